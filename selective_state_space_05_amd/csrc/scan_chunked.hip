// scan_chunked.hip -- selective-scan forward: one workgroup per (batch,
// 16-channel group) walks the whole sequence from h0 (or 0) with the fused chunk
// walk of scan_core.h.  Parallelism is over channels and state elements; the
// sequence itself is walked in order, so the recurrence is evaluated exactly
// as its sequential definition ("Mamba状态空间模型的硬件感知推理优化"
// (ybb.press) section 5: the state stays on chip across chunks).
//
// Balancing the compute units.  Workgroups are all alike, so with G of them
// on U compute units the busiest units hold ceil(G / U) and set the time.
// When G is not a multiple of U, the last r = G mod U groups are each cut in
// two parts at step S (about three quarters of L): the first part walks
// [0, S) with output; the second recomputes the state at S with the cheaper
// state-only walk over [0, S) and walks [S, L) with output.  The two parts
// cost about the same, three quarters of a whole group, and go to different
// units, so the busiest units carry ceil(G / U) - 1/4 groups of work.  The
// second part evaluates the recurrence over [0, S) in exactly the order of
// the first, so the results are identical to those of the unsplit walk.
#include <algorithm>
#include <mutex>

#include "internal.h"
#include "scan_core.h"

namespace mssm {
namespace {

using core::kCh;

template <typename T, int W, int NPL, bool GATE, bool VEC, bool CONV>
__global__ __launch_bounds__(64 * W) void scan_chunked_kernel(
    const T *__restrict__ u, const T *__restrict__ delta,
    const float *__restrict__ delta_bias, const float *__restrict__ A,
    const T *__restrict__ Bm, const T *__restrict__ Cm,
    const float *__restrict__ Dskip, const T *__restrict__ z, const float *h0, T *__restrict__ y,
    float *h_last, int64_t L, int dim, int N, int groups_per_batch, int n_whole, int n_split,
    int split_t, const float *__restrict__ conv_w, const float *__restrict__ conv_b) {
    __shared__ core::Smem<W> sm;
    // Workgroups [0, n_whole) walk groups [0, n_whole) whole; the next
    // n_split walk the first parts of groups n_whole.. up to split_t, the
    // last n_split their second parts.
    int grp = blockIdx.x, part = 0;
    if (grp >= n_whole) {
        const int i = grp - n_whole;
        part = i < n_split ? 1 : 2;
        grp = n_whole + (i < n_split ? i : i - n_split);
    }
    const int64_t b = grp / groups_per_batch;
    const int d0 = (grp - static_cast<int>(b) * groups_per_batch) * kCh;
    core::Walker<T, W, NPL, GATE, VEC, CONV> wk;
    wk.init(u, delta, delta_bias, A, Bm, Cm, Dskip, z, y, L, dim, N, b, d0, conv_w, conv_b);
    // Lanes of channels past the last one mirror the last channel (their
    // owners store its y again), so they start from its initial state too.
    float h[NPL];
    const bool row_ok = d0 + wk.j < dim;
    const int dS = min(d0 + wk.j, dim - 1);
#pragma unroll
    for (int g = 0; g < NPL; ++g)
        h[g] = (h0 && wk.nok[g])
                   ? h0[(b * dim + dS) * static_cast<int64_t>(N) + wk.prow * NPL + g]
                   : 0.0f;
    if (part == 1) {
        wk.template walk<true>(0, split_t, h, sm);
        return;
    }
    if (part == 2) {
        wk.template walk<false>(0, split_t, h, sm);
        __syncthreads();   // the state-only walk's LDS reads are done
        wk.template walk<true>(split_t, L, h, sm);
    } else {
        wk.template walk<true>(0, L, h, sm);
    }
    if (h_last && row_ok) {
#pragma unroll
        for (int g = 0; g < NPL; ++g)
            if (wk.nok[g])
                h_last[(b * dim + d0 + wk.j) * static_cast<int64_t>(N) + wk.prow * NPL + g] = h[g];
    }
}

// Compute units of the current device, queried once per device.
int device_cus() {
    static std::mutex mu;
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    std::lock_guard<std::mutex> lk(mu);
    if (cache[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) n = -1;
        cache[dev] = n;
    }
    return cache[dev];
}

// How many groups to cut in two, and where (0: none).  Only when the grid
// leaves the busiest units with one group more than others, the cut parts
// fit on the units that carry one group less, the busiest units hold at most
// three groups (so every workgroup is resident at once), and the sequence is
// long enough for a cut at a chunk boundary near three quarters of it.  The
// parts are the last workgroups of the grid, first parts before second
// parts.
struct Split { int n_split, split_t; };
Split plan_split(int64_t groups, int64_t L) {
    const int cus = device_cus();
    Split sp{0, 0};
    if (cus <= 0 || L < 16 * core::kT) return sp;
    const int64_t q = groups / cus, r = groups % cus;
    if (r == 0 || q >= 3 || 2 * r > cus) return sp;
    sp.n_split = static_cast<int>(r);
    sp.split_t = static_cast<int>((3 * L / 4) / core::kT * core::kT);
    return sp;
}

template <typename T, int W, int NPL, bool CONV>
hipError_t launch_typed(const ScanArgs &a, hipStream_t stream) {
    const int groups = static_cast<int>((a.dim + kCh - 1) / kCh);
    const int64_t total = a.batch * groups;
    // An initial state read in place of the final state (h0 == h_last) is
    // read by a group's first part and overwritten by its second, which need
    // not run after it: such calls walk every group whole.
    const Split sp = (a.h0 && a.h0 == a.h_last) ? Split{0, 0} : plan_split(total, a.L);
    const int n_whole = static_cast<int>(total - sp.n_split);
    const int64_t grid = total + sp.n_split;
    const bool vec = scan_rows_vectorizable(a);
    decltype(&scan_chunked_kernel<T, W, NPL, true, true, CONV>) kern;
    if (a.z) kern = vec ? scan_chunked_kernel<T, W, NPL, true, true, CONV> : scan_chunked_kernel<T, W, NPL, true, false, CONV>;
    else kern = vec ? scan_chunked_kernel<T, W, NPL, false, true, CONV> : scan_chunked_kernel<T, W, NPL, false, false, CONV>;
    hipLaunchKernelGGL(kern, dim3(static_cast<uint32_t>(grid)), dim3(64 * W), 0, stream,
                       static_cast<const T *>(a.u), static_cast<const T *>(a.delta),
                       a.delta_bias, a.A, static_cast<const T *>(a.B),
                       static_cast<const T *>(a.C), a.D, static_cast<const T *>(a.z), a.h0,
                       static_cast<T *>(a.y), a.h_last, a.L, static_cast<int>(a.dim),
                       static_cast<int>(a.N), groups, n_whole, sp.n_split, sp.split_t,
                       a.conv_w, a.conv_b);
    return hipGetLastError();
}

template <typename T, int W, int NPL>
hipError_t launch_conv(const ScanArgs &a, hipStream_t stream) {
    return a.conv_w ? launch_typed<T, W, NPL, true>(a, stream) : launch_typed<T, W, NPL, false>(a, stream);
}

// Four waves with one state element per lane: the most waves in flight, and
// the partial sums of a wave's four state rows are added in registers.
// Larger N puts more state elements on each lane (four per lane for N <= 32
// in two waves, four per lane in four waves up to N = 64).
template <typename T>
hipError_t launch_by_n(const ScanArgs &a, hipStream_t stream) {
    if (a.N <= 8) return launch_conv<T, 2, 1>(a, stream);
    if (a.N <= 16) return launch_conv<T, 4, 1>(a, stream);
    if (a.N <= 32) return launch_conv<T, 2, 4>(a, stream);
    return launch_conv<T, 4, 4>(a, stream);
}

}  // namespace

bool scan_rows_vectorizable(const ScanArgs &a) {
    auto aligned = [](const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
    return (a.L % 8 == 0) && aligned(a.u) && aligned(a.delta) && aligned(a.y) &&
           (!a.z || aligned(a.z));
}

bool scan_offsets_fit(const ScanArgs &a) {
    const int64_t esz = a.io == IO_F32 ? 4 : 2;
    return (a.N > kCh ? a.N : kCh) * a.L * esz < (int64_t(1) << 31);
}

bool scan_chunked_supported(const ScanArgs &a) {
    const int64_t groups = (a.dim + kCh - 1) / kCh;
    return a.N >= 1 && a.N <= 64 && a.dim <= (int64_t(1) << 30) && scan_offsets_fit(a) &&
           a.batch * groups < (int64_t(1) << 30);
}

int64_t scan_chunked_waves(const ScanArgs &a) {
    const int64_t groups = a.batch * ((a.dim + kCh - 1) / kCh);
    return groups * ((a.N > 8 && a.N <= 16) || a.N > 32 ? 4 : 2);
}

hipError_t launch_scan_chunked(const ScanArgs &a, hipStream_t stream) {
    if (a.io == IO_F32) return launch_by_n<float>(a, stream);
    return launch_by_n<uint16_t>(a, stream);
}

}  // namespace mssm
