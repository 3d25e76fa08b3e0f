// scan_lookback.hip -- chunk-parallel selective-scan forward for shapes whose
// channels alone cannot fill the GPU (few channels, very long sequences).
//
// The sequence is cut into segments; every (segment k, 16-channel group)
// pair is one workgroup.  Over a segment the recurrence
// h_t = a_t h_{t-1} + b_t composes into one pair (P, h_loc): the product of
// the decays and the state reached from h = 0, and a segment's pair applied
// to the state entering it gives the state leaving it -- the pair operator
// (P1,h1) (+) (P2,h2) = (P2 P1, P2 h1 + h2) (www.mhpq.cn/news/984979 essay
// section 2.3, and its three-phase grid scan: local sweep, carry of block
// tails, fix-up).  Each workgroup:
//
//   1. walks its segment from h = 0 without output (the state-only walk of
//      scan_core.h), giving h_loc, and forms P = exp(A * sum dl) in log space
//      ("Mamba状态空间模型的硬件感知推理优化" (ybb.press) section 6.2); the
//      last segment, whose pair nobody reads, skips this walk;
//   2. publishes its pair (P, h_loc), waits for the pairs of segments
//      0 .. k-1, and folds them in that order from the caller's initial
//      state: h = P_j h + h_loc_j, one fused multiply-add per state element
//      and predecessor, gives its incoming state h_in;
//   3. walks its segment again from h_in, now forming y.
//
// Steps 1 and 3 -- all of the exponentials -- run in parallel over every
// segment, and so does step 2: every segment folds its predecessors' pairs
// itself instead of waiting for a chain of inclusive states handed from
// segment to segment (which put one hand-over latency per segment on the
// critical path).  The fold is the same sequence of fused multiply-adds, in
// the same order, for every segment and every run, so results are bitwise
// repeatable.
//
// Work is handed out by an atomic ticket in segment-major order, so a
// workgroup only ever waits for a ticket taken before its own, by a
// workgroup that is already running: every wait ends.  Published states
// cross the eight XCDs' separate L2 caches.  Every access to them and to the
// flags is an agent-scope (coherent) atomic: a writer waits for its state
// stores to be acknowledged, synchronises the workgroup, then stores the
// flag; a reader polls the flag, synchronises the workgroup, then loads.
//
// The result differs from the sequential loop only by the association of
// the carried state across segment boundaries and the rounding of P.  Every
// workgroup reads the initial state before it publishes its pair, so when h0
// is the h_last buffer, the last segment (which waits for every pair before
// its output walk) writes h_last after all the reads.
#include <algorithm>
#include <mutex>

#include "internal.h"
#include "mssm.h"
#include "scan_core.h"

namespace mssm {

// Status bits of this device (mssm_device_status): kernels set them with an
// atomic OR, the host reads and clears them.  Each device's copy of the code
// object holds its own word.
__device__ uint32_t g_device_status_bits;

// Scratch of the entry point that allocates nothing: a fixed array per
// device, held until the process ends.  Host code never passes the array's
// name to a kernel (on the host it is only a stand-in for the symbol): it
// takes the device address from hipGetSymbolAddress once per device.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

using core::kCh;

constexpr uint32_t kFlagPair = 1;        // the segment's pair (P, h_loc) published
constexpr uint32_t kFlagTimedOut = 2;    // local marker: the wait gave up
constexpr uint32_t kMaxSpins = 1u << 24;

__device__ __forceinline__ void store_agent(float *p, float v) {
    __hip_atomic_store(reinterpret_cast<uint32_t *>(p), __float_as_uint(v), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until this wave's stores have been acknowledged.  The published
// states are agent-scope (coherent) stores, so once they are acknowledged any
// agent-scope load sees them; no cache write-back or invalidate is needed --
// the release/acquire fences of the memory model would write back or drop
// the whole L2 of this XCD at every hand-over.
__device__ __forceinline__ void stores_done() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ float load_agent(const float *p) {
    return __uint_as_float(__hip_atomic_load(reinterpret_cast<const uint32_t *>(p), __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT));
}

// Scratch layout: per item (segment k, global group index gidx) the pair:
// P (`slots` floats) then h_loc (`slots` floats); then one flag per item, then
// the ticket counter.
struct Scratch {
    float *pay;
    uint32_t *flags;
    uint32_t *ticket;
};

template <typename T, int W, int NPL, bool GATE, bool VEC, bool CONV>
__global__ __launch_bounds__(64 * W) void scan_lookback_kernel(
    const T *__restrict__ u, const T *__restrict__ delta,
    const float *__restrict__ delta_bias, const float *__restrict__ A,
    const T *__restrict__ Bm, const T *__restrict__ Cm,
    const float *__restrict__ Dskip, const T *__restrict__ z, const float *h0, T *__restrict__ y,
    float *h_last, int64_t L, int dim, int N, int groups_per_batch,
    int total_groups, int64_t seg_len, int nseg, Scratch s, const float *__restrict__ conv_w,
    const float *__restrict__ conv_b) {
    constexpr int kSlots = 4 * W * NPL * kCh;
    __shared__ core::Smem<W> sm;
    __shared__ uint32_t sh_item, sh_flag;

    const int tid = threadIdx.x;
    if (tid == 0) sh_item = __hip_atomic_fetch_add(s.ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const int item = static_cast<int>(sh_item);
    const int k = item / total_groups;               // segment
    const int gidx = item - k * total_groups;        // (batch, group)
    const int64_t b = gidx / groups_per_batch;
    const int d0 = (gidx - static_cast<int>(b) * groups_per_batch) * kCh;

    core::Walker<T, W, NPL, GATE, VEC, CONV> wk;
    wk.init(u, delta, delta_bias, A, Bm, Cm, Dskip, z, y, L, dim, N, b, d0, conv_w, conv_b);
    const int t_begin = static_cast<int>(static_cast<int64_t>(k) * seg_len);
    const int t_end = static_cast<int>(min(L, static_cast<int64_t>(t_begin) + seg_len));

    // ---- 1. local pair of the segment ---------------------------------------
    // (the last segment's pair is never used: it skips this walk)
    float h[NPL], P[NPL];
#pragma unroll
    for (int g = 0; g < NPL; ++g) h[g] = 0.0f, P[g] = 0.0f;
    if (k < nseg - 1) {
        wk.template walk<false>(t_begin, t_end, h, sm);
        const float sdl = wk.channel_dl_sum(sm);
#pragma unroll
        for (int g = 0; g < NPL; ++g) P[g] = fast_exp2(wk.A2[g] * sdl);
    }

    // ---- 2. publish the pair, fold the predecessors' pairs ---------------------
    auto slot = [&](int g) { return (wk.prow * NPL + g) * kCh + wk.j; };
    auto pair = [&](int seg) {
        return s.pay + (static_cast<int64_t>(seg) * total_groups + gidx) * (2 * kSlots);
    };
    // The fold starts from the caller's initial state (lanes of channels past
    // the last one mirror the last channel, whose y their owners store again,
    // so they take its initial state).  It is read before the pair is
    // published: the flag store below comes after the read has returned.
    float h_in[NPL];
    const bool row_ok = d0 + wk.j < dim;
    const int dS = min(d0 + wk.j, dim - 1);
#pragma unroll
    for (int g = 0; g < NPL; ++g)
        h_in[g] = (h0 && wk.nok[g])
                      ? h0[(b * dim + dS) * static_cast<int64_t>(N) + wk.prow * NPL + g]
                      : 0.0f;
    if (k < nseg - 1) {
        float *mine = pair(k);
#pragma unroll
        for (int g = 0; g < NPL; ++g) {
            store_agent(mine + slot(g), P[g]);
            store_agent(mine + kSlots + slot(g), h[g]);
        }
    }
    stores_done();
    __syncthreads();
    if (tid == 0 && k < nseg - 1)
        __hip_atomic_store(s.flags + static_cast<int64_t>(k) * total_groups + gidx, kFlagPair,
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (k > 0) {
        // The first wave polls the predecessors' flags, one lane per flag.
        // Each of them publishes before it waits for anything, so every wait
        // ends; the bound (about a second per lane) only guards against a
        // bug: the state becomes NaN instead of the kernel hanging, and the
        // device's MSSM_DEVICE_LOOKBACK_TIMEOUT status bit is set.
        if (tid < 64) {
            bool bad = false;
            for (int j0 = 0; j0 < k; j0 += 64) {
                const int j = j0 + tid;
                if (j < k) {
                    const uint32_t *f = s.flags + static_cast<int64_t>(j) * total_groups + gidx;
                    uint32_t spins = 0;
                    while (__hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0) {
                        __builtin_amdgcn_s_sleep(2);
                        if (++spins == kMaxSpins) { bad = true; break; }
                    }
                }
            }
            const bool any_bad = __any(bad);
            if (tid == 0) {
                sh_flag = any_bad ? kFlagTimedOut : kFlagPair;
                if (any_bad)
                    __hip_atomic_fetch_or(&g_device_status_bits, MSSM_DEVICE_LOOKBACK_TIMEOUT,
                                          __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        __syncthreads();
        if (sh_flag == kFlagTimedOut) {
#pragma unroll
            for (int g = 0; g < NPL; ++g) h_in[g] = __builtin_nanf("");
        } else {
            // h = P_j h + h_loc_j for j = 0 .. k-1, in that order.  The pairs
            // are loaded a batch at a time so their latencies overlap.
            constexpr int kBatch = NPL == 1 ? 16 : 4;
            for (int j0 = 0; j0 < k; j0 += kBatch) {
                float pv[kBatch][NPL], hv[kBatch][NPL];
#pragma unroll
                for (int i = 0; i < kBatch; ++i) {
                    const float *pj = pair(min(j0 + i, k - 1));   // past k-1: loaded, unused
#pragma unroll
                    for (int g = 0; g < NPL; ++g) {
                        pv[i][g] = load_agent(pj + slot(g));
                        hv[i][g] = load_agent(pj + kSlots + slot(g));
                    }
                }
#pragma unroll
                for (int i = 0; i < kBatch; ++i)
                    if (j0 + i < k) {
#pragma unroll
                        for (int g = 0; g < NPL; ++g) h_in[g] = fmaf(pv[i][g], h_in[g], hv[i][g]);
                    }
            }
        }
    }

    // ---- 3. output walk from the true incoming state ---------------------------
#pragma unroll
    for (int g = 0; g < NPL; ++g) h[g] = h_in[g];
    wk.template walk<true>(t_begin, t_end, h, sm);
    if (k == nseg - 1 && h_last && row_ok) {
#pragma unroll
        for (int g = 0; g < NPL; ++g)
            if (wk.nok[g])
                h_last[(b * dim + d0 + wk.j) * static_cast<int64_t>(N) + wk.prow * NPL + g] = h[g];
    }
}

__global__ void zero_u32_kernel(uint32_t *p, int64_t n) {
    int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (; i < n; i += stride) p[i] = 0u;
}

struct Plan {
    int groups_per_batch, total_groups, nseg;
    int64_t seg_len;
};

// Segments: about as many (segment, group) workgroups as the chip holds at
// once (three per compute unit, 256 units), so every segment runs
// concurrently and no segment waits for a predecessor that has not yet been
// scheduled; each segment is a whole number of 32-step chunks and at least
// 256 steps long.
Plan make_plan(const ScanArgs &a) {
    Plan p;
    p.groups_per_batch = static_cast<int>((a.dim + kCh - 1) / kCh);
    p.total_groups = static_cast<int>(a.batch * p.groups_per_batch);
    const int64_t target_items = 3 * 256;
    int64_t nseg = (target_items + p.total_groups - 1) / p.total_groups;
    int64_t seg = (a.L + nseg - 1) / nseg;
    seg = (seg + core::kT - 1) / core::kT * core::kT;
    if (seg < 256) seg = 256;
    p.seg_len = seg;
    p.nseg = static_cast<int>((a.L + seg - 1) / seg);
    return p;
}

// Layout of the look-back scratch: the pairs of every (segment, group) item
// (2 * kSlots floats each), then one flag per item and the ticket.
template <int W, int NPL>
void scratch_layout(const ScanArgs &a, int64_t *items, size_t *pay_bytes, size_t *flag_bytes) {
    constexpr int kSlots = 4 * W * NPL * kCh;
    const Plan p = make_plan(a);
    *items = static_cast<int64_t>(p.nseg) * p.total_groups;
    *pay_bytes = static_cast<size_t>(*items) * (2 * kSlots) * sizeof(float);
    *flag_bytes = static_cast<size_t>(*items + 1) * sizeof(uint32_t);
}

// `pre`: caller-provided scratch of at least the layout's size (the no-alloc
// entry point); null: allocated and freed stream-ordered here.
template <typename T, int W, int NPL, bool CONV>
hipError_t launch_typed(const ScanArgs &a, hipStream_t stream, void *pre) {
    const Plan p = make_plan(a);
    int64_t items;
    size_t pay_bytes, flag_bytes;
    scratch_layout<W, NPL>(a, &items, &pay_bytes, &flag_bytes);
    void *mem = pre;
    hipError_t e = hipSuccess;
    if (!pre) {
        e = scratch_alloc(&mem, pay_bytes + flag_bytes, stream);
        if (e != hipSuccess) return e;
    }
    Scratch s;
    s.pay = static_cast<float *>(mem);
    s.flags = reinterpret_cast<uint32_t *>(static_cast<char *>(mem) + pay_bytes);
    s.ticket = s.flags + items;
    const int64_t nflags = items + 1;
    const int zb = static_cast<int>(std::min<int64_t>((nflags + 255) / 256, 1024));
    hipLaunchKernelGGL(zero_u32_kernel, dim3(zb), dim3(256), 0, stream, s.flags, nflags);
    e = hipGetLastError();
    if (e == hipSuccess) {
        const bool vec = scan_rows_vectorizable(a);
        decltype(&scan_lookback_kernel<T, W, NPL, true, true, CONV>) kern;
        if (a.z) kern = vec ? scan_lookback_kernel<T, W, NPL, true, true, CONV> : scan_lookback_kernel<T, W, NPL, true, false, CONV>;
        else kern = vec ? scan_lookback_kernel<T, W, NPL, false, true, CONV> : scan_lookback_kernel<T, W, NPL, false, false, CONV>;
        hipLaunchKernelGGL(kern, dim3(static_cast<uint32_t>(items)), dim3(64 * W), 0, stream,
                           static_cast<const T *>(a.u), static_cast<const T *>(a.delta),
                           a.delta_bias, a.A, static_cast<const T *>(a.B),
                           static_cast<const T *>(a.C), a.D, static_cast<const T *>(a.z), a.h0,
                           static_cast<T *>(a.y), a.h_last, a.L, static_cast<int>(a.dim),
                           static_cast<int>(a.N), p.groups_per_batch, p.total_groups, p.seg_len,
                           p.nseg, s, a.conv_w, a.conv_b);
        e = hipGetLastError();
    }
    if (pre) return e;
    const hipError_t ef = scratch_free(mem, stream);
    return e != hipSuccess ? e : ef;
}

template <typename T, int W, int NPL>
hipError_t launch_conv(const ScanArgs &a, hipStream_t stream, void *pre) {
    return a.conv_w ? launch_typed<T, W, NPL, true>(a, stream, pre)
                    : launch_typed<T, W, NPL, false>(a, stream, pre);
}

template <typename T>
hipError_t launch_by_n(const ScanArgs &a, hipStream_t stream, void *pre) {
    if (a.N <= 16) return launch_conv<T, 4, 1>(a, stream, pre);
    if (a.N <= 32) return launch_conv<T, 2, 4>(a, stream, pre);
    return launch_conv<T, 4, 4>(a, stream, pre);
}

// Device address of this device's scratch array, looked up once per device
// (with that device current) and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

hipError_t device_scratch(void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace

size_t scan_lookback_scratch_bytes(const ScanArgs &a) {
    int64_t items;
    size_t pay, flags;
    if (a.N <= 16) scratch_layout<4, 1>(a, &items, &pay, &flags);
    else if (a.N <= 32) scratch_layout<2, 4>(a, &items, &pay, &flags);
    else scratch_layout<4, 4>(a, &items, &pay, &flags);
    return pay + flags;
}

hipError_t launch_scan_lookback_noalloc(const ScanArgs &a, hipStream_t stream) {
    if (scan_lookback_scratch_bytes(a) > kNoAllocScratchBytes) return hipErrorInvalidValue;
    void *pre = nullptr;
    const hipError_t e = device_scratch(&pre);
    if (e != hipSuccess) return e;
    if (a.io == IO_F32) return launch_by_n<float>(a, stream, pre);
    return launch_by_n<uint16_t>(a, stream, pre);
}

bool scan_lookback_supported(const ScanArgs &a) {
    if (a.N < 1 || a.N > 64 || !scan_offsets_fit(a)) return false;
    const int64_t groups = a.batch * ((a.dim + kCh - 1) / kCh);
    if (groups >= (int64_t(1) << 20)) return false;
    const Plan p = make_plan(a);
    return static_cast<int64_t>(p.nseg) * p.total_groups < (int64_t(1) << 31);
}

hipError_t device_status(uint32_t *bits, bool clear) {
    void *p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(g_device_status_bits));
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e == hipSuccess) e = hipMemcpy(bits, p, sizeof(uint32_t), hipMemcpyDeviceToHost);
    if (e == hipSuccess && clear) {
        const uint32_t zero = 0;
        e = hipMemcpy(p, &zero, sizeof(uint32_t), hipMemcpyHostToDevice);
    }
    return e;
}

hipError_t launch_scan_lookback(const ScanArgs &a, hipStream_t stream) {
    if (a.io == IO_F32) return launch_by_n<float>(a, stream, nullptr);
    return launch_by_n<uint16_t>(a, stream, nullptr);
}

}  // namespace mssm
