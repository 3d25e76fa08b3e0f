// state_update.hip -- one decode step of the selective scan: the recurrence
// advanced by a single time step on a state kept between calls.
//
// Per batch b and channel d ("Mamba状态空间模型的硬件感知推理优化" (ybb.press)
// sections 1 and 3.1: h_t = exp(A dl) h_{t-1} + dl B x_t, y = C.h + D x; the
// tencentcloud.csdn.net article on Mamba, section 3: the SiLU gate; the
// www.mhpq.cn essay, section 2.2: the zero-order-hold decay):
//
//   dl       = softplus(dt[b,d] + dt_bias[d])
//   state[n] = exp(dl * A[d,n]) * state[n] + dl * B[b,n] * x[b,d]
//   y[b,d]   = (sum_n C[b,n] * state[n] + D[d] * x[b,d]) * silu(z[b,d])
//
// The step reads and writes the whole float32 state once and does a handful
// of operations per element, so it is bound by HBM bandwidth.  The layout
// follows from that: a group of GS lanes owns one (b, d) row, each lane four
// consecutive state elements moved as one 16-byte load and store, so a wave
// streams 64 x 16 contiguous bytes of state per sequence; the output dot
// product is summed across the group with lane shuffles.
#include "device_math.h"
#include "internal.h"

namespace mssm {
namespace {

template <typename T> struct Quad;
template <> struct Quad<float> {
    // four consecutive elements at p (16-byte aligned)
    __device__ __forceinline__ static float4 load(const float *p) { return *reinterpret_cast<const float4 *>(p); }
};
template <> struct Quad<uint16_t> {
    // four consecutive elements at p (8-byte aligned)
    __device__ __forceinline__ static float4 load(const uint16_t *p) {
        const uint2 v = *reinterpret_cast<const uint2 *>(p);
        return make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u),
                           __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xffff0000u));
    }
};

// Elements n0 .. n0 + 3 of a row of length N; VEC: all four exist and the
// row start is aligned for a vector load; otherwise missing ones read as 0.
template <bool VEC, typename T>
__device__ __forceinline__ float4 load4(const T *row, int n0, int N) {
    if (VEC) return Quad<T>::load(row + n0);
    float v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = n0 + k < N ? Io<T>::load(row, n0 + k) : 0.0f;
    return make_float4(v[0], v[1], v[2], v[3]);
}

// Sequences per thread: each thread advances the same channel d (and the
// same four state elements) of RB sequences, so its row of A is loaded once
// and RB independent 16-byte state loads are in flight at a time.  Measured
// on the 256-sequence Mamba-2.8B step: RB = 2 reaches 5.3 TB/s, against
// 4.7 TB/s for RB = 1 or 4 and 3.2 TB/s for RB = 8.
constexpr int kRB = 2;

typedef float vf4 __attribute__((ext_vector_type(4)));

// The state is streamed: read once, written once, not reused by this step,
// so its loads and stores carry the nontemporal hint (5.3 against 4.6 TB/s).
__device__ __forceinline__ float4 load_state4(const float *p) {
    const vf4 t = __builtin_nontemporal_load(reinterpret_cast<const vf4 *>(p));
    return make_float4(t.x, t.y, t.z, t.w);
}
__device__ __forceinline__ void store_state4(float *p, float4 v) {
    const vf4 t = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(t, reinterpret_cast<vf4 *>(p));
}

// v where ok, else 0, through a mask the optimiser cannot see through: a
// select between a freshly loaded value and zero is turned into a branch
// around the load that waits for it, which serialises the loads.
__device__ __forceinline__ float keep_if(float v, bool ok) {
    uint32_t m = ok ? ~0u : 0u;
    asm("" : "+v"(m));
    return __uint_as_float(__float_as_uint(v) & m);
}

template <typename T, int GS, bool VEC>
__global__ __launch_bounds__(256) void state_update_kernel(
    float *__restrict__ state, const T *__restrict__ x, const T *__restrict__ dt,
    const float *__restrict__ dt_bias, const float *__restrict__ A, const T *__restrict__ B,
    const T *__restrict__ C, const float *__restrict__ Dskip, const T *__restrict__ z,
    T *__restrict__ y, int64_t batch, int dim, int N, int dblocks) {
    constexpr int kRows = 256 / GS;                      // channels per workgroup
    const int q = threadIdx.x % GS;                      // quad of this lane
    const int dblk = static_cast<int>(blockIdx.x % static_cast<uint32_t>(dblocks));
    const int64_t b0 = static_cast<int64_t>(blockIdx.x / static_cast<uint32_t>(dblocks)) * kRB;
    const int d = dblk * kRows + static_cast<int>(threadIdx.x) / GS;
    if (d >= dim) return;                                // whole groups leave together
    const int n0 = 4 * q;
    const bool live = n0 < N;
    // Vector path: lanes past the last quad load quad 0 (in bounds) and their
    // term of the sum is zeroed, so no load sits behind a branch.
    const int nl = live ? n0 : 0;
    const float4 a = VEC ? load4<true>(A + static_cast<int64_t>(d) * N, nl, N)
                         : (live ? load4<false>(A + static_cast<int64_t>(d) * N, n0, N) : make_float4(0, 0, 0, 0));
    // optional operands: read from a valid row (A has at least dim floats) and masked
    const float bias = keep_if((dt_bias ? dt_bias : A)[d], dt_bias != nullptr);
    const float skip = keep_if((Dskip ? Dskip : A)[d], Dskip != nullptr);

    // All loads first (sequences past the batch read the last one's operands
    // and store nothing), then the arithmetic.
    float xv[kRB], dv[kRB], zv[kRB];
    float4 h[kRB], bq[kRB], cq[kRB];
#pragma unroll
    for (int i = 0; i < kRB; ++i) {
        const int64_t b = min(b0 + i, batch - 1);
        const int64_t row = b * dim + d;
        xv[i] = Io<T>::load(x, row);
        dv[i] = Io<T>::load(dt, row);
        zv[i] = Io<T>::load(z ? z : x, row);   // used only when z is given
        if (VEC) {
            h[i] = load_state4(state + row * N + nl);
            bq[i] = load4<true>(B + b * N, nl, N);
            cq[i] = load4<true>(C + b * N, nl, N);
        } else if (live) {
            h[i] = VEC ? load_state4(state + row * N + n0) : load4<VEC>(state + row * N, n0, N);
            bq[i] = load4<VEC>(B + b * N, n0, N);
            cq[i] = load4<VEC>(C + b * N, n0, N);
        } else {
            h[i] = bq[i] = cq[i] = make_float4(0, 0, 0, 0);
        }
    }
#pragma unroll
    for (int i = 0; i < kRB; ++i) {
        const int64_t b = b0 + i;
        const int64_t row = b * dim + d;
        const float dl = softplus(dv[i] + bias);
        const float dx = dl * xv[i];
        const float s = dl * kLog2e;
        float4 hn;
        hn.x = fmaf(fast_exp2(s * a.x), h[i].x, dx * bq[i].x);
        hn.y = fmaf(fast_exp2(s * a.y), h[i].y, dx * bq[i].y);
        hn.z = fmaf(fast_exp2(s * a.z), h[i].z, dx * bq[i].z);
        hn.w = fmaf(fast_exp2(s * a.w), h[i].w, dx * bq[i].w);
        float acc = fmaf(cq[i].x, hn.x, fmaf(cq[i].y, hn.y, fmaf(cq[i].z, hn.z, cq[i].w * hn.w)));
        if (VEC) acc = live ? acc : 0.0f;
        // sum over the group's lanes (aligned runs of GS lanes of one wave)
#pragma unroll
        for (int m = GS / 2; m >= 1; m /= 2) acc += __shfl_xor(acc, m, GS);
        if (b < batch) {
            if (live) {
                float *srow = state + row * N;
                if (VEC) {
                    store_state4(srow + n0, hn);
                } else {
                    const float hv[4] = {hn.x, hn.y, hn.z, hn.w};
#pragma unroll
                    for (int k = 0; k < 4; ++k)
                        if (n0 + k < N) srow[n0 + k] = hv[k];
                }
            }
            if (q == 0) {
                float yv = fmaf(skip, xv[i], acc);
                if (z) yv *= silu(zv[i]);
                Io<T>::store(y, row, yv);
            }
        }
    }
}

template <typename T, int GS>
hipError_t launch_gs(const StepArgs &a, hipStream_t stream) {
    constexpr int kRows = 256 / GS;
    const int64_t dblocks = (a.dim + kRows - 1) / kRows;
    const int64_t grid = dblocks * ((a.batch + kRB - 1) / kRB);
    // Vector path: every quad complete, rows of state / A / B / C aligned.
    const int64_t bsz = a.io == IO_F32 ? 16 : 8;
    auto al = [](const void *p, int64_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; };
    const bool vec = a.N % 4 == 0 && al(a.state, 16) && al(a.A, 16) && al(a.B, bsz) && al(a.C, bsz);
    auto kern = vec ? state_update_kernel<T, GS, true> : state_update_kernel<T, GS, false>;
    hipLaunchKernelGGL(kern, dim3(static_cast<uint32_t>(grid)), dim3(256), 0, stream, a.state,
                       static_cast<const T *>(a.x), static_cast<const T *>(a.dt), a.dt_bias, a.A,
                       static_cast<const T *>(a.B), static_cast<const T *>(a.C), a.D,
                       static_cast<const T *>(a.z), static_cast<T *>(a.y), a.batch,
                       static_cast<int>(a.dim), static_cast<int>(a.N), static_cast<int>(dblocks));
    return hipGetLastError();
}

// Lanes per row: the quads of a row, rounded up to a power of two.
template <typename T>
hipError_t launch_typed(const StepArgs &a, hipStream_t stream) {
    const int64_t quads = (a.N + 3) / 4;
    if (quads <= 1) return launch_gs<T, 1>(a, stream);
    if (quads <= 2) return launch_gs<T, 2>(a, stream);
    if (quads <= 4) return launch_gs<T, 4>(a, stream);
    if (quads <= 8) return launch_gs<T, 8>(a, stream);
    return launch_gs<T, 16>(a, stream);
}

}  // namespace

bool state_update_supported(const StepArgs &a) {
    if (a.N < 1 || a.N > 64 || a.dim > (int64_t(1) << 31) - 1) return false;
    const int64_t quads = (a.N + 3) / 4;
    int gs = 1;
    while (gs < quads) gs *= 2;
    const int64_t dblocks = (a.dim + 256 / gs - 1) / (256 / gs);
    // 256-thread workgroups: the grid's thread count stays below 2^32
    return dblocks * ((a.batch + kRB - 1) / kRB) < (int64_t(1) << 24);
}

hipError_t launch_state_update(const StepArgs &a, hipStream_t stream) {
    if (a.io == IO_F32) return launch_typed<float>(a, stream);
    return launch_typed<uint16_t>(a, stream);
}

}  // namespace mssm
