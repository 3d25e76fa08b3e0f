// scan_bwd_rowserial.hip -- backward of the selective scan in its plainest
// GPU form: one lane owns one (batch, channel) row, as in the row-serial
// forward, and differentiates its walk in reverse.
//
// Forward per step ("Mamba状态空间模型的硬件感知推理优化" (ybb.press) sections 1
// and 3.1; www.mhpq.cn/news/984979 essay section 2.2; the tencentcloud.csdn.net
// Mamba article, sections 2-3):
//   x = delta + bias, dl = softplus(x), a[n] = exp(dl A[n])
//   h[n] = a[n] h[n] + dl B[n] u,  s = sum_n C[n] h[n] + D u,  y = s silu(z)
// Reverse, from dh = dh_last at the end (the chain rule through each step):
//   ds = dy silu(z), dz = dy s silu'(z), dh[n] += ds C[n],
//   dC[n] += ds h[n], dD += ds u, dA[n] += dh[n] h_prev[n] a[n] dl,
//   dB[n] += dh[n] dl u, du = ds D + sum_n dh[n] dl B[n],
//   d(dl) = sum_n dh[n] (h_prev[n] a[n] A[n] + B[n] u), ddelta = d(dl) sigmoid(x),
//   dh[n] <- a[n] dh[n]  (carried to the step before); dh0 = dh at the start.
//
// The reverse walk needs h_prev at every step.  The forward walk stores the
// state every K steps (K * N floats stay in registers); the reverse walk
// recomputes each K-step segment from its stored state, keeps the segment's
// states in registers and walks them backwards.  The stored states take
// rows * ceil(L / K) * N floats of scratch, allocated stream-ordered.
//
// dB and dC sum over channels, dA, dD and the bias gradient over batches:
// a wave first sums over its 64 rows (when they share a batch) with lane
// shuffles, then one lane adds the sum atomically.  This is the parity form
// (few waves for few rows, many atomics); the summation order of the
// atomics makes those sums order-dependent in the last bits.
#include "device_math.h"
#include "internal.h"

namespace mssm {
namespace {

// Segment length: the K states of a segment stay in registers (K * NS floats).
template <int NS>
constexpr int seg_steps() { return NS <= 4 ? 32 : NS <= 8 ? 16 : NS <= 16 ? 8 : NS <= 32 ? 4 : 2; }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}

// v summed over the rows of this wave into *p: one atomic per wave when all
// 64 rows share the address, else one per lane.
__device__ __forceinline__ void add_rows(float *p, float v, bool shared, int lane) {
    if (shared) {
        v = wave_sum(v);
        if (lane == 0) atomicAdd(p, v);
    } else {
        atomicAdd(p, v);
    }
}

template <typename T, int NS>
__global__ __launch_bounds__(64) void scan_bwd_rowserial_kernel(BwdArgs a, float *__restrict__ ck,
                                                                int nseg) {
    constexpr int K = seg_steps<NS>();
    const T *u = static_cast<const T *>(a.u);
    const T *delta = static_cast<const T *>(a.delta);
    const T *Bm = static_cast<const T *>(a.B);
    const T *Cm = static_cast<const T *>(a.C);
    const T *z = static_cast<const T *>(a.z);
    const T *dy = static_cast<const T *>(a.dy);
    const int64_t rows = a.batch * a.dim, L = a.L;
    const int N = static_cast<int>(a.N);
    const int lane = threadIdx.x;
    const int64_t row = static_cast<int64_t>(blockIdx.x) * 64 + lane;
    const bool valid = row < rows;
    // lanes past the last row walk the last row with zero output gradients,
    // so every lane takes part in the wave sums and contributes nothing
    const int64_t r = valid ? row : rows - 1;
    const int64_t b = r / a.dim;
    const int64_t d = r - b * a.dim;
    // all rows of the wave in one batch (the common case): sums over rows can
    // go through the wave first
    const int64_t r_first = static_cast<int64_t>(blockIdx.x) * 64;
    const int64_t r_last = min(r_first + 63, rows - 1);
    const bool one_batch = r_first / a.dim == r_last / a.dim;

    float A2[NS];
#pragma unroll
    for (int n = 0; n < NS; ++n) A2[n] = n < N ? a.A[d * N + n] * kLog2e : 0.0f;
    const float bias = a.delta_bias ? a.delta_bias[d] : 0.0f;
    const float skip = a.D ? a.D[d] : 0.0f;
    const int64_t rb = r * L;
    const T *Bb = Bm + b * N * L;
    const T *Cb = Cm + b * N * L;
    float *ckr = ck + r * static_cast<int64_t>(nseg) * N;

    // ---- forward: the state before every segment ---------------------------
    float h[NS];
#pragma unroll
    for (int n = 0; n < NS; ++n) h[n] = (a.h0 && n < N) ? a.h0[r * N + n] : 0.0f;
    for (int s = 0; s < nseg; ++s) {
        if (valid) {
#pragma unroll
            for (int n = 0; n < NS; ++n)
                if (n < N) ckr[s * N + n] = h[n];
        }
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int64_t t = static_cast<int64_t>(s) * K + k;
            if (t < L) {
                const float dl = softplus_libm(Io<T>::load(delta, rb + t) + bias);
                const float du = dl * Io<T>::load(u, rb + t);
#pragma unroll
                for (int n = 0; n < NS; ++n)
                    if (n < N) h[n] = fmaf(fast_exp2(dl * A2[n]), h[n], du * Io<T>::load(Bb, n * L + t));
            }
        }
    }

    // ---- reverse ---------------------------------------------------------
    float dh[NS], dAacc[NS];
#pragma unroll
    for (int n = 0; n < NS; ++n) {
        dh[n] = (valid && a.dh_last && n < N) ? a.dh_last[r * N + n] : 0.0f;
        dAacc[n] = 0.0f;
    }
    float dDacc = 0.0f, dbacc = 0.0f;
    for (int s = nseg - 1; s >= 0; --s) {
        const int64_t t0 = static_cast<int64_t>(s) * K;
        float hb[NS], hs[K][NS];
#pragma unroll
        for (int n = 0; n < NS; ++n) hb[n] = n < N ? ckr[s * N + n] : 0.0f;
        // the segment's states, recomputed
#pragma unroll
        for (int n = 0; n < NS; ++n) h[n] = hb[n];
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int64_t t = t0 + k;
            if (t < L) {
                const float dl = softplus_libm(Io<T>::load(delta, rb + t) + bias);
                const float du = dl * Io<T>::load(u, rb + t);
#pragma unroll
                for (int n = 0; n < NS; ++n)
                    if (n < N) h[n] = fmaf(fast_exp2(dl * A2[n]), h[n], du * Io<T>::load(Bb, n * L + t));
            }
#pragma unroll
            for (int n = 0; n < NS; ++n) hs[k][n] = h[n];
        }
        // walked backwards
#pragma unroll
        for (int k = K - 1; k >= 0; --k) {
            const int64_t t = t0 + k;
            if (t >= L) continue;
            const float x = Io<T>::load(delta, rb + t) + bias;
            const float dl = softplus_libm(x);
            const float sig = 1.0f / (1.0f + expf(-x));
            const float ut = Io<T>::load(u, rb + t);
            const float dyt = valid ? Io<T>::load(dy, rb + t) : 0.0f;
            float ds = dyt;
            if (z) {
                const float zt = Io<T>::load(z, rb + t);
                float sv = skip * ut;
#pragma unroll
                for (int n = 0; n < NS; ++n)
                    if (n < N) sv = fmaf(Io<T>::load(Cb, n * L + t), hs[k][n], sv);
                const float sz = 1.0f / (1.0f + expf(-zt));
                ds = dyt * zt * sz;
                if (valid && a.dz) a.dz[rb + t] = dyt * sv * sz * (1.0f + zt * (1.0f - sz));
            }
            dDacc = fmaf(ds, ut, dDacc);
            float dut = ds * skip, ddl = 0.0f;
#pragma unroll
            for (int n = 0; n < NS; ++n) {
                if (n < N) {
                    const float Bt = Io<T>::load(Bb, n * L + t);
                    const float Ct = Io<T>::load(Cb, n * L + t);
                    const float an = fast_exp2(dl * A2[n]);
                    const float hp = k > 0 ? hs[k > 0 ? k - 1 : 0][n] : hb[n];
                    dh[n] = fmaf(ds, Ct, dh[n]);
                    if (a.dC) add_rows(a.dC + (b * N + n) * L + t, ds * hs[k][n], one_batch, lane);
                    const float ha = hp * an;
                    dAacc[n] = fmaf(dh[n] * ha, dl, dAacc[n]);
                    if (a.dB) add_rows(a.dB + (b * N + n) * L + t, dh[n] * dl * ut, one_batch, lane);
                    dut = fmaf(dh[n] * dl, Bt, dut);
                    ddl = fmaf(dh[n], fmaf(ha, A2[n] * kLn2, Bt * ut), ddl);
                    dh[n] *= an;
                }
            }
            if (valid) {
                a.du[rb + t] = dut;
                a.ddelta[rb + t] = ddl * sig;
            }
            dbacc = fmaf(ddl, sig, dbacc);
        }
    }
    if (valid) {
        if (a.dh0) {
#pragma unroll
            for (int n = 0; n < NS; ++n)
                if (n < N) a.dh0[r * N + n] = dh[n];
        }
        if (a.dA) {
#pragma unroll
            for (int n = 0; n < NS; ++n)
                if (n < N) atomicAdd(a.dA + d * N + n, dAacc[n]);
        }
        if (a.dD) atomicAdd(a.dD + d, dDacc);
        if (a.ddelta_bias) atomicAdd(a.ddelta_bias + d, dbacc);
    }
}

template <typename T, int NS>
hipError_t launch_typed(const BwdArgs &a, hipStream_t stream) {
    constexpr int K = seg_steps<NS>();
    const int64_t rows = a.batch * a.dim;
    const int nseg = static_cast<int>((a.L + K - 1) / K);
    void *mem = nullptr;
    hipError_t e = hipMallocAsync(&mem, static_cast<size_t>(rows) * nseg * a.N * sizeof(float), stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((scan_bwd_rowserial_kernel<T, NS>), dim3(static_cast<uint32_t>((rows + 63) / 64)),
                       dim3(64), 0, stream, a, static_cast<float *>(mem), nseg);
    e = hipGetLastError();
    const hipError_t ef = hipFreeAsync(mem, stream);
    return e != hipSuccess ? e : ef;
}

template <typename T>
hipError_t launch_by_n(const BwdArgs &a, hipStream_t stream) {
    if (a.N <= 4) return launch_typed<T, 4>(a, stream);
    if (a.N <= 8) return launch_typed<T, 8>(a, stream);
    if (a.N <= 16) return launch_typed<T, 16>(a, stream);
    if (a.N <= 32) return launch_typed<T, 32>(a, stream);
    return launch_typed<T, 64>(a, stream);
}

}  // namespace

bool scan_bwd_supported(const BwdArgs &a) {
    return a.N >= 1 && a.N <= 64 && (a.batch * a.dim + 63) / 64 < (int64_t(1) << 31) &&
           a.L < (int64_t(1) << 31);
}

hipError_t launch_scan_bwd(const BwdArgs &a, hipStream_t stream) {
    if (a.io == IO_F32) return launch_by_n<float>(a, stream);
    return launch_by_n<uint16_t>(a, stream);
}

}  // namespace mssm
