// ssd_recurrent.hip -- Mamba-2 scalar-decay (SSD) forward as a plain
// recurrence: one lane owns one (batch, head, headdim) row and keeps its
// N-element slice of the state in registers.
//
// With a scalar decay per (step, head) ("Mamba状态空间模型的硬件感知推理优化"
// (ybb.press) section 4), every headdim index p evolves independently:
//   dl   = softplus(dt + dt_bias[h]);  a = exp(dl * A[h])
//   S[n] = a * S[n] + (dl * x[p]) * B[n]
//   y[p] = (sum_n C[n] * S[n] + D[h] * x[p]) * silu(z[p])   (z optional)
// The 64 lanes of a wave are consecutive p of one (b, h), so B and C reads
// are uniform across the wave.  This is the parity form; the chunked
// matrix-core form is the fast path for long sequences.
#include "device_math.h"
#include "internal.h"

namespace mssm {
namespace {

template <typename T, int NS>
__global__ __launch_bounds__(64) void ssd_recurrent_kernel(
    const T *__restrict__ x, const T *__restrict__ dt,
    const float *__restrict__ dt_bias, const float *__restrict__ A,
    const T *__restrict__ B, const T *__restrict__ C,
    const float *__restrict__ Dskip, const T *__restrict__ z, const float *h0, T *__restrict__ y,
    float *h_last, int64_t L, int H, int P, int N, int G) {
    // grid: x = p-tiles of 64, y = head, z = batch
    const int p = blockIdx.x * 64 + threadIdx.x;
    const int h = blockIdx.y;
    const int64_t b = blockIdx.z;
    const int g = h / (H / G);
    const bool live = p < P;

    const int64_t sbase = ((b * H + h) * static_cast<int64_t>(P) + p) * N;
    float S[NS];
#pragma unroll
    for (int n = 0; n < NS; ++n) S[n] = (h0 && live && n < N) ? h0[sbase + n] : 0.0f;
    const float A2 = A[h] * kLog2e;
    const float bias = dt_bias ? dt_bias[h] : 0.0f;
    const float skip = Dskip ? Dskip[h] : 0.0f;

    for (int64_t t = 0; t < L; ++t) {
        const float dl = softplus_libm(Io<T>::load(dt, (b * L + t) * H + h) + bias);
        const float a = fast_exp2(dl * A2);
        const int64_t xi = ((b * L + t) * H + h) * static_cast<int64_t>(P) + p;
        const float xp = live ? Io<T>::load(x, xi) : 0.0f;
        const float dx = dl * xp;
        const int64_t bc = ((b * L + t) * G + g) * static_cast<int64_t>(N);
        float acc = 0.0f;
#pragma unroll
        for (int n = 0; n < NS; ++n) {
            if (n < N) {
                S[n] = fmaf(a, S[n], dx * Io<T>::load(B, bc + n));
                acc = fmaf(Io<T>::load(C, bc + n), S[n], acc);
            }
        }
        if (live) {
            float yv = fmaf(skip, xp, acc);
            if (z) yv *= silu_libm(Io<T>::load(z, xi));
            Io<T>::store(y, xi, yv);
        }
    }
    if (h_last && live) {
#pragma unroll
        for (int n = 0; n < NS; ++n)
            if (n < N) h_last[sbase + n] = S[n];
    }
}

template <typename T, int NS>
hipError_t launch_typed(const SSDArgs &a, hipStream_t stream) {
    dim3 grid(static_cast<uint32_t>((a.P + 63) / 64), static_cast<uint32_t>(a.H),
              static_cast<uint32_t>(a.batch));
    hipLaunchKernelGGL((ssd_recurrent_kernel<T, NS>), grid, dim3(64), 0, stream,
                       static_cast<const T *>(a.x), static_cast<const T *>(a.dt),
                       a.dt_bias, a.A, static_cast<const T *>(a.B),
                       static_cast<const T *>(a.C), a.D, static_cast<const T *>(a.z), a.h0,
                       static_cast<T *>(a.y),
                       a.h_last, a.L, static_cast<int>(a.H), static_cast<int>(a.P),
                       static_cast<int>(a.N), static_cast<int>(a.G));
    return hipGetLastError();
}

template <typename T>
hipError_t launch_by_n(const SSDArgs &a, hipStream_t stream) {
    if (a.N <= 16) return launch_typed<T, 16>(a, stream);
    if (a.N <= 32) return launch_typed<T, 32>(a, stream);
    if (a.N <= 64) return launch_typed<T, 64>(a, stream);
    if (a.N <= 128) return launch_typed<T, 128>(a, stream);
    return launch_typed<T, 256>(a, stream);
}

}  // namespace

bool ssd_recurrent_supported(const SSDArgs &a) {
    return a.N >= 1 && a.N <= 256 && a.P >= 1 && a.P <= 256 && a.H <= 65535 &&
           a.batch <= 65535;
}

hipError_t launch_ssd_recurrent(const SSDArgs &a, hipStream_t stream) {
    if (a.io == IO_F32) return launch_by_n<float>(a, stream);
    return launch_by_n<uint16_t>(a, stream);
}

}  // namespace mssm
