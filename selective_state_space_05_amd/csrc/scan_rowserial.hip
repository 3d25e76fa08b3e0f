// scan_rowserial.hip -- the plainest GPU form of the selective-scan forward:
// one lane owns one (batch, channel) row and walks the whole sequence
// serially, its N-element state in registers.
//
// Per step ("Mamba状态空间模型的硬件感知推理优化" (ybb.press) sections 1 and
// 3.1; www.mhpq.cn/news/984979 essay sections 2.2 and 3.1):
//   dl   = softplus(delta + delta_bias)
//   h[n] = exp(dl * A[n]) * h[n] + dl * u * B[n]
//   y    = (sum_n C[n] * h[n] + D * u) * silu(z)
//
// This variant has no cross-lane traffic at all, so it is the first parity
// kernel and the choice for short sequences, where the per-chunk work of the
// parallel variants does not pay for itself (the ybb.press page, section 6.2,
// makes the same observation for sequences under ~128 steps).
#include "device_math.h"
#include "internal.h"

namespace mssm {
namespace {

template <typename T, int NS>
__global__ __launch_bounds__(256) void scan_rowserial_kernel(
    const T *__restrict__ u, const T *__restrict__ delta,
    const float *__restrict__ delta_bias, const float *__restrict__ A,
    const T *__restrict__ B, const T *__restrict__ C,
    const float *__restrict__ Dskip, const T *__restrict__ z, const float *h0, T *__restrict__ y,
    float *h_last, int64_t batch, int64_t L, int64_t dim, int N, const float *__restrict__ conv_w,
    const float *__restrict__ conv_b) {
    const int64_t row = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (row >= batch * dim) return;
    const int64_t b = row / dim;
    const int64_t d = row - b * dim;

    float A2[NS], h[NS];
#pragma unroll
    for (int n = 0; n < NS; ++n) {
        A2[n] = n < N ? A[d * N + n] * kLog2e : 0.0f;   // exp(x) = 2^(x log2 e)
        h[n] = (h0 && n < N) ? h0[row * N + n] : 0.0f;
    }
    const float bias = delta_bias ? delta_bias[d] : 0.0f;
    const float skip = Dskip ? Dskip[d] : 0.0f;
    // convolution prologue: taps, bias and the three previous inputs
    float cw[4] = {0.0f, 0.0f, 0.0f, 0.0f}, cb = 0.0f, xp[3] = {0.0f, 0.0f, 0.0f};
    if (conv_w) {
#pragma unroll
        for (int k = 0; k < 4; ++k) cw[k] = conv_w[d * 4 + k];
        cb = conv_b ? conv_b[d] : 0.0f;
    }
    const int64_t rbase = row * L;
    const int64_t bbase = b * N * L;

    for (int64_t t = 0; t < L; ++t) {
        const float dl = softplus_libm(Io<T>::load(delta, rbase + t) + bias);
        float ut = Io<T>::load(u, rbase + t);
        if (conv_w) {
            // u_t = silu(cb + w0 x_{t-3} + w1 x_{t-2} + w2 x_{t-1} + w3 x_t)
            const float xt = ut;
            ut = silu_libm(fmaf(cw[3], xt, fmaf(cw[2], xp[2], fmaf(cw[1], xp[1], fmaf(cw[0], xp[0], cb)))));
            xp[0] = xp[1];
            xp[1] = xp[2];
            xp[2] = xt;
        }
        const float du = dl * ut;
        float acc = 0.0f;
#pragma unroll
        for (int n = 0; n < NS; ++n) {
            if (n < N) {
                const float a = fast_exp2(dl * A2[n]);
                const float bn = Io<T>::load(B, bbase + n * L + t);
                const float cn = Io<T>::load(C, bbase + n * L + t);
                h[n] = fmaf(a, h[n], du * bn);
                acc = fmaf(cn, h[n], acc);
            }
        }
        float yv = fmaf(skip, ut, acc);
        if (z) yv *= silu_libm(Io<T>::load(z, rbase + t));
        Io<T>::store(y, rbase + t, yv);
    }
    if (h_last) {
#pragma unroll
        for (int n = 0; n < NS; ++n)
            if (n < N) h_last[row * N + n] = h[n];
    }
}

template <typename T, int NS>
hipError_t launch_typed(const ScanArgs &a, hipStream_t stream) {
    const int64_t rows = a.batch * a.dim;
    const int block = 256;
    const int64_t grid = (rows + block - 1) / block;
    hipLaunchKernelGGL((scan_rowserial_kernel<T, NS>), dim3(static_cast<uint32_t>(grid)),
                       dim3(block), 0, stream, static_cast<const T *>(a.u),
                       static_cast<const T *>(a.delta), a.delta_bias, a.A,
                       static_cast<const T *>(a.B), static_cast<const T *>(a.C), a.D,
                       static_cast<const T *>(a.z), a.h0, static_cast<T *>(a.y), a.h_last,
                       a.batch, a.L, a.dim, static_cast<int>(a.N), a.conv_w, a.conv_b);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_by_n(const ScanArgs &a, hipStream_t stream) {
    if (a.N <= 4) return launch_typed<T, 4>(a, stream);
    if (a.N <= 8) return launch_typed<T, 8>(a, stream);
    if (a.N <= 16) return launch_typed<T, 16>(a, stream);
    if (a.N <= 32) return launch_typed<T, 32>(a, stream);
    return launch_typed<T, 64>(a, stream);
}

}  // namespace

bool scan_rowserial_supported(const ScanArgs &a) {
    return a.N >= 1 && a.N <= 64 && a.batch * a.dim <= (int64_t(1) << 31) * 256;
}

hipError_t launch_scan_rowserial(const ScanArgs &a, hipStream_t stream) {
    if (a.io == IO_F32) return launch_by_n<float>(a, stream);
    return launch_by_n<uint16_t>(a, stream);
}

}  // namespace mssm
