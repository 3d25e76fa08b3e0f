// peak_probes.hip -- measurement kernels behind include/mssm_probes.h: the
// ceilings the roofline of the scan kernels is read against, measured on
// the device the kernels run on rather than taken from a data sheet
// ("Mamba状态空间模型的硬件感知推理优化" (ybb.press) section 1.1 reads the
// scan against the memory-bandwidth roof; on this chip the vector-ALU roof
// matters as well).
//
//   probe_copy_kernel   a plain copy, one 16-byte load and store per
//                       thread: the HBM rate a simple kernel reaches
//                       (read + write bytes / time).
//   probe_valu_kernel   eight independent dependency chains per lane of one
//                       vector ALU operation (fused multiply-add, 2^x,
//                       log2 x or 1/x), on enough waves to fill every SIMD:
//                       the issue rate of that operation, in lane-operations
//                       per second.  The ratio of the multiply-add rate to a
//                       transcendental's rate is what the transcendental
//                       costs in multiply-add issue slots.
#include <hip/hip_runtime.h>

#include "internal.h"
#include "mssm_probes.h"

namespace mssm {
namespace {

constexpr int kCopyThreads = 256;

// One 16-byte element per thread over a grid that covers the buffer.  On
// MI355X this flat form copies 1 GiB at about 6.2 TB/s (read + write),
// against 4.3-5.2 TB/s for grid-stride loops of 2048-16384 workgroups with
// four or eight elements in flight per thread.
__global__ __launch_bounds__(kCopyThreads) void probe_copy_kernel(const uint4 *__restrict__ src,
                                                                    uint4 *__restrict__ dst,
                                                                    int64_t n16) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * kCopyThreads + threadIdx.x;
    if (i < n16) dst[i] = src[i];
}

template <int OP>
__device__ __forceinline__ float valu_op(float x, float a, float b) {
    if constexpr (OP == MSSM_PROBE_FMA) return fmaf(x, a, b);
    else if constexpr (OP == MSSM_PROBE_EXP2) return __builtin_amdgcn_exp2f(x);
    else if constexpr (OP == MSSM_PROBE_LOG2) return __builtin_amdgcn_logf(x);
    else return __builtin_amdgcn_rcpf(x);
}

template <int OP>
__global__ __launch_bounds__(MSSM_PROBE_VALU_BLOCK) void probe_valu_kernel(float a, float b,
                                                                           int iters, float *out) {
    const int gid = blockIdx.x * MSSM_PROBE_VALU_BLOCK + threadIdx.x;
    float x[MSSM_PROBE_VALU_CHAINS];
#pragma unroll
    for (int k = 0; k < MSSM_PROBE_VALU_CHAINS; ++k) x[k] = b + 1e-3f * static_cast<float>(threadIdx.x + k);
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int r = 0; r < MSSM_PROBE_VALU_OPS_PER_ITER / MSSM_PROBE_VALU_CHAINS; ++r) {
#pragma unroll
            for (int k = 0; k < MSSM_PROBE_VALU_CHAINS; ++k) x[k] = valu_op<OP>(x[k], a, b);
        }
    }
    float s = 0.0f;
#pragma unroll
    for (int k = 0; k < MSSM_PROBE_VALU_CHAINS; ++k) s += x[k];
    out[gid] = s;
}

}  // namespace

hipError_t launch_probe_copy(const void *src, void *dst, int64_t bytes, hipStream_t stream) {
    const int64_t n16 = bytes / 16;
    const int64_t blocks = (n16 + kCopyThreads - 1) / kCopyThreads;
    if (blocks < 1) return hipSuccess;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(probe_copy_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(kCopyThreads), 0,
                       stream, static_cast<const uint4 *>(src), static_cast<uint4 *>(dst), n16);
    return hipGetLastError();
}

hipError_t launch_probe_valu(int op, int iters, float *out, hipStream_t stream) {
    decltype(&probe_valu_kernel<MSSM_PROBE_FMA>) k;
    switch (op) {
        case MSSM_PROBE_FMA: k = probe_valu_kernel<MSSM_PROBE_FMA>; break;
        case MSSM_PROBE_EXP2: k = probe_valu_kernel<MSSM_PROBE_EXP2>; break;
        case MSSM_PROBE_LOG2: k = probe_valu_kernel<MSSM_PROBE_LOG2>; break;
        case MSSM_PROBE_RCP: k = probe_valu_kernel<MSSM_PROBE_RCP>; break;
        default: return hipErrorInvalidValue;
    }
    hipLaunchKernelGGL(k, dim3(MSSM_PROBE_VALU_THREADS / MSSM_PROBE_VALU_BLOCK),
                       dim3(MSSM_PROBE_VALU_BLOCK), 0, stream, 0.999f, 1e-7f, iters, out);
    return hipGetLastError();
}

}  // namespace mssm
