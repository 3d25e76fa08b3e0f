// device_math.h -- small device helpers shared by the HIP kernels: storage
// conversions and the scalar nonlinearities of the selective scan.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mssm {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---- storage conversions --------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint16_t v) {
    return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

// float32 -> bfloat16, round to nearest, ties to even; NaN stays NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t bits = __float_as_uint(f);
    if ((bits & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((bits >> 16) | 0x40u);
    bits += 0x7fffu + ((bits >> 16) & 1u);
    return static_cast<uint16_t>(bits >> 16);
}

template <typename T> struct Io;
template <> struct Io<float> {
    __device__ __forceinline__ static float load(const float *p, int64_t i) { return p[i]; }
    __device__ __forceinline__ static void store(float *p, int64_t i, float v) { p[i] = v; }
};
template <> struct Io<uint16_t> {
    __device__ __forceinline__ static float load(const uint16_t *p, int64_t i) { return bf16_to_f32(p[i]); }
    __device__ __forceinline__ static void store(uint16_t *p, int64_t i, float v) { p[i] = f32_to_bf16(v); }
};

// ---- nonlinearities -------------------------------------------------------
// 2^x on the hardware exponential unit (v_exp_f32).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
// log2(x) on the hardware unit (v_log_f32).
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// log(1 + w) for w in [0, 1], accurate to about 1 ulp for every w including
// w < 2^-24, where 1 + w rounds to 1.  With s = fl(1 + w), the rounding
// error c = w - (s - 1) is exact (both subtractions are exact by Sterbenz's
// lemma), 1 + w = s + c, and log(1 + w) = log(s) + c/s + O(c^2); replacing
// c/s by c costs at most |c| (s - 1) <= 2^-24 w.  v_log_f32 is accurate to
// ~1 ulp on (1, 2].
__device__ __forceinline__ float log1p_unit(float w) {
    const float s = 1.0f + w;
    const float c = w - (s - 1.0f);
    return fmaf(fast_log2(s), kLn2, c);
}

// softplus(x) = log(1 + e^x) = max(x, 0) + log(1 + e^{-|x|}), through the
// device math library (correctly rounded to ~1 ulp; used where clarity
// matters more than speed).
__device__ __forceinline__ float softplus_libm(float x) {
    return fmaxf(x, 0.0f) + log1pf(expf(-fabsf(x)));
}

// silu through the device math library.
__device__ __forceinline__ float silu_libm(float z) { return z / (1.0f + expf(-z)); }

// softplus on the hardware exponential/logarithm units.
__device__ __forceinline__ float softplus(float x) {
    const float w = fast_exp2(-fabsf(x) * kLog2e);
    return fmaxf(x, 0.0f) + log1p_unit(w);
}

// silu(z) = z * sigmoid(z) = z / (1 + e^{-z}).
__device__ __forceinline__ float silu(float z) {
    float e = fast_exp2(-z * kLog2e);
    return z * __builtin_amdgcn_rcpf(1.0f + e);
}

}  // namespace mssm
