// mssm_api.cpp -- the C ABI of libmssm (declared in include/mssm.h):
// argument validation, kernel-variant choice and launch on the caller's
// stream.  Validation runs before any HIP call, so every error path can be
// exercised without a GPU.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <string>

#include "internal.h"
#include "mssm.h"
#include "mssm_probes.h"

namespace {

thread_local std::string g_last_error;
thread_local mssm_variant g_forced = MSSM_VARIANT_AUTO;
thread_local mssm_variant g_last_variant = MSSM_VARIANT_AUTO;

mssm_status fail(mssm_status s, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

mssm_status hip_fail(hipError_t e, const char *what) {
    if (e == hipErrorOutOfMemory || e == hipErrorMemoryAllocation)
        return fail(MSSM_ERR_ALLOC, "%s: %s (%d)", what, hipGetErrorString(e), static_cast<int>(e));
    return fail(MSSM_ERR_HIP, "%s: %s (%d)", what, hipGetErrorString(e), static_cast<int>(e));
}

bool mul_ok(int64_t a, int64_t b, int64_t *out) {
    return !__builtin_mul_overflow(a, b, out);
}

// Byte range [p, p + n) of one operand, for the overlap check.
struct Range {
    const char *name;
    uintptr_t lo, hi;
};

Range range(const char *name, const void *p, int64_t bytes) {
    uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Range{name, lo, p ? lo + static_cast<uintptr_t>(bytes) : lo};
}

bool overlaps(const Range &a, const Range &b) {
    if (a.lo == a.hi || b.lo == b.hi) return false;
    return a.lo < b.hi && b.lo < a.hi;
}

// Fill n floats with zero.  A kernel rather than hipMemsetAsync so that the
// call stays safe to record into a HIP graph.
__global__ void zero_fill_kernel(float *p, int64_t n) {
    int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (; i < n; i += stride) p[i] = 0.0f;
}

hipError_t zero_fill(float *p, int64_t n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(zero_fill_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, s, p, n);
    return hipGetLastError();
}

mssm_status check_dtypes(mssm_dtypes dt) {
    if (dt.io != MSSM_F32 && dt.io != MSSM_BF16)
        return fail(MSSM_ERR_INVALID_ARG, "unknown io dtype %d", dt.io);
    if (dt.param != MSSM_F32 && dt.param != MSSM_BF16)
        return fail(MSSM_ERR_INVALID_ARG, "unknown param dtype %d", dt.param);
    if (dt.param != MSSM_F32)
        return fail(MSSM_ERR_UNSUPPORTED, "param dtype must be MSSM_F32");
    return MSSM_OK;
}

// Shape-based choice.  Short sequences take the row-serial walk (its single
// lane per row has nothing to amortise).  Long sequences whose channels give
// the chunked kernel waves for under four fifths of the 1024 SIMDs of the
// chip are cut into segments and take the look-back kernel; everything else
// takes the chunked kernel, which walks each row in order.  The look-back
// kernel walks every segment twice (state only, then with output), about
// 1.47 times the chunked kernel's vector instructions, but keeps three
// workgroups on every compute unit: measured on the Mamba-130M layer (768
// waves, three quarters of the SIMDs), 237 us against 244 us for the
// chunked kernel, which at one wave per SIMD keeps its SIMDs about 58 %
// busy against the look-back's 66 %.  Nearer a full chip of waves the
// second walk no longer pays.
mssm_variant choose_scan_variant(const mssm::ScanArgs &a) {
    if (a.L < 128 || !mssm::scan_chunked_supported(a)) return MSSM_VARIANT_ROWSERIAL;
    if (a.L >= 2048 && 5 * mssm::scan_chunked_waves(a) < 4 * 1024 && mssm::scan_lookback_supported(a))
        return MSSM_VARIANT_LOOKBACK;
    return MSSM_VARIANT_CHUNKED;
}

// Outputs may not overlap inputs, nor each other; the one exception is an
// initial-state input passed as the final-state output itself (the same
// buffer, exactly), which continues a sequence in place.
mssm_status check_overlaps(const Range *ins, int nin, const Range *outs, int nout,
                           const void *h0, const void *h_last) {
    const bool in_place = h0 && h0 == h_last;
    for (int o = 0; o < nout; ++o)
        for (int i = 0; i < nin; ++i) {
            if (in_place && std::strcmp(ins[i].name, "h0") == 0 &&
                std::strcmp(outs[o].name, "h_last") == 0)
                continue;
            if (overlaps(outs[o], ins[i]))
                return fail(MSSM_ERR_INVALID_ARG, "output %s overlaps input %s", outs[o].name,
                            ins[i].name);
        }
    for (int o = 0; o < nout; ++o)
        for (int p = o + 1; p < nout; ++p)
            if (overlaps(outs[o], outs[p]))
                return fail(MSSM_ERR_INVALID_ARG, "%s overlaps %s", outs[o].name, outs[p].name);
    return MSSM_OK;
}

mssm_status scan_fwd(const void *u, const void *delta, const float *delta_bias, const float *A,
                     const void *B, const void *C, const float *D, const void *z, const float *h0,
                     void *y, float *h_last, mssm_scan_dims dims, mssm_dtypes dtypes,
                     void *stream, const float *conv_w = nullptr, const float *conv_b = nullptr,
                     bool no_alloc = false) {
    g_last_error.clear();
    if (mssm_status s = check_dtypes(dtypes)) return s;
    const int64_t batch = dims.batch, L = dims.seqlen, dim = dims.dim, N = dims.dstate;
    if (batch < 0 || L < 0 || dim < 0)
        return fail(MSSM_ERR_INVALID_ARG, "negative size (batch %lld, L %lld, dim %lld)",
                    (long long)batch, (long long)L, (long long)dim);
    if (N < 1) return fail(MSSM_ERR_INVALID_ARG, "dstate must be >= 1, got %lld", (long long)N);
    if (N > MSSM_MAX_DSTATE)
        return fail(MSSM_ERR_UNSUPPORTED, "dstate %lld exceeds MSSM_MAX_DSTATE (%d)",
                    (long long)N, MSSM_MAX_DSTATE);
    const int64_t esz = dtypes.io == MSSM_F32 ? 4 : 2;
    int64_t rows, act, act_bytes, bc, bc_bytes, dn, hl;
    if (!mul_ok(batch, dim, &rows) || !mul_ok(rows, L, &act) || !mul_ok(act, esz, &act_bytes) ||
        !mul_ok(batch, N, &bc) || !mul_ok(bc, L, &bc) || !mul_ok(bc, esz, &bc_bytes) ||
        !mul_ok(dim, N, &dn) || !mul_ok(rows, N, &hl) || !mul_ok(hl, 4, &hl))
        return fail(MSSM_ERR_INVALID_ARG, "sizes overflow int64");
    if (rows == 0) {
        g_last_variant = MSSM_VARIANT_AUTO;
        return MSSM_OK;
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (L == 0) {
        if (h_last && h0 != h_last) {
            if (h0) {
                if (overlaps(range("h_last", h_last, hl), range("h0", h0, hl)))
                    return fail(MSSM_ERR_INVALID_ARG, "output h_last overlaps input h0");
                hipError_t e = hipMemcpyAsync(h_last, h0, hl, hipMemcpyDeviceToDevice, st);
                if (e != hipSuccess) return hip_fail(e, "copy of h0 to h_last");
            } else {
                hipError_t e = zero_fill(h_last, rows * N, st);
                if (e != hipSuccess) return hip_fail(e, "zero-fill of h_last");
            }
        }
        g_last_variant = MSSM_VARIANT_AUTO;
        return MSSM_OK;
    }
    if (!u) return fail(MSSM_ERR_INVALID_ARG, "u is null");
    if (!delta) return fail(MSSM_ERR_INVALID_ARG, "delta is null");
    if (!A) return fail(MSSM_ERR_INVALID_ARG, "A is null");
    if (!B) return fail(MSSM_ERR_INVALID_ARG, "B is null");
    if (!C) return fail(MSSM_ERR_INVALID_ARG, "C is null");
    if (!y) return fail(MSSM_ERR_INVALID_ARG, "y is null");

    const Range ins[] = {
        range("u", u, act_bytes),          range("delta", delta, act_bytes),
        range("z", z, act_bytes),          range("B", B, bc_bytes),
        range("C", C, bc_bytes),           range("A", A, dn * 4),
        range("D", D, dim * 4),            range("delta_bias", delta_bias, dim * 4),
        range("h0", h0, hl),               range("conv_w", conv_w, dim * 4 * MSSM_CONV_WIDTH),
        range("conv_b", conv_b, dim * 4)};
    const Range outs[] = {range("y", y, act_bytes), range("h_last", h_last, hl)};
    if (mssm_status c = check_overlaps(ins, 11, outs, 2, h0, h_last)) return c;

    mssm::ScanArgs a{u, delta, delta_bias, A, B, C, D, z, h0, y, h_last, batch, L, dim, N,
                     dtypes.io == MSSM_F32 ? mssm::IO_F32 : mssm::IO_BF16, conv_w, conv_b};

    mssm_variant v = g_forced;
    if (v == MSSM_VARIANT_AUTO) v = choose_scan_variant(a);
    hipError_t e;
    switch (v) {
        case MSSM_VARIANT_ROWSERIAL:
            if (!mssm::scan_rowserial_supported(a))
                return fail(MSSM_ERR_UNSUPPORTED, "row-serial variant does not support this shape");
            e = mssm::launch_scan_rowserial(a, st);
            break;
        case MSSM_VARIANT_CHUNKED:
            if (!mssm::scan_chunked_supported(a))
                return fail(MSSM_ERR_UNSUPPORTED, "chunked variant does not support this shape");
            e = mssm::launch_scan_chunked(a, st);
            break;
        case MSSM_VARIANT_LOOKBACK:
            if (!mssm::scan_lookback_supported(a))
                return fail(MSSM_ERR_UNSUPPORTED, "look-back variant does not support this shape");
            if (no_alloc) {
                const size_t need = mssm::scan_lookback_scratch_bytes(a);
                if (need > mssm::kNoAllocScratchBytes)
                    return fail(MSSM_ERR_UNSUPPORTED,
                                "look-back scratch of %zu bytes exceeds the %zu bytes of the "
                                "no-alloc entry point", need, mssm::kNoAllocScratchBytes);
                e = mssm::launch_scan_lookback_noalloc(a, st);
            } else {
                e = mssm::launch_scan_lookback(a, st);
            }
            break;
        case MSSM_VARIANT_PAIRSCAN:
        case MSSM_VARIANT_PAIRSCAN2:
            if (!mssm::scan_pairscan_supported(a))
                return fail(MSSM_ERR_UNSUPPORTED, "pair-scan variant does not support this shape "
                            "(N <= 16, no convolution prologue)");
            e = mssm::launch_scan_pairscan(a, st, v == MSSM_VARIANT_PAIRSCAN2 ? 2 : 1);
            break;
        default:
            return fail(MSSM_ERR_UNSUPPORTED, "variant %d does not apply to the selective scan",
                        static_cast<int>(v));
    }
    if (e != hipSuccess) return hip_fail(e, "selective-scan launch");
    g_last_variant = v;
    return MSSM_OK;
}

mssm_status ssd_fwd(const void *x, const void *dt, const float *dt_bias, const float *A,
                    const void *B, const void *C, const float *D, const void *z, const float *h0,
                    void *y, float *h_last, mssm_ssd_dims dims, mssm_dtypes dtypes,
                    void *stream) {
    g_last_error.clear();
    if (mssm_status s = check_dtypes(dtypes)) return s;
    const int64_t batch = dims.batch, L = dims.seqlen, H = dims.nheads, P = dims.headdim,
                  N = dims.dstate, G = dims.ngroups, Q = dims.chunk;
    if (batch < 0 || L < 0 || H < 0)
        return fail(MSSM_ERR_INVALID_ARG, "negative size (batch %lld, L %lld, H %lld)",
                    (long long)batch, (long long)L, (long long)H);
    if (P < 1 || N < 1) return fail(MSSM_ERR_INVALID_ARG, "headdim and dstate must be >= 1");
    if (G < 1) return fail(MSSM_ERR_INVALID_ARG, "ngroups must be >= 1");
    if (H % G != 0)
        return fail(MSSM_ERR_INVALID_ARG, "nheads %lld is not a multiple of ngroups %lld",
                    (long long)H, (long long)G);
    if (Q < 0) return fail(MSSM_ERR_INVALID_ARG, "chunk must be >= 0");
    if (P > MSSM_SSD_MAX_HEADDIM || N > MSSM_SSD_MAX_DSTATE)
        return fail(MSSM_ERR_UNSUPPORTED, "headdim %lld / dstate %lld beyond limits (%d / %d)",
                    (long long)P, (long long)N, MSSM_SSD_MAX_HEADDIM, MSSM_SSD_MAX_DSTATE);
    const int64_t esz = dtypes.io == MSSM_F32 ? 4 : 2;
    int64_t bl, xs, x_bytes, dts, dt_bytes, bcs, bc_bytes, pairs, hl;
    if (!mul_ok(batch, L, &bl) || !mul_ok(bl, H, &dts) || !mul_ok(dts, P, &xs) ||
        !mul_ok(xs, esz, &x_bytes) || !mul_ok(dts, esz, &dt_bytes) ||
        !mul_ok(bl, G, &bcs) || !mul_ok(bcs, N, &bcs) || !mul_ok(bcs, esz, &bc_bytes) ||
        !mul_ok(batch, H, &pairs) || !mul_ok(pairs, P, &hl) || !mul_ok(hl, N, &hl) ||
        !mul_ok(hl, 4, &hl))
        return fail(MSSM_ERR_INVALID_ARG, "sizes overflow int64");
    if (pairs == 0) {
        g_last_variant = MSSM_VARIANT_AUTO;
        return MSSM_OK;
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (L == 0) {
        if (h_last && h0 != h_last) {
            if (h0) {
                if (overlaps(range("h_last", h_last, hl), range("h0", h0, hl)))
                    return fail(MSSM_ERR_INVALID_ARG, "output h_last overlaps input h0");
                hipError_t e = hipMemcpyAsync(h_last, h0, hl, hipMemcpyDeviceToDevice, st);
                if (e != hipSuccess) return hip_fail(e, "copy of h0 to h_last");
            } else {
                hipError_t e = zero_fill(h_last, hl / 4, st);
                if (e != hipSuccess) return hip_fail(e, "zero-fill of h_last");
            }
        }
        g_last_variant = MSSM_VARIANT_AUTO;
        return MSSM_OK;
    }
    if (!x) return fail(MSSM_ERR_INVALID_ARG, "x is null");
    if (!dt) return fail(MSSM_ERR_INVALID_ARG, "dt is null");
    if (!A) return fail(MSSM_ERR_INVALID_ARG, "A is null");
    if (!B) return fail(MSSM_ERR_INVALID_ARG, "B is null");
    if (!C) return fail(MSSM_ERR_INVALID_ARG, "C is null");
    if (!y) return fail(MSSM_ERR_INVALID_ARG, "y is null");
    const Range ins[] = {range("x", x, x_bytes),   range("dt", dt, dt_bytes),
                         range("B", B, bc_bytes),  range("C", C, bc_bytes),
                         range("A", A, H * 4),     range("D", D, H * 4),
                         range("dt_bias", dt_bias, H * 4), range("h0", h0, hl),
                         range("z", z, x_bytes)};
    const Range outs[] = {range("y", y, x_bytes), range("h_last", h_last, hl)};
    if (mssm_status c = check_overlaps(ins, 9, outs, 2, h0, h_last)) return c;

    mssm::SSDArgs a{x, dt, dt_bias, A, B, C, D, z, h0, y, h_last, batch, L, H, P, N, G,
                    Q == 0 ? 256 : Q, dtypes.io == MSSM_F32 ? mssm::IO_F32 : mssm::IO_BF16};
    // The matrix-core form needs bf16 operands and a few chunks to pay off;
    // everything else takes the recurrent form.
    mssm_variant v = g_forced;
    if (v == MSSM_VARIANT_AUTO)
        v = (mssm::ssd_chunked_supported(a) && a.L >= 2 * a.chunk) ? MSSM_VARIANT_SSD_CHUNKED
                                                                    : MSSM_VARIANT_SSD_RECURRENT;
    hipError_t e;
    switch (v) {
        case MSSM_VARIANT_SSD_RECURRENT:
            if (!mssm::ssd_recurrent_supported(a))
                return fail(MSSM_ERR_UNSUPPORTED, "recurrent SSD variant does not support this shape");
            e = mssm::launch_ssd_recurrent(a, st);
            break;
        case MSSM_VARIANT_SSD_CHUNKED:
            if (!mssm::ssd_chunked_supported(a))
                return fail(MSSM_ERR_UNSUPPORTED, "chunked SSD variant needs bf16 I/O, dstate <= 128 "
                            "and chunk 64, 128 or 256");
            e = mssm::launch_ssd_chunked(a, st);
            break;
        default:
            return fail(MSSM_ERR_UNSUPPORTED, "variant %d does not apply to the SSD scan",
                        static_cast<int>(v));
    }
    if (e != hipSuccess) return hip_fail(e, "SSD launch");
    g_last_variant = v;
    return MSSM_OK;
}

}  // namespace

namespace mssm {

namespace {
constexpr int kPoolDevices = 64;
std::mutex g_pool_mu;
hipMemPool_t g_pool[kPoolDevices] = {};
}  // namespace

// The current device's scratch pool, created on first use with an unlimited
// release threshold.
hipError_t scratch_alloc(void **ptr, size_t bytes, hipStream_t stream) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kPoolDevices) return hipErrorInvalidDevice;
    hipMemPool_t pool;
    {
        std::lock_guard<std::mutex> lk(g_pool_mu);
        if (!g_pool[dev]) {
            hipMemPoolProps props;
            std::memset(&props, 0, sizeof props);
            props.allocType = hipMemAllocationTypePinned;
            props.location.type = hipMemLocationTypeDevice;
            props.location.id = dev;
            hipMemPool_t p = nullptr;
            e = hipMemPoolCreate(&p, &props);
            if (e != hipSuccess) return e;
            uint64_t keep = UINT64_MAX;
            e = hipMemPoolSetAttribute(p, hipMemPoolAttrReleaseThreshold, &keep);
            if (e != hipSuccess) {
                (void)hipMemPoolDestroy(p);
                return e;
            }
            g_pool[dev] = p;
        }
        pool = g_pool[dev];
    }
    return hipMallocFromPoolAsync(ptr, bytes, pool, stream);
}

hipError_t scratch_free(void *ptr, hipStream_t stream) { return hipFreeAsync(ptr, stream); }

}  // namespace mssm

extern "C" {

mssm_status mssm_selective_scan_fwd(const void *u, const void *delta,
                                    const float *delta_bias, const float *A,
                                    const void *B, const void *C,
                                    const float *D, const void *z, void *y,
                                    float *h_last, mssm_scan_dims dims,
                                    mssm_dtypes dtypes, void *stream) {
    return scan_fwd(u, delta, delta_bias, A, B, C, D, z, nullptr, y, h_last, dims, dtypes,
                    stream);
}

mssm_status mssm_selective_scan_fwd_h0(const void *u, const void *delta,
                                       const float *delta_bias, const float *A,
                                       const void *B, const void *C, const float *D,
                                       const void *z, const float *h0, void *y,
                                       float *h_last, mssm_scan_dims dims,
                                       mssm_dtypes dtypes, void *stream) {
    return scan_fwd(u, delta, delta_bias, A, B, C, D, z, h0, y, h_last, dims, dtypes, stream);
}

mssm_status mssm_selective_scan_fwd_h0_noalloc(const void *u, const void *delta,
                                               const float *delta_bias, const float *A,
                                               const void *B, const void *C, const float *D,
                                               const void *z, const float *h0, void *y,
                                               float *h_last, mssm_scan_dims dims,
                                               mssm_dtypes dtypes, void *stream) {
    return scan_fwd(u, delta, delta_bias, A, B, C, D, z, h0, y, h_last, dims, dtypes, stream,
                    nullptr, nullptr, true);
}

mssm_status mssm_selective_scan_fwd_conv(const void *x, const float *conv_w,
                                         const float *conv_b, const void *delta,
                                         const float *delta_bias, const float *A, const void *B,
                                         const void *C, const float *D, const void *z,
                                         const float *h0, void *y, float *h_last,
                                         mssm_scan_dims dims, mssm_dtypes dtypes, void *stream) {
    if (!conv_w) {
        g_last_error.clear();
        return fail(MSSM_ERR_INVALID_ARG, "conv_w is null");
    }
    return scan_fwd(x, delta, delta_bias, A, B, C, D, z, h0, y, h_last, dims, dtypes, stream,
                    conv_w, conv_b);
}

mssm_status mssm_selective_scan_bwd(const void *u, const void *delta, const float *delta_bias,
                                    const float *A, const void *B, const void *C, const float *D,
                                    const void *z, const float *h0, const void *dy,
                                    const float *dh_last, float *du, float *ddelta,
                                    float *ddelta_bias, float *dA, float *dB, float *dC, float *dD,
                                    float *dz, float *dh0, mssm_scan_dims dims, mssm_dtypes dtypes,
                                    void *stream) {
    g_last_error.clear();
    if (mssm_status s = check_dtypes(dtypes)) return s;
    const int64_t batch = dims.batch, L = dims.seqlen, dim = dims.dim, N = dims.dstate;
    if (batch < 0 || L < 0 || dim < 0)
        return fail(MSSM_ERR_INVALID_ARG, "negative size (batch %lld, L %lld, dim %lld)",
                    (long long)batch, (long long)L, (long long)dim);
    if (N < 1) return fail(MSSM_ERR_INVALID_ARG, "dstate must be >= 1, got %lld", (long long)N);
    if (N > MSSM_MAX_DSTATE)
        return fail(MSSM_ERR_UNSUPPORTED, "dstate %lld exceeds MSSM_MAX_DSTATE (%d)",
                    (long long)N, MSSM_MAX_DSTATE);
    if (dz && !z) return fail(MSSM_ERR_INVALID_ARG, "dz given without z");
    const int64_t esz = dtypes.io == MSSM_F32 ? 4 : 2;
    int64_t rows, act, act_bytes, act4, bc, bc_bytes, bc4, dn, hl;
    if (!mul_ok(batch, dim, &rows) || !mul_ok(rows, L, &act) || !mul_ok(act, esz, &act_bytes) ||
        !mul_ok(act, 4, &act4) || !mul_ok(batch, N, &bc) || !mul_ok(bc, L, &bc) ||
        !mul_ok(bc, esz, &bc_bytes) || !mul_ok(bc, 4, &bc4) || !mul_ok(dim, N, &dn) ||
        !mul_ok(rows, N, &hl) || !mul_ok(hl, 4, &hl))
        return fail(MSSM_ERR_INVALID_ARG, "sizes overflow int64");
    hipStream_t st = static_cast<hipStream_t>(stream);
    // the accumulated gradients start from zero, whatever else happens
    auto zero_sums = [&]() -> hipError_t {
        hipError_t e = hipSuccess;
        if (e == hipSuccess && dB) e = zero_fill(dB, bc, st);
        if (e == hipSuccess && dC) e = zero_fill(dC, bc, st);
        if (e == hipSuccess && dA) e = zero_fill(dA, dn, st);
        if (e == hipSuccess && dD) e = zero_fill(dD, dim, st);
        if (e == hipSuccess && ddelta_bias) e = zero_fill(ddelta_bias, dim, st);
        return e;
    };
    if (rows == 0 || L == 0) {
        const Range outs0[] = {range("dB", dB, bc4), range("dC", dC, bc4), range("dA", dA, dn * 4),
                               range("dD", dD, dim * 4), range("ddelta_bias", ddelta_bias, dim * 4),
                               range("dh0", dh0, hl)};
        for (int i = 0; i < 6; ++i)
            for (int j = i + 1; j < 6; ++j)
                if (overlaps(outs0[i], outs0[j]))
                    return fail(MSSM_ERR_INVALID_ARG, "%s overlaps %s", outs0[i].name, outs0[j].name);
        hipError_t e = zero_sums();
        // with L == 0 the initial state is the final state: dh0 = dh_last
        if (e == hipSuccess && dh0 && rows > 0) {
            e = dh_last ? hipMemcpyAsync(dh0, dh_last, hl, hipMemcpyDeviceToDevice, st)
                        : zero_fill(dh0, rows * N, st);
        }
        if (e != hipSuccess) return hip_fail(e, "zero-fill of the gradients");
        g_last_variant = MSSM_VARIANT_AUTO;
        return MSSM_OK;
    }
    if (!u) return fail(MSSM_ERR_INVALID_ARG, "u is null");
    if (!delta) return fail(MSSM_ERR_INVALID_ARG, "delta is null");
    if (!A) return fail(MSSM_ERR_INVALID_ARG, "A is null");
    if (!B) return fail(MSSM_ERR_INVALID_ARG, "B is null");
    if (!C) return fail(MSSM_ERR_INVALID_ARG, "C is null");
    if (!dy) return fail(MSSM_ERR_INVALID_ARG, "dy is null");
    if (!du) return fail(MSSM_ERR_INVALID_ARG, "du is null");
    if (!ddelta) return fail(MSSM_ERR_INVALID_ARG, "ddelta is null");
    const Range ins[] = {
        range("u", u, act_bytes),          range("delta", delta, act_bytes),
        range("z", z, act_bytes),          range("B", B, bc_bytes),
        range("C", C, bc_bytes),           range("A", A, dn * 4),
        range("D", D, dim * 4),            range("delta_bias", delta_bias, dim * 4),
        range("h0", h0, hl),               range("dy", dy, act_bytes),
        range("dh_last", dh_last, hl)};
    const Range outs[] = {
        range("du", du, act4),             range("ddelta", ddelta, act4),
        range("dz", dz, act4),             range("dB", dB, bc4),
        range("dC", dC, bc4),              range("dA", dA, dn * 4),
        range("dD", dD, dim * 4),          range("ddelta_bias", ddelta_bias, dim * 4),
        range("dh0", dh0, hl)};
    if (mssm_status c = check_overlaps(ins, 11, outs, 9, nullptr, nullptr)) return c;

    mssm::BwdArgs a{u, delta, delta_bias, A, B, C, D, z, h0, dy, dh_last, du, ddelta, ddelta_bias,
                    dA, dB, dC, dD, dz, dh0, batch, L, dim, N,
                    dtypes.io == MSSM_F32 ? mssm::IO_F32 : mssm::IO_BF16};
    // AUTO: the chunked backward where it applies (N <= 16), else the
    // row-serial one; either can be forced
    mssm_variant v = g_forced;
    if (v == MSSM_VARIANT_AUTO)
        v = mssm::scan_bwd_chunked_supported(a) ? MSSM_VARIANT_CHUNKED : MSSM_VARIANT_ROWSERIAL;
    if (v == MSSM_VARIANT_CHUNKED) {
        if (!mssm::scan_bwd_chunked_supported(a))
            return fail(MSSM_ERR_UNSUPPORTED, "chunked backward needs N <= 16");
    } else if (v == MSSM_VARIANT_ROWSERIAL) {
        if (!mssm::scan_bwd_supported(a))
            return fail(MSSM_ERR_UNSUPPORTED, "backward does not support this shape");
    } else {
        return fail(MSSM_ERR_UNSUPPORTED, "variant %d does not apply to the backward",
                    static_cast<int>(v));
    }
    hipError_t e = zero_sums();
    if (e == hipSuccess)
        e = v == MSSM_VARIANT_CHUNKED ? mssm::launch_scan_bwd_chunked(a, st) : mssm::launch_scan_bwd(a, st);
    if (e != hipSuccess) return hip_fail(e, "selective-scan backward launch");
    g_last_variant = v;
    return MSSM_OK;
}

mssm_status mssm_ssd_scalar_fwd(const void *x, const void *dt, const float *dt_bias,
                                const float *A, const void *B, const void *C,
                                const float *D, void *y, float *h_last,
                                mssm_ssd_dims dims, mssm_dtypes dtypes, void *stream) {
    return ssd_fwd(x, dt, dt_bias, A, B, C, D, nullptr, nullptr, y, h_last, dims, dtypes, stream);
}

mssm_status mssm_ssd_scalar_fwd_h0(const void *x, const void *dt, const float *dt_bias,
                                   const float *A, const void *B, const void *C,
                                   const float *D, const float *h0, void *y, float *h_last,
                                   mssm_ssd_dims dims, mssm_dtypes dtypes, void *stream) {
    return ssd_fwd(x, dt, dt_bias, A, B, C, D, nullptr, h0, y, h_last, dims, dtypes, stream);
}

mssm_status mssm_ssd_scalar_fwd_gated(const void *x, const void *dt, const float *dt_bias,
                                      const float *A, const void *B, const void *C,
                                      const float *D, const void *z, const float *h0, void *y,
                                      float *h_last, mssm_ssd_dims dims, mssm_dtypes dtypes,
                                      void *stream) {
    return ssd_fwd(x, dt, dt_bias, A, B, C, D, z, h0, y, h_last, dims, dtypes, stream);
}

mssm_status mssm_selective_state_update(float *state, const void *x, const void *dt,
                                        const float *dt_bias, const float *A, const void *B,
                                        const void *C, const float *D, const void *z, void *y,
                                        mssm_step_dims dims, mssm_dtypes dtypes, void *stream) {
    g_last_error.clear();
    if (mssm_status s = check_dtypes(dtypes)) return s;
    const int64_t batch = dims.batch, dim = dims.dim, N = dims.dstate;
    if (batch < 0 || dim < 0)
        return fail(MSSM_ERR_INVALID_ARG, "negative size (batch %lld, dim %lld)", (long long)batch,
                    (long long)dim);
    if (N < 1) return fail(MSSM_ERR_INVALID_ARG, "dstate must be >= 1, got %lld", (long long)N);
    if (N > MSSM_MAX_DSTATE)
        return fail(MSSM_ERR_UNSUPPORTED, "dstate %lld exceeds MSSM_MAX_DSTATE (%d)",
                    (long long)N, MSSM_MAX_DSTATE);
    const int64_t esz = dtypes.io == MSSM_F32 ? 4 : 2;
    int64_t rows, row_bytes, st_bytes, bc_bytes, dn;
    if (!mul_ok(batch, dim, &rows) || !mul_ok(rows, esz, &row_bytes) ||
        !mul_ok(rows, N, &st_bytes) || !mul_ok(st_bytes, 4, &st_bytes) ||
        !mul_ok(batch, N, &bc_bytes) || !mul_ok(bc_bytes, esz, &bc_bytes) ||
        !mul_ok(dim, N, &dn))
        return fail(MSSM_ERR_INVALID_ARG, "sizes overflow int64");
    if (rows == 0) {
        g_last_variant = MSSM_VARIANT_AUTO;
        return MSSM_OK;
    }
    if (!state) return fail(MSSM_ERR_INVALID_ARG, "state is null");
    if (!x) return fail(MSSM_ERR_INVALID_ARG, "x is null");
    if (!dt) return fail(MSSM_ERR_INVALID_ARG, "dt is null");
    if (!A) return fail(MSSM_ERR_INVALID_ARG, "A is null");
    if (!B) return fail(MSSM_ERR_INVALID_ARG, "B is null");
    if (!C) return fail(MSSM_ERR_INVALID_ARG, "C is null");
    if (!y) return fail(MSSM_ERR_INVALID_ARG, "y is null");
    const Range ins[] = {range("x", x, row_bytes),   range("dt", dt, row_bytes),
                         range("z", z, row_bytes),   range("B", B, bc_bytes),
                         range("C", C, bc_bytes),    range("A", A, dn * 4),
                         range("D", D, dim * 4),     range("dt_bias", dt_bias, dim * 4)};
    const Range outs[] = {range("y", y, row_bytes), range("state", state, st_bytes)};
    if (mssm_status c = check_overlaps(ins, 8, outs, 2, nullptr, nullptr)) return c;

    mssm::StepArgs a{state, x, dt, dt_bias, A, B, C, D, z, y, batch, dim, N,
                     dtypes.io == MSSM_F32 ? mssm::IO_F32 : mssm::IO_BF16};
    if (!mssm::state_update_supported(a))
        return fail(MSSM_ERR_UNSUPPORTED, "state update does not support this shape");
    const hipError_t e = mssm::launch_state_update(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "state-update launch");
    g_last_variant = MSSM_VARIANT_AUTO;
    return MSSM_OK;
}

mssm_variant mssm_force_variant(mssm_variant v) {
    mssm_variant prev = g_forced;
    g_forced = v;
    return prev;
}

mssm_variant mssm_last_variant(void) { return g_last_variant; }

const char *mssm_status_string(mssm_status s) {
    switch (s) {
        case MSSM_OK: return "MSSM_OK";
        case MSSM_ERR_INVALID_ARG: return "MSSM_ERR_INVALID_ARG";
        case MSSM_ERR_UNSUPPORTED: return "MSSM_ERR_UNSUPPORTED";
        case MSSM_ERR_HIP: return "MSSM_ERR_HIP";
        case MSSM_ERR_ALLOC: return "MSSM_ERR_ALLOC";
    }
    return "MSSM_ERR_UNKNOWN";
}

const char *mssm_last_error(void) { return g_last_error.c_str(); }

int mssm_version(void) { return 100; }

mssm_status mssm_device_status(uint32_t *bits, int clear) {
    g_last_error.clear();
    if (!bits) return fail(MSSM_ERR_INVALID_ARG, "bits is null");
    const hipError_t e = mssm::device_status(bits, clear != 0);
    if (e != hipSuccess) return hip_fail(e, "device status read");
    return MSSM_OK;
}

mssm_status mssm_probe_copy(const void *src, void *dst, int64_t bytes, void *stream) {
    g_last_error.clear();
    if (!src || !dst) return fail(MSSM_ERR_INVALID_ARG, "src and dst must not be null");
    if (bytes <= 0 || bytes % 16 != 0 || bytes >= (int64_t(1) << 43))
        return fail(MSSM_ERR_INVALID_ARG,
                    "bytes must be a positive multiple of 16 below 2^43, got %lld", (long long)bytes);
    if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15u)
        return fail(MSSM_ERR_INVALID_ARG, "src and dst must be 16-byte aligned");
    if (overlaps(range("src", src, bytes), range("dst", dst, bytes)))
        return fail(MSSM_ERR_INVALID_ARG, "src and dst overlap");
    const hipError_t e = mssm::launch_probe_copy(src, dst, bytes, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "copy probe launch");
    return MSSM_OK;
}

mssm_status mssm_probe_valu(int op, int32_t iters, float *out, void *stream) {
    g_last_error.clear();
    if (op < MSSM_PROBE_FMA || op > MSSM_PROBE_RCP)
        return fail(MSSM_ERR_INVALID_ARG, "unknown probe operation %d", op);
    if (iters < 1) return fail(MSSM_ERR_INVALID_ARG, "iters must be >= 1");
    if (!out) return fail(MSSM_ERR_INVALID_ARG, "out is null");
    const hipError_t e = mssm::launch_probe_valu(op, iters, out, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "ALU probe launch");
    return MSSM_OK;
}

#ifndef MSSM_SOURCE_HASH
#define MSSM_SOURCE_HASH "unknown"
#endif
const char *mssm_source_hash(void) { return MSSM_SOURCE_HASH; }

}  // extern "C"
