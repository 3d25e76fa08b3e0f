// scan_bwd_rowserial.hip -- backward of the selective scan, walking each
// (batch, channel) row in reverse as the row-serial forward walks it forward.
// For N <= 16 a group of 8 (or, for N <= 8, 4) lanes owns a row, each lane a
// slice of its state elements (the lane-group kernel below); for larger N one
// lane owns a row with all its state elements.
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
// dB and dC sum over channels.  At every step a wave sums its rows'
// contributions (2 x 16 values per group of 16 state elements) with a
// transposed reduction -- cross-row swaps in registers, then a wave-private
// LDS pass or a row rotation -- and stores the 32 sums with one store
// into a per-wave partial buffer; a second kernel adds the partials of the
// waves of each batch in a fixed order and writes dB and dC, so they are
// deterministic.  (Atomic additions from every wave to the same (n, t) at the
// same time serialised in the caches.)  A wave whose rows span several
// batches reduces each batch's rows into a partial slot of its own.  dA, dD
// and the bias gradient are added atomically once per lane at the end, so
// their last bits depend on the order.
#include <algorithm>

#include "device_math.h"
#include "internal.h"

namespace mssm {
namespace {

// Segment length: the K states of a segment stay in registers (K * NS floats).
template <int NS>
constexpr int seg_steps() { return NS <= 4 ? 32 : NS <= 8 ? 16 : NS <= 16 ? 8 : NS <= 32 ? 4 : 2; }

constexpr int kRedPitch = 36;   // LDS row pitch (floats) of the wave's reduction pass

// Sum over the wave's 64 lanes of v[k], k < 32; lane l returns the sum for
// k = l % 32.  v_permlane32_swap pairs lanes l and l + 32 for k and k + 16,
// v_permlane16_swap rows (0, 1) and (2, 3) for k and k + 8, so that lane (row
// r, column c) holds the four-row sums of k = 8 r + i, i < 8, for its column;
// those go through LDS (row c of `red`), and each lane adds the 16 columns of
// its k.  The same wave writes and reads `red`, in order, so no barrier.
__device__ __forceinline__ float reduce32(const float (&v)[32], float *red) {
    float w[16], x[8];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[k]), __float_as_uint(v[k + 16]),
                                                        false, false);
        w[k] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(w[k]), __float_as_uint(w[k + 8]),
                                                        false, false);
        x[k] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    const int lane = threadIdx.x & 63;
    float4 *dst = reinterpret_cast<float4 *>(red + (lane & 15) * kRedPitch + 8 * (lane >> 4));
    dst[0] = make_float4(x[0], x[1], x[2], x[3]);
    dst[1] = make_float4(x[4], x[5], x[6], x[7]);
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < 16; ++c) s += red[c * kRedPitch + (lane & 31)];
    return s;
}

// Groups of 16 state elements the partial sums are formed in.
template <int NS>
constexpr int n_groups() { return (NS + 15) / 16; }

template <typename T, int NS>
__global__ __launch_bounds__(64) void scan_bwd_rowserial_kernel(BwdArgs a, float *__restrict__ ck,
                                                                int nseg, float *__restrict__ part,
                                                                int nslots) {
    constexpr int K = seg_steps<NS>();
    constexpr int NG = n_groups<NS>();
    __shared__ float red[16 * kRedPitch];
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
    // batches this wave's rows span (wave-uniform): slot s holds the sums over
    // its rows of batch b_first + s
    const int nspan = static_cast<int>(r_last / a.dim - r_first / a.dim) + 1;
    const int64_t b_first = r_first / a.dim;
    const bool want_bc = a.dB || a.dC;
    // this wave's partial sums: [slot][t][NG][32]
    float *pw = part + static_cast<int64_t>(blockIdx.x) * nslots * L * (NG * 32);

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
                const float dl = softplus(Io<T>::load(delta, rb + t) + bias);
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
                const float dl = softplus(Io<T>::load(delta, rb + t) + bias);
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
            const float dl = softplus(x);
            const float sig = __builtin_amdgcn_rcpf(1.0f + fast_exp2(-x * kLog2e));
            const float ut = Io<T>::load(u, rb + t);
            const float dyt = valid ? Io<T>::load(dy, rb + t) : 0.0f;
            float ds = dyt;
            if (z) {
                const float zt = Io<T>::load(z, rb + t);
                float sv = skip * ut;
#pragma unroll
                for (int n = 0; n < NS; ++n)
                    if (n < N) sv = fmaf(Io<T>::load(Cb, n * L + t), hs[k][n], sv);
                const float sz = __builtin_amdgcn_rcpf(1.0f + fast_exp2(-zt * kLog2e));
                ds = dyt * zt * sz;
                if (valid && a.dz) a.dz[rb + t] = dyt * sv * sz * (1.0f + zt * (1.0f - sz));
            }
            dDacc = fmaf(ds, ut, dDacc);
            float dut = ds * skip, ddl = 0.0f;
            // this row's dC (k < 16) and dB (k >= 16) terms of each group
            // of 16 state elements
            float vbc[NG][32];
#pragma unroll
            for (int n = 0; n < NS; ++n) {
                float cterm = 0.0f, bterm = 0.0f;
                if (n < N) {
                    const float Bt = Io<T>::load(Bb, n * L + t);
                    const float Ct = Io<T>::load(Cb, n * L + t);
                    const float an = fast_exp2(dl * A2[n]);
                    const float hp = k > 0 ? hs[k > 0 ? k - 1 : 0][n] : hb[n];
                    dh[n] = fmaf(ds, Ct, dh[n]);
                    cterm = ds * hs[k][n];
                    const float ha = hp * an;
                    dAacc[n] = fmaf(dh[n] * ha, dl, dAacc[n]);
                    bterm = dh[n] * dl * ut;
                    dut = fmaf(dh[n] * dl, Bt, dut);
                    ddl = fmaf(dh[n], fmaf(ha, A2[n] * kLn2, Bt * ut), ddl);
                    dh[n] *= an;
                }
                vbc[n / 16][n % 16] = cterm;
                vbc[n / 16][16 + n % 16] = bterm;
            }
#pragma unroll
            for (int n = NS; n < NG * 16; ++n) {
                vbc[n / 16][n % 16] = 0.0f;
                vbc[n / 16][16 + n % 16] = 0.0f;
            }
            if (want_bc) {
                // sums over the wave's rows of each batch it holds, one
                // coalesced store of 32 sums per group (lanes 0..31)
                for (int slot = 0; slot < nspan; ++slot) {
                    const bool mine = one_batch || b == b_first + slot;
#pragma unroll
                    for (int gi = 0; gi < NG; ++gi) {
                        float vm[32];
#pragma unroll
                        for (int q = 0; q < 32; ++q) vm[q] = mine ? vbc[gi][q] : 0.0f;
                        const float sum = reduce32(vm, red);
                        if (lane < 32)
                            pw[(static_cast<int64_t>(slot) * L + t) * (NG * 32) + gi * 32 + lane] = sum;
                    }
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

// dB[b, n, t] and dC[b, n, t] from the per-wave partial sums: one thread per
// (b, t, column) adds the partials of the waves holding rows of batch b, in
// wave order (slot b - b_first for a wave whose first row is in batch
// b_first).
__global__ __launch_bounds__(256) void scan_bwd_bc_kernel(const float *__restrict__ part, int nslots,
                                                          int ng, int rpw, int64_t batch, int64_t dim,
                                                          int64_t L, int N, float *dB, float *dC) {
    // one thread per four consecutive partial columns of one (batch, step):
    // 16-byte loads, so a wave reads 1 KB of each wave's partial plane
    const int64_t cols = static_cast<int64_t>(ng) * 32;
    const int64_t quads = cols / 4;
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= batch * L * quads) return;
    const int col = static_cast<int>(i % quads) * 4;
    const int64_t t = (i / quads) % L;
    const int64_t b = i / (quads * L);
    const int gi = col / 32, kk = col % 32;
    const int n = 16 * gi + kk % 16;            // state elements n .. n + 3
    if (n >= N) return;
    const int64_t w_lo = (b * dim) / rpw, w_hi = ((b + 1) * dim - 1) / rpw;
    float s[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    // unrolled so that several waves' partials are in flight at once (the
    // adds stay in wave order)
#pragma unroll 8
    for (int64_t w = w_lo; w <= w_hi; ++w) {
        const int64_t slot = b - (w * rpw) / dim;
        const float4 v = *reinterpret_cast<const float4 *>(&part[((w * nslots + slot) * L + t) * cols + col]);
        s[0] += v.x;
        s[1] += v.y;
        s[2] += v.z;
        s[3] += v.w;
    }
    float *out = kk < 16 ? dC : dB;
    if (out) {
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (n + k < N) out[(b * N + n + k) * L + t] = s[k];
    }
}

template <typename T, int NS>
hipError_t launch_typed(const BwdArgs &a, hipStream_t stream) {
    constexpr int K = seg_steps<NS>();
    constexpr int NG = n_groups<NS>();
    const int64_t rows = a.batch * a.dim;
    const int64_t waves = (rows + 63) / 64;
    const int nseg = static_cast<int>((a.L + K - 1) / K);
    // partial slots: the most batches any 64 consecutive rows span
    const int64_t span = a.dim % 64 == 0 ? 1 : 63 / a.dim + 2;
    const int nslots = static_cast<int>(std::min<int64_t>(std::min<int64_t>(a.batch, span), 64));
    const bool want_bc = a.dB || a.dC;
    const size_t ck_bytes = static_cast<size_t>(rows) * nseg * a.N * sizeof(float);
    const size_t part_bytes =
        want_bc ? static_cast<size_t>(waves) * nslots * a.L * NG * 32 * sizeof(float) : 0;
    void *mem = nullptr;
    hipError_t e = scratch_alloc(&mem, ck_bytes + part_bytes, stream);
    if (e != hipSuccess) return e;
    float *ck = static_cast<float *>(mem);
    float *part = reinterpret_cast<float *>(static_cast<char *>(mem) + ck_bytes);
    hipLaunchKernelGGL((scan_bwd_rowserial_kernel<T, NS>), dim3(static_cast<uint32_t>(waves)), dim3(64), 0,
                       stream, a, ck, nseg, part, nslots);
    e = hipGetLastError();
    if (e == hipSuccess && want_bc) {
        const int64_t n = a.batch * a.L * NG * 32 / 4;   // column quads
        hipLaunchKernelGGL(scan_bwd_bc_kernel, dim3(static_cast<uint32_t>((n + 255) / 256)), dim3(256), 0,
                           stream, part, nslots, NG, 64, a.batch, a.dim, a.L, static_cast<int>(a.N), a.dB,
                           a.dC);
        e = hipGetLastError();
    }
    const hipError_t ef = scratch_free(mem, stream);
    return e != hipSuccess ? e : ef;
}


// ---------------------------------------------------------------------------
// Lane-group forms for N <= 16: LPR lanes per row (4 or 8), each with NPL =
// 16 / LPR state elements (lane = LPR i + g: row i of the wave's 64 / LPR,
// elements n = NPL g .. NPL g + NPL - 1), so a layer has LPR times the waves
// of the one-lane-per-row form and each lane 1 / LPR of its serial work.  The
// row's scalars are formed by all LPR lanes; sums over n (the output before
// the gate, du and d(dl)) are DPP swaps within the lane group; dB and dC use
// the per-wave partial buffer as above.
// ---------------------------------------------------------------------------
constexpr int kQuadRedPitch = 8;  // floats per column of the four-lane form's reduction pass

template <int LPR> constexpr int grp_steps() { return 16; }   // steps per stored segment

template <int LPR>
__device__ __forceinline__ float group_sum(float v) {
    // quad_perm [1,0,3,2] then [2,3,0,1]: every lane of a quad gets the quad's
    // sum; for eight lanes, row_half_mirror then adds the other quad
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xb1, 0xf, 0xf, true));
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4e, 0xf, 0xf, true));
    if (LPR == 8)
        v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x141, 0xf, 0xf, true));
    return v;
}

// Four lanes per row: sum over the wave's 16 rows of v[q] (q < 4: dC terms of
// n = 4 g + q; q >= 4: dB terms of n = 4 g + q - 4).  Lanes l and l + 32 are
// paired for q, q + 4 (v_permlane32_swap), then l and l + 16 for q, q + 2
// (v_permlane16_swap), so lane l holds the sums over its column l % 16 of
// q = 4 b5 + 2 b4 + {0, 1}; the four columns of group g go through LDS.  Lane
// o < 32 returns the sum for group o % 4 and q = o / 4, the partial column
// (q < 4 ? 0 : 16) + 4 g + q % 4.
__device__ __forceinline__ float reduce_quad8(const float (&v)[8], float *red) {
    float w[4], x[2];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[k]), __float_as_uint(v[k + 4]),
                                                        false, false);
        w[k] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(w[k]), __float_as_uint(w[k + 2]),
                                                        false, false);
        x[k] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    const int lane = threadIdx.x & 63;
    *reinterpret_cast<float2 *>(red + (lane & 15) * kQuadRedPitch + 4 * ((lane >> 5) & 1) +
                                2 * ((lane >> 4) & 1)) = make_float2(x[0], x[1]);
    const int o = lane & 31, g = o & 3, q = o >> 2;
    float s = 0.0f;
#pragma unroll
    for (int m = 0; m < 4; ++m) s += red[(g + 4 * m) * kQuadRedPitch + q];
    return s;
}

// Eight lanes per row: sum over the wave's 8 rows of v[q] (q < 2: dC terms of
// n = 2 g + q; q >= 2: dB terms of n = 2 g + q - 2).  v_permlane32_swap pairs
// lanes l, l + 32 for q, q + 2; v_permlane16_swap pairs l, l + 16 for the two
// left; a row rotation by 8 adds the other row of the 16-lane DPP row.  Lane
// l then holds the sum for group l % 8 and q = 2 b5 + b4, the partial column
// (b5 ? 16 : 0) + 2 g + b4; the lanes with bit 3 clear store it.
__device__ __forceinline__ float reduce_octo4(const float (&v)[4]) {
    float w[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[k]), __float_as_uint(v[k + 2]),
                                                        false, false);
        w[k] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(w[0]), __float_as_uint(w[1]), false, false);
    float x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x128, 0xf, 0xf, true));
    return x;
}

// Value of v held by lane `src` of this lane's group of LPR lanes, through an
// LDS-free swizzle (broadcast mode: and-mask keeps the group bits, or-mask
// selects the lane).  src must fold to a constant.
template <int LPR, int SRC>
__device__ __forceinline__ float grp_bcast_c(float v) {
    constexpr int pat = (0x20 - LPR) | (SRC << 5);
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), pat));
}
template <int LPR>
__device__ __forceinline__ float grp_bcast(float v, int src) {
    switch (src) {
    case 0: return grp_bcast_c<LPR, 0>(v);
    case 1: return grp_bcast_c<LPR, 1>(v);
    case 2: return grp_bcast_c<LPR, 2>(v);
    case 3: return grp_bcast_c<LPR, 3>(v);
    case 4: return grp_bcast_c<LPR, 4 % LPR>(v);
    case 5: return grp_bcast_c<LPR, 5 % LPR>(v);
    case 6: return grp_bcast_c<LPR, 6 % LPR>(v);
    default: return grp_bcast_c<LPR, 7 % LPR>(v);
    }
}

// B or C of one state row over the K steps of a segment, as 32-bit words
// (two bf16 per word, or one float).  Full segments of aligned rows come in
// with 16-byte loads; otherwise element by element, zero past L.
template <typename T, int K>
struct SegRow {
    static constexpr int W = K * static_cast<int>(sizeof(T)) / 4;
    uint32_t w[W];
    __device__ void load(const T *row, int64_t t0, int64_t L, bool vec) {
        if (vec && t0 + K <= L) {
#pragma unroll
            for (int q = 0; q < W / 4; ++q) {
                const uint4 v = *reinterpret_cast<const uint4 *>(row + t0 + q * (16 / sizeof(T)));
                w[4 * q] = v.x; w[4 * q + 1] = v.y; w[4 * q + 2] = v.z; w[4 * q + 3] = v.w;
            }
        } else {
#pragma unroll
            for (int k = 0; k < K; k += 4 / sizeof(T)) {
                uint32_t v;
                if constexpr (sizeof(T) == 4) {
                    v = t0 + k < L ? __float_as_uint(row[t0 + k]) : 0u;
                } else {
                    const uint32_t lo = t0 + k < L ? row[t0 + k] : 0u;
                    const uint32_t hi = t0 + k + 1 < L ? row[t0 + k + 1] : 0u;
                    v = lo | (hi << 16);
                }
                w[k * sizeof(T) / 4] = v;
            }
        }
    }
    __device__ void zero() {
#pragma unroll
        for (int q = 0; q < W; ++q) w[q] = 0u;
    }
    // float32 value at step k of the segment
    __device__ float at(int k) const {
        if constexpr (sizeof(T) == 4) return __uint_as_float(w[k]);
        else return __uint_as_float((k & 1) ? (w[k >> 1] & 0xffff0000u) : (w[k >> 1] << 16));
    }
};

template <typename T, int LPR>
__global__ __launch_bounds__(64, LPR == 8 ? 2 : 1) void scan_bwd_group_kernel(BwdArgs a, float *__restrict__ ck, int nseg,
                                                            float *__restrict__ part, int nslots) {
    constexpr int K = grp_steps<LPR>();
    constexpr int NPL = 16 / LPR;     // state elements per lane
    constexpr int RPW = 64 / LPR;     // rows per wave
    constexpr int SPL = K / LPR;      // steps of a segment whose row scalars each lane forms
    static_assert(SPL * LPR == K && LPR <= 8, "segment steps split evenly over the lane group");
    const T *u = static_cast<const T *>(a.u);
    const T *delta = static_cast<const T *>(a.delta);
    const T *Bm = static_cast<const T *>(a.B);
    const T *Cm = static_cast<const T *>(a.C);
    const T *z = static_cast<const T *>(a.z);
    const T *dy = static_cast<const T *>(a.dy);
    __shared__ float red[16 * kQuadRedPitch];
    const int64_t rows = a.batch * a.dim, L = a.L;
    const int N = static_cast<int>(a.N);
    const int lane = threadIdx.x;
    const int g = lane % LPR;
    const int64_t row = static_cast<int64_t>(blockIdx.x) * RPW + lane / LPR;
    const bool valid = row < rows;
    // lanes past the last row walk the last row with zero output gradients
    const int64_t r = valid ? row : rows - 1;
    const int64_t b = r / a.dim;
    const int64_t d = r - b * a.dim;
    const int64_t r_first = static_cast<int64_t>(blockIdx.x) * RPW;
    const int64_t r_last = min(r_first + RPW - 1, rows - 1);
    const int nspan = static_cast<int>(r_last / a.dim - r_first / a.dim) + 1;
    const int64_t b_first = r_first / a.dim;
    const bool want_bc = a.dB || a.dC;
    float *pw = part + static_cast<int64_t>(blockIdx.x) * nslots * L * 32;

    float A2[NPL];
    bool nok[NPL];
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
        const int n = NPL * g + i;
        nok[i] = n < N;
        A2[i] = nok[i] ? a.A[d * N + n] * kLog2e : 0.0f;
    }
    const float bias = a.delta_bias ? a.delta_bias[d] : 0.0f;
    const float skip = a.D ? a.D[d] : 0.0f;
    const int64_t rb = r * L;
    const T *Bb = Bm + b * N * L;
    const T *Cb = Cm + b * N * L;
    // stored states: 16 floats per (row, segment), this lane's NPL at NPL g
    float *ckr = ck + r * static_cast<int64_t>(nseg) * 16 + NPL * g;
    // B and C rows 16-byte aligned at every segment start
    const bool vbc = L % 8 == 0 &&
                     ((reinterpret_cast<uintptr_t>(a.B) | reinterpret_cast<uintptr_t>(a.C)) & 15u) == 0;
    auto load_rows = [&](SegRow<T, K> (&rows)[NPL], const T *base, int64_t t0) {
#pragma unroll
        for (int i = 0; i < NPL; ++i) {
            if (nok[i]) rows[i].load(base + (NPL * g + i) * L, t0, L, vbc);
            else rows[i].zero();
        }
    };

    // Inputs of one segment for this lane, exactly as loaded: its SPL steps
    // of the row's delta and u (and, for the reverse, dy, z and the stored
    // state), and its rows of B (and C).  With eight lanes per row each pass
    // loads segment s + 1 (or s - 1) into the second of two sets while
    // segment s is worked on, so the loads' latency is covered by a segment
    // of work; two sets used in turn need no copy (the kernel is held to two
    // waves per SIMD, at the cost of a small register spill).  Steps past L
    // are read at L - 1 and never used.
    struct FwdIn {
        T rd[SPL], ru[SPL];
        SegRow<T, K> b[NPL];
    };
    struct RevIn {
        float hb[NPL];
        T rd[SPL], ru[SPL], ry[SPL], rz[SPL];
        SegRow<T, K> b[NPL], c[NPL];
    };
    auto load_fwd = [&](int s, FwdIn &in) {
        const int64_t t0 = static_cast<int64_t>(s) * K;
#pragma unroll
        for (int m = 0; m < SPL; ++m) {
            const int64_t t = min(t0 + SPL * g + m, L - 1);
            in.rd[m] = delta[rb + t];
            in.ru[m] = u[rb + t];
        }
        load_rows(in.b, Bb, t0);
    };
    auto load_rev = [&](int s, RevIn &in) {
        const int64_t t0 = static_cast<int64_t>(s) * K;
#pragma unroll
        for (int i = 0; i < NPL; ++i) in.hb[i] = ckr[s * 16 + i];
#pragma unroll
        for (int m = 0; m < SPL; ++m) {
            const int64_t t = min(t0 + SPL * g + m, L - 1);
            in.rd[m] = delta[rb + t];
            in.ru[m] = u[rb + t];
            in.ry[m] = dy[rb + t];
            in.rz[m] = z ? z[rb + t] : T(0);
        }
        load_rows(in.b, Bb, t0);
        load_rows(in.c, Cb, t0);
    };
    auto to_f = [](T v) -> float {
        if constexpr (sizeof(T) == 4) return v;
        else return __uint_as_float(static_cast<uint32_t>(v) << 16);
    };

    // ---- forward: the state before every segment ---------------------------
    float h[NPL];
#pragma unroll
    for (int i = 0; i < NPL; ++i) h[i] = (a.h0 && nok[i]) ? a.h0[r * N + NPL * g + i] : 0.0f;
    auto fwd_seg = [&](int s, const FwdIn &in) {
        if (valid) {
#pragma unroll
            for (int i = 0; i < NPL; ++i) ckr[s * 16 + i] = h[i];
        }
        // dl and dl*u of this lane's SPL steps
        float sdl[SPL], sdu[SPL];
#pragma unroll
        for (int m = 0; m < SPL; ++m) {
            sdl[m] = softplus(to_f(in.rd[m]) + bias);
            sdu[m] = sdl[m] * to_f(in.ru[m]);
        }
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int64_t t = static_cast<int64_t>(s) * K + k;
            if (t < L) {
                const float dl = grp_bcast<LPR>(sdl[k % SPL], k / SPL);
                const float du = grp_bcast<LPR>(sdu[k % SPL], k / SPL);
#pragma unroll
                for (int i = 0; i < NPL; ++i)
                    if (nok[i]) h[i] = fmaf(fast_exp2(dl * A2[i]), h[i], du * in.b[i].at(k));
            }
        }
    };
    if constexpr (LPR == 8) {
        FwdIn f0, f1;
        load_fwd(0, f0);
        int s = 0;
        for (; s + 1 < nseg; s += 2) {
            load_fwd(s + 1, f1);
            fwd_seg(s, f0);
            load_fwd(s + 2, f0);
            fwd_seg(s + 1, f1);
        }
        if (s < nseg) fwd_seg(s, f0);
    } else {
        // four lanes per row hold twice the state elements per lane: one
        // input set, loaded at each segment's start, keeps them in registers
        for (int s = 0; s < nseg; ++s) {
            FwdIn f0;
            load_fwd(s, f0);
            fwd_seg(s, f0);
        }
    }

    // ---- reverse ---------------------------------------------------------
    float dh[NPL], dAacc[NPL];
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
        dh[i] = (valid && a.dh_last && nok[i]) ? a.dh_last[r * N + NPL * g + i] : 0.0f;
        dAacc[i] = 0.0f;
    }
    float dDacc = 0.0f, dbacc = 0.0f;
    auto rev_seg = [&](int s, const RevIn &in) {
        const int64_t t0 = static_cast<int64_t>(s) * K;
        // this lane's SPL steps of the row's per-step scalars: dl, dl*u, the
        // logistic of x, u, ds = dy silu(z) and the gate-gradient factor
        // dz / s = dy sigmoid(z) (1 + z (1 - sigmoid(z)))
        float sdl[SPL], sdu[SPL], ssig[SPL], sut[SPL], sds[SPL], sdzf[SPL];
#pragma unroll
        for (int m = 0; m < SPL; ++m) {
            const int64_t t = t0 + SPL * g + m;
            const float x = to_f(in.rd[m]) + bias;
            const float ut = to_f(in.ru[m]);
            sdl[m] = softplus(x);
            sdu[m] = sdl[m] * ut;
            ssig[m] = __builtin_amdgcn_rcpf(1.0f + fast_exp2(-x * kLog2e));
            sut[m] = ut;
            const float dyt = (valid && t < L) ? to_f(in.ry[m]) : 0.0f;
            if (z) {
                const float zt = to_f(in.rz[m]);
                const float sz = __builtin_amdgcn_rcpf(1.0f + fast_exp2(-zt * kLog2e));
                sds[m] = dyt * zt * sz;
                sdzf[m] = dyt * sz * (1.0f + zt * (1.0f - sz));
            } else {
                sds[m] = dyt;
                sdzf[m] = 0.0f;
            }
        }
        // the segment's states, recomputed
        float hs[K][NPL];
#pragma unroll
        for (int i = 0; i < NPL; ++i) h[i] = in.hb[i];
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int64_t t = t0 + k;
            if (t < L) {
                const float dl = grp_bcast<LPR>(sdl[k % SPL], k / SPL);
                const float du = grp_bcast<LPR>(sdu[k % SPL], k / SPL);
#pragma unroll
                for (int i = 0; i < NPL; ++i)
                    if (nok[i]) h[i] = fmaf(fast_exp2(dl * A2[i]), h[i], du * in.b[i].at(k));
            }
#pragma unroll
            for (int i = 0; i < NPL; ++i) hs[k][i] = h[i];
        }
        // this lane's SPL steps of du, ddelta and dz, stored after the segment
        float odu[SPL], odd[SPL], odz[SPL];
#pragma unroll
        for (int m = 0; m < SPL; ++m) odu[m] = odd[m] = odz[m] = 0.0f;
#pragma unroll
        for (int k = K - 1; k >= 0; --k) {
            const int64_t t = t0 + k;
            if (t >= L) continue;
            const int src = k / SPL, ms = k % SPL;
            const float dl = grp_bcast<LPR>(sdl[ms], src);
            const float sig = grp_bcast<LPR>(ssig[ms], src);
            const float ut = grp_bcast<LPR>(sut[ms], src);
            const float ds = grp_bcast<LPR>(sds[ms], src);
            if (z) {
                float sp = 0.0f;
#pragma unroll
                for (int i = 0; i < NPL; ++i)
                    if (nok[i]) sp = fmaf(in.c[i].at(k), hs[k][i], sp);
                const float sv = fmaf(skip, ut, group_sum<LPR>(sp));
                const float dzv = grp_bcast<LPR>(sdzf[ms], src) * sv;
                if (g == src) odz[ms] = dzv;
            }
            dDacc = fmaf(ds, ut, dDacc);
            float dup = 0.0f, ddlp = 0.0f;
            float vbc[2 * NPL];
#pragma unroll
            for (int i = 0; i < NPL; ++i) {
                float cterm = 0.0f, bterm = 0.0f;
                if (nok[i]) {
                    const float Bt = in.b[i].at(k);
                    const float Ct = in.c[i].at(k);
                    const float an = fast_exp2(dl * A2[i]);
                    const float hp = k > 0 ? hs[k > 0 ? k - 1 : 0][i] : in.hb[i];
                    dh[i] = fmaf(ds, Ct, dh[i]);
                    cterm = ds * hs[k][i];
                    const float ha = hp * an;
                    dAacc[i] = fmaf(dh[i] * ha, dl, dAacc[i]);
                    bterm = dh[i] * dl * ut;
                    dup = fmaf(dh[i] * dl, Bt, dup);
                    ddlp = fmaf(dh[i], fmaf(ha, A2[i] * kLn2, Bt * ut), ddlp);
                    dh[i] *= an;
                }
                vbc[i] = cterm;
                vbc[NPL + i] = bterm;
            }
            const float dut = fmaf(ds, skip, group_sum<LPR>(dup));
            const float ddl = group_sum<LPR>(ddlp);
            if (g == src) {
                odu[ms] = dut;
                odd[ms] = ddl * sig;
            }
            dbacc = fmaf(ddl, sig, dbacc);
            if (want_bc) {
                // sums over the wave's rows of each batch it holds, stored as
                // partial column dC n (< 16) or 16 + dB n
                for (int slot = 0; slot < nspan; ++slot) {
                    const bool mine = nspan == 1 || b == b_first + slot;
                    float vm[2 * NPL];
#pragma unroll
                    for (int q = 0; q < 2 * NPL; ++q) vm[q] = mine ? vbc[q] : 0.0f;
                    float* dst = pw + (static_cast<int64_t>(slot) * L + t) * 32;
                    if constexpr (LPR == 4) {
                        const float sum = reduce_quad8(vm, red);
                        const int o = lane & 31, og = o & 3, oq = o >> 2;
                        if (lane < 32) dst[(oq < 4 ? 0 : 16) + 4 * og + (oq & 3)] = sum;
                    } else {
                        const float sum = reduce_octo4(vm);
                        if ((lane & 8) == 0)
                            dst[((lane >> 5) & 1 ? 16 : 0) + 2 * (lane & 7) + ((lane >> 4) & 1)] = sum;
                    }
                }
            }
        }
        // the segment's du, ddelta (and dz): SPL consecutive steps per lane
        if (valid) {
#pragma unroll
            for (int m = 0; m < SPL; ++m) {
                const int64_t t = t0 + SPL * g + m;
                if (t < L) {
                    a.du[rb + t] = odu[m];
                    a.ddelta[rb + t] = odd[m];
                    if (z && a.dz) a.dz[rb + t] = odz[m];
                }
            }
        }
    };
    if constexpr (LPR == 8) {
        RevIn r0, r1;
        load_rev(nseg - 1, r0);
        int s = nseg - 1;
        for (; s - 1 >= 0; s -= 2) {
            load_rev(s - 1, r1);
            rev_seg(s, r0);
            if (s - 2 >= 0) load_rev(s - 2, r0);
            rev_seg(s - 1, r1);
        }
        if (s >= 0) rev_seg(s, r0);
    } else {
        for (int s = nseg - 1; s >= 0; --s) {
            RevIn r0;
            load_rev(s, r0);
            rev_seg(s, r0);
        }
    }
    if (valid) {
#pragma unroll
        for (int i = 0; i < NPL; ++i) {
            if (!nok[i]) continue;
            if (a.dh0) a.dh0[r * N + NPL * g + i] = dh[i];
            if (a.dA) atomicAdd(a.dA + d * N + NPL * g + i, dAacc[i]);
        }
        if (g == 0) {
            if (a.dD) atomicAdd(a.dD + d, dDacc);
            if (a.ddelta_bias) atomicAdd(a.ddelta_bias + d, dbacc);
        }
    }
}

template <typename T, int LPR>
hipError_t launch_group(const BwdArgs &a, hipStream_t stream) {
    constexpr int K = grp_steps<LPR>();
    constexpr int RPW = 64 / LPR;
    const int64_t rows = a.batch * a.dim;
    const int64_t waves = (rows + RPW - 1) / RPW;
    const int nseg = static_cast<int>((a.L + K - 1) / K);
    // partial slots: the most batches any RPW consecutive rows span
    const int64_t span = a.dim % RPW == 0 ? 1 : (RPW - 1) / a.dim + 2;
    const int nslots = static_cast<int>(std::min<int64_t>(std::min<int64_t>(a.batch, span), RPW));
    const bool want_bc = a.dB || a.dC;
    const size_t ck_bytes = static_cast<size_t>(rows) * nseg * 16 * sizeof(float);
    const size_t part_bytes = want_bc ? static_cast<size_t>(waves) * nslots * a.L * 32 * sizeof(float) : 0;
    void *mem = nullptr;
    hipError_t e = scratch_alloc(&mem, ck_bytes + part_bytes, stream);
    if (e != hipSuccess) return e;
    float *ck = static_cast<float *>(mem);
    float *part = reinterpret_cast<float *>(static_cast<char *>(mem) + ck_bytes);
    hipLaunchKernelGGL((scan_bwd_group_kernel<T, LPR>), dim3(static_cast<uint32_t>(waves)), dim3(64), 0, stream,
                       a, ck, nseg, part, nslots);
    e = hipGetLastError();
    if (e == hipSuccess && want_bc) {
        const int64_t n = a.batch * a.L * 32 / 4;   // column quads
        hipLaunchKernelGGL(scan_bwd_bc_kernel, dim3(static_cast<uint32_t>((n + 255) / 256)), dim3(256), 0,
                           stream, part, nslots, 1, RPW, a.batch, a.dim, a.L, static_cast<int>(a.N), a.dB,
                           a.dC);
        e = hipGetLastError();
    }
    const hipError_t ef = scratch_free(mem, stream);
    return e != hipSuccess ? e : ef;
}

template <typename T>
hipError_t launch_by_n(const BwdArgs &a, hipStream_t stream) {
    if (a.N <= 8) return launch_group<T, 4>(a, stream);
    if (a.N <= 16) return launch_group<T, 8>(a, stream);
    if (a.N <= 32) return launch_typed<T, 32>(a, stream);
    return launch_typed<T, 64>(a, stream);
}

}  // namespace

bool scan_bwd_supported(const BwdArgs &a) {
    return a.N >= 1 && a.N <= 64 && (a.batch * a.dim + 7) / 8 < (int64_t(1) << 31) &&
           a.L < (int64_t(1) << 31);
}

hipError_t launch_scan_bwd(const BwdArgs &a, hipStream_t stream) {
    if (a.io == IO_F32) return launch_by_n<float>(a, stream);
    return launch_by_n<uint16_t>(a, stream);
}

}  // namespace mssm
