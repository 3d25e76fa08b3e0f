// ssd_chunked.hip -- Mamba-2 scalar-decay (SSD) forward in the chunked
// matrix form, on the gfx950 matrix cores (v_mfma_f32_32x32x16_bf16).
//
// Per batch b and head h, with dl_t = softplus(dt_t + dt_bias[h]) and the
// log decay l_t = dl_t A[h] ("Mamba状态空间模型的硬件感知推理优化" (ybb.press)
// section 4: one scalar decay per step and head; section 6.2: cumulative
// products taken in log space), the sequence is cut into chunks of Q steps.
// Inside a chunk, with cum_t the inclusive sum of l over the chunk up to t:
//
//   Y_diag[t,p] = sum_{s<=t} (C_t . B_s) exp(cum_t - cum_s) dl_s x_s[p]
//   Y_off[t,p]  = exp(cum_t) sum_n C_t[n] h_prev[p,n]
//   S[p,n]      = sum_s exp(cum_end - cum_s) dl_s x_s[p] B_s[n]
//   h[p,n]      = exp(cum_end) h_prev[p,n] + S[p,n]
//   y[t,p]      = Y_diag + Y_off + D[h] x_t[p]
//
// which is the recurrence S_t = a_t S_{t-1} + dl_t x_t B_t^T, y = C_t S_t +
// D x_t unrolled over the chunk (the cumulative-product closed form of the
// same ybb.press section).  Chunks are walked in order, so h never leaves
// the chip.
//
// Work decomposition.  A workgroup of four waves owns one (batch, head,
// 32-wide slice of the head dimension) and walks every chunk.  Per chunk:
//   * B (Q x N) is staged in LDS as bf16, x (Q x 32) transposed to (32 x Q),
//     and x * exp(cum_end - cum_s) dl_s split into bf16 high and low parts;
//   * wave w takes the 32-row time blocks w and Q/32-1-w (balanced causal
//     work).  For each earlier-or-equal source block it forms
//     G' = B_s C_t^T on the matrix cores, scales it by exp(cum_t - cum_s)
//     dl_s under the causal mask in registers, splits the result into bf16
//     high/low parts, and feeds them straight back as the A operand of the
//     product with x -- the accumulator layout of G' (column = target step)
//     is the operand layout with a permuted K order, and x is read in the
//     same permuted order, so no LDS round trip is needed;
//   * the off-diagonal term C_t h_prev^T reads h_prev (bf16 high/low) from
//     LDS; y is assembled in registers and stored;
//   * wave w also forms the chunk state S for state columns 32w..32w+31.
// Products whose operands are not exact bf16 values (the masked decay
// matrix, x * decay, the carried state) use a two-term bf16 split, so every
// product carries about 16 significant bits; accumulation is float32.
#include "device_math.h"
#include "internal.h"

namespace mssm {
namespace {

typedef __bf16 bf8 __attribute__((ext_vector_type(8)));
typedef float f16x __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kPt = 32;                 // head-dimension columns per workgroup

__device__ __forceinline__ f16x mfma(bf8 a, bf8 b, f16x c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint16_t bf16_bits(__bf16 v) { return __builtin_bit_cast(uint16_t, v); }
__device__ __forceinline__ float bf16_val(__bf16 v) {
    return __uint_as_float(static_cast<uint32_t>(bf16_bits(v)) << 16);
}
// Two floats rounded to bf16 (nearest even), packed low half first.
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
    const bf2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
    return __builtin_bit_cast(uint32_t, v);
}
// Two-term split: v ~= hi + lo with both parts bf16 (about 16 significant bits).
__device__ __forceinline__ void split(float v, __bf16 &hi, __bf16 &lo) {
    hi = static_cast<__bf16>(v);
    lo = static_cast<__bf16>(v - bf16_val(hi));
}

// Eight consecutive bf16 of row `t` starting at column c8 of a row-major
// (rows x cols) slice with row stride `stride`; zero past the last row or
// column.  Branch-free: out-of-range reads are redirected to element 0 and
// the value is discarded, so all loads of a phase are in flight together.
// vec: rows start 16-byte aligned and cols % 8 == 0.
__device__ __forceinline__ uint4 load_row8(const uint16_t *base, int64_t t, int c8, int64_t rows,
                                           int cols, int64_t stride, bool vec) {
    const bool okt = t < rows;
    if (vec) {
        const bool ok = okt && c8 < cols;
        const uint4 v = *reinterpret_cast<const uint4 *>(base + (ok ? t * stride + c8 : 0));
        return ok ? v : make_uint4(0, 0, 0, 0);
    }
    uint16_t e[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        const bool ok = okt && c8 + r < cols;
        const uint16_t w = base[ok ? t * stride + c8 + r : 0];
        e[r] = ok ? w : 0;
    }
    uint4 v;
    __builtin_memcpy(&v, e, 16);
    return v;
}

template <typename T> struct Ld;
template <> struct Ld<uint16_t> {
    __device__ static float f(const uint16_t *p, int64_t i) { return bf16_to_f32(p[i]); }
};

// LDS of one workgroup (bf16 data held as raw uint16_t).
template <int Q, int NP>
struct __align__(16) Smem {
    // Row pitches (elements) chosen so the operand reads of one instruction
    // fall in distinct LDS banks: 8-byte reads of X need a row stride of
    // 2 mod 64 dwords, 16-byte reads of Xw, B and h_prev 4 mod 64 dwords.
    static constexpr int BP = NP + 8;   // B[s][n]
    static constexpr int XP = Q + 4;    // x[s][p] stored as X[p][s]
    static constexpr int WP = Q + 8;    // x * w, stored like X
    static constexpr int HP = NP + 8;   // h_prev[p][n]
    uint16_t B[Q * BP];
    uint16_t X[kPt * XP];
    uint16_t Xwh[kPt * WP], Xwl[kPt * WP];   // high / low bf16 parts
    uint16_t Hh[kPt * HP], Hl[kPt * HP];     // high / low bf16 parts
    float cum[Q];      // inclusive sum of the log2 decay over the chunk
    float dl[Q];
    float fs[Q];       // 2^(cum at the end of s's 32-step block - cum_s) dl_s
    float wsum[kThreads / 64];
};

template <int Q, int NP>
__global__ __launch_bounds__(kThreads) void ssd_chunked_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ dt,
    const float *__restrict__ dt_bias, const float *__restrict__ A,
    const uint16_t *__restrict__ Bm, const uint16_t *__restrict__ Cm,
    const float *__restrict__ Dskip, uint16_t *__restrict__ y,
    float *__restrict__ h_last, int64_t L, int H, int P, int N, int G, int ptiles, bool vec,
    bool vecx) {
    // vec: B and C rows start 16-byte aligned (N % 8 == 0 and aligned bases);
    // vecx: the same for x (P % 8 == 0 and an aligned base)
    using S = Smem<Q, NP>;
    constexpr int NT = Q / 32;          // 32-step time blocks per chunk
    constexpr int KN = NP / 16;         // K steps over the state index
    constexpr int KQ = Q / 16;          // K steps over a chunk
    __shared__ S sm;

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int half = lane >> 5;
    const int pt = blockIdx.x % ptiles;
    const int hh = (blockIdx.x / ptiles) % H;
    const int64_t b = blockIdx.x / (static_cast<int64_t>(ptiles) * H);
    const int g = hh / (H / G);
    const int p0 = pt * kPt;
    const float A2 = A[hh] * kLog2e;
    const float bias = dt_bias ? dt_bias[hh] : 0.0f;
    const float skip = Dskip ? Dskip[hh] : 0.0f;
    const int64_t rowBC = static_cast<int64_t>(G) * N;   // stride of B/C between steps
    const int64_t rowX = static_cast<int64_t>(H) * P;    // stride of x/y between steps
    const uint16_t *Bg = Bm + (b * L * G + g) * N;
    const uint16_t *Cg = Cm + (b * L * G + g) * N;
    const uint16_t *xg = x + b * L * rowX + static_cast<int64_t>(hh) * P + p0;
    uint16_t *yg = y + b * L * rowX + static_cast<int64_t>(hh) * P + p0;
    const uint16_t *dtg = dt + b * L * H + hh;

    // State h[p][n] for p = p(v), n = 32 * wave + l32, in the 32x32 result
    // layout: p(v) = 8 (v / 4) + 4 half + v % 4.
    f16x hst;
#pragma unroll
    for (int v = 0; v < 16; ++v) hst[v] = 0.0f;
    const int nS = 32 * wave + l32;      // this lane's state column
    for (int i = tid; i < kPt * S::HP; i += kThreads) { sm.Hh[i] = 0; sm.Hl[i] = 0; }

    const int64_t nchunks = (L + Q - 1) / Q;
    for (int64_t c = 0; c < nchunks; ++c) {
        const int64_t t0 = c * Q;
        // ---- stage B (Q x NP) and x (Q x 32, transposed); dl and its scan ---
        for (int u = tid; u < Q * (NP / 8); u += kThreads) {
            const int s = u / (NP / 8), n8 = (u % (NP / 8)) * 8;
            *reinterpret_cast<uint4 *>(&sm.B[s * S::BP + n8]) = load_row8(Bg, t0 + s, n8, L, N, rowBC, vec);
        }
        // x: units of (two consecutive steps, 8 head-dim columns); each unit
        // is written transposed as 8 dwords (step pair packed) -- no
        // sub-dword LDS writes.  Q / 128 units per thread (one half of the
        // threads when Q = 64).
        constexpr int XU = (2 * Q + kThreads - 1) / kThreads;
        float xr[XU][2][8];
#pragma unroll
        for (int k = 0; k < XU; ++k) {
            const int u = tid + k * kThreads;
            if (u < 2 * Q) {
                const int s2 = 2 * (u / (kPt / 8)), pg = (u % (kPt / 8)) * 8;
                const uint4 v0 = load_row8(xg, t0 + s2, pg, L, P - p0, rowX, vecx);
                const uint4 v1 = load_row8(xg, t0 + s2 + 1, pg, L, P - p0, rowX, vecx);
                uint16_t e0[8], e1[8];
                __builtin_memcpy(e0, &v0, 16);
                __builtin_memcpy(e1, &v1, 16);
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    xr[k][0][r] = __uint_as_float(static_cast<uint32_t>(e0[r]) << 16);
                    xr[k][1][r] = __uint_as_float(static_cast<uint32_t>(e1[r]) << 16);
                    *reinterpret_cast<uint32_t *>(&sm.X[(pg + r) * S::XP + s2]) =
                        static_cast<uint32_t>(e0[r]) | (static_cast<uint32_t>(e1[r]) << 16);
                }
            }
        }
        // dl and the log decay of step tid (threads >= Q idle here)
        float ell = 0.0f;
        if (tid < Q) {
            const bool okt = t0 + tid < L;
            const float dr = Ld<uint16_t>::f(dtg, okt ? (t0 + tid) * H : 0);
            const float dlv = okt ? softplus(dr + bias) : 0.0f;
            sm.dl[tid] = dlv;
            ell = dlv * A2;                          // log2 of the step decay
        }
        // inclusive scan of ell over the chunk: within waves, then across
        float sc = ell;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float o = __shfl_up(sc, off, 64);
            if (lane >= off) sc += o;
        }
        if (lane == 63) sm.wsum[wave] = sc;
        __syncthreads();
        if (tid < Q) {
            float base = 0.0f;
            for (int w2 = 0; w2 < wave; ++w2) base += sm.wsum[w2];
            sm.cum[tid] = sc + base;
        }
        __syncthreads();

        const float cum_end = sm.cum[Q - 1];
        // ---- per-step factors of the decay, x * w as bf16 high / low --------
        if (tid < Q) {
            const float cb = sm.cum[(tid | 31)];
            sm.fs[tid] = fast_exp2(cb - sm.cum[tid]) * sm.dl[tid];
        }
#pragma unroll
        for (int k = 0; k < XU; ++k) {
            const int u = tid + k * kThreads;
            if (u < 2 * Q) {
                const int s2 = 2 * (u / (kPt / 8)), pg = (u % (kPt / 8)) * 8;
                // w_s = 2^(cum_end - cum_s) dl_s: the weight of step s in the
                // state at the chunk end
                const float w0 = fast_exp2(cum_end - sm.cum[s2]) * sm.dl[s2];
                const float w1 = fast_exp2(cum_end - sm.cum[s2 + 1]) * sm.dl[s2 + 1];
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    const float a0 = xr[k][0][r] * w0, a1 = xr[k][1][r] * w1;
                    const uint32_t hi = pack2(a0, a1);
                    const uint32_t lo = pack2(a0 - __uint_as_float(hi << 16),
                                              a1 - __uint_as_float(hi & 0xffff0000u));
                    *reinterpret_cast<uint32_t *>(&sm.Xwh[(pg + r) * S::WP + s2]) = hi;
                    *reinterpret_cast<uint32_t *>(&sm.Xwl[(pg + r) * S::WP + s2]) = lo;
                }
            }
        }
        __syncthreads();

        // ---- output rows: time blocks tb = wave and NT - 1 - wave -----------
        // (with NT < 8 blocks, only waves 0 .. NT/2 - 1 have rows)
#pragma unroll 1
        for (int which = 0; which < 2 && 2 * wave < NT; ++which) {
            const int tb = which == 0 ? wave : NT - 1 - wave;
            const int tl = tb * 32 + l32;            // this lane's target step (in chunk)
            // C fragments of the 32 target steps: row tl, n = 16 j + 8 half + r
            bf8 cf[KN];
#pragma unroll
            for (int jn = 0; jn < KN; ++jn) {
                cf[jn] = __builtin_bit_cast(bf8, load_row8(Cg, t0 + tl, 16 * jn + 8 * half, L, N, rowBC, vec));
            }
            const float cum_t = sm.cum[tl];
            f16x yd;
#pragma unroll
            for (int v = 0; v < 16; ++v) yd[v] = 0.0f;
            for (int sb = 0; sb <= tb; ++sb) {
                // G'[s][t] = B_s . C_t for s in block sb, t in block tb
                f16x gacc;
#pragma unroll
                for (int v = 0; v < 16; ++v) gacc[v] = 0.0f;
#pragma unroll
                for (int jn = 0; jn < KN; ++jn) {
                    const bf8 a = *reinterpret_cast<const bf8 *>(
                        &sm.B[(sb * 32 + l32) * S::BP + 16 * jn + 8 * half]);
                    gacc = mfma(a, cf[jn], gacc);
                }
                // M[t][s] = G'[s][t] 2^(cum_t - cum_s) dl_s for s <= t, else 0.
                // This lane holds column t = tl and rows s(v) = 8(v/4) + 4 half + v%4.
                // Off the diagonal block every s < t and the decay factors as
                // 2^(cum_t - cb) * fs[s], cb the cum at the end of block sb:
                // both factors are <= 1 (and <= dl_s), so nothing overflows.
                // On the diagonal block the exponent is formed directly and
                // steps s > t are masked out by selection.
                float mval[16];
                if (sb < tb) {
                    const float et = fast_exp2(cum_t - sm.cum[sb * 32 + 31]);
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int sl = sb * 32 + 8 * (v / 4) + 4 * half + (v % 4);
                        mval[v] = gacc[v] * (et * sm.fs[sl]);
                    }
                } else {
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int sl = sb * 32 + 8 * (v / 4) + 4 * half + (v % 4);
                        const float mv = gacc[v] * fast_exp2(cum_t - sm.cum[sl]) * sm.dl[sl];
                        mval[v] = sl <= tl ? mv : 0.0f;
                    }
                }
                bf8 mh[2], ml[2];
#pragma unroll
                for (int v = 0; v < 16; v += 2) {
                    const uint32_t hi = pack2(mval[v], mval[v + 1]);
                    const uint32_t lo = pack2(mval[v] - __uint_as_float(hi << 16),
                                              mval[v + 1] - __uint_as_float(hi & 0xffff0000u));
                    mh[v / 8][v % 8] = __builtin_bit_cast(__bf16, static_cast<uint16_t>(hi));
                    mh[v / 8][v % 8 + 1] = __builtin_bit_cast(__bf16, static_cast<uint16_t>(hi >> 16));
                    ml[v / 8][v % 8] = __builtin_bit_cast(__bf16, static_cast<uint16_t>(lo));
                    ml[v / 8][v % 8 + 1] = __builtin_bit_cast(__bf16, static_cast<uint16_t>(lo >> 16));
                }
                // Y_diag[t][p] += sum_s M[t][s] x[s][p], K order s(v) as above:
                // operand lane (p = l32, half) reads x[s(v)][p] for the same v.
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    const int sA = sb * 32 + 16 * kk + 4 * half;   // s(8kk + 0..3)
                    const uint16_t *xp = &sm.X[l32 * S::XP];
                    uint2 lo4 = *reinterpret_cast<const uint2 *>(xp + sA);
                    uint2 hi4 = *reinterpret_cast<const uint2 *>(xp + sA + 8);
                    const uint4 xv4 = make_uint4(lo4.x, lo4.y, hi4.x, hi4.y);
                    const bf8 xb = __builtin_bit_cast(bf8, xv4);
                    yd = mfma(mh[kk], xb, yd);
                    yd = mfma(ml[kk], xb, yd);
                }
            }
            // Y_off[t][p] = sum_n C_t[n] h_prev[p][n]
            f16x yo;
#pragma unroll
            for (int v = 0; v < 16; ++v) yo[v] = 0.0f;
#pragma unroll
            for (int jn = 0; jn < KN; ++jn) {
                const int n8 = 16 * jn + 8 * half;
                const bf8 bh = *reinterpret_cast<const bf8 *>(&sm.Hh[l32 * S::HP + n8]);
                const bf8 bl = *reinterpret_cast<const bf8 *>(&sm.Hl[l32 * S::HP + n8]);
                yo = mfma(cf[jn], bh, yo);
                yo = mfma(cf[jn], bl, yo);
            }
            // y[t][p], this lane: p = l32, t(v) = 8(v/4) + 4 half + v%4
            const int p = p0 + l32;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int tv = tb * 32 + 8 * (v / 4) + 4 * half + (v % 4);
                const float xs = __uint_as_float(static_cast<uint32_t>(sm.X[l32 * S::XP + tv]) << 16);
                const float yv = yd[v] + fast_exp2(sm.cum[tv]) * yo[v] + skip * xs;
                if (t0 + tv < L && p < P) yg[(t0 + tv) * rowX + l32] = f32_to_bf16(yv);
            }
        }

        // ---- chunk state for state columns n = 32 wave .. 32 wave + 31 -------
        f16x sacc;
#pragma unroll
        for (int v = 0; v < 16; ++v) sacc[v] = 0.0f;
        if (32 * wave < NP) {
#pragma unroll 4
            for (int kq = 0; kq < KQ; ++kq) {
                const int s8 = 16 * kq + 8 * half;
                const bf8 ah = *reinterpret_cast<const bf8 *>(&sm.Xwh[l32 * S::WP + s8]);
                const bf8 al = *reinterpret_cast<const bf8 *>(&sm.Xwl[l32 * S::WP + s8]);
                bf8 bb;
#pragma unroll
                for (int r = 0; r < 8; ++r)
                    bb[r] = __builtin_bit_cast(__bf16, sm.B[(s8 + r) * S::BP + nS]);
                sacc = mfma(ah, bb, sacc);
                sacc = mfma(al, bb, sacc);
            }
        }
        __syncthreads();   // every wave is done with B, x, x*w and h_prev

        // ---- h = 2^(cum_end) h + S; publish h_prev for the next chunk -------
        const float decay = fast_exp2(cum_end);
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            hst[v] = fmaf(decay, hst[v], sacc[v]);
            const int pv = 8 * (v / 4) + 4 * half + (v % 4);
            if (32 * wave < NP) {
                __bf16 hi, lo;
                split(hst[v], hi, lo);
                sm.Hh[pv * S::HP + nS] = bf16_bits(hi);
                sm.Hl[pv * S::HP + nS] = bf16_bits(lo);
            }
        }
        __syncthreads();
    }

    if (h_last && 32 * wave < NP && nS < N) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int pv = p0 + 8 * (v / 4) + 4 * half + (v % 4);
            if (pv < P) h_last[((b * H + hh) * static_cast<int64_t>(P) + pv) * N + nS] = hst[v];
        }
    }
}

template <int Q, int NP>
hipError_t launch_typed(const SSDArgs &a, hipStream_t stream) {
    const int ptiles = static_cast<int>((a.P + kPt - 1) / kPt);
    const int64_t grid = a.batch * a.H * ptiles;
    auto aligned = [](const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
    const bool vec = a.N % 8 == 0 && aligned(a.B) && aligned(a.C);
    const bool vecx = a.P % 8 == 0 && aligned(a.x);
    hipLaunchKernelGGL((ssd_chunked_kernel<Q, NP>), dim3(static_cast<uint32_t>(grid)), dim3(kThreads),
                       0, stream, static_cast<const uint16_t *>(a.x),
                       static_cast<const uint16_t *>(a.dt), a.dt_bias, a.A,
                       static_cast<const uint16_t *>(a.B), static_cast<const uint16_t *>(a.C), a.D,
                       static_cast<uint16_t *>(a.y), a.h_last, a.L, static_cast<int>(a.H),
                       static_cast<int>(a.P), static_cast<int>(a.N), static_cast<int>(a.G), ptiles, vec, vecx);
    return hipGetLastError();
}

template <int Q>
hipError_t launch_by_n(const SSDArgs &a, hipStream_t stream) {
    if (a.N <= 32) return launch_typed<Q, 32>(a, stream);
    if (a.N <= 64) return launch_typed<Q, 64>(a, stream);
    if (a.N <= 96) return launch_typed<Q, 96>(a, stream);
    return launch_typed<Q, 128>(a, stream);
}

}  // namespace

bool ssd_chunked_supported(const SSDArgs &a) {
    return a.io == IO_BF16 && a.N >= 1 && a.N <= 128 && a.P >= 1 &&
           (a.chunk == 64 || a.chunk == 128 || a.chunk == 256) &&
           a.batch * a.H * ((a.P + kPt - 1) / kPt) < (int64_t(1) << 31);
}

hipError_t launch_ssd_chunked(const SSDArgs &a, hipStream_t stream) {
    if (a.chunk == 64) return launch_by_n<64>(a, stream);
    if (a.chunk == 128) return launch_by_n<128>(a, stream);
    return launch_by_n<256>(a, stream);
}

}  // namespace mssm
