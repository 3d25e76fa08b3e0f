// ssd_chunked.hip -- Mamba-2 scalar-decay (SSD) forward in the chunked matrix
// form on the gfx950 matrix cores (v_mfma_f32_32x32x16_bf16), parallel over
// chunks.
//
// Per batch b and head h, with dl_t = softplus(dt_t + dt_bias[h]) and the log
// decay l_t = dl_t A[h] ("Mamba状态空间模型的硬件感知推理优化" (ybb.press)
// section 4: one scalar decay per step and head; section 6.2: cumulative
// products taken in log space), the sequence is cut into chunks of Q steps.
// With cum_t the inclusive sum of l over the chunk up to t and h_in the state
// entering the chunk:
//
//   S[p,n]      = sum_s exp(cum_end - cum_s) dl_s x_s[p] B_s[n]      (chunk state)
//   h_out       = exp(cum_end) h_in + S                                (state pass)
//   Y_diag[t,p] = sum_{s<=t} (C_t . B_s) exp(cum_t - cum_s) dl_s x_s[p]
//   Y_off[t,p]  = exp(cum_t) sum_n C_t[n] h_in[p,n]
//   y[t,p]      = (Y_diag + Y_off + D[h] x_t[p]) silu(z[t,p])   (gate optional)
//
// which is the recurrence S_t = a_t S_{t-1} + dl_t x_t B_t^T, y = C_t S_t +
// D x_t unrolled over a chunk (the cumulative-product closed form of the
// same ybb.press section; its chunk-by-chunk state carry is section 5).
//
// Three kernels, so that every chunk is worked on at once:
//   1. ssd_state_kernel: the chunk state S as a matrix-core product
//      (x * weight)^T B over the chunk's steps, and the chunk's total log2
//      decay;
//   2. ssd_pass_kernel: walks the chunks of each (batch, head) in order,
//      elementwise over the P x N state and starting from the initial state
//      (zero unless given), replacing each chunk state by the state entering
//      that chunk and writing h_last;
//   3. ssd_output_kernel: the outputs, computed transposed
//      (Y^T = X^T M^T + H C^T) so that each lane owns one step t: the decay
//      factors become per-lane scalars and each lane stores four consecutive
//      head-dimension values at once.
// Kernels 1 and 3 give each workgroup one (batch, chunk) and a run of heads
// of one B / C group: B (and C) of the chunk are staged once and serve every
// head of the run, and the next head's x rows are prefetched into registers
// while the current head is computed.
// Products whose operands are not exact bf16 values (x * weight, the masked
// decay matrix, the carried state) use a two-term bf16 split (hi + lo), so
// each product carries about 16 significant bits; accumulation is float32.
#include <type_traits>

#include "device_math.h"
#include "internal.h"

namespace mssm {
namespace {

typedef __bf16 bf8 __attribute__((ext_vector_type(8)));
typedef float f16x __attribute__((ext_vector_type(16)));

constexpr int kPG = 64;     // head-dimension columns per workgroup (two 32-wide tiles)

__device__ __forceinline__ f16x mfma(bf8 a, bf8 b, f16x c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f16x zero16() {
    f16x z;
#pragma unroll
    for (int v = 0; v < 16; ++v) z[v] = 0.0f;
    return z;
}

// Two floats rounded to bf16 (nearest even), packed low half first.
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
    const bf2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
    return __builtin_bit_cast(uint32_t, v);
}
// Two-term split of two floats: hi = bf16(v), lo = bf16(v - hi).
__device__ __forceinline__ void split2(float a, float b, uint32_t &hi, uint32_t &lo) {
    hi = pack2(a, b);
    lo = pack2(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xffff0000u));
}

// Eight consecutive bf16 of row t starting at column c8 of a row-major slice
// with row stride `stride`; zero past the last row or column.  Out-of-range
// reads are redirected to element 0 (always valid) and discarded, so the
// load needs no branch.  VEC: rows 16-byte aligned and cols % 8 == 0.
// Element offsets within a slice fit in 31 bits (checked by the launcher).
//
// Masks are applied with a bitwise AND on a mask the optimiser cannot see
// through: a select between a freshly loaded value and zero is turned into a
// branch around the load that waits for it, which serialises loads that
// should all be in flight together.
__device__ __forceinline__ uint32_t opaque_mask(bool ok) {
    uint32_t m = ok ? ~0u : 0u;
    asm("" : "+v"(m));
    return m;
}
__device__ __forceinline__ uint4 and4(uint4 v, uint32_t m) {
    return make_uint4(v.x & m, v.y & m, v.z & m, v.w & m);
}

// The same without the mask applied: the load is issued at a clamped index
// and m receives the mask for and4, so a prefetch stays in flight until the
// value is used.
template <bool VEC>
__device__ __forceinline__ uint4 load_row8_raw(const uint16_t *base, int t, int c8, int rows,
                                               int cols, int stride, uint32_t &m);

template <bool VEC>
__device__ __forceinline__ uint4 load_row8(const uint16_t *base, int t, int c8, int rows, int cols,
                                           int stride) {
    uint32_t m;
    const uint4 v = load_row8_raw<VEC>(base, t, c8, rows, cols, stride, m);
    return VEC ? and4(v, m) : v;
}

template <bool VEC>
__device__ __forceinline__ uint4 load_row8_raw(const uint16_t *base, int t, int c8, int rows,
                                               int cols, int stride, uint32_t &m) {
    const bool okt = t < rows;
    if (VEC) {
        const bool ok = okt && c8 < cols;
        const uint32_t i = ok ? static_cast<uint32_t>(t) * static_cast<uint32_t>(stride) + c8 : 0u;
        m = opaque_mask(ok);
        return *reinterpret_cast<const uint4 *>(base + i);
    }
    m = ~0u;
    uint16_t e[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        const bool ok = okt && c8 + r < cols;
        const uint32_t i = ok ? static_cast<uint32_t>(t) * static_cast<uint32_t>(stride) + c8 + r : 0u;
        const uint16_t w = base[i];
        e[r] = ok ? w : 0;
    }
    uint4 v;
    __builtin_memcpy(&v, e, 16);
    return v;
}

__device__ __forceinline__ float bits_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bits_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

struct Geom {
    int L, H, P, N, G, nch, npg;
};

// Work item of the state and output kernels: one (batch, chunk) and a run of
// heads that read the same B / C group, so B and C are staged once and reused
// by every head of the run; within a run, item i covers head h0 + i / npg and
// head-dimension slice i % npg.
struct Run {
    int64_t b;
    int c, h0, items, grp;
};

__device__ __forceinline__ Run decode_run(const Geom &g, int runs_per_chunk, int heads_per_run) {
    int64_t id = blockIdx.x;
    const int r = static_cast<int>(id % runs_per_chunk);
    id /= runs_per_chunk;
    Run run;
    run.c = static_cast<int>(id % g.nch);
    run.b = id / g.nch;
    run.h0 = r * heads_per_run;
    const int h1 = min(g.H, run.h0 + heads_per_run);
    run.items = (h1 - run.h0) * g.npg;
    run.grp = run.h0 / (g.H / g.G);
    return run;
}

// ---------------------------------------------------------------------------
// 1. chunk states
// ---------------------------------------------------------------------------
// Threads of the chunk-state kernel: eight waves (two per SIMD, so one
// wave's matrix-core work overlaps the other's staging) when the chunk has
// enough steps to give each thread a unit of x.
template <int Q>
constexpr int state_threads() { return Q >= 128 ? 512 : 256; }

// Row pitches (elements) of the transposed tiles.  B^T rows are read as
// 16-byte pieces (pitch a multiple of 8).  The x tiles are written as 4-byte
// step pairs by groups of 8 lanes whose rows lie 8 apart, and read as 8-byte
// pieces: a pitch of Q + 4 (an odd number of 8-byte pieces) spreads those
// 8 rows over 4 bank groups instead of 2.
template <int Q, int NP>
struct __align__(16) StateSmem {
    static constexpr int XP = Q + 8;     // B^T row pitch
    static constexpr int XQ = Q + 4;     // (x w)^T row pitch
    uint16_t BT[NP * XP];                // B^T of the chunk
    uint16_t Xh[kPG * XQ], Xl[kPG * XQ]; // (x * weight)^T, bf16 high / low parts
    float cum[Q], dl[Q], wsum[8];
};

// Eight consecutive bf16 of an LDS row as two 8-byte reads (8-byte aligned).
__device__ __forceinline__ bf8 lds_read8(const uint16_t *p) {
    const uint2 a = *reinterpret_cast<const uint2 *>(p);
    const uint2 b = *reinterpret_cast<const uint2 *>(p + 4);
    return __builtin_bit_cast(bf8, make_uint4(a.x, a.y, b.x, b.y));
}

// x rows of one item, prefetched into registers by NT threads: unit u of
// this thread covers steps 2 s2, 2 s2 + 1 and head-dimension columns
// p8 .. p8 + 7.
template <int Q, int NT>
struct XRegs {
    static constexpr int U = (Q / 2) * (kPG / 8) / NT;
    static_assert(U >= 1 && U * NT == (Q / 2) * (kPG / 8), "every thread holds whole units");
    uint4 v[U][2];       // raw loads; apply the masks m with and4 before use
    uint32_t m[U][2];
    float dt;
};

template <int Q, int NT, bool VEC>
__device__ __forceinline__ void load_x(XRegs<Q, NT> &r, const uint16_t *x, const uint16_t *dt,
                                       const Geom &g, const Run &run, int item) {
    const int tid = threadIdx.x;
    const int hh = run.h0 + item / g.npg, pbase = (item % g.npg) * kPG;
    const int t0 = run.c * Q;
    const int rowX = g.H * g.P;
    const uint16_t *xg = x + run.b * g.L * static_cast<int64_t>(rowX) + hh * g.P + pbase;
#pragma unroll
    for (int k = 0; k < XRegs<Q, NT>::U; ++k) {
        const int u = tid + NT * k;
        const int s2 = 2 * (u / (kPG / 8)), p8 = (u % (kPG / 8)) * 8;
        r.v[k][0] = load_row8_raw<VEC>(xg, t0 + s2, p8, g.L, g.P - pbase, rowX, r.m[k][0]);
        r.v[k][1] = load_row8_raw<VEC>(xg, t0 + s2 + 1, p8, g.L, g.P - pbase, rowX, r.m[k][1]);
    }
    const int t = t0 + (tid < Q ? tid : 0);
    r.dt = bf16_to_f32(dt[run.b * g.L * static_cast<int64_t>(g.H) + (t < g.L ? t : g.L - 1) * g.H + hh]);
}

// dl and the inclusive sum of the log2 decay over the chunk's Q steps from a
// prefetched raw dt value (thread s < Q holds step s; s_wsum holds one float
// per wave of the workgroup).  Ends with a barrier.
template <int Q>
__device__ void chunk_decay_from(float dr, int t0, int L, float A2, float bias,
                                 float *s_cum, float *s_dl, float *s_wsum) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    float dlv = 0.0f, ell = 0.0f;
    if (tid < Q && t0 + tid < L) {
        dlv = softplus(dr + bias);
        ell = dlv * A2;
    }
    float sc = ell;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float o = __shfl_up(sc, off, 64);
        if (lane >= off) sc += o;
    }
    if (lane == 63) s_wsum[wave] = sc;
    __syncthreads();
    if (tid < Q) {
        float base = 0.0f;
        for (int w2 = 0; w2 < wave; ++w2) base += s_wsum[w2];
        s_cum[tid] = sc + base;
        s_dl[tid] = dlv;
    }
    __syncthreads();
}

template <int Q, int NP, bool VEC>
__global__ __launch_bounds__(state_threads<Q>()) void ssd_state_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ dt,
    const float *__restrict__ dt_bias, const float *__restrict__ A,
    const uint16_t *__restrict__ Bm, float *__restrict__ S, float *__restrict__ ce, Geom g,
    int runs_per_chunk, int heads_per_run) {
    using Sm = StateSmem<Q, NP>;
    constexpr int XP = Sm::XP, XQ = Sm::XQ;
    constexpr int NT = state_threads<Q>();
    constexpr int kWaves = NT / 64;
    // output tiles of 32 x 32: eight waves take one each (pt = wave & 1,
    // nt = wave / 2), four waves take both head-dimension tiles of one nt
    constexpr int kPtPerWave = kWaves == 8 ? 1 : 2;
    __shared__ Sm sm;
    const int tid = threadIdx.x;
    // wave index as a scalar, so control flow that depends on it stays uniform
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l32 = lane & 31, half = lane >> 5;
    const Run run = decode_run(g, runs_per_chunk, heads_per_run);
    const int t0 = run.c * Q;
    const int rowBC = g.G * g.N;
    const uint16_t *Bg = Bm + run.b * g.L * static_cast<int64_t>(rowBC) + run.grp * g.N;

    XRegs<Q, NT> xr;
    load_x<Q, NT, VEC>(xr, x, dt, g, run, 0);
    // B^T of the chunk, exact bf16 values re-packed as step pairs
    constexpr int kTotBT = (Q / 2) * (NP / 8);
#pragma unroll
    for (int k = 0; k < (kTotBT + NT - 1) / NT; ++k) {
        const int u = tid + NT * k;
        if (kTotBT % NT != 0 && u >= kTotBT) break;
        const int s2 = 2 * (u / (NP / 8)), n8 = (u % (NP / 8)) * 8;
        const uint4 v0 = load_row8<VEC>(Bg, t0 + s2, n8, g.L, g.N, rowBC);
        const uint4 v1 = load_row8<VEC>(Bg, t0 + s2 + 1, n8, g.L, g.N, rowBC);
        const uint32_t a[4] = {v0.x, v0.y, v0.z, v0.w}, e[4] = {v1.x, v1.y, v1.z, v1.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            *reinterpret_cast<uint32_t *>(&sm.BT[(n8 + 2 * r) * XP + s2]) = (a[r] & 0xffffu) | (e[r] << 16);
            *reinterpret_cast<uint32_t *>(&sm.BT[(n8 + 2 * r + 1) * XP + s2]) = (a[r] >> 16) | (e[r] & 0xffff0000u);
        }
    }
    const int nt = kWaves == 8 ? wave >> 1 : wave;     // 32-wide tile of the state index
    const int pt0 = kWaves == 8 ? wave & 1 : 0;        // first 32-wide head-dimension tile
#pragma unroll 1
    for (int item = 0; item < run.items; ++item) {
        const int hh = run.h0 + item / g.npg, pbase = (item % g.npg) * kPG;
        const int pcols = g.P - pbase;
        // (the decay scan starts with a barrier: the previous item's MFMA
        // reads of Xh / Xl are done before they are overwritten below)
        __syncthreads();
        chunk_decay_from<Q>(xr.dt, t0, g.L, A[hh] * kLog2e, dt_bias ? dt_bias[hh] : 0.0f, sm.cum,
                            sm.dl, sm.wsum);
        const float cum_end = sm.cum[Q - 1];
        // (x * w)^T with w_s = 2^(cum_end - cum_s) dl_s, split into bf16 parts
#pragma unroll
        for (int k = 0; k < XRegs<Q, NT>::U; ++k) {
            const int u = tid + NT * k;
            const int s2 = 2 * (u / (kPG / 8)), p8 = (u % (kPG / 8)) * 8;
            const float w0 = fast_exp2(cum_end - sm.cum[s2]) * sm.dl[s2];
            const float w1 = fast_exp2(cum_end - sm.cum[s2 + 1]) * sm.dl[s2 + 1];
            const uint4 v0 = and4(xr.v[k][0], xr.m[k][0]), v1 = and4(xr.v[k][1], xr.m[k][1]);
            const uint32_t a[4] = {v0.x, v0.y, v0.z, v0.w}, e[4] = {v1.x, v1.y, v1.z, v1.w};
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                uint32_t hi, lo;
                split2(bits_lo(a[r]) * w0, bits_lo(e[r]) * w1, hi, lo);
                *reinterpret_cast<uint32_t *>(&sm.Xh[(p8 + 2 * r) * XQ + s2]) = hi;
                *reinterpret_cast<uint32_t *>(&sm.Xl[(p8 + 2 * r) * XQ + s2]) = lo;
                split2(bits_hi(a[r]) * w0, bits_hi(e[r]) * w1, hi, lo);
                *reinterpret_cast<uint32_t *>(&sm.Xh[(p8 + 2 * r + 1) * XQ + s2]) = hi;
                *reinterpret_cast<uint32_t *>(&sm.Xl[(p8 + 2 * r + 1) * XQ + s2]) = lo;
            }
        }
        __syncthreads();
        // next item's x (the last item re-reads its own rows; unused)
        load_x<Q, NT, VEC>(xr, x, dt, g, run, item + 1 < run.items ? item + 1 : item);
        // S[p][n] = sum_s (x w)^T[p][s] B^T[n][s]: A rows p, B operand columns n
        f16x acc[kPtPerWave];
#pragma unroll
        for (int i = 0; i < kPtPerWave; ++i) acc[i] = zero16();
        if (nt * 32 < NP) {
#pragma unroll 2
            for (int kq = 0; kq < Q / 16; ++kq) {
                const int s8 = 16 * kq + 8 * half;
                const bf8 bb = *reinterpret_cast<const bf8 *>(&sm.BT[(nt * 32 + l32) * XP + s8]);
#pragma unroll
                for (int i = 0; i < kPtPerWave; ++i) {
                    const int pt = pt0 + i;
                    const bf8 ah = lds_read8(&sm.Xh[(pt * 32 + l32) * XQ + s8]);
                    const bf8 al = lds_read8(&sm.Xl[(pt * 32 + l32) * XQ + s8]);
                    acc[i] = mfma(ah, bb, acc[i]);
                    acc[i] = mfma(al, bb, acc[i]);
                }
            }
            // lane (column n, half) holds S[p(v)][n], p(v) = 8 (v / 4) + 4 half + v % 4
            const int n = nt * 32 + l32;
            if (n < g.N) {
                float *Sg = S + ((run.b * g.nch + run.c) * g.H + hh) * static_cast<int64_t>(g.P) * g.N;
#pragma unroll
                for (int i = 0; i < kPtPerWave; ++i)
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int p = (pt0 + i) * 32 + 8 * (v / 4) + 4 * half + (v % 4);
                        if (p < pcols) Sg[static_cast<int64_t>(pbase + p) * g.N + n] = acc[i][v];
                    }
            }
        }
        if (pbase == 0 && tid == 0) ce[(run.b * g.nch + run.c) * g.H + hh] = cum_end;
    }
}

// ---------------------------------------------------------------------------
// 2. state pass: S[chunk] <- state entering the chunk; h_last <- final state
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void ssd_pass_kernel(float *__restrict__ S,
                                                       const float *__restrict__ ce,
                                                       const float *h0, float *h_last, Geom g,
                                                       int blocks_per_head) {
    const int64_t PN = static_cast<int64_t>(g.P) * g.N;
    const int64_t bh = blockIdx.x / blocks_per_head;         // batch * H + head
    const int64_t e = static_cast<int64_t>(blockIdx.x % blocks_per_head) * 256 + threadIdx.x;
    if (e >= PN) return;
    const int64_t b = bh / g.H, hh = bh % g.H;
    float h = h0 ? h0[bh * PN + e] : 0.0f;   // state entering the first chunk
    constexpr int U = 4;    // chunks whose states are loaded ahead of the chain
    int c = 0;
    for (; c + U <= g.nch; c += U) {
        float s[U], a[U];
        int64_t idx[U];
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int64_t bc = (b * g.nch + c + k) * g.H + hh;
            idx[k] = bc * PN + e;
            s[k] = S[idx[k]];
            a[k] = fast_exp2(ce[bc]);
        }
#pragma unroll
        for (int k = 0; k < U; ++k) {
            S[idx[k]] = h;
            h = fmaf(a[k], h, s[k]);
        }
    }
    for (; c < g.nch; ++c) {
        const int64_t bc = (b * g.nch + c) * g.H + hh;
        const float s = S[bc * PN + e];
        S[bc * PN + e] = h;
        h = fmaf(fast_exp2(ce[bc]), h, s);
    }
    if (h_last) h_last[bh * PN + e] = h;
}

// ---------------------------------------------------------------------------
// 3. outputs
// ---------------------------------------------------------------------------
template <int Q, int NP>
struct __align__(16) OutSmem {
    static constexpr int BP = NP + 8;    // B row pitch (elements)
    static constexpr int XP = Q + 4;     // x^T row pitch (8-byte reads; see StateSmem)
    static constexpr int HP = NP + 8;    // h_in row pitch
    uint16_t B[Q * BP];                  // B of the chunk, exact bf16
    uint16_t XT[kPG * XP];               // x^T, exact bf16
    uint16_t Hh[kPG * HP], Hl[kPG * HP]; // state entering the chunk, bf16 parts
    float cum[Q], dl[Q];
    float fs[Q];   // 2^(cum at the end of s's 32-step block - cum_s) dl_s
    float wsum[4];
};

// h_in of one item prefetched into registers: unit u covers row p, columns
// n2, n2 + 1 of the 64 x NP tile.
template <int NP>
struct HRegs {
    static constexpr int U = kPG * (NP / 2) / 256;
    float2 v[U];
};

template <int Q, int NP>
__device__ __forceinline__ void load_h(HRegs<NP> &r, const float *Hin, const Geom &g, const Run &run,
                                       int item) {
    const int tid = threadIdx.x;
    const int hh = run.h0 + item / g.npg, pbase = (item % g.npg) * kPG;
    const int pcols = g.P - pbase;
    const float *Hg = Hin + ((run.b * g.nch + run.c) * g.H + hh) * static_cast<int64_t>(g.P) * g.N;
    // Every load is issued first, at an index clamped into the slice, and the
    // masks are applied afterwards with selects: a load guarded by its mask
    // is placed in a branch that waits for it, which serialises the loads.
    float raw[HRegs<NP>::U][2];
#pragma unroll
    for (int k = 0; k < HRegs<NP>::U; ++k) {
        const int u = tid + 256 * k;
        const int p = u / (NP / 2), n2 = (u % (NP / 2)) * 2;
        const int64_t base = static_cast<int64_t>(pbase + (p < pcols ? p : 0)) * g.N;
        raw[k][0] = Hg[base + (n2 < g.N ? n2 : 0)];
        raw[k][1] = Hg[base + (n2 + 1 < g.N ? n2 + 1 : 0)];
    }
#pragma unroll
    for (int k = 0; k < HRegs<NP>::U; ++k) {
        const int u = tid + 256 * k;
        const int p = u / (NP / 2), n2 = (u % (NP / 2)) * 2;
        const bool okp = p < pcols;
        const bool m0 = okp & (n2 < g.N), m1 = okp & (n2 + 1 < g.N);
        r.v[k] = make_float2(m0 ? raw[k][0] : 0.0f, m1 ? raw[k][1] : 0.0f);
    }
}

template <int Q, int NP, bool VEC, bool GATE>
__global__ __launch_bounds__(256) void ssd_output_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ dt,
    const float *__restrict__ dt_bias, const float *__restrict__ A,
    const uint16_t *__restrict__ Bm, const uint16_t *__restrict__ Cm,
    const float *__restrict__ Dskip, const uint16_t *__restrict__ z, const float *__restrict__ Hin,
    uint16_t *__restrict__ y, Geom g, int runs_per_chunk, int heads_per_run) {
    using Sm = OutSmem<Q, NP>;
    constexpr int BP = Sm::BP, XP = Sm::XP, HP = Sm::HP;
    constexpr int NT = Q / 32;          // 32-step blocks per chunk
    constexpr int KN = NP / 16;         // K steps over the state index
    __shared__ Sm sm;
    const int tid = threadIdx.x;
    // wave index as a scalar, so control flow that depends on it stays uniform
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l32 = lane & 31, half = lane >> 5;
    const Run run = decode_run(g, runs_per_chunk, heads_per_run);
    const int t0 = run.c * Q;
    const int rowX = g.H * g.P;
    const int rowBC = g.G * g.N;
    const uint16_t *Bg = Bm + run.b * g.L * static_cast<int64_t>(rowBC) + run.grp * g.N;
    const uint16_t *Cg = Cm + run.b * g.L * static_cast<int64_t>(rowBC) + run.grp * g.N;

    XRegs<Q, 256> xr;
    load_x<Q, 256, VEC>(xr, x, dt, g, run, 0);
    // B of the chunk (rows s), shared by every head of the run
    static_assert(Q * (NP / 8) % 256 == 0, "whole units of B per thread");
#pragma unroll
    for (int k = 0; k < Q * (NP / 8) / 256; ++k) {
        const int u = tid + 256 * k;
        const int s = u / (NP / 8), n8 = (u % (NP / 8)) * 8;
        *reinterpret_cast<uint4 *>(&sm.B[s * BP + n8]) = load_row8<VEC>(Bg, t0 + s, n8, g.L, g.N, rowBC);
    }
    // Each wave owns the 32-step blocks tb = wave and NT-1-wave (balanced
    // causal work); with fewer than 8 blocks only the first NT/2 waves work.
    // C_t fragments of those blocks: row t, state indices 16 jn + 8 half ...
    const bool active = 2 * wave < NT;
    bf8 cf[2][KN];
#pragma unroll
    for (int which = 0; which < 2; ++which) {
        const int tb = which == 0 ? wave : NT - 1 - wave;
#pragma unroll
        for (int jn = 0; jn < KN; ++jn)
            cf[which][jn] = __builtin_bit_cast(
                bf8, load_row8<VEC>(Cg, t0 + (active ? tb : 0) * 32 + l32, 16 * jn + 8 * half, g.L, g.N, rowBC));
    }

#pragma unroll 1
    for (int item = 0; item < run.items; ++item) {
        const int hh = run.h0 + item / g.npg, pbase = (item % g.npg) * kPG;
        const int pcols = g.P - pbase;
        const float skip = Dskip ? Dskip[hh] : 0.0f;
        uint16_t *yg = y + run.b * g.L * static_cast<int64_t>(rowX) + hh * g.P + pbase;
        const uint16_t *zg = GATE ? z + run.b * g.L * static_cast<int64_t>(rowX) + hh * g.P + pbase : nullptr;
        __syncthreads();   // the previous item's LDS reads are done
        // state entering the chunk; its loads overlap the decay scan
        HRegs<NP> hr;
        load_h<Q, NP>(hr, Hin, g, run, item);
        chunk_decay_from<Q>(xr.dt, t0, g.L, A[hh] * kLog2e, dt_bias ? dt_bias[hh] : 0.0f, sm.cum,
                            sm.dl, sm.wsum);
        if (tid < Q) sm.fs[tid] = fast_exp2(sm.cum[tid | 31] - sm.cum[tid]) * sm.dl[tid];
        // x^T as step pairs; h_in split into bf16 parts
#pragma unroll
        for (int k = 0; k < XRegs<Q, 256>::U; ++k) {
            const int u = tid + 256 * k;
            const int s2 = 2 * (u / (kPG / 8)), p8 = (u % (kPG / 8)) * 8;
            const uint4 v0 = and4(xr.v[k][0], xr.m[k][0]), v1 = and4(xr.v[k][1], xr.m[k][1]);
            const uint32_t a[4] = {v0.x, v0.y, v0.z, v0.w}, e[4] = {v1.x, v1.y, v1.z, v1.w};
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                *reinterpret_cast<uint32_t *>(&sm.XT[(p8 + 2 * r) * XP + s2]) = (a[r] & 0xffffu) | (e[r] << 16);
                *reinterpret_cast<uint32_t *>(&sm.XT[(p8 + 2 * r + 1) * XP + s2]) = (a[r] >> 16) | (e[r] & 0xffff0000u);
            }
        }
#pragma unroll
        for (int k = 0; k < HRegs<NP>::U; ++k) {
            const int u = tid + 256 * k;
            const int p = u / (NP / 2), n2 = (u % (NP / 2)) * 2;
            uint32_t hi, lo;
            split2(hr.v[k].x, hr.v[k].y, hi, lo);
            *reinterpret_cast<uint32_t *>(&sm.Hh[p * HP + n2]) = hi;
            *reinterpret_cast<uint32_t *>(&sm.Hl[p * HP + n2]) = lo;
        }
        __syncthreads();
        // next item's x (the last item re-reads its own; unused)
        load_x<Q, 256, VEC>(xr, x, dt, g, run, item + 1 < run.items ? item + 1 : item);
        if (!active) continue;

        // Output tiles Y^T[p][t]: lane (column t, half) holds rows
        // p(v) = 8 (v / 4) + 4 half + v % 4.
#pragma unroll
        for (int which = 0; which < 2; ++which) {
            const int tb = which == 0 ? wave : NT - 1 - wave;
            const int tl = tb * 32 + l32;            // this lane's step within the chunk
            const float cum_t = sm.cum[tl];
            f16x yd[2] = {zero16(), zero16()};
            // G'[s][t] = B_s . C_t of source block sb: A operand rows s of B.
            // The block's LDS operands are all read up front, so their
            // latencies overlap one another and the matrix-core work instead
            // of being exposed one product at a time.
            auto gblock = [&](int sb) {
                bf8 ab[KN];
#pragma unroll
                for (int jn = 0; jn < KN; ++jn)
                    ab[jn] = *reinterpret_cast<const bf8 *>(&sm.B[(sb * 32 + l32) * BP + 16 * jn + 8 * half]);
                f16x g = zero16();
#pragma unroll
                for (int jn = 0; jn < KN; ++jn) g = mfma(ab[jn], cf[which][jn], g);
                return g;
            };
            // One source block's contribution: build the masked decay tile from
            // G' and add x^T M^T to the output tile.  DIAG (a compile-time tag)
            // selects the diagonal block sb = tb.
            auto mstep = [&](int sb, const f16x &gacc, auto diag_tag) {
                constexpr bool DIAG = decltype(diag_tag)::value;
                // x^T operands of the block: A operand row p reads x at
                // s(8 kk + 0..3) and s(8 kk + 4..7), s(v) as below
                bf8 xa[2][2];
#pragma unroll
                for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                    for (int pt = 0; pt < 2; ++pt) {
                        const uint16_t *xp = &sm.XT[(pt * 32 + l32) * XP + sb * 32 + 16 * kk + 4 * half];
                        const uint2 lo4 = *reinterpret_cast<const uint2 *>(xp);
                        const uint2 hi4 = *reinterpret_cast<const uint2 *>(xp + 8);
                        xa[kk][pt] = __builtin_bit_cast(bf8, make_uint4(lo4.x, lo4.y, hi4.x, hi4.y));
                    }
                // M[t][s] = G'[s][t] 2^(cum_t - cum_s) dl_s for s <= t (else 0),
                // at s(v) = 32 sb + 8 (v / 4) + 4 half + v % 4, plus the skip
                // weight D on the diagonal s = t, so the product with x^T also
                // forms D x_t.  Off the diagonal block the decay factors as
                // 2^(cum_t - cb) fs[s], cb the cum at the end of block sb, both
                // factors <= 1.
                float mval[16];
                if constexpr (!DIAG) {
                    const float et = fast_exp2(cum_t - sm.cum[sb * 32 + 31]);
#pragma unroll
                    for (int v = 0; v < 16; ++v)
                        mval[v] = gacc[v] * (et * sm.fs[sb * 32 + 8 * (v / 4) + 4 * half + (v % 4)]);
                } else {
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int sl = sb * 32 + 8 * (v / 4) + 4 * half + (v % 4);
                        const float mv = gacc[v] * fast_exp2(cum_t - sm.cum[sl]) * sm.dl[sl];
                        mval[v] = sl < tl ? mv : (sl == tl ? mv + skip : 0.0f);
                    }
                }
                uint32_t mh[8], ml[8];
#pragma unroll
                for (int v = 0; v < 16; v += 2) split2(mval[v], mval[v + 1], mh[v / 2], ml[v / 2]);
                // Y^T[p][t] += sum_s x^T[p][s] M[t][s], K slot order s(v) as above
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    const bf8 bh = __builtin_bit_cast(bf8, make_uint4(mh[4 * kk], mh[4 * kk + 1], mh[4 * kk + 2], mh[4 * kk + 3]));
                    const bf8 bl = __builtin_bit_cast(bf8, make_uint4(ml[4 * kk], ml[4 * kk + 1], ml[4 * kk + 2], ml[4 * kk + 3]));
#pragma unroll
                    for (int pt = 0; pt < 2; ++pt) {
                        yd[pt] = mfma(xa[kk][pt], bh, yd[pt]);
                        yd[pt] = mfma(xa[kk][pt], bl, yd[pt]);
                    }
                }
            };
            // Two-stage pipeline over the blocks below the diagonal: block
            // sb + 1's G' products are issued in the same straight-line body as
            // block sb's decay tile and output products, so the matrix cores
            // work while the vector units build the tile.  The diagonal block,
            // whose tile needs per-element exponentials and the causal mask,
            // follows the loop.
            f16x gnext = gblock(0);
#pragma unroll 1
            for (int sb = 0; sb < tb; ++sb) {
                const f16x gacc = gnext;
                gnext = gblock(sb + 1);
                mstep(sb, gacc, std::false_type{});
            }
            mstep(tb, gnext, std::true_type{});
            // Y_off^T[p][t] = sum_n h_in[p][n] C_t[n]; y = (Y_diag (with D x) +
            // 2^cum_t Y_off) * silu(z) when gated
            const float et = fast_exp2(cum_t);
            const int t = t0 + tl;
            const uint32_t row = static_cast<uint32_t>(t < g.L ? t : 0) * static_cast<uint32_t>(rowX);
            // Both head-dimension tiles, with the hi and lo parts of h_in in
            // accumulators of their own: four independent chains of matrix-core
            // products instead of one dependent chain per tile.  (Rows of a
            // tile past the slice's columns compute values that are not
            // stored.)
            f16x yo2[2][2] = {{zero16(), zero16()}, {zero16(), zero16()}};
#pragma unroll
            for (int jn = 0; jn < KN; ++jn) {
                const int n8 = 16 * jn + 8 * half;
#pragma unroll
                for (int pt = 0; pt < 2; ++pt) {
                    const bf8 ah = *reinterpret_cast<const bf8 *>(&sm.Hh[(pt * 32 + l32) * HP + n8]);
                    const bf8 al = *reinterpret_cast<const bf8 *>(&sm.Hl[(pt * 32 + l32) * HP + n8]);
                    yo2[pt][0] = mfma(ah, cf[which][jn], yo2[pt][0]);
                    yo2[pt][1] = mfma(al, cf[which][jn], yo2[pt][1]);
                }
            }
#pragma unroll
            for (int pt = 0; pt < 2; ++pt) {
                if (pt * 32 >= pcols) break;
                // gate values of this lane's step for the tile's 16 head-dimension
                // columns (vector path; the element path loads them at the
                // stores)
                uint2 zq[4];
                if (VEC && GATE) {
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4) {
                        const int p = pt * 32 + 8 * q4 + 4 * half;
                        zq[q4] = p < pcols ? *reinterpret_cast<const uint2 *>(zg + row + p) : make_uint2(0, 0);
                    }
                }
                const f16x yo = yo2[pt][0] + yo2[pt][1];
                if (t < g.L) {
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4) {
                        // four consecutive p = pt*32 + 8 q4 + 4 half + 0..3
                        const int p = pt * 32 + 8 * q4 + 4 * half;
                        float yv[4];
#pragma unroll
                        for (int k = 0; k < 4; ++k) yv[k] = fmaf(et, yo[4 * q4 + k], yd[pt][4 * q4 + k]);
                        if (GATE) {
                            float zf[4];
                            if (VEC) {
                                zf[0] = bits_lo(zq[q4].x);
                                zf[1] = bits_hi(zq[q4].x);
                                zf[2] = bits_lo(zq[q4].y);
                                zf[3] = bits_hi(zq[q4].y);
                            } else {
#pragma unroll
                                for (int k = 0; k < 4; ++k)
                                    zf[k] = p + k < pcols ? bf16_to_f32(zg[row + p + k]) : 0.0f;
                            }
#pragma unroll
                            for (int k = 0; k < 4; ++k) yv[k] *= silu(zf[k]);
                        }
                        if (VEC) {
                            if (p < pcols)
                                *reinterpret_cast<uint2 *>(yg + row + p) =
                                    make_uint2(pack2(yv[0], yv[1]), pack2(yv[2], yv[3]));
                        } else {
#pragma unroll
                            for (int k = 0; k < 4; ++k)
                                if (p + k < pcols) yg[row + p + k] = f32_to_bf16(yv[k]);
                        }
                    }
                }
            }
        }
    }
}

// Heads per run: runs never straddle a B / C group, and the grid keeps at
// least two runs per compute unit when the problem allows.
int heads_per_run(const SSDArgs &a, int64_t nch) {
    const int hpg = static_cast<int>(a.H / a.G);
    int best = 1;
    for (int d = 1; d <= hpg; ++d) {
        if (hpg % d) continue;
        if (a.batch * nch * a.G * (hpg / d) >= 512) best = d;
    }
    return best;
}

template <int Q, int NP>
hipError_t launch_typed(const SSDArgs &a, hipStream_t stream) {
    Geom g;
    g.L = static_cast<int>(a.L);
    g.H = static_cast<int>(a.H);
    g.P = static_cast<int>(a.P);
    g.N = static_cast<int>(a.N);
    g.G = static_cast<int>(a.G);
    g.nch = static_cast<int>((a.L + Q - 1) / Q);
    g.npg = static_cast<int>((a.P + kPG - 1) / kPG);
    auto aligned = [](const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
    const bool vecB = a.N % 8 == 0 && aligned(a.B) && aligned(a.C);
    const bool vecX = a.P % 8 == 0 && aligned(a.x) && aligned(a.y) && (!a.z || aligned(a.z));
    const int hpr = heads_per_run(a, g.nch);
    const int rpc = static_cast<int>((a.H + hpr - 1) / hpr);

    const int64_t chunks = a.batch * g.nch * a.H;
    const int64_t PN = a.P * a.N;
    const size_t s_bytes = static_cast<size_t>(chunks * PN) * sizeof(float);
    const size_t ce_bytes = static_cast<size_t>(chunks) * sizeof(float);
    void *mem = nullptr;
    hipError_t e = hipMallocAsync(&mem, s_bytes + ce_bytes, stream);
    if (e != hipSuccess) return e;
    float *S = static_cast<float *>(mem);
    float *ce = reinterpret_cast<float *>(static_cast<char *>(mem) + s_bytes);

    const auto *x = static_cast<const uint16_t *>(a.x);
    const auto *dt = static_cast<const uint16_t *>(a.dt);
    const auto *B = static_cast<const uint16_t *>(a.B);
    const auto *C = static_cast<const uint16_t *>(a.C);
    const auto *zz = static_cast<const uint16_t *>(a.z);
    const int64_t grid = a.batch * g.nch * rpc;
    const bool vec = vecB && vecX;
    constexpr int nts = state_threads<Q>();
    if (vec)
        hipLaunchKernelGGL((ssd_state_kernel<Q, NP, true>), dim3(static_cast<uint32_t>(grid)), dim3(nts), 0,
                           stream, x, dt, a.dt_bias, a.A, B, S, ce, g, rpc, hpr);
    else
        hipLaunchKernelGGL((ssd_state_kernel<Q, NP, false>), dim3(static_cast<uint32_t>(grid)), dim3(nts), 0,
                           stream, x, dt, a.dt_bias, a.A, B, S, ce, g, rpc, hpr);
    e = hipGetLastError();
    if (e == hipSuccess) {
        const int bph = static_cast<int>((PN + 255) / 256);
        hipLaunchKernelGGL(ssd_pass_kernel, dim3(static_cast<uint32_t>(a.batch * a.H * bph)),
                           dim3(256), 0, stream, S, ce, a.h0, a.h_last, g, bph);
        e = hipGetLastError();
    }
    if (e == hipSuccess) {
        decltype(&ssd_output_kernel<Q, NP, true, true>) kern;
        if (zz) kern = vec ? ssd_output_kernel<Q, NP, true, true> : ssd_output_kernel<Q, NP, false, true>;
        else kern = vec ? ssd_output_kernel<Q, NP, true, false> : ssd_output_kernel<Q, NP, false, false>;
        hipLaunchKernelGGL(kern, dim3(static_cast<uint32_t>(grid)), dim3(256), 0, stream, x, dt, a.dt_bias,
                           a.A, B, C, a.D, zz, S, static_cast<uint16_t *>(a.y), g, rpc, hpr);
        e = hipGetLastError();
    }
    const hipError_t ef = hipFreeAsync(mem, stream);
    return e != hipSuccess ? e : ef;
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
    const int64_t nch = (a.L + a.chunk - 1) / (a.chunk > 0 ? a.chunk : 1);
    // element offsets within one batch's x and B / C slices fit in 31 bits
    const int64_t lim = int64_t(1) << 31;
    if (a.L * a.H * a.P >= lim || a.L * a.G * a.N >= lim || a.L * a.H >= lim) return false;
    return a.io == IO_BF16 && a.N >= 1 && a.N <= 128 && a.P >= 1 &&
           (a.chunk == 64 || a.chunk == 128 || a.chunk == 256) &&
           a.batch * nch * a.H * ((a.P + kPG - 1) / kPG) < (int64_t(1) << 31) &&
           nch < (int64_t(1) << 30);
}

hipError_t launch_ssd_chunked(const SSDArgs &a, hipStream_t stream) {
    if (a.chunk == 64) return launch_by_n<64>(a, stream);
    if (a.chunk == 128) return launch_by_n<128>(a, stream);
    return launch_by_n<256>(a, stream);
}

}  // namespace mssm
