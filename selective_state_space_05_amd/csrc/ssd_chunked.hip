// ssd_chunked.hip -- Mamba-2 scalar-decay (SSD) forward in the chunked matrix
// form on the gfx950 matrix cores (v_mfma_f32_16x16x32_bf16), parallel over
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
//   y[t,p]      = (C_t . h_t[p,:] + D[h] x_t[p]) silu(z[t,p])   (gate optional)
//
// where h_t is the state after step t of the recurrence
// h_t = a_t h_{t-1} + dl_t x_t B_t^T started from h_in (the cumulative-product
// closed form of the same ybb.press section; its chunk-by-chunk state carry
// is section 5).
//
// Three kernels, so that every pair of consecutive chunks is worked on at
// once:
//   1. ssd_state_kernel: the state of each pair of chunks (2 m, 2 m + 1) from
//      zero, 2^(e_{2m+1}) S_{2m} + S_{2m+1} (e: a chunk's total log2 decay),
//      accumulated block by block of 32 steps as a matrix-core product
//      (x w)^T B, and the pair's total log2 decay; extra workgroups of the
//      same launch form the C . B Gram products within each 32-step block,
//      which depend on the group only;
//   2. ssd_pass_kernel: walks the pairs of each (batch, head) in order,
//      elementwise over the P x N state and starting from the initial state
//      (zero unless given), storing the state entering every pair (or every
//      other pair) over the aggregates already read, and writing h_last;
//   3. ssd_output_kernel: the outputs, walking the 32-step blocks of two or
//      four consecutive chunks from the state entering the first, with the
//      state carried in matrix-core accumulators; within a block the outputs
//      come from the state entering it and the block's own 32 x 32
//      decay-masked C B^T tile (the Gram products scaled by the decays).
// Two or four chunks rather than one per workgroup halve (or quarter) the
// chunk states written, passed and read again.  Both walks give each
// workgroup a 64-column slice of the head dimension and each of its four
// waves 16 columns, and stage a block's B, C and x in LDS (transposed where
// a product contracts over the steps) while the next block's rows are in
// flight.
// Products whose operands are not exact bf16 values (x * weight, the masked
// decay tile, the carried state) use a two-term bf16 split (hi + lo), so each
// product carries about 16 significant bits; accumulation is float32.
#include "device_math.h"
#include "internal.h"

namespace mssm {
namespace {

typedef __bf16 bf8 __attribute__((ext_vector_type(8)));

constexpr int kPG = 64;     // head-dimension columns per workgroup (four 16-wide wave slices)

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

typedef float f4x __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f4x mfma16(bf8 a, bf8 b, f4x c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f4x zero4() {
    f4x z = {0.0f, 0.0f, 0.0f, 0.0f};
    return z;
}
__device__ __forceinline__ bf8 cat8(uint2 a, uint2 b) {
    return __builtin_bit_cast(bf8, make_uint4(a.x, a.y, b.x, b.y));
}
// Column of step s in row r of a transposed (rows x 32 steps) LDS tile:
// steps are swizzled by 8 ((r / 16) mod 4), which keeps every aligned run of
// four steps contiguous, gives the 16 rows read together one swizzle, and
// spreads the step-pair writes of rows 8 apart (the staging pattern below)
// over distinct banks.
__device__ __forceinline__ int swz(int s, int r) { return s ^ (8 * ((r >> 4) & 3)); }
// Two floats rounded to bf16 (nearest even) and packed, low half first, as
// one instruction the optimiser cannot re-derive: the split below then
// widens the packed halves with a shift and a mask, six instructions per
// pair in all.
__device__ __forceinline__ uint32_t cvt_pk(float lo, float hi) {
    uint32_t r;
    asm("v_cvt_pk_bf16_f32 %0, %1, %2" : "=v"(r) : "v"(lo), "v"(hi));
    return r;
}
__device__ __forceinline__ void split_pk(float a, float b, uint32_t &hi, uint32_t &lo) {
    hi = cvt_pk(a, b);
    lo = cvt_pk(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xffff0000u));
}

// Buffer resources (gfx9 raw-buffer format word): a load at a byte offset
// at or past `bytes` returns zero, a store there is dropped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t brsrc(const void *base, int64_t bytes) {
    const int32_t n = static_cast<int32_t>(bytes < 0 ? 0 : (bytes > 0x7fffffff ? 0x7fffffff : bytes));
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, n, 0x00020000);
}
__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    return make_uint4(v[0], v[1], v[2], v[3]);
}

// One 32-step block of B, C and x in LDS.
template <int NP, int HPW = 1>
struct __align__(16) BlockStage {
    static constexpr int XH = HPW;       // heads of x staged
    static constexpr int TP = 36;        // BT / XT row pitch (elements; rows 8-byte aligned)
    static constexpr int CP = NP + 4;    // CR row pitch (8-byte reads of 16 rows: distinct banks)
    uint16_t BT[NP * TP];                // BT[n][s] = B at step s, state n
    uint16_t CR[32 * CP];                // CR[t][n] = C at step t, state n
    uint16_t XT[HPW * kPG * TP];         // XT[head][p][s] = x at step s, column p
};
template <int Q, int NP, int HPW>
struct __align__(16) OutSmem {
    BlockStage<NP, HPW> st[2];           // blocks k and k + 1 of the walk
    uint4 M[HPW][2][2][64];              // diagonal decay tile: [head][t tile][hi, lo][lane]
    float cum[HPW][Q], dl[HPW][Q];
    float fs[HPW][Q];                    // 2^(cum at the end of s's block - cum_s) dl_s
    float wsum[HPW][4];
};

// A block's B, C and x rows as loaded.  Unit u of B and x: step pair
// 2 (u / (NP / 8)) (x: 2 (u / 8)) of the block, 8 states (columns) from
// 8 (u % (NP / 8)) (x: 8 (u % 8)), so consecutive lanes read consecutive
// 16-byte pieces of a row; unit u of C:
// step u / (NP / 8), 8 states.  Rows past the sequence end are read as zero
// (vector path) or clamped (element path); their values meet only zero
// weights (dl = 0 there) and outputs that are not stored.  States past N
// are zeroed (cm, bm): they would enter the sums over n.  Columns past the
// slice's head dimension are not masked: every column p is computed on its
// own and those are not stored.
template <int NP, bool WC = true>
struct BlockRegs {
    static constexpr int NCU = WC ? (4 * NP + 255) / 256 : 0;   // C units per thread
    uint4 b[2], x[2], c[NCU > 0 ? NCU : 1];
};

// Per-thread load geometry, fixed over the walk.
template <int NP, bool WC = true>
struct BlockGeom {
    static constexpr int NC = BlockRegs<NP, WC>::NCU > 0 ? BlockRegs<NP, WC>::NCU : 1;
    uint32_t ob, ox, oc[NC];                     // byte offsets within a block
    uint32_t bm, cm[NC];                         // state masks of the B and C units
    int sb, sx, scu[NC];                         // step of the unit
    int nb, px, ncu[NC];                         // first state / column of the unit
};

template <int NP, bool WC>
__device__ __forceinline__ void block_geom(BlockGeom<NP, WC> &q, const Geom &g, int rowBC, int rowX) {
    const int tid = threadIdx.x;
    {
        const int u = min(tid, 2 * NP - 1);
        q.sb = 2 * (u / (NP / 8));
        q.nb = (u % (NP / 8)) * 8;
        q.ob = static_cast<uint32_t>(q.sb * rowBC + q.nb) * 2u;
        q.bm = q.nb < g.N ? ~0u : 0u;
    }
    {
        const int u = tid & 127;
        q.sx = 2 * (u / (kPG / 8));
        q.px = (u % (kPG / 8)) * 8;
        q.ox = static_cast<uint32_t>(q.sx * rowX + q.px) * 2u;
    }
#pragma unroll
    for (int i = 0; i < BlockRegs<NP, WC>::NCU; ++i) {
        const int u = min(tid + 256 * i, 4 * NP - 1);
        q.scu[i] = u / (NP / 8);
        q.ncu[i] = (u % (NP / 8)) * 8;
        q.oc[i] = static_cast<uint32_t>(q.scu[i] * rowBC + q.ncu[i]) * 2u;
        q.cm[i] = q.ncu[i] < g.N ? ~0u : 0u;
    }
}

template <int NP, bool VEC, bool WC>
__device__ __forceinline__ void load_block(BlockRegs<NP, WC> &r, const BlockGeom<NP, WC> &q, const uint16_t *Bg,
                                           const uint16_t *Cg, const uint16_t *xg, int tb, const Geom &g,
                                           int rowBC, int rowX, int pcols) {
    if (VEC) {
        // resources from the block's first row to the end of the sequence
        const int64_t rows = g.L - tb;
        const auto rB = brsrc(Bg + static_cast<int64_t>(tb) * rowBC, rows * rowBC * 2 - (rowBC - g.N) * 2);
        const auto rX = brsrc(xg + static_cast<int64_t>(tb) * rowX, rows * rowX * 2 - (rowX - pcols) * 2);
        r.b[0] = bload16(rB, q.ob);
        r.b[1] = bload16(rB, q.ob + rowBC * 2);
        r.x[0] = bload16(rX, q.ox);
        r.x[1] = bload16(rX, q.ox + rowX * 2);
        if constexpr (WC) {
            const auto rC = brsrc(Cg + static_cast<int64_t>(tb) * rowBC, rows * rowBC * 2 - (rowBC - g.N) * 2);
#pragma unroll
            for (int i = 0; i < BlockRegs<NP, WC>::NCU; ++i) r.c[i] = bload16(rC, q.oc[i]);
        }
    } else {
        uint32_t m;
        r.b[0] = load_row8_raw<false>(Bg, tb + q.sb, q.nb, g.L, g.N, rowBC, m);
        r.b[1] = load_row8_raw<false>(Bg, tb + q.sb + 1, q.nb, g.L, g.N, rowBC, m);
        r.x[0] = load_row8_raw<false>(xg, tb + q.sx, q.px, g.L, pcols, rowX, m);
        r.x[1] = load_row8_raw<false>(xg, tb + q.sx + 1, q.px, g.L, pcols, rowX, m);
#pragma unroll
        for (int i = 0; i < BlockRegs<NP, WC>::NCU; ++i)
            r.c[i] = load_row8_raw<false>(Cg, tb + q.scu[i], q.ncu[i], g.L, g.N, rowBC, m);
    }
}

// `nmask`: N < NP (workgroup-uniform), so state columns past N are zeroed.
template <int NP, bool VEC, bool WC, class Stage>
__device__ __forceinline__ void store_block(const BlockRegs<NP, WC> &r, const BlockGeom<NP, WC> &q, bool nmask,
                                            Stage &st) {
    constexpr int TP = Stage::TP;
    const int tid = threadIdx.x;
    // two step rows as 4-byte step pairs of the transposed tiles (the eight
    // rows of a unit share one swizzle)
    auto pairs = [](uint16_t *T, int row8, int s2, uint4 v0, uint4 v1) {
        const uint32_t a[4] = {v0.x, v0.y, v0.z, v0.w}, e[4] = {v1.x, v1.y, v1.z, v1.w};
        const int sc = swz(s2, row8);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            *reinterpret_cast<uint32_t *>(&T[(row8 + 2 * k) * TP + sc]) = (a[k] & 0xffffu) | (e[k] << 16);
            *reinterpret_cast<uint32_t *>(&T[(row8 + 2 * k + 1) * TP + sc]) = (a[k] >> 16) | (e[k] & 0xffff0000u);
        }
    };
    const bool vm = VEC && nmask;
    if (tid < 2 * NP) pairs(st.BT, q.nb, q.sb, vm ? and4(r.b[0], q.bm) : r.b[0], vm ? and4(r.b[1], q.bm) : r.b[1]);
    // x: threads 128 q + u hold unit u of head q's tile (Stage::XH heads)
    if (Stage::XH == 2) pairs(st.XT + (tid >> 7) * (kPG * TP), q.px, q.sx, r.x[0], r.x[1]);
    else if (tid < 128) pairs(st.XT, q.px, q.sx, r.x[0], r.x[1]);
    if constexpr (WC) {
        constexpr int CP = Stage::CP;
#pragma unroll
        for (int i = 0; i < BlockRegs<NP, WC>::NCU; ++i) {
            if (tid + 256 * i < 4 * NP) {
                const uint4 v = vm ? and4(r.c[i], q.cm[i]) : r.c[i];
                *reinterpret_cast<uint2 *>(&st.CR[q.scu[i] * CP + q.ncu[i]]) = make_uint2(v.x, v.y);
                *reinterpret_cast<uint2 *>(&st.CR[q.scu[i] * CP + q.ncu[i] + 4]) = make_uint2(v.z, v.w);
            }
        }
    }
}

// dl and the inclusive sum of the log2 decay over the chunk's Q steps for
// HPW heads at once, from prefetched raw dt values (thread s < Q holds step
// s of every head; wsum holds one float per head and wave).  The scans of
// the heads are interleaved and share the two barriers; each is the same
// sequence of additions as a scan of one head.  Ends with a barrier.
template <int Q, int HPW>
__device__ void chunk_decay(const float (&dr)[HPW], int t0, int L, const float (&A2)[HPW],
                            const float (&bias)[HPW], float (*s_cum)[Q], float (*s_dl)[Q], float (*s_wsum)[4]) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    float dlv[HPW], sc[HPW];
#pragma unroll
    for (int hd = 0; hd < HPW; ++hd) {
        dlv[hd] = 0.0f;
        sc[hd] = 0.0f;
        if (tid < Q && t0 + tid < L) {
            dlv[hd] = softplus(dr[hd] + bias[hd]);
            sc[hd] = dlv[hd] * A2[hd];
        }
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
#pragma unroll
        for (int hd = 0; hd < HPW; ++hd) {
            const float o = __shfl_up(sc[hd], off, 64);
            if (lane >= off) sc[hd] += o;
        }
    }
    if (lane == 63) {
#pragma unroll
        for (int hd = 0; hd < HPW; ++hd) s_wsum[hd][wave] = sc[hd];
    }
    __syncthreads();
    if (tid < Q) {
#pragma unroll
        for (int hd = 0; hd < HPW; ++hd) {
            float base = 0.0f;
            for (int w2 = 0; w2 < wave; ++w2) base += s_wsum[hd][w2];
            s_cum[hd][tid] = sc[hd] + base;
            s_dl[hd][tid] = dlv[hd];
        }
    }
    __syncthreads();
}

// ---------------------------------------------------------------------------
// Gram tiles of the blocks' diagonals (formed by extra workgroups of the
// state kernel's launch, which the output kernel reads)
// ---------------------------------------------------------------------------
// C_t . B_s for s, t in the same 32-step block, in the three 16 x 16
// quadrants (s tile, t tile) = (0, 0), (0, 1), (1, 1) that hold every s <= t.
// They depend only on the B / C group, not on the head, so they are formed
// once instead of in each of the group's heads' output workgroups, whose LDS
// operand layouts (steps along a row) would need a gather per element for
// this contraction over the states.  One wave per task = ((b G + group) nblk
// + block) 3 + quadrant w, with the states in K slots 8 g + i of K step kk
// (state 32 kk + 8 g + i; past N: zero; rows past the sequence end: zero).
// Stored as one float4 per lane at Gm[task * 64 + lane], D layout (column
// t = l16, rows s = 4 g + v of the quadrant).
template <int NP, bool VEC>
__device__ __forceinline__ void gram_quadrant(const uint16_t *__restrict__ Bm, const uint16_t *__restrict__ Cm,
                                              f4x *__restrict__ Gm, const Geom &g, int nblk, int64_t task,
                                              int lane) {
    const int l16 = lane & 15, g4 = lane >> 4;
    const int w = static_cast<int>(task % 3);
    int64_t id = task / 3;
    const int blk = static_cast<int>(id % nblk);
    id /= nblk;
    const int grp = static_cast<int>(id % g.G);
    const int64_t b = id / g.G;
    const int sq = w == 2 ? 1 : 0, tq = w == 0 ? 0 : 1;
    const int rowBC = g.G * g.N;
    const int s = 32 * blk + 16 * sq + l16, t = 32 * blk + 16 * tq + l16;
    const bool oks = s < g.L, okt = t < g.L;
    const uint16_t *bp = Bm + (b * g.L + (oks ? s : 0)) * static_cast<int64_t>(rowBC) + grp * g.N;
    const uint16_t *cp = Cm + (b * g.L + (okt ? t : 0)) * static_cast<int64_t>(rowBC) + grp * g.N;
    f4x G = zero4();
#pragma unroll
    for (int kk = 0; kk < NP / 32; ++kk) {
        const int n0 = 32 * kk + 8 * g4;
        uint4 av, cv;
        if (VEC) {
            // N % 8 == 0: the eight states are all inside the row or all past it
            const bool ia = oks && n0 < g.N, ic = okt && n0 < g.N;
            const uint4 a4 = *reinterpret_cast<const uint4 *>(bp + (ia ? n0 : 0));
            const uint4 c4 = *reinterpret_cast<const uint4 *>(cp + (ic ? n0 : 0));
            av = ia ? a4 : make_uint4(0, 0, 0, 0);
            cv = ic ? c4 : make_uint4(0, 0, 0, 0);
        } else {
            uint16_t ae[8], ce[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const bool in = n0 + i < g.N;
                ae[i] = oks && in ? bp[n0 + i] : 0;
                ce[i] = okt && in ? cp[n0 + i] : 0;
            }
            __builtin_memcpy(&av, ae, 16);
            __builtin_memcpy(&cv, ce, 16);
        }
        G = mfma16(__builtin_bit_cast(bf8, av), __builtin_bit_cast(bf8, cv), G);
    }
    Gm[task * 64 + lane] = G;
}

// ---------------------------------------------------------------------------
// 1. chunk states, block-walk form
// ---------------------------------------------------------------------------
// S[p][n] = sum_s w_s x_s[p] B_s[n], w_s = 2^(cum_end - cum_s) dl_s: the
// output kernel's state update (section 3) without the outputs.  One
// workgroup per (batch, chunk pair, 64-column slice) and HPW heads of one
// B / C group (two where the group's head count is even): the block's B^T is
// staged once and each of its operand reads serves both heads.  The second
// chunk of a pair continues from the first one's state decayed over the
// second chunk, so the pair's state is written once.  Wave w
// accumulates columns p = 16 w + 0..15 of every head over the chunk's
// 32-step blocks with the same operand orders (B^T rows n and K = steps;
// (x w) columns p).
template <int NP, int HPW>
struct __align__(16) StateStage {
    static constexpr int XH = HPW;
    static constexpr int TP = 36;
    uint16_t BT[NP * TP];                // BT[n][s]
    uint16_t XT[HPW * kPG * TP];         // XT[head][p][s]
};
template <int Q, int NP, int HPW>
struct __align__(16) StateSmem {
    StateStage<NP, HPW> st[2];
    float cum[HPW][Q], dl[HPW][Q], w[HPW][Q];
    float wsum[HPW][4];
};

template <int Q, int NP, bool VEC, int HPW>
__global__ __launch_bounds__(256, VEC ? (HPW == 2 ? 3 : 4) : 2) void ssd_state_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ dt,
    const float *__restrict__ dt_bias, const float *__restrict__ A,
    const uint16_t *__restrict__ Bm, float *__restrict__ S, float *__restrict__ ce, Geom g,
    const uint16_t *__restrict__ Cm, f4x *__restrict__ Gm, int nstate, int nblk, int ntask) {
    constexpr int NB = Q / 32;
    constexpr int NJ = NP / 16;
    constexpr int TP = StateStage<NP, HPW>::TP;
    __shared__ StateSmem<Q, NP, HPW> sm;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l16 = lane & 15, g4 = lane >> 4;

    // workgroups past the states' ones: four Gram quadrants each
    if (static_cast<int>(blockIdx.x) >= nstate) {
        const int64_t task = static_cast<int64_t>(blockIdx.x - nstate) * 4 + wave;
        if (task < ntask) gram_quadrant<NP, VEC>(Bm, Cm, Gm, g, nblk, task, lane);
        return;
    }
    // (batch, chunk pair m, heads h0.., slice pg): chunks 2 m and 2 m + 1
    int64_t id = blockIdx.x;
    const int pg = static_cast<int>(id % g.npg);
    id /= g.npg;
    const int h0 = static_cast<int>(id % (g.H / HPW)) * HPW;
    id /= g.H / HPW;
    const int npair = (g.nch + 1) / 2;
    const int m = static_cast<int>(id % npair);
    const int64_t b = id / npair;
    const int pbase = pg * kPG, pcols = g.P - pbase;
    const int rowX = g.H * g.P, rowBC = g.G * g.N;
    const int grp = h0 / (g.H / g.G);
    const uint16_t *Bg = Bm + b * g.L * static_cast<int64_t>(rowBC) + grp * g.N;
    // x rows of this thread's staging head (wave-uniform: waves 0-1 head 0)
    const int hx = HPW == 2 ? (wave >> 1) : 0;
    const uint16_t *xg = x + b * g.L * static_cast<int64_t>(rowX) + (h0 + hx) * g.P + pbase;
    const bool nmask = g.N < NP;
    const int pl = 16 * wave + l16;
    float a2[HPW], bs[HPW];
#pragma unroll
    for (int hd = 0; hd < HPW; ++hd) {
        a2[hd] = A[h0 + hd] * kLog2e;
        bs[hd] = dt_bias ? dt_bias[h0 + hd] : 0.0f;
    }
    BlockGeom<NP, false> q;
    block_geom<NP, false>(q, g, rowBC, rowX);

    f4x acc[HPW][NJ];
    float ce_pair[HPW];
#pragma unroll
    for (int hd = 0; hd < HPW; ++hd) {
        ce_pair[hd] = 0.0f;
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[hd][j] = zero4();
    }
#pragma unroll 1
    for (int cc = 0; cc < 2; ++cc) {
        const int c = 2 * m + cc;
        if (c >= g.nch) break;
        if (cc > 0) __syncthreads();   // every read of the previous chunk's LDS is done
        const int t0 = c * Q;
        // dt first, then the first two blocks (one register set ahead, as in
        // the output kernel)
        const int tdt = t0 + (tid < Q ? tid : 0);
        const int64_t dto = b * g.L * static_cast<int64_t>(g.H) + static_cast<int64_t>(tdt < g.L ? tdt : g.L - 1) * g.H + h0;
        float dtr[HPW];
#pragma unroll
        for (int hd = 0; hd < HPW; ++hd) dtr[hd] = bf16_to_f32(dt[dto + hd]);
        BlockRegs<NP, false> r0, ra;
        load_block<NP, VEC, false>(r0, q, Bg, nullptr, xg, t0, g, rowBC, rowX, pcols);
        if (NB > 1) load_block<NP, VEC, false>(ra, q, Bg, nullptr, xg, t0 + 32, g, rowBC, rowX, pcols);
        float cum_end[HPW];
        chunk_decay<Q, HPW>(dtr, t0, g.L, a2, bs, sm.cum, sm.dl, sm.wsum);
#pragma unroll
        for (int hd = 0; hd < HPW; ++hd) {
            cum_end[hd] = sm.cum[hd][Q - 1];
            if (tid < Q) sm.w[hd][tid] = fast_exp2(cum_end[hd] - sm.cum[hd][tid]) * sm.dl[hd][tid];
            // the second chunk continues from the first one's state:
            // acc = 2^(its decay) S_{2m} + (its own terms) = the pair's
            // aggregate
            if (cc > 0) {
                const float a = fast_exp2(cum_end[hd]);
#pragma unroll
                for (int j = 0; j < NJ; ++j) acc[hd][j] = acc[hd][j] * a;
            }
            ce_pair[hd] += cum_end[hd];
        }
        store_block<NP, VEC, false>(r0, q, nmask, sm.st[0]);
        __syncthreads();

        auto step = [&](const int k, BlockRegs<NP, false> &rg) {
            const StateStage<NP, HPW> &st = sm.st[k & 1];
            const int base = 32 * k;
            // (x w) of the block for each head: column p = pl, K slots
            // s = 16 (i / 4) + 4 g4 + i % 4
            bf8 xwh[HPW], xwl[HPW];
#pragma unroll
            for (int hd = 0; hd < HPW; ++hd) {
                const uint16_t *xp = &st.XT[(hd * kPG + pl) * TP];
                const uint2 x0 = *reinterpret_cast<const uint2 *>(xp + swz(4 * g4, pl));
                const uint2 x1 = *reinterpret_cast<const uint2 *>(xp + swz(16 + 4 * g4, pl));
                const float4 f0 = *reinterpret_cast<const float4 *>(&sm.w[hd][base + 4 * g4]);
                const float4 f1 = *reinterpret_cast<const float4 *>(&sm.w[hd][base + 16 + 4 * g4]);
                uint32_t xh[4], xl[4];
                split_pk(bits_lo(x0.x) * f0.x, bits_hi(x0.x) * f0.y, xh[0], xl[0]);
                split_pk(bits_lo(x0.y) * f0.z, bits_hi(x0.y) * f0.w, xh[1], xl[1]);
                split_pk(bits_lo(x1.x) * f1.x, bits_hi(x1.x) * f1.y, xh[2], xl[2]);
                split_pk(bits_lo(x1.y) * f1.z, bits_hi(x1.y) * f1.w, xh[3], xl[3]);
                xwh[hd] = __builtin_bit_cast(bf8, make_uint4(xh[0], xh[1], xh[2], xh[3]));
                xwl[hd] = __builtin_bit_cast(bf8, make_uint4(xl[0], xl[1], xl[2], xl[3]));
            }
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const uint16_t *bp = &st.BT[(16 * j + l16) * TP];
                const bf8 bt = cat8(*reinterpret_cast<const uint2 *>(bp + swz(4 * g4, 16 * j)),
                                    *reinterpret_cast<const uint2 *>(bp + swz(16 + 4 * g4, 16 * j)));
#pragma unroll
                for (int hd = 0; hd < HPW; ++hd) {
                    acc[hd][j] = mfma16(bt, xwh[hd], acc[hd][j]);
                    acc[hd][j] = mfma16(bt, xwl[hd], acc[hd][j]);
                }
            }
            if (k + 1 < NB) {
                // the next block into LDS: its buffer was last read in the
                // previous block, before that block's barrier
                store_block<NP, VEC, false>(rg, q, nmask, sm.st[(k + 1) & 1]);
                __syncthreads();
                if (k + 2 < NB)
                    load_block<NP, VEC, false>(rg, q, Bg, nullptr, xg, t0 + base + 64, g, rowBC, rowX, pcols);
            }
        };
#pragma unroll 1
        for (int k = 0; k < NB; k += 2) {
            step(k, ra);
            step(k + 1, ra);
        }
    }
    // the pair's aggregate (a last chunk without a partner: its own state)
    // and total log2 decay.  Lane (l16, g4) holds [pl][16 j + 4 g4 + v] of
    // each head.
    {
        if (pl < pcols) {
#pragma unroll
            for (int hd = 0; hd < HPW; ++hd) {
                float *Sg = S + (((b * npair + m) * g.H + h0 + hd) * static_cast<int64_t>(g.P) + pbase + pl) * g.N;
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    const int n4 = 16 * j + 4 * g4;
                    if (VEC) {
                        if (n4 < g.N)
                            *reinterpret_cast<float4 *>(Sg + n4) =
                                make_float4(acc[hd][j][0], acc[hd][j][1], acc[hd][j][2], acc[hd][j][3]);
                    } else {
#pragma unroll
                        for (int v = 0; v < 4; ++v)
                            if (n4 + v < g.N) Sg[n4 + v] = acc[hd][j][v];
                    }
                }
            }
        }
        if (pbase == 0 && tid < HPW) ce[(b * npair + m) * g.H + h0 + tid] = ce_pair[tid];
    }
}

// ---------------------------------------------------------------------------
// 2. state pass over chunk pairs: slot j <- state entering chunk 2 GSZ j;
//    h_last <- final state
// ---------------------------------------------------------------------------
// Slot m holds the aggregate of chunks 2 m and 2 m + 1,
// 2^(e_{2m+1}) S_{2m} + S_{2m+1} (e: a chunk's total log2 decay, S: its state
// from zero; a last chunk without a partner: its own S), and ce[m] the pair's
// total decay, so one fused multiply-add per pair, h <- 2^(ce[m]) h + slot,
// carries the state across two chunks.  The output kernel walks GSZ pairs
// (GSZ = 1 or 2) from the state entering the first, so only every GSZ-th
// entering state is stored, into slot m / GSZ (a slot already read: the
// aggregates are read ahead of the stores).
template <int GSZ>
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
    const int npair = (g.nch + 1) / 2;
    constexpr int U = 4;    // pairs whose aggregates are loaded ahead of the chain
    int m = 0;
    for (; m + U <= npair; m += U) {
        float s[U], a[U];
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int64_t bc = (b * npair + m + k) * g.H + hh;
            s[k] = S[bc * PN + e];
            a[k] = fast_exp2(ce[bc]);
        }
#pragma unroll
        for (int k = 0; k < U; ++k) {
            if ((m + k) % GSZ == 0) S[((b * npair + (m + k) / GSZ) * g.H + hh) * PN + e] = h;
            h = fmaf(a[k], h, s[k]);
        }
    }
    for (; m < npair; ++m) {
        const int64_t bc = (b * npair + m) * g.H + hh;
        const float s = S[bc * PN + e];
        if (m % GSZ == 0) S[((b * npair + m / GSZ) * g.H + hh) * PN + e] = h;
        h = fmaf(fast_exp2(ce[bc]), h, s);
    }
    if (h_last) h_last[bh * PN + e] = h;
}

// ---------------------------------------------------------------------------
// 3. outputs, block-state form
// ---------------------------------------------------------------------------
// One workgroup per (batch, chunk, head, 64-column head-dimension slice).  The
// chunk is walked in 32-step blocks k carrying the slice's state: with c_k
// the cumulative log2 decay before block k (c_0 = 0), e_k the one at its end
// and H_k the state entering it (H_0 = h_in),
//
//   y_t     = 2^(cum_t - c_k) C_t . H_k[p,:]
//             + sum_{s in block k, s <= t} (C_t . B_s) 2^(cum_t - cum_s) dl_s x_s[p]
//             + D x_t[p]
//   H_{k+1} = 2^(e_k - c_k) H_k + sum_{s in block k} 2^(e_k - cum_s) dl_s x_s[p] B_s
//
// -- the chunk's unrolled recurrence ("Mamba状态空间模型的硬件感知推理优化"
// (ybb.press) section 4) taken block by block, with the state carried from
// block to block as section 5 carries it from chunk to chunk.  Only the
// 32 x 32 diagonal tile of each block needs a decay matrix; everything before
// the block reaches y through the carried state.
//
// Products run on v_mfma_f32_16x16x32_bf16 (A: lane l holds row l % 16 and K
// indices 8 (l / 16) + 0..7; B: column l % 16 and the same K indices; D:
// column l % 16, rows 4 (l / 16) + 0..3).  Wave w owns head-dimension columns
// p = 16 w + 0..15 and keeps H^T of them as accumulators: lane (l16 = l % 16,
// g = l / 16) holds H[16 w + l16][16 j + 4 g + v] of state tile j.  As the A
// operand of the output product (rows p, K = n) those registers put state
// index 32 kk + 16 (i / 4) + 4 g + i % 4 in K slot 8 g + i, and the C operand
// is read in the same order.  Every product over the steps s of a block uses
// the order s = 16 (i / 4) + 4 g + i % 4 likewise, so the diagonal tile's
// accumulators (rows s, column t) are already B operands of its product with
// x.  Waves 0-2 form the tile's three causal 16 x 16 quadrants one block
// ahead and share them through LDS.
// Waves 0, 1, 2: quadrant (sq, tq) = (0, 0), (0, 1), (1, 1) of the diagonal
// tile of the block at chunk step `base`, for each of the HPW heads:
//   M[t][s] = (C_t . B_s) 2^(cum_t - cum_s) dl_s for s < t, plus D at s = t,
// split into bf16 parts (hi pair 0-1, hi pair 2-3, lo pair 0-1, lo pair 2-3)
// that diag_store writes as K slots 4 sq .. 4 sq + 3 of the B operand of t
// tile tq.  G holds the quadrant's C_t . B_s as ssd_gram_kernel laid it out:
// G[v] at step s = 16 sq + 4 g + v, column t = 16 tq + l16 of the block.
// (Wave 3 may form the values of quadrant (0, 1) too; it stores none.)
template <int Q, int NP, int HPW>
__device__ __forceinline__ void diag_vals(const f4x G, const OutSmem<Q, NP, HPW> &sm, int base,
                                          const float (&skip)[HPW], int wave, int lane,
                                          uint4 (&mv)[HPW]) {
    const int sq = wave == 2 ? 1 : 0, tq = wave == 0 ? 0 : 1;
    const int l16 = lane & 15, g4 = lane >> 4;
    const int t = base + 16 * tq + l16, s0 = base + 16 * sq + 4 * g4;
#pragma unroll
    for (int hd = 0; hd < HPW; ++hd) {
        const float ct = sm.cum[hd][t];
        const float4 cs = *reinterpret_cast<const float4 *>(&sm.cum[hd][s0]);
        const float4 ds = *reinterpret_cast<const float4 *>(&sm.dl[hd][s0]);
        const float csv[4] = {cs.x, cs.y, cs.z, cs.w}, dsv[4] = {ds.x, ds.y, ds.z, ds.w};
        float m[4];
        // causal mask s <= t, D on the diagonal (2^(ct - cs) overflows only
        // where s > t, which the mask replaces by 0)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const float e = G[v] * fast_exp2(ct - csv[v]) * dsv[v];
            const int sv = 16 * sq + 4 * g4 + v, tv = 16 * tq + l16;
            m[v] = sv <= tv ? e + (sv == tv ? skip[hd] : 0.0f) : 0.0f;
        }
        split_pk(m[0], m[1], mv[hd].x, mv[hd].z);
        split_pk(m[2], m[3], mv[hd].y, mv[hd].w);
    }
}
template <int Q, int NP, int HPW>
__device__ __forceinline__ void diag_store(OutSmem<Q, NP, HPW> &sm, const uint4 (&mv)[HPW], int wave,
                                           int lane) {
    const int sq = wave == 2 ? 1 : 0, tq = wave == 0 ? 0 : 1;
#pragma unroll
    for (int hd = 0; hd < HPW; ++hd) {
        reinterpret_cast<uint2 *>(&sm.M[hd][tq][0][lane])[sq] = make_uint2(mv[hd].x, mv[hd].y);
        reinterpret_cast<uint2 *>(&sm.M[hd][tq][1][lane])[sq] = make_uint2(mv[hd].z, mv[hd].w);
    }
}

// cpw (2 or 4) consecutive chunks per workgroup: the walk over one chunk
// ends holding the state entering the next, so only the state entering the
// first is read.  HPW heads of one B / C group per workgroup (the launcher
// takes one, so that the layer's chunk groups and heads fill the chip in
// whole rounds; two would share the block's staged B and C and every B and C
// operand read).  Workgroups per compute unit: three for one head on the
// vector path, gated or not (LDS and registers allow it), two otherwise.
template <int Q, int NP, bool VEC, bool GATE, int HPW>
__global__ __launch_bounds__(256, (HPW == 1 && VEC) ? 3 : 2) void ssd_output_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ dt,
    const float *__restrict__ dt_bias, const float *__restrict__ A,
    const uint16_t *__restrict__ Bm, const uint16_t *__restrict__ Cm,
    const float *__restrict__ Dskip, const uint16_t *__restrict__ z, const float *__restrict__ Hin,
    const f4x *__restrict__ Gm, uint16_t *__restrict__ y, Geom g, int cpw) {
    constexpr int NB = Q / 32;          // blocks per chunk
    constexpr int NJ = NP / 16;         // 16-wide state tiles
    constexpr int KK = NP / 32;         // K steps over the state index
    using St = BlockStage<NP, HPW>;
    constexpr int TP = St::TP, CP = St::CP;
    __shared__ OutSmem<Q, NP, HPW> sm;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l16 = lane & 15, g4 = lane >> 4;

    int64_t id = blockIdx.x;
    const int pg = static_cast<int>(id % g.npg);
    id /= g.npg;
    const int h0 = static_cast<int>(id % (g.H / HPW)) * HPW;
    id /= g.H / HPW;
    const int npair = (g.nch + 1) / 2, ngrp = (g.nch + cpw - 1) / cpw;
    const int m = static_cast<int>(id % ngrp);       // chunks cpw m .. cpw m + cpw - 1
    const int64_t b = id / ngrp;
    const int pbase = pg * kPG, pcols = g.P - pbase;
    const int rowX = g.H * g.P, rowBC = g.G * g.N;
    const int grp = h0 / (g.H / g.G);
    const uint16_t *Bg = Bm + b * g.L * static_cast<int64_t>(rowBC) + grp * g.N;
    const uint16_t *Cg = Cm + b * g.L * static_cast<int64_t>(rowBC) + grp * g.N;
    // element offset of head h0's slice in its batch's first row (head
    // h0 + hd: hd P further)
    const int64_t xoff = b * g.L * static_cast<int64_t>(rowX) + h0 * g.P + pbase;
    // x rows of this thread's staging head (wave-uniform: waves 0-1 head 0)
    const uint16_t *xg = x + xoff + (HPW == 2 ? (wave >> 1) : 0) * g.P;
    const bool nmask = g.N < NP;
    const int pl = 16 * wave + l16;     // column of this lane's A rows / B columns
    const int p4 = 16 * wave + 4 * g4;  // first of this lane's four output columns
    float skip[HPW];
#pragma unroll
    for (int hd = 0; hd < HPW; ++hd) skip[hd] = Dskip ? Dskip[h0 + hd] : 0.0f;

    // the state entering chunk cpw m, from the pass (slot m)
    f4x H[HPW][NJ];
    const int64_t PNs = static_cast<int64_t>(g.P) * g.N;
#pragma unroll
    for (int hd = 0; hd < HPW; ++hd) {
        const float *Hg = Hin + ((b * npair + m) * g.H + h0 + hd) * PNs;
        const bool okp = pl < pcols;
        const float *hrow = Hg + static_cast<int64_t>(okp ? pbase + pl : 0) * g.N;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int n4 = 16 * j + 4 * g4;
            if (VEC) {
                // N % 8 == 0: the four states are all inside the row or all past it
                const bool ok = okp && n4 < g.N;
                const uint32_t mk = opaque_mask(ok);
                const float4 v = *reinterpret_cast<const float4 *>(hrow + (ok ? n4 : 0));
                H[hd][j][0] = __uint_as_float(__float_as_uint(v.x) & mk);
                H[hd][j][1] = __uint_as_float(__float_as_uint(v.y) & mk);
                H[hd][j][2] = __uint_as_float(__float_as_uint(v.z) & mk);
                H[hd][j][3] = __uint_as_float(__float_as_uint(v.w) & mk);
            } else {
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const bool ok = okp && n4 + v < g.N;
                    const float e = hrow[ok ? n4 + v : 0];
                    H[hd][j][v] = ok ? e : 0.0f;
                }
            }
        }
    }
    float a2[HPW], bs[HPW];
#pragma unroll
    for (int hd = 0; hd < HPW; ++hd) {
        a2[hd] = A[h0 + hd] * kLog2e;
        bs[hd] = dt_bias ? dt_bias[h0 + hd] : 0.0f;
    }
    // K slots 4..7 of t tile 0 (steps 16..31, after every step of the tile)
    // stay zero; no quadrant writes them
    if (wave == 3) {
#pragma unroll
        for (int hd = 0; hd < HPW; ++hd)
#pragma unroll
            for (int hl = 0; hl < 2; ++hl) reinterpret_cast<uint2 *>(&sm.M[hd][0][hl][lane])[1] = make_uint2(0, 0);
    }
    BlockGeom<NP, true> q;
    block_geom<NP, true>(q, g, rowBC, rowX);
    uint16_t *yg = y + xoff;
    // Each head's state is carried as H = sig * Hs with sig a
    // workgroup-uniform scalar, so a block's decay multiplies sig (and the
    // block's new terms by 1 / sig) instead of every state element; when sig
    // would fall below 2^-64 it is folded back into Hs.  It carries on from
    // the first chunk of the pair to the second.
    float sig[HPW];
#pragma unroll
    for (int hd = 0; hd < HPW; ++hd) sig[hd] = 1.0f;
    // this wave's Gram quadrant of the group's first block (waves 0-2; one
    // block further: 3 * 64 float4)
    const f4x *Gw = Gm + ((b * g.G + grp) * static_cast<int64_t>(g.nch) * NB * 3 + (wave < 3 ? wave : 0)) * 64 + lane;

#pragma unroll 1
    for (int cc = 0; cc < cpw; ++cc) {
    const int c = cpw * m + cc;
    if (c >= g.nch) break;
    if (cc > 0) __syncthreads();   // every read of the previous chunk's LDS is done
    const int t0 = c * Q;
    // the walk continues into the next chunk after this one's last block
    const bool cont = cc + 1 < cpw && c + 1 < g.nch;
    // dt first (the decay scan waits for it), then the first two blocks'
    // rows: block j + 1 is stored to LDS at the end of block j from the
    // register set ra, which then receives block j + 2
    const int tdt = t0 + (tid < Q ? tid : 0);
    const int64_t dto = b * g.L * static_cast<int64_t>(g.H) + static_cast<int64_t>(tdt < g.L ? tdt : g.L - 1) * g.H + h0;
    float dtr[HPW];
#pragma unroll
    for (int hd = 0; hd < HPW; ++hd) dtr[hd] = bf16_to_f32(dt[dto + hd]);
    // Gram quadrant of block 0, then (in flight through each block) of the
    // block after the next
    f4x gq = Gw[static_cast<int64_t>(c * NB) * 192];
    BlockRegs<NP, true> r0, ra;
    load_block<NP, VEC, true>(r0, q, Bg, Cg, xg, t0, g, rowBC, rowX, pcols);
    if (NB > 1) load_block<NP, VEC, true>(ra, q, Bg, Cg, xg, t0 + 32, g, rowBC, rowX, pcols);
    chunk_decay<Q, HPW>(dtr, t0, g.L, a2, bs, sm.cum, sm.dl, sm.wsum);
#pragma unroll
    for (int hd = 0; hd < HPW; ++hd)
        if (tid < Q) sm.fs[hd][tid] = fast_exp2(sm.cum[hd][tid | 31] - sm.cum[hd][tid]) * sm.dl[hd][tid];
    store_block<NP, VEC, true>(r0, q, nmask, sm.st[0]);
    __syncthreads();
    {
        uint4 mv[HPW];
        diag_vals<Q, NP, HPW>(gq, sm, 0, skip, wave, lane, mv);
        if (wave < 3) diag_store<Q, NP, HPW>(sm, mv, wave, lane);
    }
    gq = Gw[static_cast<int64_t>(c * NB + 1) * 192];
    // gate values of this lane's steps of the current block, four columns each
    uint2 zr[HPW][2];
#pragma unroll
    for (int hd = 0; hd < HPW; ++hd) zr[hd][0] = zr[hd][1] = make_uint2(0, 0);
    auto load_z = [&](int kb) {
#pragma unroll
        for (int hd = 0; hd < HPW; ++hd)
#pragma unroll
            for (int tq = 0; tq < 2; ++tq) {
                const int t = t0 + 32 * kb + 16 * tq + l16;
                const int tc = t < g.L ? t : g.L - 1;
                const uint16_t *zp = z + xoff + hd * g.P + static_cast<int64_t>(tc) * rowX;
                if (VEC) {
                    const uint32_t mk = opaque_mask(p4 < pcols);
                    const uint2 v = *reinterpret_cast<const uint2 *>(zp + (p4 < pcols ? p4 : 0));
                    zr[hd][tq] = make_uint2(v.x & mk, v.y & mk);
                } else {
                    uint16_t e[4];
#pragma unroll
                    for (int v = 0; v < 4; ++v) e[v] = p4 + v < pcols ? zp[p4 + v] : 0;
                    zr[hd][tq] = make_uint2(e[0] | (static_cast<uint32_t>(e[1]) << 16),
                                            e[2] | (static_cast<uint32_t>(e[3]) << 16));
                }
            }
    };
    if (GATE) load_z(0);
    // y of the chunk's rows from head h0's slice on (the second head's columns
    // are P further), stores past the sequence end dropped
    const auto ry = brsrc(yg + static_cast<int64_t>(t0) * rowX,
                          static_cast<int64_t>(g.L - t0) * rowX * 2 -
                              static_cast<int64_t>(rowX - pcols - (HPW - 1) * g.P) * 2);
    __syncthreads();

    auto step = [&](const int k, BlockRegs<NP, true> &rg) {
        const St &st = sm.st[k & 1];
        const int base = 32 * k;
        float ck[HPW];
        uint2 x0[HPW], x1[HPW];
        bf8 xa[HPW];
#pragma unroll
        for (int hd = 0; hd < HPW; ++hd) {
            ck[hd] = k > 0 ? sm.cum[hd][base - 1] : 0.0f;
            // x of the block: row p = pl, K slots s = 16 (i / 4) + 4 g4 + i % 4
            const uint16_t *xp = &st.XT[(hd * kPG + pl) * TP];
            x0[hd] = *reinterpret_cast<const uint2 *>(xp + swz(4 * g4, pl));
            x1[hd] = *reinterpret_cast<const uint2 *>(xp + swz(16 + 4 * g4, pl));
            xa[hd] = cat8(x0[hd], x1[hd]);
        }
        // output: Y^T = Hs_k C^T (state part; one head: hi and lo parts of Hs_k
        // in chains of their own) and the diagonal tile's x^T M^T
        constexpr int YC = HPW == 1 ? 2 : 1;
        // the block's products at raised wave priority (back to normal for
        // the outputs and the staging): a wave that reaches them issues
        // first, so its matrix-core work overlaps the other waves' vector work
        // the next block into LDS first (its buffer was last read in the
        // previous block, before that block's barriers), so that the writes
        // overlap this block's products; rg then receives block k + 2
        if (k + 1 < NB) {
            store_block<NP, VEC, true>(rg, q, nmask, sm.st[(k + 1) & 1]);
            if (k + 2 < NB) load_block<NP, VEC, true>(rg, q, Bg, Cg, xg, t0 + base + 64, g, rowBC, rowX, pcols);
        }
        __builtin_amdgcn_s_setprio(1);
        f4x ys[HPW][2][YC], yd[HPW][2];
#pragma unroll
        for (int hd = 0; hd < HPW; ++hd)
#pragma unroll
            for (int tq = 0; tq < 2; ++tq)
#pragma unroll
                for (int e = 0; e < YC; ++e) ys[hd][tq][e] = zero4();
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            bf8 cb[2];
#pragma unroll
            for (int tq = 0; tq < 2; ++tq) {
                const uint16_t *cp = &st.CR[(16 * tq + l16) * CP + 32 * kk + 4 * g4];
                cb[tq] = cat8(*reinterpret_cast<const uint2 *>(cp), *reinterpret_cast<const uint2 *>(cp + 16));
            }
#pragma unroll
            for (int hd = 0; hd < HPW; ++hd) {
                uint32_t hw[4], lw[4];
                split_pk(H[hd][2 * kk][0], H[hd][2 * kk][1], hw[0], lw[0]);
                split_pk(H[hd][2 * kk][2], H[hd][2 * kk][3], hw[1], lw[1]);
                split_pk(H[hd][2 * kk + 1][0], H[hd][2 * kk + 1][1], hw[2], lw[2]);
                split_pk(H[hd][2 * kk + 1][2], H[hd][2 * kk + 1][3], hw[3], lw[3]);
                const bf8 ah = __builtin_bit_cast(bf8, make_uint4(hw[0], hw[1], hw[2], hw[3]));
                const bf8 al = __builtin_bit_cast(bf8, make_uint4(lw[0], lw[1], lw[2], lw[3]));
#pragma unroll
                for (int tq = 0; tq < 2; ++tq) {
                    ys[hd][tq][0] = mfma16(ah, cb[tq], ys[hd][tq][0]);
                    ys[hd][tq][YC - 1] = mfma16(al, cb[tq], ys[hd][tq][YC - 1]);
                }
            }
        }
#pragma unroll
        for (int hd = 0; hd < HPW; ++hd)
#pragma unroll
            for (int tq = 0; tq < 2; ++tq) {
                const bf8 mh = __builtin_bit_cast(bf8, sm.M[hd][tq][0][lane]);
                const bf8 ml = __builtin_bit_cast(bf8, sm.M[hd][tq][1][lane]);
                yd[hd][tq] = mfma16(xa[hd], mh, zero4());
                yd[hd][tq] = mfma16(xa[hd], ml, yd[hd][tq]);
            }
        float sig_k[HPW];
#pragma unroll
        for (int hd = 0; hd < HPW; ++hd) sig_k[hd] = sig[hd];
        // state entering the next block: H_{k+1} = 2^(e_k - c_k) H_k + dH_k
        // (after the chunk's last block: the state entering the next chunk)
        if (k + 1 < NB || cont) {
            bf8 xwh[HPW], xwl[HPW];
#pragma unroll
            for (int hd = 0; hd < HPW; ++hd) {
                const float rk = fast_exp2(sm.cum[hd][base + 31] - ck[hd]);
                const float sn = sig[hd] * rk;
                float wsc = 1.0f;             // weight of the block's new terms
                if (sn >= 0x1p-64f) {
                    wsc = __builtin_amdgcn_rcpf(sn);
                    sig[hd] = sn;
                } else {
#pragma unroll
                    for (int j = 0; j < NJ; ++j) H[hd][j] = H[hd][j] * sn;
                    sig[hd] = 1.0f;
                }
                const float4 f0 = *reinterpret_cast<const float4 *>(&sm.fs[hd][base + 4 * g4]);
                const float4 f1 = *reinterpret_cast<const float4 *>(&sm.fs[hd][base + 16 + 4 * g4]);
                uint32_t xh[4], xl[4];
                split_pk(bits_lo(x0[hd].x) * f0.x * wsc, bits_hi(x0[hd].x) * f0.y * wsc, xh[0], xl[0]);
                split_pk(bits_lo(x0[hd].y) * f0.z * wsc, bits_hi(x0[hd].y) * f0.w * wsc, xh[1], xl[1]);
                split_pk(bits_lo(x1[hd].x) * f1.x * wsc, bits_hi(x1[hd].x) * f1.y * wsc, xh[2], xl[2]);
                split_pk(bits_lo(x1[hd].y) * f1.z * wsc, bits_hi(x1[hd].y) * f1.w * wsc, xh[3], xl[3]);
                xwh[hd] = __builtin_bit_cast(bf8, make_uint4(xh[0], xh[1], xh[2], xh[3]));
                xwl[hd] = __builtin_bit_cast(bf8, make_uint4(xl[0], xl[1], xl[2], xl[3]));
            }
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const uint16_t *bp = &st.BT[(16 * j + l16) * TP];
                const bf8 bt = cat8(*reinterpret_cast<const uint2 *>(bp + swz(4 * g4, 16 * j)),
                                    *reinterpret_cast<const uint2 *>(bp + swz(16 + 4 * g4, 16 * j)));
#pragma unroll
                for (int hd = 0; hd < HPW; ++hd) {
                    H[hd][j] = mfma16(bt, xwh[hd], H[hd][j]);
                    H[hd][j] = mfma16(bt, xwl[hd], H[hd][j]);
                }
            }
        }
        __builtin_amdgcn_s_setprio(0);
        // the next block's decay tile values (stored after this block's
        // reads of M), then the Gram quadrant of the block after it; past
        // the chunk's last block both are formed from in-range indices and
        // left unused
        uint4 mv[HPW];
        diag_vals<Q, NP, HPW>(gq, sm, k + 1 < NB ? base + 32 : base, skip, wave, lane, mv);
        gq = Gw[static_cast<int64_t>(c * NB + (k + 2 < NB ? k + 2 : NB - 1)) * 192];
        // y at this lane's steps of the block, four columns each
#pragma unroll
        for (int hd = 0; hd < HPW; ++hd)
#pragma unroll
            for (int tq = 0; tq < 2; ++tq) {
                const int tl = base + 16 * tq + l16;
                const float ft = fast_exp2(sm.cum[hd][tl] - ck[hd]) * sig_k[hd];
                float yv[4];
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    yv[v] = fmaf(ft, YC == 2 ? ys[hd][tq][0][v] + ys[hd][tq][YC - 1][v] : ys[hd][tq][0][v],
                                 yd[hd][tq][v]);
                if (GATE) {
                    yv[0] *= silu(bits_lo(zr[hd][tq].x));
                    yv[1] *= silu(bits_hi(zr[hd][tq].x));
                    yv[2] *= silu(bits_lo(zr[hd][tq].y));
                    yv[3] *= silu(bits_hi(zr[hd][tq].y));
                }
                if (VEC) {
                    // rows past the sequence end fall outside the resource
                    if (p4 < pcols)
                        __builtin_amdgcn_raw_buffer_store_b64(
                            __builtin_bit_cast(__attribute__((ext_vector_type(2))) uint32_t,
                                               make_uint2(cvt_pk(yv[0], yv[1]), cvt_pk(yv[2], yv[3]))),
                            ry, static_cast<uint32_t>((tl * rowX + hd * g.P + p4) * 2), 0, 0);
                } else if (t0 + tl < g.L) {
                    uint16_t *py = yg + hd * g.P + static_cast<int64_t>(t0 + tl) * rowX + p4;
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        if (p4 + v < pcols) py[v] = f32_to_bf16(yv[v]);
                }
            }
        if (k + 1 < NB) {
            // the next block's decay tiles, after every read of this block's
            // (the first barrier also publishes the next block's rows)
            __syncthreads();
            if (wave < 3) diag_store<Q, NP, HPW>(sm, mv, wave, lane);
            if (GATE) load_z(k + 1);
            __syncthreads();
        }
    };
    // NB is even
#pragma unroll 1
    for (int k = 0; k < NB; k += 2) {
        step(k, ra);
        step(k + 1, ra);
    }
    }
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

    // chunk-pair states and decays (one per pair of consecutive chunks)
    const int64_t chunks = a.batch * ((g.nch + 1) / 2) * a.H;
    const int64_t PN = a.P * a.N;
    const size_t s_bytes = static_cast<size_t>(chunks * PN) * sizeof(float);
    const size_t ce_bytes = static_cast<size_t>(chunks) * sizeof(float);
    // Gram quadrants: 3 x 64 float4 per (batch, group, 32-step block)
    const int nblk = g.nch * (Q / 32);
    const size_t g_bytes = static_cast<size_t>(a.batch * a.G * nblk) * 3 * 64 * sizeof(f4x);
    // (each part 256-byte aligned)
    const size_t s_pad = (s_bytes + 255) & ~size_t(255), ce_pad = (ce_bytes + 255) & ~size_t(255);
    void *mem = nullptr;
    hipError_t e = scratch_alloc(&mem, s_pad + ce_pad + g_bytes, stream);
    if (e != hipSuccess) return e;
    float *S = static_cast<float *>(mem);
    float *ce = reinterpret_cast<float *>(static_cast<char *>(mem) + s_pad);
    f4x *Gq = reinterpret_cast<f4x *>(static_cast<char *>(mem) + s_pad + ce_pad);

    const auto *x = static_cast<const uint16_t *>(a.x);
    const auto *dt = static_cast<const uint16_t *>(a.dt);
    const auto *B = static_cast<const uint16_t *>(a.B);
    const auto *C = static_cast<const uint16_t *>(a.C);
    const auto *zz = static_cast<const uint16_t *>(a.z);
    const bool vec = vecB && vecX;
    // one workgroup per (batch, pair of consecutive chunks, 64-column
    // head-dimension slice) and one head, or in the state kernel two where
    // each group's head count is even
    const bool pairs = (a.H / a.G) % 2 == 0;
    const int64_t npair = (g.nch + 1) / 2;
    // chunks per output workgroup: four where that still gives at least
    // three workgroups per compute unit of a 256-CU device (half the
    // entering states stored and read), else two.  Only the vector path
    // runs three output workgroups per CU; the element path runs two, where
    // four-chunk walks would leave a half-filled last round.
    const bool three_per_cu = vec;
    const int cpw = three_per_cu && a.batch * ((g.nch + 3) / 4) * a.H * g.npg >= 768 ? 4 : 2;
    // the state workgroups, then those of the Gram quadrants (four each)
    const int nstate = static_cast<int>(a.batch * npair * (pairs ? a.H / 2 : a.H) * g.npg);
    const int ntask = static_cast<int>(a.batch * a.G * nblk * 3);
    const dim3 sgrid(static_cast<uint32_t>(nstate + (ntask + 3) / 4));
    if (vec && pairs)
        hipLaunchKernelGGL((ssd_state_kernel<Q, NP, true, 2>), sgrid, dim3(256), 0, stream, x, dt, a.dt_bias, a.A,
                           B, S, ce, g, C, Gq, nstate, nblk, ntask);
    else if (vec)
        hipLaunchKernelGGL((ssd_state_kernel<Q, NP, true, 1>), sgrid, dim3(256), 0, stream, x, dt, a.dt_bias, a.A,
                           B, S, ce, g, C, Gq, nstate, nblk, ntask);
    else if (pairs)
        hipLaunchKernelGGL((ssd_state_kernel<Q, NP, false, 2>), sgrid, dim3(256), 0, stream, x, dt, a.dt_bias, a.A,
                           B, S, ce, g, C, Gq, nstate, nblk, ntask);
    else
        hipLaunchKernelGGL((ssd_state_kernel<Q, NP, false, 1>), sgrid, dim3(256), 0, stream, x, dt, a.dt_bias, a.A,
                           B, S, ce, g, C, Gq, nstate, nblk, ntask);
    e = hipGetLastError();
    if (e == hipSuccess) {
        const int bph = static_cast<int>((PN + 255) / 256);
        const dim3 pgrid(static_cast<uint32_t>(a.batch * a.H * bph));
        if (cpw == 4)
            hipLaunchKernelGGL(ssd_pass_kernel<2>, pgrid, dim3(256), 0, stream, S, ce, a.h0, a.h_last, g, bph);
        else
            hipLaunchKernelGGL(ssd_pass_kernel<1>, pgrid, dim3(256), 0, stream, S, ce, a.h0, a.h_last, g, bph);
        e = hipGetLastError();
    }
    if (e == hipSuccess) {
        // one head and cpw consecutive chunks per workgroup
        decltype(&ssd_output_kernel<Q, NP, true, true, 1>) kern;
        if (zz) kern = vec ? ssd_output_kernel<Q, NP, true, true, 1> : ssd_output_kernel<Q, NP, false, true, 1>;
        else kern = vec ? ssd_output_kernel<Q, NP, true, false, 1> : ssd_output_kernel<Q, NP, false, false, 1>;
        const dim3 ogrid(static_cast<uint32_t>(a.batch * ((g.nch + cpw - 1) / cpw) * a.H * g.npg));
        hipLaunchKernelGGL(kern, ogrid, dim3(256), 0, stream, x, dt, a.dt_bias, a.A, B, C, a.D, zz, S, Gq,
                           static_cast<uint16_t *>(a.y), g, cpw);
        e = hipGetLastError();
    }
    const hipError_t ef = scratch_free(mem, stream);
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
    // byte offsets of a chunk's rows from its first row fit in 31 bits
    if (a.chunk * a.H * a.P * 2 >= lim || a.chunk * a.G * a.N * 2 >= lim) return false;
    if (!(a.io == IO_BF16 && a.N >= 1 && a.N <= 128 && a.P >= 1 &&
          (a.chunk == 64 || a.chunk == 128 || a.chunk == 256) && nch < (int64_t(1) << 30)))
        return false;
    // each launch's grid in work-items (256 per workgroup) stays below 2^32
    const int64_t wmax = int64_t(1) << 24;
    const int64_t npair = (nch + 1) / 2, npg = (a.P + kPG - 1) / kPG;
    const int64_t nstate = a.batch * npair * a.H * npg;
    const int64_t ntask = a.batch * a.G * nch * (a.chunk / 32) * 3;
    return nstate < wmax && nstate + (ntask + 3) / 4 < wmax &&
           a.batch * a.H * ((a.P * a.N + 255) / 256) < wmax;
}

hipError_t launch_ssd_chunked(const SSDArgs &a, hipStream_t stream) {
    if (a.chunk == 64) return launch_by_n<64>(a, stream);
    if (a.chunk == 128) return launch_by_n<128>(a, stream);
    return launch_by_n<256>(a, stream);
}

}  // namespace mssm
