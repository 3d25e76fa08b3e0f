// scan_pairscan.hip -- selective-scan forward with the sequence of every row
// split across the lanes of a workgroup: a scan of (decay, state) pairs
// inside the workgroup, for shapes whose channels alone give the chunked
// kernel too few waves to keep the SIMDs issuing (one wave or less per SIMD).
//
// The recurrence h_t = a_t h_{t-1} + b_t (a_t = exp(dl_t A), b_t = dl_t u_t
// B_t) over a run of steps composes into one pair (P, h): the product of the
// decays and the state reached from h = 0; the pair of a run applied to the
// state entering it gives the state leaving it, and pairs compose with the
// associative operator (P1,h1) (+) (P2,h2) = (P2 P1, P2 h1 + h2)
// (www.mhpq.cn/news/984979 essay section 2.3: the pair operator, and the
// scan of a sequence as local sweeps, a scan of the block totals, and a
// fix-up; section 3.3: the same at warp, block and grid level).
//
// A workgroup owns one batch and 16 channels and walks the sequence in
// chunks of kChunk steps, carrying the state between chunks in registers.
// Lane (slice th, state wave sg, row r, column j) holds channel j and the
// state elements n = 2 sg + g (g < 2) for the SEG steps of time segment
// (th, r) of the chunk.  Per chunk:
//
//   A. owner threads compute the per-step scalars once per (channel, step):
//      dl = softplus(delta + bias), dl*u, D*u and silu(z), and publish dl
//      and dl*u in LDS;
//   B. every lane walks its SEG steps from h = 0, keeping the local state
//      h_loc_t and the running decay product P_t of every step in
//      registers;
//   C. the segments' pairs (P, h_loc) are scanned across the four rows of
//      the wave with two cross-row swap levels (v_permlane16_swap pairs rows
//      0-1 and 2-3, v_permlane32_swap pairs rows 0-1 with 2-3), which gives
//      every row its exclusive prefix and the wave's total; with two time
//      slices per chunk, the slices' totals are combined through LDS;
//   D. the carried state h_in of the segment is the prefix applied to the
//      state entering the chunk, and every step's state is
//      h_t = P_t h_in + h_loc_t -- one fused multiply-add per element;
//      C.h over the lane's two state elements goes to LDS, the owner of
//      (channel, step) adds the eight state waves' sums, the skip term and
//      the gate, and stores y.
//
// B values are shared by the 16 channels of a row: lane j of a row holds
// B[n, t] of step j of the row's segment, and the multiply takes it through
// a DPP row broadcast (the same device as the chunked kernel).  Every
// element costs one exponential, as in a serial walk, plus the running
// product and the fix-up: the work per element grows by about a third, and
// the number of waves by eight (one slice) or sixteen (two slices) per
// 16-channel group instead of four.
//
// The chunk's carry is the last segment's inclusive pair applied to the
// entering state, the same in every lane, so results are bitwise
// repeatable; they differ from the sequential loop by the association of
// the pairs inside a chunk.
#include <type_traits>
#include <utility>

#include "internal.h"
#include "scan_core.h"

namespace mssm {
namespace {

using core::buffer_ld;
using core::buffer_rsrc;
using core::kCh;
using core::Pack;
using core::row_bcast;

template <int... S, typename F>
__device__ __forceinline__ void for_each_step(std::integer_sequence<int, S...>, F &&f) {
    (f(std::integral_constant<int, S>{}), ...);
}

// A run of steps as a pair: decay product p and state h reached from 0.
struct Pair {
    float p, h;
};
// x followed by y.
__device__ __forceinline__ Pair compose(Pair x, Pair y) { return {y.p * x.p, fmaf(y.p, x.h, y.h)}; }

// Value of v in the even and in the odd row of this lane's row pair
// (rows 0-1, 2-3), in every lane of the pair: v_permlane16_swap exchanges
// the odd rows of its first operand with the even rows of its second, so
// with v in both, the first result holds the even row's v and the second
// the odd row's.
__device__ __forceinline__ void row_pair(float v, float &even, float &odd) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    even = __uint_as_float(r[0]);
    odd = __uint_as_float(r[1]);
}
// The same between the lower half (rows 0-1) and the upper half (rows 2-3).
__device__ __forceinline__ void half_pair(float v, float &lo, float &hi) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    lo = __uint_as_float(r[0]);
    hi = __uint_as_float(r[1]);
}

template <typename T, int TH, int SEG, bool GATE, bool VEC>
struct PairScan {
    static constexpr int SG = 8;                        // state waves per slice
    static constexpr int NPL = 2;                       // state elements per lane
    static constexpr int W = TH * SG;                   // waves
    static constexpr int NT = 64 * W;                   // threads
    static constexpr int kSlice = 4 * SEG;              // steps of one slice (four rows)
    static constexpr int kChunk = TH * kSlice;
    static constexpr int kPitch = kChunk + 4;           // LDS row pitch (floats)
    static constexpr int OS0 = kCh * kChunk / NT;
    static constexpr int OS = OS0 >= 2 ? OS0 : 2;       // steps per owner thread
    static constexpr int NOWN = kCh * kChunk / OS;      // owner threads: tid < NOWN
    static constexpr int OPC = kChunk / OS;             // owner threads per channel
    static_assert(SEG % 4 == 0 && SEG <= 16, "a segment is at most one row of steps");
    static_assert(NOWN % 64 == 0 && NOWN <= NT, "owners are whole waves");
    using Raw = typename Pack<T, OS>::raw;

    struct Smem {
        float dl[2][kCh * kPitch];
        float du[2][kCh * kPitch];
        float part[2][SG][kCh * kPitch];                // C.h of state wave sg per (channel, step)
        float tot[TH][2][SG * NPL * kCh];               // totals of the slices (P, h)
    };

    struct In {
        Raw ru, rd, rz;                                 // owner: OS steps of u, delta (and z)
        T rb[NPL], rc[NPL];                             // lane: B, C of step j % SEG of its segment
    };
    struct Own {
        float uu[OS], gz[OS];
        int rem;
    };

    // lane role
    int th, sg, r, j, seg_off;
    float A2[NPL];
    bool nok[NPL];
    uint32_t bcj[NPL];
    const T *Bb, *Cb;
    int32_t rec_a, rec_bc;
    // owner role
    bool owner;
    int oc, ok;
    uint32_t oo;
    const T *ub, *db, *zb;
    T *yb;
    float bias, skip;
    int L;

    __device__ void init(const T *u, const T *delta, const float *delta_bias, const float *A,
                         const T *B, const T *C, const float *Dskip, const T *z, T *y, int64_t L_,
                         int dim, int N, int64_t b, int d0) {
        const int tid = threadIdx.x;
        const int w = tid >> 6;
        th = w / SG;
        sg = w - th * SG;
        r = (tid >> 4) & 3;
        j = tid & 15;
        seg_off = th * kSlice + r * SEG;
        L = static_cast<int>(L_);
        Bb = B + b * N * L_;
        Cb = C + b * N * L_;
        const int dS = min(d0 + j, dim - 1);
#pragma unroll
        for (int g = 0; g < NPL; ++g) {
            const int n = NPL * sg + g;
            nok[g] = n < N;
            A2[g] = nok[g] ? A[static_cast<int64_t>(dS) * N + n] * kLog2e : 0.0f;
            // rows past N load through an offset past every buffer's end,
            // which reads zero
            bcj[g] = nok[g] ? (static_cast<uint32_t>(n) * static_cast<uint32_t>(L) +
                               static_cast<uint32_t>(seg_off + (j % SEG))) * sizeof(T)
                            : 0xffffff00u;
        }
        owner = tid < NOWN;
        oc = tid / OPC;
        ok = tid - oc * OPC;
        if (!owner) oc = 0, ok = 0;
        // channels past the last one compute on the last channel's inputs
        // and store the same values into its row
        const int dO = min(d0 + oc, dim - 1);
        const int64_t row0 = (b * dim + d0) * L_;
        oo = static_cast<uint32_t>(dO - d0) * static_cast<uint32_t>(L) * sizeof(T);
        bias = delta_bias ? delta_bias[dO] : 0.0f;
        skip = Dskip ? Dskip[dO] : 0.0f;
        ub = u + row0;
        db = delta + row0;
        zb = GATE ? z + row0 : nullptr;
        yb = y + row0;
        rec_a = min(kCh, dim - d0) * L * static_cast<int32_t>(sizeof(T));
        rec_bc = N * L * static_cast<int32_t>(sizeof(T));
    }

    // Loads of the chunk at t0, issued a chunk before their use.
    __device__ void load(int t0, In &in) const {
        const int32_t tb = t0 * static_cast<int32_t>(sizeof(T));
        if (owner) {
            if constexpr (VEC) {
                // rows 16-byte aligned, L % 8 == 0, OS | 8: the OS steps are
                // all inside the row or all past its end (then discarded)
                const uint32_t o = oo + static_cast<uint32_t>(OS * ok) * sizeof(T);
                in.ru = buffer_ld<Raw>(buffer_rsrc(reinterpret_cast<const char *>(ub) + tb, rec_a - tb), o);
                in.rd = buffer_ld<Raw>(buffer_rsrc(reinterpret_cast<const char *>(db) + tb, rec_a - tb), o);
                if (GATE)
                    in.rz = buffer_ld<Raw>(buffer_rsrc(reinterpret_cast<const char *>(zb) + tb, rec_a - tb), o);
            } else {
                T su[OS], sd[OS], sz[OS];
                const int off = t0 + OS * ok;
#pragma unroll
                for (int i = 0; i < OS; ++i) {
                    const int t = off + i < L ? off + i : L - 1;
                    const uint32_t o = oo + static_cast<uint32_t>(t) * sizeof(T);
                    su[i] = *reinterpret_cast<const T *>(reinterpret_cast<const char *>(ub) + o);
                    sd[i] = *reinterpret_cast<const T *>(reinterpret_cast<const char *>(db) + o);
                    sz[i] = GATE ? *reinterpret_cast<const T *>(reinterpret_cast<const char *>(zb) + o) : T(0);
                }
                __builtin_memcpy(&in.ru, su, sizeof(Raw));
                __builtin_memcpy(&in.rd, sd, sizeof(Raw));
                __builtin_memcpy(&in.rz, sz, sizeof(Raw));
            }
        }
        const auto rB = buffer_rsrc(reinterpret_cast<const char *>(Bb) + tb, rec_bc - tb);
        const auto rC = buffer_rsrc(reinterpret_cast<const char *>(Cb) + tb, rec_bc - tb);
#pragma unroll
        for (int g = 0; g < NPL; ++g) {
            in.rb[g] = buffer_ld<T>(rB, bcj[g]);
            in.rc[g] = buffer_ld<T>(rC, bcj[g]);
        }
    }

    __device__ static float to_f32(T v) {
        if constexpr (sizeof(T) == 4) return v;
        else return __uint_as_float(static_cast<uint32_t>(v) << 16);
    }

    // ---- A: per-step scalars of the owner's OS steps of the chunk at t0 ----
    template <bool FULL>
    __device__ void phase_a(int t0, int t_end, const In &in, Smem &sm, int buf, Own &o) const {
        if (!owner) return;
        float u[OS], dr[OS], zz[OS];
        Pack<T, OS>::unpack(in.ru, u);
        Pack<T, OS>::unpack(in.rd, dr);
        if (GATE) Pack<T, OS>::unpack(in.rz, zz);
        int rem = OS;
        if (!FULL) rem = min(t_end - (t0 + OS * ok), OS);
        o.rem = rem;
        float dl[OS], du[OS];
#pragma unroll
        for (int i = 0; i < OS; ++i) {
            // steps past the end become the identity step dl = 0, dl*u = 0
            const float sp = softplus(dr[i] + bias);
            dl[i] = (FULL || i < rem) ? sp : 0.0f;
            du[i] = (FULL || i < rem) ? sp * u[i] : 0.0f;
            o.uu[i] = u[i];
            o.gz[i] = GATE ? silu(zz[i]) : 1.0f;
        }
#pragma unroll
        for (int i = 0; i < OS; i += 2) {
            *reinterpret_cast<float2 *>(sm.dl[buf] + oc * kPitch + OS * ok + i) = make_float2(dl[i], dl[i + 1]);
            *reinterpret_cast<float2 *>(sm.du[buf] + oc * kPitch + OS * ok + i) = make_float2(du[i], du[i + 1]);
        }
    }

    // ---- B-D: the lane's segment of the chunk at t0, from the carried state
    // `carry` (updated to the state leaving the chunk); p[s] = C.h of its
    // state elements at step s of its segment.  Every thread calls it.
    template <bool FULL>
    __device__ void lanes(int t0, int t_end, const In &in, Smem &sm, int buf, float (&carry)[NPL],
                          float (&p)[SEG]) const {
        float dls[SEG], dus[SEG];
        const float4 *pdl = reinterpret_cast<const float4 *>(sm.dl[buf] + j * kPitch + seg_off);
        const float4 *pdu = reinterpret_cast<const float4 *>(sm.du[buf] + j * kPitch + seg_off);
#pragma unroll
        for (int k = 0; k < SEG / 4; ++k) {
            const float4 a = pdl[k], e = pdu[k];
            dls[4 * k] = a.x; dls[4 * k + 1] = a.y; dls[4 * k + 2] = a.z; dls[4 * k + 3] = a.w;
            dus[4 * k] = e.x; dus[4 * k + 1] = e.y; dus[4 * k + 2] = e.z; dus[4 * k + 3] = e.w;
        }
        // B, C of the row broadcasts (zero past the end; state rows past N
        // loaded zero)
        const bool tok = FULL || t0 + seg_off + (j % SEG) < t_end;
        float cb[NPL], cc[NPL];
#pragma unroll
        for (int g = 0; g < NPL; ++g) {
            cb[g] = tok ? to_f32(in.rb[g]) : 0.0f;
            cc[g] = tok ? to_f32(in.rc[g]) : 0.0f;
        }
        // B. local walk from h = 0: h_loc and the running decay product
        float hl[NPL][SEG], pc[NPL][SEG];
        for_each_step(std::make_integer_sequence<int, SEG>{}, [&](auto s_) {
            constexpr int S = decltype(s_)::value;
#pragma unroll
            for (int g = 0; g < NPL; ++g) {
                const float a = fast_exp2(dls[S] * A2[g]);
                const float bu = row_bcast<S>(cb[g]) * dus[S];
                if constexpr (S == 0) {
                    hl[g][0] = bu;
                    pc[g][0] = a;
                } else {
                    hl[g][S] = fmaf(a, hl[g][S - 1], bu);
                    pc[g][S] = pc[g][S - 1] * a;
                }
            }
        });
        // C. scan of the four rows' segment pairs: exclusive prefix e of this
        // row and the total t of the wave
        Pair e[NPL], t[NPL];
        const bool odd = (r & 1) != 0, upper = r >= 2;
#pragma unroll
        for (int g = 0; g < NPL; ++g) {
            Pair xe, xo;
            row_pair(pc[g][SEG - 1], xe.p, xo.p);
            row_pair(hl[g][SEG - 1], xe.h, xo.h);
            const Pair t1 = compose(xe, xo);
            const Pair lx = odd ? xe : Pair{1.0f, 0.0f};
            Pair lo, hi;
            half_pair(t1.p, lo.p, hi.p);
            half_pair(t1.h, lo.h, hi.h);
            t[g] = compose(lo, hi);
            e[g] = upper ? compose(lo, lx) : lx;
        }
        // state entering this slice, and the state leaving the chunk
        float c_in[NPL];
        if constexpr (TH == 1) {
#pragma unroll
            for (int g = 0; g < NPL; ++g) {
                c_in[g] = carry[g];
                carry[g] = fmaf(t[g].p, carry[g], t[g].h);
            }
        } else {
            if (r == 0) {
#pragma unroll
                for (int g = 0; g < NPL; ++g) {
                    sm.tot[th][0][(sg * NPL + g) * kCh + j] = t[g].p;
                    sm.tot[th][1][(sg * NPL + g) * kCh + j] = t[g].h;
                }
            }
            __syncthreads();
#pragma unroll
            for (int g = 0; g < NPL; ++g) {
                float c = carry[g];
                c_in[g] = c;
#pragma unroll
                for (int s = 0; s < TH; ++s) {
                    c = fmaf(sm.tot[s][0][(sg * NPL + g) * kCh + j], c,
                             sm.tot[s][1][(sg * NPL + g) * kCh + j]);
                    if (s + 1 == th) c_in[g] = c;
                }
                carry[g] = c;
            }
        }
        // D. fix-up: h_t = P_t h_in + h_loc_t, and C.h
        float hin[NPL];
#pragma unroll
        for (int g = 0; g < NPL; ++g) hin[g] = fmaf(e[g].p, c_in[g], e[g].h);
        for_each_step(std::make_integer_sequence<int, SEG>{}, [&](auto s_) {
            constexpr int S = decltype(s_)::value;
            float acc = 0.0f;
#pragma unroll
            for (int g = 0; g < NPL; ++g) {
                const float h = fmaf(pc[g][S], hin[g], hl[g][S]);
                acc = g == 0 ? row_bcast<S>(cc[g]) * h : fmaf(row_bcast<S>(cc[g]), h, acc);
            }
            p[S] = acc;
        });
    }

    __device__ void store_part(const float (&p)[SEG], Smem &sm, int pbuf) const {
        float4 *dst = reinterpret_cast<float4 *>(sm.part[pbuf][sg] + j * kPitch + seg_off);
#pragma unroll
        for (int k = 0; k < SEG / 4; ++k) dst[k] = make_float4(p[4 * k], p[4 * k + 1], p[4 * k + 2], p[4 * k + 3]);
    }

    // ---- output: the owner adds the state waves' sums of its OS steps ----
    template <bool FULL>
    __device__ void phase_c(int t0, const Own &o, const Smem &sm, int pbuf) const {
        if (!owner) return;
        float yv[OS];
#pragma unroll
        for (int i = 0; i < OS; ++i) yv[i] = 0.0f;
#pragma unroll
        for (int w = 0; w < SG; ++w) {
            const float *src = sm.part[pbuf][w] + oc * kPitch + OS * ok;
#pragma unroll
            for (int i = 0; i < OS; i += 2) {
                const float2 v = *reinterpret_cast<const float2 *>(src + i);
                yv[i] += v.x;
                yv[i + 1] += v.y;
            }
        }
#pragma unroll
        for (int i = 0; i < OS; ++i) yv[i] = fmaf(skip, o.uu[i], yv[i]) * o.gz[i];
        T *py = reinterpret_cast<T *>(reinterpret_cast<char *>(yb) + oo) + (t0 + OS * ok);
        if (FULL) {
            if (VEC) {
                Pack<T, OS>::store(py, yv);
            } else {
#pragma unroll
                for (int i = 0; i < OS; ++i) Io<T>::store(py, i, yv[i]);
            }
        } else {
#pragma unroll
            for (int i = 0; i < OS; ++i)
                if (i < o.rem) Io<T>::store(py, i, yv[i]);
        }
    }

    // Stage k: publish chunk k + 1's step scalars and chunk k's sums, one
    // barrier, chunk k's outputs, chunk k + 1's lanes.  Loads run two chunks
    // ahead: xk is free once chunk k's lanes are done.  FN: chunk k + 1 is
    // full; chunk k is.  LDS buffers alternate with the chunk, and each is
    // rewritten two stages after it was written, past a barrier that all its
    // readers passed.
    template <bool FN>
    __device__ void stage(int k, int t_end, In &xk, const In &xk1, const Own &ok_, Own &ok1,
                          float (&carry)[NPL], float (&p)[SEG], Smem &sm) const {
        const int tk = k * kChunk;
        load(tk + 2 * kChunk, xk);
        phase_a<FN>(tk + kChunk, t_end, xk1, sm, (k + 1) & 1, ok1);
        store_part(p, sm, k & 1);
        __syncthreads();
        phase_c<true>(tk, ok_, sm, k & 1);
        lanes<FN>(tk + kChunk, t_end, xk1, sm, (k + 1) & 1, carry, p);
    }

    __device__ void last(int k, bool full, const float (&p)[SEG], const Own &o, Smem &sm) const {
        store_part(p, sm, k & 1);
        __syncthreads();
        if (full) phase_c<true>(k * kChunk, o, sm, k & 1);
        else phase_c<false>(k * kChunk, o, sm, k & 1);
    }

    // The whole row group from the state `carry` (updated to the final state).
    __device__ void walk(float (&carry)[NPL], Smem &sm) const {
        const int t_end = L;
        const int nfull = L / kChunk;
        const int nch = (L + kChunk - 1) / kChunk;
        In xa, xb;
        Own oa, ob;
        float p[SEG];
        load(0, xa);
        load(kChunk, xb);
        if (nfull > 0) {
            phase_a<true>(0, t_end, xa, sm, 0, oa);
            __syncthreads();
            lanes<true>(0, t_end, xa, sm, 0, carry, p);
        } else {
            phase_a<false>(0, t_end, xa, sm, 0, oa);
            __syncthreads();
            lanes<false>(0, t_end, xa, sm, 0, carry, p);
        }
        int k = 0;
        for (; k + 2 < nfull; k += 2) {
            stage<true>(k, t_end, xa, xb, oa, ob, carry, p, sm);
            stage<true>(k + 1, t_end, xb, xa, ob, oa, carry, p, sm);
        }
        const bool last_full = nch == nfull;
        if (k + 1 < nch) {
            if (k + 1 < nfull) stage<true>(k, t_end, xa, xb, oa, ob, carry, p, sm);
            else stage<false>(k, t_end, xa, xb, oa, ob, carry, p, sm);
            ++k;
            if (k + 1 < nch) {
                stage<false>(k, t_end, xb, xa, ob, oa, carry, p, sm);
                ++k;
                last(k, last_full, p, oa, sm);
            } else {
                last(k, last_full, p, ob, sm);
            }
        } else {
            last(k, last_full, p, oa, sm);
        }
    }
};

template <typename T, int TH, int SEG, bool GATE, bool VEC>
__global__ __launch_bounds__(512 * TH) void scan_pairscan_kernel(
    const T *__restrict__ u, const T *__restrict__ delta, const float *__restrict__ delta_bias,
    const float *__restrict__ A, const T *__restrict__ Bm, const T *__restrict__ Cm,
    const float *__restrict__ Dskip, const T *__restrict__ z, const float *h0, T *__restrict__ y,
    float *h_last, int64_t L, int dim, int N, int groups_per_batch) {
    using PS = PairScan<T, TH, SEG, GATE, VEC>;
    static_assert(PS::NT == 512 * TH, "eight state waves per slice");
    __shared__ typename PS::Smem sm;
    const int grp = blockIdx.x;
    const int64_t b = grp / groups_per_batch;
    const int d0 = (grp - static_cast<int>(b) * groups_per_batch) * kCh;
    PS ps;
    ps.init(u, delta, delta_bias, A, Bm, Cm, Dskip, z, y, L, dim, N, b, d0);
    // lanes of channels past the last one mirror the last channel
    const int dS = min(d0 + ps.j, dim - 1);
    float carry[PS::NPL];
#pragma unroll
    for (int g = 0; g < PS::NPL; ++g)
        carry[g] = (h0 && ps.nok[g])
                       ? h0[(b * dim + dS) * static_cast<int64_t>(N) + PS::NPL * ps.sg + g]
                       : 0.0f;
    ps.walk(carry, sm);
    // every lane holds the final state of its (channel, state element); the
    // lanes of the first row of the first slice store it
    if (h_last && ps.th == 0 && ps.r == 0 && d0 + ps.j < dim) {
#pragma unroll
        for (int g = 0; g < PS::NPL; ++g)
            if (ps.nok[g])
                h_last[(b * dim + d0 + ps.j) * static_cast<int64_t>(N) + PS::NPL * ps.sg + g] = carry[g];
    }
}

template <typename T, int TH, int SEG>
hipError_t launch_typed(const ScanArgs &a, hipStream_t stream) {
    const int groups = static_cast<int>((a.dim + kCh - 1) / kCh);
    const int64_t total = a.batch * groups;
    const bool vec = scan_rows_vectorizable(a);
    using K = decltype(&scan_pairscan_kernel<T, TH, SEG, true, true>);
    K kern;
    if (a.z) kern = vec ? scan_pairscan_kernel<T, TH, SEG, true, true> : scan_pairscan_kernel<T, TH, SEG, true, false>;
    else kern = vec ? scan_pairscan_kernel<T, TH, SEG, false, true> : scan_pairscan_kernel<T, TH, SEG, false, false>;
    hipLaunchKernelGGL(kern, dim3(static_cast<uint32_t>(total)), dim3(PairScan<T, TH, SEG, true, true>::NT), 0,
                       stream, static_cast<const T *>(a.u), static_cast<const T *>(a.delta), a.delta_bias,
                       a.A, static_cast<const T *>(a.B), static_cast<const T *>(a.C), a.D,
                       static_cast<const T *>(a.z), a.h0, static_cast<T *>(a.y), a.h_last, a.L,
                       static_cast<int>(a.dim), static_cast<int>(a.N), groups);
    return hipGetLastError();
}

}  // namespace

bool scan_pairscan_supported(const ScanArgs &a) {
    const int64_t groups = (a.dim + kCh - 1) / kCh;
    return a.N >= 1 && a.N <= 16 && !a.conv_w && scan_offsets_fit(a) &&
           a.batch * groups < (int64_t(1) << 30) && a.L < (int64_t(1) << 30);
}

hipError_t launch_scan_pairscan(const ScanArgs &a, hipStream_t stream, int slices) {
    if (slices == 2) {
        if (a.io == IO_F32) return launch_typed<float, 2, 8>(a, stream);
        return launch_typed<uint16_t, 2, 8>(a, stream);
    }
    if (a.io == IO_F32) return launch_typed<float, 1, 16>(a, stream);
    return launch_typed<uint16_t, 1, 16>(a, stream);
}

}  // namespace mssm
