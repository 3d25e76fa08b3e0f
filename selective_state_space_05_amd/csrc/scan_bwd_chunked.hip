// scan_bwd_chunked.hip -- backward of the selective scan for N <= 16 with
// the chunked forward's decomposition: a workgroup owns one batch and 16
// channels, lane (wave w, row r, column j) holds channel j and state element
// n = 4 w + r, and the sequence is walked in chunks of 32 steps.
//
// Forward per step ("Mamba状态空间模型的硬件感知推理优化" (ybb.press) sections 1
// and 3.1; www.mhpq.cn/news/984979 essay section 2.2; the tencentcloud.csdn.net
// Mamba article, sections 2-3):
//   x = delta + bias, dl = softplus(x), a[n] = exp(dl A[n])
//   h[n] = a[n] h[n] + dl B[n] u,  s = sum_n C[n] h[n] + D u,  y = s silu(z)
// Reverse (the chain rule through each step, from dh = dh_last at the end;
// the block is trained forward and backward, www.mlqm.cn/news/983902 essay
// section 3.2, and its intermediate states are recomputed rather than kept,
// the tencentcloud.csdn.net article section 1):
//   ds = dy silu(z), dz = dy s silu'(z)
//   dh_t[n] = ds_t C_t[n] + g_t[n],     g_{t-1}[n] = a_t[n] dh_t[n]
//   q_t[n]  = g_{t-1}[n] h_{t-1}[n]     (= dh_t a_t h_{t-1})
//   dA[n] += q_t[n] dl_t,  dC_t[n] += ds_t h_t[n],  dB_t[n] += dh_t[n] dl_t u_t
//   du_t = ds_t D + dl_t sum_n dh_t[n] B_t[n]
//   d(dl_t) = sum_n q_t[n] A[n] + u_t sum_n dh_t[n] B_t[n]
//   ddelta_t = d(dl_t) sigmoid(x_t),  dbias += ddelta_t,  dD += ds_t u_t
//   dh0 = g_{-1}.
//
// Three kernels:
//   1. scan_bwd_ckpt_kernel: the forward's state-only chunk walk
//      (scan_core.h), storing every lane's state at the start of every
//      chunk (one float per lane and chunk);
//   2. scan_bwd_chunked_kernel: the chunks in reverse.  Per chunk the owner
//      of each (channel, step) forms dl, dl*u and ds once and publishes them
//      in LDS; every lane recomputes its 32 states and decays from the
//      stored state, then walks the steps backwards.  Sums over n (C.h for
//      dz, dh.B for du and d(dl), q.A for d(dl)) go through the cross-row
//      swap reduction and LDS, as the forward's output; sums over the
//      workgroup's 16 channels (dB, dC) go through an LDS tile of 16 steps
//      and are stored as the workgroup's partial sums;
//   3. scan_bwd_chunked_bc_kernel: dB and dC as the sums of the workgroups'
//      partials of each batch, in workgroup order (deterministic).
// dA, dD and the bias gradient are added atomically once per lane or owner,
// so their last bits depend on the order.
#include <algorithm>
#include <mutex>
#include <type_traits>

#include "internal.h"
#include "scan_core.h"

namespace mssm {
namespace {

using core::buffer_ld;
using core::buffer_rsrc;
using core::kCh;
using core::kT;
using core::Pack;
using core::row_bcast;
using core::rows_reduce;

constexpr int kPitch = kT + 4;          // LDS row pitch of per-(channel, step) arrays
constexpr int kHalf = 16;               // steps per channel-sum tile
constexpr int kCbT = 20;                // floats per step in the channel-sum tile (16 + pad)
constexpr int kCbN = kHalf * kCbT + 4;  // floats per state element in the tile (bank offset)

// ---------------------------------------------------------------------------
// The walker of the reverse walk (shared with the adjoint-only walk)
// ---------------------------------------------------------------------------
struct BwdSmem {
    float dl[kCh * kPitch], du[kCh * kPitch], ds[kCh * kPitch];  // per (channel, step)
    float p[3][4][kCh * kPitch];    // per wave sums over its four state rows: C.h, dh.B, q.A
    float cb[2][16 * kCbN];         // channel terms of 16 steps: [dC | dB][n][t][channel]
};

template <typename T, bool GATE, bool VEC>
struct BwdWalker {
    static constexpr int OS = 2;                // steps per owner thread
    using Raw = typename Pack<T, OS>::raw;
    struct In {
        Raw ru, rd, rz, ry;                     // owner: u, delta, z, dy of OS steps
        T rb[2], rc[2];                         // lane: B, C at steps 16 q + j of the chunk
    };
    struct Own {
        float u[OS], sig[OS], gz[OS], ds[OS], dl[OS];
        bool ok[OS];
    };

    // lane role
    int w, r, j, n;
    bool nok, chok;
    float A2, Aval;
    uint32_t bcj;
    const T *Bb, *Cb;
    int32_t rec_a, rec_bc;
    // owner role
    int oc, ok;
    bool ochok;
    uint32_t oo;
    const T *ub, *db, *zb, *yb;
    float bias, skip;
    int L, dim;

    __device__ void init(const BwdArgs &a, int64_t b, int d0) {
        const int tid = threadIdx.x;
        w = tid >> 6;
        r = (tid >> 4) & 3;
        j = tid & 15;
        n = 4 * w + r;
        L = static_cast<int>(a.L);
        dim = static_cast<int>(a.dim);
        const int N = static_cast<int>(a.N);
        nok = n < N;
        chok = d0 + j < dim;
        const int dS = min(d0 + j, dim - 1);
        Aval = nok ? a.A[static_cast<int64_t>(dS) * N + n] : 0.0f;
        A2 = Aval * kLog2e;
        const T *B = static_cast<const T *>(a.B);
        const T *C = static_cast<const T *>(a.C);
        Bb = B + b * N * a.L;
        Cb = C + b * N * a.L;
        // rows past N load through an offset past every buffer's end (zero)
        bcj = nok ? (static_cast<uint32_t>(n) * static_cast<uint32_t>(L) + static_cast<uint32_t>(j)) *
                        sizeof(T)
                  : 0xffffff00u;
        oc = tid >> 4;
        ok = tid & 15;
        ochok = d0 + oc < dim;
        const int dO = min(d0 + oc, dim - 1);
        oo = static_cast<uint32_t>(dO - d0) * static_cast<uint32_t>(L) * sizeof(T);
        bias = a.delta_bias ? a.delta_bias[dO] : 0.0f;
        skip = a.D ? a.D[dO] : 0.0f;
        const int64_t row0 = (b * dim + d0) * a.L;
        ub = static_cast<const T *>(a.u) + row0;
        db = static_cast<const T *>(a.delta) + row0;
        zb = GATE ? static_cast<const T *>(a.z) + row0 : nullptr;
        yb = static_cast<const T *>(a.dy) + row0;
        rec_a = min(kCh, dim - d0) * L * static_cast<int32_t>(sizeof(T));
        rec_bc = N * L * static_cast<int32_t>(sizeof(T));
    }

    __device__ void load(int t0, In &in) const {
        const int32_t tb = t0 * static_cast<int32_t>(sizeof(T));
        if constexpr (VEC) {
            // rows 16-byte aligned, L % 8 == 0: the OS steps are all inside
            // the row or all past its end (zero or the next row, discarded)
            const uint32_t o = oo + static_cast<uint32_t>(OS * ok) * sizeof(T);
            in.ru = buffer_ld<Raw>(buffer_rsrc(reinterpret_cast<const char *>(ub) + tb, rec_a - tb), o);
            in.rd = buffer_ld<Raw>(buffer_rsrc(reinterpret_cast<const char *>(db) + tb, rec_a - tb), o);
            in.ry = buffer_ld<Raw>(buffer_rsrc(reinterpret_cast<const char *>(yb) + tb, rec_a - tb), o);
            if (GATE) in.rz = buffer_ld<Raw>(buffer_rsrc(reinterpret_cast<const char *>(zb) + tb, rec_a - tb), o);
        } else {
            T su[OS], sd[OS], sz[OS], sy[OS];
            const int off = t0 + OS * ok;
#pragma unroll
            for (int i = 0; i < OS; ++i) {
                const int t = off + i < L ? off + i : L - 1;
                const uint32_t o = oo + static_cast<uint32_t>(t) * sizeof(T);
                su[i] = *reinterpret_cast<const T *>(reinterpret_cast<const char *>(ub) + o);
                sd[i] = *reinterpret_cast<const T *>(reinterpret_cast<const char *>(db) + o);
                sy[i] = *reinterpret_cast<const T *>(reinterpret_cast<const char *>(yb) + o);
                sz[i] = GATE ? *reinterpret_cast<const T *>(reinterpret_cast<const char *>(zb) + o) : T(0);
            }
            __builtin_memcpy(&in.ru, su, sizeof(Raw));
            __builtin_memcpy(&in.rd, sd, sizeof(Raw));
            __builtin_memcpy(&in.ry, sy, sizeof(Raw));
            __builtin_memcpy(&in.rz, sz, sizeof(Raw));
        }
        const auto rB = buffer_rsrc(reinterpret_cast<const char *>(Bb) + tb, rec_bc - tb);
        const auto rC = buffer_rsrc(reinterpret_cast<const char *>(Cb) + tb, rec_bc - tb);
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const uint32_t o = bcj + static_cast<uint32_t>(16 * q) * sizeof(T);
            in.rb[q] = buffer_ld<T>(rB, o);
            in.rc[q] = buffer_ld<T>(rC, o);
        }
    }

    __device__ static float to_f32(T v) {
        if constexpr (sizeof(T) == 4) return v;
        else return __uint_as_float(static_cast<uint32_t>(v) << 16);
    }

    // Owner: the per-step scalars of its OS steps.  Steps past L and
    // channels past the last one get dl = dl*u = ds = 0, so they contribute
    // nothing.  The reverse walk and the adjoint-only walk both take them
    // from here, so the two compute identical values.
    __device__ void step_scalars(int t0, const In &in, float (&dl)[OS], float (&du)[OS], float (&dsv)[OS],
                                 Own &o) const {
        float u[OS], dr[OS], dy[OS], zz[OS];
        Pack<T, OS>::unpack(in.ru, u);
        Pack<T, OS>::unpack(in.rd, dr);
        Pack<T, OS>::unpack(in.ry, dy);
        if (GATE) Pack<T, OS>::unpack(in.rz, zz);
#pragma unroll
        for (int i = 0; i < OS; ++i) {
            const bool ok_t = ochok && t0 + OS * ok + i < L;
            const float x = dr[i] + bias;
            const float sp = softplus(x);
            // sigmoid(x) = 1 - exp(-softplus(x))
            o.sig[i] = 1.0f - fast_exp2(-sp * kLog2e);
            float dsx = dy[i];
            o.gz[i] = 0.0f;
            if (GATE) {
                const float sz = __builtin_amdgcn_rcpf(1.0f + fast_exp2(-zz[i] * kLog2e));
                dsx = dy[i] * (zz[i] * sz);
                // d silu / dz = sz (1 + z (1 - sz)); dz = dy s silu'(z)
                o.gz[i] = dy[i] * sz * fmaf(zz[i], 1.0f - sz, 1.0f);
            }
            dl[i] = ok_t ? sp : 0.0f;
            du[i] = ok_t ? sp * u[i] : 0.0f;
            dsv[i] = ok_t ? dsx : 0.0f;
            o.u[i] = u[i];
            o.ds[i] = dsv[i];
            o.dl[i] = dl[i];
            o.ok[i] = ok_t;
        }
    }

    // Owner: the chunk's per-step scalars published in LDS, and kept for its
    // outputs.
    __device__ void owner_scalars(int t0, const In &in, BwdSmem &sm, Own &o) const {
        float dl[OS], du[OS], dsv[OS];
        step_scalars(t0, in, dl, du, dsv, o);
        const int at = oc * kPitch + OS * ok;
        *reinterpret_cast<float2 *>(sm.dl + at) = make_float2(dl[0], dl[1]);
        *reinterpret_cast<float2 *>(sm.du + at) = make_float2(du[0], du[1]);
        *reinterpret_cast<float2 *>(sm.ds + at) = make_float2(dsv[0], dsv[1]);
    }

    // Owner, adjoint-only walk: dl and ds only.
    template <typename Sm>
    __device__ void owner_adjoint(int t0, const In &in, Sm &sm) const {
        float dl[OS], du[OS], dsv[OS];
        Own o;
        step_scalars(t0, in, dl, du, dsv, o);
        const int at = oc * kPitch + OS * ok;
        *reinterpret_cast<float2 *>(sm.dl + at) = make_float2(dl[0], dl[1]);
        *reinterpret_cast<float2 *>(sm.ds + at) = make_float2(dsv[0], dsv[1]);
    }

    // The same for the 16 steps of half `half` of the chunk: lane (row r,
    // column j) writes the four-row sums of steps 16 half + 4 r .. + 3
    // (v_permlane32_swap pairs rows {0,1}/{2,3} for steps k, k + 8, then
    // v_permlane16_swap rows 0/1 and 2/3 for k, k + 4).
    __device__ void reduce_store16(const float (&p)[16], BwdSmem &sm, int q, int half) const {
        float z[8], s[4];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(p[k]), __float_as_uint(p[k + 8]),
                                                            false, false);
            z[k] = __uint_as_float(x[0]) + __uint_as_float(x[1]);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const auto x = __builtin_amdgcn_permlane16_swap(__float_as_uint(z[k]), __float_as_uint(z[k + 4]),
                                                            false, false);
            s[k] = __uint_as_float(x[0]) + __uint_as_float(x[1]);
        }
        *reinterpret_cast<float4 *>(sm.p[q][w] + j * kPitch + 16 * half + 4 * r) = make_float4(s[0], s[1], s[2], s[3]);
    }

    // The wave's four state rows of p summed (cross-row swaps), then to LDS
    // slot q: lane (row r, column j) writes steps 8 r .. 8 r + 7.
    __device__ void reduce_store(const float (&p)[kT], BwdSmem &sm, int q) const {
        float s[8];
        rows_reduce(p, s);
        float4 *dst = reinterpret_cast<float4 *>(sm.p[q][w] + j * kPitch + 8 * r);
        dst[0] = make_float4(s[0], s[1], s[2], s[3]);
        dst[1] = make_float4(s[4], s[5], s[6], s[7]);
    }

    // Sums over the workgroup's 16 channels of the 16-step tile `half`: thread
    // (step t, state element m) adds the dC and dB terms of its 16 channels and
    // stores them as the workgroup's partial sums of step t0 + 16 half + t.
    __device__ static void channel_sums(int t0, int half, int L, const BwdSmem &sm, float *pg) {
        const int tid = threadIdx.x;
        const int t = tid >> 4, m = tid & 15;
        const int tt = t0 + kHalf * half + t;
        float s[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const float4 *src = reinterpret_cast<const float4 *>(sm.cb[q] + m * kCbN + t * kCbT);
            float acc = 0.0f;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float4 v = src[k];
                acc += v.x;
                acc += v.y;
                acc += v.z;
                acc += v.w;
            }
            s[q] = acc;
        }
        if (tt < L) {
            pg[static_cast<int64_t>(tt) * 32 + m] = s[0];
            pg[static_cast<int64_t>(tt) * 32 + 16 + m] = s[1];
        }
    }

    // Owner: du, ddelta (and dz) of its steps from the sums over n.
    __device__ void owner_outputs(int t0, const Own &o, const BwdSmem &sm, const BwdArgs &a,
                                  int64_t row_out, float &dD, float &dbias) const {
        const int at = oc * kPitch + OS * ok;
        float su[OS] = {0.0f, 0.0f}, sq[OS] = {0.0f, 0.0f}, sc[OS] = {0.0f, 0.0f};
#pragma unroll
        for (int ww = 0; ww < 4; ++ww) {
            const float2 vu = *reinterpret_cast<const float2 *>(sm.p[1][ww] + at);
            const float2 vq = *reinterpret_cast<const float2 *>(sm.p[2][ww] + at);
            su[0] += vu.x; su[1] += vu.y;
            sq[0] += vq.x; sq[1] += vq.y;
            if (GATE) {
                const float2 vc = *reinterpret_cast<const float2 *>(sm.p[0][ww] + at);
                sc[0] += vc.x; sc[1] += vc.y;
            }
        }
#pragma unroll
        for (int i = 0; i < OS; ++i) {
            if (!o.ok[i]) continue;
            const int64_t t = t0 + OS * ok + i;
            const float du = fmaf(o.ds[i], skip, o.dl[i] * su[i]);
            const float ddl = fmaf(o.u[i], su[i], sq[i]);
            const float ddelta = ddl * o.sig[i];
            a.du[row_out + t] = du;
            a.ddelta[row_out + t] = ddelta;
            if (GATE && a.dz) a.dz[row_out + t] = fmaf(skip, o.u[i], sc[i]) * o.gz[i];
            dD = fmaf(o.ds[i], o.u[i], dD);
            dbias += ddelta;
        }
    }
};

// ---------------------------------------------------------------------------
// 1. checkpoints: the state at the start of every chunk, and the adjoint
//    carries where the reverse walk of a group is cut into parts
// ---------------------------------------------------------------------------
// LDS of the adjoint-only walk: the chunk's dl and ds, double-buffered so a
// chunk needs one barrier.
struct AdjSmem {
    float dl[2][kCh * kPitch], ds[2][kCh * kPitch];
};
struct AdjBuf {
    float *dl, *ds;
};
union CkptSmem {
    core::Smem<4> walk;
    AdjSmem adj;
};

// How the reverse walk of the last groups is cut: the first n_whole groups
// are walked whole; each of the others is cut into `parts` ranges of whole
// chunks, part p covering chunks [p nch / parts, (p + 1) nch / parts).
struct BwdSplit {
    int n_whole, parts;
};

// Adjoint-only walk of group grp from the end down to the end of its first
// part: per chunk, the owners' dl and ds, then per lane, in the reverse
// walk's order and with its arithmetic,
//   dh = ds C + g,   g <- exp(dl A) dh,
// so that g at each cut equals, bit for bit, the carry the whole walk would
// reach there.  out[p * 256 + thread] receives the carry entering part p
// (p < parts - 1) from the parts after it.
template <typename T, bool GATE, bool VEC>
__device__ void adjoint_walk(const BwdArgs &a, int grp, int groups_per_batch, int nch, int parts,
                             float *__restrict__ out, AdjSmem &sm) {
    using BW = BwdWalker<T, GATE, VEC>;
    const int64_t b = grp / groups_per_batch;
    const int d0 = (grp - static_cast<int>(b) * groups_per_batch) * kCh;
    BW bw;
    bw.init(a, b, d0);
    const int L = bw.L;
    const int N = static_cast<int>(a.N);
    float g = (a.dh_last && bw.nok && bw.chok)
                  ? a.dh_last[(b * a.dim + d0 + bw.j) * static_cast<int64_t>(N) + bw.n]
                  : 0.0f;
    const int c_stop = nch / parts;   // the first part's end
    typename BW::In xa, xb;
    bw.load((nch - 1) * kT, xa);
    // (a buffer is rewritten two chunks after it was read, with this
    // chunk's barrier between)
    auto chunk = [&](int k, typename BW::In &cur, typename BW::In &nxt) {
        const int t0 = k * kT;
        if (k > c_stop) bw.load(t0 - kT, nxt);
        AdjBuf buf{sm.dl[k & 1], sm.ds[k & 1]};
        bw.owner_adjoint(t0, cur, buf);
        __syncthreads();
        float ccv[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const bool tok = t0 + 16 * q + bw.j < L;
            ccv[q] = tok ? BW::to_f32(cur.rc[q]) : 0.0f;
        }
        const float4 *pdl = reinterpret_cast<const float4 *>(buf.dl + bw.j * kPitch);
        const float4 *pds = reinterpret_cast<const float4 *>(buf.ds + bw.j * kPitch);
#pragma unroll
        for (int qq = 1; qq >= 0; --qq) {
            float dlh[16], dsh[16];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 x = pdl[4 * qq + q], y = pds[4 * qq + q];
                dlh[4 * q] = x.x; dlh[4 * q + 1] = x.y; dlh[4 * q + 2] = x.z; dlh[4 * q + 3] = x.w;
                dsh[4 * q] = y.x; dsh[4 * q + 1] = y.y; dsh[4 * q + 2] = y.z; dsh[4 * q + 3] = y.w;
            }
#define MSSM_ADJ(S)                                                                    \
    {                                                                                  \
        const float av = fast_exp2(dlh[S] * bw.A2);                                    \
        const float dh = fmaf(row_bcast<S>(ccv[qq]), dsh[S], g);                       \
        g = av * dh;                                                                   \
    }
            MSSM_ADJ(15) MSSM_ADJ(14) MSSM_ADJ(13) MSSM_ADJ(12) MSSM_ADJ(11) MSSM_ADJ(10)
            MSSM_ADJ(9) MSSM_ADJ(8) MSSM_ADJ(7) MSSM_ADJ(6) MSSM_ADJ(5) MSSM_ADJ(4)
            MSSM_ADJ(3) MSSM_ADJ(2) MSSM_ADJ(1) MSSM_ADJ(0)
#undef MSSM_ADJ
        }
        for (int p = 0; p + 1 < parts; ++p)
            if (k == (p + 1) * nch / parts) out[p * 256 + threadIdx.x] = g;
    };
    int k = nch - 1;
    for (; k >= c_stop + 1; k -= 2) {
        chunk(k, xa, xb);
        chunk(k - 1, xb, xa);
    }
    if (k == c_stop) chunk(k, xa, xb);
}

// Workgroups [0, groups) store the checkpoints of their group; workgroup
// groups + i walks the adjoint carries of group split.n_whole + i.
template <typename T, bool GATE, bool VEC>
__global__ __launch_bounds__(256) void scan_bwd_ckpt_kernel(BwdArgs a, float *__restrict__ ck, int nch,
                                                             int groups_per_batch, int groups, BwdSplit split,
                                                             float *__restrict__ adj) {
    using Wk = core::Walker<T, 4, 1, false, VEC, false>;
    __shared__ CkptSmem smu;
    if (static_cast<int>(blockIdx.x) >= groups) {
        const int i = static_cast<int>(blockIdx.x) - groups;
        adjoint_walk<T, GATE, VEC>(a, split.n_whole + i, groups_per_batch, nch, split.parts,
                                   adj + static_cast<int64_t>(i) * (split.parts - 1) * 256, smu.adj);
        return;
    }
    core::Smem<4> &sm = smu.walk;
    const int grp = blockIdx.x;
    const int64_t b = grp / groups_per_batch;
    const int d0 = (grp - static_cast<int>(b) * groups_per_batch) * kCh;
    const int dim = static_cast<int>(a.dim), N = static_cast<int>(a.N);
    Wk wk;
    wk.init(static_cast<const T *>(a.u), static_cast<const T *>(a.delta), a.delta_bias, a.A,
            static_cast<const T *>(a.B), static_cast<const T *>(a.C), nullptr, nullptr, nullptr, a.L, dim,
            N, b, d0);
    const int dS = min(d0 + wk.j, dim - 1);
    float h[1];
    h[0] = (a.h0 && wk.nok[0]) ? a.h0[(b * dim + dS) * static_cast<int64_t>(N) + wk.prow] : 0.0f;
    float *cg = ck + static_cast<int64_t>(grp) * nch * 256 + threadIdx.x;
    const int L = static_cast<int>(a.L);
    const int nfull = L / kT;
    typename Wk::In x0, x1;
    wk.template load<false>(0, x0);
    int c = 0;
    // two input sets used in turn, loads one chunk ahead (as the forward's
    // state-only walk); chunk c's state is stored before the chunk
    for (; c + 1 < nfull; c += 2) {
        wk.template load<false>((c + 1) * kT, x1);
        cg[static_cast<int64_t>(c) * 256] = h[0];
        wk.template state_chunk<true>(c * kT, L, x0, h, sm, 0);
        wk.template load<false>((c + 2) * kT, x0);
        cg[static_cast<int64_t>(c + 1) * 256] = h[0];
        wk.template state_chunk<true>((c + 1) * kT, L, x1, h, sm, 1);
    }
    if (c < nfull) {
        wk.template load<false>((c + 1) * kT, x1);
        cg[static_cast<int64_t>(c) * 256] = h[0];
        wk.template state_chunk<true>(c * kT, L, x0, h, sm, 0);
        if (c + 1 < nch) {
            cg[static_cast<int64_t>(c + 1) * 256] = h[0];
            wk.template state_chunk<false>((c + 1) * kT, L, x1, h, sm, 1);
        }
    } else if (c < nch) {
        cg[static_cast<int64_t>(c) * 256] = h[0];
        wk.template state_chunk<false>(c * kT, L, x0, h, sm, 0);
    }
}


// ---------------------------------------------------------------------------
// 2. the reverse walk
// ---------------------------------------------------------------------------
template <typename T, bool GATE, bool VEC>
__global__ __launch_bounds__(256, 2) void scan_bwd_chunked_kernel(BwdArgs a, const float *__restrict__ ck, int nch,
                                                                   int groups_per_batch, float *__restrict__ part,
                                                                   BwdSplit split, const float *__restrict__ adj) {
    using BW = BwdWalker<T, GATE, VEC>;
    __shared__ BwdSmem sm;
    // Workgroups [0, n_whole) walk their group whole; the others walk part p
    // of group n_whole + i, starting from the carry the adjoint-only walk
    // stored for it (the last part from dh_last, as a whole group).
    int grp = blockIdx.x, c_begin = 0, c_end = nch;
    const float *g_in = nullptr;
    if (grp >= split.n_whole) {
        const int i = (grp - split.n_whole) / split.parts, pp = (grp - split.n_whole) % split.parts;
        grp = split.n_whole + i;
        c_begin = pp * nch / split.parts;
        c_end = (pp + 1) * nch / split.parts;
        if (pp + 1 < split.parts) g_in = adj + (static_cast<int64_t>(i) * (split.parts - 1) + pp) * 256;
    }
    const int64_t b = grp / groups_per_batch;
    const int d0 = (grp - static_cast<int>(b) * groups_per_batch) * kCh;
    BW bw;
    bw.init(a, b, d0);
    const int N = static_cast<int>(a.N);
    const int L = bw.L;
    const bool want_bc = a.dB || a.dC;
    float *pg = part ? part + static_cast<int64_t>(grp) * a.L * 32 : nullptr;
    const float *cg = ck + static_cast<int64_t>(grp) * nch * 256 + threadIdx.x;
    const int64_t orow = (b * a.dim + (d0 + bw.oc)) * a.L;   // owner's output row
    // carry g = a_{t+1} dh_{t+1}: dh_last at the end
    float g = g_in ? g_in[threadIdx.x]
                   : ((a.dh_last && bw.nok && bw.chok)
                          ? a.dh_last[(b * a.dim + d0 + bw.j) * static_cast<int64_t>(N) + bw.n]
                          : 0.0f);
    float dA = 0.0f, dD = 0.0f, dbias = 0.0f;

    typename BW::In xa, xb;
    bw.load((c_end - 1) * kT, xa);
    auto chunk = [&](int k, typename BW::In &cur, typename BW::In &nxt) {
        const int t0 = k * kT;
        if (k > c_begin) bw.load(t0 - kT, nxt);
        typename BW::Own own;
        bw.owner_scalars(t0, cur, sm, own);
        __syncthreads();
        // recompute the chunk's states from the stored one
        float dls[kT], dus[kT], hs[kT], as[kT];
        {
            const float4 *pdl = reinterpret_cast<const float4 *>(sm.dl + bw.j * kPitch);
            const float4 *pdu = reinterpret_cast<const float4 *>(sm.du + bw.j * kPitch);
#pragma unroll
            for (int q = 0; q < kT / 4; ++q) {
                const float4 x = pdl[q], y = pdu[q];
                dls[4 * q] = x.x; dls[4 * q + 1] = x.y; dls[4 * q + 2] = x.z; dls[4 * q + 3] = x.w;
                dus[4 * q] = y.x; dus[4 * q + 1] = y.y; dus[4 * q + 2] = y.z; dus[4 * q + 3] = y.w;
            }
        }
        float cbv[2], ccv[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            // B, C past L: zero (the buffer loads return the next row or zero)
            const bool tok = t0 + 16 * q + bw.j < L;
            cbv[q] = tok ? BW::to_f32(cur.rb[q]) : 0.0f;
            ccv[q] = tok ? BW::to_f32(cur.rc[q]) : 0.0f;
        }
        const float hstart = cg[static_cast<int64_t>(k) * 256];
        {
            float h = hstart;
            float pc[kT];
#pragma unroll
            for (int qq = 0; qq < 2; ++qq) {
#define MSSM_FWD(S)                                                                    \
    {                                                                                  \
        const float av = fast_exp2(dls[16 * qq + S] * bw.A2);                          \
        h = fmaf(av, h, row_bcast<S>(cbv[qq]) * dus[16 * qq + S]);                     \
        as[16 * qq + S] = av;                                                          \
        hs[16 * qq + S] = h;                                                           \
        if (GATE) pc[16 * qq + S] = row_bcast<S>(ccv[qq]) * h;                         \
    }
                MSSM_FWD(0) MSSM_FWD(1) MSSM_FWD(2) MSSM_FWD(3) MSSM_FWD(4) MSSM_FWD(5)
                MSSM_FWD(6) MSSM_FWD(7) MSSM_FWD(8) MSSM_FWD(9) MSSM_FWD(10) MSSM_FWD(11)
                MSSM_FWD(12) MSSM_FWD(13) MSSM_FWD(14) MSSM_FWD(15)
#undef MSSM_FWD
            }
            if (GATE) bw.reduce_store(pc, sm, 0);
        }
        // reverse walk: steps 31 .. 16, the tile of channel sums, 15 .. 0;
        // the per-step scalars are read from LDS again (fewer live registers)
        float pu[kHalf], pq[kHalf];
        auto rev_step = [&](auto s_, auto qq_) {
            constexpr int S = decltype(s_)::value;      // lane of the row broadcast
            constexpr int QQ = decltype(qq_)::value;    // half of the chunk
            constexpr int s = 16 * QQ + S;
            const int qq = QQ;
            const float dsv = sm.ds[bw.j * kPitch + s];
            const float dlv = sm.dl[bw.j * kPitch + s];
            const float duv = sm.du[bw.j * kPitch + s];
            const float dh = fmaf(row_bcast<S>(ccv[qq]), dsv, g);
            float hp;
            if constexpr (s > 0) hp = hs[s - 1];
            else hp = hstart;
            sm.cb[0][bw.n * kCbN + S * kCbT + bw.j] = dsv * hs[s];       // dC term
            sm.cb[1][bw.n * kCbN + S * kCbT + bw.j] = dh * duv;          // dB term
            pu[S] = row_bcast<S>(cbv[qq]) * dh;
            g = as[s] * dh;
            const float q = g * hp;
            dA = fmaf(q, dlv, dA);
            pq[S] = q * bw.Aval;
        };
        auto rev_half = [&](auto qq_) {
#define MSSM_REV(S) rev_step(std::integral_constant<int, S>{}, qq_);
            MSSM_REV(15) MSSM_REV(14) MSSM_REV(13) MSSM_REV(12) MSSM_REV(11) MSSM_REV(10)
            MSSM_REV(9) MSSM_REV(8) MSSM_REV(7) MSSM_REV(6) MSSM_REV(5) MSSM_REV(4)
            MSSM_REV(3) MSSM_REV(2) MSSM_REV(1) MSSM_REV(0)
#undef MSSM_REV
        };
        rev_half(std::integral_constant<int, 1>{});
        bw.reduce_store16(pu, sm, 1, 1);
        bw.reduce_store16(pq, sm, 2, 1);
        __syncthreads();
        if (want_bc) BW::channel_sums(t0, 1, L, sm, pg);
        __syncthreads();
        rev_half(std::integral_constant<int, 0>{});
        bw.reduce_store16(pu, sm, 1, 0);
        bw.reduce_store16(pq, sm, 2, 0);
        __syncthreads();
        bw.owner_outputs(t0, own, sm, a, orow, dD, dbias);
        if (want_bc) BW::channel_sums(t0, 0, L, sm, pg);
        // (the next chunk's owners rewrite dl / du / ds after all of this
        // chunk's readers passed the barrier above)
    };
    int k = c_end - 1;
    for (; k >= c_begin + 1; k -= 2) {
        chunk(k, xa, xb);
        chunk(k - 1, xb, xa);
    }
    if (k == c_begin) chunk(k, xa, xb);

    if (bw.nok && bw.chok) {
        const int64_t d = d0 + bw.j;
        if (a.dh0 && c_begin == 0) a.dh0[(b * a.dim + d) * static_cast<int64_t>(N) + bw.n] = g;
        if (a.dA) atomicAdd(a.dA + d * N + bw.n, dA);
    }
    if (bw.ochok) {
        if (a.dD) atomicAdd(a.dD + d0 + bw.oc, dD);
        if (a.ddelta_bias) atomicAdd(a.ddelta_bias + d0 + bw.oc, dbias);
    }
}

// ---------------------------------------------------------------------------
// 3. dB, dC: the workgroups' partials of each batch added in workgroup order
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void scan_bwd_chunked_bc_kernel(const float *__restrict__ part,
                                                                  int groups_per_batch, int64_t batch,
                                                                  int64_t L, int N, float *dB, float *dC) {
    // one thread per four consecutive partial columns of one (batch, step)
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= batch * L * 8) return;
    const int col = static_cast<int>(i % 8) * 4;
    const int64_t t = (i / 8) % L;
    const int64_t b = i / (8 * L);
    const int n = col % 16;
    if (n >= N) return;
    float s[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    const float *p = part + (b * groups_per_batch * L + t) * 32 + col;
#pragma unroll 8
    for (int g = 0; g < groups_per_batch; ++g) {
        const float4 v = *reinterpret_cast<const float4 *>(p + static_cast<int64_t>(g) * L * 32);
        s[0] += v.x;
        s[1] += v.y;
        s[2] += v.z;
        s[3] += v.w;
    }
    float *out = col < 16 ? dC : dB;
    if (out) {
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (n + k < N) out[(b * N + n + k) * L + t] = s[k];
    }
}

// Compute units of the current device, queried once per device (0 if the
// query fails).
int device_cus() {
    static std::mutex mu;
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    std::lock_guard<std::mutex> lk(mu);
    if (cache[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) n = -1;
        cache[dev] = n;
    }
    return cache[dev] > 0 ? cache[dev] : 0;
}

// The reverse kernel holds two workgroups per compute unit (its registers
// and LDS), so U units walk 2 U groups at a time.  When the last round is
// partly empty (r = groups mod 2 U > 0, with at least one full round before
// it), the last r groups are each cut into parts = min(4, 2 U / r) ranges,
// which fill the last round with shorter work; every part is at least four
// chunks long.
BwdSplit plan_bwd_split(int64_t groups, int nch) {
    BwdSplit sp{static_cast<int>(groups), 1};
    const int cus = device_cus();
    const int64_t slots = 2 * static_cast<int64_t>(cus);
    if (cus <= 0 || groups <= slots) return sp;
    const int64_t r = groups % slots;
    if (r == 0) return sp;
    const int parts = static_cast<int>(std::min<int64_t>(4, slots / r));
    if (parts < 2 || nch < 4 * parts) return sp;
    sp.n_whole = static_cast<int>(groups - r);
    sp.parts = parts;
    return sp;
}

template <typename T, bool GATE, bool VEC>
hipError_t launch_typed(const BwdArgs &a, hipStream_t stream) {
    const int gpb = static_cast<int>((a.dim + kCh - 1) / kCh);
    const int64_t total = a.batch * gpb;
    const int nch = static_cast<int>((a.L + kT - 1) / kT);
    const bool want_bc = a.dB || a.dC;
    const BwdSplit sp = plan_bwd_split(total, nch);
    const int n_cut = static_cast<int>(total) - sp.n_whole;   // groups walked in parts
    const size_t ck_bytes = static_cast<size_t>(total) * nch * 256 * sizeof(float);
    const size_t part_bytes = want_bc ? static_cast<size_t>(total) * a.L * 32 * sizeof(float) : 0;
    const size_t adj_bytes = static_cast<size_t>(n_cut) * (sp.parts - 1) * 256 * sizeof(float);
    void *mem = nullptr;
    hipError_t e = scratch_alloc(&mem, ck_bytes + part_bytes + adj_bytes, stream);
    if (e != hipSuccess) return e;
    float *ck = static_cast<float *>(mem);
    float *part = want_bc ? reinterpret_cast<float *>(static_cast<char *>(mem) + ck_bytes) : nullptr;
    float *adj = reinterpret_cast<float *>(static_cast<char *>(mem) + ck_bytes + part_bytes);
    hipLaunchKernelGGL((scan_bwd_ckpt_kernel<T, GATE, VEC>), dim3(static_cast<uint32_t>(total + n_cut)), dim3(256),
                       0, stream, a, ck, nch, gpb, static_cast<int>(total), sp, adj);
    e = hipGetLastError();
    if (e == hipSuccess) {
        const int64_t grid = sp.n_whole + static_cast<int64_t>(n_cut) * sp.parts;
        hipLaunchKernelGGL((scan_bwd_chunked_kernel<T, GATE, VEC>), dim3(static_cast<uint32_t>(grid)),
                           dim3(256), 0, stream, a, ck, nch, gpb, part, sp, adj);
        e = hipGetLastError();
    }
    if (e == hipSuccess && want_bc) {
        const int64_t n = a.batch * a.L * 8;   // column quads
        hipLaunchKernelGGL(scan_bwd_chunked_bc_kernel, dim3(static_cast<uint32_t>((n + 255) / 256)), dim3(256),
                           0, stream, part, gpb, a.batch, a.L, static_cast<int>(a.N), a.dB, a.dC);
        e = hipGetLastError();
    }
    const hipError_t ef = scratch_free(mem, stream);
    return e != hipSuccess ? e : ef;
}

template <typename T>
hipError_t launch_gate(const BwdArgs &a, hipStream_t stream) {
    auto aligned = [](const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
    const bool vec = a.L % 8 == 0 && aligned(a.u) && aligned(a.delta) && aligned(a.dy) &&
                     (!a.z || aligned(a.z));
    if (a.z) return vec ? launch_typed<T, true, true>(a, stream) : launch_typed<T, true, false>(a, stream);
    return vec ? launch_typed<T, false, true>(a, stream) : launch_typed<T, false, false>(a, stream);
}

}  // namespace

bool scan_bwd_chunked_supported(const BwdArgs &a) {
    const int64_t esz = a.io == IO_F32 ? 4 : 2;
    const int64_t gpb = (a.dim + kCh - 1) / kCh;
    // 32-bit byte offsets over 16 channel rows and the N rows of B / C
    return a.N >= 1 && a.N <= 16 && kCh * a.L * esz < (int64_t(1) << 31) &&
           a.batch * gpb < (int64_t(1) << 30) && a.L < (int64_t(1) << 30);
}

hipError_t launch_scan_bwd_chunked(const BwdArgs &a, hipStream_t stream) {
    if (a.io == IO_F32) return launch_gate<float>(a, stream);
    return launch_gate<uint16_t>(a, stream);
}

}  // namespace mssm
