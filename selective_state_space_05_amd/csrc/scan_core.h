// scan_core.h -- the fused selective-scan chunk walk shared by the chunked
// kernel (scan_chunked.hip) and the chunk-parallel look-back kernel
// (scan_lookback.hip).
//
// Computes, for every (batch b, channel d) and step t
// ("Mamba状态空间模型的硬件感知推理优化" (ybb.press) sections 1 and 3.1;
// www.mhpq.cn/news/984979 essay sections 2.2-2.3):
//   dl   = softplus(delta + delta_bias[d])
//   h[n] = exp(dl * A[d,n]) * h[n] + (dl * u) * B[b,n,t]
//   y    = (sum_n C[b,n,t] * h[n] + D[d] * u) * silu(z)
// walking a range of steps in order from a given state, so the recurrence is
// evaluated exactly as the sequential definition over that range (one
// exponential per state element and step, no re-association inside it).
//
// Work decomposition (gfx950, wave64).  A workgroup of W waves (W = 2 or 4)
// owns 16 channels of one batch and all N state elements.  Lane (wave w, row
// r, column j) -- r = lane / 16, j = lane % 16 -- holds channel j and the NPL
// state elements n = (4w + r) * NPL + g, g < NPL, in registers, so the 4W
// rows of the workgroup cover 4W * NPL >= N state elements.  Steps are walked
// in chunks of 32:
//
//   A. Every thread owns 8/W consecutive steps of one channel: it loads u,
//      delta (and z) for them with one vector load each, computes the
//      per-step scalars dl, dl*u, D*u and silu(z) once, and publishes dl and
//      dl*u in LDS.  Loads for the next chunk are issued here, so their
//      latency overlaps the scan of this chunk.
//   B. Every lane walks the 32 steps for its channel and state elements.
//      B[b,n,t] and C[b,n,t] are the same for the 16 channels of a row; lane j
//      of the row holds the values of step 16q + j, and the product with them
//      takes that lane's value through a DPP row broadcast folded into the
//      multiply itself (row_newbcast), so sharing them costs no instruction.
//      Each lane accumulates C.h over its NPL state elements per step and
//      writes the 32 partial sums to LDS.
//   C. The owner of each (channel, step) adds the 4W partial sums, applies
//      the skip term and the gate, rounds and stores y.
//
// A state-only walk (no output) skips the C terms and phase C and keeps a
// running sum of dl per channel, which gives the range's total decay
// exp(A * sum dl) -- the cumulative product of the decays taken in log space
// (ybb.press section 6.2).
//
// Steps past the end of the range get dl = 0 and dl*u = 0, i.e. the identity
// pair (decay 1, input 0), so the state passes through unchanged.  Channels
// beyond the last compute on clamped inputs and store nothing.
//
// With the convolution prologue (CONV), the activation row holds the input x
// of a causal width-4 depthwise convolution, and the owner forms
// u_t = silu(conv_b + sum_k conv_w[k] x_{t-3+k}) (x = 0 before step 0) from
// its own steps and the four before them (the tencentcloud.csdn.net article
// on Mamba, section 3: a local convolution and SiLU precede the selective
// SSM), so u never goes through HBM.
#pragma once

#include "device_math.h"

namespace mssm {
namespace core {

constexpr int kCh = 16;            // channels per workgroup
constexpr int kT = 32;             // steps per chunk
constexpr int kPitch = kT + 4;     // LDS row pitch (floats)

// Value of `v` held by lane S of this lane's 16-lane row.
template <int S>
__device__ __forceinline__ float row_bcast(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(
        __builtin_bit_cast(int, v), 0x150 + S, 0xf, 0xf, true));
}

// Two float32 values rounded to bf16 (nearest even) and packed, low half
// first, with one v_cvt_pk_bf16_f32.  Written as an instruction rather than
// through the __bf16 type: with that type in a kernel the compiler stops
// folding the row broadcasts above into the multiplies that consume them.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    uint32_t r;
    asm("v_cvt_pk_bf16_f32 %0, %1, %2" : "=v"(r) : "v"(lo), "v"(hi));
    return r;
}

// OS consecutive steps of one activation row, moved as one vector.
template <int BYTES> struct RawT;
template <> struct RawT<4> { using type = uint32_t; };
template <> struct RawT<8> { using type = uint2; };
template <> struct RawT<16> { using type = uint4; };

template <typename T, int OS>
struct Pack {
    using raw = typename RawT<OS * sizeof(T)>::type;
    __device__ static raw load(const T *p) { return *reinterpret_cast<const raw *>(p); }
    __device__ static void unpack(raw v, float *o) {
        uint32_t w[OS * sizeof(T) / 4];
        __builtin_memcpy(w, &v, sizeof(raw));
        if constexpr (sizeof(T) == 4) {
#pragma unroll
            for (int i = 0; i < OS; ++i) o[i] = __uint_as_float(w[i]);
        } else {
#pragma unroll
            for (int i = 0; i < OS / 2; ++i) {
                o[2 * i] = __uint_as_float(w[i] << 16);
                o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
            }
        }
    }
    __device__ static void store(T *p, const float *v) {
        uint32_t w[OS * sizeof(T) / 4];
        if constexpr (sizeof(T) == 4) {
#pragma unroll
            for (int i = 0; i < OS; ++i) w[i] = __float_as_uint(v[i]);
        } else {
#pragma unroll
            for (int i = 0; i < OS / 2; ++i) w[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
        }
        raw r;
        __builtin_memcpy(&r, w, sizeof(raw));
        *reinterpret_cast<raw *>(p) = r;
    }
};

// Buffer loads.  A buffer resource names a base address and a size in
// bytes; a lane's load at a byte offset at or past the size returns zero
// instead of touching memory.  Walks move the base along the rows chunk by
// chunk in scalar registers, so per-lane offsets stay fixed and loads past
// the end of a tensor need no clamping.
// Sizes are below 2^31 bytes (the launchers check the rows' extent), so
// they stay in 32-bit scalar arithmetic.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *base, int32_t bytes) {
    // 0x00020000: the raw-buffer format word of the gfx9 family (32-bit data)
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, bytes > 0 ? bytes : 0, 0x00020000);
}
template <typename V> __device__ V buffer_ld(__amdgpu_buffer_rsrc_t r, uint32_t off);
template <> __device__ __forceinline__ uint16_t buffer_ld<uint16_t>(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}
template <> __device__ __forceinline__ float buffer_ld<float>(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
template <> __device__ __forceinline__ uint32_t buffer_ld<uint32_t>(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
template <> __device__ __forceinline__ uint2 buffer_ld<uint2>(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    return make_uint2(v[0], v[1]);
}
template <> __device__ __forceinline__ uint4 buffer_ld<uint4>(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    return make_uint4(v[0], v[1], v[2], v[3]);
}

// LDS of one workgroup.  dl / dl*u and the partial sums are double-buffered
// so that every walk needs one barrier per chunk.
template <int W>
struct Smem {
    float dl[2][kCh * kPitch];
    float du[2][kCh * kPitch];
    float p[2][W * kCh * kPitch];   // per wave: partial sums over its 4 state rows
};

// Sum of a value over the four 16-lane rows of a wave, for 32 values at
// once (p[k] belongs to step k), with cross-row swaps instead of LDS:
// v_permlane32_swap pairs rows (0, 2) and (1, 3) for steps k and k + 16,
// v_permlane16_swap then pairs rows (0, 1) and (2, 3) for steps k and k + 8.
// On return lane (row r, column j) holds in q[i] the four-row sum of step
// 8 r + i for its column.
__device__ __forceinline__ void rows_reduce(const float (&p)[32], float (&q)[8]) {
    float z[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(p[k]), __float_as_uint(p[k + 16]),
                                                        false, false);
        // rows 0, 1: step k, rows {0, 2} / {1, 3}; rows 2, 3: step k + 16
        z[k] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(z[k]), __float_as_uint(z[k + 8]),
                                                        false, false);
        // row 0: step k, row 1: k + 8, row 2: k + 16, row 3: k + 24
        q[k] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
}

constexpr int kConv = 4;           // width of the convolution prologue

// Per-thread view of one (batch, 16-channel group) problem slice.
template <typename T, int W, int NPL, bool GATE, bool VEC, bool CONV = false>
struct Walker {
    static constexpr int kRows = 4 * W;            // rows of 16 lanes
    static constexpr int OS = kT * kCh / (64 * W); // steps per owner thread (4 or 2)
    static constexpr int OPC = kT / OS;            // owner threads per channel
    static constexpr int kPrev = kConv / OS;       // raws holding the 4 steps before
    using Raw = typename Pack<T, OS>::raw;

    // Inputs of one chunk exactly as loaded; they are converted where they
    // are first used, a chunk after the loads were issued, so the loads
    // overlap a whole chunk of work.
    struct In {
        Raw ru, rd, rz;            // owner: OS steps of u (CONV: x), delta (and z)
        Raw rp[CONV ? kPrev : 1];  // CONV: x at the 4 steps before the owner's first
        T rb[2][NPL], rc[2][NPL];  // scan lane: B, C at steps t0 + 16 q + j
    };

    // scan-lane role
    int prow, j;
    float A2[NPL];
    uint32_t bco[NPL];     // byte offset of this lane's B / C rows in the batch
    uint32_t bcj[NPL];     // bco + this lane's step j within a 16-step half
    bool nok[NPL];
    int32_t rec_a, rec_bc; // bytes from ub / Bb to the end of their rows (< 2^31)
    const T *Bb, *Cb;      // B, C of this batch (workgroup-uniform)
    // owner role
    int oc, ok;
    uint32_t oo;           // byte offset of the owner's channel row
    const T *ub, *db, *zb; // rows of the workgroup's first channel (uniform)
    T *yb;
    float bias, skip;
    float cw[kConv], cbias; // CONV: the owner channel's taps and bias
    int L;
    float sdl;             // owner's running sum of dl over the walked steps

    // Offsets are 32-bit byte offsets from workgroup-uniform bases, which
    // keeps per-load address arithmetic to one 32-bit add; the launchers
    // guarantee 16 * L and N * L elements fit in 2^31 bytes.
    template <typename V>
    __device__ static V ld(const T *base, uint32_t off) {
        return *reinterpret_cast<const V *>(reinterpret_cast<const char *>(base) + off);
    }

    __device__ void init(const T *u, const T *delta, const float *delta_bias, const float *A,
                         const T *B, const T *C, const float *Dskip, const T *z, T *y,
                         int64_t L_, int dim, int N, int64_t b, int d0,
                         const float *conv_w = nullptr, const float *conv_b = nullptr) {
        const int tid = threadIdx.x;
        const int lane = tid & 63;
        prow = (tid >> 6) * 4 + (lane >> 4);
        j = lane & 15;
        L = static_cast<int>(L_);
        Bb = B + b * N * L_;
        Cb = C + b * N * L_;
        const int dS = min(d0 + j, dim - 1);
#pragma unroll
        for (int g = 0; g < NPL; ++g) {
            const int n = prow * NPL + g;
            nok[g] = n < N;
            A2[g] = nok[g] ? A[static_cast<int64_t>(dS) * N + n] * kLog2e : 0.0f;
            bco[g] = static_cast<uint32_t>(min(n, N - 1)) * static_cast<uint32_t>(L) * sizeof(T);
            // rows past N load through an offset past every buffer's end,
            // which reads zero: their B and C vanish with no select
            bcj[g] = nok[g] ? bco[g] + static_cast<uint32_t>(j) * sizeof(T) : 0xffffff00u;
        }
        oc = tid / OPC;
        ok = tid % OPC;
        // Channels past the last one compute on the last channel's inputs
        // (scan lanes and owners alike), so their outputs equal that
        // channel's outputs bit for bit; storing them into its row rewrites
        // the same values and needs no branch around the store.
        const int dO = min(d0 + oc, dim - 1);
        const int64_t row0 = (b * dim + d0) * L_;
        oo = static_cast<uint32_t>(dO - d0) * static_cast<uint32_t>(L) * sizeof(T);
        bias = delta_bias ? delta_bias[dO] : 0.0f;
        skip = Dskip ? Dskip[dO] : 0.0f;
        if constexpr (CONV) {
#pragma unroll
            for (int k = 0; k < kConv; ++k) cw[k] = conv_w[static_cast<int64_t>(dO) * kConv + k];
            cbias = conv_b ? conv_b[dO] : 0.0f;
        }
        ub = u + row0;
        db = delta + row0;
        zb = GATE ? z + row0 : nullptr;
        yb = y ? y + row0 : nullptr;
        rec_a = min(kCh, dim - d0) * L * static_cast<int32_t>(sizeof(T));
        rec_bc = N * L * static_cast<int32_t>(sizeof(T));
        sdl = 0.0f;
    }

    // Issue the loads of the chunk starting at step t0, from indices clamped
    // into the row and with no branch, so that nothing waits for them before
    // their use.  Values of steps past the walked range are discarded there.
    template <bool OUT>
    __device__ void load(int t0, In &in) const {
        const int off = t0 + OS * ok;
        // byte offset of step t0 in a row: the resources below start there
        const int32_t tb = t0 * static_cast<int32_t>(sizeof(T));
        if constexpr (VEC) {
            // rows 16-byte aligned and L % 8 == 0 with OS | 8: the OS steps
            // are all inside the row or all past its end; past the end of the
            // row they read the next row (or zero past the last one), values
            // the chunk discards
            static_assert(8 % OS == 0, "vector owner loads need OS | 8");
            const uint32_t o = oo + static_cast<uint32_t>(OS * ok) * sizeof(T);
            in.ru = buffer_ld<Raw>(buffer_rsrc(reinterpret_cast<const char *>(ub) + tb, rec_a - tb), o);
            in.rd = buffer_ld<Raw>(buffer_rsrc(reinterpret_cast<const char *>(db) + tb, rec_a - tb), o);
            if (GATE && OUT)
                in.rz = buffer_ld<Raw>(buffer_rsrc(reinterpret_cast<const char *>(zb) + tb, rec_a - tb), o);
            if constexpr (CONV) {
                // the 4 steps before, as kPrev aligned raws; indices clamped
                // into the row (those before step 0 are zeroed at the use)
#pragma unroll
                for (int m = 0; m < kPrev; ++m) {
                    const int s = off - kConv + m * OS;
                    const int sc = s < 0 ? 0 : (s + OS <= L ? s : L - OS);
                    in.rp[m] = ld<Raw>(ub, oo + static_cast<uint32_t>(sc) * sizeof(T));
                }
            }
        } else {
            T su[OS], sd[OS], sz[OS];
#pragma unroll
            for (int i = 0; i < OS; ++i) {
                const uint32_t o = oo + static_cast<uint32_t>(off + i < L ? off + i : L - 1) * sizeof(T);
                su[i] = ld<T>(ub, o);
                sd[i] = ld<T>(db, o);
                sz[i] = (GATE && OUT) ? ld<T>(zb, o) : T(0);
            }
            __builtin_memcpy(&in.ru, su, sizeof(Raw));
            __builtin_memcpy(&in.rd, sd, sizeof(Raw));
            __builtin_memcpy(&in.rz, sz, sizeof(Raw));
            if constexpr (CONV) {
                T sp[kConv];
#pragma unroll
                for (int k = 0; k < kConv; ++k) {
                    const int s = off - kConv + k;
                    const int sc = s < 0 ? 0 : (s < L ? s : L - 1);
                    sp[k] = ld<T>(ub, oo + static_cast<uint32_t>(sc) * sizeof(T));
                }
                __builtin_memcpy(in.rp, sp, sizeof(sp));
            }
        }
        // B, C at steps t0 + 16 q + j (past the end of an n row: the next
        // row or zero, discarded)
        const auto rB = buffer_rsrc(reinterpret_cast<const char *>(Bb) + tb, rec_bc - tb);
        const auto rC = buffer_rsrc(reinterpret_cast<const char *>(Cb) + tb, rec_bc - tb);
#pragma unroll
        for (int q = 0; q < 2; ++q) {
#pragma unroll
            for (int g = 0; g < NPL; ++g) {
                const uint32_t o = bcj[g] + static_cast<uint32_t>(16 * q) * sizeof(T);
                in.rb[q][g] = buffer_ld<T>(rB, o);
                if (OUT) in.rc[q][g] = buffer_ld<T>(rC, o);
            }
        }
    }

    __device__ static float to_f32(T v) {
        if constexpr (sizeof(T) == 4) return v;
        else return __uint_as_float(static_cast<uint32_t>(v) << 16);
    }

    // Per-step values an owner thread keeps from phase A of a chunk to its
    // phase C: the scan input u (for the skip term), the gate factor, and the
    // number of its steps inside the range.
    struct Own {
        float uu[OS], gz[OS];
        int rem;
    };

    // ---- phase A: per-step scalars of this thread's OS steps of the chunk at
    // t0, published in LDS buffer buf.  FULL: all kT steps lie inside
    // [t0, t_end).  OUT: keep the skip term and gate for phase C; otherwise
    // add dl to the owner's running sum.
    template <bool OUT, bool FULL>
    __device__ void phase_a(int t0, int t_end, const In &in, Smem<W> &sm, int buf, Own &o) {
        float u[OS], dr[OS], zz[OS];
        Pack<T, OS>::unpack(in.ru, u);
        Pack<T, OS>::unpack(in.rd, dr);
        if constexpr (CONV) {
            // xx[0..3]: x at the 4 steps before the owner's first (0 before
            // step 0), xx[4..]: the owner's own steps
            float xx[kConv + OS];
#pragma unroll
            for (int m = 0; m < kPrev; ++m) Pack<T, OS>::unpack(in.rp[m], xx + m * OS);
            const int first = t0 + OS * ok;
#pragma unroll
            for (int k = 0; k < kConv; ++k)
                if (first - kConv + k < 0) xx[k] = 0.0f;
#pragma unroll
            for (int i = 0; i < OS; ++i) xx[kConv + i] = u[i];
#pragma unroll
            for (int i = 0; i < OS; ++i) {
                float c = cbias;
#pragma unroll
                for (int k = 0; k < kConv; ++k) c = fmaf(cw[k], xx[i + 1 + k], c);
                u[i] = silu(c);
            }
        }
        if (GATE && OUT) Pack<T, OS>::unpack(in.rz, zz);
        int rem = OS;                       // steps of this owner inside the range
        if (!FULL) rem = min(t_end - (t0 + OS * ok), OS);
        o.rem = rem;
        float dl[OS], du[OS];
#pragma unroll
        for (int i = 0; i < OS; ++i) {
            // computed unconditionally; steps past the end become the
            // identity step dl = 0, dl*u = 0
            const float sp = softplus(dr[i] + bias);
            dl[i] = (FULL || i < rem) ? sp : 0.0f;
            du[i] = (FULL || i < rem) ? sp * u[i] : 0.0f;
            if (OUT) {
                o.uu[i] = u[i];
                o.gz[i] = GATE ? silu(zz[i]) : 1.0f;
            } else {
                sdl += dl[i];
            }
        }
#pragma unroll
        for (int i = 0; i < OS; i += 2) {
            *reinterpret_cast<float2 *>(sm.dl[buf] + oc * kPitch + OS * ok + i) = make_float2(dl[i], dl[i + 1]);
            *reinterpret_cast<float2 *>(sm.du[buf] + oc * kPitch + OS * ok + i) = make_float2(du[i], du[i + 1]);
        }
    }

    // dl and dl*u of the 32 steps of this lane's channel, from LDS buffer buf.
    __device__ static void read_steps(const Smem<W> &sm, int buf, int jj, float (&dls)[kT], float (&dus)[kT]) {
        const float4 *pdl = reinterpret_cast<const float4 *>(sm.dl[buf] + jj * kPitch);
        const float4 *pdu = reinterpret_cast<const float4 *>(sm.du[buf] + jj * kPitch);
#pragma unroll
        for (int k = 0; k < kT / 4; ++k) {
            const float4 a = pdl[k], e = pdu[k];
            dls[4 * k] = a.x; dls[4 * k + 1] = a.y; dls[4 * k + 2] = a.z; dls[4 * k + 3] = a.w;
            dus[4 * k] = e.x; dus[4 * k + 1] = e.y; dus[4 * k + 2] = e.z; dus[4 * k + 3] = e.w;
        }
    }

    // ---- phase B: 32 steps of the recurrence for this lane from the step
    // scalars dls / dus; with OUT, p[k] is this lane's part of C.h at step k.
    template <bool OUT, bool FULL>
    __device__ void phase_b(int t0, int t_end, const In &in, const float (&dls)[kT], const float (&dus)[kT],
                            float (&h)[NPL], float (&p)[kT]) const {
        // B, C of the row broadcasts: zero past the end (state rows past N
        // loaded zero)
        float cb[2][NPL], cc[2][NPL];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const bool tok = FULL || t0 + 16 * q + j < t_end;
#pragma unroll
            for (int g = 0; g < NPL; ++g) {
                cb[q][g] = tok ? to_f32(in.rb[q][g]) : 0.0f;
                cc[q][g] = (OUT && tok) ? to_f32(in.rc[q][g]) : 0.0f;
            }
        }
#pragma unroll
        for (int q = 0; q < 2; ++q) {
#define MSSM_STEP(S)                                                           \
    {                                                                          \
        float acc = 0.0f;                                                      \
        _Pragma("unroll") for (int g = 0; g < NPL; ++g) {                      \
            const float a = fast_exp2(dls[16 * q + S] * A2[g]);                \
            h[g] = fmaf(a, h[g], row_bcast<S>(cb[q][g]) * dus[16 * q + S]);    \
            if (OUT) acc = g == 0 ? row_bcast<S>(cc[q][g]) * h[g]              \
                                  : fmaf(row_bcast<S>(cc[q][g]), h[g], acc);   \
        }                                                                      \
        p[16 * q + S] = acc;                                                   \
    }
            MSSM_STEP(0) MSSM_STEP(1) MSSM_STEP(2) MSSM_STEP(3)
            MSSM_STEP(4) MSSM_STEP(5) MSSM_STEP(6) MSSM_STEP(7)
            MSSM_STEP(8) MSSM_STEP(9) MSSM_STEP(10) MSSM_STEP(11)
            MSSM_STEP(12) MSSM_STEP(13) MSSM_STEP(14) MSSM_STEP(15)
#undef MSSM_STEP
        }
    }

    // The wave's four state rows of p summed in registers; lane (row r,
    // column j) writes steps 8 r .. 8 r + 7 of channel j to partial-sum
    // buffer pbuf.
    __device__ void reduce_store(const float (&p)[kT], Smem<W> &sm, int pbuf) const {
        float qs[8];
        rows_reduce(p, qs);
        const int r = (threadIdx.x >> 4) & 3;
        float4 *dst = reinterpret_cast<float4 *>(sm.p[pbuf] + ((threadIdx.x >> 6) * kCh + j) * kPitch + 8 * r);
        dst[0] = make_float4(qs[0], qs[1], qs[2], qs[3]);
        dst[1] = make_float4(qs[4], qs[5], qs[6], qs[7]);
    }

    // ---- phase C: the owner adds the W waves' partial sums of its OS steps
    // of the chunk at t0, applies the skip term and the gate, and stores y.
    template <bool FULL>
    __device__ void phase_c(int t0, const Own &o, const Smem<W> &sm, int pbuf) const {
        float yv[OS];
#pragma unroll
        for (int i = 0; i < OS; ++i) yv[i] = 0.0f;
#pragma unroll
        for (int r = 0; r < W; ++r) {
            const float *src = sm.p[pbuf] + (r * kCh + oc) * kPitch + OS * ok;
#pragma unroll
            for (int i = 0; i < OS; i += 2) {
                const float2 v = *reinterpret_cast<const float2 *>(src + i);
                yv[i] += v.x;
                yv[i + 1] += v.y;
            }
        }
        // The skip term as one explicit fused multiply-add: left to the
        // compiler, D*u + sum is contracted in some inlined copies of this
        // phase and not in others, which changes the last bit of y between
        // walks of the same steps.
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

    // One state-only chunk of kT steps at t0 (no output; the owner's sum of
    // dl grows).  Buffer buf alternates between chunks, so one barrier per
    // chunk orders the LDS reuse.
    template <bool FULL>
    __device__ void state_chunk(int t0, int t_end, const In &in, float (&h)[NPL], Smem<W> &sm, int buf) {
        Own o;
        phase_a<false, FULL>(t0, t_end, in, sm, buf, o);
        __syncthreads();
        float dls[kT], dus[kT], p[kT];
        read_steps(sm, buf, j, dls, dus);
        phase_b<false, FULL>(t0, t_end, in, dls, dus, h, p);
    }

    // One stage of the output pipeline, at chunk k of a walk from t_begin:
    // issues the loads of chunk k + 2 into xk (free: chunk k's scan is done),
    // publishes chunk k + 1's step scalars and chunk k's partial sums, then,
    // after the one barrier of the stage, stores chunk k's outputs and runs
    // chunk k + 1's scan into p.  FN: chunk k + 1 is full.  Chunk k is full.
    //
    // LDS reuse: step scalars of chunk c live in buffer c % 2 and partial
    // sums in partial buffer c % 2.  Each buffer is rewritten two stages after
    // it was written, and the stage in between holds a barrier that every
    // reader of the old contents passed first.
    template <bool FN>
    __device__ void out_stage(int t_begin, int t_end, int k, In &xk, const In &xk1, const Own &ok_,
                              Own &ok1, float (&h)[NPL], float (&p)[kT], Smem<W> &sm) {
        const int tk = t_begin + k * kT;
        load<true>(tk + 2 * kT, xk);
        phase_a<true, FN>(tk + kT, t_end, xk1, sm, (k + 1) & 1, ok1);
        reduce_store(p, sm, k & 1);
        __syncthreads();
        float dls[kT], dus[kT];
        read_steps(sm, (k + 1) & 1, j, dls, dus);
        phase_c<true>(tk, ok_, sm, k & 1);
        phase_b<true, FN>(tk + kT, t_end, xk1, dls, dus, h, p);
    }

    // The last chunk k of a walk: its partial sums, one barrier, its outputs.
    __device__ void out_last(int t_begin, int k, bool full, const float (&p)[kT], const Own &o, Smem<W> &sm) {
        reduce_store(p, sm, k & 1);
        __syncthreads();
        if (full) phase_c<true>(t_begin + k * kT, o, sm, k & 1);
        else phase_c<false>(t_begin + k * kT, o, sm, k & 1);
    }

    // Walk steps [t_begin, t_end) from state h (updated in place).  OUT: also
    // form and store y; otherwise only the state and the owner's sum of dl.
    // t_begin must be a multiple of OS; every thread of the workgroup calls
    // this with the same range, after a barrier that follows any earlier use
    // of the workgroup's LDS.
    //
    // The output walk is a pipeline with one barrier per chunk: chunk k's
    // partial sums and chunk k + 1's step scalars are published together,
    // so the reduction's cross-lane work and phase A's transcendental chains
    // fill each other's latencies, and chunk k's stores overlap chunk
    // k + 1's scan.  Loads run two chunks ahead of the scan.
    template <bool OUT>
    __device__ void walk(int t_begin, int t_end, float (&h)[NPL], Smem<W> &sm) {
        const int len = t_end - t_begin;
        if (len <= 0) return;
        const int nfull = len / kT;
        if constexpr (!OUT) {
            // Two input sets used in turn: the loads of chunk c + 1 go
            // straight into the registers that chunk c + 1 reads, with no
            // copy in between (a copy would have to wait for the loads).
            In x0, x1;
            load<false>(t_begin, x0);
            int c = 0;
            for (; c + 1 < nfull; c += 2) {
                const int t0 = t_begin + c * kT;
                load<false>(t0 + kT, x1);
                state_chunk<true>(t0, t_end, x0, h, sm, 0);
                load<false>(t0 + 2 * kT, x0);
                state_chunk<true>(t0 + kT, t_end, x1, h, sm, 1);
            }
            // x0 holds the inputs of chunk c; loads past the range are
            // clamped and their values unused
            const int t0 = t_begin + c * kT;
            if (c < nfull) {
                load<false>(t0 + kT, x1);
                state_chunk<true>(t0, t_end, x0, h, sm, 0);
                if (t0 + kT < t_end) state_chunk<false>(t0 + kT, t_end, x1, h, sm, 1);
            } else if (t0 < t_end) {
                state_chunk<false>(t0, t_end, x0, h, sm, 0);
            }
        } else {
            const int nch = (len + kT - 1) / kT;
            In xa, xb;
            Own oa, ob;
            float p[kT];
            load<true>(t_begin, xa);
            load<true>(t_begin + kT, xb);
            {
                float dls[kT], dus[kT];
                if (nfull > 0) {
                    phase_a<true, true>(t_begin, t_end, xa, sm, 0, oa);
                    __syncthreads();
                    read_steps(sm, 0, j, dls, dus);
                    phase_b<true, true>(t_begin, t_end, xa, dls, dus, h, p);
                } else {
                    phase_a<true, false>(t_begin, t_end, xa, sm, 0, oa);
                    __syncthreads();
                    read_steps(sm, 0, j, dls, dus);
                    phase_b<true, false>(t_begin, t_end, xa, dls, dus, h, p);
                }
            }
            // Stage k needs chunk k + 1 to exist; stages with both chunks
            // full run two at a time, so the input sets swap roles without a
            // copy.  At most two stages remain after the loop, the second
            // one for the partial last chunk.
            int k = 0;
            for (; k + 2 < nfull; k += 2) {
                out_stage<true>(t_begin, t_end, k, xa, xb, oa, ob, h, p, sm);
                out_stage<true>(t_begin, t_end, k + 1, xb, xa, ob, oa, h, p, sm);
            }
            const bool last_full = nch == nfull;
            if (k + 1 < nch) {
                if (k + 1 < nfull) out_stage<true>(t_begin, t_end, k, xa, xb, oa, ob, h, p, sm);
                else out_stage<false>(t_begin, t_end, k, xa, xb, oa, ob, h, p, sm);
                ++k;
                if (k + 1 < nch) {
                    out_stage<false>(t_begin, t_end, k, xb, xa, ob, oa, h, p, sm);
                    ++k;
                    out_last(t_begin, k, last_full, p, oa, sm);
                } else {
                    out_last(t_begin, k, last_full, p, ob, sm);
                }
            } else {
                out_last(t_begin, k, last_full, p, oa, sm);
            }
        }
    }

    // Sum of dl over the walked steps for this lane's channel j, gathered
    // from the OPC owners of the channel through LDS.  Call after a state-only
    // walk; every thread of the workgroup must call it.
    __device__ float channel_dl_sum(Smem<W> &sm) const {
        __syncthreads();                           // last chunk's readers are done
        sm.p[0][oc * OPC + ok] = sdl;
        __syncthreads();
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < OPC; ++i) s += sm.p[0][j * OPC + i];
        __syncthreads();                           // sm.p is reused afterwards
        return s;
    }
};

}  // namespace core
}  // namespace mssm
