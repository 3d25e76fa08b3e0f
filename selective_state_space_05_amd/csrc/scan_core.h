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

// Owner loads of one chunk: OS steps of u, delta (and z) of one channel.
template <typename T, int OS, bool VEC, bool GATE>
struct OwnerIn {
    float u[OS], dr[OS], z[OS];
    typename Pack<T, OS>::raw ru, rd, rz;
    __device__ void load(const T *pu, const T *pd, const T *pz, int64_t off, int64_t nvalid) {
        if (VEC && nvalid >= OS) {
            ru = Pack<T, OS>::load(pu + off);
            rd = Pack<T, OS>::load(pd + off);
            if (GATE) rz = Pack<T, OS>::load(pz + off);
        } else {
            // tail (or unaligned rows): gather the valid steps, zero the rest
            T su[OS], sd[OS], sz[OS];
#pragma unroll
            for (int i = 0; i < OS; ++i) {
                const bool ok = i < nvalid;
                su[i] = ok ? pu[off + i] : T(0);
                sd[i] = ok ? pd[off + i] : T(0);
                sz[i] = (ok && GATE) ? pz[off + i] : T(0);
            }
            __builtin_memcpy(&ru, su, sizeof(ru));
            __builtin_memcpy(&rd, sd, sizeof(rd));
            __builtin_memcpy(&rz, sz, sizeof(rz));
        }
    }
    __device__ void unpack() {
        Pack<T, OS>::unpack(ru, u);
        Pack<T, OS>::unpack(rd, dr);
        if (GATE) Pack<T, OS>::unpack(rz, z);
    }
};

// LDS of one workgroup.  dl / dl*u are double-buffered so that the
// state-only walk needs one barrier per chunk.
template <int W>
struct Smem {
    float dl[2][kCh * kPitch];
    float du[2][kCh * kPitch];
    float p[4 * W * kCh * kPitch];
};

// Per-thread view of one (batch, 16-channel group) problem slice.
template <typename T, int W, int NPL, bool GATE, bool VEC>
struct Walker {
    static constexpr int kRows = 4 * W;            // rows of 16 lanes
    static constexpr int OS = kT * kCh / (64 * W); // steps per owner thread (4 or 2)
    static constexpr int OPC = kT / OS;            // owner threads per channel

    // scan-lane role
    int prow, j;
    float A2[NPL];
    int64_t bcrow[NPL];
    bool nok[NPL];
    const T *Bm, *Cm;
    // owner role
    int oc, ok;
    const T *pu, *pd, *pz;
    T *py;                 // null when the owner's channel is past the end
    float bias, skip;
    int64_t L;
    float sdl;             // owner's running sum of dl over the walked steps

    __device__ void init(const T *u, const T *delta, const float *delta_bias, const float *A,
                         const T *B, const T *C, const float *Dskip, const T *z, T *y,
                         int64_t L_, int dim, int N, int64_t b, int d0) {
        const int tid = threadIdx.x;
        const int lane = tid & 63;
        prow = (tid >> 6) * 4 + (lane >> 4);
        j = lane & 15;
        L = L_;
        Bm = B;
        Cm = C;
        const int dS = min(d0 + j, dim - 1);
#pragma unroll
        for (int g = 0; g < NPL; ++g) {
            const int n = prow * NPL + g;
            nok[g] = n < N;
            A2[g] = nok[g] ? A[static_cast<int64_t>(dS) * N + n] * kLog2e : 0.0f;
            bcrow[g] = (b * N + min(n, N - 1)) * L;
        }
        oc = tid / OPC;
        ok = tid % OPC;
        const int dO = min(d0 + oc, dim - 1);
        const int64_t orow = (b * dim + dO) * L;
        bias = delta_bias ? delta_bias[dO] : 0.0f;
        skip = Dskip ? Dskip[dO] : 0.0f;
        pu = u + orow;
        pd = delta + orow;
        pz = GATE ? z + orow : nullptr;
        py = (y && d0 + oc < dim) ? y + orow : nullptr;
        sdl = 0.0f;
    }

    // B / C values this lane contributes to the row broadcasts of one chunk.
    __device__ void load_bc(int64_t t0, int64_t t_end, float (&bs)[2][NPL], float (&cs)[2][NPL],
                            bool with_c) const {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int64_t t = t0 + 16 * q + j;
#pragma unroll
            for (int g = 0; g < NPL; ++g) {
                const bool ok2 = t < t_end && nok[g];
                bs[q][g] = ok2 ? Io<T>::load(Bm, bcrow[g] + t) : 0.0f;
                cs[q][g] = (ok2 && with_c) ? Io<T>::load(Cm, bcrow[g] + t) : 0.0f;
            }
        }
    }

    // Walk steps [t_begin, t_end) from state h (updated in place).  OUT: also
    // form and store y; otherwise only the state and the owner's sum of dl.
    // t_begin must be a multiple of OS; every thread of the workgroup calls
    // this with the same range.
    template <bool OUT>
    __device__ void walk(int64_t t_begin, int64_t t_end, float (&h)[NPL], Smem<W> &sm) {
        const int64_t nchunks = (t_end - t_begin + kT - 1) / kT;
        OwnerIn<T, OS, VEC, GATE && OUT> nxt;
        float nb[2][NPL], nc[2][NPL];
        {
            const int64_t off = t_begin + OS * ok;
            nxt.load(pu, pd, pz, off, t_end - off);
            load_bc(t_begin, t_end, nb, nc, OUT);
        }
        for (int64_t c = 0; c < nchunks; ++c) {
            const int64_t t0 = t_begin + c * kT;
            const int buf = OUT ? 0 : static_cast<int>(c & 1);
            OwnerIn<T, OS, VEC, GATE && OUT> cur = nxt;
            float cb[2][NPL], cc[2][NPL];
#pragma unroll
            for (int q = 0; q < 2; ++q)
#pragma unroll
                for (int g = 0; g < NPL; ++g) { cb[q][g] = nb[q][g]; cc[q][g] = nc[q][g]; }
            if (c + 1 < nchunks) {
                const int64_t off = t0 + kT + OS * ok;
                nxt.load(pu, pd, pz, off, t_end - off);
                load_bc(t0 + kT, t_end, nb, nc, OUT);
            }

            // ---- A: per-step scalars of this thread's OS steps --------------
            cur.unpack();
            float dl[OS], du[OS], sk[OS], gz[OS];
#pragma unroll
            for (int i = 0; i < OS; ++i) {
                // computed unconditionally (inputs past the end are zero),
                // then steps past the end become the identity step dl = 0
                const float sp = softplus(cur.dr[i] + bias);
                dl[i] = t0 + OS * ok + i < t_end ? sp : 0.0f;
                du[i] = dl[i] * cur.u[i];
                if (OUT) {
                    sk[i] = skip * cur.u[i];
                    gz[i] = GATE ? silu(cur.z[i]) : 1.0f;
                } else {
                    sdl += dl[i];
                }
            }
#pragma unroll
            for (int i = 0; i < OS; i += 2) {
                *reinterpret_cast<float2 *>(sm.dl[buf] + oc * kPitch + OS * ok + i) = make_float2(dl[i], dl[i + 1]);
                *reinterpret_cast<float2 *>(sm.du[buf] + oc * kPitch + OS * ok + i) = make_float2(du[i], du[i + 1]);
            }
            __syncthreads();

            // ---- B: 32 steps of the recurrence for this lane ----------------
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                float dls[16], dus[16], p[16];
                const float4 *pdl = reinterpret_cast<const float4 *>(sm.dl[buf] + j * kPitch + 16 * q);
                const float4 *pdu = reinterpret_cast<const float4 *>(sm.du[buf] + j * kPitch + 16 * q);
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const float4 a = pdl[k], e = pdu[k];
                    dls[4 * k] = a.x; dls[4 * k + 1] = a.y; dls[4 * k + 2] = a.z; dls[4 * k + 3] = a.w;
                    dus[4 * k] = e.x; dus[4 * k + 1] = e.y; dus[4 * k + 2] = e.z; dus[4 * k + 3] = e.w;
                }
#define MSSM_STEP(S)                                                           \
    {                                                                          \
        float acc = 0.0f;                                                      \
        _Pragma("unroll") for (int g = 0; g < NPL; ++g) {                      \
            const float a = fast_exp2(dls[S] * A2[g]);                         \
            h[g] = fmaf(a, h[g], row_bcast<S>(cb[q][g]) * dus[S]);             \
            if (OUT) acc = g == 0 ? row_bcast<S>(cc[q][g]) * h[g]              \
                                  : fmaf(row_bcast<S>(cc[q][g]), h[g], acc);   \
        }                                                                      \
        p[S] = acc;                                                            \
    }
                MSSM_STEP(0) MSSM_STEP(1) MSSM_STEP(2) MSSM_STEP(3)
                MSSM_STEP(4) MSSM_STEP(5) MSSM_STEP(6) MSSM_STEP(7)
                MSSM_STEP(8) MSSM_STEP(9) MSSM_STEP(10) MSSM_STEP(11)
                MSSM_STEP(12) MSSM_STEP(13) MSSM_STEP(14) MSSM_STEP(15)
#undef MSSM_STEP
                if (OUT) {
                    float4 *dst = reinterpret_cast<float4 *>(sm.p + (prow * kCh + j) * kPitch + 16 * q);
#pragma unroll
                    for (int k = 0; k < 4; ++k)
                        dst[k] = make_float4(p[4 * k], p[4 * k + 1], p[4 * k + 2], p[4 * k + 3]);
                }
            }
            if (!OUT) continue;
            __syncthreads();

            // ---- C: reduce the partial sums, skip term, gate, store ---------
            float yv[OS];
#pragma unroll
            for (int i = 0; i < OS; ++i) yv[i] = 0.0f;
#pragma unroll
            for (int r = 0; r < kRows; ++r) {
                const float *src = sm.p + (r * kCh + oc) * kPitch + OS * ok;
#pragma unroll
                for (int i = 0; i < OS; i += 2) {
                    const float2 v = *reinterpret_cast<const float2 *>(src + i);
                    yv[i] += v.x;
                    yv[i + 1] += v.y;
                }
            }
#pragma unroll
            for (int i = 0; i < OS; ++i) yv[i] = (yv[i] + sk[i]) * gz[i];
            const int64_t tt = t0 + OS * ok;
            if (py) {
                if (VEC && tt + OS <= t_end) {
                    Pack<T, OS>::store(py + tt, yv);
                } else {
#pragma unroll
                    for (int i = 0; i < OS; ++i)
                        if (tt + i < t_end) Io<T>::store(py, tt + i, yv[i]);
                }
            }
        }
    }

    // Sum of dl over the walked steps for this lane's channel j, gathered
    // from the OPC owners of the channel through LDS.  Call after a state-only
    // walk; every thread of the workgroup must call it.
    __device__ float channel_dl_sum(Smem<W> &sm) const {
        __syncthreads();                           // last chunk's readers are done
        sm.p[oc * OPC + ok] = sdl;
        __syncthreads();
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < OPC; ++i) s += sm.p[j * OPC + i];
        __syncthreads();                           // sm.p is reused afterwards
        return s;
    }
};

}  // namespace core
}  // namespace mssm
