// scan_chunked.hip -- selective-scan forward, fused, one lane per (channel,
// group of state elements).
//
// Computes, for every (batch b, channel d) and step t
// ("Mamba状态空间模型的硬件感知推理优化" (ybb.press) sections 1 and 3.1;
// www.mhpq.cn/news/984979 essay sections 2.2-2.3):
//   dl   = softplus(delta + delta_bias[d])
//   h[n] = exp(dl * A[d,n]) * h[n] + (dl * u) * B[b,n,t]
//   y    = (sum_n C[b,n,t] * h[n] + D[d] * u) * silu(z)
// walking the sequence in order, so the recurrence is evaluated exactly as the
// sequential definition (no re-association, no second pass, one exponential
// per state element and step).
//
// Work decomposition (gfx950, wave64).  A workgroup of W waves (W = 2 or 4)
// owns 16 channels of one batch and all N state elements.  Lane (wave w, row
// r, column j) -- r = lane / 16, j = lane % 16 -- holds channel j and the NPL
// state elements n = (4w + r) * NPL + g, g < NPL, in registers, so the 4W
// rows of the workgroup cover 4W * NPL >= N state elements.  The sequence is
// walked in chunks of 32 steps:
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
// W = 4 with one state element per lane gives twice the waves of W = 2 with
// two per lane (better latency hiding when channels are few); W = 2 halves
// the partial sums written to LDS.
//
// Ragged lengths: steps t >= L get dl = 0 and dl*u = 0, i.e. the identity pair
// (decay 1, input 0), so the state passes through unchanged.  Channels beyond
// the last compute on clamped inputs and store nothing.
#include "device_math.h"
#include "internal.h"

namespace mssm {
namespace {

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
        if constexpr (sizeof(T) == 4) {
            raw r;
            uint32_t w[OS];
#pragma unroll
            for (int i = 0; i < OS; ++i) w[i] = __float_as_uint(v[i]);
            __builtin_memcpy(&r, w, sizeof(raw));
            *reinterpret_cast<raw *>(p) = r;
        } else {
            uint32_t w[OS / 2];
#pragma unroll
            for (int i = 0; i < OS / 2; ++i) w[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
            raw r;
            __builtin_memcpy(&r, w, sizeof(raw));
            *reinterpret_cast<raw *>(p) = r;
        }
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

template <typename T, int W, int NPL, bool GATE, bool VEC>
__global__ __launch_bounds__(64 * W) void scan_chunked_kernel(
    const T *__restrict__ u, const T *__restrict__ delta,
    const float *__restrict__ delta_bias, const float *__restrict__ A,
    const T *__restrict__ Bm, const T *__restrict__ Cm,
    const float *__restrict__ Dskip, const T *__restrict__ z, T *__restrict__ y,
    float *__restrict__ h_last, int64_t L, int dim, int N, int groups_per_batch) {
    constexpr int kRows = 4 * W;           // rows of 16 lanes: state-element groups
    constexpr int OS = kT * kCh / (64 * W); // steps per owner thread (4 or 2)
    constexpr int OPC = kT / OS;            // owner threads per channel
    __shared__ __align__(16) float sDL[kCh * kPitch];
    __shared__ __align__(16) float sDU[kCh * kPitch];
    __shared__ __align__(16) float sP[kRows * kCh * kPitch];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int prow = (tid >> 6) * 4 + (lane >> 4);   // state-element group
    const int j = lane & 15;                          // channel within the workgroup
    const int64_t b = blockIdx.x / groups_per_batch;
    const int d0 = (blockIdx.x - static_cast<int>(b) * groups_per_batch) * kCh;

    // ---- scan lane: channel d0 + j, state elements prow * NPL + g ----------
    const int dS = min(d0 + j, dim - 1);
    float A2[NPL], h[NPL];
    int64_t bcrow[NPL];
#pragma unroll
    for (int g = 0; g < NPL; ++g) {
        const int n = prow * NPL + g;
        A2[g] = n < N ? A[static_cast<int64_t>(dS) * N + n] * kLog2e : 0.0f;
        h[g] = 0.0f;
        bcrow[g] = (b * N + min(n, N - 1)) * L;
    }

    // ---- owner: channel d0 + oc, steps OS * ok .. OS * ok + OS - 1 ---------
    const int oc = tid / OPC;
    const int ok = tid % OPC;
    const int dO = min(d0 + oc, dim - 1);
    const bool own_store = d0 + oc < dim;
    const int64_t orow = (b * dim + dO) * L;
    const float bias = delta_bias ? delta_bias[dO] : 0.0f;
    const float skip = Dskip ? Dskip[dO] : 0.0f;
    const T *pu = u + orow;
    const T *pd = delta + orow;
    const T *pz = GATE ? z + orow : nullptr;

    const int64_t nchunks = (L + kT - 1) / kT;

    // B / C values this lane contributes to the row broadcasts of one chunk.
    auto load_bc = [&](int64_t t0, float (&bs)[2][NPL], float (&cs)[2][NPL]) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int64_t t = t0 + 16 * q + j;
#pragma unroll
            for (int g = 0; g < NPL; ++g) {
                const bool ok2 = t < L && prow * NPL + g < N;
                bs[q][g] = ok2 ? Io<T>::load(Bm, bcrow[g] + t) : 0.0f;
                cs[q][g] = ok2 ? Io<T>::load(Cm, bcrow[g] + t) : 0.0f;
            }
        }
    };

    OwnerIn<T, OS, VEC, GATE> nxt;
    float nb[2][NPL], nc[2][NPL];
    nxt.load(pu, pd, pz, OS * ok, L - OS * ok);
    load_bc(0, nb, nc);

    for (int64_t c = 0; c < nchunks; ++c) {
        const int64_t t0 = c * kT;
        OwnerIn<T, OS, VEC, GATE> cur = nxt;
        float cb[2][NPL], cc[2][NPL];
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int g = 0; g < NPL; ++g) { cb[q][g] = nb[q][g]; cc[q][g] = nc[q][g]; }
        if (c + 1 < nchunks) {
            const int64_t off = t0 + kT + OS * ok;
            nxt.load(pu, pd, pz, off, L - off);
            load_bc(t0 + kT, nb, nc);
        }

        // ---- A: per-step scalars of this thread's OS steps ------------------
        cur.unpack();
        float dl[OS], du[OS], sk[OS], gz[OS];
#pragma unroll
        for (int i = 0; i < OS; ++i) {
            // computed unconditionally (inputs past the end are zero), then
            // steps past the end become the identity step dl = 0
            const float sp = softplus(cur.dr[i] + bias);
            dl[i] = t0 + OS * ok + i < L ? sp : 0.0f;
            du[i] = dl[i] * cur.u[i];
            sk[i] = skip * cur.u[i];
            gz[i] = GATE ? silu(cur.z[i]) : 1.0f;
        }
#pragma unroll
        for (int i = 0; i < OS; i += 2) {
            *reinterpret_cast<float2 *>(sDL + oc * kPitch + OS * ok + i) = make_float2(dl[i], dl[i + 1]);
            *reinterpret_cast<float2 *>(sDU + oc * kPitch + OS * ok + i) = make_float2(du[i], du[i + 1]);
        }
        __syncthreads();

        // ---- B: 32 steps of the recurrence for this lane's state elements --
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            float dls[16], dus[16], p[16];
            const float4 *pdl = reinterpret_cast<const float4 *>(sDL + j * kPitch + 16 * q);
            const float4 *pdu = reinterpret_cast<const float4 *>(sDU + j * kPitch + 16 * q);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float4 a = pdl[k], e = pdu[k];
                dls[4 * k] = a.x; dls[4 * k + 1] = a.y; dls[4 * k + 2] = a.z; dls[4 * k + 3] = a.w;
                dus[4 * k] = e.x; dus[4 * k + 1] = e.y; dus[4 * k + 2] = e.z; dus[4 * k + 3] = e.w;
            }
#define MSSM_STEP(S)                                                       \
    {                                                                      \
        float acc;                                                         \
        _Pragma("unroll") for (int g = 0; g < NPL; ++g) {                  \
            const float a = fast_exp2(dls[S] * A2[g]);                     \
            h[g] = fmaf(a, h[g], row_bcast<S>(cb[q][g]) * dus[S]);         \
            acc = g == 0 ? row_bcast<S>(cc[q][g]) * h[g]                   \
                         : fmaf(row_bcast<S>(cc[q][g]), h[g], acc);        \
        }                                                                  \
        p[S] = acc;                                                        \
    }
            MSSM_STEP(0) MSSM_STEP(1) MSSM_STEP(2) MSSM_STEP(3)
            MSSM_STEP(4) MSSM_STEP(5) MSSM_STEP(6) MSSM_STEP(7)
            MSSM_STEP(8) MSSM_STEP(9) MSSM_STEP(10) MSSM_STEP(11)
            MSSM_STEP(12) MSSM_STEP(13) MSSM_STEP(14) MSSM_STEP(15)
#undef MSSM_STEP
            float4 *dst = reinterpret_cast<float4 *>(sP + (prow * kCh + j) * kPitch + 16 * q);
#pragma unroll
            for (int k = 0; k < 4; ++k)
                dst[k] = make_float4(p[4 * k], p[4 * k + 1], p[4 * k + 2], p[4 * k + 3]);
        }
        __syncthreads();

        // ---- C: reduce the partial sums, skip term, gate, store ------------
        float yv[OS];
#pragma unroll
        for (int i = 0; i < OS; ++i) yv[i] = 0.0f;
#pragma unroll
        for (int r = 0; r < kRows; ++r) {
            const float *src = sP + (r * kCh + oc) * kPitch + OS * ok;
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
        if (own_store) {
            if (VEC && tt + OS <= L) {
                Pack<T, OS>::store(y + orow + tt, yv);
            } else {
#pragma unroll
                for (int i = 0; i < OS; ++i)
                    if (tt + i < L) Io<T>::store(y, orow + tt + i, yv[i]);
            }
        }
    }

    if (h_last && d0 + j < dim) {
#pragma unroll
        for (int g = 0; g < NPL; ++g) {
            const int n = prow * NPL + g;
            if (n < N) h_last[(b * dim + d0 + j) * static_cast<int64_t>(N) + n] = h[g];
        }
    }
}

template <typename T, int W, int NPL>
hipError_t launch_typed(const ScanArgs &a, hipStream_t stream) {
    const int groups = static_cast<int>((a.dim + kCh - 1) / kCh);
    const int64_t grid = a.batch * groups;
    auto aligned = [](const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
    const bool vec = (a.L % 4 == 0) && aligned(a.u) && aligned(a.delta) && aligned(a.y) &&
                     (!a.z || aligned(a.z));
    decltype(&scan_chunked_kernel<T, W, NPL, true, true>) kern;
    if (a.z) kern = vec ? scan_chunked_kernel<T, W, NPL, true, true> : scan_chunked_kernel<T, W, NPL, true, false>;
    else kern = vec ? scan_chunked_kernel<T, W, NPL, false, true> : scan_chunked_kernel<T, W, NPL, false, false>;
    hipLaunchKernelGGL(kern, dim3(static_cast<uint32_t>(grid)), dim3(64 * W), 0, stream,
                       static_cast<const T *>(a.u), static_cast<const T *>(a.delta),
                       a.delta_bias, a.A, static_cast<const T *>(a.B),
                       static_cast<const T *>(a.C), a.D, static_cast<const T *>(a.z),
                       static_cast<T *>(a.y), a.h_last, a.L, static_cast<int>(a.dim),
                       static_cast<int>(a.N), groups);
    return hipGetLastError();
}

// Four waves with one state element per lane double the waves in flight,
// which matters when the grid is small; two waves with two per lane write
// half the partial sums.  Chosen by how many waves the W = 2 form would put
// on each of the chip's 1024 SIMDs.
template <typename T>
hipError_t launch_by_n(const ScanArgs &a, hipStream_t stream) {
    const int64_t groups = a.batch * ((a.dim + kCh - 1) / kCh);
    const bool few = groups * 2 < 4 * 1024;
    if (a.N <= 16 && few) return launch_typed<T, 4, 1>(a, stream);
    if (a.N <= 8) return launch_typed<T, 2, 1>(a, stream);
    if (a.N <= 16) return launch_typed<T, 2, 2>(a, stream);
    if (a.N <= 32) return launch_typed<T, 2, 4>(a, stream);
    return launch_typed<T, 2, 8>(a, stream);
}

}  // namespace

bool scan_chunked_supported(const ScanArgs &a) {
    const int64_t groups = (a.dim + kCh - 1) / kCh;
    return a.N >= 1 && a.N <= 64 && a.dim <= (int64_t(1) << 30) &&
           a.batch * groups < (int64_t(1) << 31);
}

hipError_t launch_scan_chunked(const ScanArgs &a, hipStream_t stream) {
    if (a.io == IO_F32) return launch_by_n<float>(a, stream);
    return launch_by_n<uint16_t>(a, stream);
}

}  // namespace mssm
