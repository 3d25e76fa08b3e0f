/*
 * mssm.h -- C ABI of libmssm, the MI355X (gfx950) selective-scan forward.
 *
 * Sources (web pages on selective state-space models, cited by title and
 * section):
 *   [ybb]  "Mamba状态空间模型的硬件感知推理优化：从选择性扫描到并行前缀和"
 *          (ybb.press/llm/14642) -- section 1: recurrence h_t = A h_{t-1} +
 *          B x_t, output y_t = C h_t; section 3.1: one fused kernel computing
 *          the decay exp(A*softplus(dt)), the input term, the scan and
 *          y = C.h + D*x, returning the final state; section 4: the Mamba-2
 *          scalar per-step decay; section 5: chunked walk keeping the state
 *          on chip.
 *   [mhpq] essay at www.mhpq.cn/news/984979 -- section 2.2: zero-order-hold
 *          step A_d = exp(A dt) and the skip term D u; section 2.3: the pair
 *          operator (A1,B1) (+) (A2,B2) = (A2 A1, A2 B1 + B2) whose prefix is
 *          the scan; section 3.1: diagonal A, elementwise exponential.
 *   [csdn] "从硬件感知到算法革命：Mamba如何重塑序列建模的计算效率"
 *          (tencentcloud.csdn.net) -- section 2: Delta = softplus(.), B and C
 *          input-dependent; section 3: SSM output merged with a SiLU gate.
 *   [mlqm] essay at www.mlqm.cn/news/983902 -- section 5.4: token-by-token
 *          decoding keeps only the fixed-size evolving state between steps.
 * [ybb] section 2.1 also writes the recurrence as a product of augmented
 * matrices applied to [h_0; 1], and its section 5 walks the chunks from an
 * initial state h0; [mhpq] section 4.2 keeps the state in a preallocated
 * buffer updated in place.
 *
 * Conventions shared by every entry point:
 *   - Tensor arguments are DEVICE pointers owned by the caller, contiguous in
 *     the stated row-major layouts, 16-byte aligned for the fast path (any
 *     4-byte (f32) / 2-byte (bf16) aligned pointer is accepted).  They must
 *     stay valid until the work queued on `stream` has finished.  The library
 *     keeps no pointer after a call returns.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Calls are
 *     asynchronous: a return of MSSM_OK means the work was queued.  Faults
 *     inside a kernel surface at the caller's next synchronisation.
 *   - Outputs are overwritten, never accumulated into.  Outputs must not
 *     overlap any input (checked on the pointer ranges; MSSM_ERR_INVALID_ARG).
 *   - Validation happens before any HIP call.  On failure nothing is queued,
 *     the status is returned and mssm_last_error() (thread-local) describes
 *     it.  No call aborts, throws or prints.
 *   - Arithmetic is float32 with float32 state whatever the I/O dtype; bf16
 *     outputs are rounded to nearest even.
 *   - Scratch memory, where a kernel variant needs it, is allocated and freed
 *     stream-ordered on `stream` from a memory pool the library creates per
 *     device (hipMallocFromPoolAsync/hipFreeAsync).  The pool keeps freed
 *     memory for later calls (its release threshold is unlimited), so it
 *     holds up to the largest scratch in use at once until the process ends.
 */
#ifndef MSSM_H
#define MSSM_H

#include <stdint.h>

#if defined(MSSM_BUILDING_LIBRARY)
#define MSSM_API __attribute__((visibility("default")))
#else
#define MSSM_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MSSM_OK = 0,
    MSSM_ERR_INVALID_ARG = 1,   /* null required pointer, bad dims, aliasing   */
    MSSM_ERR_UNSUPPORTED = 2,   /* valid but outside this build's limits       */
    MSSM_ERR_HIP = 3,           /* a HIP runtime call or launch failed          */
    MSSM_ERR_ALLOC = 4          /* scratch allocation failed                    */
} mssm_status;

typedef enum {
    MSSM_F32 = 0,
    MSSM_BF16 = 1
} mssm_dtype;

/* Kernel variant selection (for tests and tuning; AUTO picks by shape). */
typedef enum {
    MSSM_VARIANT_AUTO = 0,
    MSSM_VARIANT_ROWSERIAL = 1, /* one lane per (b,d) row, whole-L serial walk */
    MSSM_VARIANT_CHUNKED = 2,   /* lanes over (row, n), L walked in chunks     */
    MSSM_VARIANT_LOOKBACK = 3,  /* L split across workgroups, decoupled carry  */
    MSSM_VARIANT_SSD_RECURRENT = 4,
    MSSM_VARIANT_SSD_CHUNKED = 5,
    MSSM_VARIANT_PAIRSCAN = 6,  /* steps of a chunk split across lanes: pair
                                   scan across rows, N <= 16, no prologue   */
    MSSM_VARIANT_PAIRSCAN2 = 7  /* the same with two slices of waves per
                                   chunk, combined through LDS               */
} mssm_variant;

/* Sizes of a selective-scan problem. */
typedef struct {
    int64_t batch;   /* >= 0 */
    int64_t seqlen;  /* L >= 0 */
    int64_t dim;     /* channels D >= 0 */
    int64_t dstate;  /* state size N, 1 <= N <= MSSM_MAX_DSTATE */
} mssm_scan_dims;

/* Storage dtypes.  `io` covers the activations (u, delta, B, C, z, y; for
 * SSD x, dt, B, C, y).  `param` covers A, D, delta_bias / dt_bias and must
 * be MSSM_F32.  h_last is always float32. */
typedef struct {
    int32_t io;      /* mssm_dtype */
    int32_t param;   /* mssm_dtype, MSSM_F32 only */
} mssm_dtypes;

#define MSSM_MAX_DSTATE 64      /* selective scan: largest N this build runs */
#define MSSM_SSD_MAX_DSTATE 256 /* SSD: largest N */
#define MSSM_SSD_MAX_HEADDIM 256

/*
 * Selective-scan forward ([ybb] sections 1, 3.1; [mhpq] sections 2.2-2.3,
 * 3.1; [csdn] sections 2-3).  For every batch b and channel d, from h = 0:
 *
 *   dl        = softplus(delta[b,d,t] + delta_bias[d])
 *   h[n]      = exp(dl * A[d,n]) * h[n] + dl * B[b,n,t] * u[b,d,t]
 *   y[b,d,t]  = (sum_n C[b,n,t] * h[n] + D[d] * u[b,d,t]) * silu(z[b,d,t])
 *   h_last[b,d,n] = h[n] after t = L-1
 *
 * The recurrence is evaluated as a parallel scan over the pair operator
 * (a1,b1) (+) (a2,b2) = (a2 a1, a2 b1 + b2); the result equals the
 * sequential loop up to float32 rounding order.
 *
 * Arguments (device pointers unless stated):
 *   u, delta   (batch, dim, L), dtype `io`           required
 *   delta_bias (dim) float32                         nullable -> 0
 *   A          (dim, N) float32 (expected < 0)       required
 *   B, C       (batch, N, L), dtype `io`             required
 *   D          (dim) float32                         nullable -> no skip term
 *   z          (batch, dim, L), dtype `io`           nullable -> no gate
 *   y          (batch, dim, L), dtype `io`           required (output)
 *   h_last     (batch, dim, N) float32               nullable (output)
 * Errors: MSSM_ERR_INVALID_ARG for a null required pointer, a negative
 * size, N < 1, an unknown dtype, or an output overlapping an input;
 * MSSM_ERR_UNSUPPORTED for N > MSSM_MAX_DSTATE or param dtype != F32.
 * batch == 0 or dim == 0: nothing to do, MSSM_OK.  L == 0: h_last is
 * zero-filled, y is empty.
 */
MSSM_API mssm_status mssm_selective_scan_fwd(const void *u, const void *delta,
                                    const float *delta_bias, const float *A,
                                    const void *B, const void *C,
                                    const float *D, const void *z, void *y,
                                    float *h_last, mssm_scan_dims dims,
                                    mssm_dtypes dtypes, void *stream);

/*
 * The selective-scan forward fed by its convolution prologue ([csdn]
 * section 3: a local convolution and a SiLU precede the selective SSM in the
 * Mamba block, kernel size 4; [mlqm] section 3.3: d_conv = 4).  The scan
 * input is formed on chip from x and never stored:
 *
 *   u[b,d,t] = silu(conv_b[d] + sum_{k=0..3} conv_w[d,k] * x[b,d,t-3+k])
 *
 * with x = 0 before step 0 (a causal, zero-padded depthwise convolution);
 * then the selective scan of mssm_selective_scan_fwd_h0 on u, including
 * the skip term D[d] * u.
 *
 *   x       (batch, dim, L), dtype `io`        required (the prologue input)
 *   conv_w  (dim, MSSM_CONV_WIDTH) float32     required
 *   conv_b  (dim) float32                      nullable -> 0
 * Everything else (delta ... h_last, errors, variants) is as for
 * mssm_selective_scan_fwd_h0; h0 does not carry the convolution's window,
 * so a continued sequence restarts it from zero.
 */
#define MSSM_CONV_WIDTH 4
MSSM_API mssm_status mssm_selective_scan_fwd_conv(const void *x, const float *conv_w,
                                         const float *conv_b, const void *delta,
                                         const float *delta_bias, const float *A,
                                         const void *B, const void *C,
                                         const float *D, const void *z,
                                         const float *h0, void *y, float *h_last,
                                         mssm_scan_dims dims, mssm_dtypes dtypes,
                                         void *stream);

/*
 * Backward of the selective scan (the reverse-mode derivative of
 * mssm_selective_scan_fwd_h0; [mlqm] section 3.2: the block is trained,
 * forward and backward).  Given the forward's inputs and the gradients of a
 * loss with respect to y (dy) and h_last (dh_last), it writes the loss's
 * gradients with respect to every input.  The states are recomputed from
 * the inputs (stored every few steps in stream-ordered scratch), not read
 * from the forward.
 *
 * Inputs: u ... h0 as for mssm_selective_scan_fwd_h0;
 *   dy       (batch, dim, L), dtype `io`     required
 *   dh_last  (batch, dim, N) float32         nullable -> 0
 * Outputs, all float32 whatever the I/O dtype (like h_last):
 *   du, ddelta    (batch, dim, L) float32      required
 *   dz            (batch, dim, L) float32      nullable; needs z
 *   dB, dC        (batch, N, L) float32        nullable
 *   dA            (dim, N) float32             nullable
 *   dD, ddelta_bias (dim) float32              nullable (gradients at D
 *                                              = 0 / bias = 0 when those
 *                                              inputs are null)
 *   dh0           (batch, dim, N) float32      nullable
 * dB and dC sum over channels in a fixed order (deterministic); dA, dD and
 * ddelta_bias sum over batches with float32 atomic additions, so their last
 * bits depend on the order.  Scratch is allocated and freed stream-ordered:
 * the states every 16 steps (batch * dim * ceil(L / 16) * 64 bytes for
 * N <= 16) and, when dB or dC is requested,
 * per-wave partial sums of about batch * dim / 8 * L * 128 bytes for
 * 8 < N <= 16 (half that for N <= 8; 4.3 GB for L = 2^20 with 256
 * channels); an allocation failure returns MSSM_ERR_ALLOC.  Errors as for
 * the forward, plus MSSM_ERR_INVALID_ARG for dz without z or any output
 * overlapping an input or another output.
 */
MSSM_API mssm_status mssm_selective_scan_bwd(const void *u, const void *delta,
                                    const float *delta_bias, const float *A,
                                    const void *B, const void *C, const float *D,
                                    const void *z, const float *h0, const void *dy,
                                    const float *dh_last, float *du, float *ddelta,
                                    float *ddelta_bias, float *dA, float *dB,
                                    float *dC, float *dD, float *dz, float *dh0,
                                    mssm_scan_dims dims, mssm_dtypes dtypes,
                                    void *stream);

/* Sizes of a Mamba-2 scalar-decay (SSD) problem. */
typedef struct {
    int64_t batch;
    int64_t seqlen;   /* L */
    int64_t nheads;   /* H */
    int64_t headdim;  /* P, 1 <= P <= MSSM_SSD_MAX_HEADDIM */
    int64_t dstate;   /* N, 1 <= N <= MSSM_SSD_MAX_DSTATE */
    int64_t ngroups;  /* G >= 1, H % G == 0; head h reads group h / (H/G) */
    int64_t chunk;    /* chunk length of the matrix-core form; 0 -> 256 */
} mssm_ssd_dims;

/*
 * Mamba-2 scalar-decay forward ([ybb] section 4: one decay per step and head,
 * shared by all state elements; section 6.2: cumulative products taken in
 * log space).  For every batch b and head h (group g), from S = 0:
 *
 *   dl          = softplus(dt[b,t,h] + dt_bias[h])
 *   S[p][n]     = exp(dl * A[h]) * S[p][n] + dl * x[b,t,h,p] * B[b,t,g,n]
 *   y[b,t,h,p]  = sum_n C[b,t,g,n] * S[p][n] + D[h] * x[b,t,h,p]
 *   h_last[b,h,p,n] = S[p][n] after t = L-1
 *
 * Arguments (device pointers unless stated):
 *   x        (batch, L, H, P), dtype `io`     required
 *   dt       (batch, L, H),    dtype `io`     required
 *   dt_bias  (H) float32                      nullable -> 0
 *   A        (H) float32                      required
 *   B, C     (batch, L, G, N), dtype `io`     required
 *   D        (H) float32                      nullable -> no skip term
 *   y        (batch, L, H, P), dtype `io`     required (output)
 *   h_last   (batch, H, P, N) float32         nullable (output)
 * Errors as for mssm_selective_scan_fwd; also MSSM_ERR_INVALID_ARG when
 * H % G != 0 or chunk < 0, MSSM_ERR_UNSUPPORTED beyond the P/N limits.
 */
MSSM_API mssm_status mssm_ssd_scalar_fwd(const void *x, const void *dt,
                                const float *dt_bias, const float *A,
                                const void *B, const void *C, const float *D,
                                void *y, float *h_last, mssm_ssd_dims dims,
                                mssm_dtypes dtypes, void *stream);

/*
 * Both forwards from a given initial state ([ybb] sections 2.1 and 5): the
 * recurrence starts at h0 instead of 0, so a long sequence can be processed
 * in pieces, each call continuing from the h_last of the previous one.
 *
 *   h0  (batch, dim, N) float32 for the selective scan,
 *       (batch, H, P, N) float32 for SSD          nullable -> 0
 *
 * h0 may be the very buffer passed as h_last (same pointer): the state is
 * then advanced in place.  Any other overlap of h0 with an output is
 * MSSM_ERR_INVALID_ARG.  L == 0 copies h0 to h_last.  Everything else --
 * layouts, variants, errors -- is as for the entry points without h0, which
 * equal these with h0 = NULL.
 */
MSSM_API mssm_status mssm_selective_scan_fwd_h0(const void *u, const void *delta,
                                       const float *delta_bias, const float *A,
                                       const void *B, const void *C,
                                       const float *D, const void *z,
                                       const float *h0, void *y, float *h_last,
                                       mssm_scan_dims dims, mssm_dtypes dtypes,
                                       void *stream);
MSSM_API mssm_status mssm_ssd_scalar_fwd_h0(const void *x, const void *dt,
                                   const float *dt_bias, const float *A,
                                   const void *B, const void *C, const float *D,
                                   const float *h0, void *y, float *h_last,
                                   mssm_ssd_dims dims, mssm_dtypes dtypes,
                                   void *stream);

/*
 * mssm_selective_scan_fwd_h0 for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  It calls no hipMalloc, hipMallocAsync, hipFree or other
 * allocating routine.  The look-back variant's scratch (its published
 * carries, flags and work ticket) lives in a fixed device array of
 * MSSM_NOALLOC_SCRATCH_BYTES on each device the library runs on, held until
 * the process ends; the other variants need no scratch.  The flags and the
 * ticket are cleared by a kernel at the start of each call.
 *
 * Arguments, layouts, variants and results are those of
 * mssm_selective_scan_fwd_h0 (bitwise the same outputs).  The caller still
 * provides every input and output.
 * Limit: a problem whose look-back scratch exceeds the array returns
 * MSSM_ERR_UNSUPPORTED before anything is queued (the look-back variant
 * needs about 2 KB per (segment, 16-channel group) for N <= 16 and up to
 * 8 KB for larger N, with about 768 of them when AUTO chooses it: 1.5 MB for
 * a million-step sequence of 256 channels).
 * Every call on a device shares that device's array, so calls that overlap
 * on one device (on different streams or threads) race and must be
 * serialised by the caller.
 */
#define MSSM_NOALLOC_SCRATCH_BYTES (8u << 20)
MSSM_API mssm_status mssm_selective_scan_fwd_h0_noalloc(const void *u, const void *delta,
                                               const float *delta_bias, const float *A,
                                               const void *B, const void *C,
                                               const float *D, const void *z,
                                               const float *h0, void *y, float *h_last,
                                               mssm_scan_dims dims, mssm_dtypes dtypes,
                                               void *stream);

/*
 * The SSD forward with a SiLU gate on its output ([csdn] section 3: a SiLU
 * branch gates the SSM output; the same reading as the selective scan's z):
 *
 *   y[b,t,h,p] = (sum_n C[b,t,g,n] * S[p][n] + D[h] * x[b,t,h,p]) * silu(z[b,t,h,p])
 *
 *   z    (batch, L, H, P), dtype `io`, like x   nullable -> no gate
 *   h0   (batch, H, P, N) float32               nullable -> 0 (as in the
 *                                               _h0 entry point)
 * Everything else is as for mssm_ssd_scalar_fwd_h0, which equals this with
 * z = NULL.
 */
MSSM_API mssm_status mssm_ssd_scalar_fwd_gated(const void *x, const void *dt,
                                      const float *dt_bias, const float *A,
                                      const void *B, const void *C,
                                      const float *D, const void *z,
                                      const float *h0, void *y, float *h_last,
                                      mssm_ssd_dims dims, mssm_dtypes dtypes,
                                      void *stream);

/* Sizes of one decode step. */
typedef struct {
    int64_t batch;   /* >= 0 */
    int64_t dim;     /* channels D >= 0 */
    int64_t dstate;  /* state size N, 1 <= N <= MSSM_MAX_DSTATE */
} mssm_step_dims;

/*
 * One decode step of the selective scan ([mlqm] section 5.4: incremental
 * decoding carries only the fixed-size state; [mhpq] section 4.2: the state
 * cache is a preallocated buffer; the step itself is the recurrence of
 * mssm_selective_scan_fwd at a single time t):
 *
 *   dl              = softplus(dt[b,d] + dt_bias[d])
 *   state[b,d,n]    = exp(dl * A[d,n]) * state[b,d,n] + dl * B[b,n] * x[b,d]
 *   y[b,d]          = (sum_n C[b,n] * state[b,d,n] + D[d] * x[b,d]) * silu(z[b,d])
 *
 * It equals mssm_selective_scan_fwd_h0 with L = 1 and h0 = h_last = state.
 *
 * Arguments (device pointers unless stated):
 *   state    (batch, dim, N) float32       required, read and overwritten
 *   x, dt    (batch, dim), dtype `io`      required
 *   dt_bias  (dim) float32                 nullable -> 0
 *   A        (dim, N) float32              required
 *   B, C     (batch, N), dtype `io`        required
 *   D        (dim) float32                 nullable -> no skip term
 *   z        (batch, dim), dtype `io`      nullable -> no gate
 *   y        (batch, dim), dtype `io`      required (output)
 * Errors: as for mssm_selective_scan_fwd; state and y must not overlap any
 * input or each other.  batch == 0 or dim == 0: nothing to do, MSSM_OK.
 */
MSSM_API mssm_status mssm_selective_state_update(float *state, const void *x,
                                        const void *dt, const float *dt_bias,
                                        const float *A, const void *B,
                                        const void *C, const float *D,
                                        const void *z, void *y,
                                        mssm_step_dims dims, mssm_dtypes dtypes,
                                        void *stream);

/* Force a kernel variant for subsequent calls made by THIS thread
 * (MSSM_VARIANT_AUTO restores the shape-based choice).  A variant that does
 * not apply to the entry point or shape makes that call return
 * MSSM_ERR_UNSUPPORTED.  Returns the previous setting. */
MSSM_API mssm_variant mssm_force_variant(mssm_variant v);

/* The variant the most recent successful call on this thread launched. */
MSSM_API mssm_variant mssm_last_variant(void);

/* Static description of a status code (never NULL). */
MSSM_API const char *mssm_status_string(mssm_status s);

/* Thread-local text of the last error on this thread ("" if none).  The
 * pointer stays valid until the next library call on the same thread. */
MSSM_API const char *mssm_last_error(void);

/* Library version as major*10000 + minor*100 + patch. */
MSSM_API int mssm_version(void);

/* Identity of the sources this binary was built from: 16 hex digits of a
 * SHA-256 over the kernel and host sources, this header and the compile
 * flags.  A binding compares it with the hash of the sources it ships with
 * and refuses a binary built from others.  Never NULL. */
MSSM_API const char *mssm_source_hash(void);

/* Status bits that kernels set on a device while they run. */
#define MSSM_DEVICE_LOOKBACK_TIMEOUT 0x1u /* a look-back wait gave up */

/*
 * Device status of the CURRENT device.  Waits for all work queued on the
 * device (hipDeviceSynchronize), then writes into *bits the status bits set
 * by this library's kernels since they were last cleared, and clears them
 * when `clear` is nonzero.  The bits are the device's, shared by every
 * stream and thread.
 *
 * MSSM_DEVICE_LOOKBACK_TIMEOUT: a workgroup of the look-back variant
 * (MSSM_VARIANT_LOOKBACK) waited about a second per predecessor for a
 * predecessor's published carry and gave up.  Predecessors always publish
 * before they wait, so this marks a defect, not a slow device; that call's
 * outputs from the affected segment on (y and h_last) are NaN rather than
 * wrong numbers, and the call itself returned MSSM_OK when it was queued.
 *
 * Errors: MSSM_ERR_INVALID_ARG if bits is NULL; MSSM_ERR_HIP if the
 * synchronisation or a copy fails (including a fault of earlier work).
 */
MSSM_API mssm_status mssm_device_status(uint32_t *bits, int clear);

#ifdef __cplusplus
}
#endif

#endif /* MSSM_H */
