// internal.h -- interface between the C-ABI front end (mssm_api.cpp) and the
// kernel translation units.  Not installed; not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mssm.h"

namespace mssm {

enum IoType : int { IO_F32 = 0, IO_BF16 = 1 };

// One selective-scan problem, already validated.  Layouts as in mssm.h:
// u, delta, z, y (batch, dim, L); B, C (batch, N, L); A (dim, N);
// delta_bias, D (dim); h0, h_last (batch, dim, N).  h0 may be the same
// buffer as h_last (each element is read before it is overwritten) but
// overlaps nothing else.
struct ScanArgs {
    const void *u;
    const void *delta;
    const float *delta_bias;  // may be null
    const float *A;
    const void *B;
    const void *C;
    const float *D;           // may be null
    const void *z;            // may be null
    const float *h0;          // may be null -> the state starts at 0
    void *y;
    float *h_last;            // may be null
    int64_t batch, L, dim, N;
    IoType io;
    // Convolution prologue: when conv_w is set, u holds the input x of a
    // causal width-4 depthwise convolution (conv_w (dim, 4), conv_b (dim)
    // may be null) and the scan runs on silu(conv(x)).
    const float *conv_w = nullptr;
    const float *conv_b = nullptr;
};

// Scratch memory of the variants that need it, stream-ordered on `stream`,
// from a memory pool the library keeps per device.  The pool keeps freed
// memory (release threshold: unlimited) instead of returning it at every
// synchronisation, so calls separated by synchronisations reuse it rather
// than map it again; it holds up to the largest scratch in use at once until
// the process ends.
hipError_t scratch_alloc(void **ptr, size_t bytes, hipStream_t stream);
hipError_t scratch_free(void *ptr, hipStream_t stream);

// One SSD problem, already validated.  Layouts as in mssm.h.
struct SSDArgs {
    const void *x;
    const void *dt;
    const float *dt_bias;     // may be null
    const float *A;
    const void *B;
    const void *C;
    const float *D;           // may be null
    const void *z;            // may be null -> no gate; (batch, L, H, P) like x
    const float *h0;          // may be null; may be the same buffer as h_last
    void *y;
    float *h_last;            // may be null
    int64_t batch, L, H, P, N, G, chunk;
    IoType io;
};

// One decode step of the selective scan, already validated: state
// (batch, dim, N) float32 updated in place; x, dt, z, y (batch, dim);
// B, C (batch, N); A (dim, N); dt_bias, D (dim).
struct StepArgs {
    float *state;
    const void *x;
    const void *dt;
    const float *dt_bias;     // may be null
    const float *A;
    const void *B;
    const void *C;
    const float *D;           // may be null
    const void *z;            // may be null
    void *y;
    int64_t batch, dim, N;
    IoType io;
};

// One selective-scan backward, already validated: the forward's inputs (as in
// ScanArgs), the output gradients dy (like u) and dh_last (batch, dim, N;
// may be null), and the gradient outputs, all float32: du, ddelta, dz
// (batch, dim, L), dB, dC (batch, N, L), dA (dim, N), dD and ddelta_bias
// (dim), dh0 (batch, dim, N).  dA, dB, dC, dD and ddelta_bias are
// accumulated into and must hold zeros on entry.  Optional outputs may be
// null.
struct BwdArgs {
    const void *u;
    const void *delta;
    const float *delta_bias;
    const float *A;
    const void *B;
    const void *C;
    const float *D;
    const void *z;
    const float *h0;
    const void *dy;
    const float *dh_last;
    float *du;
    float *ddelta;
    float *ddelta_bias;
    float *dA;
    float *dB;
    float *dC;
    float *dD;
    float *dz;
    float *dh0;
    int64_t batch, L, dim, N;
    IoType io;
};

// Each launcher queues its kernel(s) on `stream` and returns the launch
// status.  Shapes have been checked against the launcher's limits by the
// caller (see the *_supported helpers).
hipError_t launch_scan_rowserial(const ScanArgs &a, hipStream_t stream);
bool scan_rowserial_supported(const ScanArgs &a);

hipError_t launch_scan_chunked(const ScanArgs &a, hipStream_t stream);
bool scan_chunked_supported(const ScanArgs &a);
int64_t scan_chunked_waves(const ScanArgs &a);
// Rows start 16-byte aligned and L % 8 == 0: activations move as vectors.
// The chunk walk addresses 16 channel rows and the N rows of B / C with
// 32-bit byte offsets: max(16, N) * L elements must fit in 2^31 bytes.
bool scan_offsets_fit(const ScanArgs &a);
bool scan_rows_vectorizable(const ScanArgs &a);

// Steps of each chunk split across the lanes of the workgroup (a scan of
// (decay, state) pairs across rows and, with slices = 2, across waves).
hipError_t launch_scan_pairscan(const ScanArgs &a, hipStream_t stream, int slices);
bool scan_pairscan_supported(const ScanArgs &a);

// Chunk-parallel variant; allocates its look-back scratch stream-ordered.
hipError_t launch_scan_lookback(const ScanArgs &a, hipStream_t stream);
bool scan_lookback_supported(const ScanArgs &a);
// Bytes of look-back scratch a problem needs, and the variant that takes it
// from the device's fixed array of kNoAllocScratchBytes instead of
// allocating (the caller checks the size first).
constexpr size_t kNoAllocScratchBytes = MSSM_NOALLOC_SCRATCH_BYTES;
size_t scan_lookback_scratch_bytes(const ScanArgs &a);
hipError_t launch_scan_lookback_noalloc(const ScanArgs &a, hipStream_t stream);

// Status bits of the current device (mssm_device_status): waits for the
// device, reads them into *bits and clears them when asked.
hipError_t device_status(uint32_t *bits, bool clear);

// Backward: one lane per (batch, channel) row; stream-ordered scratch for the
// stored states.
hipError_t launch_scan_bwd(const BwdArgs &a, hipStream_t stream);
bool scan_bwd_supported(const BwdArgs &a);
// Backward with the chunked forward's decomposition (N <= 16): lanes over
// (channel, state element), states stored every 32 steps, per-workgroup
// partial sums of dB and dC; stream-ordered scratch.
hipError_t launch_scan_bwd_chunked(const BwdArgs &a, hipStream_t stream);
bool scan_bwd_chunked_supported(const BwdArgs &a);

// Measurement probes (include/mssm_probes.h); arguments already checked.
hipError_t launch_probe_copy(const void *src, void *dst, int64_t bytes, hipStream_t stream);
hipError_t launch_probe_valu(int op, int iters, float *out, hipStream_t stream);

hipError_t launch_state_update(const StepArgs &a, hipStream_t stream);
bool state_update_supported(const StepArgs &a);

hipError_t launch_ssd_recurrent(const SSDArgs &a, hipStream_t stream);
bool ssd_recurrent_supported(const SSDArgs &a);

// Chunked matrix-core form (bf16 I/O, N <= 128, chunk 64 / 128 / 256).
hipError_t launch_ssd_chunked(const SSDArgs &a, hipStream_t stream);
bool ssd_chunked_supported(const SSDArgs &a);

}  // namespace mssm
