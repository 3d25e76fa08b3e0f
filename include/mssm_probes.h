/*
 * mssm_probes.h -- measurement probes exported by libmssm, for reading the
 * scan kernels against ceilings measured on the device itself.
 *
 * "Mamba状态空间模型的硬件感知推理优化" (ybb.press) section 1.1 places the
 * selective scan on a roofline: about one to two operations per byte, so
 * memory bandwidth bounds it.  A roofline needs two roofs; these probes
 * measure them where the kernels run:
 *   - the HBM rate a plain streaming copy reaches (mssm_probe_copy);
 *   - the issue rate of the vector-ALU operations the scan is made of
 *     (mssm_probe_valu): fused multiply-add, 2^x (v_exp_f32), log2 x
 *     (v_log_f32) and 1/x (v_rcp_f32).
 * Neither probe computes anything of the method.  Conventions as in mssm.h:
 * device pointers owned by the caller, asynchronous on `stream`, validation
 * before any HIP call, errors in mssm_last_error().
 */
#ifndef MSSM_PROBES_H
#define MSSM_PROBES_H

#include <stdint.h>

#include "mssm.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Copy `bytes` from src to dst with a plain kernel: one 16-byte load and
 * store per thread, in a grid of bytes / 4096 workgroups of 256 threads.
 * Timing it gives the copy ceiling: 2 * bytes / time.
 *   src, dst  device buffers of `bytes` bytes, 16-byte aligned, not
 *             overlapping
 *   bytes     > 0, a multiple of 16, below 2^43
 * Errors: MSSM_ERR_INVALID_ARG for a null pointer, a size that is not a
 * positive multiple of 16, misaligned or overlapping buffers; MSSM_ERR_HIP
 * if the launch fails.
 */
MSSM_API mssm_status mssm_probe_copy(const void *src, void *dst, int64_t bytes, void *stream);

/* Operations of mssm_probe_valu. */
#define MSSM_PROBE_FMA 0   /* x = fma(x, a, b)  (v_fma_f32) */
#define MSSM_PROBE_EXP2 1  /* x = 2^x           (v_exp_f32) */
#define MSSM_PROBE_LOG2 2  /* x = log2 x        (v_log_f32) */
#define MSSM_PROBE_RCP 3   /* x = 1 / x         (v_rcp_f32) */

/* Launch shape of mssm_probe_valu: MSSM_PROBE_VALU_THREADS threads in
 * workgroups of MSSM_PROBE_VALU_BLOCK (eight waves per SIMD on a 256-CU
 * device), each running MSSM_PROBE_VALU_CHAINS independent chains and
 * MSSM_PROBE_VALU_OPS_PER_ITER operations per iteration. */
#define MSSM_PROBE_VALU_BLOCK 256
#define MSSM_PROBE_VALU_THREADS (2048 * 256)
#define MSSM_PROBE_VALU_CHAINS 8
#define MSSM_PROBE_VALU_OPS_PER_ITER 128

/*
 * Run `iters` iterations of operation `op` on every thread of the launch
 * shape above: MSSM_PROBE_VALU_THREADS * iters * MSSM_PROBE_VALU_OPS_PER_ITER
 * lane-operations.  Timing it gives the issue rate of the operation.
 *   op    one of MSSM_PROBE_*
 *   iters >= 1
 *   out   device float buffer of MSSM_PROBE_VALU_THREADS elements; each
 *         thread writes the sum of its chains (so no work is optimised
 *         away); the values mean nothing
 * Errors: MSSM_ERR_INVALID_ARG for an unknown op, iters < 1 or a null out;
 * MSSM_ERR_HIP if the launch fails.
 */
MSSM_API mssm_status mssm_probe_valu(int op, int32_t iters, float *out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MSSM_PROBES_H */
