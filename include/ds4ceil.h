/* ds4ceil.h — measured ceilings for the roofline fractions of libds4attn's kernels.
 *
 * Not steps of the method: two plain kernels that show what this GPU delivers to the units
 * the hot path is bound by, so that bench.py can report each kernel's fraction of the
 * published peak and of this measured ceiling.  Both are asynchronous on `stream`.
 * Return 0, DS4A_CEIL_EINVAL for a bad argument (nothing launched), DS4A_CEIL_ELAUNCH for a
 * launch error.
 */
#ifndef DS4CEIL_H
#define DS4CEIL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DS4A_CEIL_EINVAL (-1)
#define DS4A_CEIL_ELAUNCH (-7)

/* HBM read stream: reads `bytes` (a multiple of 16, >= 16) of device memory at `src` (16-byte
 * aligned) once, 16 bytes per thread per iteration, non-temporal, with `grid` workgroups of
 * 256 threads (1..2^20); writes one uint32 per thread to sink[grid * 256] (device memory). */
int ds4a_ceiling_read(const void *src, int64_t bytes, int grid, uint32_t *sink, void *stream);

/* bf16 matrix cores: `grid` workgroups of 4 waves, each wave running `iters` rounds of 8
 * independent v_mfma_f32_16x16x32_bf16 (operands in registers); writes one float per thread
 * to sink[grid * 256] and, if flops is not NULL, the launch's dense flop count to *flops (host
 * memory). */
int ds4a_ceiling_mfma(int64_t iters, int grid, float *sink, double *flops, void *stream);

#ifdef __cplusplus
}
#endif
#endif
