/*
 * fa_probe.h — roofline probes of the exact tiled attention library.
 *
 * Two measurements of what the current device sustains, used to report the
 * attention kernels' rates against measured ceilings next to the published
 * ones (the attention kernels are bound by the matrix cores, the backward
 * pre-pass and short sequences by HBM). They are not part of the attention
 * computation defined in "Flash attention and efficient attention — Hinglish
 * notes"; that page's "Memory Hierarchy" section motivates measuring the two
 * rates the method trades against each other: on-chip compute versus HBM
 * traffic.
 *
 * Both calls enqueue their kernel on `stream` (a hipStream_t; NULL means the
 * default stream), WAIT for it, and return the measured rate through the
 * last argument. They allocate no device memory.
 */
#ifndef FA_PROBE_H
#define FA_PROBE_H

#include <stddef.h>

#include "fa.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Matrix-core probe: every wave of a full-device grid (two workgroups of
 * four waves per compute unit) issues `iters` rounds of eight independent
 * bf16 32x32x16 MFMAs with float32 accumulation on register operands.
 * *tflops receives 2*32*32*16 * 8 * iters * waves / elapsed seconds / 1e12.
 * Errors: FA_ERR_NULL (tflops NULL), FA_ERR_SHAPE (iters < 1 or > 2^24),
 * FA_ERR_LAUNCH (a HIP call failed). */
fa_status fa_probe_mfma_bf16(int iters, void* stream, double* tflops);

/* HBM probe: a grid-stride copy of `bytes` bytes from src to dst with
 * 16-byte non-temporal loads and stores (four workgroups of 256 threads per
 * compute unit), run `reps` times back to back. *gbs receives
 * 2 * bytes * reps / elapsed seconds / 1e9 (bytes read plus bytes written).
 * src and dst are device pointers owned by the caller, 16-byte aligned and
 * non-overlapping; bytes is a positive multiple of 16. Errors: FA_ERR_NULL,
 * FA_ERR_ALIGN (pointer or size not a multiple of 16), FA_ERR_SHAPE
 * (bytes == 0, reps < 1), FA_ERR_ALIAS (ranges overlap), FA_ERR_LAUNCH. */
fa_status fa_probe_copy(const void* src, void* dst, size_t bytes, int reps, void* stream,
                        double* gbs);

#ifdef __cplusplus
}
#endif

#endif /* FA_PROBE_H */
