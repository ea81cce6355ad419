/*
 * fa_tuning.h — explicit kernel-shape selection for timing comparisons.
 *
 * fa_fwd and fa_bwd (fa.h) always run the kernel shapes measured fastest on
 * MI355X; nothing in the environment changes that. These two entry points run
 * the same operation with an alternative shape chosen by `cfg`, so that tile
 * sizes can be compared by interleaved timing and every alternative can be
 * held to the same parity bar as the default. The tile sizes themselves are
 * the subject of "What the tiling is actually constrained by" (sections "The
 * formula, which the title only gestures at" and "The successor tunes rather
 * than derives"): a derived formula against a hand-tuned set.
 *
 * Arguments, conventions, results and errors are those of fa_fwd / fa_bwd,
 * plus FA_ERR_CONFIG for a cfg outside the list below. cfg = 0 is exactly
 * fa_fwd / fa_bwd. Every cfg computes the same attention; only the rounding
 * order of the float32 sums may differ.
 *
 * Forward, bf16 (query rows per wave x waves per workgroup, keys per tile):
 *   d = 128: 1 = 32 x 8, 64 keys;  2 = block-pipelined 32 x 8, 128 keys;
 *            3 = block-pipelined 32 x 8, 64 keys;  4 = 32 x 4, 64 keys;
 *            7 = 32 x 4, 160 keys (the derived tile: B_c = ceil(M / 4d) with
 *                M = 160 KiB of LDS in bf16 elements, B_r = 128);
 *            8 = 32 x 8, 160 keys (the derived B_c with the default 256 rows);
 *            9 = ping-pong schedule, 32 x 8, 128 keys (the two waves of each
 *                SIMD one phase apart: one on the matrix core while the
 *                other runs the softmax);
 *            5, 6 = the default.
 *   d = 64:  1 = 32 x 8, 64 keys;  2 = block-pipelined 32 x 8, 128 keys;
 *            3 = 32 x 8, 128 keys;  4 = 32 x 4, 64 keys;
 *            5 = block-pipelined 32 x 8, 64 keys;
 *            6 = 64 x 4 or 64 x 8 (the workgroup size the mask does not pick);
 *            7 = 32 x 2, 320 keys (the derived tile at d = 64: B_c = 320,
 *                B_r = 64);
 *            8 = 64 x 4, 320 keys (the derived B_c with 256 rows);
 *            9 = ping-pong schedule, 64 x 8, 64 keys.
 *   float32: only cfg = 0.
 * Backward, bf16: 2 = the other workgroup size (4 or 8 waves) than the mask
 *   picks; float32: only cfg = 0.
 */
#ifndef FA_TUNING_H
#define FA_TUNING_H

#include <stddef.h>

#include "fa.h"

#ifdef __cplusplus
extern "C" {
#endif

fa_status fa_fwd_tuned(const void* q, const void* k, const void* v, void* o, float* lse,
                       int B, int H, int N, int d, fa_dtype dtype,
                       float scale, fa_mask mask, int window, int cfg, void* stream);

fa_status fa_bwd_tuned(const void* q, const void* k, const void* v, const void* o,
                       const void* dout, const float* lse, void* dq, void* dk, void* dv,
                       void* workspace, size_t workspace_bytes,
                       int B, int H, int N, int d, fa_dtype dtype,
                       float scale, fa_mask mask, int window, int cfg, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_TUNING_H */
