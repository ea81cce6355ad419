// Host-side argument handling shared by every attention entry point of the
// C ABI (fa_api.hip, fa_bwd_api.hip): problem validation, the band radius the
// kernels receive, pointer checks and the folding of the scale's sign into the
// bf16 operands. One copy, so that a rule changed here holds for all calls.
#pragma once
#include <math.h>
#include <stdint.h>
#include <stddef.h>

#include "fa.h"

namespace fa {
namespace host {

constexpr int64_t kI32Max = 2147483647;
// Longest sequence accepted. The kernels form sums such as
// (first row of a block) + 32 + window in 32-bit integers; with N below 2^29
// and the band radius clamped to N - 1 (below) every such sum stays below
// 2^30 + 512.
constexpr int64_t kMaxN = int64_t(1) << 29;

inline size_t elem_bytes(fa_dtype dt) { return dt == FA_BF16 ? 2 : 4; }

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// [a, a+na) and [b, b+nb) overlap.
inline bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

// Shape, dtype, head dimension, mask and scale of one problem.
inline fa_status check_problem(int B, int H, int N, int d, fa_dtype dtype, float scale,
                               fa_mask mask, int window) {
  if (B < 1 || H < 1 || N < 1) return FA_ERR_SHAPE;
  if ((int64_t)B * H > kI32Max) return FA_ERR_SHAPE;
  if ((int64_t)N > kMaxN) return FA_ERR_SHAPE;
  if (dtype != FA_BF16 && dtype != FA_F32) return FA_ERR_DTYPE;
  if (dtype == FA_BF16 && d != 64 && d != 128) return FA_ERR_HEADDIM;
  if (dtype == FA_F32 && (d < 1 || d > 128)) return FA_ERR_HEADDIM;
  if ((int64_t)N * d > kI32Max) return FA_ERR_SHAPE;
  // one workgroup per 32 query rows at most, per head
  if (((int64_t)N + 31) / 32 * ((int64_t)B * H) > kI32Max) return FA_ERR_SHAPE;
  if (mask != FA_MASK_NONE && mask != FA_MASK_CAUSAL && mask != FA_MASK_LOCAL) return FA_ERR_MASK;
  if (mask == FA_MASK_LOCAL && window < 0) return FA_ERR_MASK;
  if (!isfinite(scale)) return FA_ERR_SCALE;
  return FA_OK;
}

// The band radius the kernels see: 0 unless the mask is the band; for the
// band min(window, N - 1). Every |i - j| of one sequence is at most N - 1, so
// the clamp allows exactly the same pairs, and it keeps the kernels' index
// sums (row + window) inside 32-bit integers for any window up to 2^31 - 1.
inline int kernel_window(fa_mask mask, int window, int N) {
  if (mask != FA_MASK_LOCAL) return 0;
  return window < N - 1 ? window : N - 1;
}

// How the bf16 kernels take the scale. Their exp2 argument needs a positive
// factor, so a negative scale negates Q (or K: exact in bf16) and a zero or
// underflowing scale zeroes it, which makes every logit exactly 0 as a zero
// scale does. The operand bits become (x & q_and) ^ q_xor.
struct ScaleFold {
  float scale_abs;   // |scale|; 1 when the operand is zeroed
  float scale_log2;  // scale_abs * log2(e), a normal positive float
  unsigned q_and;
  unsigned q_xor;
};

inline ScaleFold fold_scale(float scale) {
  const double LOG2E = 1.4426950408889634;
  ScaleFold f;
  double s = fabs((double)scale);
  f.q_and = 0xFFFFFFFFu;
  f.q_xor = scale < 0 ? 0x80008000u : 0u;
  float c = (float)(s * LOG2E);
  if (!(c >= 1.17549435e-38f)) {  // zero, or too small for a normal float factor
    f.q_and = 0u;
    f.q_xor = 0u;
    s = 1.0;
    c = (float)LOG2E;
  }
  f.scale_abs = (float)s;
  f.scale_log2 = c;
  return f;
}

}  // namespace host
}  // namespace fa
