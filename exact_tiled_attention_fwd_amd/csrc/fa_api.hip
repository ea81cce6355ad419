// C ABI entry points (include/fa.h): argument validation, kernel selection
// and launch on the caller's stream. Nothing here allocates device memory or
// synchronizes.
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#include "fa.h"
#include "fa_kernels.h"

namespace {

constexpr int64_t kI32Max = 2147483647;

size_t elem_bytes(fa_dtype dt) { return dt == FA_BF16 ? 2 : 4; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// [a, a+na) and [b, b+nb) overlap.
bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

fa_status check_problem(int B, int H, int N, int d, fa_dtype dtype, float scale, fa_mask mask,
                        int window) {
  if (B < 1 || H < 1 || N < 1) return FA_ERR_SHAPE;
  if ((int64_t)B * H > kI32Max) return FA_ERR_SHAPE;
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

int tuning_cfg(const char* name) {
  const char* s = getenv(name);
  return s ? atoi(s) : 0;
}

// Sign handling of the scale for the bf16 kernels: the kernel's exp2
// argument needs a positive factor, so a negative scale negates Q (exact in
// bf16) and a zero (or underflowing) scale zeroes Q, which makes every logit
// exactly 0 as scale = 0 does.
void bf16_scale(float scale, fa::FwdArgs& a) {
  const double LOG2E = 1.4426950408889634;
  double s = fabs((double)scale);
  a.q_and = 0xFFFFFFFFu;
  a.q_xor = scale < 0 ? 0x80008000u : 0u;
  float c = (float)(s * LOG2E);
  if (!(c >= 1.17549435e-38f)) {  // zero, or too small for a normal float factor
    a.q_and = 0u;
    a.q_xor = 0u;
    s = 1.0;
    c = (float)LOG2E;
  }
  a.scale_abs = (float)s;
  a.scale_log2 = c;
}

}  // namespace

extern "C" {

const char* fa_status_string(fa_status s) {
  switch (s) {
    case FA_OK: return "FA_OK: success";
    case FA_ERR_NULL: return "FA_ERR_NULL: a required pointer is NULL";
    case FA_ERR_SHAPE: return "FA_ERR_SHAPE: B, H, N must be >= 1 and within the size limits";
    case FA_ERR_DTYPE: return "FA_ERR_DTYPE: unknown dtype";
    case FA_ERR_HEADDIM: return "FA_ERR_HEADDIM: head dimension not supported for this dtype";
    case FA_ERR_MASK: return "FA_ERR_MASK: unknown mask or negative local window";
    case FA_ERR_SCALE: return "FA_ERR_SCALE: scale must be finite";
    case FA_ERR_ALIGN: return "FA_ERR_ALIGN: pointers must be 16-byte aligned";
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE: workspace missing or too small";
    case FA_ERR_LAUNCH: return "FA_ERR_LAUNCH: kernel launch failed";
    case FA_ERR_ALIAS: return "FA_ERR_ALIAS: an output overlaps an input";
  }
  return "unknown fa_status";
}

fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                 int N, int d, fa_dtype dtype, float scale, fa_mask mask, int window,
                 void* stream) {
  fa_status st = check_problem(B, H, N, d, dtype, scale, mask, window);
  if (st != FA_OK) return st;
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return FA_ERR_ALIGN;
  const size_t tb = (size_t)B * H * N * d * elem_bytes(dtype);
  const size_t lb = (size_t)B * H * N * sizeof(float);
  if (overlap(o, tb, q, tb) || overlap(o, tb, k, tb) || overlap(o, tb, v, tb) ||
      overlap(lse, lb, q, tb) || overlap(lse, lb, k, tb) || overlap(lse, lb, v, tb) ||
      overlap(o, tb, lse, lb))
    return FA_ERR_ALIAS;
  if (mask != FA_MASK_LOCAL) window = 0;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if (dtype == FA_BF16) {
    fa::FwdArgs a;
    a.q = (const bf16*)q;
    a.k = (const bf16*)k;
    a.v = (const bf16*)v;
    a.o = (bf16*)o;
    a.lse = lse;
    a.BH = B * H;
    a.N = N;
    a.n_qtiles = 0;
    a.window = window;
    bf16_scale(scale, a);
    e = fa::launch_fwd_bf16(a, d, (int)mask, tuning_cfg("FA_FWD_CFG"), s);
  } else {
    fa::FwdF32Args a;
    a.q = (const float*)q;
    a.k = (const float*)k;
    a.v = (const float*)v;
    a.o = (float*)o;
    a.lse = lse;
    a.BH = B * H;
    a.N = N;
    a.d = d;
    a.window = window;
    a.scale = scale;
    e = fa::launch_fwd_f32(a, (int)mask, s);
  }
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

// Standard (unfused) attention: workspace = S (float32, rows padded to 4)
// then P (bf16, rows padded to 8), each region 256-byte aligned.
static bool std_layout(int B, int H, int N, size_t& s_bytes, size_t& total) {
  const size_t bh = (size_t)B * H, lds = ((size_t)N + 3) & ~(size_t)3, ldp = ((size_t)N + 7) & ~(size_t)7;
  const long double need = (long double)bh * N * (lds * 4.0L + ldp * 2.0L) + 512.0L;
  if (need > 1.0e15L) return false;  // far beyond any device memory
  s_bytes = (bh * N * lds * 4 + 255) & ~(size_t)255;
  total = s_bytes + ((bh * N * ldp * 2 + 255) & ~(size_t)255);
  return true;
}

size_t fa_fwd_standard_workspace_bytes(int B, int H, int N, int d, fa_dtype dtype) {
  if (dtype != FA_BF16) return 0;
  if (check_problem(B, H, N, d, dtype, 1.0f, FA_MASK_NONE, 0) != FA_OK) return 0;
  size_t sb, total;
  if (!std_layout(B, H, N, sb, total)) return 0;
  return total;
}

fa_status fa_fwd_standard(const void* q, const void* k, const void* v, void* o, float* lse,
                          void* workspace, size_t workspace_bytes, int B, int H, int N, int d,
                          fa_dtype dtype, float scale, fa_mask mask, int window, void* stream) {
  fa_status st = check_problem(B, H, N, d, dtype, scale, mask, window);
  if (st != FA_OK) return st;
  if (dtype != FA_BF16) return FA_ERR_DTYPE;
  if ((int64_t)B * H * N > kI32Max) return FA_ERR_SHAPE;  // one softmax workgroup per row
  size_t sb, total;
  if (!std_layout(B, H, N, sb, total)) return FA_ERR_SHAPE;
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  if (!workspace || workspace_bytes < total) return FA_ERR_WORKSPACE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse) ||
      !aligned16(workspace))
    return FA_ERR_ALIGN;
  const size_t tb = (size_t)B * H * N * d * 2;
  const size_t lb = (size_t)B * H * N * sizeof(float);
  const void* ins[3] = {q, k, v};
  for (const void* in : ins)
    if (overlap(o, tb, in, tb) || overlap(lse, lb, in, tb) || overlap(workspace, total, in, tb))
      return FA_ERR_ALIAS;
  if (overlap(o, tb, lse, lb) || overlap(workspace, total, o, tb) || overlap(workspace, total, lse, lb))
    return FA_ERR_ALIAS;
  fa::StdArgs a;
  a.q = (const bf16*)q;
  a.k = (const bf16*)k;
  a.v = (const bf16*)v;
  a.o = (bf16*)o;
  a.lse = lse;
  a.s = (float*)workspace;
  a.p = (bf16*)((char*)workspace + sb);
  a.BH = B * H;
  a.N = N;
  a.lds = (N + 3) & ~3;
  a.ldp = (N + 7) & ~7;
  a.window = mask == FA_MASK_LOCAL ? window : 0;
  a.scale = scale;
  const hipError_t e = fa::launch_std_bf16(a, d, (int)mask, (hipStream_t)stream);
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

size_t fa_fwd_keymajor_workspace_bytes(int B, int H, int N, int d, fa_dtype dtype) {
  if (dtype != FA_BF16) return 0;
  if (check_problem(B, H, N, d, dtype, 1.0f, FA_MASK_NONE, 0) != FA_OK) return 0;
  return fa::km_state_bytes(B * H, N, d);
}

fa_status fa_fwd_keymajor(const void* q, const void* k, const void* v, void* o, float* lse,
                          void* workspace, size_t workspace_bytes, int B, int H, int N, int d,
                          fa_dtype dtype, float scale, fa_mask mask, int window, int block_keys,
                          void* stream) {
  fa_status st = check_problem(B, H, N, d, dtype, scale, mask, window);
  if (st != FA_OK) return st;
  if (dtype != FA_BF16) return FA_ERR_DTYPE;
  const bool bc_ok = block_keys == 32 || block_keys == 64 || block_keys == 128 ||
                     (block_keys == 256 && d == 64);
  if (!bc_ok) return FA_ERR_SHAPE;
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  const size_t total = fa::km_state_bytes(B * H, N, d);
  if (!workspace || workspace_bytes < total) return FA_ERR_WORKSPACE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse) ||
      !aligned16(workspace))
    return FA_ERR_ALIGN;
  const size_t tb = (size_t)B * H * N * d * 2;
  const size_t lb = (size_t)B * H * N * sizeof(float);
  const void* ins[3] = {q, k, v};
  for (const void* in : ins)
    if (overlap(o, tb, in, tb) || overlap(lse, lb, in, tb) || overlap(workspace, total, in, tb))
      return FA_ERR_ALIAS;
  if (overlap(o, tb, lse, lb) || overlap(workspace, total, o, tb) || overlap(workspace, total, lse, lb))
    return FA_ERR_ALIAS;
  fa::FwdArgs f;
  bf16_scale(scale, f);
  fa::KmArgs a;
  a.q = (const bf16*)q;
  a.k = (const bf16*)k;
  a.v = (const bf16*)v;
  a.o = (bf16*)o;
  a.lse = lse;
  a.state = (float*)workspace;
  a.BH = B * H;
  a.N = N;
  a.n_qtiles = 0;
  a.window = mask == FA_MASK_LOCAL ? window : 0;
  a.scale_log2 = f.scale_log2;
  a.scale_abs = f.scale_abs;
  a.q_and = f.q_and;
  a.q_xor = f.q_xor;
  const hipError_t e = fa::launch_fwd_keymajor(a, d, block_keys, (int)mask, (hipStream_t)stream);
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // extern "C"
