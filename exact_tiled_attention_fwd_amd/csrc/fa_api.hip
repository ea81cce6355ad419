// C ABI entry points (include/fa.h): argument validation, kernel selection
// and launch on the caller's stream. Nothing here allocates device memory or
// synchronizes.
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#include "fa.h"
#include "fa_host.h"
#include "fa_kernels.h"

using namespace fa::host;

namespace {

// Kernel choice of the forward: 0 is the measured default; other values
// select the alternative shapes kept for timing comparisons (fa_tuning.h).
constexpr int kFwdCfgMax = 9;

void set_scale(const ScaleFold& f, fa::FwdArgs& a) {
  a.scale_abs = f.scale_abs;
  a.scale_log2 = f.scale_log2;
  a.q_and = f.q_and;
  a.q_xor = f.q_xor;
}

fa_status fwd_impl(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                   int N, int d, fa_dtype dtype, float scale, fa_mask mask, int window, int cfg,
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
    a.window = kernel_window(mask, window, N);
    set_scale(fold_scale(scale), a);
    e = fa::launch_fwd_bf16(a, d, (int)mask, cfg, s);
  } else {
    if (cfg != 0) return FA_ERR_CONFIG;
    fa::FwdF32Args a;
    a.q = (const float*)q;
    a.k = (const float*)k;
    a.v = (const float*)v;
    a.o = (float*)o;
    a.lse = lse;
    a.BH = B * H;
    a.N = N;
    a.d = d;
    a.window = kernel_window(mask, window, N);
    a.scale = scale;
    e = fa::launch_fwd_f32(a, (int)mask, s);
  }
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
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
    case FA_ERR_CONFIG: return "FA_ERR_CONFIG: unknown kernel configuration";
  }
  return "unknown fa_status";
}

fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                 int N, int d, fa_dtype dtype, float scale, fa_mask mask, int window,
                 void* stream) {
  return fwd_impl(q, k, v, o, lse, B, H, N, d, dtype, scale, mask, window, 0, stream);
}

fa_status fa_fwd_tuned(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                       int H, int N, int d, fa_dtype dtype, float scale, fa_mask mask, int window,
                       int cfg, void* stream) {
  if (cfg < 0 || cfg > kFwdCfgMax) return FA_ERR_CONFIG;
  return fwd_impl(q, k, v, o, lse, B, H, N, d, dtype, scale, mask, window, cfg, stream);
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
  fa::StdArgs a = {};
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
  a.window = kernel_window(mask, window, N);
  a.scale = scale;
  const hipError_t e = fa::launch_std_bf16(a, d, (int)mask, (hipStream_t)stream);
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

size_t fa_bwd_standard_workspace_bytes(int B, int H, int N, int d, fa_dtype dtype) {
  return fa_fwd_standard_workspace_bytes(B, H, N, d, dtype);
}

fa_status fa_bwd_standard(const void* q, const void* k, const void* v, const void* dout,
                          const void* fwd_workspace, size_t fwd_workspace_bytes, void* dq,
                          void* dk, void* dv, void* workspace, size_t workspace_bytes, int B,
                          int H, int N, int d, fa_dtype dtype, float scale, void* stream) {
  fa_status st = check_problem(B, H, N, d, dtype, scale, FA_MASK_NONE, 0);
  if (st != FA_OK) return st;
  if (dtype != FA_BF16) return FA_ERR_DTYPE;
  if ((int64_t)B * H * N > kI32Max) return FA_ERR_SHAPE;  // one row workgroup per query row
  size_t sb, total;
  if (!std_layout(B, H, N, sb, total)) return FA_ERR_SHAPE;
  if (!q || !k || !v || !dout || !dq || !dk || !dv) return FA_ERR_NULL;
  if (!fwd_workspace || fwd_workspace_bytes < total || !workspace || workspace_bytes < total)
    return FA_ERR_WORKSPACE;
  const void* all[] = {q, k, v, dout, fwd_workspace, dq, dk, dv, workspace};
  for (const void* p : all)
    if (!aligned16(p)) return FA_ERR_ALIGN;
  const size_t tb = (size_t)B * H * N * d * 2;
  const void* ins[] = {q, k, v, dout};
  void* outs[] = {dq, dk, dv};
  for (void* o : outs) {
    for (const void* in : ins)
      if (overlap(o, tb, in, tb)) return FA_ERR_ALIAS;
    if (overlap(o, tb, fwd_workspace, total) || overlap(o, tb, workspace, total)) return FA_ERR_ALIAS;
  }
  if (overlap(dq, tb, dk, tb) || overlap(dq, tb, dv, tb) || overlap(dk, tb, dv, tb))
    return FA_ERR_ALIAS;
  for (const void* in : ins)
    if (overlap(workspace, total, in, tb)) return FA_ERR_ALIAS;
  if (overlap(workspace, total, fwd_workspace, total)) return FA_ERR_ALIAS;
  fa::StdArgs a;
  a.q = (const bf16*)q;
  a.k = (const bf16*)k;
  a.v = (const bf16*)v;
  a.dout = (const bf16*)dout;
  a.o = nullptr;
  a.lse = nullptr;
  a.p = (bf16*)((char*)fwd_workspace + sb);  // the forward's P, read only
  a.s = (float*)workspace;                   // dP
  a.ds = (bf16*)((char*)workspace + sb);     // dS
  a.dq = (bf16*)dq;
  a.dk = (bf16*)dk;
  a.dv = (bf16*)dv;
  a.BH = B * H;
  a.N = N;
  a.lds = (N + 3) & ~3;
  a.ldp = (N + 7) & ~7;
  a.window = 0;
  a.scale = scale;
  const hipError_t e = fa::launch_std_bwd_bf16(a, d, (hipStream_t)stream);
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
  const ScaleFold f = fold_scale(scale);
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
  a.window = kernel_window(mask, window, N);
  a.scale_log2 = f.scale_log2;
  a.scale_abs = f.scale_abs;
  a.q_and = f.q_and;
  a.q_xor = f.q_xor;
  const hipError_t e = fa::launch_fwd_keymajor(a, d, block_keys, (int)mask, (hipStream_t)stream);
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // extern "C"
