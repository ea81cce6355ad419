// C ABI of the backward pass (include/fa.h): validation and workspace layout.
#include <math.h>
#include <stdint.h>

#include "fa.h"
#include "fa_kernels.h"

namespace fa {

static size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

// The workspace holds D_i = <dO_i, O_i> for every row, float32 [BH][N].
size_t bwd_workspace_bytes(int BH, int N) { return round256((size_t)BH * N * sizeof(float)); }

}  // namespace fa

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

fa_status check_problem(int B, int H, int N, int d, fa_dtype dtype) {
  if (B < 1 || H < 1 || N < 1) return FA_ERR_SHAPE;
  if ((int64_t)B * H > 2147483647) return FA_ERR_SHAPE;
  if (dtype != FA_BF16 && dtype != FA_F32) return FA_ERR_DTYPE;
  if (dtype == FA_BF16 && d != 64 && d != 128) return FA_ERR_HEADDIM;
  if (dtype == FA_F32 && (d < 1 || d > 128)) return FA_ERR_HEADDIM;
  if ((int64_t)N * d > 2147483647) return FA_ERR_SHAPE;
  if (((int64_t)N + 31) / 32 * ((int64_t)B * H) > 2147483647) return FA_ERR_SHAPE;
  return FA_OK;
}

}  // namespace

extern "C" {

size_t fa_bwd_workspace_bytes(int B, int H, int N, int d, fa_dtype dtype) {
  if (check_problem(B, H, N, d, dtype) != FA_OK) return 0;
  return fa::bwd_workspace_bytes(B * H, N);
}

fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                 const float* lse, void* dq, void* dk, void* dv, void* workspace,
                 size_t workspace_bytes, int B, int H, int N, int d, fa_dtype dtype, float scale,
                 fa_mask mask, int window, void* stream) {
  fa_status st = check_problem(B, H, N, d, dtype);
  if (st != FA_OK) return st;
  if (mask != FA_MASK_NONE && mask != FA_MASK_CAUSAL && mask != FA_MASK_LOCAL) return FA_ERR_MASK;
  if (mask == FA_MASK_LOCAL && window < 0) return FA_ERR_MASK;
  if (!isfinite(scale)) return FA_ERR_SCALE;
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return FA_ERR_NULL;
  const void* ptrs[] = {q, k, v, o, dout, lse, dq, dk, dv, workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return FA_ERR_ALIGN;
  const size_t need = fa::bwd_workspace_bytes(B * H, N);
  if (!workspace || workspace_bytes < need) return FA_ERR_WORKSPACE;
  const size_t tb = (size_t)B * H * N * d * (dtype == FA_BF16 ? 2 : 4);
  const size_t lb = (size_t)B * H * N * sizeof(float);
  const void* ins[] = {q, k, v, o, dout};
  void* outs[] = {dq, dk, dv};
  for (void* out : outs) {
    for (const void* in : ins)
      if (overlap(out, tb, in, tb)) return FA_ERR_ALIAS;
    if (overlap(out, tb, lse, lb) || overlap(out, tb, workspace, need)) return FA_ERR_ALIAS;
  }
  if (overlap(dq, tb, dk, tb) || overlap(dq, tb, dv, tb) || overlap(dk, tb, dv, tb))
    return FA_ERR_ALIAS;
  for (const void* in : ins)
    if (overlap(workspace, need, in, tb)) return FA_ERR_ALIAS;
  if (overlap(workspace, need, lse, lb)) return FA_ERR_ALIAS;

  fa::BwdArgs a;
  a.q = q; a.k = k; a.v = v; a.o = o; a.dout = dout; a.lse = lse;
  a.dq = dq; a.dk = dk; a.dv = dv;
  a.delta = (float*)workspace;
  a.BH = B * H;
  a.N = N;
  a.d = d;
  a.window = mask == FA_MASK_LOCAL ? window : 0;
  a.scale = scale;
  {
    const double LOG2E = 1.4426950408889634;
    double s = fabs((double)scale);
    a.q_and = 0xFFFFFFFFu;
    a.q_xor = scale < 0 ? 0x80008000u : 0u;
    float c = (float)(s * LOG2E);
    if (!(c >= 1.17549435e-38f)) {
      a.q_and = 0u;
      a.q_xor = 0u;
      s = 1.0;
      c = (float)LOG2E;
    }
    a.scale_abs = (float)s;
    a.scale_log2 = c;
  }
  hipError_t e = fa::launch_bwd(a, dtype == FA_BF16, (int)mask, (hipStream_t)stream);
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // extern "C"
