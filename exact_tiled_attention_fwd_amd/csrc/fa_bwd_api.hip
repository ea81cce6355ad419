// C ABI of the backward pass (include/fa.h): validation and workspace layout.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "fa.h"
#include "fa_host.h"
#include "fa_kernels.h"

namespace fa {

static size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

// The workspace holds D_i = <dO_i, O_i> for every row, float32 [BH][N].
size_t bwd_workspace_bytes(int BH, int N) { return round256((size_t)BH * N * sizeof(float)); }

}  // namespace fa

using namespace fa::host;

namespace {

// Kernel choice of the backward: 0 is the measured default, 2 the other
// workgroup size (fa_tuning.h).
bool bwd_cfg_ok(int cfg) { return cfg == 0 || cfg == 2; }

// Validation of everything but the workspace, and the kernel arguments.
fa_status bwd_prepare(const void* q, const void* k, const void* v, const void* o, const void* dout,
                      const float* lse, void* dq, void* dk, void* dv, const void* workspace,
                      size_t ws_bytes, int B, int H, int N, int d, fa_dtype dtype, float scale,
                      fa_mask mask, int window, fa::BwdArgs& a) {
  fa_status st = check_problem(B, H, N, d, dtype, scale, mask, window);
  if (st != FA_OK) return st;
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return FA_ERR_NULL;
  const void* ptrs[] = {q, k, v, o, dout, lse, dq, dk, dv, workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return FA_ERR_ALIGN;
  const size_t tb = (size_t)B * H * N * d * elem_bytes(dtype);
  const size_t lb = (size_t)B * H * N * sizeof(float);
  const void* ins[] = {q, k, v, o, dout};
  void* outs[] = {dq, dk, dv};
  for (void* out : outs) {
    for (const void* in : ins)
      if (overlap(out, tb, in, tb)) return FA_ERR_ALIAS;
    if (overlap(out, tb, lse, lb)) return FA_ERR_ALIAS;
    if (workspace && overlap(out, tb, workspace, ws_bytes)) return FA_ERR_ALIAS;
  }
  if (overlap(dq, tb, dk, tb) || overlap(dq, tb, dv, tb) || overlap(dk, tb, dv, tb))
    return FA_ERR_ALIAS;
  if (workspace) {
    for (const void* in : ins)
      if (overlap(workspace, ws_bytes, in, tb)) return FA_ERR_ALIAS;
    if (overlap(workspace, ws_bytes, lse, lb)) return FA_ERR_ALIAS;
  }
  a.q = q; a.k = k; a.v = v; a.o = o; a.dout = dout; a.lse = lse;
  a.dq = dq; a.dk = dk; a.dv = dv;
  a.delta = (float*)workspace;
  a.BH = B * H;
  a.N = N;
  a.d = d;
  a.window = kernel_window(mask, window, N);
  a.scale = scale;
  const ScaleFold f = fold_scale(scale);
  a.scale_abs = f.scale_abs;
  a.scale_log2 = f.scale_log2;
  a.q_and = f.q_and;
  a.q_xor = f.q_xor;
  return FA_OK;
}

fa_status bwd_impl(const void* q, const void* k, const void* v, const void* o, const void* dout,
                   const float* lse, void* dq, void* dk, void* dv, void* workspace,
                   size_t workspace_bytes, int B, int H, int N, int d, fa_dtype dtype, float scale,
                   fa_mask mask, int window, int cfg, void* stream) {
  fa_status st = check_problem(B, H, N, d, dtype, scale, mask, window);
  if (st != FA_OK) return st;
  const size_t need = fa::bwd_workspace_bytes(B * H, N);
  fa::BwdArgs a;
  st = bwd_prepare(q, k, v, o, dout, lse, dq, dk, dv, workspace, need, B, H, N, d, dtype, scale,
                   mask, window, a);
  if (st != FA_OK) return st;
  if (!workspace || workspace_bytes < need) return FA_ERR_WORKSPACE;
  const hipError_t e = fa::launch_bwd(a, dtype == FA_BF16, (int)mask, cfg, (hipStream_t)stream);
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

// ---- allocation-free variant: D in a static device array
// Every GPU the library runs on holds one copy of `scratch` (64 MiB) until the
// process ends. In host code `scratch` names a host-side stand-in, never the
// device memory: host code uses only the per-device address that
// hipGetSymbolAddress returns, taken once per device with that device current.
constexpr size_t kNoallocRows = FA_BWD_NOALLOC_MAX_ROWS;
static __device__ __align__(256) float scratch[kNoallocRows];

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// Device address of `scratch` on the current device.
fa_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FA_ERR_LAUNCH;
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = p;
  });
  if (g_scratch_err[dev] != hipSuccess || g_scratch_ptr[dev] == nullptr) return FA_ERR_LAUNCH;
  *out = g_scratch_ptr[dev];
  return FA_OK;
}

}  // namespace

extern "C" {

fa_status fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                         const void* dout, const float* lse, void* dq, void* dk, void* dv, int B,
                         int H, int N, int d, fa_dtype dtype, float scale, fa_mask mask,
                         int window, void* stream) {
  fa_status st = check_problem(B, H, N, d, dtype, scale, mask, window);
  if (st != FA_OK) return st;
  if ((size_t)B * H * N > kNoallocRows) return FA_ERR_WORKSPACE;
  fa::BwdArgs a;
  st = bwd_prepare(q, k, v, o, dout, lse, dq, dk, dv, nullptr, 0, B, H, N, d, dtype, scale, mask,
                   window, a);
  if (st != FA_OK) return st;
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != FA_OK) return st;
  // D is written for every row (by the dQ kernel, or the float32 pre-pass)
  // before anything reads it, so the array needs no clearing between calls.
  a.delta = (float*)ws;
  const hipError_t e = fa::launch_bwd(a, dtype == FA_BF16, (int)mask, 0, (hipStream_t)stream);
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

size_t fa_bwd_workspace_bytes(int B, int H, int N, int d, fa_dtype dtype) {
  if (check_problem(B, H, N, d, dtype, 1.0f, FA_MASK_NONE, 0) != FA_OK) return 0;
  return fa::bwd_workspace_bytes(B * H, N);
}

fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                 const float* lse, void* dq, void* dk, void* dv, void* workspace,
                 size_t workspace_bytes, int B, int H, int N, int d, fa_dtype dtype, float scale,
                 fa_mask mask, int window, void* stream) {
  return bwd_impl(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, B, H, N, d,
                  dtype, scale, mask, window, 0, stream);
}

fa_status fa_bwd_tuned(const void* q, const void* k, const void* v, const void* o,
                       const void* dout, const float* lse, void* dq, void* dk, void* dv,
                       void* workspace, size_t workspace_bytes, int B, int H, int N, int d,
                       fa_dtype dtype, float scale, fa_mask mask, int window, int cfg,
                       void* stream) {
  if (!bwd_cfg_ok(cfg) || (cfg != 0 && dtype != FA_BF16)) return FA_ERR_CONFIG;
  return bwd_impl(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, B, H, N, d,
                  dtype, scale, mask, window, cfg, stream);
}

}  // extern "C"
