// Internal kernel launch interface between the C ABI layer and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include "fa_common.h"

namespace fa {

struct FwdArgs {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  bf16* o;
  float* lse;
  int BH;
  int N;
  int n_qtiles;       // filled by the launcher
  int window;
  float scale_log2;   // |scale| * log2(e), > 0
  float scale_abs;    // |scale| (0 becomes 1 with Q zeroed)
  unsigned q_and;     // Q bits are (q & q_and) ^ q_xor: identity, negate or zero
  unsigned q_xor;
};

struct FwdF32Args {
  const float* q;
  const float* k;
  const float* v;
  float* o;
  float* lse;
  int BH;
  int N;
  int d;
  int window;
  float scale;
};

// Standard (unfused) attention: S, P and the LSE through device memory.
struct StdArgs {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  bf16* o;
  float* lse;
  float* s;    // workspace: [BH][N][lds] float32 scaled, masked logits
  bf16* p;     // workspace: [BH][N][ldp] bf16 probabilities (zero padded)
  int BH;
  int N;
  int lds;     // N rounded up to 4
  int ldp;     // N rounded up to 8
  int window;
  float scale;  // signed scale as given
  // standard backward only
  const bf16* dout;   // dO
  bf16* ds;           // workspace: [BH][N][ldp] bf16 dS (the P region's layout)
  bf16* dq;
  bf16* dk;
  bf16* dv;
};

// Key-major forward: per key block one launch updating a running state.
struct KmArgs {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  bf16* o;
  float* lse;
  float* state;       // workspace: km_state_bytes(BH, N, d)
  int BH;
  int N;
  int n_qtiles;       // filled by the launcher
  int window;
  float scale_log2;   // as FwdArgs
  float scale_abs;
  unsigned q_and;
  unsigned q_xor;
};
size_t km_state_bytes(int BH, int N, int d);
hipError_t launch_fwd_keymajor(const KmArgs& a, int d, int bc, int mask, hipStream_t stream);

// cfg selects a tile configuration (0 = default); tuning only.
hipError_t launch_fwd_bf16(const FwdArgs& a, int d, int mask, int cfg, hipStream_t stream);
hipError_t launch_std_bf16(const StdArgs& a, int d, int mask, hipStream_t stream);
// standard backward: dP = dO V^T into a.s, dV = P^T dO, D and dS into a.ds,
// dQ = scale dS K, dK = scale dS^T Q (P read from a.p)
hipError_t launch_std_bwd_bf16(const StdArgs& a, int d, hipStream_t stream);
hipError_t launch_fwd_f32(const FwdF32Args& a, int mask, hipStream_t stream);

}  // namespace fa

namespace fa {

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* delta;    // workspace: [BH][N] float32, D_i = <dO_i, O_i>
  int BH;
  int N;
  int d;
  int window;
  float scale;       // signed scale as given
  float scale_log2;  // |scale| * log2(e) (bf16 path)
  float scale_abs;
  unsigned q_and;    // bf16 path: Q bits are (q & q_and) ^ q_xor
  unsigned q_xor;
};

// Workspace layout shared by fa_bwd_workspace_bytes and the launcher.
size_t bwd_workspace_bytes(int BH, int N);

// cfg selects an alternative workgroup size (0 = default); tuning only.
hipError_t launch_bwd(const BwdArgs& a, int bf16, int mask, int cfg, hipStream_t stream);

}  // namespace fa
