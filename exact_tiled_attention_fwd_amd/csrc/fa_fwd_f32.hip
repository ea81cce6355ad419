// Forward exact attention in float32 (storage and arithmetic), 1 <= d <= 128.
//
// Same method as the bf16 kernel — the incremental softmax merge of the
// Hinglish notes' "Derivation: Incremental Softmax" over a query-major tile
// schedule — but on the vector ALUs: float32 is the precision-reference
// path for small head dimensions (the TensorViz toy run is 6 x 4), where
// matrix cores buy nothing. One lane owns one query row; a 32-key K/V tile
// sits in LDS and every lane reads the same key row (an LDS broadcast).
#include "fa_common.h"
#include "fa_kernels.h"

namespace fa {

constexpr int F32_BR = 128;  // query rows per workgroup (one per thread)
constexpr int F32_BC = 32;   // keys per LDS tile

template <int DP, int MASK>
__global__ __launch_bounds__(F32_BR) void fwd_f32_kernel(FwdF32Args a) {
  __shared__ float sK[F32_BC][DP];
  __shared__ float sV[F32_BC][DP];
  const int N = a.N, d = a.d;
  const int n_qt = (N + F32_BR - 1) / F32_BR;
  const int bh = blockIdx.x / n_qt;
  const int q0 = (blockIdx.x - bh * n_qt) * F32_BR;
  const int qi = q0 + (int)threadIdx.x;
  const size_t base = (size_t)bh * N * d;
  const float* __restrict__ Q = a.q + base;
  const float* __restrict__ K = a.k + base;
  const float* __restrict__ V = a.v + base;

  float q[DP], acc[DP];
#pragma unroll
  for (int c = 0; c < DP; ++c) {
    q[c] = (qi < N && c < d) ? Q[(size_t)qi * d + c] : 0.f;
    acc[c] = 0.f;
  }
  float m = -INFINITY, l = 0.f;

  int k_lo, k_hi;
  key_range<MASK>(q0, q0 + F32_BR, N, a.window, k_lo, k_hi);
  for (int k0 = (k_lo / F32_BC) * F32_BC; k0 < k_hi; k0 += F32_BC) {
    for (int idx = threadIdx.x; idx < F32_BC * DP; idx += F32_BR) {
      const int r = idx / DP, c = idx % DP, key = k0 + r;
      const bool ok = key < N && c < d;
      sK[r][c] = ok ? K[(size_t)key * d + c] : 0.f;
      sV[r][c] = ok ? V[(size_t)key * d + c] : 0.f;
    }
    __syncthreads();
    float z[F32_BC];
    float tmax = -INFINITY;
#pragma unroll
    for (int j = 0; j < F32_BC; ++j) {
      float s = 0.f;
#pragma unroll
      for (int c = 0; c < DP; ++c) s = fmaf(q[c], sK[j][c], s);
      const int key = k0 + j;
      z[j] = (key < N && allowed<MASK>(qi, key, a.window)) ? a.scale * s : -INFINITY;
      tmax = fmaxf(tmax, z[j]);
    }
    const float m_new = fmaxf(m, tmax);
    if (m_new != -INFINITY) {
      const float alpha = (m == -INFINITY) ? 0.f : expf(m - m_new);
      float ps = 0.f;
#pragma unroll
      for (int c = 0; c < DP; ++c) acc[c] *= alpha;
#pragma unroll
      for (int j = 0; j < F32_BC; ++j) {
        const float p = (z[j] == -INFINITY) ? 0.f : expf(z[j] - m_new);
        ps += p;
#pragma unroll
        for (int c = 0; c < DP; ++c) acc[c] = fmaf(p, sV[j][c], acc[c]);
      }
      l = alpha * l + ps;
      m = m_new;
    }
    __syncthreads();
  }
  if (qi < N) {
    const float inv = 1.f / l;
    for (int c = 0; c < d && c < DP; ++c) a.o[base + (size_t)qi * d + c] = acc[c] * inv;
    a.lse[(size_t)bh * N + qi] = m + logf(l);
  }
}

template <int DP>
static hipError_t launch_f32_dp(const FwdF32Args& a, int mask, hipStream_t stream) {
  const int n_qt = (a.N + F32_BR - 1) / F32_BR;
  dim3 grid((unsigned)(n_qt * a.BH)), block(F32_BR);
  switch (mask) {
    case MASK_CAUSAL: hipLaunchKernelGGL((fwd_f32_kernel<DP, MASK_CAUSAL>), grid, block, 0, stream, a); break;
    case MASK_LOCAL: hipLaunchKernelGGL((fwd_f32_kernel<DP, MASK_LOCAL>), grid, block, 0, stream, a); break;
    default: hipLaunchKernelGGL((fwd_f32_kernel<DP, MASK_NONE>), grid, block, 0, stream, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_fwd_f32(const FwdF32Args& a, int mask, hipStream_t stream) {
  if (a.d <= 8) return launch_f32_dp<8>(a, mask, stream);
  if (a.d <= 32) return launch_f32_dp<32>(a, mask, stream);
  if (a.d <= 64) return launch_f32_dp<64>(a, mask, stream);
  return launch_f32_dp<128>(a, mask, stream);
}

}  // namespace fa
