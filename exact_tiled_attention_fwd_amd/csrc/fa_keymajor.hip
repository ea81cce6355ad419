// Key-major forward (the loop order of the FlashAttention paper's
// Algorithm 1, LIT-074, as quoted in "What the tiling is actually
// constrained by": K and V split into T_c = ceil(N / B_c) blocks in the
// outer loop, Q blocks in the inner one; the TensorViz card's fidelity note
// contrasts it with the query-major loop of the fused kernel). For every key
// block j one launch updates the running state (m, l, unnormalized O) of
// every query row with the incremental-softmax rule of the Hinglish notes'
// "Derivation: Incremental Softmax", reading the state from device memory
// and writing it back. The state traffic, T_c * N * (d + 2) * 4 bytes each
// way, is what makes the HBM accesses of this order scale as N^2 d / B_c,
// i.e. Theta(N^2 d^2 / M) with M = 4 B_c d (the paper's Theorem 2).
//
// State layout (workspace): per workgroup of 256 query rows and per wave of
// 32 rows, the wave's accumulator registers as [DT*16/4][64 lanes] float4
// (one coalesced 1 KiB access per group of four registers), then m and l as
// [64 lanes] floats each, then the sum of the bf16-rounded weights (the
// output's normalizer, as in the query-major kernel) as [64 lanes] floats.
// Lanes l and l+32 share query row l mod 32: m is the same in both, the two
// sums hold each half's part.
#include "fa_common.h"
#include "fa_kernels.h"
#include "fa_tile_ops.h"

namespace fa {

template <int D>
__device__ __forceinline__ size_t km_wave_floats() { return (size_t)64 * (D / 32 * 16 + 3); }

// state pointer of wave wv of workgroup w
template <int D>
__device__ __forceinline__ float* km_state(float* ws, int w, int wv) {
  return ws + ((size_t)w * 8 + wv) * km_wave_floats<D>();
}

// m = -inf, l = 0, rounded-weight sum = 0, acc = 0 for every row
template <int D>
__global__ __launch_bounds__(512) void km_init_kernel(float* ws, size_t n_wg) {
  constexpr int NACC = D / 32 * 16;
  const size_t w = blockIdx.x;
  if (w >= n_wg) return;
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float* st = km_state<D>(ws, (int)w, wv);
  for (int r = 0; r < NACC; ++r) st[(size_t)r * 64 + lane] = 0.f;
  st[(size_t)NACC * 64 + lane] = -INFINITY;
  st[(size_t)(NACC + 1) * 64 + lane] = 0.f;
  st[(size_t)(NACC + 2) * 64 + lane] = 0.f;
}

// One key block j of BC keys: workgroup = 256 query rows (8 waves x 32),
// K_j and V_j in LDS, scores transposed (S^T = K Q^T) and the P V product as
// in the query-major kernel, the state loaded and stored around them.
template <int D, int BC, int MASK>
__global__ __launch_bounds__(512, 2) void km_step_kernel(KmArgs a, int j) {
  constexpr int KC = D / 16, DT = D / 32, KB = BC / 32, ROWB = D * 2, TILEB = BC * ROWB;
  constexpr int CPR = D / 8, NACC = DT * 16;
  constexpr int CPT = (BC * CPR + 511) / 512;
  __shared__ __attribute__((aligned(16))) char smem[2 * TILEB];  // K_j, V_j
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, l32 = lane & 31, h = lane >> 5;
  const int N = a.N;
  const int w = blockIdx.x;
  const int bh = w / a.n_qtiles, qt = w - bh * a.n_qtiles;
  const int q0 = qt * 256, qw0 = q0 + wv * 32, qi = qw0 + l32;
  const int k0 = j * BC;

  // the workgroup (and each wave) only works where some pair is allowed
  int k_lo, k_hi, wk_lo, wk_hi;
  key_range<MASK>(q0, q0 + 256, N, a.window, k_lo, k_hi);
  if (!(k0 < k_hi && k0 + BC > k_lo)) return;
  key_range<MASK>(qw0, qw0 + 32, N, a.window, wk_lo, wk_hi);
  const bool active = qw0 < N && k0 < wk_hi && k0 + BC > wk_lo;

  const size_t base = (size_t)bh * N * D;
  char* sK = smem;
  char* sV = smem + TILEB;
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int slot = (wv * CPT + i) * 64;
    if (slot < BC * CPR) {
      const int p = slot + lane;
      const int row = p / CPR;
      int gr = k0 + row;
      gr = gr < N ? gr : N - 1;  // keys past N are masked
      lds_dma16(a.k + base + (size_t)gr * D + ((p % CPR) ^ swz_k16<D>(row)) * 8, lds_addr(sK + slot * 16));
      lds_dma16(a.v + base + (size_t)gr * D + ((p % CPR) ^ swz_v16<D>(row)) * 8, lds_addr(sV + slot * 16));
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();
  if (!active) return;

  // state in
  float* st = km_state<D>(a.state, w, wv);
  f32x16 oacc[DT];
#pragma unroll
  for (int g = 0; g < NACC / 4; ++g) {
    const f32x4 x = *(const f32x4*)(st + ((size_t)g * 64 + lane) * 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) oacc[(4 * g + e) >> 4][(4 * g + e) & 15] = x[e];
  }
  float m_ref = st[(size_t)NACC * 64 + lane];
  float l_run = st[(size_t)(NACC + 1) * 64 + lane];
  float lb_run = st[(size_t)(NACC + 2) * 64 + lane];
  const float c = a.scale_log2;

  bf16x8 qop[KC];
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) {
    u32x4 x = {0u, 0u, 0u, 0u};
    if (qi < N) x = *(const u32x4*)(a.q + base + (size_t)qi * D + kc * 16 + h * 8);
    x = (x & a.q_and) ^ a.q_xor;
    qop[kc] = __builtin_bit_cast(bf16x8, x);
  }

  // S^T = K_j Q^T
  f32x16 sacc[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
#pragma unroll
  for (int kc = 0; kc < KC; ++kc)
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int row = kb * 32 + l32;
      const bf16x8 kop = *(const bf16x8*)(sK + row * ROWB + (((2 * kc + h) ^ swz_k16<D>(row)) << 4));
      sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qop[kc], sacc[kb], 0, 0, 0);
    }
  // mask
  if ((k0 + BC > N) || !tile_full<MASK>(qw0, qw0 + 32, k0, k0 + BC, a.window)) {
    const int q_hi_key = MASK == MASK_CAUSAL ? min(qi, N - 1)
                         : MASK == MASK_LOCAL ? min(qi + a.window, N - 1) : N - 1;
    const int q_lo_key = MASK == MASK_LOCAL ? qi - a.window : 0;
    const int hi_rel = q_hi_key - k0 - 4 * h, lo_rel = q_lo_key - k0 - 4 * h;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kr = kb * 32 + acc_key(r);
        const bool ok = (MASK == MASK_LOCAL) ? (kr <= hi_rel && kr >= lo_rel) : (kr <= hi_rel);
        sacc[kb][r] = ok ? sacc[kb][r] : -INFINITY;
      }
  }
  // incremental softmax: the reference moves when a row's block maximum
  // exceeds it by more than 2^RESCALE_LOG2 in exp2 units (any reference keeps
  // numerator and denominator consistent)
  float mx = max16(sacc[0]);
#pragma unroll
  for (int kb = 1; kb < KB; ++kb) mx = fmaxf(mx, max16(sacc[kb]));
  mx = pair_max(mx);
  if (__builtin_amdgcn_ballot_w64((mx - m_ref) * c > RESCALE_LOG2)) {
    const float m_new = fmaxf(m_ref, mx);
    const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f((m_ref - m_new) * c);
    m_ref = m_new;
    l_run *= alpha;
    lb_run *= alpha;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
  }
  const float mc = (m_ref == -INFINITY ? 0.f : m_ref) * c;
  const int g16 = lane >> 4, s16 = lane & 15;
  const int tr_row = 4 * h + (s16 >> 2), tr_ch8 = 4 * (g16 & 1) + (s16 & 3);
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) sacc[kb][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][r], c, -mc));
    l_run += sum16(sacc[kb]);
    bf16x8 pops[2];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) pops[u][e] = (bf16)sacc[kb][8 * u + e];
    lb_run = sum_bf16x16(pops, lb_run);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const bf16x8 pop = pops[u];
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int rlo = kb * 32 + 16 * u + tr_row, rhi = rlo + 8;
        const int clo = ((dt * 8 + tr_ch8) ^ (swz_v16<D>(rlo) << 1)) * 8;
        const int chi = ((dt * 8 + tr_ch8) ^ (swz_v16<D>(rhi) << 1)) * 8;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)(sV + rlo * ROWB + clo));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)(sV + rhi * ROWB + chi));
        const bf16x8 vop = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pop, oacc[dt], 0, 0, 0);
      }
    }
  }
  // state out
#pragma unroll
  for (int g = 0; g < NACC / 4; ++g) {
    f32x4 x;
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = oacc[(4 * g + e) >> 4][(4 * g + e) & 15];
    *(f32x4*)(st + ((size_t)g * 64 + lane) * 4) = x;
  }
  st[(size_t)NACC * 64 + lane] = m_ref;
  st[(size_t)(NACC + 1) * 64 + lane] = l_run;
  st[(size_t)(NACC + 2) * 64 + lane] = lb_run;
}

// O = acc / (rounded-weight sum) and LSE = m scale + ln l from the final state
template <int D>
__global__ __launch_bounds__(512) void km_finalize_kernel(KmArgs a) {
  constexpr int DT = D / 32, NACC = DT * 16;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, l32 = lane & 31, h = lane >> 5;
  const int N = a.N;
  const int w = blockIdx.x;
  const int bh = w / a.n_qtiles, qt = w - bh * a.n_qtiles;
  const int qi = qt * 256 + wv * 32 + l32;
  const float* st = km_state<D>(a.state, w, wv);
  const float m_ref = st[(size_t)NACC * 64 + lane];
  const float lt = pair_sum(st[(size_t)(NACC + 1) * 64 + lane]);
  const float lbt = pair_sum(st[(size_t)(NACC + 2) * 64 + lane]);
  if (qi >= N) return;
  const float inv = 1.f / lbt;
  bf16* O = a.o + (size_t)bh * N * D + (size_t)qi * D;
#pragma unroll
  for (int g = 0; g < NACC / 4; ++g) {
    const f32x4 x = *(const f32x4*)(st + ((size_t)g * 64 + lane) * 4);
    // registers 4g..4g+3 of tile dt = g / 4: value columns dt*32 + 8 r4 + 4h + e
    const int dt = g >> 2, r4 = g & 3;
    bf16x4 y;
#pragma unroll
    for (int e = 0; e < 4; ++e) y[e] = (bf16)(x[e] * inv);
    *(bf16x4*)(O + dt * 32 + 8 * r4 + 4 * h) = y;
  }
  if (h == 0) a.lse[(size_t)bh * N + qi] = m_ref * a.scale_abs + logf(lt);
}

template <int D, int BC, int MASK>
static hipError_t km_run(const KmArgs& a, hipStream_t stream) {
  const size_t n_wg = (size_t)a.BH * a.n_qtiles;
  hipLaunchKernelGGL((km_init_kernel<D>), dim3((unsigned)n_wg), dim3(512), 0, stream, a.state, n_wg);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int tc = (a.N + BC - 1) / BC;
  for (int j = 0; j < tc; ++j) {
    hipLaunchKernelGGL((km_step_kernel<D, BC, MASK>), dim3((unsigned)n_wg), dim3(512), 0, stream, a, j);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((km_finalize_kernel<D>), dim3((unsigned)n_wg), dim3(512), 0, stream, a);
  return hipGetLastError();
}

template <int D, int BC>
static hipError_t km_mask(const KmArgs& a, int mask, hipStream_t stream) {
  if (mask == MASK_CAUSAL) return km_run<D, BC, MASK_CAUSAL>(a, stream);
  if (mask == MASK_LOCAL) return km_run<D, BC, MASK_LOCAL>(a, stream);
  return km_run<D, BC, MASK_NONE>(a, stream);
}

size_t km_state_bytes(int BH, int N, int d) {
  const size_t n_wg = (size_t)BH * ((N + 255) / 256);
  return n_wg * 8 * 64 * (size_t)(d / 32 * 16 + 3) * sizeof(float);
}

hipError_t launch_fwd_keymajor(const KmArgs& a0, int d, int bc, int mask, hipStream_t stream) {
  KmArgs a = a0;
  a.n_qtiles = (a.N + 255) / 256;
  if (d == 128) {
    switch (bc) {
      case 32: return km_mask<128, 32>(a, mask, stream);
      case 64: return km_mask<128, 64>(a, mask, stream);
      default: return km_mask<128, 128>(a, mask, stream);
    }
  }
  switch (bc) {
    case 32: return km_mask<64, 32>(a, mask, stream);
    case 64: return km_mask<64, 64>(a, mask, stream);
    case 128: return km_mask<64, 128>(a, mask, stream);
    default: return km_mask<64, 256>(a, mask, stream);
  }
}

}  // namespace fa
