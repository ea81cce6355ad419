// Forward exact attention, bf16 storage, fp32 accumulation, gfx950 MFMA.
//
// Method (Hinglish notes "Flash attention and efficient attention",
// "Derivation: Incremental Softmax", Steps 1–3): for each query row keep a
// running maximum m, a running denominator l and an unnormalized numerator;
// every key tile updates them with m' = max(m, rowmax), alpha = exp(m - m'),
// l = alpha l + sum p, acc = alpha acc + p V. The schedule is query-major
// (TensorViz "Compute attention one tile at a time", step "tiles"): one
// workgroup owns a block of query rows and streams every K/V tile it needs
// through LDS.
//
// gfx950 mapping
//  * A wave owns QB blocks of 32 query rows. Scores are produced transposed,
//    S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: the accumulator of lane l
//    holds 16 keys of query column (l mod 32), so row max / row sum are
//    in-lane plus one exchange between lanes l and l+32, and the running
//    statistics are per-lane scalars.
//  * That accumulator, rounded to bf16, is already the B operand of
//    O^T = V^T P^T (same lane <-> query, 8 keys per lane), so P never goes
//    through LDS. The matching A operand (8 keys of one value column per
//    lane) is read from the row-major V tile with ds_read_b64_tr_b16.
//  * O^T accumulates in registers with the query on the lane, so the
//    rescale by alpha is one multiply per accumulator register.
//  * K/V tiles are double-buffered in LDS with an XOR swizzle (no padding)
//    chosen so that the 16-byte K reads and the 8-byte transposed V reads
//    are bank-conflict free; the next tile's global loads are in flight
//    while the current one is computed.
//  * exp is computed as exp2 with scale*log2(e) folded into one FMA.
#include "fa_common.h"
#include "fa_kernels.h"

namespace fa {

// 16-byte chunk swizzle of a K row (D/8 chunks per row).
template <int D>
__device__ __forceinline__ int swz_k16(int row) {
  if constexpr (D == 128) return row & 15;
  else return (row >> 1) & 7;
}
// 16-byte chunk swizzle of a V row; 8-byte chunk index c maps to
// c ^ (2 * swz_v16(row)).
template <int D>
__device__ __forceinline__ int swz_v16(int row) {
  if constexpr (D == 128) return (row & 3) << 2;
  else return ((row >> 1) & 1) << 2;
}

template <int D, int QB, int NW, int BC, int MASK>
__global__ __launch_bounds__(NW * 64, 1) void fwd_bf16_kernel(FwdArgs a) {
  constexpr int NT = NW * 64;
  constexpr int BR = NW * QB * 32;  // query rows per workgroup
  constexpr int KC = D / 16;        // 16-wide chunks of the QK^T contraction
  constexpr int DT = D / 32;        // 32-column tiles of O^T
  constexpr int KB = BC / 32;       // 32-key blocks per K/V tile
  constexpr int ROWB = D * 2;       // bytes of one K/V row in LDS
  constexpr int TILEB = BC * ROWB;
  constexpr int CPR = D / 8;        // 16-byte chunks per row
  constexpr int CPT = BC * CPR / NT;  // 16-byte chunks per thread per tile
  static_assert((BC * CPR) % NT == 0, "tile chunks must divide evenly");
  static_assert(BC % 32 == 0 && (D == 64 || D == 128), "unsupported tile");

  __shared__ __attribute__((aligned(16))) char smem[4 * TILEB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int l32 = lane & 31;
  const int h = lane >> 5;
  const int N = a.N;

  // Workgroup -> (head, query tile). Consecutive workgroup ids land on
  // different XCDs, so the ids are regrouped to give every XCD a contiguous
  // run of heads (their K/V stay in that XCD's L2); within a head the query
  // tiles with the most keys go first.
  const int total = a.BH * a.n_qtiles;
  int w = blockIdx.x;
  if ((total & 7) == 0) w = (w & 7) * (total >> 3) + (w >> 3);
  const int bh = w / a.n_qtiles;
  int qt = w - bh * a.n_qtiles;
  if (MASK == MASK_CAUSAL) qt = a.n_qtiles - 1 - qt;

  const size_t base = (size_t)bh * (size_t)N * D;
  const bf16* __restrict__ Q = a.q + base;
  const bf16* __restrict__ K = a.k + base;
  const bf16* __restrict__ V = a.v + base;
  const int q0 = qt * BR;
  const int qw0 = q0 + wv * QB * 32;  // first query row of this wave

  // Q as the B operand of S^T = K Q^T: lane holds Q[row][16kc + 8h .. +7].
  bf16x8 qop[QB][KC];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = qw0 + qb * 32 + l32;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (row < N) x = *(const u32x4*)(Q + (size_t)row * D + kc * 16 + h * 8);
      x = (x & a.q_and) ^ a.q_xor;
      qop[qb][kc] = __builtin_bit_cast(bf16x8, x);
    }
  }

  f32x16 oacc[QB][DT];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[qb][dt][r] = 0.f;
  float m_run[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.f;
  }
  const float c = a.scale_log2;  // > 0

  int k_lo, k_hi;
  key_range<MASK>(q0, q0 + BR, N, a.window, k_lo, k_hi);
  const int t_begin = k_lo / BC;
  const int t_end = (k_hi + BC - 1) / BC;

  u32x4 stK[CPT], stV[CPT];
  auto gload = [&](int t) {
    const int k0 = t * BC;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int ch = tid + NT * i;
      const int row = ch / CPR, cc = ch % CPR;
      const int gr = k0 + row;
      u32x4 zk = {0u, 0u, 0u, 0u}, zv = {0u, 0u, 0u, 0u};
      if (gr < N) {
        zk = *(const u32x4*)(K + (size_t)gr * D + cc * 8);
        zv = *(const u32x4*)(V + (size_t)gr * D + cc * 8);
      }
      stK[i] = zk;
      stV[i] = zv;
    }
  };
  auto lstore = [&](int buf) {
    char* sK = smem + buf * TILEB;
    char* sV = smem + (2 + buf) * TILEB;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int ch = tid + NT * i;
      const int row = ch / CPR, cc = ch % CPR;
      *(u32x4*)(sK + row * ROWB + ((cc ^ swz_k16<D>(row)) << 4)) = stK[i];
      *(u32x4*)(sV + row * ROWB + ((cc ^ swz_v16<D>(row)) << 4)) = stV[i];
    }
  };

  if (t_begin < t_end) {
    gload(t_begin);
    lstore(0);
  }
  __syncthreads();

  // Per-lane constants of the transposed V read: within each 16-lane group,
  // lane s points at row 4*(s/4)+... of a 4-key x 16-column block.
  const int g16 = lane >> 4;      // 16-lane group 0..3
  const int s16 = lane & 15;
  const int tr_row = 4 * h + (s16 >> 2);               // + 32kb + 16u + 8t
  const int tr_ch8 = 4 * (g16 & 1) + (s16 & 3);        // + 8dt  (8-byte chunks)

  for (int t = t_begin; t < t_end; ++t) {
    const int buf = (t - t_begin) & 1;
    const char* sK = smem + buf * TILEB;
    const char* sV = smem + (2 + buf) * TILEB;
    if (t + 1 < t_end) gload(t + 1);
    const int k0 = t * BC;

    // ---- S^T = K Q^T for BC keys x 32*QB queries
    f32x16 sacc[QB][KB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[qb][kb][r] = 0.f;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const int row = kb * 32 + l32;
        const bf16x8 ka =
            *(const bf16x8*)(sK + row * ROWB + (((2 * kc + h) ^ swz_k16<D>(row)) << 4));
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          sacc[qb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qop[qb][kc], sacc[qb][kb], 0, 0, 0);
      }
    }

    // ---- mask (only where the tile is not fully visible to this wave)
    const bool need_mask =
        (k0 + BC > N) || !tile_full<MASK>(qw0, qw0 + QB * 32, k0, k0 + BC, a.window);
    if (need_mask) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int qi = qw0 + qb * 32 + l32;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
            if (!(key < N && allowed<MASK>(qi, key, a.window))) sacc[qb][kb][r] = -INFINITY;
          }
      }
    }

    // ---- online softmax update (per lane: one query, 16 keys per block)
    bf16x8 pop[QB][KB][2];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[qb][kb][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run[qb], mx);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float mc = m_use * c;
      const float alpha = __builtin_amdgcn_exp2f(m_run[qb] * c - mc);
      float ls = 0.f;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[qb][kb][r], c, -mc));
          sacc[qb][kb][r] = p;
          ls += p;
        }
      l_run[qb] = alpha * l_run[qb] + ls;
      m_run[qb] = m_new;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[qb][dt][r] *= alpha;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int s = 0; s < 8; ++s) pop[qb][kb][u][s] = (bf16)sacc[qb][kb][8 * u + s];
    }

    // ---- O^T += V^T P^T
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          i16x4 lo, hi;
          {
            const int row = kb * 32 + 16 * u + tr_row;
            const int ch = (dt * 8 + tr_ch8) ^ (swz_v16<D>(row) << 1);
            lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)(sV + row * ROWB + ch * 8));
          }
          {
            const int row = kb * 32 + 16 * u + 8 + tr_row;
            const int ch = (dt * 8 + tr_ch8) ^ (swz_v16<D>(row) << 1);
            hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)(sV + row * ROWB + ch * 8));
          }
          const bf16x8 va = __builtin_bit_cast(
              bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            oacc[qb][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pop[qb][kb][u], oacc[qb][dt], 0, 0, 0);
        }

    if (t + 1 < t_end) lstore(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O = acc / l, LSE = m*scale + ln l
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = l_run[qb] + __shfl_xor(l_run[qb], 32);
    const float inv = 1.f / lt;
    const int qi = qw0 + qb * 32 + l32;
    if (qi < N) {
      bf16* O = a.o + base + (size_t)qi * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          bf16x4 y;
#pragma unroll
          for (int e = 0; e < 4; ++e) y[e] = (bf16)(oacc[qb][dt][4 * r4 + e] * inv);
          *(bf16x4*)(O + dt * 32 + 8 * r4 + 4 * h) = y;
        }
      if (h == 0) a.lse[(size_t)bh * N + qi] = m_run[qb] * a.scale_abs + logf(lt);
    }
  }
}

template <int D, int QB, int NW, int BC>
static hipError_t launch_fwd_bf16_cfg(const FwdArgs& a0, int mask, hipStream_t stream) {
  FwdArgs a = a0;
  constexpr int BR = NW * QB * 32;
  a.n_qtiles = (a.N + BR - 1) / BR;
  dim3 grid((unsigned)(a.n_qtiles * a.BH)), block(NW * 64);
  switch (mask) {
    case MASK_CAUSAL: hipLaunchKernelGGL((fwd_bf16_kernel<D, QB, NW, BC, MASK_CAUSAL>), grid, block, 0, stream, a); break;
    case MASK_LOCAL: hipLaunchKernelGGL((fwd_bf16_kernel<D, QB, NW, BC, MASK_LOCAL>), grid, block, 0, stream, a); break;
    default: hipLaunchKernelGGL((fwd_bf16_kernel<D, QB, NW, BC, MASK_NONE>), grid, block, 0, stream, a); break;
  }
  return hipGetLastError();
}

// Tile configurations (QB x 32 query rows per wave, NW waves, BC keys per
// tile). The default was picked by measurement on MI355X: one 32-row query
// block per wave and eight waves (two per SIMD) beat the register-heavy
// two-block waves, which leave no second wave to overlap softmax with MFMA.
hipError_t launch_fwd_bf16(const FwdArgs& a, int d, int mask, int cfg, hipStream_t stream) {
  if (d == 128) {
    switch (cfg) {
      case 1: return launch_fwd_bf16_cfg<128, 1, 4, 64>(a, mask, stream);
      case 2: return launch_fwd_bf16_cfg<128, 2, 4, 32>(a, mask, stream);
      case 4: return launch_fwd_bf16_cfg<128, 2, 4, 64>(a, mask, stream);
      default: return launch_fwd_bf16_cfg<128, 1, 8, 64>(a, mask, stream);
    }
  }
  switch (cfg) {
    case 1: return launch_fwd_bf16_cfg<64, 1, 4, 64>(a, mask, stream);
    case 2: return launch_fwd_bf16_cfg<64, 2, 4, 32>(a, mask, stream);
    case 4: return launch_fwd_bf16_cfg<64, 2, 4, 64>(a, mask, stream);
    default: return launch_fwd_bf16_cfg<64, 1, 8, 64>(a, mask, stream);
  }
}

}  // namespace fa
