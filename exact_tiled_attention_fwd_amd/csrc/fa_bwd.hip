// Backward exact attention by recomputation.
//
// The notes ("Flash attention and efficient attention — Hinglish notes",
// "Backward Pass: Recomputation") only say that S and P are recomputed on
// chip from Q, K, V instead of being read back from device memory. The
// gradient of sum(dO * O) follows from the definition by the chain rule:
//   P_ij = exp(z_ij - LSE_i),      D_i  = <dO_i, O_i>
//   dV_j = sum_i P_ij dO_i,        dS_ij = P_ij (<dO_i, v_j> - D_i)
//   dK_j = scale sum_i dS_ij q_i,  dQ_i = scale sum_j dS_ij k_j
// where LSE is the forward's saved log-sum-exp.
//
// Two launches on the caller's stream (bf16), no atomics, deterministic:
//  1. dQ, query-major (the forward's layout): S^T = K Q^T and dP^T = V dO^T
//     put the query on the lane, so LSE_i and D_i are per-lane scalars, and
//     dS^T is the B operand of dQ^T += K^T dS^T (K read transposed). Each
//     query row belongs to one wave, which also computes D_i from its dO and
//     O rows and stores it in the workspace.
//  2. dK/dV, key-major: a workgroup owns a block of keys (K in registers and
//     V in LDS as MFMA B operands) and streams every query tile that sees
//     them (Q, dO, LSE, D) through LDS. S = Q K^T puts the key on the lane,
//     so P^T and dS^T are already the A operands of dV += P^T dO and
//     dK += dS^T Q; the B operands (dO, Q with the query along the lane
//     vector) come from ds_read_b64_tr_b16.
// Recomputing S and dP in the dQ kernel costs two extra contractions (7
// instead of the 5 the gradient needs), the price of determinism without
// atomics. The float32 path keeps a separate preprocess launch for D.
// Under the band mask both kernels visit their tiles in a rotated order (by
// tile index modulo the window's tile count), so that neighbouring
// workgroups read each shared tile at the same step, and the dK/dV kernel
// takes its key blocks in descending order, opposite to the dQ kernel
// launched just before it.
#include "fa_common.h"
#include "fa_kernels.h"
#include "fa_tile_ops.h"

namespace fa {

// XOR swizzle of 16-byte chunks for tiles read both as rows (16-byte
// reads, 32 rows at one column) and transposed (ds_read_b64_tr_b16,
// 8 rows x 64 bytes): both patterns are bank-conflict free.
template <int D>
__device__ __forceinline__ int swz_dual(int row) {
  if constexpr (D == 128) return ((row & 3) << 2) | ((row >> 2) & 3);
  else {
    const int x = (row >> 1) & 7;
    return ((x & 1) << 2) | ((x >> 1) & 3);
  }
}


// ------------------------------------------------------------------ dK / dV
// dK/dV, key-major: NW waves (two per SIMD) of 32 keys each. To fit two
// waves per SIMD next to the dK/dV accumulators, the V operand of
// dP = dO V^T is read from an LDS copy of the workgroup's V rows (loaded
// once) instead of registers; K stays in registers. Q/dO tiles of 32 rows
// arrive by direct global->LDS loads, and every LDS operand is read one step
// ahead of the MFMA that consumes it.
template <int D>
__device__ __forceinline__ int swz_rows(int row) {  // 16-byte chunk swizzle for row reads
  if constexpr (D == 128) return row & 15;
  else return (row >> 1) & 7;
}

template <int D, int NW, int BRQ, int MASK>
__global__ __launch_bounds__(NW * 64, 2) void bwd_dkdv2_bf16_kernel(BwdArgs a) {
  constexpr int BC = NW * 32;       // keys per workgroup (32 per wave)
  constexpr int KC = D / 16;
  constexpr int DT = D / 32;
  constexpr int QBN = BRQ / 32;
  constexpr int ROWB = D * 2;
  constexpr int QTILEB = BRQ * ROWB;
  constexpr int CPR = D / 8;
  constexpr int NINS = BRQ * CPR / 64;  // 64-lane DMA instructions per query tile
  static_assert((BRQ * CPR) % 64 == 0 && BRQ <= NW * 64, "tile must divide over the lanes");

  __shared__ __attribute__((aligned(16))) char sVt[BC * ROWB];      // V rows of this workgroup
  __shared__ __attribute__((aligned(16))) char sQO[4 * QTILEB];     // Q[2], dO[2]
  __shared__ __attribute__((aligned(16))) float sL[2][BRQ];         // LSE * log2(e)
  __shared__ __attribute__((aligned(16))) float sD[2][BRQ];         // -D

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  const int N = a.N;
  const int n_kt = (N + BC - 1) / BC;
  int bh, kt;  // ascending: under a causal mask the first key tiles see most rows
  wg_tile(blockIdx.x, a.BH, n_kt, bh, kt);
  // Under the band every key tile has about the same work, so the order is
  // free: descending, the opposite of the dQ kernel launched just before,
  // whose last query tiles (the same rows) may still be in the L2 and the
  // memory-side cache (band backward 501.2 -> 484.1 us on [1, 32, 16384, 128]).
  if (MASK == MASK_LOCAL) kt = n_kt - 1 - kt;
  const size_t base = (size_t)bh * N * D;
  const bf16* __restrict__ Q = (const bf16*)a.q + base;
  const bf16* __restrict__ K = (const bf16*)a.k + base;
  const bf16* __restrict__ V = (const bf16*)a.v + base;
  const bf16* __restrict__ dO = (const bf16*)a.dout + base;
  const float* __restrict__ LSE = a.lse + (size_t)bh * N;
  const float* __restrict__ Dl = a.delta + (size_t)bh * N;
  const int k0 = kt * BC;
  const int kw0 = k0 + wv * 32;
  const int key = kw0 + l32;

  // this wave's 32 V rows -> LDS (rows past N clamped; their keys are never stored)
#pragma unroll
  for (int j = 0; j < 32 * CPR / 64; ++j) {
    const int p = j * 64 + lane;           // chunk index within the wave's rows
    const int row = wv * 32 + p / CPR;     // row within the workgroup's V block
    int gr = k0 + row;
    gr = gr < N ? gr : N - 1;
    const int cc = (p % CPR) ^ swz_rows<D>(row);
    lds_dma16(V + (size_t)gr * D + cc * 8, lds_addr(sVt + (wv * 32 * CPR + j * 64) * 16));
  }
  bf16x8 kop[KC];
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) {
    u32x4 x = {0u, 0u, 0u, 0u};
    if (key < N) x = *(const u32x4*)(K + (size_t)key * D + kc * 16 + h * 8);
    x = (x & a.q_and) ^ a.q_xor;  // sign / zero of the scale folded into K
    kop[kc] = __builtin_bit_cast(bf16x8, x);
  }
  f32x16 dk[DT], dv[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dk[dt][r] = 0.f;
      dv[dt][r] = 0.f;
    }
  const float c = a.scale_log2;
  const float LOG2E = 1.4426950408889634f;

  int q_lo = 0, q_hi = N;
  if (MASK == MASK_CAUSAL) q_lo = k0;
  if (MASK == MASK_LOCAL) {
    q_lo = k0 - a.window > 0 ? k0 - a.window : 0;
    const long long hh = (long long)k0 + BC + a.window;
    q_hi = hh < N ? (int)hh : N;
  }
  const int t_begin = q_lo / BRQ, t_end = q_lo < q_hi ? (q_hi + BRQ - 1) / BRQ : t_begin;
  const int n_t = t_end - t_begin;
  // i-th query tile visited: in index order, except under the band mask
  // (rotated so that neighbouring workgroups read shared tiles together)
  const int t_rot = MASK == MASK_LOCAL ? band_tile_rotation(BC, BRQ, a.window, t_begin, n_t) : 0;
  auto tile_at = [&](int i) {
    if constexpr (MASK != MASK_LOCAL) return t_begin + i;
    const int j = i + t_rot;
    return t_begin + (j >= n_t ? j - n_t : j);
  };
  // query rows that can see this wave's keys
  int wq_lo = 0, wq_hi = N;
  if (MASK == MASK_CAUSAL) wq_lo = kw0;
  if (MASK == MASK_LOCAL) {
    wq_lo = kw0 - a.window;
    wq_hi = kw0 + 32 + a.window;
  }
  const bool wave_live = kw0 < N;

  // Q/dO tile t -> LDS: per-lane byte offsets within a tile computed once,
  // the tile's first row as a wave-uniform base; rows past N (last tile
  // only) read row N-1 (their P is 0)
  constexpr int IPW = (NINS + NW - 1) / NW;  // DMA instructions per wave
  const int wvu = __builtin_amdgcn_readfirstlane(wv);
  unsigned qoff[IPW];
#pragma unroll
  for (int j = 0; j < IPW; ++j) {
    const int p = (wvu + j * NW) * 64 + lane;
    const int row = p / CPR;
    qoff[j] = row * ROWB + (((p % CPR) ^ swz_dual<D>(row)) << 4);
  }
  auto dma = [&](int t, int buf) {
    char* sQ = sQO + buf * QTILEB;
    char* sO = sQO + (2 + buf) * QTILEB;
    const int r0 = t * BRQ;
    const char* gQ = (const char*)Q + (size_t)r0 * ROWB;
    const char* gO = (const char*)dO + (size_t)r0 * ROWB;
    if (r0 + BRQ <= N) {
#pragma unroll
      for (int j = 0; j < IPW; ++j) {
        const int ins = wvu + j * NW;
        if (ins < NINS) {
          lds_dma16_s(gQ, qoff[j], lds_addr(sQ + ins * 64 * 16));
          lds_dma16_s(gO, qoff[j], lds_addr(sO + ins * 64 * 16));
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < IPW; ++j) {
        const int ins = wvu + j * NW;
        if (ins < NINS) {
          const int p = ins * 64 + lane;
          const int row = p / CPR;
          const unsigned off =
              min(row, N - 1 - r0) * ROWB + (((p % CPR) ^ swz_dual<D>(row)) << 4);
          lds_dma16_s(gQ, off, lds_addr(sQ + ins * 64 * 16));
          lds_dma16_s(gO, off, lds_addr(sO + ins * 64 * 16));
        }
      }
    }
  };
  float stL = 0.f, stD = 0.f;
  auto ld_stats = [&](int t) {
    if (tid < BRQ) {
      const int gr = t * BRQ + tid;
      stL = gr < N ? LSE[gr] * LOG2E : INFINITY;  // padded rows get P = 0
      stD = gr < N ? Dl[gr] : 0.f;
    }
  };
  auto st_stats = [&](int buf) {
    if (tid < BRQ) {
      sL[buf][tid] = stL;
      sD[buf][tid] = -stD;
    }
  };

  if (n_t > 0) {
    dma(tile_at(0), 0);
    ld_stats(tile_at(0));
    st_stats(0);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): V rows and the first tile are in LDS
  __syncthreads();

  const int g16 = lane >> 4, s16 = lane & 15;
  const int tr_row = 4 * h + (s16 >> 2);
  const int tr_ch8 = 4 * (g16 & 1) + (s16 & 3);
  const int vrow = wv * 32 + l32;  // this lane's V row in sVt

  for (int i = 0; i < n_t; ++i) {
    const int buf = i & 1;
    const char* sQ = sQO + buf * QTILEB;
    const char* sO = sQO + (2 + buf) * QTILEB;
    if (i + 1 < n_t) {
      dma(tile_at(i + 1), buf ^ 1);
      ld_stats(tile_at(i + 1));
    }
    const int q0 = tile_at(i) * BRQ;
#pragma unroll 1
    for (int qb = 0; qb < QBN; ++qb) {
      const int qr0 = q0 + qb * 32;
      if (!(wave_live && qr0 < wq_hi && qr0 + 32 > wq_lo)) continue;  // no allowed pair
      // S = Q K^T and dP = dO V^T (lane <-> key, 16 query rows); operands
      // read one 16-wide chunk ahead
      // dP starts from -D (its 16 query rows): the MFMAs then produce dP - D,
      // the factor that dS = P (dP - D) needs, with no subtraction
      f32x16 sa, dp;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const f32x4 nD4 = *(const f32x4*)&sD[buf][qb * 32 + 8 * rr + 4 * h];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sa[4 * rr + e] = 0.f;
          dp[4 * rr + e] = nD4[e];
        }
      }
      const int arow = qb * 32 + l32;
      bf16x8 qa[2], oa[2], va[2];
      auto rd = [&](int kc, int sl) {
        const int off = arow * ROWB + (((2 * kc + h) ^ swz_dual<D>(arow)) << 4);
        qa[sl] = *(const bf16x8*)(sQ + off);
        oa[sl] = *(const bf16x8*)(sO + off);
        va[sl] = *(const bf16x8*)(sVt + vrow * ROWB + (((2 * kc + h) ^ swz_rows<D>(vrow)) << 4));
      };
      rd(0, 0);
      // the first chunk's reads stand alone, so that every group below pairs
      // the reads of chunk kc + 1 with the MFMAs of chunk kc
      __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        if (kc + 1 < KC) rd(kc + 1, (kc + 1) & 1);
        sa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[kc & 1], kop[kc], sa, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa[kc & 1], va[kc & 1], dp, 0, 0, 0);
        if (kc + 1 < KC) __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      const bool need_mask = !tile_full<MASK>(qr0, qr0 + 32, kw0, kw0 + 32, a.window);
      if (need_mask) {  // a uniform branch: full tiles run no per-element compare
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (!allowed<MASK>(qr0 + 8 * (r >> 2) + 4 * h + (r & 3), key, a.window)) sa[r] = -INFINITY;
      }
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const f32x4 L4 = *(const f32x4*)&sL[buf][qb * 32 + 8 * rr + 4 * h];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * rr + e;
          const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sa[r], c, -L4[e]));
          sa[r] = pv;
          dp[r] = pv * dp[r];
        }
      }
      // dV += P^T dO and dK += dS^T Q; B operands by transposed reads
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        bf16x8 pa, da;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pa[e] = (bf16)sa[8 * u + e];
          da[e] = (bf16)dp[8 * u + e];
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const int rlo = qb * 32 + 16 * u + tr_row, rhi = rlo + 8;
          const int clo = ((dt * 8 + tr_ch8) ^ (swz_dual<D>(rlo) << 1)) * 8;
          const int chi = ((dt * 8 + tr_ch8) ^ (swz_dual<D>(rhi) << 1)) * 8;
          const i16x4 olo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)(sO + rlo * ROWB + clo));
          const i16x4 ohi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)(sO + rhi * ROWB + chi));
          const i16x4 qlo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)(sQ + rlo * ROWB + clo));
          const i16x4 qhi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)(sQ + rhi * ROWB + chi));
          const bf16x8 ob = __builtin_bit_cast(bf16x8, __builtin_shufflevector(olo, ohi, 0, 1, 2, 3, 4, 5, 6, 7));
          const bf16x8 qbv = __builtin_bit_cast(bf16x8, __builtin_shufflevector(qlo, qhi, 0, 1, 2, 3, 4, 5, 6, 7));
          dv[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa, ob, dv[dt], 0, 0, 0);
          dk[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da, qbv, dk[dt], 0, 0, 0);
        }
      }
    }
    if (i + 1 < n_t) st_stats(buf ^ 1);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the next tile landed in LDS
    __syncthreads();
  }

  bf16* __restrict__ dK = (bf16*)a.dk + base;
  bf16* __restrict__ dV = (bf16*)a.dv + base;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int kr = kw0 + 8 * (r >> 2) + 4 * h + (r & 3);
    if (kr < N) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        dK[(size_t)kr * D + dt * 32 + l32] = (bf16)(dk[dt][r] * a.scale);
        dV[(size_t)kr * D + dt * 32 + l32] = (bf16)dv[dt][r];
      }
    }
  }
}

// ----------------------------------------------------------------------- dQ
// Query-major, laid out like the forward: S^T = K Q^T and dP^T = V dO^T put
// the query on the lane, so LSE_i and D_i are per-lane scalars, and dS^T is
// the B operand of dQ^T += K^T dS^T (K read transposed). K/V tiles arrive
// by direct global->LDS loads; operands are read one step ahead.
template <int D, int NW, int BC, int MASK>
__global__ __launch_bounds__(NW * 64, 2) void bwd_dq_bf16_kernel(BwdArgs a) {
  constexpr int BR = NW * 32;
  constexpr int KC = D / 16;
  constexpr int DT = D / 32;
  constexpr int KB = BC / 32;
  constexpr int ROWB = D * 2;
  constexpr int TILEB = BC * ROWB;
  constexpr int CPR = D / 8;
  constexpr int NINS = BC * CPR / 64;  // 64-lane DMA instructions per tile
  static_assert((BC * CPR) % 64 == 0, "tile chunks must divide evenly");

  __shared__ __attribute__((aligned(16))) char smem[4 * TILEB];  // K[2] (dual), V[2]

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  const int N = a.N;
  const int n_qt = (N + BR - 1) / BR;
  int bh, qt;
  wg_tile(blockIdx.x, a.BH, n_qt, bh, qt);
  if (MASK == MASK_CAUSAL) qt = n_qt - 1 - qt;
  const size_t base = (size_t)bh * N * D;
  const bf16* __restrict__ Q = (const bf16*)a.q + base;
  const bf16* __restrict__ K = (const bf16*)a.k + base;
  const bf16* __restrict__ V = (const bf16*)a.v + base;
  const bf16* __restrict__ dO = (const bf16*)a.dout + base;
  const int q0 = qt * BR;
  const int qw0 = q0 + wv * 32;
  const int qi = qw0 + l32;  // this lane's query row

  bf16x8 qop[KC], oop[KC];
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) {
    u32x4 x = {0u, 0u, 0u, 0u}, y = {0u, 0u, 0u, 0u};
    if (qi < N) {
      x = *(const u32x4*)(Q + (size_t)qi * D + kc * 16 + h * 8);
      y = *(const u32x4*)(dO + (size_t)qi * D + kc * 16 + h * 8);
    }
    x = (x & a.q_and) ^ a.q_xor;
    qop[kc] = __builtin_bit_cast(bf16x8, x);
    oop[kc] = __builtin_bit_cast(bf16x8, y);
  }
  const float Lq = qi < N ? a.lse[(size_t)bh * N + qi] * 1.4426950408889634f : INFINITY;
  // D_i = <dO_i, O_i>, the row term of dS = P (dP - D). This kernel owns
  // every query row once, so it computes D_i here (lanes l and l + 32 hold
  // the two halves of row l) and stores it for the dK/dV kernel, which runs
  // after it on the stream.
  const bf16* __restrict__ Op = (const bf16*)a.o + base;
  float dpart = 0.f;
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) {
    u32x4 z = {0u, 0u, 0u, 0u};
    if (qi < N) z = *(const u32x4*)(Op + (size_t)qi * D + kc * 16 + h * 8);
    const bf16x8 ov = __builtin_bit_cast(bf16x8, z);
#pragma unroll
    for (int e = 0; e < 8; ++e) dpart = __builtin_fmaf((float)ov[e], (float)oop[kc][e], dpart);
  }
  const float Dq = pair_sum(dpart);
  if (h == 0 && qi < N) a.delta[(size_t)bh * N + qi] = Dq;
  // dP^T starts from -D_i (this lane's query): the MFMAs then produce
  // dP - D, the factor that dS = P (dP - D) needs, with no subtraction
  f32x16 negD;
#pragma unroll
  for (int r = 0; r < 16; ++r) negD[r] = -Dq;
  const float c = a.scale_log2;

  f32x16 dq[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[dt][r] = 0.f;

  int k_lo, k_hi;
  key_range<MASK>(q0, q0 + BR, N, a.window, k_lo, k_hi);
  const int t_begin = k_lo / BC, t_end = (k_hi + BC - 1) / BC;
  const int n_t = t_end - t_begin;
  // i-th key tile visited (rotated under the band mask, as in the dK/dV kernel)
  const int t_rot = MASK == MASK_LOCAL ? band_tile_rotation(BR, BC, a.window, t_begin, n_t) : 0;
  auto tile_at = [&](int i) {
    if constexpr (MASK != MASK_LOCAL) return t_begin + i;
    const int j = i + t_rot;
    return t_begin + (j >= n_t ? j - n_t : j);
  };
  int wk_lo, wk_hi;
  key_range<MASK>(qw0, qw0 + 32, N, a.window, wk_lo, wk_hi);
  const bool wave_live = qw0 < N;

  // K/V tile t -> LDS, addressed as in the dK/dV kernel (keys past N, last
  // tile only, read row N-1 and are masked)
  constexpr int IPW = (NINS + NW - 1) / NW;
  const int wvu = __builtin_amdgcn_readfirstlane(wv);
  unsigned koff[IPW];
#pragma unroll
  for (int j = 0; j < IPW; ++j) {
    const int p = (wvu + j * NW) * 64 + lane;
    const int row = p / CPR;
    koff[j] = row * ROWB + (((p % CPR) ^ swz_dual<D>(row)) << 4);
  }
  auto dma = [&](int t, int buf) {
    char* sK = smem + buf * TILEB;
    char* sV = smem + (2 + buf) * TILEB;
    const int k0 = t * BC;
    const char* gK = (const char*)K + (size_t)k0 * ROWB;
    const char* gV = (const char*)V + (size_t)k0 * ROWB;
    if (k0 + BC <= N) {
#pragma unroll
      for (int j = 0; j < IPW; ++j) {
        const int ins = wvu + j * NW;
        if (ins < NINS) {
          lds_dma16_s(gK, koff[j], lds_addr(sK + ins * 64 * 16));
          lds_dma16_s(gV, koff[j], lds_addr(sV + ins * 64 * 16));
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < IPW; ++j) {
        const int ins = wvu + j * NW;
        if (ins < NINS) {
          const int p = ins * 64 + lane;
          const int row = p / CPR;
          const unsigned off =
              min(row, N - 1 - k0) * ROWB + (((p % CPR) ^ swz_dual<D>(row)) << 4);
          lds_dma16_s(gK, off, lds_addr(sK + ins * 64 * 16));
          lds_dma16_s(gV, off, lds_addr(sV + ins * 64 * 16));
        }
      }
    }
  };
  if (n_t > 0) dma(tile_at(0), 0);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();

  const int g16 = lane >> 4, s16 = lane & 15;
  const int tr_row = 4 * h + (s16 >> 2);
  const int tr_ch8 = 4 * (g16 & 1) + (s16 & 3);

  // the tile loop unrolled by two, so that the double-buffer index is a
  // compile-time constant (LDS addresses take it as an immediate offset)
  auto tile_step = [&](int i, auto buf_tag) {
    constexpr int buf = decltype(buf_tag)::value;
    const char* sK = smem + buf * TILEB;
    const char* sV = smem + (2 + buf) * TILEB;
    if (i + 1 < n_t) dma(tile_at(i + 1), buf ^ 1);
    const int k0 = tile_at(i) * BC;
    if (wave_live && k0 < wk_hi && k0 + BC > wk_lo) {
      bf16x8 dsb[KB][2];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        f32x16 sa, dp = negD;
#pragma unroll
        for (int r = 0; r < 16; ++r) sa[r] = 0.f;
        const int arow = kb * 32 + l32;
        bf16x8 ka[2], va[2];
        auto rd = [&](int kc, int sl) {
          const int off = arow * ROWB + (((2 * kc + h) ^ swz_dual<D>(arow)) << 4);
          ka[sl] = *(const bf16x8*)(sK + off);
          va[sl] = *(const bf16x8*)(sV + off);
        };
        rd(0, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // as in the dK/dV kernel
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
          if (kc + 1 < KC) rd(kc + 1, (kc + 1) & 1);
          sa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[kc & 1], qop[kc], sa, 0, 0, 0);
          dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[kc & 1], oop[kc], dp, 0, 0, 0);
          if (kc + 1 < KC) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        const int kb0 = k0 + kb * 32;
        const bool need_mask =
            (kb0 + 32 > N) || !tile_full<MASK>(qw0, qw0 + 32, kb0, kb0 + 32, a.window);
        if (need_mask) {  // a uniform branch: full tiles run no per-element compare
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kk = kb0 + 8 * (r >> 2) + 4 * h + (r & 3);
            if (!(kk < N && allowed<MASK>(qi, kk, a.window))) sa[r] = -INFINITY;
          }
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sa[r], c, -Lq));
          sa[r] = pv * dp[r];
        }
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int e = 0; e < 8; ++e) dsb[kb][u][e] = (bf16)sa[8 * u + e];
        // dQ^T += K^T dS^T for this key block (K read transposed)
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) {
            const int rlo = kb * 32 + 16 * u + tr_row, rhi = rlo + 8;
            const int clo = ((dt * 8 + tr_ch8) ^ (swz_dual<D>(rlo) << 1)) * 8;
            const int chi = ((dt * 8 + tr_ch8) ^ (swz_dual<D>(rhi) << 1)) * 8;
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)(sK + rlo * ROWB + clo));
            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)(sK + rhi * ROWB + chi));
            const bf16x8 kt = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            dq[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kt, dsb[kb][u], dq[dt], 0, 0, 0);
          }
      }
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the next tile landed in LDS
    __syncthreads();
  };
  for (int i = 0; i < n_t; i += 2) {
    tile_step(i, ic<0>{});
    if (i + 1 < n_t) tile_step(i + 1, ic<1>{});
  }

  if (qi < N) {
    bf16* __restrict__ dQ = (bf16*)a.dq + base + (size_t)qi * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        bf16x4 y;
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = (bf16)(dq[dt][4 * r4 + e] * a.scale);
        *(bf16x4*)(dQ + dt * 32 + 8 * r4 + 4 * h) = y;
      }
  }
}

// ------------------------------------------------------------ float32 path
constexpr int F32B_T = 128;  // rows (keys or queries) per workgroup, one per thread
constexpr int F32B_TILE = 32;

__global__ __launch_bounds__(256) void bwd_pre_f32_kernel(const float* __restrict__ o,
                                                          const float* __restrict__ dout,
                                                          float* __restrict__ delta, long rows,
                                                          int d) {
  const long row = (long)blockIdx.x * 256 + threadIdx.x;
  if (row >= rows) return;
  float acc = 0.f;
  for (int c = 0; c < d; ++c) acc = fmaf(o[row * d + c], dout[row * d + c], acc);
  delta[row] = acc;
}

template <int DP, int MASK>
__global__ __launch_bounds__(F32B_T) void bwd_dkdv_f32_kernel(BwdArgs a) {
  __shared__ float sQ[F32B_TILE][DP], sO[F32B_TILE][DP], sL[F32B_TILE], sDl[F32B_TILE];
  const int N = a.N, d = a.d;
  const int n_t = (N + F32B_T - 1) / F32B_T;
  const int bh = blockIdx.x / n_t;
  const int k0 = (blockIdx.x - bh * n_t) * F32B_T;
  const int kj = k0 + (int)threadIdx.x;
  const size_t base = (size_t)bh * N * d;
  const float* Q = (const float*)a.q + base;
  const float* K = (const float*)a.k + base;
  const float* V = (const float*)a.v + base;
  const float* dO = (const float*)a.dout + base;
  float k[DP], v[DP], dk[DP], dv[DP];
#pragma unroll
  for (int cc = 0; cc < DP; ++cc) {
    const bool ok = kj < N && cc < d;
    k[cc] = ok ? K[(size_t)kj * d + cc] : 0.f;
    v[cc] = ok ? V[(size_t)kj * d + cc] : 0.f;
    dk[cc] = 0.f;
    dv[cc] = 0.f;
  }
  int q_lo = 0, q_hi = N;
  if (MASK == MASK_CAUSAL) q_lo = k0;
  if (MASK == MASK_LOCAL) {
    q_lo = k0 - a.window > 0 ? k0 - a.window : 0;
    const long long hh = (long long)k0 + F32B_T + a.window;
    q_hi = hh < N ? (int)hh : N;
  }
  for (int r0 = (q_lo / F32B_TILE) * F32B_TILE; r0 < q_hi; r0 += F32B_TILE) {
    for (int idx = threadIdx.x; idx < F32B_TILE * DP; idx += F32B_T) {
      const int r = idx / DP, cc = idx % DP, qi = r0 + r;
      const bool ok = qi < N && cc < d;
      sQ[r][cc] = ok ? Q[(size_t)qi * d + cc] : 0.f;
      sO[r][cc] = ok ? dO[(size_t)qi * d + cc] : 0.f;
    }
    if (threadIdx.x < F32B_TILE) {
      const int qi = r0 + threadIdx.x;
      sL[threadIdx.x] = qi < N ? a.lse[(size_t)bh * N + qi] : 0.f;
      sDl[threadIdx.x] = qi < N ? a.delta[(size_t)bh * N + qi] : 0.f;
    }
    __syncthreads();
    for (int r = 0; r < F32B_TILE; ++r) {
      const int qi = r0 + r;
      if (qi >= N || kj >= N || !allowed<MASK>(qi, kj, a.window)) continue;
      float s = 0.f, dpv = 0.f;
#pragma unroll
      for (int cc = 0; cc < DP; ++cc) {
        s = fmaf(sQ[r][cc], k[cc], s);
        dpv = fmaf(sO[r][cc], v[cc], dpv);
      }
      const float p = expf(a.scale * s - sL[r]);
      const float ds = p * (dpv - sDl[r]);
#pragma unroll
      for (int cc = 0; cc < DP; ++cc) {
        dv[cc] = fmaf(p, sO[r][cc], dv[cc]);
        dk[cc] = fmaf(ds, sQ[r][cc], dk[cc]);
      }
    }
    __syncthreads();
  }
  if (kj < N) {
    for (int cc = 0; cc < d && cc < DP; ++cc) {
      ((float*)a.dk)[base + (size_t)kj * d + cc] = a.scale * dk[cc];
      ((float*)a.dv)[base + (size_t)kj * d + cc] = dv[cc];
    }
  }
}

template <int DP, int MASK>
__global__ __launch_bounds__(F32B_T) void bwd_dq_f32_kernel(BwdArgs a) {
  __shared__ float sK[F32B_TILE][DP], sV[F32B_TILE][DP];
  const int N = a.N, d = a.d;
  const int n_t = (N + F32B_T - 1) / F32B_T;
  const int bh = blockIdx.x / n_t;
  const int q0 = (blockIdx.x - bh * n_t) * F32B_T;
  const int qi = q0 + (int)threadIdx.x;
  const size_t base = (size_t)bh * N * d;
  const float* Q = (const float*)a.q + base;
  const float* K = (const float*)a.k + base;
  const float* V = (const float*)a.v + base;
  const float* dO = (const float*)a.dout + base;
  float q[DP], o[DP], dq[DP];
#pragma unroll
  for (int cc = 0; cc < DP; ++cc) {
    const bool ok = qi < N && cc < d;
    q[cc] = ok ? Q[(size_t)qi * d + cc] : 0.f;
    o[cc] = ok ? dO[(size_t)qi * d + cc] : 0.f;
    dq[cc] = 0.f;
  }
  const float L = qi < N ? a.lse[(size_t)bh * N + qi] : 0.f;
  const float Dv = qi < N ? a.delta[(size_t)bh * N + qi] : 0.f;
  int k_lo, k_hi;
  key_range<MASK>(q0, q0 + F32B_T, N, a.window, k_lo, k_hi);
  for (int r0 = (k_lo / F32B_TILE) * F32B_TILE; r0 < k_hi; r0 += F32B_TILE) {
    for (int idx = threadIdx.x; idx < F32B_TILE * DP; idx += F32B_T) {
      const int r = idx / DP, cc = idx % DP, kj = r0 + r;
      const bool ok = kj < N && cc < d;
      sK[r][cc] = ok ? K[(size_t)kj * d + cc] : 0.f;
      sV[r][cc] = ok ? V[(size_t)kj * d + cc] : 0.f;
    }
    __syncthreads();
    for (int r = 0; r < F32B_TILE; ++r) {
      const int kj = r0 + r;
      if (qi >= N || kj >= N || !allowed<MASK>(qi, kj, a.window)) continue;
      float s = 0.f, dpv = 0.f;
#pragma unroll
      for (int cc = 0; cc < DP; ++cc) {
        s = fmaf(q[cc], sK[r][cc], s);
        dpv = fmaf(o[cc], sV[r][cc], dpv);
      }
      const float p = expf(a.scale * s - L);
      const float ds = p * (dpv - Dv);
#pragma unroll
      for (int cc = 0; cc < DP; ++cc) dq[cc] = fmaf(ds, sK[r][cc], dq[cc]);
    }
    __syncthreads();
  }
  if (qi < N)
    for (int cc = 0; cc < d && cc < DP; ++cc)
      ((float*)a.dq)[base + (size_t)qi * d + cc] = a.scale * dq[cc];
}

// ------------------------------------------------------------------ launch
// dK/dV (KNW waves of 32 keys) and dQ (QNW waves of 32 queries) launches.
template <int D, int MASK, int KNW, int QNW>
static hipError_t launch_bwd_main(const BwdArgs& a, hipStream_t stream) {
  // dQ first: it also writes D, which the dK/dV kernel reads
  const int n_qt = (a.N + QNW * 32 - 1) / (QNW * 32);
  hipLaunchKernelGGL((bwd_dq_bf16_kernel<D, QNW, 64, MASK>), dim3((unsigned)(n_qt * a.BH)),
                     dim3(QNW * 64), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int n_kt = (a.N + KNW * 32 - 1) / (KNW * 32);
  hipLaunchKernelGGL((bwd_dkdv2_bf16_kernel<D, KNW, 32, MASK>), dim3((unsigned)(n_kt * a.BH)),
                     dim3(KNW * 64), 0, stream, a);
  return hipGetLastError();
}

template <int D, int MASK>
static hipError_t launch_bwd_bf16_mask(const BwdArgs& a, int cfg, hipStream_t stream) {
  // Under a band mask a wave needs only the query (key) rows within the
  // window of its own 32 keys (queries), while a workgroup streams the union
  // over its waves: four waves per workgroup keep more of each streamed tile
  // useful than eight. cfg 2 swaps the choice (timing comparisons).
  if ((MASK == MASK_LOCAL) != (cfg == 2)) return launch_bwd_main<D, MASK, 4, 4>(a, stream);
  return launch_bwd_main<D, MASK, 8, 8>(a, stream);
}

template <int DP, int MASK>
static hipError_t launch_bwd_f32_mask(const BwdArgs& a, hipStream_t stream) {
  const long rows = (long)a.BH * a.N;
  hipLaunchKernelGGL(bwd_pre_f32_kernel, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, stream,
                     (const float*)a.o, (const float*)a.dout, a.delta, rows, a.d);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int n_t = (a.N + F32B_T - 1) / F32B_T;
  hipLaunchKernelGGL((bwd_dkdv_f32_kernel<DP, MASK>), dim3((unsigned)(n_t * a.BH)), dim3(F32B_T), 0,
                     stream, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_dq_f32_kernel<DP, MASK>), dim3((unsigned)(n_t * a.BH)), dim3(F32B_T), 0,
                     stream, a);
  return hipGetLastError();
}

template <int MASK>
static hipError_t launch_bwd_mask(const BwdArgs& a, int bf16_path, int cfg, hipStream_t stream) {
  if (bf16_path) {
    if (a.d == 128) return launch_bwd_bf16_mask<128, MASK>(a, cfg, stream);
    return launch_bwd_bf16_mask<64, MASK>(a, cfg, stream);
  }
  if (a.d <= 8) return launch_bwd_f32_mask<8, MASK>(a, stream);
  if (a.d <= 32) return launch_bwd_f32_mask<32, MASK>(a, stream);
  if (a.d <= 64) return launch_bwd_f32_mask<64, MASK>(a, stream);
  return launch_bwd_f32_mask<128, MASK>(a, stream);
}

hipError_t launch_bwd(const BwdArgs& a, int bf16_path, int mask, int cfg, hipStream_t stream) {
  switch (mask) {
    case MASK_CAUSAL: return launch_bwd_mask<MASK_CAUSAL>(a, bf16_path, cfg, stream);
    case MASK_LOCAL: return launch_bwd_mask<MASK_LOCAL>(a, bf16_path, cfg, stream);
    default: return launch_bwd_mask<MASK_NONE>(a, bf16_path, cfg, stream);
  }
}

}  // namespace fa
