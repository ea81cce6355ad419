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
//  * Three schedules: the tile kernel runs all scores of a K tile, then the
//    softmax, then P V with the exp of the next 32-key block interleaved;
//    the block-pipelined kernel (an alternative) overlaps the scores of
//    block b+1 with the exp of block b and P V of block b with the maximum
//    of block b+1, keeping the online-softmax state per 32-key block; the
//    ping-pong kernel (another alternative) runs the two waves of each SIMD
//    one phase apart, one on the matrix core while the other runs the
//    softmax.
//  * Under the band mask the key tiles are visited in a rotated order (by
//    tile index modulo the window's tile count), so that neighbouring
//    workgroups read each shared tile at the same step.
//  * The subtracted maximum is refreshed lazily: the reference m only moves
//    when some row's tile maximum exceeds it by more than 2^RESCALE_LOG2 in
//    exp2 units, so most tiles skip the rescale of the accumulator (p then
//    stays below 2^RESCALE_LOG2, harmless in float32 and bf16). Numerator
//    and denominator share the reference, so the result is unchanged.
#include <type_traits>

#include "fa_common.h"
#include "fa_kernels.h"
#include "fa_tile_ops.h"

namespace fa {



// WPE: waves per SIMD the register budget is sized for (2: 256 registers per
// lane; 1: 512, for workgroups whose LDS use leaves room for one per CU).
template <int D, int QB, int NW, int BC, int MASK, int WPE = 2>
__global__ __launch_bounds__(NW * 64, WPE) void fwd_bf16_kernel(FwdArgs a) {
  constexpr int NT = NW * 64;
  constexpr int QW = QB * 32;       // query rows per wave
  constexpr int BR = NW * QW;       // query rows per workgroup
  constexpr int KC = D / 16;        // 16-wide chunks of the QK^T contraction
  constexpr int DT = D / 32;        // 32-column tiles of O^T
  constexpr int KB = BC / 32;       // 32-key blocks per K/V tile
  constexpr int ROWB = D * 2;       // bytes of one K/V row in LDS
  constexpr int TILEB = BC * ROWB;
  constexpr int CPR = D / 8;        // 16-byte chunks per row
  constexpr int CPT = BC * CPR / NT;  // 16-byte chunks per thread per tile
  static_assert((BC * CPR) % NT == 0, "tile chunks must divide evenly");
  static_assert(BC % 32 == 0 && (D == 64 || D == 128), "unsupported tile");

  __shared__ __attribute__((aligned(16))) char smem[4 * TILEB];  // K[2], V[2]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int l32 = lane & 31;
  const int h = lane >> 5;
  const int N = a.N;

  // Workgroup -> (head, query tile); under a causal mask the query tiles
  // with the most keys go first.
  int bh, qt;
  wg_tile(blockIdx.x, a.BH, a.n_qtiles, bh, qt);
  if (MASK == MASK_CAUSAL) qt = a.n_qtiles - 1 - qt;

  const size_t base = (size_t)bh * (size_t)N * D;
  const bf16* __restrict__ Q = a.q + base;
  const bf16* __restrict__ K = a.k + base;
  const bf16* __restrict__ V = a.v + base;
  const int q0 = qt * BR;
  const int qw0 = q0 + wv * QW;  // first query row of this wave

  // Q as the B operand of S^T = K Q^T: lane holds Q[row][16kc + 8h .. +7]
  // for row = qw0 + 32 qb + l32.
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
  // reference maximum (raw units); the lane's part of l (float32 sum of the
  // weights, for the LSE) and of the sum of the bf16-rounded weights (the
  // output's normalizer, in four running parts)
  float m_ref[QB], l_run[QB], lb_run[QB][4];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_ref[qb] = -INFINITY;
    l_run[qb] = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) lb_run[qb][i] = 0.f;
  }
  const float c = a.scale_log2;  // > 0

  // key tiles of the workgroup, and the contiguous sub-range this wave needs
  int k_lo, k_hi;
  key_range<MASK>(q0, q0 + BR, N, a.window, k_lo, k_hi);
  const int t_begin = k_lo / BC;
  const int t_end = (k_hi + BC - 1) / BC;
  const int n_t = t_end - t_begin;
  // i-th key tile visited: in index order, except under the band mask
  // (rotated so that neighbouring workgroups read shared tiles together)
  const int t_rot = MASK == MASK_LOCAL ? band_tile_rotation(BR, BC, a.window, t_begin, n_t) : 0;
  auto tile_at = [&](int i) {
    if constexpr (MASK != MASK_LOCAL) return t_begin + i;
    const int j = i + t_rot;
    return t_begin + (j >= n_t ? j - n_t : j);
  };
  int wk_lo, wk_hi;
  key_range<MASK>(qw0, qw0 + QW, N, a.window, wk_lo, wk_hi);
  const bool wave_live = qw0 < N;

  // K/V staging: global_load_lds_dwordx4 writes lane i's 16 bytes to LDS at
  // the wave's base + 16 i, so each lane fetches the global chunk that
  // belongs at its LDS slot under the XOR swizzle. The byte offsets of those
  // chunks within a tile are the same for every tile, so they are computed
  // once; the tile's first row is a wave-uniform base. In a last, partial
  // tile, rows past N are clamped to row N-1: their keys are masked, so only
  // finiteness of the data matters.
  const int wvu = __builtin_amdgcn_readfirstlane(wv);
  unsigned koff[CPT], voff[CPT];
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    const int p = (wvu * CPT + j) * 64 + lane;
    const int row = p / CPR;
    koff[j] = row * ROWB + (((p % CPR) ^ swz_k16<D>(row)) << 4);
    voff[j] = row * ROWB + (((p % CPR) ^ swz_v16<D>(row)) << 4);
  }
  auto dma = [&](int t, int buf) {
    const int k0 = t * BC;
    const char* gK = (const char*)K + (size_t)k0 * ROWB;
    const char* gV = (const char*)V + (size_t)k0 * ROWB;
    char* sK = smem + buf * TILEB;
    char* sV = smem + (2 + buf) * TILEB;
    if (k0 + BC <= N) {
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
        const int slot = (wvu * CPT + j) * 64;  // first LDS chunk of this instruction
        if constexpr (BC <= 128) {
          lds_dma16_s(gK, koff[j], lds_addr(sK + slot * 16));
          lds_dma16_s(gV, voff[j], lds_addr(sV + slot * 16));
        } else {
          // tiles longer than 128 keys leave too few scalar registers for the
          // base-plus-offset form: full per-lane addresses instead
          lds_dma16(gK + koff[j], lds_addr(sK + slot * 16));
          lds_dma16(gV + voff[j], lds_addr(sV + slot * 16));
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
        const int slot = (wvu * CPT + j) * 64;
        const int p = slot + lane;
        const int row = p / CPR;
        const int gr = min(row, N - 1 - k0);
        const unsigned ko = gr * ROWB + (((p % CPR) ^ swz_k16<D>(row)) << 4);
        const unsigned vo = gr * ROWB + (((p % CPR) ^ swz_v16<D>(row)) << 4);
        if constexpr (BC <= 128) {
          lds_dma16_s(gK, ko, lds_addr(sK + slot * 16));
          lds_dma16_s(gV, vo, lds_addr(sV + slot * 16));
        } else {
          lds_dma16(gK + ko, lds_addr(sK + slot * 16));
          lds_dma16(gV + vo, lds_addr(sV + slot * 16));
        }
      }
    }
  };

  if (n_t > 0) {
    dma(tile_at(0), 0);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the tile is in LDS
  }
  __syncthreads();

  // Per-lane constants of the transposed V read: within each 16-lane group,
  // lane s addresses row 4h + s/4 and 8-byte chunk 4*(group&1) + s%4.
  const int g16 = lane >> 4;
  const int s16 = lane & 15;
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

    // Skip tiles that hold no allowed key for any row of this wave.
    if (wave_live && k0 < wk_hi && k0 + BC > wk_lo) {
      // ---- S^T = K Q^T for BC keys x QW queries; each K read feeds QB MFMAs.
      // K operands are double-buffered in registers one 16-wide chunk ahead,
      // so each LDS read has KB*QB MFMAs of time to land.
      f32x16 sacc[QB][KB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) sacc[qb][kb][r] = 0.f;
      bf16x8 kop[2][KB];
      auto kread = [&](int kc, int slot) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const int row = kb * 32 + l32;
          kop[slot][kb] =
              *(const bf16x8*)(sK + row * ROWB + (((2 * kc + h) ^ swz_k16<D>(row)) << 4));
        }
      };
      kread(0, 0);
      // the first chunk's reads stand alone, so that every group below pairs
      // the reads of chunk kc + 1 with the MFMAs of chunk kc
      __builtin_amdgcn_sched_group_barrier(0x100, KB, 0);
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        if (kc + 1 < KC) kread(kc + 1, (kc + 1) & 1);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            sacc[qb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[kc & 1][kb], qop[qb][kc], sacc[qb][kb], 0, 0, 0);
        if (kc + 1 < KC) __builtin_amdgcn_sched_group_barrier(0x100, KB, 0);  // next chunk's reads
        __builtin_amdgcn_sched_group_barrier(0x008, KB * QB, 0);             // this chunk's MFMAs
      }
      __builtin_amdgcn_sched_barrier(0);

      // ---- mask, only where the tile is not fully visible to this wave
      if ((k0 + BC > N) || !tile_full<MASK>(qw0, qw0 + QW, k0, k0 + BC, a.window)) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          // key allowed iff lo_rel <= 32 kb + acc_key(r) <= hi_rel
          const int qi = qw0 + qb * 32 + l32;
          const int q_hi_key = MASK == MASK_CAUSAL ? min(qi, N - 1)
                               : MASK == MASK_LOCAL ? min(qi + a.window, N - 1) : N - 1;
          const int hoff = 4 * h;
          const int hi_rel = q_hi_key - k0 - hoff;
          const int lo_rel = (MASK == MASK_LOCAL ? qi - a.window : 0) - k0 - hoff;
#pragma unroll
          for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int kr = kb * 32 + acc_key(r);
              const bool ok =
                  (MASK == MASK_LOCAL) ? (kr <= hi_rel && kr >= lo_rel) : (kr <= hi_rel);
              sacc[qb][kb][r] = ok ? sacc[qb][kb][r] : -INFINITY;
            }
        }
      }

      // ---- online softmax (one query per lane and query block)
      float mc[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        float mx = max16(sacc[qb][0]);
#pragma unroll
        for (int kb = 1; kb < KB; ++kb) mx = fmaxf(mx, max16(sacc[qb][kb]));
        mx = pair_max(mx);
        // refresh the reference only when a row's maximum outgrew it
        if (__builtin_amdgcn_ballot_w64((mx - m_ref[qb]) * c > RESCALE_LOG2)) {
          const float m_new = fmaxf(m_ref[qb], mx);
          // 0 when the row had no key before; 1 while it still has none
          const float alpha =
              m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f((m_ref[qb] - m_new) * c);
          m_ref[qb] = m_new;
          l_run[qb] *= alpha;
#pragma unroll
          for (int i = 0; i < 4; ++i) lb_run[qb][i] *= alpha;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[qb][dt][r] *= alpha;
        }
        mc[qb] = (m_ref[qb] == -INFINITY ? 0.f : m_ref[qb]) * c;
      }
      bf16x8 pop[QB][KB][2];
      float ls[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) ls[qb] = 0.f;
      // exp of one 32-key block (all query blocks), its row-sum part and its
      // bf16 MFMA operand
      auto exp_block = [&](int kb) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
          for (int r = 0; r < 16; ++r)
            sacc[qb][kb][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[qb][kb][r], c, -mc[qb]));
          ls[qb] += sum16(sacc[qb][kb]);
#pragma unroll
          for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int e = 0; e < 8; ++e) pop[qb][kb][u][e] = (bf16)sacc[qb][kb][8 * u + e];
          sum_bf16x16_4(pop[qb][kb], lb_run[qb]);
        }
      };
      // O^T += V^T P^T for one 32-key block; each V read feeds QB MFMAs.
      bf16x8 vop[2][DT];
      auto vread = [&](int kb, int u) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const int rlo = kb * 32 + 16 * u + tr_row, rhi = rlo + 8;
          const int clo = ((dt * 8 + tr_ch8) ^ (swz_v16<D>(rlo) << 1)) * 8;
          const int chi = ((dt * 8 + tr_ch8) ^ (swz_v16<D>(rhi) << 1)) * 8;
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)(sV + rlo * ROWB + clo));
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)(sV + rhi * ROWB + chi));
          vop[u][dt] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
      };
      auto pv_mfma = [&](int kb, int u) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            oacc[qb][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[u][dt], pop[qb][kb][u], oacc[qb][dt], 0, 0, 0);
      };
      // Software pipeline over the key blocks: block kb-1's V operands are
      // read first, then its PV MFMAs share a scheduling region with the exp /
      // convert VALU work of block kb (a few VALU ops per MFMA), so LDS
      // latency, the matrix core and the vector ALU overlap.
      // Two waves share each SIMD (wave w and w + NW/2); the older one wins
      // issue arbitration, finishes its tile first and then idles at the
      // barrier while the younger one runs alone. From its exponentials to
      // the end of the tile the younger wave takes priority instead.
      if (NW == 8 && wvu >= NW / 2) __builtin_amdgcn_s_setprio(1);
      exp_block(0);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kb = 1; kb <= KB; ++kb) {
        vread(kb - 1, 0);
        vread(kb - 1, 1);
        if (kb < KB) exp_block(kb);
        pv_mfma(kb - 1, 0);
        pv_mfma(kb - 1, 1);
        __builtin_amdgcn_sched_group_barrier(0x100, 4 * DT, 0);  // all V reads of the block
        if (kb < KB) {
          __builtin_amdgcn_sched_group_barrier(0x002, 16, 0);     // VALU while they land
#pragma unroll
          for (int i = 0; i < 2 * DT; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, QB, 0);      // QB MFMAs
            __builtin_amdgcn_sched_group_barrier(0x002, 5 * QB, 0);  // VALU
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) l_run[qb] += ls[qb];
      if (NW == 8 && wvu >= NW / 2) __builtin_amdgcn_s_setprio(0);
    }

    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): next tile landed in LDS
    __syncthreads();
  };
  for (int i = 0; i < n_t; i += 2) {
    tile_step(i, ic<0>{});
    if (i + 1 < n_t) tile_step(i + 1, ic<1>{});
  }

  // ---- epilogue: O = acc / (sum of the rounded weights), LSE = m * scale + ln l
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = pair_sum(l_run[qb]);
    const float lbt = pair_sum((lb_run[qb][0] + lb_run[qb][1]) + (lb_run[qb][2] + lb_run[qb][3]));
    const int qi = qw0 + qb * 32 + l32;
    if (qi < N) {
      const float inv = 1.f / lbt;
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
      if (h == 0) a.lse[(size_t)bh * N + qi] = m_ref[qb] * a.scale_abs + logf(lt);
    }
  }
}


// ---------------------------------------------------------------------------
// Block-pipelined variant. The online softmax runs per 32-key block (the
// lazily refreshed reference makes any key grouping valid), and inside each
// LDS tile every wave alternates two phases per block b:
//   A: S(b+1) = K(b+1) Q^T on the matrix core, beside exp / row sum / bf16
//      convert of block b on the vector ALU;
//   B: O += P(b) V(b) on the matrix core, beside mask and row maximum of
//      block b+1, followed by the reference check for block b+1.
// Each stretch of matrix work thus has independent vector work next to it
// in the same instruction stream, and only two 32-key score blocks are live.
template <int D, int BC, int MASK>
__global__ __launch_bounds__(512) void fwd_bf16_xb_kernel(FwdArgs a) {
  constexpr int NW = 8;
  constexpr int NT = NW * 64;
  constexpr int BR = NW * 32;
  constexpr int KC = D / 16;
  constexpr int DT = D / 32;
  constexpr int KB = BC / 32;
  constexpr int ROWB = D * 2;
  constexpr int TILEB = BC * ROWB;
  constexpr int CPR = D / 8;
  constexpr int CPW = BC * CPR / NT;  // DMA chunks per lane per tile (K or V)
  static_assert((BC * CPR) % NT == 0 && CPW >= 1, "tile chunks must divide evenly");
  static_assert(KC % 4 == 0, "four exp pieces spread over the QK steps");

  __shared__ __attribute__((aligned(16))) char smem[4 * TILEB];  // K[2], V[2]

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  const int N = a.N;

  int bh, qt;
  wg_tile(blockIdx.x, a.BH, a.n_qtiles, bh, qt);
  if (MASK == MASK_CAUSAL) qt = a.n_qtiles - 1 - qt;

  const size_t base = (size_t)bh * (size_t)N * D;
  const bf16* __restrict__ Q = a.q + base;
  const bf16* __restrict__ K = a.k + base;
  const bf16* __restrict__ V = a.v + base;
  const int q0 = qt * BR;
  const int qw0 = q0 + wv * 32;
  const int qi = qw0 + l32;

  bf16x8 qop[KC];
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) {
    u32x4 x = {0u, 0u, 0u, 0u};
    if (qi < N) x = *(const u32x4*)(Q + (size_t)qi * D + kc * 16 + h * 8);
    x = (x & a.q_and) ^ a.q_xor;
    qop[kc] = __builtin_bit_cast(bf16x8, x);
  }
  f32x16 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.f;
  // running reference, float32 weight sum (LSE), rounded weight sum (output)
  float m_ref = -INFINITY, l_run = 0.f, lb_run = 0.f, mc = 0.f;
  const float c = a.scale_log2;

  int k_lo, k_hi;
  key_range<MASK>(q0, q0 + BR, N, a.window, k_lo, k_hi);
  const int t_begin = k_lo / BC;
  const int t_end = (k_hi + BC - 1) / BC;
  int wk_lo, wk_hi;
  key_range<MASK>(qw0, qw0 + 32, N, a.window, wk_lo, wk_hi);
  const bool wave_live = qw0 < N;
  const int q_hi_key = MASK == MASK_CAUSAL ? min(qi, N - 1)
                       : MASK == MASK_LOCAL ? min(qi + a.window, N - 1) : N - 1;
  const int q_lo_key = MASK == MASK_LOCAL ? qi - a.window : 0;

  // direct global->LDS copy of key tile t into buffer buf (K) and 2 + buf (V):
  // per-lane byte offsets within a tile computed once, the tile's first row
  // as a wave-uniform base; rows past N (last tile only) read row N-1, as
  // their keys are masked
  const int wvu = __builtin_amdgcn_readfirstlane(wv);
  unsigned koff[CPW], voff[CPW];
#pragma unroll
  for (int i = 0; i < CPW; ++i) {
    const int p = (wvu * CPW + i) * 64 + lane;
    const int row = p / CPR;
    koff[i] = row * ROWB + (((p % CPR) ^ swz_k16<D>(row)) << 4);
    voff[i] = row * ROWB + (((p % CPR) ^ swz_v16<D>(row)) << 4);
  }
  auto dma = [&](int t, int buf) {
    const int k0 = t * BC;
    const char* gK = (const char*)K + (size_t)k0 * ROWB;
    const char* gV = (const char*)V + (size_t)k0 * ROWB;
    if (k0 + BC <= N) {
#pragma unroll
      for (int i = 0; i < CPW; ++i) {
        const int slot = (wvu * CPW + i) * 64;
        if constexpr (BC <= 128) {
          lds_dma16_s(gK, koff[i], lds_addr(smem + buf * TILEB + slot * 16));
          lds_dma16_s(gV, voff[i], lds_addr(smem + (2 + buf) * TILEB + slot * 16));
        } else {
          // the longer unrolled block loop of these tiles leaves too few
          // scalar registers for the base-plus-offset form: full per-lane
          // addresses instead
          lds_dma16(gK + koff[i], lds_addr(smem + buf * TILEB + slot * 16));
          lds_dma16(gV + voff[i], lds_addr(smem + (2 + buf) * TILEB + slot * 16));
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < CPW; ++i) {
        const int slot = (wvu * CPW + i) * 64;
        const int p = slot + lane;
        const int row = p / CPR;
        const int gr = min(row, N - 1 - k0);
        const unsigned ko = gr * ROWB + (((p % CPR) ^ swz_k16<D>(row)) << 4);
        const unsigned vo = gr * ROWB + (((p % CPR) ^ swz_v16<D>(row)) << 4);
        if constexpr (BC <= 128) {
          lds_dma16_s(gK, ko, lds_addr(smem + buf * TILEB + slot * 16));
          lds_dma16_s(gV, vo, lds_addr(smem + (2 + buf) * TILEB + slot * 16));
        } else {
          lds_dma16(gK + ko, lds_addr(smem + buf * TILEB + slot * 16));
          lds_dma16(gV + vo, lds_addr(smem + (2 + buf) * TILEB + slot * 16));
        }
      }
    }
  };

  const int g16 = lane >> 4, s16 = lane & 15;
  const int tr_row = 4 * h + (s16 >> 2);
  const int tr_ch8 = 4 * (g16 & 1) + (s16 & 3);

  if (t_begin < t_end) dma(t_begin, 0);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();

  for (int t = t_begin; t < t_end; ++t) {
    const int buf = (t - t_begin) & 1;
    const char* sK = smem + buf * TILEB;
    const char* sV = smem + (2 + buf) * TILEB;
    if (t + 1 < t_end) dma(t + 1, buf ^ 1);
    const int k0 = t * BC;

    if (wave_live && k0 < wk_hi && k0 + BC > wk_lo) {
      f32x16 sacc[2];
      bf16x8 pop[2][2];
      auto kread = [&](int kb, int kc, bf16x8& kop) {
        const int row = kb * 32 + l32;
        kop = *(const bf16x8*)(sK + row * ROWB + (((2 * kc + h) ^ swz_k16<D>(row)) << 4));
      };
      auto vread = [&](int kb, int u, bf16x8 (&vop)[DT]) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const int rlo = kb * 32 + 16 * u + tr_row, rhi = rlo + 8;
          const int clo = ((dt * 8 + tr_ch8) ^ (swz_v16<D>(rlo) << 1)) * 8;
          const int chi = ((dt * 8 + tr_ch8) ^ (swz_v16<D>(rhi) << 1)) * 8;
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)(sV + rlo * ROWB + clo));
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)(sV + rhi * ROWB + chi));
          vop[dt] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
      };
      // mask of block kb (tiles this wave does not see whole)
      auto mask_block = [&](f32x16& S, int kb) {
        const int kb0 = k0 + kb * 32;
        const int hi_rel = q_hi_key - kb0 - 4 * h;
        const int lo_rel = q_lo_key - kb0 - 4 * h;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kr = acc_key(r);
          const bool ok = (MASK == MASK_LOCAL) ? (kr <= hi_rel && kr >= lo_rel) : (kr <= hi_rel);
          S[r] = ok ? S[r] : -INFINITY;
        }
      };
      auto rescale = [&](float mx) {
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
        mc = (m_ref == -INFINITY ? 0.f : m_ref) * c;
      };
      // exp piece q of block scores S (registers 4q..4q+3); the last piece
      // adds the row-sum part (to l_run, which a later rescale scales with
      // the numerator) and writes the bf16 operand P
      auto exp_piece = [&](f32x16& S, int q, bf16x8 (&P)[2]) {
#pragma unroll
        for (int r = 4 * q; r < 4 * q + 4; ++r)
          S[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[r], c, -mc));
        if (q == 3) {
          l_run += sum16(S);
#pragma unroll
          for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int e = 0; e < 8; ++e) P[u][e] = (bf16)S[8 * u + e];
          lb_run = sum_bf16x16(P, lb_run);
        }
      };

      // The tile body, with the per-element mask compiled in (tiles this
      // wave does not see whole) or out (all other tiles: no branch inside).
      auto body = [&](auto masked) {
      constexpr bool MASKED = decltype(masked)::value;
      // block 0: scores, mask, maximum
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[0][r] = 0.f;
      {
        bf16x8 kop[2];
        kread(0, 0, kop[0]);
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
          if (kc + 1 < KC) kread(0, kc + 1, kop[(kc + 1) & 1]);
          sacc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[kc & 1], qop[kc], sacc[0], 0, 0, 0);
        }
      }
      if constexpr (MASKED) mask_block(sacc[0], 0);
      rescale(pair_max(max16(sacc[0])));

#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const int P0 = kb & 1, P1 = P0 ^ 1;
        bf16x8 vop[2][DT];
        // ---- phase A: S(kb+1) beside exp of block kb; then the V operands
        // of block kb are requested
        if (kb + 1 < KB) {
#pragma unroll
          for (int r = 0; r < 16; ++r) sacc[P1][r] = 0.f;
          bf16x8 kop[KC];
#pragma unroll
          for (int kc = 0; kc < KC; ++kc) kread(kb + 1, kc, kop[kc]);
          __builtin_amdgcn_sched_group_barrier(0x100, KC, 0);
#pragma unroll
          for (int kc = 0; kc < KC; ++kc) {
            sacc[P1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[kc], qop[kc], sacc[P1], 0, 0, 0);
            if (kc % (KC / 4) == KC / 4 - 1) exp_piece(sacc[P0], kc / (KC / 4), pop[P0]);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 28 / KC, 0);
          }
          // keep the exp work in this stretch (it would otherwise sink to its
          // use in the P V step below)
          asm volatile("" : "+v"(pop[P0][0]), "+v"(pop[P0][1]), "+v"(l_run), "+v"(lb_run));
          vread(kb, 0, vop[0]);
          vread(kb, 1, vop[1]);
          __builtin_amdgcn_sched_barrier(0);
        } else {
          vread(kb, 0, vop[0]);
          vread(kb, 1, vop[1]);
#pragma unroll
          for (int q = 0; q < 4; ++q) exp_piece(sacc[P0], q, pop[P0]);
        }
        // ---- phase B: O += P(kb) V(kb) beside mask / maximum of block kb+1
        float mx = -INFINITY;
        {
          if (MASKED && kb + 1 < KB) mask_block(sacc[P1], kb + 1);
#pragma unroll
          for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
              oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[u][dt], pop[P0][u], oacc[dt], 0, 0, 0);
          if (kb + 1 < KB) mx = pair_max(max16(sacc[P1]));
#pragma unroll
          for (int i = 0; i < 2 * DT; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        if (kb + 1 < KB) rescale(mx);
      }
      };
      if ((k0 + BC > N) || !tile_full<MASK>(qw0, qw0 + 32, k0, k0 + BC, a.window)) body(ic<1>{});
      else body(ic<0>{});
    }

    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): next tile landed in LDS
    __syncthreads();
  }

  const float lt = pair_sum(l_run);
  const float lbt = pair_sum(lb_run);
  if (qi < N) {
    const float inv = 1.f / lbt;
    bf16* O = a.o + base + (size_t)qi * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        bf16x4 y;
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = (bf16)(oacc[dt][4 * r4 + e] * inv);
        *(bf16x4*)(O + dt * 32 + 8 * r4 + 4 * h) = y;
      }
    if (h == 0) a.lse[(size_t)bh * N + qi] = m_ref * a.scale_abs + logf(lt);
  }
}

// Ping-pong variant of the tile kernel. The two waves that share a SIMD
// (w and w + 4 of the eight) run the same per-tile program,
//   M(t): O^T += V^T P^T for tile t-1, then S^T = K Q^T for tile t
//         (matrix core and LDS reads only);
//   X(t): mask, row maximum, reference check and exp of tile t
//         (vector ALU only),
// with a workgroup barrier after each phase, but the second wave of each
// SIMD starts one phase late. From then on every SIMD holds one wave in an
// M phase and one in an X phase, so the matrix core and the vector ALU work
// at the same time instead of taking turns. P of tile t waits in registers
// (bf16) until the next M phase.
// LDS: K of tile t is read in the M(t) phases of both waves, V of tile t in
// their M(t+1) phases, so the loads of K(t+1) and V(t) share one window of
// two phases: the first wave of each SIMD issues all of them at the start of
// its M(t) phase and waits for them before the barrier that ends its X(t).
template <int D, int QB, int BC, int MASK>
__global__ __launch_bounds__(512, 2) void fwd_bf16_pp_kernel(FwdArgs a) {
  constexpr int NW = 8;
  constexpr int NT = NW * 64;
  constexpr int QW = QB * 32;
  constexpr int BR = NW * QW;
  constexpr int KC = D / 16;
  constexpr int DT = D / 32;
  constexpr int KB = BC / 32;
  constexpr int ROWB = D * 2;
  constexpr int TILEB = BC * ROWB;
  constexpr int CPR = D / 8;
  constexpr int CPT = BC * CPR / NT;
  static_assert((BC * CPR) % NT == 0 && BC <= 128, "tile chunks must divide evenly");
  static_assert(BC % 32 == 0 && (D == 64 || D == 128), "unsupported tile");

  __shared__ __attribute__((aligned(16))) char smem[4 * TILEB];  // K[2], V[2]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int l32 = lane & 31;
  const int h = lane >> 5;
  const int N = a.N;

  int bh, qt;
  wg_tile(blockIdx.x, a.BH, a.n_qtiles, bh, qt);
  if (MASK == MASK_CAUSAL) qt = a.n_qtiles - 1 - qt;

  const size_t base = (size_t)bh * (size_t)N * D;
  const bf16* __restrict__ Q = a.q + base;
  const bf16* __restrict__ K = a.k + base;
  const bf16* __restrict__ V = a.v + base;
  const int q0 = qt * BR;
  const int qw0 = q0 + wv * QW;

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
  float m_ref[QB], l_run[QB], lb_run[QB][4];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_ref[qb] = -INFINITY;
    l_run[qb] = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) lb_run[qb][i] = 0.f;
  }
  const float c = a.scale_log2;

  int k_lo, k_hi;
  key_range<MASK>(q0, q0 + BR, N, a.window, k_lo, k_hi);
  const int t_begin = k_lo / BC;
  const int t_end = (k_hi + BC - 1) / BC;
  int wk_lo, wk_hi;
  key_range<MASK>(qw0, qw0 + QW, N, a.window, wk_lo, wk_hi);
  const bool wave_live = qw0 < N;

  const int wvu = __builtin_amdgcn_readfirstlane(wv);
  const bool lead = wvu < NW / 2;
  // The first wave of each SIMD issues all tile loads (CPL chunks each), at
  // the start of its M phases; the second never touches global memory in
  // the loop. Offsets are recomputed at each load from an opaque copy of the
  // lane index, so that no per-load address stays live across the loop.
  constexpr int CPL = 2 * CPT;
  auto dma = [&](auto is_v, const bf16* G, int t, char* dst) {
    constexpr bool ISV = decltype(is_v)::value;
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int k0 = t * BC;
    const char* g = (const char*)G + (size_t)k0 * ROWB;
    const int rmax = N - 1 - k0;  // rows past N are clamped (their keys are masked)
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int slot = (wvu * CPL + j) * 64;
      const int p = slot + ln;
      const int row = p / CPR;
      const int gr = min(row, rmax);
      const unsigned off = gr * ROWB + (((p % CPR) ^ (ISV ? swz_v16<D>(row) : swz_k16<D>(row))) << 4);
      lds_dma16_s(g, off, lds_addr(dst + slot * 16));
    }
  };
  char* const sK0 = smem;
  char* const sK1 = smem + TILEB;
  char* const sV0 = smem + 2 * TILEB;
  char* const sV1 = smem + 3 * TILEB;
  // loads of window j (tile t = t_begin + j): K(t + 1) into K buffer
  // (j + 1) & 1 and V(t) into V buffer j & 1
  auto window_dma = [&](int t, auto jpar) {
    constexpr int JP = decltype(jpar)::value;
    if (t + 1 < t_end) dma(std::false_type{}, K, t + 1, JP ? sK0 : sK1);
    if (t < t_end) dma(std::true_type{}, V, t, JP ? sV1 : sV0);
  };

  const int g16 = lane >> 4;
  const int s16 = lane & 15;
  const int tr_row = 4 * h + (s16 >> 2);
  const int tr_ch8 = 4 * (g16 & 1) + (s16 & 3);

  if (lead && t_begin < t_end) {
    dma(std::false_type{}, K, t_begin, sK0);
    __builtin_amdgcn_s_waitcnt(0x0F70);
  }
  __syncthreads();
  if (!lead) __syncthreads();  // the second wave of each SIMD runs one phase late

  f32x16 sacc[QB][KB];
  bf16x8 pop[QB][KB][2];
  bool have_p = false;  // pop holds P of the previous tile

  // one (M, X) pair of tile t = t_begin + j; JP = j & 1 (buffer parity)
  auto step = [&](int t, auto jpar) {
    constexpr int JP = decltype(jpar)::value;
    const char* sK = JP ? sK1 : sK0;       // K(t)
    const char* sV = JP ? sV0 : sV1;       // V(t - 1)
    const int k0 = t * BC;
    const bool live = t < t_end && wave_live && k0 < wk_hi && k0 + BC > wk_lo;

    // ---------------- M phase
    if (lead) window_dma(t, jpar);
    if (have_p) {
      bf16x8 vop[2][DT];
      auto vread = [&](int kb, int u) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const int rlo = kb * 32 + 16 * u + tr_row, rhi = rlo + 8;
          const int clo = ((dt * 8 + tr_ch8) ^ (swz_v16<D>(rlo) << 1)) * 8;
          const int chi = ((dt * 8 + tr_ch8) ^ (swz_v16<D>(rhi) << 1)) * 8;
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)(sV + rlo * ROWB + clo));
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)(sV + rhi * ROWB + chi));
          vop[u][dt] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
      };
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          vread(kb, u);
#pragma unroll
          for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
              oacc[qb][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[u][dt], pop[qb][kb][u], oacc[qb][dt], 0, 0, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (live) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) sacc[qb][kb][r] = 0.f;
      bf16x8 kop[2][KB];
      auto kread = [&](int kc, int slot) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const int row = kb * 32 + l32;
          kop[slot][kb] = *(const bf16x8*)(sK + row * ROWB + (((2 * kc + h) ^ swz_k16<D>(row)) << 4));
        }
      };
      kread(0, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, KB, 0);
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        if (kc + 1 < KC) kread(kc + 1, (kc + 1) & 1);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            sacc[qb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[kc & 1][kb], qop[qb][kc], sacc[qb][kb], 0, 0, 0);
        if (kc + 1 < KC) __builtin_amdgcn_sched_group_barrier(0x100, KB, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, KB * QB, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();

    // ---------------- X phase
    have_p = live;
    if (live) {
      if ((k0 + BC > N) || !tile_full<MASK>(qw0, qw0 + QW, k0, k0 + BC, a.window)) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const int qi = qw0 + qb * 32 + l32;
          const int q_hi_key = MASK == MASK_CAUSAL ? min(qi, N - 1)
                               : MASK == MASK_LOCAL ? min(qi + a.window, N - 1) : N - 1;
          const int hoff = 4 * h;
          const int hi_rel = q_hi_key - k0 - hoff;
          const int lo_rel = (MASK == MASK_LOCAL ? qi - a.window : 0) - k0 - hoff;
#pragma unroll
          for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int kr = kb * 32 + acc_key(r);
              const bool ok =
                  (MASK == MASK_LOCAL) ? (kr <= hi_rel && kr >= lo_rel) : (kr <= hi_rel);
              sacc[qb][kb][r] = ok ? sacc[qb][kb][r] : -INFINITY;
            }
        }
      }
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        float mx = max16(sacc[qb][0]);
#pragma unroll
        for (int kb = 1; kb < KB; ++kb) mx = fmaxf(mx, max16(sacc[qb][kb]));
        mx = pair_max(mx);
        if (__builtin_amdgcn_ballot_w64((mx - m_ref[qb]) * c > RESCALE_LOG2)) {
          const float m_new = fmaxf(m_ref[qb], mx);
          const float alpha =
              m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f((m_ref[qb] - m_new) * c);
          m_ref[qb] = m_new;
          l_run[qb] *= alpha;
#pragma unroll
          for (int i = 0; i < 4; ++i) lb_run[qb][i] *= alpha;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[qb][dt][r] *= alpha;
        }
        const float mc = (m_ref[qb] == -INFINITY ? 0.f : m_ref[qb]) * c;
        float ls = 0.f;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
          for (int r = 0; r < 16; ++r)
            sacc[qb][kb][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[qb][kb][r], c, -mc));
          ls += sum16(sacc[qb][kb]);
#pragma unroll
          for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int e = 0; e < 8; ++e) pop[qb][kb][u][e] = (bf16)sacc[qb][kb][8 * u + e];
          sum_bf16x16_4(pop[qb][kb], lb_run[qb]);
        }
        l_run[qb] += ls;
      }
    } else {
      // (nothing reads P after a skipped tile; a defined value here ends the
      // previous P's live range at the last P V instead of carrying it on)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int u = 0; u < 2; ++u) pop[qb][kb][u] = bf16x8{};
    }
    if (lead) __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
  };
  // t runs one past the last tile: its M phase holds the last P V
  int t = t_begin;
  for (; t + 1 <= t_end; t += 2) {
    step(t, ic<0>{});
    step(t + 1, ic<1>{});
  }
  if (t <= t_end) step(t, ic<0>{});
  if (lead) __syncthreads();

#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = pair_sum(l_run[qb]);
    const float lbt = pair_sum((lb_run[qb][0] + lb_run[qb][1]) + (lb_run[qb][2] + lb_run[qb][3]));
    const int qi = qw0 + qb * 32 + l32;
    if (qi < N) {
      const float inv = 1.f / lbt;
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
      if (h == 0) a.lse[(size_t)bh * N + qi] = m_ref[qb] * a.scale_abs + logf(lt);
    }
  }
}

template <int D, int QB, int BC>
static hipError_t launch_fwd_bf16_pp(const FwdArgs& a0, int mask, hipStream_t stream) {
  FwdArgs a = a0;
  constexpr int BR = 8 * QB * 32;
  a.n_qtiles = (a.N + BR - 1) / BR;
  dim3 grid((unsigned)(a.n_qtiles * a.BH)), block(512);
  switch (mask) {
    case MASK_CAUSAL: hipLaunchKernelGGL((fwd_bf16_pp_kernel<D, QB, BC, MASK_CAUSAL>), grid, block, 0, stream, a); break;
    case MASK_LOCAL: hipLaunchKernelGGL((fwd_bf16_pp_kernel<D, QB, BC, MASK_LOCAL>), grid, block, 0, stream, a); break;
    default: hipLaunchKernelGGL((fwd_bf16_pp_kernel<D, QB, BC, MASK_NONE>), grid, block, 0, stream, a); break;
  }
  return hipGetLastError();
}

template <int D, int BC>
static hipError_t launch_fwd_bf16_xb(const FwdArgs& a0, int mask, hipStream_t stream) {
  FwdArgs a = a0;
  a.n_qtiles = (a.N + 255) / 256;
  dim3 grid((unsigned)(a.n_qtiles * a.BH)), block(512);
  switch (mask) {
    case MASK_CAUSAL: hipLaunchKernelGGL((fwd_bf16_xb_kernel<D, BC, MASK_CAUSAL>), grid, block, 0, stream, a); break;
    case MASK_LOCAL: hipLaunchKernelGGL((fwd_bf16_xb_kernel<D, BC, MASK_LOCAL>), grid, block, 0, stream, a); break;
    default: hipLaunchKernelGGL((fwd_bf16_xb_kernel<D, BC, MASK_NONE>), grid, block, 0, stream, a); break;
  }
  return hipGetLastError();
}

template <int D, int QB, int NW, int BC, int WPE = 2>
static hipError_t launch_fwd_bf16_cfg(const FwdArgs& a0, int mask, hipStream_t stream) {
  FwdArgs a = a0;
  constexpr int BR = NW * QB * 32;
  a.n_qtiles = (a.N + BR - 1) / BR;
  dim3 grid((unsigned)(a.n_qtiles * a.BH)), block(NW * 64);
  switch (mask) {
    case MASK_CAUSAL: hipLaunchKernelGGL((fwd_bf16_kernel<D, QB, NW, BC, MASK_CAUSAL, WPE>), grid, block, 0, stream, a); break;
    case MASK_LOCAL: hipLaunchKernelGGL((fwd_bf16_kernel<D, QB, NW, BC, MASK_LOCAL, WPE>), grid, block, 0, stream, a); break;
    default: hipLaunchKernelGGL((fwd_bf16_kernel<D, QB, NW, BC, MASK_NONE, WPE>), grid, block, 0, stream, a); break;
  }
  return hipGetLastError();
}

// Kernel choice per head dimension, picked by interleaved timing on MI355X
// (causal 8192 x 128, 4096 x 128, unmasked 2048 x 64, band 16384 x 128):
// d = 128 uses the tile kernel with 128-key tiles. d = 64 uses the tile
// kernel with two 32-row query blocks per wave (each K and V operand read
// feeds two MFMAs) and 64-key tiles: against the block-pipelined kernel
// 82.2 -> 78.8 us on [4, 16, 2048, 64], 316 -> 302 us on [16, 16, 2048, 64],
// 602 -> 577 us on causal [4, 16, 8192, 64] with four-wave workgroups (two
// per CU), which the causal and band masks keep; without a mask eight-wave
// workgroups are another 1-3% faster (77.0 -> 75.0 us, 2124 -> 2098 us on
// [2, 16, 16384, 64]). At d = 128 two blocks per wave do not fit the
// registers.
// Under a band mask a wave needs only the key tiles within the window of its
// rows while the workgroup streams the union over its waves, so d = 128
// bands use four-wave workgroups: 218 -> 174 us on [1, 32, 16384, 128] with
// radius 128 (64-key tiles, two per CU). With 32-key tiles the kernel needs
// 158 VGPRs, so three waves share each SIMD, which hides more of the band's
// memory latency: 163 -> 156 and 158.6 -> 154.3 us on two cards. At d = 64
// the band takes one query block per wave and 32-key tiles (100 VGPRs, five
// waves per SIMD): 112 -> 76 us on [1, 32, 16384, 64] with radius 128.
// cfg 9 is the ping-pong schedule (fwd_bf16_pp_kernel). It passes the same
// parity tests but is slower at d = 128 (534.6 vs 498.4 us on causal
// [2, 16, 8192, 128]) and even at d = 64 (77.5 vs 76.9 us on [4, 16, 2048,
// 64]). A per-phase timeline shows why: the M phase of the four first waves
// alone takes about 4200 cycles for 2048 cycles of MFMA work. Issuing the
// tile loads costs about 1250 of them, and the P V part is held to the rate
// of the transposed LDS reads. When the two phases overlap, the X phase
// slows from about 1950 to 3300 cycles. So a step costs about as much as
// the two phases back to back.
// cfg selects the alternatives for timing comparisons. cfg 7 and 8 are the
// tile that "What the tiling is actually constrained by" derives from the
// on-chip memory ("The formula, which the title only gestures at"):
// B_c = ceil(M / 4d) keys with M = 160 KiB of LDS counted in bf16 elements
// (160 at d = 128, 320 at d = 64; double-buffered K and V then fill the LDS
// exactly) and B_r = min(B_c, d) rows (128, 64). cfg 7 takes both literally
// in the tile kernel (one workgroup per compute unit, so one wave per SIMD
// with the register file to itself); cfg 8 keeps B_c in the block-pipelined
// kernel, whose live score registers do not grow with the tile, at 256 rows.
hipError_t launch_fwd_bf16(const FwdArgs& a, int d, int mask, int cfg, hipStream_t stream) {
  if (d == 128) {
    switch (cfg) {
      case 1: return launch_fwd_bf16_cfg<128, 1, 8, 64>(a, mask, stream);
      case 2: return launch_fwd_bf16_xb<128, 128>(a, mask, stream);
      case 3: return launch_fwd_bf16_xb<128, 64>(a, mask, stream);
      case 4: return launch_fwd_bf16_cfg<128, 1, 4, 64>(a, mask, stream);
      case 7: return launch_fwd_bf16_cfg<128, 1, 4, 160, 1>(a, mask, stream);
      case 8: return launch_fwd_bf16_xb<128, 160>(a, mask, stream);
      case 9: return launch_fwd_bf16_pp<128, 1, 128>(a, mask, stream);
      default:
        if (mask == MASK_LOCAL) return launch_fwd_bf16_cfg<128, 1, 4, 32>(a, mask, stream);
        return launch_fwd_bf16_cfg<128, 1, 8, 128>(a, mask, stream);
    }
  }
  switch (cfg) {
    case 1: return launch_fwd_bf16_cfg<64, 1, 8, 64>(a, mask, stream);
    case 2: return launch_fwd_bf16_xb<64, 128>(a, mask, stream);
    case 3: return launch_fwd_bf16_cfg<64, 1, 8, 128>(a, mask, stream);
    case 4: return launch_fwd_bf16_cfg<64, 1, 4, 64>(a, mask, stream);
    case 5: return launch_fwd_bf16_xb<64, 64>(a, mask, stream);
    case 6:  // the other workgroup size of the default
      if (mask == MASK_NONE) return launch_fwd_bf16_cfg<64, 2, 4, 64>(a, mask, stream);
      return launch_fwd_bf16_cfg<64, 2, 8, 64>(a, mask, stream);
    case 7: return launch_fwd_bf16_cfg<64, 1, 2, 320, 1>(a, mask, stream);
    case 8: return launch_fwd_bf16_xb<64, 320>(a, mask, stream);
    case 9: return launch_fwd_bf16_pp<64, 2, 64>(a, mask, stream);
    default:
      if (mask == MASK_NONE) return launch_fwd_bf16_cfg<64, 2, 8, 64>(a, mask, stream);
      if (mask == MASK_LOCAL) return launch_fwd_bf16_cfg<64, 1, 4, 32>(a, mask, stream);
      return launch_fwd_bf16_cfg<64, 2, 4, 64>(a, mask, stream);
  }
}

}  // namespace fa
