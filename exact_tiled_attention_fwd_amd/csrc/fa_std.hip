// Standard (unfused) attention, bf16 storage, for comparison with the fused
// forward. The three steps of the notes' "The Standard Attention Problem"
// each make a round trip through device memory, as that page's "Memory
// Hierarchy" section counts them:
//   1. S = scale Q K^T, float32, every (query, key) pair; masked pairs -inf;
//   2. row softmax: m_i, l_i, LSE_i = m_i + ln l_i, and P = exp(S - m) / l
//      written as bf16;
//   3. O = P V, divided by the row sum of the bf16-rounded P (1 up to that
//      rounding), so that each output row is a convex combination of value
//      rows with the weights the product actually used.
// Workspace layout (fa_fwd_standard_workspace_bytes): S as [BH][N][lds]
// float32 with lds = N rounded up to 4, then P as [BH][N][ldp] bf16 with
// ldp = N rounded up to 8 (16-byte aligned rows).
//
// The standard backward (the notes' "Backward Pass: Recomputation" contrasts
// it with the recomputing one) reads the stored P instead of recomputing it,
// and makes each N x N intermediate a round trip through device memory too:
//   4. dP = dO V^T, float32, into a workspace of the forward's layout (S region);
//   5. dV = P^T dO;
//   6. D_i = sum_j P_ij dP_ij and dS = P (dP - D), bf16 (P region of that workspace);
//   7. dQ = scale dS K (the P V kernel without normalization);
//   8. dK = scale dS^T Q.
// The chain rule behind 5-8 is the one the recomputing backward uses.
#include "fa_common.h"
#include "fa_kernels.h"
#include "fa_tile_ops.h"

namespace fa {

// ---- step 1: S = scale Q K^T. Workgroup: 256 queries (8 waves x 32) x 128
// keys. S = Q K^T with Q as the A operand puts the key on the lane, so each
// accumulator register of a half-wave is 32 consecutive keys of one query
// row: 128-byte coalesced stores.
template <int D, int MASK>
__global__ __launch_bounds__(512) void std_scores_kernel(StdArgs a) {
  constexpr int BC = 128, KC = D / 16, KB = BC / 32, ROWB = D * 2, CPR = D / 8;
  constexpr int CPT = BC * CPR / 512;
  __shared__ __attribute__((aligned(16))) char sK[BC * ROWB];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, l32 = lane & 31, h = lane >> 5;
  const int N = a.N;
  const int n_kt = (N + BC - 1) / BC, n_qt = (N + 255) / 256;
  int w = blockIdx.x;
  const int kt = w % n_kt;
  w /= n_kt;
  const int qt = w % n_qt;
  const int bh = w / n_qt;
  const size_t base = (size_t)bh * N * D;
  const int k0 = kt * BC, q0 = qt * 256 + wv * 32;

#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    const int slot = (wv * CPT + j) * 64;
    const int p = slot + lane;
    const int row = p / CPR;
    int gr = k0 + row;
    gr = gr < N ? gr : N - 1;
    lds_dma16(a.k + base + (size_t)gr * D + ((p % CPR) ^ swz_k16<D>(row)) * 8, lds_addr(sK + slot * 16));
  }
  bf16x8 qop[KC];
  const int qi = q0 + l32;
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) {
    u32x4 x = {0u, 0u, 0u, 0u};
    if (qi < N) x = *(const u32x4*)(a.q + base + (size_t)qi * D + kc * 16 + h * 8);
    qop[kc] = __builtin_bit_cast(bf16x8, x);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): K tile in LDS
  __syncthreads();
  if (q0 >= N) return;

  float* S = a.s + (size_t)bh * N * a.lds;
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
    const int row = kb * 32 + l32;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      const bf16x8 kop = *(const bf16x8*)(sK + row * ROWB + (((2 * kc + h) ^ swz_k16<D>(row)) << 4));
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qop[kc], kop, acc, 0, 0, 0);
    }
    const int key = k0 + kb * 32 + l32;
    if (key < N) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = q0 + 8 * (r >> 2) + 4 * h + (r & 3);
        if (i < N) {
          const float z = allowed<MASK>(i, key, a.window) ? a.scale * acc[r] : -INFINITY;
          S[(size_t)i * a.lds + key] = z;
        }
      }
    }
  }
}

// ---- step 2: row softmax, one workgroup of 256 threads per row: one pass
// for the maximum and the sum (online, per thread, then merged), a second
// pass writing P = exp(z - m) / l in bf16.
__device__ __forceinline__ void merge_ml(float& m, float& l, float m2, float l2) {
  const float mn = fmaxf(m, m2);
  if (mn == -INFINITY) return;
  l = l * __expf(m - mn) + l2 * __expf(m2 - mn);
  m = mn;
}

__global__ __launch_bounds__(256) void std_softmax_kernel(StdArgs a) {
  __shared__ float sm[4], sl[4];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const size_t row = blockIdx.x;  // bh * N + i
  const int N = a.N;
  const float* z = a.s + row * a.lds;
  float m = -INFINITY, l = 0.f;
  for (int j = tid; j < N; j += 256) {
    const float x = z[j];
    if (x > m) {
      l = (m == -INFINITY ? 0.f : l * __expf(m - x)) + 1.f;
      m = x;
    } else if (x != -INFINITY) {
      l += __expf(x - m);
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float m2 = __shfl_xor(m, off), l2 = __shfl_xor(l, off);
    merge_ml(m, l, m2, l2);
  }
  if (lane == 0) {
    sm[wv] = m;
    sl[wv] = l;
  }
  __syncthreads();
  m = sm[0];
  l = sl[0];
#pragma unroll
  for (int w2 = 1; w2 < 4; ++w2) merge_ml(m, l, sm[w2], sl[w2]);
  const float inv = 1.f / l;
  bf16* p = a.p + row * a.ldp;
  for (int j = tid; j < a.ldp; j += 256) p[j] = (bf16)(j < N ? __expf(z[j] - m) * inv : 0.f);
  if (tid == 0) a.lse[row] = m + logf(l);
}

// ---- step 3: O = P V. Workgroup: 256 queries (8 waves x 32); V tiles of 64
// keys through double-buffered LDS (direct loads), read transposed as the A
// operand of O^T = V^T P^T; P rows come from memory as the B operand, each
// lane taking the 8 keys of one query that match the transposed V read
// (keys 16u + 4h + {0..3} and 16u + 8 + 4h + {0..3} of step u).
// NORM: divide each row by its sum of the rounded weights (the forward's
// O = P V); otherwise multiply by out_scale (the backward's dQ = scale dS K,
// with p = dS, v = K, o = dQ).
template <int D, bool NORM>
__global__ __launch_bounds__(512) void std_pv_kernel(StdArgs a, const bf16* __restrict__ pm,
                                                     const bf16* __restrict__ vm,
                                                     bf16* __restrict__ om, float out_scale) {
  constexpr int BC = 64, DT = D / 32, KB = BC / 32, ROWB = D * 2, TILEB = BC * ROWB, CPR = D / 8;
  constexpr int CPT = BC * CPR / 512;
  __shared__ __attribute__((aligned(16))) char sV[2 * TILEB];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, l32 = lane & 31, h = lane >> 5;
  const int N = a.N;
  const int n_qt = (N + 255) / 256;
  const int bh = blockIdx.x / n_qt, qt = blockIdx.x % n_qt;
  const size_t base = (size_t)bh * N * D;
  const int qi = qt * 256 + wv * 32 + l32;
  const bf16* P = pm + ((size_t)bh * N + (qi < N ? qi : N - 1)) * a.ldp;
  const int n_tiles = (N + BC - 1) / BC;

  auto dma = [&](int t, int buf) {
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int slot = (wv * CPT + j) * 64;
      const int p = slot + lane;
      const int row = p / CPR;
      int gr = t * BC + row;
      gr = gr < N ? gr : N - 1;  // P is 0 for keys past N
      lds_dma16(vm + base + (size_t)gr * D + ((p % CPR) ^ swz_v16<D>(row)) * 8,
                lds_addr(sV + buf * TILEB + slot * 16));
    }
  };
  const int g16 = lane >> 4, s16 = lane & 15;
  const int tr_row = 4 * h + (s16 >> 2);
  const int tr_ch8 = 4 * (g16 & 1) + (s16 & 3);
  f32x16 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.f;
  float psum = 0.f;  // this lane's part of the row sum of the rounded P

  dma(0, 0);
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
  for (int t = 0; t < n_tiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < n_tiles) dma(t + 1, buf ^ 1);
    const char* sVb = sV + buf * TILEB;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int key = t * BC + kb * 32 + 16 * u + 4 * h;  // first key of this lane's two groups
        // rows hold ldp (a multiple of 8) entries, zero past N; key is a
        // multiple of 4, so each group of 4 is either inside the row or past it
        u32x2 lo = {0u, 0u}, hi = {0u, 0u};
        if (key < a.ldp) lo = *(const u32x2*)(P + key);
        if (key + 8 < a.ldp) hi = *(const u32x2*)(P + key + 8);
        const bf16x8 pb = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
        if constexpr (NORM) psum = sum_bf16x8(pb, psum);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const int rlo = kb * 32 + 16 * u + tr_row, rhi = rlo + 8;
          const int clo = ((dt * 8 + tr_ch8) ^ (swz_v16<D>(rlo) << 1)) * 8;
          const int chi = ((dt * 8 + tr_ch8) ^ (swz_v16<D>(rhi) << 1)) * 8;
          const i16x4 vlo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)(sVb + rlo * ROWB + clo));
          const i16x4 vhi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)(sVb + rhi * ROWB + chi));
          const bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(vlo, vhi, 0, 1, 2, 3, 4, 5, 6, 7));
          oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, oacc[dt], 0, 0, 0);
        }
      }
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
  }
  const float inv = NORM ? 1.f / pair_sum(psum) : out_scale;
  if (qi < N) {
    bf16* O = om + base + (size_t)qi * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        bf16x4 y;
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = (bf16)(oacc[dt][4 * r4 + e] * inv);
        *(bf16x4*)(O + dt * 32 + 8 * r4 + 4 * h) = y;
      }
  }
}

template <int D, int MASK>
static hipError_t launch_std_mask(const StdArgs& a, hipStream_t stream) {
  const long n_kt = (a.N + 127) / 128, n_qt = (a.N + 255) / 256;
  hipLaunchKernelGGL((std_scores_kernel<D, MASK>), dim3((unsigned)(n_kt * n_qt * a.BH)), dim3(512), 0,
                     stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(std_softmax_kernel, dim3((unsigned)((long)a.BH * a.N)), dim3(256), 0, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((std_pv_kernel<D, true>), dim3((unsigned)(n_qt * a.BH)), dim3(512), 0, stream, a,
                     (const bf16*)a.p, a.v, a.o, 1.f);
  return hipGetLastError();
}

// ---- standard backward, step 6: one workgroup per row: D_i = sum_j P_ij
// dP_ij (float32, reduced over the workgroup), then dS_ij = P_ij (dP_ij - D_i)
// as bf16 (rows padded to ldp with zeros).
__global__ __launch_bounds__(256) void std_ds_kernel(StdArgs a) {
  __shared__ float sd[4];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const size_t row = blockIdx.x;  // bh * N + i
  const int N = a.N;
  const float* dp = a.s + row * a.lds;
  const bf16* p = a.p + row * a.ldp;
  float acc = 0.f;
  for (int j = tid; j < N; j += 256) acc = __builtin_fmaf((float)p[j], dp[j], acc);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
  if (lane == 0) sd[wv] = acc;
  __syncthreads();
  const float Di = (sd[0] + sd[1]) + (sd[2] + sd[3]);
  bf16* ds = a.ds + row * a.ldp;
  for (int j = tid; j < a.ldp; j += 256)
    ds[j] = (bf16)(j < N ? (float)p[j] * (dp[j] - Di) : 0.f);
}

// ---- standard backward, steps 5 and 8: out = alpha X^T Y, i.e.
// out[j][c] = alpha sum_i X[i][j] Y[i][c], with X an N x N bf16 matrix of row
// stride ldp (P or dS) and Y an N x D bf16 matrix (dO or Q). Workgroup: 256
// output rows j (8 waves x 32); i runs over tiles of 32 rows staged in LDS
// (X: 32 x 256 columns, Y: 32 x D), both read transposed with
// ds_read_b64_tr_b16 so that i is the contraction index of
// out^T = Y^T X on v_mfma_f32_32x32x16_bf16: lane (j, half h) gets the rows
// 16u + 4h + {0..3} and 16u + 8 + 4h + {0..3} of its column from both tiles,
// the same row order, so the products pair up.
template <int D>
__global__ __launch_bounds__(512) void std_xty_kernel(StdArgs a, const bf16* __restrict__ X,
                                                      const bf16* __restrict__ Y,
                                                      bf16* __restrict__ out, float alpha) {
  constexpr int DT = D / 32, ROWY = D * 2, ROWX = 256 * 2, TI = 32;
  __shared__ __attribute__((aligned(16))) char sY[TI * ROWY];
  __shared__ __attribute__((aligned(16))) char sX[TI * ROWX];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, h = lane >> 5;
  const int N = a.N;
  const int n_jt = (N + 255) / 256;
  const int bh = blockIdx.x / n_jt, jt = blockIdx.x % n_jt;
  const int j0 = jt * 256;
  const bf16* Xh = X + (size_t)bh * N * a.ldp;
  const bf16* Yh = Y + (size_t)bh * N * D;
  const int g16 = lane >> 4, s16 = lane & 15;
  const int tr_row = 4 * h + (s16 >> 2);
  const int tr_ch8 = 4 * (g16 & 1) + (s16 & 3);
  f32x16 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[dt][r] = 0.f;
  for (int i0 = 0; i0 < N; i0 += TI) {
    // stage: Y rows i0.. (16-byte chunks, zero past N), X rows i0.., columns
    // j0..j0+255 (zero past the padded row length ldp)
    for (int c = tid; c < TI * D / 8; c += 512) {
      const int r = c / (D / 8), cc = c % (D / 8);
      u32x4 y = {0u, 0u, 0u, 0u};
      if (i0 + r < N) y = *(const u32x4*)(Yh + (size_t)(i0 + r) * D + cc * 8);
      *(u32x4*)(sY + r * ROWY + cc * 16) = y;
    }
    for (int c = tid; c < TI * 32; c += 512) {
      const int r = c / 32, cc = c % 32;
      u32x4 x = {0u, 0u, 0u, 0u};
      const int col = j0 + cc * 8;
      if (i0 + r < N && col < a.ldp) x = *(const u32x4*)(Xh + (size_t)(i0 + r) * a.ldp + col);
      *(u32x4*)(sX + r * ROWX + cc * 16) = x;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int rlo = 16 * u + tr_row, rhi = rlo + 8;
      const int xc = (wv * 8 + tr_ch8) * 8;  // this wave's 32 columns, in bytes
      const i16x4 xlo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)(sX + rlo * ROWX + xc));
      const i16x4 xhi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)(sX + rhi * ROWX + xc));
      const bf16x8 xb = __builtin_bit_cast(bf16x8, __builtin_shufflevector(xlo, xhi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int yc = (dt * 8 + tr_ch8) * 8;
        const i16x4 ylo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)(sY + rlo * ROWY + yc));
        const i16x4 yhi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)(sY + rhi * ROWY + yc));
        const bf16x8 ya = __builtin_bit_cast(bf16x8, __builtin_shufflevector(ylo, yhi, 0, 1, 2, 3, 4, 5, 6, 7));
        acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ya, xb, acc[dt], 0, 0, 0);
      }
    }
    __syncthreads();
  }
  const int j = j0 + wv * 32 + (lane & 31);
  if (j < N) {
    bf16* o = out + ((size_t)bh * N + j) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        bf16x4 y;
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = (bf16)(acc[dt][4 * r4 + e] * alpha);
        *(bf16x4*)(o + dt * 32 + 8 * r4 + 4 * h) = y;
      }
  }
}

template <int D>
static hipError_t launch_std_bwd_d(const StdArgs& a0, hipStream_t stream) {
  const long n_kt = (a0.N + 127) / 128, n_qt = (a0.N + 255) / 256;
  hipError_t e;
  // 4. dP = dO V^T: the score kernel with dO for Q, V for K, scale 1, no mask
  StdArgs a = a0;
  a.q = a0.dout;
  a.k = a0.v;
  a.scale = 1.f;
  hipLaunchKernelGGL((std_scores_kernel<D, MASK_NONE>), dim3((unsigned)(n_kt * n_qt * a.BH)), dim3(512), 0,
                     stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // 5. dV = P^T dO
  hipLaunchKernelGGL((std_xty_kernel<D>), dim3((unsigned)(n_qt * a0.BH)), dim3(512), 0, stream, a0,
                     (const bf16*)a0.p, a0.dout, a0.dv, 1.f);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // 6. D and dS
  hipLaunchKernelGGL(std_ds_kernel, dim3((unsigned)((long)a0.BH * a0.N)), dim3(256), 0, stream, a0);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // 7. dQ = scale dS K
  hipLaunchKernelGGL((std_pv_kernel<D, false>), dim3((unsigned)(n_qt * a0.BH)), dim3(512), 0, stream, a0,
                     (const bf16*)a0.ds, a0.k, a0.dq, a0.scale);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // 8. dK = scale dS^T Q
  hipLaunchKernelGGL((std_xty_kernel<D>), dim3((unsigned)(n_qt * a0.BH)), dim3(512), 0, stream, a0,
                     (const bf16*)a0.ds, a0.q, a0.dk, a0.scale);
  return hipGetLastError();
}

hipError_t launch_std_bwd_bf16(const StdArgs& a, int d, hipStream_t stream) {
  return d == 128 ? launch_std_bwd_d<128>(a, stream) : launch_std_bwd_d<64>(a, stream);
}

hipError_t launch_std_bf16(const StdArgs& a, int d, int mask, hipStream_t stream) {
  if (d == 128) {
    if (mask == MASK_CAUSAL) return launch_std_mask<128, MASK_CAUSAL>(a, stream);
    if (mask == MASK_LOCAL) return launch_std_mask<128, MASK_LOCAL>(a, stream);
    return launch_std_mask<128, MASK_NONE>(a, stream);
  }
  if (mask == MASK_CAUSAL) return launch_std_mask<64, MASK_CAUSAL>(a, stream);
  if (mask == MASK_LOCAL) return launch_std_mask<64, MASK_LOCAL>(a, stream);
  return launch_std_mask<64, MASK_NONE>(a, stream);
}

}  // namespace fa
