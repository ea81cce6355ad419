// Device helpers shared by the forward kernels (query-major and key-major)
// and the query-major dQ kernel: LDS swizzles of K/V tiles, the lane-pair
// reductions of the transposed score layout, and the max / sum trees over one
// 32-key accumulator block.
#pragma once
#include "fa_common.h"

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


// Rescale threshold, in exp2 units, for the lazily refreshed maximum.
constexpr float RESCALE_LOG2 = 8.0f;

// v_permlane32_swap(a, b) exchanges the upper 32 lanes of a with the lower
// 32 lanes of b. With b = a it returns {a of lanes 0..31 in both halves,
// a of lanes 32..63 in both halves}, so a symmetric operation over the two
// results gives lanes l and l^32 the same, bit-identical value. (The two
// results are copied to plain scalars before reinterpretation: applying
// __builtin_bit_cast to an element of the returned vector directly has been
// seen to read element 0 twice.)
__device__ __forceinline__ void halves(float x, float& lo, float& hi) {
  const unsigned u = __float_as_uint(x);
  auto sw = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const unsigned a0 = sw[0];
  const unsigned a1 = sw[1];
  lo = __uint_as_float(a0);
  hi = __uint_as_float(a1);
}
__device__ __forceinline__ float pair_max(float x) {
  float lo, hi;
  halves(x, lo, hi);
  return fmaxf(lo, hi);
}
__device__ __forceinline__ float pair_sum(float x) {
  float lo, hi;
  halves(x, lo, hi);
  return lo + hi;
}

__device__ __forceinline__ float max16(const f32x16& v) {
  const float t0 = fmaxf(fmaxf(v[0], v[1]), v[2]);
  const float t1 = fmaxf(fmaxf(v[3], v[4]), v[5]);
  const float t2 = fmaxf(fmaxf(v[6], v[7]), v[8]);
  const float t3 = fmaxf(fmaxf(v[9], v[10]), v[11]);
  const float t4 = fmaxf(fmaxf(v[12], v[13]), v[14]);
  return fmaxf(fmaxf(fmaxf(t0, t1), t2), fmaxf(fmaxf(t3, t4), v[15]));
}

// Pairwise (depth-4) float32 sum of 16 accumulator values.
__device__ __forceinline__ float sum16(const f32x16& v) {
  const float a0 = (v[0] + v[1]) + (v[2] + v[3]);
  const float a1 = (v[4] + v[5]) + (v[6] + v[7]);
  const float a2 = (v[8] + v[9]) + (v[10] + v[11]);
  const float a3 = (v[12] + v[13]) + (v[14] + v[15]);
  return (a0 + a1) + (a2 + a3);
}

// Sum of the 16 bf16 weights of one 32-key block's P operand (two bf16x8),
// added to acc with v_dot2c_f32_bf16 against (1, 1): the weights exactly as
// the P V product uses them. Normalizing the output by this sum, rather than
// by the float32 sum of the unrounded weights, makes each output row a convex
// combination of value rows with the rounded weights; with the lazily
// refreshed reference the dominant weight of a peaked row is a non-power of
// two whose bf16 rounding would otherwise show as a relative error of up to
// 2^-9 of the output.
// (The pairs are taken with shufflevector: bit-casting the vector to four
// dwords and each dword back to a bf16 pair has been compiled into four reads
// of the first pair.)
__device__ __forceinline__ float sum_bf16x8(const bf16x8& p, float acc) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 one = __builtin_bit_cast(bf16x2, 0x3f803f80u);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p, p, 0, 1), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p, p, 2, 3), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p, p, 4, 5), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p, p, 6, 7), one, acc, false);
  return acc;
}
__device__ __forceinline__ float sum_bf16x16(const bf16x8 (&p)[2], float acc) {
  return sum_bf16x8(p[1], sum_bf16x8(p[0], acc));
}
// The same sum spread over four running accumulators (pair i of each bf16x8
// into acc[i]), so that no two dependent dot products sit next to each other
// in a wave's instruction stream: a single chain stalls the in-order issue,
// and with it the next matrix instruction.
__device__ __forceinline__ void sum_bf16x16_4(const bf16x8 (&p)[2], float (&acc)[4]) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 one = __builtin_bit_cast(bf16x2, 0x3f803f80u);
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    acc[0] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p[u], p[u], 0, 1), one, acc[0], false);
    acc[1] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p[u], p[u], 2, 3), one, acc[1], false);
    acc[2] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p[u], p[u], 4, 5), one, acc[2], false);
    acc[3] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p[u], p[u], 6, 7), one, acc[3], false);
  }
}

// Offset of accumulator register r within a 32-key block, for the lanes of
// the lower half (the upper half adds 4): key = 8 (r / 4) + (r % 4).
__device__ __forceinline__ constexpr int acc_key(int r) { return 8 * (r >> 2) + (r & 3); }

}  // namespace fa
