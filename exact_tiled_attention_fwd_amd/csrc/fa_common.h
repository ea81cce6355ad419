// Shared device types and helpers for the gfx950 attention kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

#define FA_LDS __attribute__((address_space(3)))

namespace fa {

// 32-bit LDS address of a pointer into __shared__ memory.
__device__ __forceinline__ unsigned lds_addr(const void* p) {
  return (unsigned)(size_t)(FA_LDS const char*)p;
}

// The copies below set M0 (the LDS destination of global_load_lds_*) inside
// their assembly. The kernels keep no value of their own in M0 (none of their
// LDS instructions reads it), so the compiler's note that a clobbered reserved
// register may not be preserved across the statement does not apply.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"

// Direct global -> LDS copy of 16 bytes per lane (global_load_lds_dwordx4):
// lane i's chunk lands at lds_base + 16 i, lds_base wave-uniform (M0).
// Issued as inline assembly so that the compiler does not make later LDS
// reads of other buffers wait for it; callers wait with vmcnt(0) themselves
// before the barrier that publishes the data.
__device__ __forceinline__ void lds_dma16(const void* gptr, unsigned lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds_base)), "v"(gptr)
               : "memory", "m0");
}

// The same copy addressed as a wave-uniform 64-bit base (SGPR pair) plus a
// per-lane 32-bit byte offset: no per-lane 64-bit address arithmetic, and
// the offsets of a tile can be computed once and reused for every tile.
__device__ __forceinline__ void lds_dma16_s(const void* sbase, unsigned voff, unsigned lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds_base)), "v"(voff), "s"(sbase)
               : "memory", "m0");
}

#pragma clang diagnostic pop

// Workgroup id -> (head, tile rank); rank 0 is launched first.
// Workgroup ids are handed to the eight XCDs round-robin, so id w is the
// (w / 8)-th workgroup that XCD x = w % 8 runs. When the heads split evenly
// over the XCDs, every XCD gets a contiguous run of heads (their K/V stay in
// that XCD's L2) and walks them rank-major: rank 0 of each of its heads,
// then rank 1, ... so that the longest tiles of all its heads start first
// and the short ones fill in at the end. Otherwise the ids map head-major,
// which spreads each head's ranks over all XCDs.
__device__ __forceinline__ void wg_tile(int w, int BH, int ntiles, int& bh, int& rank) {
  const int total = BH * ntiles;
  const int per = total >> 3;
  if ((total & 7) == 0 && per % ntiles == 0) {
    const int hx = per / ntiles;  // heads per XCD
    const int x = w & 7, j = w >> 3;
    bh = x * hx + j % hx;
    rank = j / hx;
    return;
  }
  bh = w / ntiles;
  rank = w - bh * ntiles;
}

// Compile-time integer tag for generic lambdas.
template <int V>
struct ic {
  static constexpr int value = V;
};

// Mask modes, mirroring fa_mask.
enum : int { MASK_NONE = 0, MASK_CAUSAL = 1, MASK_LOCAL = 2 };

// Whether key j takes part in query i's softmax (same predicate as the
// C-ABI documents: causal j <= i, band |i - j| <= window).
template <int MASK>
__device__ __forceinline__ bool allowed(int i, int j, int window) {
  if constexpr (MASK == MASK_CAUSAL) return j <= i;
  else if constexpr (MASK == MASK_LOCAL) return (i - j <= window) && (j - i <= window);
  else return true;
}

// Key range [lo, hi) any query of [q0, q1) can see under the mask.
template <int MASK>
__device__ __forceinline__ void key_range(int q0, int q1, int N, int window, int& lo, int& hi) {
  lo = 0;
  hi = N;
  if constexpr (MASK == MASK_CAUSAL) hi = q1 < N ? q1 : N;
  if constexpr (MASK == MASK_LOCAL) {
    lo = q0 - window > 0 ? q0 - window : 0;
    long long h = (long long)q1 + window;  // last query q1-1 sees keys <= q1-1+window
    hi = h < N ? (int)h : N;
  }
}

// Visiting order of a workgroup's key tiles under the band mask. A
// workgroup of br query rows starting at a multiple of br needs the
// p = ceil((br + window) / bc) + ceil(window / bc) key tiles around its rows
// (fewer at the sequence ends), and its neighbours need most of the same
// tiles. Walked from its own first tile, a workgroup reaches a tile some
// steps after its neighbour did, by which time the L2 of an XCD running
// ~160 such workgroups has evicted it. Walked instead by tile index modulo
// p, starting at the tile whose index is a multiple of p (a rotation of the
// contiguous range), every workgroup reads tile t at step t mod p, so
// neighbours that run together read each shared tile together. Returns the
// rotation, in tiles, of the range [t_begin, t_begin + n_t).
__device__ __forceinline__ int band_tile_rotation(int br, int bc, int window, int t_begin, int n_t) {
  const int p = (br + window + bc - 1) / bc + (window + bc - 1) / bc;
  const int first = (p - t_begin % p) % p;  // first tile index that is a multiple of p
  return first < n_t ? first : 0;
}

// Whether every (query, key) pair with query in [q0, q1) and key in
// [k0, k1) is allowed (so the tile needs no per-element mask).
template <int MASK>
__device__ __forceinline__ bool tile_full(int q0, int q1, int k0, int k1, int window) {
  if constexpr (MASK == MASK_CAUSAL) return k1 - 1 <= q0;
  else if constexpr (MASK == MASK_LOCAL) {
    int a = (q1 - 1) - k0, b = (k1 - 1) - q0;
    return (a > b ? a : b) <= window;
  } else return true;
}

}  // namespace fa
