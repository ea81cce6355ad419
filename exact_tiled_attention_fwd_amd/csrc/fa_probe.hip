// Roofline probes: sustained bf16 MFMA rate and HBM copy bandwidth of the
// current device (declared in fa_probe.h).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_common.h"
#include "fa_probe.h"

namespace fa {

// Written only when an accumulator takes a value it cannot take, so the
// compiler has to keep every MFMA.
__device__ float probe_sink;

// Operands are full-entropy bf16 values (random sign, exponent near 1 and
// 7 random mantissa bits from an integer hash), four A and four B sets that
// the MFMAs cycle through: the matrix cores draw as much power as on
// attention's random data, so the sustained clock is the one attention sees.
__device__ __forceinline__ bf16 probe_value(unsigned x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  const unsigned short bits = (unsigned short)(((x & 1u) << 15) | ((126u + ((x >> 1) & 1u)) << 7) |
                                               ((x >> 2) & 0x7fu));
  return __builtin_bit_cast(bf16, bits);
}

__global__ __launch_bounds__(256) void probe_mfma_kernel(int iters) {
  bf16x8 a[4], b[4];
  const unsigned t = blockIdx.x * 256u + threadIdx.x;
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[s][i] = probe_value(t * 64u + s * 8u + i);
      b[s][i] = probe_value(t * 64u + 32u + s * 8u + i);
    }
  f32x16 c[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) c[j][r] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      c[j & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j & 3], b[(j + (j >> 2)) & 3], c[j & 3], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += c[j][r];
  if (s == -1.2345e-30f) probe_sink = s;
}

// Grid-stride copy with 16-byte non-temporal loads and stores, four
// workgroups of 256 threads per compute unit: the fastest of the copy forms
// measured on a 1 GiB buffer (6.16 TB/s, against 4.6-5.7 TB/s for plain
// loads and stores at 2-16 workgroups per compute unit, unrolled loops or
// contiguous per-workgroup chunks).
__global__ __launch_bounds__(256) void probe_copy_kernel(const u32x4* __restrict__ src,
                                                         u32x4* __restrict__ dst, size_t n) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

}  // namespace fa

namespace {

// Times `launch` (which enqueues on s) with events on s; waits for it.
template <typename F>
fa_status timed(hipStream_t s, F launch, float* ms) {
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess) return FA_ERR_LAUNCH;
  if (hipEventCreate(&e1) != hipSuccess) {
    (void)hipEventDestroy(e0);
    return FA_ERR_LAUNCH;
  }
  fa_status st = FA_OK;
  if (hipEventRecord(e0, s) != hipSuccess || !launch() || hipEventRecord(e1, s) != hipSuccess ||
      hipEventSynchronize(e1) != hipSuccess || hipEventElapsedTime(ms, e0, e1) != hipSuccess)
    st = FA_ERR_LAUNCH;
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  return st;
}

int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return cus;
}

}  // namespace

extern "C" fa_status fa_probe_mfma_bf16(int iters, void* stream, double* tflops) {
  if (!tflops) return FA_ERR_NULL;
  if (iters < 1 || iters > (1 << 24)) return FA_ERR_SHAPE;
  const int cus = device_cus();
  if (cus < 1) return FA_ERR_LAUNCH;
  hipStream_t s = (hipStream_t)stream;
  const int blocks = 2 * cus;  // 8 waves per compute unit, two per SIMD
  float ms = 0.f;
  const fa_status st = timed(s, [&] {
    hipLaunchKernelGGL(fa::probe_mfma_kernel, dim3(blocks), dim3(256), 0, s, iters);
    return hipGetLastError() == hipSuccess;
  }, &ms);
  if (st != FA_OK) return st;
  if (ms <= 0.f) return FA_ERR_LAUNCH;
  const double flops = 2.0 * 32 * 32 * 16 * 8.0 * iters * (blocks * 4.0);
  *tflops = flops / (ms * 1e-3) / 1e12;
  return FA_OK;
}

extern "C" fa_status fa_probe_copy(const void* src, void* dst, size_t bytes, int reps, void* stream,
                                   double* gbs) {
  if (!src || !dst || !gbs) return FA_ERR_NULL;
  if (bytes == 0 || reps < 1) return FA_ERR_SHAPE;
  if ((bytes & 15) || ((uintptr_t)src & 15) || ((uintptr_t)dst & 15)) return FA_ERR_ALIGN;
  const uintptr_t a = (uintptr_t)src, b = (uintptr_t)dst;
  if (a < b + bytes && b < a + bytes) return FA_ERR_ALIAS;
  const int cus = device_cus();
  if (cus < 1) return FA_ERR_LAUNCH;
  hipStream_t s = (hipStream_t)stream;
  const size_t n = bytes / 16;
  const int blocks = 4 * cus;
  float ms = 0.f;
  const fa_status st = timed(s, [&] {
    for (int r = 0; r < reps; ++r) {
      hipLaunchKernelGGL(fa::probe_copy_kernel, dim3(blocks), dim3(256), 0, s, (const u32x4*)src,
                         (u32x4*)dst, n);
      if (hipGetLastError() != hipSuccess) return false;
    }
    return true;
  }, &ms);
  if (st != FA_OK) return st;
  if (ms <= 0.f) return FA_ERR_LAUNCH;
  *gbs = 2.0 * (double)bytes * reps / (ms * 1e-3) / 1e9;
  return FA_OK;
}
