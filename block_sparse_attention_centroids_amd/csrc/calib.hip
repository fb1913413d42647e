// Sustained bf16 matrix-core rate of the GPU the library runs on.
//
// Not a step of the attention path: a measurement aid.  The attention
// kernel's rate is quoted against the chip's dense bf16 peak, which assumes
// every SIMD issues a 32x32x16 MFMA every 32 cycles at 2.4 GHz.  Whether a
// card can hold that clock depends on power, and power depends on the data
// the matrix cores switch.  This kernel issues nothing but MFMAs on operands
// that stay in registers (no memory traffic after the first loads, no LDS,
// no vector ALU work in the loop), so its rate on data of a given spread is
// a practical ceiling for bf16 MFMA work on such data on the same card:
// anything else a kernel does draws on the same power budget.
//
// Layout of a wave's work: 8 A and 8 B fragments of v_mfma_f32_32x32x16_bf16
// (8 bf16 per lane each) loaded once from a 4 MiB pool, then `iters` rounds
// of 16 MFMAs cycling through the fragments into 4 independent accumulators.
// Each thread writes the sum of its accumulator elements, so the work cannot
// be dropped and a test can check it: summed over a wave's 64 lanes that is
// the sum of every entry of the 16 * iters products.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "vsa.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kPoolFragments = 4096;   // fragments of 64 lanes x 16 bytes
constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void mfma_rate_kernel(const u32x4_t* __restrict__ pool, float* __restrict__ out, int iters) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  // Fragments f = (16 * (4 * block + wave) + j) mod 4096: every wave of a
  // launch starts from its own slice of the pool.
  const int base = 16 * (4 * (int)blockIdx.x + wave);
  bf16x8_t a[8], b[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = __builtin_bit_cast(bf16x8_t, pool[((base + j) % kPoolFragments) * 64 + lane]);
    b[j] = __builtin_bit_cast(bf16x8_t, pool[((base + 8 + j) % kPoolFragments) * 64 + lane]);
  }
  f32x16_t acc[4];
#pragma unroll
  for (int x = 0; x < 4; ++x) acc[x] = f32x16_t{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      acc[j & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j], b[(j + 3) & 7], acc[j & 3], 0, 0, 0);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      acc[j & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(j + 5) & 7], b[j], acc[j & 3], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[x][r];
  out[(size_t)blockIdx.x * kThreads + threadIdx.x] = s;
}

}  // namespace

extern "C" vsa_status vsa_calib_mfma_bf16(const void* pool, size_t pool_bytes, float* out, int n_workgroups,
                                          int iters, void* stream) {
  if (!pool || !out) return VSA_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(pool) % 16 != 0 || reinterpret_cast<uintptr_t>(out) % 4 != 0)
    return VSA_ERR_INVALID_ARG;
  if (pool_bytes < VSA_CALIB_POOL_BYTES) return VSA_ERR_INVALID_ARG;
  if (n_workgroups < 1 || n_workgroups > VSA_CALIB_MAX_WORKGROUPS) return VSA_ERR_INVALID_ARG;
  if (iters < 1 || iters > VSA_CALIB_MAX_ITERS) return VSA_ERR_INVALID_ARG;
  mfma_rate_kernel<<<n_workgroups, kThreads, 0, reinterpret_cast<hipStream_t>(stream)>>>(
      static_cast<const u32x4_t*>(pool), out, iters);
  return hipGetLastError() == hipSuccess ? VSA_OK : VSA_ERR_HIP;
}
