// Device-side helpers shared by the gfx950 kernels: block geometry, bf16
// conversion and wave-level reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vsa {

// Grid and block geometry passed by value to every kernel.
struct DGeo {
  int T, H, W;
  int bt, bh, bw;
  int nbt, nbh, nbw;
  int NB;
  int N;
  // ceil(2^32 / d) for d = nbh*nbw and d = nbw (0 encodes d = 1, whose
  // magic would not fit): for n, d < 2^16, umulhi(n, m) == n / d exactly
  // (n*d < 2^32 bounds the error below 1).
  uint32_t magic_hw, magic_w;
};

// n / d with a precomputed magic (see DGeo); n and d below 2^16.
__device__ inline int div_magic(int n, uint32_t magic) {
  return magic == 0u ? n : (int)(((uint64_t)(uint32_t)n * magic) >> 32);
}

// Box of block j using the magic divisions (block ids are below 2^16).
struct Box;
__device__ inline Box block_box_fast(const DGeo& g, int j);

// The 3D box of block j: origin (t0, h0, w0) and extents (et, eh, ew); edge
// blocks of a dimension that the box does not divide are cut short.
struct Box {
  int t0, h0, w0;
  int et, eh, ew;
  __device__ int n() const { return et * eh * ew; }
};

__device__ inline Box block_box(const DGeo& g, int j) {
  int per_t = g.nbh * g.nbw;
  int tb = j / per_t, r = j - tb * per_t;
  int hb = r / g.nbw, wb = r - hb * g.nbw;
  Box b;
  b.t0 = tb * g.bt; b.h0 = hb * g.bh; b.w0 = wb * g.bw;
  b.et = min(g.bt, g.T - b.t0);
  b.eh = min(g.bh, g.H - b.h0);
  b.ew = min(g.bw, g.W - b.w0);
  return b;
}

__device__ inline Box block_box_fast(const DGeo& g, int j) {
  const int tb = div_magic(j, g.magic_hw), r = j - tb * (g.nbh * g.nbw);
  const int hb = div_magic(r, g.magic_w), wb = r - hb * g.nbw;
  Box b;
  b.t0 = tb * g.bt; b.h0 = hb * g.bh; b.w0 = wb * g.bw;
  b.et = min(g.bt, g.T - b.t0);
  b.eh = min(g.bh, g.H - b.h0);
  b.ew = min(g.bw, g.W - b.w0);
  return b;
}

// Raster index of the u-th token (row-major (t, h, w) inside the box) of a
// block.  The two divisions use a float reciprocal: for u < 128 and
// extents <= 128 the quotient (u + 0.5) / e is at least 2^-8 away from an
// integer while the float error is below 2^-16, so the floor is exact.
struct TokenMap {
  int base;        // raster index of the box origin
  int ehw, ew;
  float inv_ehw, inv_ew;
  int HW, W;
  __device__ void init(const DGeo& g, const Box& b) {
    base = (b.t0 * g.H + b.h0) * g.W + b.w0;
    ehw = b.eh * b.ew; ew = b.ew;
    inv_ehw = 1.0f / (float)ehw; inv_ew = 1.0f / (float)ew;
    HW = g.H * g.W; W = g.W;
  }
  __device__ int operator()(int u) const {
    int ut = (int)(((float)u + 0.5f) * inv_ehw);
    int rem = u - ut * ehw;
    int uh = (int)(((float)rem + 0.5f) * inv_ew);
    int uw = rem - uh * ew;
    return base + ut * HW + uh * W + uw;
  }
};

__device__ inline float bf16_lo(uint32_t two) { return __uint_as_float(two << 16); }
__device__ inline float bf16_hi(uint32_t two) { return __uint_as_float(two & 0xffff0000u); }
__device__ inline float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// float -> bf16 bits, round to nearest even (finite inputs).
__device__ inline uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ inline int wave_sum(int v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__device__ inline uint64_t lanemask_lt() {
  int lane = threadIdx.x & 63;
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

}  // namespace vsa
