// Scheme generation for gfx950: intra-block aggregation and head-wise
// blocking-scheme selection (SPADE arXiv 2608.03335, 3.2 Schemes
// Generation, Eq. 3-5 and Algorithm 1).
//
// SICS of a block is the sum of all pairwise cosine similarities of its
// token vectors; by Eq. 5 it equals ||sum of the unit-normalized tokens||^2,
// which is what the kernel accumulates (one pass over the tensor, so the
// step is HBM-bound).  A zero token normalizes to zero and adds nothing.
// A scheme's aggregation score is the sum of its blocks' SICS (Eq. 3); a
// head's score for a candidate is AS(Q) + AS(K), and the head selects the
// first candidate with the highest score.
#include <hip/hip_runtime.h>

#include "vsa_device.h"
#include "vsa_kernels.h"

namespace vsa {

__device__ inline int sics_uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ inline __amdgpu_buffer_rsrc_t sics_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(((uint64_t)hi << 32) | lo), (short)0,
                                           (int)bytes, 0x00020000);
}

// ---------------------------------------------------------------------------
// Per-block SICS.  One wave per (tensor, row bh, block j).  A token row is
// split over LPT lanes of 16 bytes (CPL channels each), so one load
// instruction covers TPI tokens; UN instructions are in flight.  Each
// token's squared norm is reduced over its LPT lanes, the token is scaled
// by 1/norm and added to the lane's running channel sums; at the end the
// sums of the TPI token slots are combined and squared.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void sics_kernel(const T* __restrict__ x0, float* __restrict__ out0,
                                                   const T* __restrict__ x1, float* __restrict__ out1,
                                                   DGeo g, int nitems) {
  constexpr int EB = (int)sizeof(T);
  constexpr int CPL = 16 / EB;      // channels per lane
  constexpr int LPT = D / CPL;      // lanes per token
  constexpr int TPI = 64 / LPT;     // tokens per load instruction
  constexpr int UN = 4;             // load instructions in flight
  static_assert(LPT >= 1 && LPT <= 64 && (64 % LPT) == 0, "a token must fill whole lane groups");
  const int wave = sics_uniform(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int item = blockIdx.x * 4 + wave;
  if (item >= nitems) return;
  const T* x = blockIdx.y ? x1 : x0;
  float* out = blockIdx.y ? out1 : out0;
  const int bh = item / g.NB, j = item - bh * g.NB;
  const Box b = block_box(g, j);
  const int n = sics_uniform(b.n());
  TokenMap map;
  map.init(g, b);
  const __amdgpu_buffer_rsrc_t rs = sics_rsrc(x + (size_t)bh * g.N * D, (uint32_t)g.N * D * EB);
  const int slot = lane / LPT, cl = lane % LPT;

  float r[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) r[c] = 0.0f;
  for (int u0 = 0; u0 < n; u0 += TPI * UN) {
    uint32_t raw[UN][4];
#pragma unroll
    for (int e = 0; e < UN; ++e) {
      const int u = u0 + e * TPI + slot;
      const int off = u < n ? map(u) * (D * EB) + cl * 16 : (int)0x80000000;   // past the block: zeros
      const auto v4 = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
#pragma unroll
      for (int w = 0; w < 4; ++w) raw[e][w] = v4[w];
    }
#pragma unroll
    for (int e = 0; e < UN; ++e) {
      float v[CPL];
      if constexpr (EB == 2) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          v[2 * w] = bf16_lo(raw[e][w]);
          v[2 * w + 1] = bf16_hi(raw[e][w]);
        }
      } else {
#pragma unroll
        for (int w = 0; w < 4; ++w) v[w] = __uint_as_float(raw[e][w]);
      }
      float sq = 0.0f;
#pragma unroll
      for (int c = 0; c < CPL; ++c) sq += v[c] * v[c];
#pragma unroll
      for (int m = 1; m < LPT; m <<= 1) sq += __shfl_xor(sq, m, 64);
      const float inv = sq > 0.0f ? __builtin_amdgcn_rsqf(sq) : 0.0f;
#pragma unroll
      for (int c = 0; c < CPL; ++c) r[c] += v[c] * inv;
    }
  }
  // Combine the token slots, then square and sum the channels.
#pragma unroll
  for (int m = LPT; m < 64; m <<= 1)
#pragma unroll
    for (int c = 0; c < CPL; ++c) r[c] += __shfl_xor(r[c], m, 64);
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < CPL; ++c) s += r[c] * r[c];
#pragma unroll
  for (int m = 1; m < LPT; m <<= 1) s += __shfl_xor(s, m, 64);
  if (lane == 0) out[item] = s;
}

// ---------------------------------------------------------------------------
// Aggregation scores and selection.  One workgroup per row bh, one wave per
// candidate: AS(Q) and AS(K) are sums over that candidate's block SICS in a
// fixed order (lane-strided partial sums, then a butterfly), so the result
// and the choice are reproducible; after a barrier one thread takes the
// first candidate with the highest AS(Q) + AS(K).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64 * VSA_MAX_SCHEMES) void scheme_select_kernel(const float* __restrict__ sics,
                                                                             SchemeArgs sa, int BH,
                                                                             float* __restrict__ scores,
                                                                             int32_t* __restrict__ choice) {
  __shared__ float sc_s[VSA_MAX_SCHEMES];
  const int bh = blockIdx.x, lane = threadIdx.x & 63, c = threadIdx.x >> 6;
  if (c < sa.n) {
    const int nb = sa.nb[c];
    float tot[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const float* src = sics + sa.off[c] + ((size_t)t * BH + bh) * nb;
      float a = 0.0f;
      for (int jj = lane; jj < nb; jj += 64) a += src[jj];
#pragma unroll
      for (int m = 32; m > 0; m >>= 1) a += __shfl_xor(a, m, 64);
      tot[t] = a;
    }
    const float sc = tot[0] + tot[1];
    if (lane == 0) {
      scores[(size_t)c * BH + bh] = sc;
      sc_s[c] = sc;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float best = -INFINITY;
    int best_c = 0;
    for (int k = 0; k < sa.n; ++k) {
      if (sc_s[k] > best) {
        best = sc_s[k];
        best_c = k;
      }
    }
    choice[bh] = best_c;
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_sics(const void* x0, float* out0, const void* x1, float* out1, int dtype, int D,
                       const DGeo& g, int BH, hipStream_t st) {
  const int nitems = BH * g.NB;
  dim3 grid((nitems + 3) / 4, x1 ? 2 : 1), block(256);
  if (dtype == 0) {
    if (D == 128)
      hipLaunchKernelGGL((sics_kernel<uint16_t, 128>), grid, block, 0, st, (const uint16_t*)x0, out0,
                         (const uint16_t*)x1, out1, g, nitems);
    else
      hipLaunchKernelGGL((sics_kernel<uint16_t, 64>), grid, block, 0, st, (const uint16_t*)x0, out0,
                         (const uint16_t*)x1, out1, g, nitems);
  } else {
    if (D == 128)
      hipLaunchKernelGGL((sics_kernel<float, 128>), grid, block, 0, st, (const float*)x0, out0,
                         (const float*)x1, out1, g, nitems);
    else
      hipLaunchKernelGGL((sics_kernel<float, 64>), grid, block, 0, st, (const float*)x0, out0,
                         (const float*)x1, out1, g, nitems);
  }
  return hipGetLastError();
}

hipError_t launch_scheme_select(const float* sics, const SchemeArgs& sa, int BH, float* scores, int32_t* choice,
                                hipStream_t st) {
  hipLaunchKernelGGL(scheme_select_kernel, dim3(BH), dim3(64 * sa.n), 0, st, sics, sa, BH, scores, choice);
  return hipGetLastError();
}

}  // namespace vsa
