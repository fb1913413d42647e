// Block-sparse flash attention for gfx950 (SPADE arXiv 2608.03335, 2.2 Eq. 2
// and 3.3): for each query block, only the key blocks listed in its CSR row
// are visited, with an online softmax, and the output is written straight
// back to raster order (the layout restore of 3.3 is fused into the store;
// the gather into the blocked layout is fused into the loads).
//
// bf16 path.  One workgroup of 4 waves per (batch*head, query block); wave w
// owns query tokens [32w, 32w+32) of the block.  Per 64-key stage:
//   S^T (keys x queries) = K Q^T     on v_mfma_f32_32x32x16_bf16, Q in VGPRs,
//                                    K from LDS ([key][d], padded rows)
//   online softmax in float32        the lane owns one query column, so the
//                                    row max/sum are in-lane plus one swap
//                                    with the lane 32 away
//   O^T (d x queries) += V^T P^T     V^T from LDS ([d][key], transposed on
//                                    the way in), P^T straight from the S^T
//                                    accumulators (same lane, same keys)
// K/V stages are loaded into registers one stage ahead, so global latency
// overlaps the matrix work of the current stage.
#include <hip/hip_runtime.h>

#include <math.h>

#include "vsa_device.h"
#include "vsa_kernels.h"

namespace vsa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int KT = 64;        // keys per stage
constexpr int VT_LD = KT + 4; // V^T row pitch in bf16 (136 B: conflict-free b64 reads)

template <int D>
struct AttnCfg {
  static constexpr int KS_LD = D + 8;            // K row pitch in bf16 (16 B pad)
  static constexpr int PARTS = D / 8;            // 16-byte pieces per token row
  static constexpr int KPT = KT * PARTS / 256;   // K pieces per thread per stage
  static constexpr int KROWS = 256 / PARTS;      // K rows covered per pass
  static constexpr int VGROUPS = (KT / 4) * PARTS;  // (4 keys x 8 d) groups per stage
};

__device__ inline uint32_t bf16_pair(uint16_t lo, uint16_t hi) { return (uint32_t)lo | ((uint32_t)hi << 16); }

__device__ inline uint16_t u4_elem(const u32x4_t& v, int e) {
  const uint32_t w = v[e >> 1];
  return (e & 1) ? (uint16_t)(w >> 16) : (uint16_t)(w & 0xffffu);
}

template <int D>
__global__ __launch_bounds__(256, 2) void attn_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    uint16_t* __restrict__ o, const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx,
    DGeo g, float scale_log2) {
  using C = AttnCfg<D>;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[KT * C::KS_LD];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[D * VT_LD];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, g2 = lane >> 5;

  // Workgroups are dealt round-robin to the 8 XCDs; give each XCD a
  // contiguous range of (head, query block) items so that neighbouring
  // query blocks of a head, which keep overlapping key blocks, share an L2.
  const int nwg = gridDim.x;
  const int xcd = blockIdx.x & 7, loc = blockIdx.x >> 3;
  const int per = (nwg + 7) >> 3, rem = nwg & 7;
  const int logical = (rem == 0 || xcd < rem) ? xcd * per + loc : rem * per + (xcd - rem) * (per - 1) + loc;

  const int bh = logical / g.NB, i = logical - bh * g.NB;
  const Box bi = block_box(g, i);
  const int ni = bi.n();
  TokenMap qmap;
  qmap.init(g, bi);
  const size_t head_off = (size_t)bh * g.N * D;
  const uint16_t* kh = k + head_off;
  const uint16_t* vh = v + head_off;

  // Q^T fragments (B operand): query column l32, channels 16*ks + 8*g2 + [0, 8).
  const int qtok = wave * 32 + l32;
  const bool wave_active = wave * 32 < ni;
  bf16x8_t qf[D / 16];
  {
    const bool ok = qtok < ni;
    const uint16_t* qp = q + head_off + (size_t)(ok ? qmap(qtok) : 0) * D + g2 * 8;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      u32x4_t raw = ok ? *reinterpret_cast<const u32x4_t*>(qp + ks * 16) : u32x4_t{0u, 0u, 0u, 0u};
      qf[ks] = __builtin_bit_cast(bf16x8_t, raw);
    }
  }

  f32x16_t acc[D / 32];
#pragma unroll
  for (int c = 0; c < D / 32; ++c) acc[c] = f32x16_t{};
  float m_run = -INFINITY, l_run = 0.0f;

  const int row = bh * g.NB + i;
  const int e0 = row_ptr[row], e1 = row_ptr[row + 1];

  // Loader roles.  K: piece p of this thread covers key (tid / PARTS) +
  // KROWS * p, bytes [16 * (tid % PARTS), +16).  V: keys 4*kg .. 4*kg+3 at
  // channels 8*dpart .. 8*dpart+7, written transposed.
  const int kpart = tid % C::PARTS, krow0 = tid / C::PARTS;
  const int vkg = tid & 15, vdpart = tid >> 4;
  const bool vloader = tid < C::VGROUPS;
  u32x4_t kreg[C::KPT], vreg[4];

  int e = e0, c0 = 0;
  int j = 0, nj = 0, nvalid = 0;
  TokenMap kmap;
  auto fetch = [&](int jj, int cstart, int nv) {
#pragma unroll
    for (int p = 0; p < C::KPT; ++p) {
      const int key = krow0 + C::KROWS * p;
      kreg[p] = key < nv ? *reinterpret_cast<const u32x4_t*>(kh + (size_t)kmap(cstart + key) * D + kpart * 8)
                         : u32x4_t{0u, 0u, 0u, 0u};
    }
    if (vloader) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = vkg * 4 + r;
        vreg[r] = key < nv ? *reinterpret_cast<const u32x4_t*>(vh + (size_t)kmap(cstart + key) * D + vdpart * 8)
                           : u32x4_t{0u, 0u, 0u, 0u};
      }
    }
    (void)jj;
  };

  // A corrupt index must not send loads out of bounds: block ids are clamped.
  if (e < e1) {
    j = min(max(col_idx[e], 0), g.NB - 1);
    const Box bj = block_box(g, j);
    nj = bj.n();
    kmap.init(g, bj);
    nvalid = min(KT, nj);
    fetch(j, 0, nvalid);
  }

  while (e < e1) {
    const int nv_cur = nvalid;
    __syncthreads();   // every wave is done with the previous stage
#pragma unroll
    for (int p = 0; p < C::KPT; ++p)
      *reinterpret_cast<u32x4_t*>(&Ks[(krow0 + C::KROWS * p) * C::KS_LD + kpart * 8]) = kreg[p];
    if (vloader) {
#pragma unroll
      for (int dd = 0; dd < 8; ++dd) {
        u32x2_t w;
        w[0] = bf16_pair(u4_elem(vreg[0], dd), u4_elem(vreg[1], dd));
        w[1] = bf16_pair(u4_elem(vreg[2], dd), u4_elem(vreg[3], dd));
        *reinterpret_cast<u32x2_t*>(&Vt[(vdpart * 8 + dd) * VT_LD + vkg * 4]) = w;
      }
    }
    __syncthreads();

    // Advance and prefetch the next stage.
    int e_next = e, c_next = c0 + KT;
    if (c_next >= nj) { e_next = e + 1; c_next = 0; }
    if (e_next < e1) {
      if (e_next != e) {
        j = min(max(col_idx[e_next], 0), g.NB - 1);
        const Box bj = block_box(g, j);
        nj = bj.n();
        kmap.init(g, bj);
      }
      nvalid = min(KT, nj - c_next);
      fetch(j, c_next, nvalid);
    }

    if (wave_active) {
      const int halves = nv_cur > 32 ? 2 : 1;
      f32x16_t s[2];
      s[0] = f32x16_t{};
      s[1] = f32x16_t{};
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        if (hf < halves) {
#pragma unroll
          for (int ks = 0; ks < D / 16; ++ks) {
            const u32x4_t raw = *reinterpret_cast<const u32x4_t*>(&Ks[(hf * 32 + l32) * C::KS_LD + ks * 16 + g2 * 8]);
            s[hf] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, raw), qf[ks], s[hf], 0, 0, 0);
          }
        }
      }
      // Mask keys past the block's end; in-lane max over this lane's keys.
      float mx = -INFINITY;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
          const int key = hf * 32 + 8 * (rr >> 2) + 4 * g2 + (rr & 3);
          const float x = key < nv_cur ? s[hf][rr] : -INFINITY;
          s[hf][rr] = x;
          mx = fmaxf(mx, x);
        }
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * scale_log2);
      m_run = m_new;
      const float mb = m_new * scale_log2;
#pragma unroll
      for (int c = 0; c < D / 32; ++c) acc[c] *= alpha;
      l_run *= alpha;
      bf16x8_t pb[2][2];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          f32x8_t pf;
#pragma unroll
          for (int t = 0; t < 8; ++t) pf[t] = __builtin_amdgcn_exp2f(s[hf][8 * m + t] * scale_log2 - mb);
          pb[hf][m] = __builtin_convertvector(pf, bf16x8_t);
#pragma unroll
          for (int t = 0; t < 8; ++t) l_run += (float)pb[hf][m][t];
        }
      }
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        if (hf < halves) {
#pragma unroll
          for (int m = 0; m < 2; ++m) {
            const int kb = hf * 32 + 16 * m + 4 * g2;
#pragma unroll
            for (int c = 0; c < D / 32; ++c) {
              const uint16_t* vp = &Vt[(c * 32 + l32) * VT_LD + kb];
              u32x4_t raw;
              const u32x2_t lo = *reinterpret_cast<const u32x2_t*>(vp);
              const u32x2_t hi = *reinterpret_cast<const u32x2_t*>(vp + 8);
              raw[0] = lo[0]; raw[1] = lo[1]; raw[2] = hi[0]; raw[3] = hi[1];
              acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, raw), pb[hf][m], acc[c], 0, 0, 0);
            }
          }
        }
      }
    }
    e = e_next;
    c0 = c_next;
  }

  // Epilogue: O = O^T / l, rounded to bf16, stored at the query's raster row.
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (qtok < ni) {
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    uint16_t* op = o + head_off + (size_t)qmap(qtok) * D;
#pragma unroll
    for (int c = 0; c < D / 32; ++c) {
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int d = c * 32 + 8 * gq + 4 * g2;
        u32x2_t w;
        w[0] = bf16_pair(f32_to_bf16(acc[c][4 * gq + 0] * inv), f32_to_bf16(acc[c][4 * gq + 1] * inv));
        w[1] = bf16_pair(f32_to_bf16(acc[c][4 * gq + 2] * inv), f32_to_bf16(acc[c][4 * gq + 3] * inv));
        *reinterpret_cast<u32x2_t*>(op + d) = w;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// float32 path: one thread per query token, 32-key tiles staged in LDS,
// float32 dot products and an exact-exp online softmax.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(128) void attn_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    float* __restrict__ o, const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx,
    DGeo g, float scale) {
  constexpr int TK = 32;
  __shared__ float Ks[TK][D + 1];
  __shared__ float Vs[TK][D];
  const int tid = threadIdx.x;
  const int bh = blockIdx.x / g.NB, i = blockIdx.x - bh * g.NB;
  const Box bi = block_box(g, i);
  const int ni = bi.n();
  TokenMap qmap;
  qmap.init(g, bi);
  const size_t head_off = (size_t)bh * g.N * D;
  const bool active = tid < ni;
  float qv[D], ov[D];
  const float* qp = q + head_off + (size_t)(active ? qmap(tid) : 0) * D;
#pragma unroll
  for (int d = 0; d < D; ++d) {
    qv[d] = active ? qp[d] : 0.0f;
    ov[d] = 0.0f;
  }
  float m_run = -INFINITY, l_run = 0.0f;
  const int row = bh * g.NB + i;
  for (int e = row_ptr[row]; e < row_ptr[row + 1]; ++e) {
    const int j = min(max(col_idx[e], 0), g.NB - 1);
    const Box bj = block_box(g, j);
    const int nj = bj.n();
    TokenMap kmap;
    kmap.init(g, bj);
    for (int c0 = 0; c0 < nj; c0 += TK) {
      const int nv = min(TK, nj - c0);
      __syncthreads();
      for (int idx = tid; idx < nv * D; idx += 128) {
        const int key = idx / D, d = idx - key * D;
        const size_t src = head_off + (size_t)kmap(c0 + key) * D + d;
        Ks[key][d] = k[src];
        Vs[key][d] = v[src];
      }
      __syncthreads();
      for (int key = 0; key < nv; ++key) {
        float s = 0.0f;
#pragma unroll
        for (int d = 0; d < D; ++d) s += qv[d] * Ks[key][d];
        s *= scale;
        const float m_new = fmaxf(m_run, s);
        const float alpha = expf(m_run - m_new);
        const float p = expf(s - m_new);
        l_run = l_run * alpha + p;
#pragma unroll
        for (int d = 0; d < D; ++d) ov[d] = ov[d] * alpha + p * Vs[key][d];
        m_run = m_new;
      }
    }
  }
  if (active) {
    float* op = o + head_off + (size_t)qmap(tid) * D;
    const float inv = 1.0f / l_run;
#pragma unroll
    for (int d = 0; d < D; ++d) op[d] = ov[d] * inv;
  }
}

hipError_t launch_attn(const void* q, const void* k, const void* v, void* o, int dtype, int D,
                       const int32_t* row_ptr, const int32_t* col_idx, const DGeo& g, int BH,
                       float scale, hipStream_t st) {
  const unsigned nwg = (unsigned)BH * (unsigned)g.NB;
  if (dtype == VSA_BF16) {
    const float sl2 = scale * 1.4426950408889634f;
    if (D == 128)
      hipLaunchKernelGGL(attn_bf16_kernel<128>, dim3(nwg), dim3(256), 0, st, (const uint16_t*)q,
                         (const uint16_t*)k, (const uint16_t*)v, (uint16_t*)o, row_ptr, col_idx, g, sl2);
    else
      hipLaunchKernelGGL(attn_bf16_kernel<64>, dim3(nwg), dim3(256), 0, st, (const uint16_t*)q,
                         (const uint16_t*)k, (const uint16_t*)v, (uint16_t*)o, row_ptr, col_idx, g, sl2);
  } else {
    if (D == 128)
      hipLaunchKernelGGL(attn_f32_kernel<128>, dim3(nwg), dim3(128), 0, st, (const float*)q,
                         (const float*)k, (const float*)v, (float*)o, row_ptr, col_idx, g, scale);
    else
      hipLaunchKernelGGL(attn_f32_kernel<64>, dim3(nwg), dim3(128), 0, st, (const float*)q,
                         (const float*)k, (const float*)v, (float*)o, row_ptr, col_idx, g, scale);
  }
  return hipGetLastError();
}

}  // namespace vsa
