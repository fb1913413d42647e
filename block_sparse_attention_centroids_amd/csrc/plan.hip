// Planning kernels for gfx950: block means or extremes (the summarizers),
// their inter-estimators (mean dot product, DSA, DSA2) with per-row Top-K or
// Top-P selection
// united with the local temporal window and the attention-sink blocks, and
// the CSR scan/fill used when rows vary in length.  SPADE (arXiv
// 2608.03335) 3.1 Fig. 4 and the vDiT-SSR utility parameters, and 3.3.
//
// This file is built with -ffp-contract=off and every product/sum uses the
// explicitly rounded intrinsics, so the arithmetic is the fixed float32
// order that makes the index reproducible bit for bit:
//   mean  = (((+0 + x_0) + x_1) + ... + x_{n-1}) / n
//   score = ((+0 + q_0*k_0) + q_1*k_1) + ... + q_{D-1}*k_{D-1}
// Top-P weights are expf((score - row max) * scale), summed in one fixed
// order per row (see topp_cut_regs).
#include <hip/hip_runtime.h>

#include "vsa_device.h"
#include "vsa_kernels.h"

#pragma clang fp contract(off)

namespace vsa {

// ---------------------------------------------------------------------------
// Block summaries (means for the mean estimator, max/min or the midpoint for
// the box estimators).  One workgroup per (tensor, row bh, block j).  The
// workgroup loads the block's n tokens in 16-byte pieces (every load
// coalesced, as in the layout kernels) and stages them through LDS half a
// block (64 tokens) at a time; thread c walks channel c over the tokens in
// block order.  The mean adds them one by one from +0
// and divides once (correctly rounded); max and min are exact.  The query
// midpoint is fl(fl(max + min) * 0.5).  With cm1 the second tensor's
// summaries go channel-major ([BH][D][NB]).
// ---------------------------------------------------------------------------
__device__ inline int uniform_i(int x) { return __builtin_amdgcn_readfirstlane(x); }

template <typename T, int D, bool EXT, bool SICS>
__global__ __launch_bounds__(256) void summary_kernel(const T* __restrict__ x0, float* __restrict__ oa0,
                                                      float* __restrict__ ob0, int mid0,
                                                      const T* __restrict__ x1, float* __restrict__ oa1,
                                                      float* __restrict__ ob1, int mid1, DGeo g, int cm1,
                                                      float* __restrict__ sc0, float* __restrict__ sc1,
                                                      HeadMap hm) {
  constexpr int ROWB = D * (int)sizeof(T);
  constexpr int PIECES = ROWB / 16;
  extern __shared__ uint4 stage16[];   // the block's tokens, [n][D] of T (room for 128)
  const T* stage = reinterpret_cast<const T*>(stage16);
  // Workgroups are dealt round-robin to the 8 XCDs by linear id; each XCD
  // takes one contiguous run of (tensor, bh, block) items instead, so the
  // channel-major 4-byte stores of neighbouring key blocks meet in one
  // XCD's L2 and leave it as whole lines.
  const int nit = (int)gridDim.x;
  const int total = nit * (int)gridDim.y;
  const int lin = (int)blockIdx.y * nit + (int)blockIdx.x;
  const int xcd = lin & 7, loc = lin >> 3;
  const int per = (total + 7) >> 3, rem8 = total & 7;
  const int logical = (rem8 == 0 || xcd < rem8) ? xcd * per + loc : rem8 * per + (xcd - rem8) * (per - 1) + loc;
  const bool second = logical >= nit;
  const int item = second ? logical - nit : logical;   // bh * NB + j
  const T* x = second ? x1 : x0;
  float* oa = second ? oa1 : oa0;
  float* ob = second ? ob1 : ob0;
  const int mid = second ? mid1 : mid0;
  const int bh = item / g.NB, j = item - bh * g.NB;
  const Box b = block_box(g, j);
  const int n = b.n();
  TokenMap map;
  map.init(g, b);
  const uint8_t* src = reinterpret_cast<const uint8_t*>(x) + (size_t)hm.tensor_bh(bh) * g.N * ROWB;
  // Every piece a thread copies is loaded before any is stored, so the
  // loads are all in flight together.  Loads are unconditional, so no
  // branch splits them: a slot past the block's last piece re-reads that
  // piece, and the channel walk below never reads it.
  constexpr int MAXIT = (VSA_MAX_BLOCK_TOKENS * PIECES + 255) / 256;
  const int npieces = n * PIECES;
  // The LDS stage holds half a block (64 tokens): the first half's pieces
  // (pa) go to LDS first, the second half's (pb) stay in registers until
  // the walk over the first half is done.  16 KB of LDS per workgroup (bf16,
  // d = 128) lets 8 workgroups share a CU, so twice as many loads are in
  // flight per CU as with a whole-block stage.
  constexpr int HALF_IT = MAXIT / 2;
  constexpr int HALF_TOK = VSA_MAX_BLOCK_TOKENS / 2;
  static_assert(256 * HALF_IT == HALF_TOK * PIECES, "half the slots hold the first 64 tokens");
  uint4 pa[HALF_IT], pb[HALF_IT];
  auto load_piece = [&](int it) {
    const int idx = min((int)threadIdx.x + it * 256, npieces - 1);
    const int u = idx / PIECES, p = idx - u * PIECES;
    return *reinterpret_cast<const uint4*>(src + (size_t)map(u) * ROWB + p * 16);
  };
#pragma unroll
  for (int it = 0; it < HALF_IT; ++it) pa[it] = load_piece(it);
#pragma unroll
  for (int it = 0; it < HALF_IT; ++it) pb[it] = load_piece(HALF_IT + it);
#pragma unroll
  for (int it = 0; it < HALF_IT; ++it) stage16[threadIdx.x + it * 256] = pa[it];
  // SICS (SPADE 3.2, Eq. 4 rewritten as Eq. 5): ||sum of the unit-normalized
  // tokens||^2, from registers.  Slot it of this thread holds piece
  // tid % PIECES (CPL channels) of token (tid + 256*it) / PIECES, so the
  // PIECES consecutive lanes that hold one token reduce its squared norm
  // with a butterfly (a zero token gets weight 0 and adds nothing), and
  // each lane adds its channels times that weight into w.  Slots past the
  // block's end (re-read pieces) are skipped.  The lanes of the four waves
  // that hold the same piece index are combined through the staging area
  // once the channel walk below is done with it, so the workgroup needs no
  // LDS beyond the 64-token stage.
  constexpr int CPL = 16 / (int)sizeof(T);
  float w[SICS ? CPL : 1];
  if constexpr (SICS) {
    static_assert(64 % PIECES == 0, "a token's pieces must sit in one wave");
#pragma unroll
    for (int e = 0; e < CPL; ++e) w[e] = 0.0f;
#pragma unroll
    for (int it = 0; it < MAXIT; ++it) {
      float v[CPL];
      const uint4 pc = it < HALF_IT ? pa[it] : pb[it - HALF_IT];
      const uint32_t w4[4] = {pc.x, pc.y, pc.z, pc.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if constexpr (sizeof(T) == 2) {
          v[2 * e] = bf16_lo(w4[e]);
          v[2 * e + 1] = bf16_hi(w4[e]);
        } else {
          v[e] = __uint_as_float(w4[e]);
        }
      }
      float sq = 0.0f;
#pragma unroll
      for (int e = 0; e < CPL; ++e) sq = __builtin_fmaf(v[e], v[e], sq);
#pragma unroll
      for (int m = 1; m < PIECES; m <<= 1) sq += __shfl_xor(sq, m, 64);
      const int u = ((int)threadIdx.x + it * 256) / PIECES;
      const float inv = (u < n && sq > 0.0f) ? __builtin_amdgcn_rsqf(sq) : 0.0f;
#pragma unroll
      for (int e = 0; e < CPL; ++e) w[e] = __builtin_fmaf(v[e], inv, w[e]);
    }
#pragma unroll
    for (int m = PIECES; m < 64; m <<= 1)
#pragma unroll
      for (int e = 0; e < CPL; ++e) w[e] += __shfl_xor(w[e], m, 64);
  }
  __syncthreads();
  const int c = threadIdx.x;
  auto val = [&](int u, int ch) {
    if constexpr (sizeof(T) == 2)
      return bf16_to_f32(stage[u * D + ch]);
    else
      return stage[u * D + ch];
  };
  float acc = 0.0f, mx = -INFINITY, mn = INFINITY;
  const int n0 = min(n, HALF_TOK);
  if (c < D) {
    if constexpr (!EXT) {
      for (int u = 0; u < n0; ++u) acc = __fadd_rn(acc, val(u, c));
    } else {
      for (int u = 0; u < n0; ++u) {
        const float v = val(u, c);
        mx = fmaxf(mx, v);
        mn = fminf(mn, v);
      }
    }
  }
  if (n > HALF_TOK) {                       // uniform over the workgroup
    __syncthreads();                        // every read of the first half is done
#pragma unroll
    for (int it = 0; it < HALF_IT; ++it) stage16[threadIdx.x + it * 256] = pb[it];
    __syncthreads();
    if (c < D) {
      if constexpr (!EXT) {
        for (int u = 0; u < n - HALF_TOK; ++u) acc = __fadd_rn(acc, val(u, c));
      } else {
        for (int u = 0; u < n - HALF_TOK; ++u) {
          const float v = val(u, c);
          mx = fmaxf(mx, v);
          mn = fminf(mn, v);
        }
      }
    }
  }
  if (c < D) {
    float ra, rb = 0.0f;
    if constexpr (!EXT) {
      ra = __fdiv_rn(acc, (float)n);
    } else {
      ra = mid ? __fmul_rn(__fadd_rn(mx, mn), 0.5f) : mx;
      rb = mn;
    }
    const size_t o = (second && cm1) ? ((size_t)bh * D + c) * g.NB + j : (size_t)item * D + c;
    oa[o] = ra;
    if (EXT && !mid) ob[o] = rb;
  }
  if constexpr (SICS) {
    float* part = reinterpret_cast<float*>(stage16);   // [4 waves][D] after the walk
    const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
    __syncthreads();                                    // every walk read of the stage is done
    if (lane < PIECES) {
#pragma unroll
      for (int e = 0; e < CPL; ++e) part[wv * D + lane * CPL + e] = w[e];
    }
    __syncthreads();
    float p2 = 0.0f;
    if (c < D) {
      const float wc = part[c] + part[D + c] + part[2 * D + c] + part[3 * D + c];
      p2 = __builtin_fmaf(wc, wc, 0.0f);
    }
#pragma unroll
    for (int m = 32; m > 0; m >>= 1) p2 += __shfl_xor(p2, m, 64);
    __syncthreads();                                    // part[] reads done before it is reused
    if (lane == 0) part[wv] = p2;
    __syncthreads();
    if (threadIdx.x == 0) (second ? sc1 : sc0)[item] = part[0] + part[1] + part[2] + part[3];
  }
}

// dst row bh (per floats) = src row tensor_bh(bh), in 16-byte pieces.
__global__ __launch_bounds__(256) void gather_rows_kernel(const float* __restrict__ src, float* __restrict__ dst,
                                                          int per, HeadMap hm) {
  const int bh = blockIdx.y;
  const float4* s4 = reinterpret_cast<const float4*>(src + (size_t)hm.tensor_bh(bh) * per);
  float4* d4 = reinterpret_cast<float4*>(dst + (size_t)bh * per);
  for (int i = blockIdx.x * 256 + threadIdx.x; i < per / 4; i += gridDim.x * 256) d4[i] = s4[i];
}

// Scores of RG query blocks against one key block for an estimator (EST 0:
// mean, 1: DSA, 2: DSA2).  qa[x]/qb[x] are query block x's summaries (mean,
// or midpoint, or max/min; D floats each, the same for the whole wave, so
// they come through scalar loads); channel d of the key block's summaries
// is at ka[d * sd] / kb[d * sd] (mean, or max/min), so either summary
// layout reads through it.  Channel by channel, in order from +0, the mean
// adds the rounded product; DSA the larger of the midpoint's two rounded
// products with the key box corners; DSA2 the largest of the four corner
// products.
template <int EST, int RG>
__device__ inline void est_column(const float* const (&qa)[RG], const float* const (&qb)[RG],
                                  const float* __restrict__ ka, const float* __restrict__ kb, size_t sd, int D,
                                  float (&acc)[RG]) {
#pragma unroll
  for (int x = 0; x < RG; ++x) acc[x] = 0.0f;
  constexpr int UNROLL = EST == 2 ? 2 : 4;   // DSA2's second query summary doubles the scalar loads
#pragma unroll UNROLL
  for (int d = 0; d < D; d += 4) {
    float kA[4], kB[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      kA[e] = ka[(size_t)(d + e) * sd];
      kB[e] = EST != 0 ? kb[(size_t)(d + e) * sd] : 0.0f;
    }
#pragma unroll
    for (int x = 0; x < RG; ++x) {
      const float4 a4 = *reinterpret_cast<const float4*>(qa[x] + d);
      const float qA[4] = {a4.x, a4.y, a4.z, a4.w};
      float qB[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      if constexpr (EST == 2) {
        const float4 b4 = *reinterpret_cast<const float4*>(qb[x] + d);
        qB[0] = b4.x;
        qB[1] = b4.y;
        qB[2] = b4.z;
        qB[3] = b4.w;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float t;
        if constexpr (EST == 0)
          t = __fmul_rn(qA[e], kA[e]);
        else if constexpr (EST == 1)
          t = fmaxf(__fmul_rn(qA[e], kA[e]), __fmul_rn(qA[e], kB[e]));
        else
          t = fmaxf(fmaxf(__fmul_rn(qA[e], kA[e]), __fmul_rn(qA[e], kB[e])),
                    fmaxf(__fmul_rn(qB[e], kA[e]), __fmul_rn(qB[e], kB[e])));
        acc[x] = __fadd_rn(acc[x], t);
      }
    }
  }
}

// Orderable key of a score: larger float -> larger key; -0 and +0 map to
// the same key, so they tie (and the lower block id wins).
__device__ inline uint32_t order_key(float s) {
  uint32_t u = __float_as_uint(s);
  if ((u << 1) == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Float of an order key (the inverse of order_key; -0 arrives as +0).
__device__ inline float key_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Same value in every lane, taken from lane 0 (keeps decisions uniform).
__device__ inline float uniform_f(float x) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x)));
}

// Sum over the wave: each lane's partial, then a butterfly.  The pairs of a
// butterfly step add the same two numbers, so every lane ends with the same
// value.
__device__ inline float wave_sum_f(float a) {
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) a = __fadd_rn(a, __shfl_xor(a, m, 64));
  return uniform_f(a);
}

__device__ inline uint32_t wave_min_u(uint32_t v) {
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) v = min(v, (uint32_t)__shfl_xor((int)v, m, 64));
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)v);
}

__device__ inline uint32_t wave_max_u(uint32_t v) {
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, m, 64));
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)v);
}

// Top-K cut of a row of keys: thr = the k-th largest key, need = how many
// keys equal to thr are kept (the lowest ids).  thr grows bit by bit from
// the top to the largest value with at least kk keys >= thr; counts are
// ballots, and rows of at most 1280 blocks keep their keys in registers
// (4, 6, 8, 12, 16 or 20 chunks of 64, the fewest that hold the row), so
// the 32 passes read LDS once; longer rows re-read it every pass.  Once
// exactly kk keys are >= the candidate, those kk are the top kk and the
// cut is their minimum, so the remaining passes are skipped (the result is
// the same key the full search reaches).
template <int NR>
__device__ inline uint32_t topk_threshold_regs(const uint32_t* keys, int NB, int lane, int kk, int& gt) {
  uint32_t kv[NR];
#pragma unroll
  for (int s2 = 0; s2 < NR; ++s2) {
    const int j = s2 * 64 + lane;
    kv[s2] = j < NB ? keys[j] : 0u;   // below every real key
  }
  uint32_t thr = 0u;
  int bit = 31;
  for (; bit >= 0; --bit) {
    const uint32_t cand = thr | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int s2 = 0; s2 < NR; ++s2) cnt += __popcll(__ballot(kv[s2] >= cand));
    if (cnt >= kk) {
      thr = cand;
      if (cnt == kk) break;
    }
  }
  if (bit >= 0) {   // exactly kk keys are >= thr: the cut is the smallest of them
    uint32_t m = 0xffffffffu;
#pragma unroll
    for (int s2 = 0; s2 < NR; ++s2) m = min(m, kv[s2] >= thr ? kv[s2] : 0xffffffffu);
    thr = wave_min_u(m);
  }
  gt = 0;
#pragma unroll
  for (int s2 = 0; s2 < NR; ++s2) gt += __popcll(__ballot(kv[s2] > thr));
  return thr;
}

__device__ inline void topk_cut(const uint32_t* keys, int NB, int lane, int kk, uint32_t& thr_out,
                                int& need_out) {
  uint32_t thr = 0u;
  int gt = 0;
  if (NB <= 64 * 4) {
    thr = topk_threshold_regs<4>(keys, NB, lane, kk, gt);
  } else if (NB <= 64 * 6) {
    thr = topk_threshold_regs<6>(keys, NB, lane, kk, gt);
  } else if (NB <= 64 * 8) {
    thr = topk_threshold_regs<8>(keys, NB, lane, kk, gt);
  } else if (NB <= 64 * 12) {
    thr = topk_threshold_regs<12>(keys, NB, lane, kk, gt);
  } else if (NB <= 64 * 16) {
    thr = topk_threshold_regs<16>(keys, NB, lane, kk, gt);
  } else if (NB <= 64 * 20) {
    thr = topk_threshold_regs<20>(keys, NB, lane, kk, gt);
  } else {
    int bit = 31;
    for (; bit >= 0; --bit) {
      const uint32_t cand = thr | (1u << bit);
      int cnt = 0;
      for (int j0 = 0; j0 < NB; j0 += 64) {
        const int j = j0 + lane;
        cnt += __popcll(__ballot(j < NB && keys[j] >= cand));
      }
      if (cnt >= kk) {
        thr = cand;
        if (cnt == kk) break;
      }
    }
    if (bit >= 0) {
      uint32_t m = 0xffffffffu;
      for (int j = lane; j < NB; j += 64) m = min(m, keys[j] >= thr ? keys[j] : 0xffffffffu);
      thr = wave_min_u(m);
    }
    for (int j0 = 0; j0 < NB; j0 += 64) {
      const int j = j0 + lane;
      gt += __popcll(__ballot(j < NB && keys[j] > thr));
    }
  }
  thr_out = thr;
  need_out = kk - gt;   // >= 1
}

// Top-P cut of a row of keys.  Weights e_j = expf((s_j - m) * scale) with m
// the row max; M(t) = sum of the weights of keys >= t, always summed the
// same way (per lane in chunk order, then the butterfly), so M is
// non-increasing in t and M(0) is the total Z.  With T = p * Z (<= Z for
// p <= 1), thr is the largest key with M(thr) >= T, found bit by bit; every
// key above thr is kept, and keys equal to thr are added in id order until
// the running mass reaches T (at least one of them).  p = 1 keeps the
// whole row: every weight is positive in exact arithmetic, even one too
// small to change a float32 sum.
template <int NR>
__device__ inline void topp_cut_regs(const uint32_t* keys, int NB, int lane, float p, float scale,
                                     uint32_t& thr_out, int& need_out) {
  if (p >= 1.0f) {
    thr_out = 0u;
    need_out = NB;
    return;
  }
  uint32_t kv[NR];
  float ev[NR];
  uint32_t kmax = 0u;
#pragma unroll
  for (int s2 = 0; s2 < NR; ++s2) {
    const int j = s2 * 64 + lane;
    kv[s2] = j < NB ? keys[j] : 0u;
    kmax = max(kmax, kv[s2]);
  }
  const float smax = key_float(wave_max_u(kmax));
#pragma unroll
  for (int s2 = 0; s2 < NR; ++s2) {
    const int j = s2 * 64 + lane;
    ev[s2] = j < NB ? expf(__fmul_rn(__fsub_rn(key_float(kv[s2]), smax), scale)) : 0.0f;
  }
  auto mass_ge = [&](uint32_t t) {
    float a = 0.0f;
#pragma unroll
    for (int s2 = 0; s2 < NR; ++s2) a = __fadd_rn(a, kv[s2] >= t ? ev[s2] : 0.0f);
    return wave_sum_f(a);
  };
  const float target = __fmul_rn(p, mass_ge(0u));
  uint32_t thr = 0u;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = thr | (1u << bit);
    if (mass_ge(cand) >= target) thr = cand;
  }
  float acc = 0.0f;
  int neq = 0;
  {
    float a = 0.0f;
#pragma unroll
    for (int s2 = 0; s2 < NR; ++s2) {
      const int j = s2 * 64 + lane;
      a = __fadd_rn(a, kv[s2] > thr ? ev[s2] : 0.0f);
      neq += __popcll(__ballot(j < NB && kv[s2] == thr));
    }
    acc = wave_sum_f(a);
  }
  const float ethr = expf(__fmul_rn(__fsub_rn(key_float(thr), smax), scale));
  int need = 0;
  while (need < neq && acc < target) {
    acc = __fadd_rn(acc, ethr);
    ++need;
  }
  thr_out = thr;
  need_out = need > 0 ? need : 1;
}

// The same cut for rows longer than the register chunks: keys stay in LDS
// and each weight is recomputed when it is needed (the same expression, so
// the same value).
__device__ inline void topp_cut_lds(const uint32_t* keys, int NB, int lane, float p, float scale,
                                    uint32_t& thr_out, int& need_out) {
  if (p >= 1.0f) {
    thr_out = 0u;
    need_out = NB;
    return;
  }
  uint32_t kmax = 0u;
  for (int j = lane; j < NB; j += 64) kmax = max(kmax, keys[j]);
  const float smax = key_float(wave_max_u(kmax));
  auto weight = [&](uint32_t key) { return expf(__fmul_rn(__fsub_rn(key_float(key), smax), scale)); };
  auto mass_ge = [&](uint32_t t) {
    float a = 0.0f;
    for (int j0 = 0; j0 < NB; j0 += 64) {
      const int j = j0 + lane;
      const uint32_t key = j < NB ? keys[j] : 0u;
      a = __fadd_rn(a, (j < NB && key >= t) ? weight(key) : 0.0f);
    }
    return wave_sum_f(a);
  };
  const float target = __fmul_rn(p, mass_ge(0u));
  uint32_t thr = 0u;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = thr | (1u << bit);
    if (mass_ge(cand) >= target) thr = cand;
  }
  float a = 0.0f;
  int neq = 0;
  for (int j0 = 0; j0 < NB; j0 += 64) {
    const int j = j0 + lane;
    const uint32_t key = j < NB ? keys[j] : 0u;
    a = __fadd_rn(a, (j < NB && key > thr) ? weight(key) : 0.0f);
    neq += __popcll(__ballot(j < NB && key == thr));
  }
  float acc = wave_sum_f(a);
  const float ethr = weight(thr);
  int need = 0;
  while (need < neq && acc < target) {
    acc = __fadd_rn(acc, ethr);
    ++need;
  }
  thr_out = thr;
  need_out = need > 0 ? need : 1;
}

// ---------------------------------------------------------------------------
// Scores + selection.  One workgroup per (bh, tile of RT query blocks).
// Phase 1 fills LDS with the RT x NB score rows; phase 2 gives each wave a
// row: the cut (Top-K or Top-P) gives a threshold key and how many keys
// equal to it are kept, then the row is emitted in ascending block id with
// ties at the threshold going to the lowest ids, united with the window and
// the sink blocks.
// ---------------------------------------------------------------------------
template <int RT, bool TOPP, int EST>
__global__ __launch_bounds__(256) void score_select_kernel(
    Summaries sm, DGeo g, int D, int heads,
    SelectArgs sa, int32_t* __restrict__ row_ptr, int32_t* __restrict__ col_idx,
    int32_t* __restrict__ counts, uint64_t* __restrict__ bits) {
  extern __shared__ uint32_t smem[];   // [RT][NB] keys
  const int NB = g.NB;
  const int bh = blockIdx.y;
  const int i0 = blockIdx.x * RT;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int rows_here = min(RT, NB - i0);
  // Phase 1: scores.  Rows past NB reuse the last valid row (never emitted).
  // A static head reads its scores from the caller's table; a dense head
  // keeps every block, so its keys are all equal.
  const int h = bh % heads;
  const int b = bh / heads;
  const int kind = sa.kind[h];
  const size_t head = (size_t)bh * NB * D;
  const float* qa = sm.qa + head;
  const float* qb = EST == 2 ? sm.qb + head : nullptr;
  const float* ka = sm.ka + head;
  const float* kb = EST != 0 ? sm.kb + head : nullptr;
  if (kind == 1) {
    const float* tab = sa.table + ((size_t)h * NB + i0) * NB;
    for (int r = 0; r < rows_here; ++r)
      for (int j = tid; j < NB; j += 256) smem[r * NB + j] = order_key(tab[(size_t)r * NB + j]);
  } else if (kind == 2) {
    for (int r = 0; r < rows_here; ++r)
      for (int j = tid; j < NB; j += 256) smem[r * NB + j] = 0x80000000u;
  } else {
    // Estimator scores.  A task is RG rows x 64 consecutive key blocks
    // (lane = key block) and the tasks are dealt evenly to the waves; with
    // the planner's channel-major key summaries every load of a channel is
    // 256 contiguous bytes.  Rows past rows_here read the last row and are
    // not stored.
    constexpr int RG = RT < 4 ? RT : 4;
    const int wv = uniform_i(wave);
    const int chunks = (NB + 63) >> 6;
    const int tasks = chunks * ((rows_here + RG - 1) / RG);
    const size_t sj = sm.kt ? 1 : (size_t)D, sd = sm.kt ? (size_t)NB : 1;
    for (int task = wv; task < tasks; task += 4) {
      const int rg = task / chunks, ch = task - rg * chunks;
      const int j = ch * 64 + lane;
      const float* qra[RG];
      const float* qrb[RG];
#pragma unroll
      for (int x = 0; x < RG; ++x) {
        const size_t qi = (size_t)(i0 + min(rg * RG + x, rows_here - 1)) * D;
        qra[x] = qa + qi;
        qrb[x] = (EST == 2 ? qb : qa) + qi;
      }
      const size_t kj = (size_t)min(j, NB - 1) * sj;
      float acc[RG];
      est_column<EST, RG>(qra, qrb, ka + kj, (EST != 0 ? kb : ka) + kj, sd, D, acc);
      if (j < NB) {
#pragma unroll
        for (int x = 0; x < RG; ++x)
          if (rg * RG + x < rows_here) smem[(rg * RG + x) * NB + j] = order_key(acc[x]);
      }
    }
  }
  __syncthreads();

  // Phase 2: selection, one wave per row.
  const int kk = TOPP ? 0 : sa.k[h];
  const int win = sa.win[h];
  const int per_t = g.nbh * g.nbw;
  for (int r = wave; r < rows_here; r += 4) {
    const int i = i0 + r;
    const uint32_t* keys = smem + r * NB;
    uint32_t thr;
    int need;
    if constexpr (TOPP) {
      // The fewest register chunks that hold the row; the chunks left out
      // would only add +0 to each lane's non-negative partial sums.
      if (NB <= 64 * 4)
        topp_cut_regs<4>(keys, NB, lane, sa.p[h], sa.scale, thr, need);
      else if (NB <= 64 * 6)
        topp_cut_regs<6>(keys, NB, lane, sa.p[h], sa.scale, thr, need);
      else if (NB <= 64 * 8)
        topp_cut_regs<8>(keys, NB, lane, sa.p[h], sa.scale, thr, need);
      else if (NB <= 64 * 12)
        topp_cut_regs<12>(keys, NB, lane, sa.p[h], sa.scale, thr, need);
      else if (NB <= 64 * 16)
        topp_cut_regs<16>(keys, NB, lane, sa.p[h], sa.scale, thr, need);
      else if (NB <= 64 * 20)
        topp_cut_regs<20>(keys, NB, lane, sa.p[h], sa.scale, thr, need);
      else
        topp_cut_lds(keys, NB, lane, sa.p[h], sa.scale, thr, need);
    } else {
      topk_cut(keys, NB, lane, kk, thr, need);
    }
    const int tbi = i / per_t;
    const int64_t row = (int64_t)bh * NB + i;
    const int64_t out0 = TOPP ? 0 : (int64_t)b * sa.batch_stride + (int64_t)NB * sa.off[h] + (int64_t)i * kk;
    int eq_before = 0, base = 0;
    const uint64_t lt = lanemask_lt();
    for (int s = 0; s * 64 < NB; ++s) {
      const int j = s * 64 + lane;
      const bool valid = j < NB;
      const uint32_t key = valid ? keys[j] : 0u;
      const bool eq = valid && key == thr;
      const uint64_t eqm = __ballot(eq);
      const int rank_eq = eq_before + __popcll(eqm & lt);
      bool keep = valid && (key > thr || (eq && rank_eq < need));
      if (sa.bitmap && valid) {
        const int dt = j / per_t - tbi;
        keep = keep || (win >= 0 && dt <= win && -dt <= win) || j < sa.sink;
      }
      const uint64_t km = __ballot(keep);
      if (sa.bitmap) {
        if (lane == 0) bits[row * sa.words + s] = km;
      } else if (keep) {
        const int pos = base + __popcll(km & lt);
        if (pos < kk) col_idx[out0 + pos] = j;
      }
      base += __popcll(km);
      eq_before += __popcll(eqm);
    }
    if (lane == 0) {
      if (sa.bitmap) {
        counts[row] = base;
      } else {
        row_ptr[row] = (int32_t)out0;
        if (row == sa.rows - 1) row_ptr[row + 1] = (int32_t)(out0 + kk);
      }
    }
  }
}

// Exclusive scan of per-row counts into row_ptr (one workgroup).
__global__ __launch_bounds__(1024) void scan_kernel(const int32_t* __restrict__ counts,
                                                    int32_t* __restrict__ row_ptr, int64_t R) {
  __shared__ int64_t part[1024];
  const int t = threadIdx.x;
  const int64_t chunk = (R + 1023) / 1024;
  const int64_t lo = min<int64_t>(R, (int64_t)t * chunk), hi = min<int64_t>(R, lo + chunk);
  int64_t s = 0;
  for (int64_t r = lo; r < hi; ++r) s += counts[r];
  part[t] = s;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    int64_t v = t >= off ? part[t - off] : 0;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  int64_t run = part[t] - s;   // exclusive prefix of this thread's chunk
  for (int64_t r = lo; r < hi; ++r) {
    row_ptr[r] = (int32_t)run;
    run += counts[r];
  }
  if (t == 1023) row_ptr[R] = (int32_t)part[1023];
}

// Bitmap rows -> ascending column lists at row_ptr (one wave per row).
// Every write stays in [0, capacity), whatever row_ptr holds.
__global__ __launch_bounds__(256) void fill_kernel(const uint64_t* __restrict__ bits,
                                                   const int32_t* __restrict__ row_ptr,
                                                   int32_t* __restrict__ col_idx, int64_t R, int words,
                                                   int NB, int64_t capacity) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + wave;
  if (row >= R) return;
  int64_t base = row_ptr[row];
  const uint64_t lt = lanemask_lt();
  for (int s = 0; s < words; ++s) {
    const uint64_t w = bits[row * words + s];
    const int j = s * 64 + lane;
    const int64_t pos = base + __popcll(w & lt);
    if (j < NB && ((w >> lane) & 1ull) && pos >= 0 && pos < capacity) col_idx[pos] = j;
    base += __popcll(w);
  }
}

// Full score matrix (the inter-estimator alone), same order as above.
template <int EST>
__global__ __launch_bounds__(256) void scores_kernel(Summaries sm, float* __restrict__ out, int NB, int D) {
  const int bh = blockIdx.y;
  const int i = blockIdx.x;
  const size_t head = (size_t)bh * NB * D;
  const size_t qi = head + (size_t)i * D;
  const size_t sj = sm.kt ? 1 : (size_t)D, sd = sm.kt ? (size_t)NB : 1;
  const float* qra[1] = {sm.qa + qi};
  const float* qrb[1] = {(EST == 2 ? sm.qb : sm.qa) + qi};
  for (int j = threadIdx.x; j < NB; j += 256) {
    float acc[1];
    const size_t kj = head + (size_t)j * sj;
    est_column<EST, 1>(qra, qrb, sm.ka + kj, (EST != 0 ? sm.kb : sm.ka) + kj, sd, D, acc);
    out[((size_t)bh * NB + i) * NB + j] = acc[0];
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <bool EXT, bool SICS>
hipError_t launch_summary(const void* x0, float* a0, float* b0, int mid0, const void* x1, float* a1, float* b1,
                          int mid1, int dtype, int D, const DGeo& g, int BH, hipStream_t st, int cm1,
                          float* s0, float* s1, const HeadMap& hm) {
  dim3 grid((unsigned)(BH * g.NB), x1 ? 2 : 1), block(256);
  const size_t lds = (size_t)(VSA_MAX_BLOCK_TOKENS / 2) * D * (dtype == 0 ? 2 : 4);   // half a block of tokens
  if (dtype == 0) {
    if (D == 128)
      hipLaunchKernelGGL((summary_kernel<uint16_t, 128, EXT, SICS>), grid, block, lds, st, (const uint16_t*)x0, a0,
                         b0, mid0, (const uint16_t*)x1, a1, b1, mid1, g, cm1, s0, s1, hm);
    else
      hipLaunchKernelGGL((summary_kernel<uint16_t, 64, EXT, SICS>), grid, block, lds, st, (const uint16_t*)x0, a0,
                         b0, mid0, (const uint16_t*)x1, a1, b1, mid1, g, cm1, s0, s1, hm);
  } else {
    if (D == 128)
      hipLaunchKernelGGL((summary_kernel<float, 128, EXT, SICS>), grid, block, lds, st, (const float*)x0, a0, b0,
                         mid0, (const float*)x1, a1, b1, mid1, g, cm1, s0, s1, hm);
    else
      hipLaunchKernelGGL((summary_kernel<float, 64, EXT, SICS>), grid, block, lds, st, (const float*)x0, a0, b0,
                         mid0, (const float*)x1, a1, b1, mid1, g, cm1, s0, s1, hm);
  }
  return hipGetLastError();
}

hipError_t launch_pool(const void* x0, float* out0, const void* x1, float* out1, int dtype, int D,
                       const DGeo& g, int BH, hipStream_t st, bool out1_channel_major, const HeadMap* hm) {
  const HeadMap id;
  return launch_summary<false, false>(x0, out0, nullptr, 0, x1, out1, nullptr, 0, dtype, D, g, BH, st,
                                      out1_channel_major ? 1 : 0, nullptr, nullptr, hm ? *hm : id);
}

hipError_t launch_pool_sics(const void* x0, float* out0, const void* x1, float* out1, float* sics0, float* sics1,
                            int dtype, int D, const DGeo& g, int BH, hipStream_t st) {
  const HeadMap id;
  return launch_summary<false, true>(x0, out0, nullptr, 0, x1, out1, nullptr, 0, dtype, D, g, BH, st, 1, sics0,
                                     sics1, id);
}

hipError_t launch_extremes(const void* x0, float* max0, float* min0, int mid0, const void* x1, float* max1,
                           float* min1, int mid1, int dtype, int D, const DGeo& g, int BH, hipStream_t st,
                           bool out1_channel_major, const HeadMap* hm) {
  const HeadMap id;
  return launch_summary<true, false>(x0, max0, min0, mid0, x1, max1, min1, mid1, dtype, D, g, BH, st,
                                     out1_channel_major && !mid1 ? 1 : 0, nullptr, nullptr, hm ? *hm : id);
}

hipError_t launch_gather_rows(const float* src, float* dst, int per, const HeadMap& hm, int BH, hipStream_t st) {
  const int blocks = min(64, (per / 4 + 255) / 256);
  hipLaunchKernelGGL(gather_rows_kernel, dim3((unsigned)max(blocks, 1), (unsigned)BH), dim3(256), 0, st, src, dst,
                     per, hm);
  return hipGetLastError();
}

// LDS of a workgroup with RT rows: RT rows of NB uint32 keys.
size_t select_lds_bytes(int RT, int NB) { return (size_t)RT * NB * 4; }

// Rows per workgroup: up to 4 (so that a CU holds about four workgroups
// at the headline, enough to cover the load latencies of phase 1), fewer
// when the rows' LDS would pass 64 KiB.
int select_rows_per_block(int NB) {
  for (int RT = 4; RT >= 2; RT >>= 1)
    if (select_lds_bytes(RT, NB) <= 65536) return RT;
  return 1;
}

template <bool TOPP, int EST>
void launch_score_select_t(int RT, dim3 grid, dim3 block, size_t lds, hipStream_t st, const Summaries& sm,
                           const DGeo& g, int D, int heads, const SelectArgs& sa, int32_t* row_ptr,
                           int32_t* col_idx, int32_t* counts, uint64_t* bits) {
  switch (RT) {
    case 4: hipLaunchKernelGGL((score_select_kernel<4, TOPP, EST>), grid, block, lds, st, sm, g, D, heads, sa, row_ptr, col_idx, counts, bits); break;
    case 2: hipLaunchKernelGGL((score_select_kernel<2, TOPP, EST>), grid, block, lds, st, sm, g, D, heads, sa, row_ptr, col_idx, counts, bits); break;
    default: hipLaunchKernelGGL((score_select_kernel<1, TOPP, EST>), grid, block, lds, st, sm, g, D, heads, sa, row_ptr, col_idx, counts, bits); break;
  }
}

template <int EST>
void launch_score_select_e(int RT, dim3 grid, dim3 block, size_t lds, hipStream_t st, const Summaries& sm,
                           const DGeo& g, int D, int heads, const SelectArgs& sa, int32_t* row_ptr,
                           int32_t* col_idx, int32_t* counts, uint64_t* bits) {
  if (sa.topp)
    launch_score_select_t<true, EST>(RT, grid, block, lds, st, sm, g, D, heads, sa, row_ptr, col_idx, counts, bits);
  else
    launch_score_select_t<false, EST>(RT, grid, block, lds, st, sm, g, D, heads, sa, row_ptr, col_idx, counts, bits);
}

hipError_t launch_score_select(const Summaries& sm, int est, const DGeo& g, int D, int heads, int BH,
                               const SelectArgs& sa, int32_t* row_ptr, int32_t* col_idx, int32_t* counts,
                               uint64_t* bits, hipStream_t st) {
  const int RT = select_rows_per_block(g.NB);
  dim3 grid((g.NB + RT - 1) / RT, BH), block(256);
  const size_t lds = select_lds_bytes(RT, g.NB);
  if (est == 1)
    launch_score_select_e<1>(RT, grid, block, lds, st, sm, g, D, heads, sa, row_ptr, col_idx, counts, bits);
  else if (est == 2)
    launch_score_select_e<2>(RT, grid, block, lds, st, sm, g, D, heads, sa, row_ptr, col_idx, counts, bits);
  else
    launch_score_select_e<0>(RT, grid, block, lds, st, sm, g, D, heads, sa, row_ptr, col_idx, counts, bits);
  return hipGetLastError();
}

hipError_t launch_scan_fill(const int32_t* counts, const uint64_t* bits, int32_t* row_ptr,
                            int32_t* col_idx, int64_t R, int words, int NB, int64_t capacity,
                            hipStream_t st) {
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, st, counts, row_ptr, R);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fill_kernel, dim3((unsigned)((R + 3) / 4)), dim3(256), 0, st, bits, row_ptr, col_idx, R, words, NB, capacity);
  return hipGetLastError();
}

hipError_t launch_scores(const Summaries& sm, int est, float* out, int NB, int D, int BH, hipStream_t st) {
  if (est == 1)
    hipLaunchKernelGGL(scores_kernel<1>, dim3(NB, BH), dim3(256), 0, st, sm, out, NB, D);
  else if (est == 2)
    hipLaunchKernelGGL(scores_kernel<2>, dim3(NB, BH), dim3(256), 0, st, sm, out, NB, D);
  else
    hipLaunchKernelGGL(scores_kernel<0>, dim3(NB, BH), dim3(256), 0, st, sm, out, NB, D);
  return hipGetLastError();
}


}  // namespace vsa
