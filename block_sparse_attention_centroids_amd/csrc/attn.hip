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
//   O^T (d x queries) += V^T P^T     V^T fragments read from the row-major
//                                    V tile with the transposing LDS read,
//                                    P^T straight from the S^T accumulators
//                                    (same lane, same keys)
// K/V stages are loaded into registers one stage ahead through raw buffer
// loads (out-of-range reads return zero), so global latency overlaps the
// matrix work of the current stage.
#include <hip/hip_runtime.h>

#include <math.h>

#include "vsa_device.h"
#include "vsa_kernels.h"

namespace vsa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

constexpr int KS = 32;              // keys per stage
constexpr int NBUF = 3;             // LDS ring: stage t (QK and PV), stages t+1 and t+2 landing
#ifndef VSA_ATTN_NT
#define VSA_ATTN_NT 1
#endif
constexpr int NT = VSA_ATTN_NT;     // 32-query MFMA tiles per wave
constexpr int WAVES = 4 / NT;       // waves per workgroup: 128 query tokens in all
constexpr int THREADS = 64 * WAVES;
constexpr int QPW = 32 * NT;        // query tokens per wave
constexpr float LAZY_LOG2 = 8.0f;   // running max is only raised when a row max exceeds it by 2^8

// LDS tiles hold token rows of D bf16 (PARTS 16-byte pieces) with no
// padding; piece pc of row r sits at slot pc ^ swz(r) of the row.  The
// swizzle keeps both fragment reads conflict-free: the K reads (16 lanes,
// 16 rows, one piece) and the transposing V reads (32 lanes, 4 rows, 4
// consecutive pieces).
template <int PARTS>
__device__ __forceinline__ int swz(int r) {
  if constexpr (PARTS == 16) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

template <int D>
struct AttnCfg {
  static constexpr int PARTS = D / 8;                  // 16-byte pieces per token row
  static constexpr int TILE_BYTES = KS * D * 2;        // one K or V stage tile
  static constexpr int ROWS_PER_INST = 64 / PARTS;     // rows one wave instruction fills
  static constexpr int IPW = KS / ROWS_PER_INST / WAVES;  // load instructions per wave per tensor
};

// Raw buffer descriptor: loads past `bytes` return zero instead of faulting.
// The base address is made explicitly wave-uniform so the descriptor stays
// in scalar registers.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
  void* p = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, (int)bytes, 0x00020000);
}

__device__ inline int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Raw buffer descriptor as four scalar dwords (base, num_records, flags).
struct Rsrc4 {
  u32x4_t d;
};
__device__ inline Rsrc4 make_rsrc4(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  Rsrc4 r;
  r.d[0] = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r.d[1] = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));   // stride 0
  r.d[2] = bytes;
  r.d[3] = 0x00020000u;
  return r;
}

// 16 bytes per lane from a raw buffer straight into LDS at lds_base + 16*lane
// (out-of-range offsets write zeros).  Written as asm so that the
// compiler's LDS-DMA tracking does not force a wait for every in-flight
// stage before each LDS read: completion is awaited explicitly (vmcnt)
// before the barrier that publishes a stage.  The instruction has no
// register results.
__device__ __forceinline__ void dma16(const Rsrc4& r, uint32_t lds_base, uint32_t voff) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds"
      :
      : "s"(lds_base), "v"(voff), "s"(r.d)
      : "memory", "m0");
}

__device__ inline uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

__device__ inline uint32_t bf16_pair(uint16_t lo, uint16_t hi) { return (uint32_t)lo | ((uint32_t)hi << 16); }

typedef __attribute__((address_space(3))) void lds_void_t;

// The key block a CSR entry names, with everything the loaders need; all
// fields are wave-uniform.
struct KeyBlock {
  int nj;            // tokens in the block
  bool nominal;      // (h, w) extents are the nominal block's
  uint32_t jbase;    // byte offset of the block's origin token in the head
  TokenMap map;      // token index -> raster index (for the other blocks)
};

template <int D>
__device__ __forceinline__ KeyBlock open_block(const DGeo& g, const int32_t* __restrict__ col_idx, int entry,
                                               bool stage_rows) {
  const int j = uniform(min(max(col_idx[entry], 0), g.NB - 1));   // a corrupt index cannot leave the head
  const Box bj = block_box_fast(g, j);
  KeyBlock kb;
  kb.nj = uniform(bj.n());
  kb.nominal = uniform(bj.eh == g.bh && bj.ew == g.bw && stage_rows) != 0;
  kb.map.base = uniform((bj.t0 * g.H + bj.h0) * g.W + bj.w0);
  kb.jbase = (uint32_t)kb.map.base * (D * 2);
  if (!kb.nominal) kb.map.init(g, bj);   // the reciprocals are only needed off the fast path
  return kb;
}

// Value of the same lane in the other half of the wave (lane ^ 32).
__device__ __forceinline__ float other_half(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  // r[0]: lanes 32..63 now hold lanes 0..31; r[1]: lanes 0..31 hold lanes 32..63.
  return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

// First half of the online-softmax step for one 32-key x 32-query tile of
// S^T held by this lane (query column l32; 16 of the 32 keys): masks keys
// past `nv` (a block's last, partial stage only), takes the row max and
// applies the lazy rescale to the tile's O^T accumulators.  Returns the
// exponent offset m*scale*log2(e).
template <int D>
__device__ __forceinline__ float softmax_prep(f32x16_t& s, int nv, int g2, float scale_log2, float tau,
                                              float& m_run, float& l_run, f32x16_t (&acc)[D / 32]) {
  if (nv < KS) {   // kept as a real branch
    asm volatile("" ::: "memory");
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      const int key = 8 * (rr >> 2) + 4 * g2 + (rr & 3);
      s[rr] = key < nv ? s[rr] : -INFINITY;
    }
  }
  float mx = fmaxf(s[0], s[1]);
#pragma unroll
  for (int rr = 2; rr < 16; rr += 2) mx = fmaxf(mx, fmaxf(s[rr], s[rr + 1]));
  mx = fmaxf(mx, other_half(mx));
  // Lazy rescale: the running max moves only when some row max exceeds it
  // by more than 2^LAZY_LOG2; otherwise p <= 2^LAZY_LOG2 stays exact enough
  // in bf16 and the O/l rescale is skipped for the whole wave.
  if (__ballot(mx > m_run + tau) != 0ull) {
    const float m_new = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * scale_log2);
#pragma unroll
    for (int c = 0; c < D / 32; ++c) acc[c] *= alpha;
    l_run *= alpha;
    m_run = m_new;
  }
  return m_run * scale_log2;
}

template <int D>
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(3, 3))) void attn_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    uint16_t* __restrict__ o, const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx,
    DGeo g, float scale_log2) {
  using C = AttnCfg<D>;
  constexpr int PARTS = C::PARTS;
  // [buffer][K tile, V tile]
  __shared__ __attribute__((aligned(1024))) uint8_t lds[NBUF * 2 * C::TILE_BYTES];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform(tid >> 6);   // wave-uniform, so per-wave branches stay scalar
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
  const uint32_t head_bytes = (uint32_t)g.N * D * 2u;
  const Rsrc4 krs = make_rsrc4(k + head_off, head_bytes);
  const Rsrc4 vrs = make_rsrc4(v + head_off, head_bytes);
  const uint32_t lds0 = (uint32_t)uniform((int)lds_addr(lds));

  // This wave's query tiles: tokens [QPW*wave + 32*t, +32) of the block.
  const int ntiles = min(NT, max(0, (ni - QPW * wave + 31) / 32));   // wave-uniform
  // Q^T fragments (B operand): query column l32 of tile t, channels 16*ks + 8*g2 + [0, 8).
  bf16x8_t qf[NT][D / 16];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int qtok = QPW * wave + 32 * t + l32;
    const bool ok = qtok < ni;
    const uint16_t* qp = q + head_off + (size_t)(ok ? qmap(qtok) : 0) * D + g2 * 8;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      u32x4_t raw = ok ? *reinterpret_cast<const u32x4_t*>(qp + ks * 16) : u32x4_t{0u, 0u, 0u, 0u};
      qf[t][ks] = __builtin_bit_cast(bf16x8_t, raw);
    }
  }

  f32x16_t acc[NT][D / 32];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int c = 0; c < D / 32; ++c) acc[t][c] = f32x16_t{};
  float m_run[NT], l_run[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) { m_run[t] = -INFINITY; l_run[t] = 0.0f; }
  const float tau = LAZY_LOG2 / scale_log2;

  const int row = bh * g.NB + i;
  const int e_end = uniform(row_ptr[row + 1]);
  int e_ld = uniform(row_ptr[row]);

  // Loader role.  Load instruction n of this wave fills slots
  // [64*(wave*IPW + n), +64) of a tile: lane L writes row
  // r_n = (wave*IPW + n)*ROWS_PER_INST + L/PARTS, slot L%PARTS, which holds
  // piece (L%PARTS) ^ swz(r_n) of that key's token row.  When a stage spans
  // whole rows of the nominal box (KS a multiple of bw, and KS and bh*bw
  // multiples of one another) the source offset inside a nominal block is
  // the offset in the first stage plus a wave-uniform step per stage.
  const int nom_hw = g.bh * g.bw;
  const bool stage_rows = (KS % g.bw == 0) && (KS % nom_hw == 0 || nom_hw % KS == 0);
  // Offset of each 32-key stage slot of a nominal block from its origin.
  uint32_t slot_off[4];
#pragma unroll
  for (int sl = 0; sl < 4; ++sl) {
    const int u = sl * KS, ut = u / nom_hw, uh = (u - ut * nom_hw) / g.bw;
    slot_off[sl] = (uint32_t)uniform((ut * g.H + uh) * g.W * D * 2);
  }
  int ld_row[C::IPW];
  uint32_t ld_piece[C::IPW], ld_rel[C::IPW];
#pragma unroll
  for (int n = 0; n < C::IPW; ++n) {
    const int r = (wave * C::IPW + n) * C::ROWS_PER_INST + lane / PARTS;
    ld_row[n] = r;
    ld_piece[n] = (uint32_t)(((lane % PARTS) ^ swz<PARTS>(r)) * 16);
    const int ut = r / nom_hw, rr = r - ut * nom_hw;
    const int uh = rr / g.bw, uw = rr - uh * g.bw;
    ld_rel[n] = (uint32_t)((ut * g.H * g.W + uh * g.W + uw) * D * 2) + ld_piece[n];
  }

  // Loader cursor: the next stage to fetch is (entry e_ld, tokens from c_ld).
  int c_ld = 0;
  KeyBlock blk;
  blk.nj = 0;
  if (e_ld < e_end) blk = open_block<D>(g, col_idx, e_ld, stage_rows);

  // Issue the stage at the cursor as direct-to-LDS loads into buffer BUF and
  // advance; NV receives its valid key count (0 when the row is exhausted).
  // Rows past the block's end read out of range and land as zeros.
#define VSA_LOAD_STAGE(BUF, NV)                                                               \
  do {                                                                                        \
    if (e_ld < e_end) {                                                                       \
      const int nv_ = uniform(min(KS, blk.nj - c_ld));                                        \
      const bool fast_ = blk.nominal;                                                         \
      const int sl_ = c_ld >> 5;                                                              \
      const uint32_t step_ = blk.jbase + (sl_ == 0 ? slot_off[0] : sl_ == 1 ? slot_off[1]     \
                                           : sl_ == 2 ? slot_off[2] : slot_off[3]);           \
      const uint32_t kt_ = (uint32_t)uniform((int)(lds0 + (BUF) * 2 * C::TILE_BYTES + wave * C::IPW * 1024)); \
      _Pragma("unroll") for (int n = 0; n < C::IPW; ++n) {                                     \
        uint32_t off = fast_ ? step_ + ld_rel[n]                                              \
                             : (uint32_t)blk.map(c_ld + ld_row[n]) * (D * 2) + ld_piece[n];   \
        off = ld_row[n] < nv_ ? off : 0x80000000u;                                            \
        dma16(krs, kt_ + n * 1024, off);                                                      \
        dma16(vrs, kt_ + C::TILE_BYTES + n * 1024, off);                                      \
      }                                                                                       \
      (NV) = nv_;                                                                             \
      c_ld = uniform(c_ld + KS);                                                              \
      if (c_ld >= blk.nj) {                                                                   \
        c_ld = 0;                                                                             \
        e_ld = uniform(e_ld + 1);                                                             \
        if (e_ld < e_end) blk = open_block<D>(g, col_idx, e_ld, stage_rows);                  \
      }                                                                                       \
    } else {                                                                                  \
      (NV) = 0;                                                                               \
    }                                                                                         \
  } while (0)

  // Per-lane fragment byte offsets within a stage's tiles.
  // K (A operand of S^T = K Q^T): row l32, piece 2*ks + g2.
  uint32_t kaddr[D / 16];
  {
    const int sw = swz<PARTS>(l32);
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) kaddr[ks] = (uint32_t)((l32 * PARTS + ((2 * ks + g2) ^ sw)) * 16);
  }
  // V^T (A operand of O^T = V^T P^T) through the transposing read: lane
  // (r16, dhalf, g2) addresses row 16*m + 8*hi + 4*g2 + r16/4 and the 8 bytes
  // at byte 64*c + 32*dhalf + 8*(r16 & 3) of it.
  uint32_t vaddr[2][D / 32];
  {
    const int r16 = lane & 15, dhalf = (lane >> 4) & 1;
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) {
      const int r = 8 * hi + 4 * g2 + (r16 >> 2);
      const int sw = swz<PARTS>(r);
#pragma unroll
      for (int c = 0; c < D / 32; ++c) {
        const int byte = 64 * c + 32 * dhalf + 8 * (r16 & 3);
        vaddr[hi][c] = (uint32_t)(r * PARTS * 16 + (((byte >> 4) ^ sw) << 4) + (byte & 15));
      }
    }
  }

  // Prologue: stages 0 and 1 issued into buffers 0 and 1.
  int nv0 = 0, nv1 = 0;
  VSA_LOAD_STAGE(0, nv0);
  VSA_LOAD_STAGE(1, nv1);
  const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};

  // Iteration t: QK, softmax and PV of stage t (buffer t%3) while stages
  // t+1 and t+2 are in flight; stage t+2 goes into buffer (t+2)%3, last read
  // in iteration t-1, which every wave finished before this iteration's
  // barrier.  Three workgroups share a compute unit, so other waves fill
  // the matrix cores while one runs its softmax.  The loop is unrolled over
  // the ring so buffer offsets are constants.
#define VSA_ITER(BC)                                                                          \
  {                                                                                           \
    /* This wave's loads of stage t are complete (stage t+1's may still be */                 \
    /* in flight); the barrier makes every wave's visible. */                                 \
    if (nv1 > 0) __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * C::IPW));                           \
    else __builtin_amdgcn_s_waitcnt(0x0F70);                                                  \
    __syncthreads();                                                                          \
    int nv2 = 0;                                                                              \
    VSA_LOAD_STAGE(((BC) + 2) % NBUF, nv2);                                                   \
    if (ntiles > 0) {                                                                         \
      const uint8_t* kt = lds + (BC) * 2 * C::TILE_BYTES;                                     \
      const uint8_t* vt = kt + C::TILE_BYTES;                                                 \
      f32x16_t s = f32x16_t{};                                                                \
      _Pragma("unroll") for (int ks = 0; ks < D / 16; ++ks) {                                  \
        const u32x4_t kf = *reinterpret_cast<const u32x4_t*>(kt + kaddr[ks]);                 \
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, kf), qf[0][ks], s, 0, 0, 0); \
      }                                                                                       \
      const float mb = softmax_prep<D>(s, nv0, g2, scale_log2, tau, m_run[0], l_run[0], acc[0]); \
      _Pragma("unroll") for (int m = 0; m < 2; ++m) {                                          \
        f32x8_t pf;                                                                           \
        _Pragma("unroll") for (int q8 = 0; q8 < 8; ++q8)                                       \
          pf[q8] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * m + q8], scale_log2, -mb));    \
        const bf16x8_t pb = __builtin_convertvector(pf, bf16x8_t);                            \
        _Pragma("unroll") for (int q8 = 0; q8 < 8; q8 += 2) {                                  \
          const bf16x2_t pr = {pb[q8], pb[q8 + 1]};                                           \
          l_run[0] = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, l_run[0], false);              \
        }                                                                                     \
        _Pragma("unroll") for (int c = 0; c < D / 32; ++c) {                                   \
          const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(                         \
              (lds_i16x4_t*)(vt + vaddr[0][c] + m * 16 * PARTS * 16));                        \
          const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(                         \
              (lds_i16x4_t*)(vt + vaddr[1][c] + m * 16 * PARTS * 16));                        \
          const i16x8_t both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);       \
          acc[0][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(                                \
              __builtin_bit_cast(bf16x8_t, both), pb, acc[0][c], 0, 0, 0);                    \
        }                                                                                     \
      }                                                                                       \
    }                                                                                         \
    nv0 = nv1; nv1 = nv2;                                                                     \
  }

  static_assert(NBUF == 3, "the loop below is unrolled over a three-stage ring");
  while (true) {
    if (nv0 == 0) break;
    VSA_ITER(0);
    if (nv0 == 0) break;
    VSA_ITER(1);
    if (nv0 == 0) break;
    VSA_ITER(2);
  }
#undef VSA_ITER
#undef VSA_LOAD_STAGE

  // Epilogue: O = O^T / l, rounded to bf16, stored at the query's raster row.
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const float l_tot = l_run[t] + __shfl_xor(l_run[t], 32, 64);
    const int qtok = QPW * wave + 32 * t + l32;
    if (qtok < ni) {
      const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
      uint16_t* op = o + head_off + (size_t)qmap(qtok) * D;
#pragma unroll
      for (int c = 0; c < D / 32; ++c) {
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const int d = c * 32 + 8 * gq + 4 * g2;
          u32x2_t w;
          w[0] = bf16_pair(f32_to_bf16(acc[t][c][4 * gq + 0] * inv), f32_to_bf16(acc[t][c][4 * gq + 1] * inv));
          w[1] = bf16_pair(f32_to_bf16(acc[t][c][4 * gq + 2] * inv), f32_to_bf16(acc[t][c][4 * gq + 3] * inv));
          *reinterpret_cast<u32x2_t*>(op + d) = w;
        }
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
      hipLaunchKernelGGL(attn_bf16_kernel<128>, dim3(nwg), dim3(THREADS), 0, st, (const uint16_t*)q,
                         (const uint16_t*)k, (const uint16_t*)v, (uint16_t*)o, row_ptr, col_idx, g, sl2);
    else
      hipLaunchKernelGGL(attn_bf16_kernel<64>, dim3(nwg), dim3(THREADS), 0, st, (const uint16_t*)q,
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
