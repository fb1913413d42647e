// Block-sparse flash attention for gfx950 (SPADE arXiv 2608.03335, 2.2 Eq. 2
// and 3.3): for each query block, only the key blocks listed in its CSR row
// are visited, with an online softmax, and the output is written straight
// back to raster order (the layout restore of 3.3 is fused into the store;
// the gather into the blocked layout is fused into the loads).
//
// bf16 path.  One workgroup of 4 waves per (batch*head, query block); wave w
// owns query tokens [32w, 32w+32) of the block; two workgroups share a
// compute unit (two waves per SIMD, up to 256 VGPRs each).  The kept key
// blocks of the row are cut into 32-key tiles (a block of n tokens gives
// ceil(n/32) tiles) and walked in stages of two consecutive tiles, which may
// come from two blocks.  Per tile:
//   S^T (keys x queries) = K Q^T     on v_mfma_f32_32x32x16_bf16, Q in VGPRs,
//                                    K from LDS (two 32-key tiles)
//   online softmax in float32        the lane owns one query column, so the
//                                    row max/sum are in-lane plus one swap
//                                    with the lane 32 away
//   O^T (d x queries) += V^T P^T     V^T fragments read from the row-major
//                                    V tile with the transposing LDS read,
//                                    P^T straight from the S^T accumulators
//                                    (same lane, same keys)
// Software pipeline at 32-key tile granularity: while a wave turns one
// tile's scores into probabilities and accumulates them into O, it already
// computes the scores of the next tile, so matrix and vector work of the
// same wave interleave.  K and V stages arrive through direct-to-LDS buffer
// loads (rows past a block's end read out of range and land as zeros) one
// iteration ahead, double-buffered: the two 32-key K tiles of a stage live
// in separate rings, so K(t+2) tile 0 and K(t+1) tile 1 can both be issued at
// the top of iteration t, as soon as their slots are free.
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

constexpr int KS = 64;              // keys per stage
constexpr int WAVES = 4;            // waves per workgroup: 128 query tokens in all
constexpr int THREADS = 64 * WAVES;
constexpr float LAZY_LOG2 = 8.0f;   // running max is only raised when a row max exceeds it by 2^8

// LDS tiles hold token rows of D bf16 (PARTS 16-byte pieces) with no
// padding; piece pc of row r sits at slot pc ^ swz(r) of the row.  The
// swizzle keeps both fragment reads conflict-free: the K reads (16 lanes,
// 16 rows, one piece) and the transposing V reads (32 lanes, 4 rows, 4
// consecutive pieces).  It depends on r mod 16 only.
template <int PARTS>
__device__ __forceinline__ int swz(int r) {
  if constexpr (PARTS == 16) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

template <int D>
struct AttnCfg {
  static constexpr int PARTS = D / 8;                  // 16-byte pieces per token row
  static constexpr int ROW = D * 2;                    // bytes per token row
  static constexpr int TILE = KS * ROW;                // one K or V stage
  static constexpr int ROWS_PER_INST = 64 / PARTS;     // rows one wave load instruction fills
  static constexpr int IPW = KS / ROWS_PER_INST / WAVES;  // load instructions per wave per tile
  static_assert(IPW >= 1 && IPW * ROWS_PER_INST * WAVES == KS, "stage rows must split evenly over the waves");
};

__device__ inline int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Buffer resource over `bytes` bytes from `base` (stride 0, raw offsets):
// loads at or past `bytes` return zeros instead of faulting.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc4(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(((uint64_t)hi << 32) | lo), (short)0,
                                           (int)bytes, 0x00020000);
}

// 16 bytes per lane from a raw buffer straight into LDS at lds_base + 16*lane
// (out-of-range offsets write zeros), through the compiler's LDS-DMA
// builtin: the compiler sets M0 itself and folds constant LDS offsets into
// the instruction.  It adds no waits of its own here; completion is awaited
// explicitly (vmcnt) before the barrier that publishes a stage.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t lds_base, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(uintptr_t)lds_base, 16,
                                           (int)voff, 0, 0, 0);
}

__device__ inline uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

__device__ inline uint32_t bf16_pair(uint16_t lo, uint16_t hi) { return (uint32_t)lo | ((uint32_t)hi << 16); }

// Column max over the two halves of the wave: lanes l and l^32 hold the
// same query column (different keys); afterwards every lane has the max.
__device__ __forceinline__ float half_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  // r[0] holds the lower half's value in both halves, r[1] the upper half's.
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// One 32-key x 32-query tile of S^T from the K rows at kt (LDS).
template <int D>
__device__ __forceinline__ f32x16_t qk_tile(const uint8_t* kt, const uint32_t (&kaddr)[D / 16],
                                            const bf16x8_t (&qf)[D / 16]) {
  f32x16_t s = f32x16_t{};
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    const u32x4_t kf = *reinterpret_cast<const u32x4_t*>(kt + kaddr[ks]);
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, kf), qf[ks], s, 0, 0, 0);
  }
  return s;
}

// Lane (l32, g2) holds, in register rr of S^T tile kt, key
// 32*kt + 8*(rr/4) + 4*g2 + rr%4 of the stage; keys at or past nv get -inf.
__device__ __forceinline__ void mask_tile(f32x16_t& s, int kt, int nv, int g2x4) {
#pragma unroll
  for (int rr = 0; rr < 16; ++rr) {
    const int thr = nv - (32 * kt + 8 * (rr >> 2) + (rr & 3));
    s[rr] = g2x4 < thr ? s[rr] : -INFINITY;
  }
}

// Max of the 16 scores this lane holds in an S^T tile (a v_max3 tree).
__device__ __forceinline__ float tile_max(const f32x16_t& s) {
  const float a = fmaxf(fmaxf(s[0], s[1]), s[2]), b = fmaxf(fmaxf(s[3], s[4]), s[5]);
  const float c = fmaxf(fmaxf(s[6], s[7]), s[8]), d = fmaxf(fmaxf(s[9], s[10]), s[11]);
  const float e = fmaxf(fmaxf(s[12], s[13]), s[14]);
  return fmaxf(fmaxf(fmaxf(a, b), c), fmaxf(fmaxf(d, e), s[15]));
}

// Probabilities of registers [8h, 8h+8) of an S^T tile, rounded to bf16 for
// the PV product; the row sum takes the rounded values, so that it matches
// what is multiplied.
__device__ __forceinline__ bf16x8_t probs(const f32x16_t& s, int h, float sl2, float mb, float& l) {
  f32x8_t pf;
#pragma unroll
  for (int q8 = 0; q8 < 8; ++q8) pf[q8] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * h + q8], sl2, -mb));
  const bf16x8_t pb = __builtin_convertvector(pf, bf16x8_t);
  const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
  for (int q8 = 0; q8 < 8; q8 += 2) {
    const bf16x2_t pr = {pb[q8], pb[q8 + 1]};
    l = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, l, false);
  }
  return pb;
}

// O^T += V^T P^T over the 16 keys of k-step m of a stage (keys 16m + [0, 16)
// in the order the S^T registers hold them).
template <int D>
__device__ __forceinline__ void pv_step(const uint8_t* vt, const uint32_t (&vaddr)[2][D / 32], int m,
                                        const bf16x8_t& pb, f32x16_t (&acc)[D / 32]) {
#pragma unroll
  for (int c = 0; c < D / 32; ++c) {
    const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(vt + vaddr[0][c] + m * 16 * D * 2));
    const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(vt + vaddr[1][c] + m * 16 * D * 2));
    const i16x8_t both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, both), pb, acc[c], 0, 0, 0);
  }
}

template <int D>
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    uint16_t* __restrict__ o, const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx,
    DGeo g, float scale_log2, int contiguous, HeadMap hm) {
  using C = AttnCfg<D>;
  constexpr int PARTS = C::PARTS, IPW = C::IPW, ROW = C::ROW, TILE = C::TILE;
  constexpr int RPI = C::ROWS_PER_INST;
  constexpr int RSTEP = WAVES * RPI;       // stage rows between a wave's consecutive load instructions
  constexpr int HALF = TILE / 2;           // one 32-key K tile
  constexpr int IPH = IPW / 2;             // load instructions per wave per 32-key tile
  static_assert(RSTEP % 16 == 0, "the swizzle of a lane's rows must not depend on the instruction");
  // LDS: K tile-0 ring (2 x HALF), K tile-1 ring (2 x HALF), V ring (2 x TILE).
  constexpr int A0 = 0, B0 = 2 * HALF, V0 = 4 * HALF;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[4 * TILE];
  // Byte offset (raster token offset * ROW) of token u of a block from the
  // block's origin, for the four (h, w) extent combinations a block can
  // have (nominal or cut short at the grid edge in each of h and w).
  __shared__ uint32_t tok_tbl[4 * VSA_MAX_BLOCK_TOKENS];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform(tid >> 6);   // wave-uniform, so per-wave branches stay scalar
  const int l32 = lane & 31, g2 = lane >> 5, g2x4 = 4 * g2;

  {
    const int eh_edge = g.H - (g.nbh - 1) * g.bh, ew_edge = g.W - (g.nbw - 1) * g.bw;
    for (int idx = tid; idx < 4 * VSA_MAX_BLOCK_TOKENS; idx += THREADS) {
      const int type = idx / VSA_MAX_BLOCK_TOKENS, u = idx % VSA_MAX_BLOCK_TOKENS;
      const uint32_t eh = (type & 1) ? eh_edge : g.bh, ew = (type & 2) ? ew_edge : g.bw;
      const uint32_t ehw = eh * ew;
      const uint32_t ut = u / ehw, rem = u - ut * ehw, uh = rem / ew, uw = rem - uh * ew;
      // Entries past a block's token count are never used.
      tok_tbl[idx] = ((ut * (uint32_t)g.H + uh) * (uint32_t)g.W + uw) * (uint32_t)ROW;
    }
  }

  // Workgroups are dealt round-robin to the 8 XCDs, and an XCD runs its
  // workgroups in order.  Neighbouring query blocks of a head keep
  // overlapping key blocks, so each XCD gets contiguous query blocks to
  // share its L2:
  //  * heads of equal work: one contiguous run of (head, query block) rows;
  //  * otherwise an equal contiguous slice of every head, head after head,
  //    so a heavy head (dense, or a high keep rate) is spread over all XCDs.
  //    Head h's NB = 8a + bx rows give a or a + 1 to each XCD; the bx extra
  //    rows of head h go to XCDs (h*bx + t) mod 8, t < bx, which matches the
  //    hardware's deal of BH*NB workgroups exactly.
  const int nwg = gridDim.x;
  const int xcd = blockIdx.x & 7, loc = blockIdx.x >> 3;
  int bh, i;
  if (contiguous) {
    const int per = (nwg + 7) >> 3, rem = nwg & 7;
    const int logical = (rem == 0 || xcd < rem) ? xcd * per + loc : rem * per + (xcd - rem) * (per - 1) + loc;
    bh = logical / g.NB;
    i = logical - bh * g.NB;
  } else {
    const int NB = g.NB, BHn = nwg / NB;
    const int a = NB >> 3, bx = NB & 7;
    // Rows XCD xcd receives from heads 0 .. h-1.
    auto prefix = [&](int h) {
      const int t = h * bx - xcd;
      return a * h + (t > 0 ? (t + 7) >> 3 : 0);
    };
    int h = min((int)(((long long)loc * 8) / NB), BHn - 1);
    while (h > 0 && prefix(h) > loc) --h;
    while (h + 1 < BHn && prefix(h + 1) <= loc) ++h;
    int start = a * xcd;
    for (int x2 = 0; x2 < xcd; ++x2) start += (((x2 - h * bx) % 8 + 8) % 8) < bx ? 1 : 0;
    bh = h;
    i = start + loc - prefix(h);
  }
  bh = uniform(bh);
  i = uniform(i);
  const Box bi = block_box(g, i);
  const int ni = bi.n();
  TokenMap qmap;
  qmap.init(g, bi);
  const size_t head_off = (size_t)hm.tensor_bh(bh) * g.N * D;   // rows index the call's heads
  const uint32_t head_bytes = (uint32_t)g.N * D * 2u;
  const __amdgpu_buffer_rsrc_t krs = make_rsrc4(k + head_off, head_bytes);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc4(v + head_off, head_bytes);
  const uint32_t lds0 = (uint32_t)uniform((int)lds_addr(lds));

  // This wave's queries: tokens [32*qt, +32) of the block.  A block of at
  // most 64 query tokens would leave waves idle, so there the waves split
  // the key tiles instead: wave w takes query tile qt and key role kr --
  // kr 0 runs tile 0 of every stage (the pipelined step below), kr 1 tile 1
  // (one unpipelined step per stage) -- and the two partial softmax states
  // of a query tile are merged through LDS after the last stage.  With one
  // query tile, waves 2 and 3 stay idle.
  const int split = uniform(ni <= 64 ? 1 : 0);
  const int qtiles = (ni + 31) >> 5;
  const int qt = uniform(split ? (qtiles == 2 ? (wave & 1) : 0) : wave);
  const int kr = uniform(split ? (qtiles == 2 ? (wave >> 1) : (wave & 1)) : 0);
  const bool active = uniform(split ? (qtiles == 2 || wave < 2) : (32 * wave < ni)) != 0;
  // Q^T fragments (B operand): query column l32, channels 16*ks + 8*g2 + [0, 8).
  bf16x8_t qf[D / 16];
  {
    const int qtok = 32 * qt + l32;
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
  const float tau = LAZY_LOG2 / scale_log2;

  // Loader role.  Load instruction n of this wave covers stage row
  // lrow + n*RSTEP (lane L: lrow = wave*RPI + L/PARTS, 16-byte slot
  // L%PARTS, which holds piece (L%PARTS) ^ swz(row) of that key's token
  // row): instructions n < IPH fill K tile 0, the others K tile 1, and all
  // of them the V stage.
  const int lrow = wave * RPI + lane / PARTS;
  const uint32_t lpiece = (uint32_t)(((lane % PARTS) ^ swz<PARTS>(lrow)) * 16);

  // Loader cursor (wave-uniform): the next 32-key tile to fetch is tokens
  // [c_ld, c_ld + 32) of entry e_ld, a block with nj tokens, origin byte
  // offset jbase and extent type ltype (a byte offset into tok_tbl).  A
  // stage is two consecutive tiles of the row's tile sequence, so a stage
  // may take its tiles from two blocks (of at most 32 tokens each).  The
  // block ids of the next two entries are fetched ahead into jn1/jn2 by
  // scalar loads (the ids are wave-uniform).  A scalar load is waited on
  // through lgkmcnt, which the K/V loads to LDS do not touch: the id of a
  // vector load would be waited on through vmcnt, and that wait would also
  // cover the K/V direct-to-LDS loads of the stage just issued.
  // Entries are read only below e_end, inside the row.
  const int row = bh * g.NB + i;
  const int e_end = uniform(row_ptr[row + 1]);
  int e_ld = uniform(row_ptr[row]);
  const __attribute__((address_space(4))) int32_t* cid_s =
      (const __attribute__((address_space(4))) int32_t*)(uintptr_t)col_idx;
  int c_ld = 0, nj = 0;
  uint32_t jbase = 0, ltype = 0;
  int jn1 = 0, jn2 = 0;

#define VSA_OPEN_BLOCK(JRAW)                                                                  \
  do {                                                                                        \
    const int j_ = uniform(min(max((JRAW), 0), g.NB - 1)); /* a corrupt id stays in the head */ \
    const Box b_ = block_box_fast(g, j_);                                                     \
    nj = uniform(b_.n());                                                                     \
    jbase = (uint32_t)uniform(((b_.t0 * g.H + b_.h0) * g.W + b_.w0) * ROW);                   \
    ltype = (uint32_t)uniform(((b_.eh != g.bh ? 1 : 0) | (b_.ew != g.bw ? 2 : 0)) *            \
                              VSA_MAX_BLOCK_TOKENS * 4);                                      \
  } while (0)

  // Advance the cursor by one tile, opening the next block when this one is
  // exhausted.
#define VSA_ADVANCE()                                                                         \
  do {                                                                                        \
    c_ld = uniform(c_ld + 32);                                                                \
    if (c_ld >= nj) {                                                                         \
      c_ld = 0;                                                                               \
      e_ld = uniform(e_ld + 1);                                                               \
      if (e_ld < e_end) {                                                                     \
        VSA_OPEN_BLOCK(__builtin_amdgcn_readfirstlane(jn1));                                  \
        jn1 = jn2;                                                                            \
        if (e_ld + 2 < e_end) jn2 = cid_s[e_ld + 2];                                           \
      }                                                                                       \
    }                                                                                         \
  } while (0)

  // Per-lane source offsets of the stage at the cursor (two tiles): the
  // table reads are issued first, then PRE runs (DMA issue that does not
  // depend on them), then the offsets are formed into OFF; the tiles' valid
  // key counts go to NV0 and NV1 (0 for a tile past the row's end) and the
  // cursor advances by the tiles taken.
#define VSA_NEXT_STAGE(NV0, NV1, OFF, PRE)                                                    \
  do {                                                                                        \
    if (e_ld < e_end) {                                                                       \
      uint32_t t_[IPW];                                                                       \
      const int nv0_ = uniform(min(32, nj - c_ld));                                           \
      const uint32_t jb0_ = jbase;                                                            \
      {                                                                                       \
        const uint8_t* tp_ = reinterpret_cast<const uint8_t*>(tok_tbl) + ltype + c_ld * 4;   \
        _Pragma("unroll") for (int n = 0; n < IPH; ++n)                                        \
          t_[n] = *reinterpret_cast<const uint32_t*>(tp_ + (lrow + n * RSTEP) * 4);           \
      }                                                                                       \
      VSA_ADVANCE();                                                                          \
      int nv1_ = 0;                                                                           \
      uint32_t jb1_ = 0;                                                                      \
      if (e_ld < e_end) {                                                                     \
        nv1_ = uniform(min(32, nj - c_ld));                                                   \
        jb1_ = jbase;                                                                         \
        const uint8_t* tp_ = reinterpret_cast<const uint8_t*>(tok_tbl) + ltype + c_ld * 4;   \
        _Pragma("unroll") for (int n = IPH; n < IPW; ++n)                                      \
          t_[n] = *reinterpret_cast<const uint32_t*>(tp_ + (lrow + n * RSTEP - 32) * 4);      \
        VSA_ADVANCE();                                                                        \
      }                                                                                       \
      PRE;                                                                                    \
      _Pragma("unroll") for (int n = 0; n < IPH; ++n) (OFF)[n] = jb0_ + t_[n] + lpiece;        \
      if (nv0_ < 32) {                                                                        \
        _Pragma("unroll") for (int n = 0; n < IPH; ++n)                                        \
          (OFF)[n] = lrow < nv0_ - n * RSTEP ? (OFF)[n] : 0x80000000u;                        \
      }                                                                                       \
      if (nv1_ > 0) {                                                                         \
        _Pragma("unroll") for (int n = IPH; n < IPW; ++n) (OFF)[n] = jb1_ + t_[n] + lpiece;    \
        if (nv1_ < 32) {                                                                      \
          _Pragma("unroll") for (int n = IPH; n < IPW; ++n)                                    \
            (OFF)[n] = lrow < nv1_ - (n * RSTEP - 32) ? (OFF)[n] : 0x80000000u;               \
        }                                                                                     \
      } else {                                                                                \
        _Pragma("unroll") for (int n = IPH; n < IPW; ++n) (OFF)[n] = 0x80000000u;              \
      }                                                                                       \
      (NV0) = nv0_;                                                                           \
      (NV1) = nv1_;                                                                           \
    } else {                                                                                  \
      PRE;                                                                                    \
      (NV0) = 0;                                                                              \
      (NV1) = 0;                                                                              \
    }                                                                                         \
  } while (0)

  // Direct-to-LDS issue: K tile 0 / K tile 1 / V of a stage with offsets OFF
  // into the slot at LDS byte SLOT.
#define VSA_ISSUE_K0(SLOT, OFF)                                                               \
  do {                                                                                        \
    const uint32_t base_ = (uint32_t)uniform((int)(lds0 + (SLOT) + wave * 1024));             \
    _Pragma("unroll") for (int n = 0; n < IPH; ++n)                                            \
      dma16(krs, base_ + n * WAVES * 1024, (OFF)[n]);                                         \
  } while (0)
#define VSA_ISSUE_K1(SLOT, OFF)                                                               \
  do {                                                                                        \
    const uint32_t base_ = (uint32_t)uniform((int)(lds0 + (SLOT) + wave * 1024));             \
    _Pragma("unroll") for (int n = IPH; n < IPW; ++n)                                          \
      dma16(krs, base_ + (n - IPH) * WAVES * 1024, (OFF)[n]);                                 \
  } while (0)
#define VSA_ISSUE_V(SLOT, OFF)                                                                \
  do {                                                                                        \
    const uint32_t base_ = (uint32_t)uniform((int)(lds0 + (SLOT) + wave * 1024));             \
    _Pragma("unroll") for (int n = 0; n < IPW; ++n)                                            \
      dma16(vrs, base_ + n * WAVES * 1024, (OFF)[n]);                                         \
  } while (0)

  // Per-lane fragment byte offsets within a tile.
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

  __syncthreads();   // tok_tbl complete
  if (e_ld < e_end) {
    VSA_OPEN_BLOCK(cid_s[e_ld]);
    if (e_ld + 1 < e_end) jn1 = cid_s[e_ld + 1];
    if (e_ld + 2 < e_end) jn2 = cid_s[e_ld + 2];
  }

  // Prologue: all of stage 0 and K tile 0 of stage 1; S^T of stage 0 tile 0.
  uint32_t offA[IPW], offB[IPW];
  int nv0c = 0, nv1c = 0, nv0n = 0, nv1n = 0;   // valid keys of the tiles of stages t and t+1
  VSA_NEXT_STAGE(nv0c, nv1c, offA, (void)0);
  if (nv0c > 0) {
    VSA_ISSUE_K0(A0, offA);
    if (nv1c > 0) VSA_ISSUE_K1(B0, offA);
    VSA_ISSUE_V(V0, offA);
  }
  VSA_NEXT_STAGE(nv0n, nv1n, offB, (void)0);
  if (nv0n > 0) VSA_ISSUE_K0(A0 + HALF, offB);
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  __syncthreads();
  f32x16_t sc, st;   // scores of the tile to exponentiate next / the tile after it
  if (active && kr == 0 && nv0c > 0) {
    sc = qk_tile<D>(lds + A0, kaddr, qf);
    if (nv0c < 32) mask_tile(sc, 0, nv0c, g2x4);
    m_run = half_max(tile_max(sc));   // O and l are still zero: no rescale
  }

  // One 32-key tile step.  SC holds the scores of the tile whose V rows are
  // at VT (its max is already folded into m_run): its probabilities go into
  // O and l.  In the same block the scores of the next tile are computed
  // from the K rows at KT into SN (unconditionally; when there is no next
  // tile they are never used).  When HAS_NEXT, keys at or past NVN of that
  // tile are masked and its max is folded into m_run; O and l are rescaled
  // only when the max rose by more than 2^LAZY_LOG2 (a rare, wave-uniform
  // branch after the pipelined block).
#define VSA_STEP(SC, SN, VT, KT, HAS_NEXT, NVN)                                               \
  {                                                                                           \
    const float mb = m_run * scale_log2;                                                      \
    __builtin_amdgcn_s_setprio(3); /* matrix-heavy block: win issue ties with the other wave */ \
    SN = qk_tile<D>((KT), kaddr, qf);                                                         \
    const bf16x8_t p0 = probs(SC, 0, scale_log2, mb, l_run);                                  \
    const bf16x8_t p1 = probs(SC, 1, scale_log2, mb, l_run);                                  \
    pv_step<D>((VT), vaddr, 0, p0, acc);                                                      \
    pv_step<D>((VT), vaddr, 1, p1, acc);                                                      \
    float mx = half_max(tile_max(SN)); /* right for a full tile; redone below otherwise */    \
    __builtin_amdgcn_s_setprio(0);                                                            \
    if (HAS_NEXT) {                                                                           \
      const int nvn_ = (NVN);                                                                 \
      if (nvn_ < 32) {                                                                        \
        mask_tile(SN, 0, nvn_, g2x4);                                                         \
        mx = half_max(tile_max(SN));                                                          \
      }                                                                                       \
      if (__ballot(mx > m_run + tau) != 0ull) {                                               \
        const float m_new = fmaxf(m_run, mx);                                                 \
        const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * scale_log2);             \
        _Pragma("unroll") for (int c = 0; c < D / 32; ++c) acc[c] *= alpha;                    \
        l_run *= alpha;                                                                       \
        m_run = m_new;                                                                        \
      }                                                                                       \
    }                                                                                         \
  }

  // One unpipelined step over the 32-key tile of K rows at KT and V rows at
  // VT with NV valid keys (the key-split role kr 1): scores, mask, max with
  // the lazy rescale, then probabilities into O and l.  m_run starts at
  // -inf, so the first tile always takes the rescale, with alpha = 0.
#define VSA_SOLO(S, KT, VT, NV)                                                               \
  {                                                                                           \
    S = qk_tile<D>((KT), kaddr, qf);                                                          \
    if ((NV) < 32) mask_tile(S, 0, (NV), g2x4);                                               \
    const float mx = half_max(tile_max(S));                                                   \
    if (__ballot(mx > m_run + tau) != 0ull) {                                                 \
      const float m_new = fmaxf(m_run, mx);                                                   \
      const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * scale_log2);               \
      _Pragma("unroll") for (int c = 0; c < D / 32; ++c) acc[c] *= alpha;                      \
      l_run *= alpha;                                                                         \
      m_run = m_new;                                                                          \
    }                                                                                         \
    const float mb = m_run * scale_log2;                                                      \
    __builtin_amdgcn_s_setprio(3);                                                            \
    const bf16x8_t p0 = probs(S, 0, scale_log2, mb, l_run);                                   \
    const bf16x8_t p1 = probs(S, 1, scale_log2, mb, l_run);                                   \
    pv_step<D>((VT), vaddr, 0, p0, acc);                                                      \
    pv_step<D>((VT), vaddr, 1, p1, acc);                                                      \
    __builtin_amdgcn_s_setprio(0);                                                            \
  }

  // Iteration t (P = t % 2).  Resident: K(t) tile 1 in B slot P, K(t+1)
  // tile 0 in A slot 1-P, V(t) in V slot P, all issued an iteration earlier;
  // sc holds the scores of stage t tile 0.  After the barrier every wave is
  // done with iteration t-1, which last read A slot P (K(t) tile 0), B slot
  // 1-P (K(t-1) tile 1) and V slot 1-P (V(t-1)): V(t+1), K(t+1) tile 1 and
  // K(t+2) tile 0 go there.  A missing tile 1 (the row's last stage) reads
  // stale LDS, fully masked.
#define VSA_ITER(P, OFF_NEXT, OFF_NEW, COMPUTE)                                               \
  {                                                                                           \
    __builtin_amdgcn_s_waitcnt(0x0F70);                                                       \
    __syncthreads();                                                                          \
    int nv0nn = 0, nv1nn = 0;                                                                 \
    VSA_NEXT_STAGE(nv0nn, nv1nn, OFF_NEW, {                                                   \
      if (nv0n > 0) {                                                                         \
        VSA_ISSUE_V(V0 + (1 - (P)) * TILE, OFF_NEXT);                                         \
        if (nv1n > 0) VSA_ISSUE_K1(B0 + (1 - (P)) * HALF, OFF_NEXT);                          \
      }                                                                                       \
    });                                                                                       \
    if (nv0nn > 0) VSA_ISSUE_K0(A0 + (P) * HALF, OFF_NEW);                                    \
    if (active) {                                                                             \
      const uint8_t* ka_ = lds + A0 + (1 - (P)) * HALF;   /* K(t+1) tile 0 */                 \
      const uint8_t* kb_ = lds + B0 + (P) * HALF;         /* K(t) tile 1 */                   \
      const uint8_t* v0_ = lds + V0 + (P) * TILE;         /* V(t) rows 0..31 */               \
      COMPUTE                                                                                 \
    }                                                                                         \
    nv0c = nv0n; nv1c = nv1n;                                                                 \
    nv0n = nv0nn; nv1n = nv1nn;                                                               \
  }

  // Both tiles of every stage (a full query block), or one tile per stage
  // and role (the key split); two loops, so that neither path's registers
  // constrain the other's.
#define VSA_BOTH                                                                              \
  VSA_STEP(sc, st, v0_, kb_, true, nv1c)                                                      \
  VSA_STEP(st, sc, v0_ + 32 * ROW, ka_, nv0n > 0, nv0n)
#define VSA_ROLE                                                                              \
  if (kr == 0) {                                                                              \
    VSA_STEP(sc, st, v0_, ka_, nv0n > 0, nv0n)                                                \
    sc = st;                                                                                  \
  } else if (nv1c > 0) {                                                                      \
    VSA_SOLO(st, kb_, v0_ + 32 * ROW, nv1c)                                                   \
  }
  if (!split) {
    while (nv0c > 0) {
      VSA_ITER(0, offB, offA, VSA_BOTH);
      if (nv0c == 0) break;
      VSA_ITER(1, offA, offB, VSA_BOTH);
    }
  } else {
    while (nv0c > 0) {
      VSA_ITER(0, offB, offA, VSA_ROLE);
      if (nv0c == 0) break;
      VSA_ITER(1, offA, offB, VSA_ROLE);
    }
  }
#undef VSA_BOTH
#undef VSA_ROLE
#undef VSA_ITER
#undef VSA_SOLO
#undef VSA_STEP
#undef VSA_ISSUE_V
#undef VSA_ISSUE_K1
#undef VSA_ISSUE_K0
#undef VSA_NEXT_STAGE
#undef VSA_OPEN_BLOCK
#undef VSA_ADVANCE

  // Key split: the kr 1 wave of each query tile leaves O, m and l in LDS
  // (the rings are free once every wave is past the last stage); the kr 0
  // wave rescales both states to the larger max and adds them.  A wave that
  // saw no key (the kr 1 wave of a single-tile row, or both waves of an
  // empty row in an index built by hand) has m = -inf and gets weight 0; an
  // empty row keeps O = 0 and l = 0, as in the unsplit path.
  if (split) {
    constexpr int NREG = (D / 32) * 16;   // accumulator floats per lane
    static_assert(2 * (NREG + 2) * 64 * 4 <= 4 * TILE, "two exchange regions must fit in the rings");
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    __syncthreads();
    float* xch = reinterpret_cast<float*>(lds) + qt * (NREG + 2) * 64 + lane;
    if (active && kr == 1) {
#pragma unroll
      for (int c = 0; c < D / 32; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) xch[(c * 16 + r) * 64] = acc[c][r];
      xch[NREG * 64] = m_run;
      xch[(NREG + 1) * 64] = l_run;
    }
    __syncthreads();
    if (active && kr == 0) {
      const float m1 = xch[NREG * 64], l1 = xch[(NREG + 1) * 64];
      const float m = fmaxf(m_run, m1);
      const float a0 = m_run == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f((m_run - m) * scale_log2);
      const float a1 = m1 == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f((m1 - m) * scale_log2);
#pragma unroll
      for (int c = 0; c < D / 32; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[c][r] = acc[c][r] * a0 + xch[(c * 16 + r) * 64] * a1;
      l_run = l_run * a0 + l1 * a1;
    }
  }

  // Epilogue: O = O^T / l, rounded to bf16, stored at the query's raster row.
  if (kr == 0) {
    const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
    const int qtok = 32 * qt + l32;
    if (active && qtok < ni) {
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
}

// ---------------------------------------------------------------------------
// float32 path: one thread per query token, 32-key tiles staged in LDS,
// float32 dot products and an exact-exp online softmax updated once per
// group of keys.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(128) void attn_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    float* __restrict__ o, const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx,
    DGeo g, float scale, HeadMap hm) {
  constexpr int TK = 32;
  constexpr int SK = D == 64 ? 16 : 4;   // keys per score group (registers: q, o and the group's scores)
  static_assert(TK % SK == 0, "a score group must not run past the tile");
  __shared__ __attribute__((aligned(16))) float Ks[TK][D];   // every thread reads the same element: broadcasts
  __shared__ __attribute__((aligned(16))) float Vs[TK][D];
  const int tid = threadIdx.x;
  const int bh = blockIdx.x / g.NB, i = blockIdx.x - bh * g.NB;
  const Box bi = block_box(g, i);
  const int ni = bi.n();
  TokenMap qmap;
  qmap.init(g, bi);
  const size_t head_off = (size_t)hm.tensor_bh(bh) * g.N * D;
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
      // Stage the tile in 16-byte pieces, K then V, each tensor's loads all
      // issued before its stores; rows past nv repeat the last valid key
      // (finite, never used).
      constexpr int Q4 = D / 4, PER = TK * Q4 / 128;
      uint32_t src[PER];   // element offsets within the head
#pragma unroll
      for (int it = 0; it < PER; ++it) {
        const int idx = tid + it * 128, key = min(idx / Q4, nv - 1), part = idx - (idx / Q4) * Q4;
        src[it] = (uint32_t)kmap(c0 + key) * D + part * 4;
      }
      const float* kh = k + head_off;
      const float* vh = v + head_off;
      float4* ks4 = reinterpret_cast<float4*>(&Ks[0][0]);
      float4* vs4 = reinterpret_cast<float4*>(&Vs[0][0]);
      __syncthreads();   // the previous tile's readers are done with Ks and Vs
      float4 pc[PER];
#pragma unroll
      for (int it = 0; it < PER; ++it) pc[it] = *reinterpret_cast<const float4*>(kh + src[it]);
#pragma unroll
      for (int it = 0; it < PER; ++it) ks4[tid + it * 128] = pc[it];
#pragma unroll
      for (int it = 0; it < PER; ++it) pc[it] = *reinterpret_cast<const float4*>(vh + src[it]);
#pragma unroll
      for (int it = 0; it < PER; ++it) vs4[tid + it * 128] = pc[it];
      __syncthreads();
      // SK keys at a time: their dot products are independent chains, and
      // the running max and rescale are updated once per group.  Keys past
      // nv read stale LDS; their scores become -inf and they are skipped in
      // the accumulation (nv is the same for the whole workgroup).
      for (int k0 = 0; k0 < nv; k0 += SK) {
        float sv[SK];
#pragma unroll
        for (int x = 0; x < SK; ++x) sv[x] = 0.0f;
#pragma unroll
        for (int d = 0; d < D; ++d) {
#pragma unroll
          for (int x = 0; x < SK; ++x) sv[x] += qv[d] * Ks[k0 + x][d];
        }
        float mt = -INFINITY;
#pragma unroll
        for (int x = 0; x < SK; ++x) {
          sv[x] = k0 + x < nv ? sv[x] * scale : -INFINITY;
          mt = fmaxf(mt, sv[x]);
        }
        const float m_new = fmaxf(m_run, mt);
        const float alpha = expf(m_run - m_new);   // 0 on the first group (m_run = -inf)
        l_run *= alpha;
#pragma unroll
        for (int d = 0; d < D; ++d) ov[d] *= alpha;
#pragma unroll
        for (int x = 0; x < SK; ++x) {
          if (k0 + x < nv) {
            const float p = expf(sv[x] - m_new);
            l_run += p;
#pragma unroll
            for (int d = 0; d < D; ++d) ov[d] += p * Vs[k0 + x][d];
          }
        }
        m_run = m_new;
      }
    }
  }
  if (active) {
    float* op = o + head_off + (size_t)qmap(tid) * D;
    const float inv = l_run > 0.0f ? 1.0f / l_run : 0.0f;   // an empty row gives zeros
#pragma unroll
    for (int d = 0; d < D; ++d) op[d] = ov[d] * inv;
  }
}

hipError_t launch_attn(const void* q, const void* k, const void* v, void* o, int dtype, int D,
                       const int32_t* row_ptr, const int32_t* col_idx, const DGeo& g, int BH,
                       float scale, bool contiguous, hipStream_t st, const HeadMap* hm) {
  const HeadMap id;
  const HeadMap& m = hm ? *hm : id;
  const unsigned nwg = (unsigned)BH * (unsigned)g.NB;
  if (dtype == VSA_BF16) {
    const float sl2 = scale * 1.4426950408889634f;
    const int cont = contiguous ? 1 : 0;
    if (D == 128)
      hipLaunchKernelGGL(attn_bf16_kernel<128>, dim3(nwg), dim3(THREADS), 0, st, (const uint16_t*)q,
                         (const uint16_t*)k, (const uint16_t*)v, (uint16_t*)o, row_ptr, col_idx, g, sl2, cont, m);
    else
      hipLaunchKernelGGL(attn_bf16_kernel<64>, dim3(nwg), dim3(THREADS), 0, st, (const uint16_t*)q,
                         (const uint16_t*)k, (const uint16_t*)v, (uint16_t*)o, row_ptr, col_idx, g, sl2, cont, m);
  } else {
    if (D == 128)
      hipLaunchKernelGGL(attn_f32_kernel<128>, dim3(nwg), dim3(128), 0, st, (const float*)q,
                         (const float*)k, (const float*)v, (float*)o, row_ptr, col_idx, g, scale, m);
    else
      hipLaunchKernelGGL(attn_f32_kernel<64>, dim3(nwg), dim3(128), 0, st, (const float*)q,
                         (const float*)k, (const float*)v, (float*)o, row_ptr, col_idx, g, scale, m);
  }
  return hipGetLastError();
}

}  // namespace vsa
