// Kernel launchers of the gfx950 library (host-callable, enqueue only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "vsa.h"
#include "vsa_device.h"

namespace vsa {

// Per-head selection parameters, passed by value as a kernel argument.
struct SelectArgs {
  union {
    int32_t k[VSA_MAX_HEADS];   // Top-K: kept blocks per query-block row of head h
    float p[VSA_MAX_HEADS];     // Top-P: cumulative threshold of head h
  };
  int32_t off[VSA_MAX_HEADS];   // Top-K: sum of k over heads before h
  int64_t batch_stride;         // Top-K: NB * sum_h k_h, col_idx entries per batch item
  int64_t rows;                 // B * heads * NB
  const float* table;           // static heads: scores [heads][NB][NB]
  int16_t win[VSA_MAX_HEADS];   // temporal window of head h, -1: none
  int8_t kind[VSA_MAX_HEADS];   // head option: 0 dynamic, 1 static, 2 dense
  int32_t words;                // 64-bit bitmap words per row
  int32_t sink;                 // key blocks 0 .. sink-1 kept by every row
  int32_t bitmap;               // rows vary: write bitmaps and counts for scan + fill
  float scale;                  // Top-P logit scale
  int32_t topp;                 // selection mode: 0 Top-K, 1 Top-P
};

// Per-candidate layout of the block SICS in the scheme workspace: candidate
// c holds [2][BH][nb[c]] floats (Q, then K) starting at float offset off[c].
struct SchemeArgs {
  int32_t n;
  int32_t nb[VSA_MAX_SCHEMES];
  int64_t off[VSA_MAX_SCHEMES];
};

// Heads a launch covers.  Row bh = b*n + s of the launch reads and writes
// tensor head b*total + h[s] of tensors that hold `total` heads; identity
// when a launch covers every head in order (n == total, h unused).
struct HeadMap {
  int32_t n = 1;
  int32_t total = 1;
  int32_t identity = 1;
  int16_t h[VSA_MAX_HEADS] = {};
  __device__ __host__ int tensor_bh(int bh) const {
    if (identity) return bh;
    const int b = bh / n;
    return b * total + h[bh - b * n];
  }
};

// Block summaries an estimator reads, each float32 [BH][NB][D]: mean: qa =
// query means, ka = key means; DSA: qa = query midpoints, ka/kb = key
// max/min; DSA2: qa/qb = query max/min, ka/kb = key max/min.  With kt set
// the key summaries are channel-major instead, [BH][D][NB], so that a wave
// reading one channel of 64 consecutive key blocks touches 256 contiguous
// bytes (the planner's own layout; callers' centroids stay [BH][NB][D]).
struct Summaries {
  const float* qa;
  const float* qb;
  const float* ka;
  const float* kb;
  int32_t kt = 0;
};

// Block means of x0 into out0 and, when x1 is not null, of x1 into out1
// ([BH][NB][D], or [BH][D][NB] for out1 when out1_channel_major).
hipError_t launch_pool(const void* x0, float* out0, const void* x1, float* out1, int dtype, int D,
                       const DGeo& g, int BH, hipStream_t st, bool out1_channel_major = false,
                       const HeadMap* hm = nullptr);
// Block means as launch_pool (x1's channel-major) and, in the same pass,
// every block's SICS (sum of the pairwise cosine similarities of its
// tokens) of x0 into sics0 and of x1 into sics1 ([BH][NB]).
hipError_t launch_pool_sics(const void* x0, float* out0, const void* x1, float* out1, float* sics0, float* sics1,
                            int dtype, int D, const DGeo& g, int BH, hipStream_t st);
// dst[bh][0 .. per) = src[tensor_bh(bh)][0 .. per) for the BH rows of a
// launch (per a multiple of 4 floats).
hipError_t launch_gather_rows(const float* src, float* dst, int per, const HeadMap& hm, int BH, hipStream_t st);
// Block max/min of x0 (or, with mid0, the midpoint into max0) and of x1
// (channel-major when out1_channel_major and not mid1).
hipError_t launch_extremes(const void* x0, float* max0, float* min0, int mid0, const void* x1, float* max1,
                           float* min1, int mid1, int dtype, int D, const DGeo& g, int BH, hipStream_t st,
                           bool out1_channel_major = false, const HeadMap* hm = nullptr);
// est: 0 mean, 1 DSA, 2 DSA2 (vsa_estimator).
hipError_t launch_score_select(const Summaries& sm, int est, const DGeo& g, int D, int heads, int BH,
                               const SelectArgs& sa, int32_t* row_ptr, int32_t* col_idx, int32_t* counts,
                               uint64_t* bits, hipStream_t st);
hipError_t launch_scan_fill(const int32_t* counts, const uint64_t* bits, int32_t* row_ptr,
                            int32_t* col_idx, int64_t R, int words, int NB, int64_t capacity,
                            hipStream_t st);
hipError_t launch_scores(const Summaries& sm, int est, float* out, int NB, int D, int BH, hipStream_t st);
// contiguous: give each XCD one contiguous run of rows (heads of equal
// work); otherwise an equal contiguous slice of every head.
hipError_t launch_attn(const void* q, const void* k, const void* v, void* o, int dtype, int D,
                       const int32_t* row_ptr, const int32_t* col_idx, const DGeo& g, int BH,
                       float scale, bool contiguous, hipStream_t st, const HeadMap* hm = nullptr);
// Per-block SICS of x0 into out0 and, when x1 is not null, of x1 into out1.
hipError_t launch_sics(const void* x0, float* out0, const void* x1, float* out1, int dtype, int D,
                       const DGeo& g, int BH, hipStream_t st);
hipError_t launch_scheme_select(const float* sics, const SchemeArgs& sa, int BH, float* scores,
                                int32_t* choice, hipStream_t st);
hipError_t launch_permute(const void* x, void* xb, int elt, int D, const DGeo& g, int BH, int P,
                          bool inverse, hipStream_t st);

}  // namespace vsa
