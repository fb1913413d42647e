// C ABI entry points (declared in include/vsa.h): host validation, then
// kernel launches on the caller's stream.  No allocation, no device
// synchronization.  The only global state is the static plan workspace of
// vsa_plan_noalloc and its per-device address table (end of this file).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "vsa.h"
#include "vsa_host.h"
#include "vsa_kernels.h"

using namespace vsa;

namespace {

// ceil(2^32 / d) for 2 <= d < 2^16; 0 stands for d = 1.
uint32_t div_magic_for(uint32_t d) {
  if (d <= 1) return 0u;
  return (uint32_t)(((uint64_t(1) << 32) + d - 1) / d);
}

DGeo to_dgeo(const Geo& g) {
  DGeo d;
  d.T = g.T; d.H = g.H; d.W = g.W;
  d.bt = g.bt; d.bh = g.bh; d.bw = g.bw;
  d.nbt = g.nbt; d.nbh = g.nbh; d.nbw = g.nbw;
  d.NB = g.NB; d.N = g.N;
  d.magic_hw = div_magic_for(uint32_t(g.nbh * g.nbw));
  d.magic_w = div_magic_for(uint32_t(g.nbw));
  return d;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

vsa_status hip_status(hipError_t e) { return e == hipSuccess ? VSA_OK : VSA_ERR_HIP; }

// Enqueue the block summaries of the estimator into the workspace regions
// ps.off_sum and describe them for the scoring kernels.
// With qmeans/kmeans (the block means of every tensor head, as
// vsa_select_scheme_means leaves them), the means of the call's heads are
// gathered from there instead of being computed from q and k.
hipError_t summarize(const void* q, const void* k, const vsa_shape* shape, const PlanSizes& ps, char* w,
                     const DGeo& dg, int BH, hipStream_t st, Summaries* sm, const HeadMap* hm = nullptr,
                     const float* qmeans = nullptr, const float* kmeans = nullptr) {
  float* s0 = reinterpret_cast<float*>(w + ps.off_sum[0]);
  float* s1 = reinterpret_cast<float*>(w + ps.off_sum[1]);
  float* s2 = ps.n_sum > 2 ? reinterpret_cast<float*>(w + ps.off_sum[2]) : nullptr;
  float* s3 = ps.n_sum > 3 ? reinterpret_cast<float*>(w + ps.off_sum[3]) : nullptr;
  if (ps.estimator == VSA_EST_MEAN) {
    *sm = Summaries{s0, nullptr, s1, nullptr, 1};
    if (qmeans) {
      const HeadMap id;
      const HeadMap& m = hm ? *hm : id;
      hipError_t e = launch_gather_rows(qmeans, s0, dg.NB * shape->D, m, BH, st);
      if (e == hipSuccess) e = launch_gather_rows(kmeans, s1, dg.NB * shape->D, m, BH, st);
      return e;
    }
    return launch_pool(q, s0, k, s1, shape->dtype, shape->D, dg, BH, st, true, hm);
  }
  if (ps.estimator == VSA_EST_DSA) {
    *sm = Summaries{s0, nullptr, s1, s2, 1};
    return launch_extremes(q, s0, nullptr, 1, k, s1, s2, 0, shape->dtype, shape->D, dg, BH, st, true, hm);
  }
  *sm = Summaries{s0, s1, s2, s3, 1};
  return launch_extremes(q, s0, s1, 0, k, s2, s3, 0, shape->dtype, shape->D, dg, BH, st, true, hm);
}

// Head list of a call over tensors with `total` heads: n distinct heads,
// each in [0, total), at most VSA_MAX_HEADS.
vsa_status make_head_map(const int32_t* heads, int n, int total, HeadMap* hm) {
  if (!heads || n < 1 || total < 1 || n > total) return VSA_ERR_INVALID_ARG;
  if (n > VSA_MAX_HEADS) return VSA_ERR_UNSUPPORTED;
  if (total > 32767) return VSA_ERR_UNSUPPORTED;
  bool seen[VSA_MAX_HEADS] = {};
  bool identity = n == total;
  for (int s2 = 0; s2 < n; ++s2) {
    const int h = heads[s2];
    if (h < 0 || h >= total) return VSA_ERR_INVALID_ARG;
    if (h < VSA_MAX_HEADS) {
      if (seen[h]) return VSA_ERR_INVALID_ARG;
      seen[h] = true;
    } else {
      for (int t = 0; t < s2; ++t)
        if (heads[t] == h) return VSA_ERR_INVALID_ARG;
    }
    hm->h[s2] = static_cast<int16_t>(h);
    identity = identity && h == s2;
  }
  hm->n = n;
  hm->total = total;
  hm->identity = identity ? 1 : 0;
  return VSA_OK;
}

}  // namespace

extern "C" {

const char* vsa_status_str(vsa_status s) {
  switch (s) {
    case VSA_OK: return "ok";
    case VSA_ERR_INVALID_ARG: return "invalid argument";
    case VSA_ERR_UNSUPPORTED: return "unsupported shape or size";
    case VSA_ERR_WORKSPACE: return "workspace too small";
    case VSA_ERR_CAPACITY: return "index capacity too small";
    case VSA_ERR_SHAPE_MISMATCH: return "index does not match the shape";
    case VSA_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

vsa_status vsa_query(const vsa_shape* shape, const float* density, int n_density, int window_t,
                     int64_t* row_ptr_len, int64_t* col_capacity, size_t* plan_ws, size_t* attn_ws) {
  try {
    PlanSizes ps;
    vsa_status st = plan_sizes(shape, density, n_density, window_t, &ps);
    if (st != VSA_OK) return st;
    if (row_ptr_len) *row_ptr_len = ps.rows + 1;
    if (col_capacity) *col_capacity = ps.capacity;
    if (plan_ws) *plan_ws = ps.ws;
    if (attn_ws) *attn_ws = 0;
    return VSA_OK;
  } catch (...) {
    return VSA_ERR_INVALID_ARG;
  }
}

vsa_status vsa_query_select(const vsa_shape* shape, const vsa_select* sel, int64_t* row_ptr_len,
                            int64_t* col_capacity, size_t* plan_ws) {
  try {
    PlanSizes ps;
    vsa_status st = select_sizes(shape, sel, &ps);
    if (st != VSA_OK) return st;
    if (row_ptr_len) *row_ptr_len = ps.rows + 1;
    if (col_capacity) *col_capacity = ps.capacity;
    if (plan_ws) *plan_ws = ps.ws;
    return VSA_OK;
  } catch (...) {
    return VSA_ERR_INVALID_ARG;
  }
}

}  // extern "C"

namespace {

// Enqueue a plan whose sizes and per-head parameters are in ps: summaries
// (when a head is dynamic), scoring + selection, then scan + fill when rows
// vary in length.  Everything the host can check has been checked.
vsa_status run_plan(const void* q, const void* k, const vsa_shape* shape, const PlanSizes& ps, int topp,
                    int sink, const float* table, vsa_index* index, void* ws, void* stream,
                    const HeadMap* hm = nullptr, const float* qmeans = nullptr, const float* kmeans = nullptr) {
  const Geo g = make_geo(*shape);
  const DGeo dg = to_dgeo(g);
  const int BH = shape->B * shape->heads;
  hipStream_t st_ = reinterpret_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);

  SelectArgs sa;
  std::memset(&sa, 0, sizeof(sa));
  int64_t sumk = 0;
  for (int h = 0; h < shape->heads; ++h) {
    if (topp) {
      sa.p[h] = ps.p[h];
    } else {
      sa.k[h] = ps.k[h];
      sa.off[h] = static_cast<int32_t>(sumk);
      sumk += ps.k[h];
    }
    sa.win[h] = static_cast<int16_t>(ps.win[h]);
    sa.kind[h] = static_cast<int8_t>(ps.kind[h]);
  }
  sa.batch_stride = sumk * g.NB;
  sa.rows = ps.rows;
  sa.table = table;
  sa.words = ps.words;
  sa.sink = sink;
  sa.bitmap = ps.bitmap ? 1 : 0;
  sa.scale = ps.scale;
  sa.topp = topp;
  int32_t* counts = ps.bitmap ? reinterpret_cast<int32_t*>(w + ps.off_cnt) : nullptr;
  uint64_t* bits = ps.bitmap ? reinterpret_cast<uint64_t*>(w + ps.off_bits) : nullptr;

  index->shape = *shape;
  index->nb = g.NB;
  index->window_t = ps.max_win;
  index->equal_heads = 1;
  for (int h = 0; h < shape->heads; ++h)
    if (topp || ps.k[h] != ps.k[0] || ps.win[h] != ps.win[0]) index->equal_heads = 0;

  Summaries sm{nullptr, nullptr, nullptr, nullptr};
  hipError_t e = hipSuccess;
  if (ps.any_dynamic) e = summarize(q, k, shape, ps, w, dg, BH, st_, &sm, hm, qmeans, kmeans);
  if (e == hipSuccess)
    e = launch_score_select(sm, ps.estimator, dg, shape->D, shape->heads, BH, sa, index->row_ptr,
                            index->col_idx, counts, bits, st_);
  if (e == hipSuccess && ps.bitmap)
    e = launch_scan_fill(counts, bits, index->row_ptr, index->col_idx, ps.rows, ps.words, g.NB,
                         index->capacity, st_);
  return hip_status(e);
}

}  // namespace

extern "C" {

vsa_status vsa_plan_select(const void* q, const void* k, const vsa_shape* shape, const vsa_select* sel,
                           vsa_index* index, void* ws, size_t ws_bytes, void* stream) {
  try {
    if (!q || !k || !index || !ws) return VSA_ERR_INVALID_ARG;
    PlanSizes ps;
    vsa_status st = select_sizes(shape, sel, &ps);
    if (st != VSA_OK) return st;
    if (!index->row_ptr || !index->col_idx) return VSA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(ws)) return VSA_ERR_INVALID_ARG;
    if (index->capacity < ps.capacity) return VSA_ERR_CAPACITY;
    if (ws_bytes < ps.ws) return VSA_ERR_WORKSPACE;
    return run_plan(q, k, shape, ps, sel->mode == VSA_TOPP ? 1 : 0, sel->sink, nullptr, index, ws, stream);
  } catch (...) {
    return VSA_ERR_INVALID_ARG;
  }
}

vsa_status vsa_query_mixed(const vsa_shape* shape, const vsa_head_option* options, int estimator,
                           int64_t* row_ptr_len, int64_t* col_capacity, size_t* plan_ws) {
  try {
    PlanSizes ps;
    vsa_status st = mixed_sizes(shape, options, estimator, &ps);
    if (st != VSA_OK) return st;
    if (row_ptr_len) *row_ptr_len = ps.rows + 1;
    if (col_capacity) *col_capacity = ps.capacity;
    if (plan_ws) *plan_ws = ps.ws;
    return VSA_OK;
  } catch (...) {
    return VSA_ERR_INVALID_ARG;
  }
}

vsa_status vsa_plan_mixed(const void* q, const void* k, const vsa_shape* shape,
                          const vsa_head_option* options, int estimator, const float* static_scores,
                          vsa_index* index, void* ws, size_t ws_bytes, void* stream) {
  try {
    if (!index) return VSA_ERR_INVALID_ARG;
    PlanSizes ps;
    vsa_status st = mixed_sizes(shape, options, estimator, &ps);
    if (st != VSA_OK) return st;
    if (!index->row_ptr || !index->col_idx) return VSA_ERR_INVALID_ARG;
    if (ps.any_dynamic && (!q || !k || !aligned16(q) || !aligned16(k))) return VSA_ERR_INVALID_ARG;
    if (ps.any_static && !static_scores) return VSA_ERR_INVALID_ARG;
    if (ps.ws > 0 && (!ws || !aligned16(ws))) return VSA_ERR_INVALID_ARG;
    if (index->capacity < ps.capacity) return VSA_ERR_CAPACITY;
    if (ws_bytes < ps.ws) return VSA_ERR_WORKSPACE;
    return run_plan(q, k, shape, ps, 0, 0, static_scores, index, ws, stream);
  } catch (...) {
    return VSA_ERR_INVALID_ARG;
  }
}

vsa_status vsa_plan(const void* q, const void* k, const vsa_shape* shape, const float* density,
                    int n_density, int window_t, vsa_index* index, void* ws, size_t ws_bytes,
                    void* stream) {
  vsa_select sel;
  sel.mode = VSA_TOPK;
  sel.n_value = n_density;
  sel.value = density;
  sel.window_t = window_t;
  sel.sink = 0;
  sel.scale = 0.0f;
  sel.estimator = VSA_EST_MEAN;
  return vsa_plan_select(q, k, shape, &sel, index, ws, ws_bytes, stream);
}

vsa_status vsa_estimate(const void* q, const void* k, const vsa_shape* shape, int estimator, float* out,
                        void* ws, size_t ws_bytes, void* stream) {
  try {
    if (!q || !k || !out || !ws) return VSA_ERR_INVALID_ARG;
    const float one = 1.0f;
    vsa_select sel;
    sel.mode = VSA_TOPK;
    sel.n_value = 1;
    sel.value = &one;
    sel.window_t = -1;
    sel.sink = 0;
    sel.scale = 0.0f;
    sel.estimator = estimator;
    PlanSizes ps;
    vsa_status st = select_sizes(shape, &sel, &ps);
    if (st != VSA_OK) return st;
    if (!aligned16(q) || !aligned16(k) || !aligned16(ws)) return VSA_ERR_INVALID_ARG;
    size_t need = ps.off_sum[ps.n_sum - 1] + align256(size_t(ps.rows) * shape->D * sizeof(float));
    if (ws_bytes < need) return VSA_ERR_WORKSPACE;
    const Geo g = make_geo(*shape);
    const DGeo dg = to_dgeo(g);
    const int BH = shape->B * shape->heads;
    hipStream_t st_ = reinterpret_cast<hipStream_t>(stream);
    Summaries sm;
    hipError_t e = summarize(q, k, shape, ps, static_cast<char*>(ws), dg, BH, st_, &sm);
    if (e == hipSuccess) e = launch_scores(sm, ps.estimator, out, g.NB, shape->D, BH, st_);
    return hip_status(e);
  } catch (...) {
    return VSA_ERR_INVALID_ARG;
  }
}

vsa_status vsa_attn(const void* q, const void* k, const void* v, const vsa_index* index,
                    float scale, void* o, void* ws, size_t ws_bytes, void* stream) {
  (void)ws;
  (void)ws_bytes;
  if (!q || !k || !v || !o || !index) return VSA_ERR_INVALID_ARG;
  if (!index->row_ptr || !index->col_idx) return VSA_ERR_INVALID_ARG;
  vsa_status st = check_shape(&index->shape);
  if (st != VSA_OK) return st;
  const Geo g = make_geo(index->shape);
  if (index->nb != g.NB || index->window_t < -1) return VSA_ERR_SHAPE_MISMATCH;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return VSA_ERR_INVALID_ARG;
  if (scale == 0.0f) scale = 1.0f / std::sqrt(static_cast<float>(index->shape.D));
  if (!(scale > 0.0f) || !std::isfinite(scale)) return VSA_ERR_INVALID_ARG;
  const int BH = index->shape.B * index->shape.heads;
  hipError_t e = launch_attn(q, k, v, o, index->shape.dtype, index->shape.D, index->row_ptr,
                             index->col_idx, to_dgeo(g), BH, scale, index->equal_heads != 0,
                             reinterpret_cast<hipStream_t>(stream));
  return hip_status(e);
}

vsa_status vsa_permute(const void* x, const vsa_shape* shape, void* xb, void* stream) {
  vsa_status st = check_shape(shape);
  if (st != VSA_OK) return st;
  if (!x || !xb || !aligned16(x) || !aligned16(xb)) return VSA_ERR_INVALID_ARG;
  const Geo g = make_geo(*shape);
  const int P = shape->bt * shape->bh * shape->bw;
  return hip_status(launch_permute(x, xb, elt_bytes(shape->dtype), shape->D, to_dgeo(g),
                                   shape->B * shape->heads, P, false,
                                   reinterpret_cast<hipStream_t>(stream)));
}

vsa_status vsa_unpermute(const void* xb, const vsa_shape* shape, void* x, void* stream) {
  vsa_status st = check_shape(shape);
  if (st != VSA_OK) return st;
  if (!x || !xb || !aligned16(x) || !aligned16(xb)) return VSA_ERR_INVALID_ARG;
  const Geo g = make_geo(*shape);
  const int P = shape->bt * shape->bh * shape->bw;
  return hip_status(launch_permute(x, const_cast<void*>(xb), elt_bytes(shape->dtype), shape->D,
                                   to_dgeo(g), shape->B * shape->heads, P, true,
                                   reinterpret_cast<hipStream_t>(stream)));
}

vsa_status vsa_centroids(const void* x, const vsa_shape* shape, float* out, void* stream) {
  vsa_status st = check_shape(shape);
  if (st != VSA_OK) return st;
  if (!x || !out || !aligned16(x) || !aligned16(out)) return VSA_ERR_INVALID_ARG;
  const Geo g = make_geo(*shape);
  return hip_status(launch_pool(x, out, nullptr, nullptr, shape->dtype, shape->D, to_dgeo(g),
                                shape->B * shape->heads, reinterpret_cast<hipStream_t>(stream)));
}

vsa_status vsa_centroid_scores(const float* qc, const float* kc, const vsa_shape* shape, float* out,
                               void* stream) {
  vsa_status st = check_shape(shape);
  if (st != VSA_OK) return st;
  if (!qc || !kc || !out || !aligned16(qc) || !aligned16(kc)) return VSA_ERR_INVALID_ARG;
  const Geo g = make_geo(*shape);
  return hip_status(launch_scores(Summaries{qc, nullptr, kc, nullptr}, VSA_EST_MEAN, out, g.NB, shape->D,
                                  shape->B * shape->heads,
                                  reinterpret_cast<hipStream_t>(stream)));
}

vsa_status vsa_sics(const void* x, const vsa_shape* shape, float* out, void* stream) {
  vsa_status st = check_shape(shape);
  if (st != VSA_OK) return st;
  if (!x || !out || !aligned16(x)) return VSA_ERR_INVALID_ARG;
  const Geo g = make_geo(*shape);
  return hip_status(launch_sics(x, out, nullptr, nullptr, shape->dtype, shape->D, to_dgeo(g),
                                shape->B * shape->heads, reinterpret_cast<hipStream_t>(stream)));
}

// Validates the candidates and lays out the workspace: per candidate the
// block SICS of Q then K, each candidate's region 256-byte aligned.
static vsa_status scheme_layout(const vsa_shape* shape, const int32_t* cand, int n_cand, vsa::SchemeArgs* sa,
                                size_t* bytes) {
  if (!shape || !cand || n_cand < 1 || n_cand > VSA_MAX_SCHEMES) return VSA_ERR_INVALID_ARG;
  const int64_t BH = (int64_t)shape->B * shape->heads;
  size_t off = 0;
  for (int c = 0; c < n_cand; ++c) {
    vsa_shape s = *shape;
    s.bt = cand[3 * c];
    s.bh = cand[3 * c + 1];
    s.bw = cand[3 * c + 2];
    const vsa_status st = check_shape(&s);
    if (st != VSA_OK) return st;
    const Geo g = make_geo(s);
    if (sa) {
      sa->nb[c] = g.NB;
      sa->off[c] = (int64_t)(off / sizeof(float));
    }
    off = align256(off + (size_t)2 * BH * g.NB * sizeof(float));
  }
  if (sa) sa->n = n_cand;
  if (bytes) *bytes = off;
  return VSA_OK;
}

vsa_status vsa_scheme_workspace(const vsa_shape* shape, const int32_t* candidates, int n_cand,
                                size_t* ws_bytes) {
  return scheme_layout(shape, candidates, n_cand, nullptr, ws_bytes);
}

vsa_status vsa_select_scheme(const void* q, const void* k, const vsa_shape* shape, const int32_t* candidates,
                             int n_cand, float* scores, int32_t* choice, void* ws, size_t ws_bytes,
                             void* stream) {
  vsa::SchemeArgs sa{};
  size_t need = 0;
  vsa_status st = scheme_layout(shape, candidates, n_cand, &sa, &need);
  if (st != VSA_OK) return st;
  if (!q || !k || !scores || !choice || !ws || !aligned16(q) || !aligned16(k) || !aligned16(ws))
    return VSA_ERR_INVALID_ARG;
  if (ws_bytes < need) return VSA_ERR_WORKSPACE;
  hipStream_t st_ = reinterpret_cast<hipStream_t>(stream);
  const int BH = shape->B * shape->heads;
  float* sics = static_cast<float*>(ws);
  for (int c = 0; c < n_cand; ++c) {
    vsa_shape s = *shape;
    s.bt = candidates[3 * c];
    s.bh = candidates[3 * c + 1];
    s.bw = candidates[3 * c + 2];
    const Geo g = make_geo(s);
    float* base = sics + sa.off[c];
    const hipError_t e = launch_sics(q, base, k, base + (size_t)BH * g.NB, shape->dtype, shape->D,
                                     to_dgeo(g), BH, st_);
    if (e != hipSuccess) return VSA_ERR_HIP;
  }
  return hip_status(launch_scheme_select(sics, sa, BH, scores, choice, st_));
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Calls over a subset of the heads, and scheme selection that keeps each
// candidate's block means for the plans that follow it.
// ---------------------------------------------------------------------------
extern "C" vsa_status vsa_plan_heads(const void* q, const void* k, const float* qmeans, const float* kmeans,
                                     const vsa_shape* shape, const int32_t* heads, int n_heads,
                                     const float* density, int n_density, int window_t, vsa_index* index,
                                     void* ws, size_t ws_bytes, void* stream) {
  try {
    if (!shape || !index) return VSA_ERR_INVALID_ARG;
    HeadMap hm;
    vsa_status st = check_shape(shape);
    if (st != VSA_OK) return st;
    st = make_head_map(heads, n_heads, shape->heads, &hm);
    if (st != VSA_OK) return st;
    vsa_shape cs = *shape;
    cs.heads = n_heads;
    PlanSizes ps;
    st = plan_sizes(&cs, density, n_density, window_t, &ps);
    if (st != VSA_OK) return st;
    const bool from_means = qmeans != nullptr || kmeans != nullptr;
    if (from_means) {
      if (!qmeans || !kmeans || !aligned16(qmeans) || !aligned16(kmeans)) return VSA_ERR_INVALID_ARG;
    } else if (!q || !k || !aligned16(q) || !aligned16(k)) {
      return VSA_ERR_INVALID_ARG;
    }
    if (!index->row_ptr || !index->col_idx || !ws || !aligned16(ws)) return VSA_ERR_INVALID_ARG;
    if (index->capacity < ps.capacity) return VSA_ERR_CAPACITY;
    if (ws_bytes < ps.ws) return VSA_ERR_WORKSPACE;
    return run_plan(q, k, &cs, ps, 0, 0, nullptr, index, ws, stream, &hm, qmeans, kmeans);
  } catch (...) {
    return VSA_ERR_INVALID_ARG;
  }
}

extern "C" vsa_status vsa_attn_heads(const void* q, const void* k, const void* v, const vsa_index* index,
                                     const int32_t* heads, int heads_total, float scale, void* o, void* ws,
                                     size_t ws_bytes, void* stream) {
  (void)ws;
  (void)ws_bytes;
  if (!q || !k || !v || !o || !index) return VSA_ERR_INVALID_ARG;
  if (!index->row_ptr || !index->col_idx) return VSA_ERR_INVALID_ARG;
  vsa_status st = check_shape(&index->shape);
  if (st != VSA_OK) return st;
  HeadMap hm;
  st = make_head_map(heads, index->shape.heads, heads_total, &hm);
  if (st != VSA_OK) return st;
  vsa_shape full = index->shape;
  full.heads = heads_total;
  st = check_shape(&full);
  if (st != VSA_OK) return st;
  const Geo g = make_geo(index->shape);
  if (index->nb != g.NB || index->window_t < -1) return VSA_ERR_SHAPE_MISMATCH;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return VSA_ERR_INVALID_ARG;
  if (scale == 0.0f) scale = 1.0f / std::sqrt(static_cast<float>(index->shape.D));
  if (!(scale > 0.0f) || !std::isfinite(scale)) return VSA_ERR_INVALID_ARG;
  const int BH = index->shape.B * index->shape.heads;
  return hip_status(launch_attn(q, k, v, o, index->shape.dtype, index->shape.D, index->row_ptr, index->col_idx,
                                to_dgeo(g), BH, scale, index->equal_heads != 0,
                                reinterpret_cast<hipStream_t>(stream), &hm));
}

// Layout of vsa_select_scheme_means' workspace: the SICS regions of
// scheme_layout, then per candidate the query means [B*heads][nb][D] and the
// key means [B*heads][D][nb], each 256-byte aligned.
static vsa_status scheme_means_layout(const vsa_shape* shape, const int32_t* cand, int n_cand,
                                      vsa::SchemeArgs* sa, size_t* means_off, size_t* bytes) {
  size_t off = 0;
  vsa_status st = scheme_layout(shape, cand, n_cand, sa, &off);
  if (st != VSA_OK) return st;
  const size_t BH = (size_t)shape->B * shape->heads;
  for (int c = 0; c < n_cand; ++c) {
    vsa_shape s = *shape;
    s.bt = cand[3 * c];
    s.bh = cand[3 * c + 1];
    s.bw = cand[3 * c + 2];
    const Geo g = make_geo(s);
    const size_t one = align256(BH * g.NB * shape->D * sizeof(float));
    if (means_off) {
      means_off[2 * c] = off;
      means_off[2 * c + 1] = off + one;
    }
    off += 2 * one;
  }
  if (bytes) *bytes = off;
  return VSA_OK;
}

extern "C" vsa_status vsa_scheme_means_workspace(const vsa_shape* shape, const int32_t* candidates, int n_cand,
                                                 size_t* ws_bytes, size_t* means_off) {
  try {
    return scheme_means_layout(shape, candidates, n_cand, nullptr, means_off, ws_bytes);
  } catch (...) {
    return VSA_ERR_INVALID_ARG;
  }
}

extern "C" vsa_status vsa_select_scheme_means(const void* q, const void* k, const vsa_shape* shape,
                                              const int32_t* candidates, int n_cand, float* scores, int32_t* choice,
                                              void* ws, size_t ws_bytes, void* stream) {
  try {
    vsa::SchemeArgs sa{};
    size_t need = 0;
    size_t moff[2 * VSA_MAX_SCHEMES];
    vsa_status st = scheme_means_layout(shape, candidates, n_cand, &sa, moff, &need);
    if (st != VSA_OK) return st;
    if (!q || !k || !scores || !choice || !ws || !aligned16(q) || !aligned16(k) || !aligned16(ws))
      return VSA_ERR_INVALID_ARG;
    if (ws_bytes < need) return VSA_ERR_WORKSPACE;
    hipStream_t st_ = reinterpret_cast<hipStream_t>(stream);
    const int BH = shape->B * shape->heads;
    char* w = static_cast<char*>(ws);
    float* sics = static_cast<float*>(ws);
    for (int c = 0; c < n_cand; ++c) {
      vsa_shape s = *shape;
      s.bt = candidates[3 * c];
      s.bh = candidates[3 * c + 1];
      s.bw = candidates[3 * c + 2];
      const Geo g = make_geo(s);
      float* base = sics + sa.off[c];
      const hipError_t e = launch_pool_sics(q, reinterpret_cast<float*>(w + moff[2 * c]), k,
                                            reinterpret_cast<float*>(w + moff[2 * c + 1]), base,
                                            base + (size_t)BH * g.NB, shape->dtype, shape->D, to_dgeo(g), BH, st_);
      if (e != hipSuccess) return VSA_ERR_HIP;
    }
    return hip_status(launch_scheme_select(sics, sa, BH, scores, choice, st_));
  } catch (...) {
    return VSA_ERR_INVALID_ARG;
  }
}

// ---------------------------------------------------------------------------
// Plan workspace for callers that cannot allocate: one static array per GPU.
// In host code `scratch` names a host-side stand-in, not the device array;
// kernels get the device address that hipGetSymbolAddress returns for the
// device a call runs on, looked up once per device and kept.
// ---------------------------------------------------------------------------
static __device__ __attribute__((aligned(256))) unsigned char scratch[VSA_PLAN_NOALLOC_MAX_WS];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the device that `stream` belongs to (the
// current device for the null stream).
vsa_status scratch_address(hipStream_t stream, void** out) {
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return VSA_ERR_HIP;
  int dev = cur;
  if (stream != nullptr && hipStreamGetDevice(stream, &dev) != hipSuccess) return VSA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return VSA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return VSA_ERR_HIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur && hipSetDevice(cur) != hipSuccess) return VSA_ERR_HIP;
    if (e != hipSuccess || p == nullptr) return VSA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return VSA_OK;
}

}  // namespace

extern "C" vsa_status vsa_plan_noalloc(const void* q, const void* k, const vsa_shape* shape,
                                       const float* density, int n_density, int window_t, vsa_index* index,
                                       void* stream) {
  try {
    if (!q || !k || !index) return VSA_ERR_INVALID_ARG;
    PlanSizes ps;
    vsa_status st = plan_sizes(shape, density, n_density, window_t, &ps);
    if (st != VSA_OK) return st;
    if (!index->row_ptr || !index->col_idx) return VSA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k)) return VSA_ERR_INVALID_ARG;
    if (index->capacity < ps.capacity) return VSA_ERR_CAPACITY;
    if (ps.ws > VSA_PLAN_NOALLOC_MAX_WS) return VSA_ERR_WORKSPACE;
    void* ws = nullptr;
    st = scratch_address(reinterpret_cast<hipStream_t>(stream), &ws);
    if (st != VSA_OK) return st;
    return run_plan(q, k, shape, ps, 0, 0, nullptr, index, ws, stream);
  } catch (...) {
    return VSA_ERR_INVALID_ARG;
  }
}
