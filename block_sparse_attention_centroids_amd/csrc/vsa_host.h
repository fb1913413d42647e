// Host-side geometry, keep-rate rule, validation and workspace layout.
// Pure C++ (no HIP): everything here runs before any launch.
#pragma once

#include <algorithm>
#include <cmath>
#include <cstddef>
#include <cstdint>
#include <vector>

#include "vsa.h"

namespace vsa {

struct Geo {
  int T, H, W;
  int bt, bh, bw;
  int nbt, nbh, nbw;
  int NB;
  int N;
};

inline int ceil_div(int a, int b) { return (a + b - 1) / b; }
inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

inline Geo make_geo(const vsa_shape& s) {
  Geo g;
  g.T = s.T; g.H = s.H; g.W = s.W;
  g.bt = s.bt; g.bh = s.bh; g.bw = s.bw;
  g.nbt = ceil_div(s.T, s.bt);
  g.nbh = ceil_div(s.H, s.bh);
  g.nbw = ceil_div(s.W, s.bw);
  g.NB = g.nbt * g.nbh * g.nbw;
  g.N = s.T * s.H * s.W;
  return g;
}

// Tokens in block j: product of its (possibly cut-short) extents.
inline int block_tokens(const Geo& g, int j) {
  int tb = j / (g.nbh * g.nbw), r = j % (g.nbh * g.nbw);
  int hb = r / g.nbw, wb = r % g.nbw;
  int et = std::min(g.bt, g.T - tb * g.bt);
  int eh = std::min(g.bh, g.H - hb * g.bh);
  int ew = std::min(g.bw, g.W - wb * g.bw);
  return et * eh * ew;
}

// Keep-rate rule: k = min(NB, max(1, floor(density*NB + 0.5))), in double
// from the float32 density.
inline int k_rule(float density, int NB) {
  double k = std::floor(static_cast<double>(density) * NB + 0.5);
  if (k < 1) k = 1;
  if (k > NB) k = NB;
  return static_cast<int>(k);
}

// Number of key blocks within +-window_t temporal blocks of a query block in
// temporal block tb.
inline int window_count(const Geo& g, int tb, int window_t) {
  if (window_t < 0) return 0;
  int lo = std::max(0, tb - window_t), hi = std::min(g.nbt - 1, tb + window_t);
  return (hi - lo + 1) * g.nbh * g.nbw;
}

// A window radius of nbt - 1 already covers every temporal block, so a
// larger one selects the same key blocks; clamping keeps the radius in the
// 16-bit field the selection kernel reads, whatever the caller passed.
inline int clamp_window(const Geo& g, int window_t) {
  return window_t < 0 ? -1 : std::min(window_t, g.nbt - 1);
}

inline int elt_bytes(int dtype) { return dtype == VSA_F32 ? 4 : 2; }

// Shape validation shared by every entry point.
inline vsa_status check_shape(const vsa_shape* s) {
  if (!s) return VSA_ERR_INVALID_ARG;
  if (s->B < 1 || s->heads < 1 || s->D < 1 || s->T < 1 || s->H < 1 || s->W < 1 ||
      s->bt < 1 || s->bh < 1 || s->bw < 1)
    return VSA_ERR_INVALID_ARG;
  if (s->dtype != VSA_BF16 && s->dtype != VSA_F32) return VSA_ERR_INVALID_ARG;
  if (s->D != 64 && s->D != 128) return VSA_ERR_UNSUPPORTED;
  // Block box larger than the grid is allowed (it is cut short).
  int64_t box = int64_t(s->bt) * s->bh * s->bw;
  int64_t bt = std::min(s->bt, s->T), bh = std::min(s->bh, s->H), bw = std::min(s->bw, s->W);
  if (bt * bh * bw > VSA_MAX_BLOCK_TOKENS) return VSA_ERR_UNSUPPORTED;
  (void)box;
  // Products are bounded step by step so that none can overflow int64.
  const int64_t TH = int64_t(s->T) * s->H;   // < 2^62
  if (TH > (int64_t(1) << 30)) return VSA_ERR_UNSUPPORTED;
  const int64_t N = TH * s->W;               // < 2^61
  if (N > (int64_t(1) << 30)) return VSA_ERR_UNSUPPORTED;
  // One head's tensor must be addressable with 32-bit byte offsets.
  const int64_t per_head = N * s->D;         // < 2^38
  if (per_head * elt_bytes(s->dtype) >= (int64_t(1) << 31)) return VSA_ERR_UNSUPPORTED;
  // B * heads * N * D <= 2^40 elements.
  const int64_t BH = int64_t(s->B) * s->heads;   // < 2^62
  if (BH > (int64_t(1) << 40) / per_head) return VSA_ERR_UNSUPPORTED;
  Geo g = make_geo(*s);
  if (g.NB > 16384) return VSA_ERR_UNSUPPORTED;
  if (int64_t(s->B) * s->heads * g.NB >= (int64_t(1) << 31) - 1) return VSA_ERR_UNSUPPORTED;
  return VSA_OK;
}

struct PlanSizes {
  int64_t rows = 0;          // B*heads*NB
  int64_t capacity = 0;      // col_idx entries needed (an upper bound in bitmap mode)
  size_t ws = 0;             // plan workspace bytes
  size_t off_sum[4] = {0, 0, 0, 0};   // block summaries (2, 3 or 4 arrays)
  int n_sum = 2;
  int estimator = VSA_EST_MEAN;
  size_t off_cnt = 0, off_bits = 0;
  int words = 0;             // 64-bit bitmap words per row
  bool bitmap = false;       // rows vary in length: bitmap + scan + fill
  float scale = 0.0f;        // Top-P logit scale (resolved)
  std::vector<int> k;        // per head (Top-K)
  std::vector<float> p;      // per head (Top-P)
  std::vector<int> win;      // per head temporal window (-1: none)
  std::vector<int> kind;     // per head option (vsa_head_kind)
  bool any_dynamic = true;   // some head needs Q/K summaries
  bool any_static = false;   // some head reads the static score table
  int max_win = -1;
};

// Summary workspace regions for an estimator, then the bitmap regions when
// rows vary in length; sets off_sum, n_sum, off_cnt, off_bits, ws.
inline void layout_workspace(const vsa_shape* s, PlanSizes* out) {
  size_t cent = align256(size_t(out->rows) * s->D * sizeof(float));
  out->n_sum = out->estimator == VSA_EST_MEAN ? 2 : out->estimator == VSA_EST_DSA ? 3 : 4;
  size_t ws = 0;
  if (out->any_dynamic) {
    for (int i = 0; i < out->n_sum; ++i) {
      out->off_sum[i] = ws;
      ws += cent;
    }
  }
  if (out->bitmap) {
    out->off_cnt = ws;
    ws += align256(size_t(out->rows + 1) * sizeof(int32_t));
    out->off_bits = ws;
    ws += align256(size_t(out->rows) * out->words * sizeof(uint64_t));
  }
  out->ws = ws;
}

// Sizes and per-head parameters of a selection; validates everything the
// host can see.
inline vsa_status select_sizes(const vsa_shape* s, const vsa_select* sel, PlanSizes* out) {
  vsa_status st = check_shape(s);
  if (st != VSA_OK) return st;
  if (!sel || !sel->value || !out) return VSA_ERR_INVALID_ARG;
  if (sel->mode != VSA_TOPK && sel->mode != VSA_TOPP) return VSA_ERR_INVALID_ARG;
  if (sel->n_value != 1 && sel->n_value != s->heads) return VSA_ERR_INVALID_ARG;
  if (sel->window_t < -1) return VSA_ERR_INVALID_ARG;
  if (sel->estimator != VSA_EST_MEAN && sel->estimator != VSA_EST_DSA && sel->estimator != VSA_EST_DSA2)
    return VSA_ERR_INVALID_ARG;
  if (s->heads > VSA_MAX_HEADS) return VSA_ERR_UNSUPPORTED;
  Geo g = make_geo(*s);
  if (sel->sink < 0 || sel->sink > g.NB) return VSA_ERR_INVALID_ARG;
  const int window_t = clamp_window(g, sel->window_t);
  if (!(sel->scale >= 0.0f) || !std::isfinite(sel->scale)) return VSA_ERR_INVALID_ARG;
  const bool topp = sel->mode == VSA_TOPP;
  out->k.assign(s->heads, 0);
  out->p.assign(s->heads, 0.0f);
  for (int h = 0; h < s->heads; ++h) {
    float d = sel->value[sel->n_value == 1 ? 0 : h];
    if (!(d > 0.0f) || !(d <= 1.0f)) return VSA_ERR_INVALID_ARG;  // also rejects NaN
    if (topp)
      out->p[h] = d;
    else
      out->k[h] = k_rule(d, g.NB);
  }
  out->scale = sel->scale != 0.0f ? sel->scale : 1.0f / std::sqrt(static_cast<float>(s->D));
  out->rows = int64_t(s->B) * s->heads * g.NB;
  int64_t cap = 0;
  if (topp) {
    cap = out->rows * g.NB;
  } else {
    for (int h = 0; h < s->heads; ++h) {
      int64_t per_head = 0;
      for (int i = 0; i < g.NB; ++i) {
        int tb = i / (g.nbh * g.nbw);
        int64_t c = int64_t(out->k[h]) + window_count(g, tb, window_t) + sel->sink;
        per_head += std::min<int64_t>(c, g.NB);
      }
      cap += per_head;
    }
    cap *= s->B;
  }
  if (cap >= (int64_t(1) << 31) - 1) return VSA_ERR_UNSUPPORTED;
  out->capacity = cap;
  out->estimator = sel->estimator;
  out->win.assign(s->heads, window_t);
  out->kind.assign(s->heads, VSA_HEAD_DYNAMIC);
  out->any_dynamic = true;
  out->any_static = false;
  out->max_win = window_t;
  out->words = (g.NB + 63) / 64;
  out->bitmap = topp || window_t >= 0 || sel->sink > 0;
  layout_workspace(s, out);
  return VSA_OK;
}

// Mixed per-head plans: each head is dynamic (Top-K at value over the
// estimator's scores), static (Top-K at value over a caller table) or dense,
// with its own window.
inline vsa_status mixed_sizes(const vsa_shape* s, const vsa_head_option* opts, int estimator,
                              PlanSizes* out) {
  vsa_status st = check_shape(s);
  if (st != VSA_OK) return st;
  if (!opts || !out) return VSA_ERR_INVALID_ARG;
  if (estimator != VSA_EST_MEAN && estimator != VSA_EST_DSA && estimator != VSA_EST_DSA2)
    return VSA_ERR_INVALID_ARG;
  if (s->heads > VSA_MAX_HEADS) return VSA_ERR_UNSUPPORTED;
  Geo g = make_geo(*s);
  out->k.assign(s->heads, 0);
  out->p.assign(s->heads, 0.0f);
  out->win.assign(s->heads, -1);
  out->kind.assign(s->heads, VSA_HEAD_DYNAMIC);
  out->any_dynamic = out->any_static = false;
  out->max_win = -1;
  for (int h = 0; h < s->heads; ++h) {
    const vsa_head_option& o = opts[h];
    if (o.kind != VSA_HEAD_DYNAMIC && o.kind != VSA_HEAD_STATIC && o.kind != VSA_HEAD_DENSE)
      return VSA_ERR_INVALID_ARG;
    if (o.window_t < -1) return VSA_ERR_INVALID_ARG;
    if (o.kind == VSA_HEAD_DENSE) {
      out->k[h] = g.NB;
    } else {
      if (!(o.value > 0.0f) || !(o.value <= 1.0f)) return VSA_ERR_INVALID_ARG;
      out->k[h] = k_rule(o.value, g.NB);
    }
    out->kind[h] = o.kind;
    out->win[h] = clamp_window(g, o.window_t);
    out->any_dynamic = out->any_dynamic || o.kind == VSA_HEAD_DYNAMIC;
    out->any_static = out->any_static || o.kind == VSA_HEAD_STATIC;
    out->max_win = std::max(out->max_win, out->win[h]);
  }
  out->estimator = estimator;
  out->scale = 1.0f;
  out->rows = int64_t(s->B) * s->heads * g.NB;
  int64_t cap = 0;
  for (int h = 0; h < s->heads; ++h) {
    for (int i = 0; i < g.NB; ++i) {
      int tb = i / (g.nbh * g.nbw);
      cap += std::min<int64_t>(int64_t(out->k[h]) + window_count(g, tb, out->win[h]), g.NB);
    }
  }
  cap *= s->B;
  if (cap >= (int64_t(1) << 31) - 1) return VSA_ERR_UNSUPPORTED;
  out->capacity = cap;
  out->words = (g.NB + 63) / 64;
  out->bitmap = out->max_win >= 0;
  layout_workspace(s, out);
  return VSA_OK;
}

// Top-K with an optional window: the selection of vsa_query / vsa_plan.
inline vsa_status plan_sizes(const vsa_shape* s, const float* density, int n_density,
                             int window_t, PlanSizes* out) {
  vsa_select sel;
  sel.mode = VSA_TOPK;
  sel.n_value = n_density;
  sel.value = density;
  sel.window_t = window_t;
  sel.sink = 0;
  sel.scale = 0.0f;
  sel.estimator = VSA_EST_MEAN;
  return select_sizes(s, &sel, out);
}

}  // namespace vsa
