/*
 * vsa.h -- C ABI of the MI355X (gfx950) library for centroid-scored 3D
 * block-sparse self-attention over a video latent.
 *
 * What the library computes (SPADE: An Input-Adaptive Sparse Attention
 * Engine for Fast Video Diffusion Models Inference, sections 2.1, 2.2 and
 * 3.1-3.3):
 *   1. the T x H x W token grid (flattened in raster order, 2.1) is cut into
 *      bt x bh x bw boxes (3.1, Fig. 3);
 *   2. Q and K are summarized per block by their mean (MEAN-SPADE, Fig. 4(c));
 *   3. the dot products of the means give an N_Qblocks x N_Kblocks importance
 *      matrix; each query-block row keeps its top-k key blocks (3.3), with k
 *      from a keep rate, i.e. the share of key blocks retained per query
 *      block (JEV sparse comparison page, How this was measured), optionally
 *      united with a local temporal window (3.3);
 *   4. attention (Eq. 2) runs over the kept blocks only with an online
 *      softmax, and the output is restored to raster order (3.3).
 * Around that path (3.1-3.3): Top-P selection and attention-sink blocks,
 * the max/min (DSA, DSA2) summarizers and estimators, mixed per-head plans
 * (dense, static and dynamic heads with their own windows), and scheme
 * generation (per-block intra-block aggregation and head-wise selection of
 * a blocking scheme, 3.2).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Layout.  q, k, v and o are dense, contiguous [B, heads, N, D] arrays with
 *   N = T*H*W tokens in raster order n = (t*H + h)*W + w.  All four have the
 *   same element type (vsa_dtype).  Device pointers must be 16-byte aligned.
 * Blocks.  nbt = ceil(T/bt), nbh = ceil(H/bh), nbw = ceil(W/bw),
 *   NB = nbt*nbh*nbw.  Block (tb, hb, wb) has id (tb*nbh + hb)*nbw + wb and
 *   covers the box [tb*bt, min(T, tb*bt+bt)) x ... ; blocks on the far edge
 *   of a dimension that bt/bh/bw do not divide are cut short and hold fewer
 *   tokens.  Tokens inside a block are ordered row-major in (t, h, w).
 * Ownership.  The caller allocates every buffer (inputs, outputs, index
 *   arrays, workspace).  The library never allocates, never synchronizes the
 *   device and keeps no mutable global state, with one exception:
 *   vsa_plan_noalloc takes its workspace from a static per-GPU array (see
 *   there).  Calls on different streams do not interfere unless they write
 *   the same buffers (or both are vsa_plan_noalloc calls on one GPU).
 * Streams.  `stream` is a hipStream_t passed as void* (NULL = null stream).
 *   Work is only enqueued; results are valid once the caller has
 *   synchronized with the stream.  Calls enqueue kernel launches and
 *   nothing else (no memset, copy, allocation or synchronization), so they
 *   can be captured in a HIP graph on a capturing stream; a captured plan
 *   that should allocate nothing uses vsa_plan_noalloc, after one eager call
 *   on the device (its first call on a device looks up the static
 *   workspace's address).
 * Errors.  Arguments are validated on the host before anything is enqueued;
 *   on error nothing is enqueued and the status says why.  A failed kernel
 *   launch returns VSA_ERR_HIP.  No C++ exception crosses this boundary.
 */
#ifndef VSA_H_
#define VSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  VSA_OK = 0,
  VSA_ERR_INVALID_ARG = 1,    /* null pointer, non-positive size, density out of (0,1], ... */
  VSA_ERR_UNSUPPORTED = 2,    /* D not 64/128, more than 128 tokens per block, too many blocks/heads */
  VSA_ERR_WORKSPACE = 3,      /* ws_bytes smaller than vsa_query reported */
  VSA_ERR_CAPACITY = 4,       /* index->capacity smaller than vsa_query reported */
  VSA_ERR_SHAPE_MISMATCH = 5, /* an index used with a shape it was not planned for */
  VSA_ERR_HIP = 6             /* a HIP launch or runtime call failed */
} vsa_status;

typedef enum { VSA_BF16 = 0, VSA_F32 = 1 } vsa_dtype;

/* Sizes are tokens (T, H, W: latent grid; bt, bh, bw: block box). */
typedef struct {
  int32_t B, heads, D;
  int32_t T, H, W;
  int32_t bt, bh, bw;
  int32_t dtype; /* vsa_dtype */
} vsa_shape;

/* Block index in CSR form (SPADE 3.3: the binary block mask, stored as a
 * block-sparse row structure).  Row r = (b*heads + h)*nb + i lists the key
 * blocks kept by query block i of head (b, h) in ascending id order:
 * col_idx[row_ptr[r] .. row_ptr[r+1]).  row_ptr[0] = 0.
 * row_ptr: device int32[B*heads*nb + 1]; col_idx: device int32[capacity].
 * The caller owns both arrays; vsa_plan fills them and sets shape, nb,
 * window_t and equal_heads.
 * equal_heads: a scheduling hint.  The planners set 1 when every (batch,
 * head) has the same selection size and window by construction (Top-K with
 * one k and one window for all heads), else 0.  vsa_attn then gives each
 * XCD a contiguous run of (head, query block) rows; with 0 it gives each
 * XCD an equal contiguous slice of every head, which balances heads of
 * different work.  Either value gives the same result; 0 is the safe
 * choice for an index built by hand. */
typedef struct {
  vsa_shape shape;
  int32_t nb;
  int32_t window_t;
  int32_t* row_ptr;
  int32_t* col_idx;
  int64_t capacity;
  int32_t equal_heads;
} vsa_index;

/* Largest supported head count with per-head densities, and block size. */
#define VSA_MAX_HEADS 256
#define VSA_MAX_BLOCK_TOKENS 128
/* Largest number of blocking-scheme candidates vsa_select_scheme takes. */
#define VSA_MAX_SCHEMES 16

/* Host-only sizing query; touches no device.
 * density: host float[n_density], n_density = 1 (all heads) or heads; each
 *   value in (0, 1].  k_h = min(NB, max(1, floor(density_h*NB + 0.5))).
 * window_t: -1 for none, r >= 0 to also keep every key block whose temporal
 *   block index is within +-r of the query block's.  Any r >= nbt - 1
 *   covers every temporal block; such a radius is treated as nbt - 1 (the
 *   same key blocks), and a plan records nbt - 1 in index->window_t.
 *   Values below -1 are VSA_ERR_INVALID_ARG.
 * Outputs (any may be NULL): row_ptr_len = B*heads*NB + 1; col_capacity =
 *   an upper bound of the kept entries (exact without a window);
 *   plan_ws / attn_ws = workspace bytes that vsa_plan / vsa_attn need. */
vsa_status vsa_query(const vsa_shape* shape, const float* density, int n_density,
                     int window_t, int64_t* row_ptr_len, int64_t* col_capacity,
                     size_t* plan_ws, size_t* attn_ws);

/* Selection mode of vsa_plan_select (SPADE 3.1: the Top-K / Top-P mode of a
 * head's scheme). */
typedef enum { VSA_TOPK = 0, VSA_TOPP = 1 } vsa_select_mode;

/* Summarizer and inter-estimator of the planning step (SPADE 3.1, the
 * Summarizer and Estimator Expressions of Fig. 4).  Each reduces a block's
 * Q or K tokens to vectors in R^D and scores a (query block, key block)
 * pair in float32, channels in order from +0 with separately rounded
 * products (no fused multiply-add):
 *   VSA_EST_MEAN: block means; score = <q_mean, k_mean> (MEAN-SPADE).
 *   VSA_EST_DSA:  channel-wise max and min over the block's tokens; the
 *     query midpoint qm = fl(fl(q_max + q_min) * 0.5); score = sum over
 *     channels of max(qm*k_max, qm*k_min): the largest dot product of qm
 *     with any vector of the key block's [k_min, k_max] box (DSA-SPADE).
 *   VSA_EST_DSA2: score = sum over channels of the largest of the four
 *     products of {q_max, q_min} with {k_max, k_min}: the largest dot
 *     product between the query and key boxes (DSA2-SPADE).
 * Cut-short edge blocks use their valid tokens. */
typedef enum { VSA_EST_MEAN = 0, VSA_EST_DSA = 1, VSA_EST_DSA2 = 2 } vsa_estimator;

/* Selection options of vsa_query_select / vsa_plan_select (SPADE 3.1:
 * each head's scheme has a local-window length and an inter-top value that
 * is a Top-K keep or a Top-P cumulative threshold; the attention-sink
 * length is a utility parameter; 3.3: the filtered scores are united with
 * the window and sink masks).
 * mode: vsa_select_mode.
 * value: host float[n_value], n_value = 1 (all heads) or heads, each in
 *   (0, 1]: the keep rate for VSA_TOPK (k as in vsa_query), the threshold p
 *   for VSA_TOPP: a query-block row keeps the shortest prefix of its key
 *   blocks, ordered by score descending and block id ascending, whose
 *   softmax(scale * scores) mass is at least p (at least one block; p = 1
 *   keeps the whole row).
 * window_t: as in vsa_query.
 * sink: 0 <= sink <= NB; key blocks 0 .. sink-1 are kept by every row.
 * scale: VSA_TOPP logit scale, 0 means 1/sqrt(D); must be finite and
 *   non-negative.
 * estimator: vsa_estimator that produces the scores being selected. */
typedef struct {
  int32_t mode;
  int32_t n_value;
  const float* value;
  int32_t window_t;
  int32_t sink;
  float scale;
  int32_t estimator;
} vsa_select;

/* Planning (SPADE 3.3: summarizer, inter-estimator, Top-K, union with the
 * local window).  q, k: device [B, heads, N, D] of shape->dtype.  Block
 * means and their dot products are computed in float32 in a fixed order:
 * mean = (sum over the block's tokens in block order, from +0) / n, and
 * score = sum over channels in order of separately rounded products, so the
 * index is reproducible bit for bit.  Ties between equal scores keep the
 * lower block id.  index: row_ptr, col_idx and capacity set by the caller;
 * ws: device workspace of at least vsa_query's plan_ws bytes. */
vsa_status vsa_plan(const void* q, const void* k, const vsa_shape* shape,
                    const float* density, int n_density, int window_t,
                    vsa_index* index, void* ws, size_t ws_bytes, void* stream);

/* Host-only sizing for vsa_plan_select; touches no device.  Outputs as in
 * vsa_query.  col_capacity is exact for VSA_TOPK without window and sink,
 * min(NB, k + window + sink) per row with them, and NB per row for
 * VSA_TOPP (any prefix length is possible). */
vsa_status vsa_query_select(const vsa_shape* shape, const vsa_select* sel, int64_t* row_ptr_len,
                            int64_t* col_capacity, size_t* plan_ws);

/* Planning with an estimator, a selection mode and sink blocks (SPADE 3.1
 * and 3.3).  Same inputs and CSR output as vsa_plan, which equals
 * vsa_plan_select with VSA_EST_MEAN, VSA_TOPK, the density as value and
 * sink 0.
 * VSA_TOPP works in float32 on the scores of the fixed order above: the
 * row max m, weights e_j = expf((s_j - m) * scale), sums over a wave in a
 * fixed order, and the prefix cut found by a search on the score keys,
 * so the index is reproducible; ties at the cut keep the lower ids.
 * Scores are assumed finite.  index->capacity must be at least
 * vsa_query_select's col_capacity; ws at least its plan_ws bytes. */
vsa_status vsa_plan_select(const void* q, const void* k, const vsa_shape* shape,
                           const vsa_select* sel, vsa_index* index, void* ws, size_t ws_bytes,
                           void* stream);

/* Option of one head in a mixed plan (DecoupAttn Plans, introduction: a
 * compiled plan gives each (timestep, layer, head) unit one option -- dense
 * or static at a keep rate theta chosen from an offline block ranking --
 * next to the dynamic estimator; SPADE 3.1: each head's scheme has its own
 * local-window length and Top-K keep). */
typedef enum { VSA_HEAD_DYNAMIC = 0, VSA_HEAD_STATIC = 1, VSA_HEAD_DENSE = 2 } vsa_head_kind;

/* kind: vsa_head_kind.
 * value: keep rate in (0, 1] for VSA_HEAD_DYNAMIC (over the estimator's
 *   scores of this call's Q and K) and VSA_HEAD_STATIC (over the caller's
 *   static score table); k as in vsa_query.  Ignored for VSA_HEAD_DENSE,
 *   which keeps every key block.
 * window_t: -1 or r >= 0, this head's temporal window as in vsa_query
 *   (a radius above nbt - 1 is treated as nbt - 1). */
typedef struct {
  int32_t kind;
  float value;
  int32_t window_t;
} vsa_head_option;

/* Host-only sizing of a mixed plan.  options: host [heads]; estimator:
 * vsa_estimator of the dynamic heads.  col_capacity = sum over rows of
 * min(NB, k_h + window blocks), exact without windows; plan_ws covers the
 * summaries (only when a head is dynamic) and the bitmaps (only when a head
 * has a window). */
vsa_status vsa_query_mixed(const vsa_shape* shape, const vsa_head_option* options, int estimator,
                           int64_t* row_ptr_len, int64_t* col_capacity, size_t* plan_ws);

/* Mixed per-head plan: row r = (b*heads + h)*NB + i of the CSR index is
 * built by head h's option (Top-K with ties to the lower id, united with
 * that head's window).  q, k: device [B, heads, N, D]; they may be NULL
 * when no head is dynamic, and the index then depends on the table alone,
 * so it can be built once and reused across calls.  static_scores: device
 * float32 [heads][NB][NB] (row i, column j = the ranking score of key
 * block j for query block i of head h, shared by every batch item), read
 * only for static heads and otherwise may be NULL.  index->window_t is set
 * to the largest head window.  Other arguments as in vsa_plan_select. */
vsa_status vsa_plan_mixed(const void* q, const void* k, const vsa_shape* shape,
                          const vsa_head_option* options, int estimator, const float* static_scores,
                          vsa_index* index, void* ws, size_t ws_bytes, void* stream);

/* Inter-block importance matrix of an estimator alone (SPADE 3.1 Fig. 4,
 * 3.3): q, k: device [B, heads, N, D]; out: device float32
 * [B, heads, NB, NB], out[.., i, j] = the score vsa_plan_select ranks for
 * query block i and key block j.  ws: device workspace of at least the
 * plan_ws that vsa_query_select reports for the same shape and estimator. */
vsa_status vsa_estimate(const void* q, const void* k, const vsa_shape* shape, int estimator, float* out,
                        void* ws, size_t ws_bytes, void* stream);

/* Block-sparse attention (SPADE 2.2 Eq. 2 with M = 0 on kept block pairs and
 * -inf elsewhere; 3.3 flash block-sparse attention and layout restore).
 * q, k, v, o: device [B, heads, N, D] in index->shape; o is written in
 * raster order.  scale: logit scale, 0 means 1/sqrt(D).  bf16 uses bf16
 * matrix cores with float32 accumulation and a float32 online softmax; f32
 * computes in float32.  A row of the index with no key blocks (never
 * produced by the planners) gives zeros for its query tokens.  ws may be
 * NULL when attn_ws is 0.
 * The index arrays are device data, read as given (the host checks only
 * the shape): row_ptr must be non-decreasing from 0 with its last entry at
 * most capacity, and every col_idx entry in use must lie in [0, nb), as the
 * planners write them.  An index that breaks this is undefined behaviour. */
vsa_status vsa_attn(const void* q, const void* k, const void* v, const vsa_index* index,
                    float scale, void* o, void* ws, size_t ws_bytes, void* stream);

/* Layout transform (SPADE 3.3: Q, K, V rearranged into the blocked layout).
 * x: device [B, heads, N, D]; xb: device [B, heads, NB, P, D] with
 * P = bt*bh*bw; rows past a block's token count are written as zero. */
vsa_status vsa_permute(const void* x, const vsa_shape* shape, void* xb, void* stream);

/* Inverse of vsa_permute (SPADE 3.3: output blocks restored to the original
 * layout); pad rows of xb are ignored. */
vsa_status vsa_unpermute(const void* xb, const vsa_shape* shape, void* x, void* stream);

/* Block means alone (the summarizer of vsa_plan, SPADE 3.1 Fig. 4(c)):
 * x: device [B, heads, N, D]; out: device float32 [B, heads, NB, D]. */
vsa_status vsa_centroids(const void* x, const vsa_shape* shape, float* out, void* stream);

/* Centroid score matrix alone (the inter-estimator of vsa_plan, SPADE 3.3):
 * qc, kc: device float32 [B, heads, NB, D]; out: device float32
 * [B, heads, NB, NB] with out[.., i, j] = <qc_i, kc_j> in vsa_plan's order. */
vsa_status vsa_centroid_scores(const float* qc, const float* kc, const vsa_shape* shape,
                               float* out, void* stream);

/* Intra-block aggregation (SPADE 3.2, Eq. 4-5 and Algorithm 1): for every
 * block of shape's blocking, the sum of all pairwise cosine similarities of
 * its token vectors, computed as the squared norm of the sum of the
 * unit-normalized tokens in float32.  A cut-short edge block uses its own
 * tokens; a zero token vector adds nothing.  x: device [B, heads, N, D];
 * out: device float32 [B, heads, NB]. */
vsa_status vsa_sics(const void* x, const vsa_shape* shape, float* out, void* stream);

/* Workspace bytes vsa_select_scheme needs for these candidates (host only).
 * candidates: host int32 [n_cand][3] block shapes (bt, bh, bw), 1 <= n_cand
 * <= VSA_MAX_SCHEMES; each must be a valid blocking of shape's grid. */
vsa_status vsa_scheme_workspace(const vsa_shape* shape, const int32_t* candidates, int n_cand,
                                size_t* ws_bytes);

/* Head-wise blocking-scheme selection (SPADE 3.2): the aggregation score of
 * a candidate is the sum of its blocks' SICS (Eq. 3); a head's score is
 * AS(Q | c) + AS(K | c) and it selects the first candidate with the highest
 * score.  shape gives B, heads, D, grid and dtype (its block fields are not
 * used).  q, k: device [B, heads, N, D]; scores: device float32
 * [n_cand, B*heads]; choice: device int32 [B*heads] (candidate index);
 * ws: device workspace of vsa_scheme_workspace bytes.  The sums run in a
 * fixed order, so the choice is reproducible. */
vsa_status vsa_select_scheme(const void* q, const void* k, const vsa_shape* shape,
                             const int32_t* candidates, int n_cand, float* scores, int32_t* choice,
                             void* ws, size_t ws_bytes, void* stream);

/* Largest plan workspace vsa_plan_noalloc holds (32 MiB per GPU). */
#define VSA_PLAN_NOALLOC_MAX_WS ((size_t)32 << 20)

/* vsa_plan for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same plan, bit for bit, with the plan workspace (block summaries and,
 * for windowed plans, per-row counts and bitmaps) taken from a static
 * device array of VSA_PLAN_NOALLOC_MAX_WS bytes inside the library instead
 * of a caller buffer.  Each GPU the library runs on holds its own copy of
 * the array until the process ends; its address is looked up once per
 * device, on the first call that runs there.  The caller still owns q, k
 * and the index arrays.  A plan whose workspace (plan_ws of vsa_query)
 * exceeds VSA_PLAN_NOALLOC_MAX_WS returns VSA_ERR_WORKSPACE before anything
 * is enqueued; the Wan2.1-1.3B, HunyuanVideo, Wan2.1-14B and 4x long-video
 * shapes need 4.1, 11.8, 13.8 and 16.6 MB.  No call allocates or frees
 * device memory.  Every call on one GPU shares that GPU's array, and every
 * value a plan reads from it is written earlier in the same call, so
 * nothing has to start at zero; two calls that overlap in time on one GPU
 * (different streams, or host threads) race on the array and must be
 * ordered by the caller.  Other arguments as in vsa_plan. */
vsa_status vsa_plan_noalloc(const void* q, const void* k, const vsa_shape* shape, const float* density,
                            int n_density, int window_t, vsa_index* index, void* stream);

/* Calls over a subset of the heads (SPADE 3.2 selects a blocking scheme
 * per head, and 3.3 groups the heads that share one into a launch): q, k,
 * v and o hold shape->heads heads ("total": [B, total, N, D]); the call
 * covers the n_heads heads listed in `heads` (host int32, distinct, each in
 * [0, total); 1 <= n_heads <= total, n_heads <= VSA_MAX_HEADS, total <=
 * 32767), all under shape's blocking.  Index row r = (b*n_heads + s)*NB + i
 * belongs to head heads[s]; index->shape is shape with heads = n_heads, so
 * vsa_query on that shape gives the index sizes and the workspace, and
 * density has 1 or n_heads entries (one per listed head).
 * qmeans, kmeans: NULL to summarize the listed heads of q and k, or the
 *   block means of every head under shape's blocking as
 *   vsa_select_scheme_means leaves them (query means [B*total][NB][D], key
 *   means [B*total][D][NB]); then q and k are not read (may be NULL) and
 *   the plan is the one vsa_plan computes, bit for bit.
 * Bad head lists are VSA_ERR_INVALID_ARG (VSA_ERR_UNSUPPORTED past the
 * limits).  Other arguments and errors as in vsa_plan. */
vsa_status vsa_plan_heads(const void* q, const void* k, const float* qmeans, const float* kmeans,
                          const vsa_shape* shape, const int32_t* heads, int n_heads, const float* density,
                          int n_density, int window_t, vsa_index* index, void* ws, size_t ws_bytes,
                          void* stream);

/* vsa_attn for an index from vsa_plan_heads: heads (host int32) lists the
 * index->shape.heads heads it covers, in its row order, among the
 * heads_total heads of q, k, v and o; only those heads of o are written.
 * Other arguments and errors as in vsa_attn. */
vsa_status vsa_attn_heads(const void* q, const void* k, const void* v, const vsa_index* index,
                          const int32_t* heads, int heads_total, float scale, void* o, void* ws,
                          size_t ws_bytes, void* stream);

/* Workspace of vsa_select_scheme_means (host only): ws_bytes, and, when
 * means_off (host [2*n_cand]) is not NULL, the byte offsets in it of each
 * candidate c's query means (means_off[2c], float32 [B*heads][NB_c][D]) and
 * key means (means_off[2c+1], float32 [B*heads][D][NB_c]).  Candidates as
 * in vsa_scheme_workspace. */
vsa_status vsa_scheme_means_workspace(const vsa_shape* shape, const int32_t* candidates, int n_cand,
                                      size_t* ws_bytes, size_t* means_off);

/* vsa_select_scheme (same scores and choice, up to float32 rounding of the
 * SICS sums) that, in the same pass over Q and K per candidate, also leaves
 * every candidate's block means of Q and K in ws at the offsets
 * vsa_scheme_means_workspace reports, in the planner's float32 order.  A
 * head's plan at its chosen candidate can then start from them
 * (vsa_plan_heads with qmeans/kmeans) without reading Q and K again:
 * SPADE 3.3 fuses blocking, summarization and intra-block estimation into
 * one pass. */
vsa_status vsa_select_scheme_means(const void* q, const void* k, const vsa_shape* shape,
                                   const int32_t* candidates, int n_cand, float* scores, int32_t* choice,
                                   void* ws, size_t ws_bytes, void* stream);

/* Measurement aid, not a step of the method: the bf16 matrix-core rate
 * this GPU sustains, the ceiling against which the attention kernel's rate
 * can be read beside the published dense peak (which assumes the full
 * 2.4 GHz clock; under load the clock depends on power, and power on the
 * data the matrix cores switch).  n_workgroups workgroups of 4 waves each
 * run `iters` rounds of 16 v_mfma_f32_32x32x16_bf16 on register operands
 * loaded once from pool; nothing else runs in the loop.  Work per call:
 * n_workgroups * 4 * iters * 16 * 32768 FLOP.
 * pool: device, at least VSA_CALIB_POOL_BYTES bytes, 16-byte aligned: 4096
 *   fragments of 64 lanes x 8 bf16, lane l of fragment f at byte
 *   (f*64 + l)*16.  Wave w of workgroup g uses fragments
 *   (16*(4g + w) + j) mod 4096 for j = 0..15, 0-7 as A operands and 8-15 as
 *   B operands (A lane l holds row l mod 32, B lane l column l mod 32, both
 *   with inner indices 8*(l/32) .. 8*(l/32)+7).  Round r multiplies
 *   A_j x B_(j+3 mod 8) and A_(j+5 mod 8) x B_j for j = 0..7.
 * out: device float32 [n_workgroups * 256]: thread t of workgroup g writes
 *   the sum of its accumulator elements at g*256 + t, so a wave's 64 values
 *   add up to the sum of every entry of its products.
 * Limits: 1 <= n_workgroups <= VSA_CALIB_MAX_WORKGROUPS, 1 <= iters <=
 * VSA_CALIB_MAX_ITERS, else VSA_ERR_INVALID_ARG (also for NULL or
 * misaligned pointers); a failed launch is VSA_ERR_HIP.  Allocates nothing. */
#define VSA_CALIB_POOL_BYTES ((size_t)4 << 20)
#define VSA_CALIB_MAX_WORKGROUPS 65536
#define VSA_CALIB_MAX_ITERS 100000
vsa_status vsa_calib_mfma_bf16(const void* pool, size_t pool_bytes, float* out, int n_workgroups, int iters,
                               void* stream);

/* Static description of a status code. */
const char* vsa_status_str(vsa_status s);

#ifdef __cplusplus
}
#endif
#endif /* VSA_H_ */
