// Host validation of the C ABI (block geometry, keep rate, selection and
// mixed-plan sizing, workspace layout) built without HIP by g++ with
// AddressSanitizer and UndefinedBehaviorSanitizer, driven through every
// error path and a set of valid shapes.  Exit status 0 and "host checks ok"
// on success; a failed check prints its line and exits 1.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <limits>
#include <vector>

#include "vsa_host.h"

using namespace vsa;

static int g_checks = 0;
#define CHECK(cond)                                                     \
  do {                                                                  \
    ++g_checks;                                                         \
    if (!(cond)) {                                                      \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      std::exit(1);                                                     \
    }                                                                   \
  } while (0)

static vsa_shape shape(int B, int heads, int D, int T, int H, int W, int bt, int bh, int bw, int dtype = VSA_BF16) {
  vsa_shape s;
  s.B = B; s.heads = heads; s.D = D;
  s.T = T; s.H = H; s.W = W;
  s.bt = bt; s.bh = bh; s.bw = bw;
  s.dtype = dtype;
  return s;
}

static vsa_select topk(const float* v, int n, int window = -1, int sink = 0, float scale = 0.0f, int est = VSA_EST_MEAN) {
  vsa_select s;
  s.mode = VSA_TOPK; s.n_value = n; s.value = v; s.window_t = window; s.sink = sink; s.scale = scale;
  s.estimator = est;
  return s;
}

static void shapes() {
  const vsa_shape wan = shape(1, 12, 128, 21, 30, 52, 4, 4, 8);
  CHECK(check_shape(&wan) == VSA_OK);
  CHECK(check_shape(nullptr) == VSA_ERR_INVALID_ARG);
  const int bad_fields[9][9] = {{0, 12, 128, 21, 30, 52, 4, 4, 8}, {1, 0, 128, 21, 30, 52, 4, 4, 8},
                                {1, 12, 0, 21, 30, 52, 4, 4, 8},  {1, 12, 128, 0, 30, 52, 4, 4, 8},
                                {1, 12, 128, 21, 0, 52, 4, 4, 8}, {1, 12, 128, 21, 30, -1, 4, 4, 8},
                                {1, 12, 128, 21, 30, 52, 0, 4, 8}, {1, 12, 128, 21, 30, 52, 4, -3, 8},
                                {1, 12, 128, 21, 30, 52, 4, 4, 0}};
  for (const auto& f : bad_fields) {
    const vsa_shape s = shape(f[0], f[1], f[2], f[3], f[4], f[5], f[6], f[7], f[8]);
    CHECK(check_shape(&s) == VSA_ERR_INVALID_ARG);
  }
  vsa_shape s = wan;
  s.dtype = 7;
  CHECK(check_shape(&s) == VSA_ERR_INVALID_ARG);
  s = wan; s.D = 96;
  CHECK(check_shape(&s) == VSA_ERR_UNSUPPORTED);
  s = wan; s.bt = 8; s.bh = 8; s.bw = 8;                       // 512 tokens per block
  CHECK(check_shape(&s) == VSA_ERR_UNSUPPORTED);
  s = wan; s.bt = 64; s.bh = 64; s.bw = 64; s.T = 1; s.H = 8; s.W = 16;   // box larger than the grid: cut to 128
  CHECK(check_shape(&s) == VSA_OK);
  s = shape(1, 1, 128, 1 << 11, 1 << 10, 1 << 10, 4, 4, 8);   // 2^31 tokens
  CHECK(check_shape(&s) == VSA_ERR_UNSUPPORTED);
  s = shape(1, 1, 128, 1 << 10, 1 << 10, 8, 1, 1, 8);         // one head past 2^31 bytes
  CHECK(check_shape(&s) == VSA_ERR_UNSUPPORTED);
  s = shape(1, 1, 64, 256, 256, 1, 1, 1, 1);                  // 65536 blocks
  CHECK(check_shape(&s) == VSA_ERR_UNSUPPORTED);
  s = shape(std::numeric_limits<int>::max(), std::numeric_limits<int>::max(), 64, 8, 8, 8, 2, 2, 2);
  CHECK(check_shape(&s) == VSA_ERR_UNSUPPORTED);              // element count overflow guarded
  s = shape(1, 1, 64, std::numeric_limits<int>::max(), std::numeric_limits<int>::max(), 2, 1, 1, 1);
  CHECK(check_shape(&s) == VSA_ERR_UNSUPPORTED);              // token count overflow guarded
}

static void keep_rate_and_geometry() {
  CHECK(k_rule(0.2f, 336) == 67);
  CHECK(k_rule(0.15f, 480) == 72);
  CHECK(k_rule(0.0675f, 1176) == 79);
  CHECK(k_rule(1e-9f, 336) == 1);
  CHECK(k_rule(1.0f, 336) == 336);
  const Geo g = make_geo(shape(1, 12, 128, 21, 30, 52, 4, 4, 8));
  CHECK(g.nbt == 6 && g.nbh == 8 && g.nbw == 7 && g.NB == 336 && g.N == 32760);
  int total = 0;
  for (int j = 0; j < g.NB; ++j) total += block_tokens(g, j);
  CHECK(total == g.N);
  CHECK(clamp_window(g, -1) == -1);
  CHECK(clamp_window(g, 3) == 3);
  CHECK(clamp_window(g, std::numeric_limits<int>::max()) == g.nbt - 1);
  CHECK(window_count(g, 0, 1) == 2 * 56 && window_count(g, 3, 1) == 3 * 56 && window_count(g, 2, -1) == 0);
}

static void selection() {
  const vsa_shape wan = shape(1, 12, 128, 21, 30, 52, 4, 4, 8);
  const float d02 = 0.2f;
  PlanSizes ps;
  vsa_select sel = topk(&d02, 1);
  CHECK(select_sizes(&wan, &sel, &ps) == VSA_OK);
  CHECK(ps.rows == 12 * 336 && ps.capacity == 12 * 336 * 67 && !ps.bitmap);
  CHECK(ps.ws == 2 * align256(size_t(ps.rows) * 128 * 4));
  CHECK(select_sizes(&wan, nullptr, &ps) == VSA_ERR_INVALID_ARG);
  CHECK(select_sizes(&wan, &sel, nullptr) == VSA_ERR_INVALID_ARG);
  vsa_select s2 = sel;
  s2.value = nullptr;
  CHECK(select_sizes(&wan, &s2, &ps) == VSA_ERR_INVALID_ARG);
  s2 = sel; s2.mode = 5;
  CHECK(select_sizes(&wan, &s2, &ps) == VSA_ERR_INVALID_ARG);
  s2 = sel; s2.n_value = 3;
  CHECK(select_sizes(&wan, &s2, &ps) == VSA_ERR_INVALID_ARG);
  s2 = sel; s2.window_t = -2;
  CHECK(select_sizes(&wan, &s2, &ps) == VSA_ERR_INVALID_ARG);
  s2 = sel; s2.estimator = 9;
  CHECK(select_sizes(&wan, &s2, &ps) == VSA_ERR_INVALID_ARG);
  s2 = sel; s2.sink = -1;
  CHECK(select_sizes(&wan, &s2, &ps) == VSA_ERR_INVALID_ARG);
  s2 = sel; s2.sink = 337;
  CHECK(select_sizes(&wan, &s2, &ps) == VSA_ERR_INVALID_ARG);
  s2 = sel; s2.scale = -1.0f;
  CHECK(select_sizes(&wan, &s2, &ps) == VSA_ERR_INVALID_ARG);
  s2 = sel; s2.scale = std::nanf("");
  CHECK(select_sizes(&wan, &s2, &ps) == VSA_ERR_INVALID_ARG);
  s2 = sel; s2.scale = INFINITY;
  CHECK(select_sizes(&wan, &s2, &ps) == VSA_ERR_INVALID_ARG);
  for (float bad : {0.0f, -0.1f, 1.5f, std::nanf(""), INFINITY}) {
    vsa_select s3 = topk(&bad, 1);
    CHECK(select_sizes(&wan, &s3, &ps) == VSA_ERR_INVALID_ARG);
  }
  vsa_shape many = wan;
  many.heads = VSA_MAX_HEADS + 1;
  CHECK(select_sizes(&many, &sel, &ps) == VSA_ERR_UNSUPPORTED);
  // windows, sinks and Top-P use the bitmap regions; huge radii are the full window
  for (int r : {1, 5, 32768, std::numeric_limits<int>::max()}) {
    vsa_select s3 = topk(&d02, 1, r, 2);
    CHECK(select_sizes(&wan, &s3, &ps) == VSA_OK);
    CHECK(ps.bitmap && ps.max_win == std::min(r, 5) && ps.off_bits > ps.off_cnt && ps.ws > ps.off_bits);
    for (int h = 0; h < 12; ++h) CHECK(ps.win[h] == std::min(r, 5));
  }
  vsa_select tp = sel;
  tp.mode = VSA_TOPP;
  CHECK(select_sizes(&wan, &tp, &ps) == VSA_OK);
  CHECK(ps.capacity == int64_t(12) * 336 * 336 && ps.bitmap);
  std::vector<float> per(12, 0.1f);
  per[5] = 1.0f;
  vsa_select ph = topk(per.data(), 12);
  CHECK(select_sizes(&wan, &ph, &ps) == VSA_OK);
  CHECK(ps.k[5] == 336 && ps.k[0] == 34);
  // the CSR capacity must stay addressable with int32 offsets
  const vsa_shape huge = shape(64, 256, 64, 64, 64, 64, 1, 4, 8);
  const float one = 1.0f;
  vsa_select all = topk(&one, 1);
  CHECK(select_sizes(&huge, &all, &ps) == VSA_ERR_UNSUPPORTED);
  PlanSizes pq;
  CHECK(plan_sizes(&wan, &d02, 1, -1, &pq) == VSA_OK && pq.capacity == 12 * 336 * 67);
  CHECK(plan_sizes(&wan, nullptr, 1, -1, &pq) == VSA_ERR_INVALID_ARG);
}

static void mixed() {
  const vsa_shape wan = shape(1, 3, 128, 21, 30, 52, 4, 4, 8);
  PlanSizes ps;
  vsa_head_option o[3] = {{VSA_HEAD_DYNAMIC, 0.2f, -1}, {VSA_HEAD_STATIC, 0.3f, 1}, {VSA_HEAD_DENSE, 0.0f, -1}};
  CHECK(mixed_sizes(&wan, o, VSA_EST_MEAN, &ps) == VSA_OK);
  CHECK(ps.k[0] == 67 && ps.k[1] == 101 && ps.k[2] == 336 && ps.any_dynamic && ps.any_static && ps.bitmap);
  CHECK(mixed_sizes(&wan, nullptr, VSA_EST_MEAN, &ps) == VSA_ERR_INVALID_ARG);
  CHECK(mixed_sizes(&wan, o, 3, &ps) == VSA_ERR_INVALID_ARG);
  CHECK(mixed_sizes(&wan, o, VSA_EST_MEAN, nullptr) == VSA_ERR_INVALID_ARG);
  vsa_head_option b[3] = {o[0], o[1], o[2]};
  b[0].kind = 7;
  CHECK(mixed_sizes(&wan, b, VSA_EST_MEAN, &ps) == VSA_ERR_INVALID_ARG);
  b[0] = o[0]; b[0].window_t = -2;
  CHECK(mixed_sizes(&wan, b, VSA_EST_MEAN, &ps) == VSA_ERR_INVALID_ARG);
  b[0] = o[0]; b[0].value = 0.0f;
  CHECK(mixed_sizes(&wan, b, VSA_EST_MEAN, &ps) == VSA_ERR_INVALID_ARG);
  b[0] = o[0]; b[0].value = std::nanf("");
  CHECK(mixed_sizes(&wan, b, VSA_EST_MEAN, &ps) == VSA_ERR_INVALID_ARG);
  b[0] = o[2]; b[0].value = -4.0f;                   // dense ignores its value
  CHECK(mixed_sizes(&wan, b, VSA_EST_MEAN, &ps) == VSA_OK);
  b[0] = o[0]; b[0].window_t = std::numeric_limits<int>::max();
  CHECK(mixed_sizes(&wan, b, VSA_EST_MEAN, &ps) == VSA_OK && ps.win[0] == 5 && ps.max_win == 5);
  vsa_head_option st[3] = {{VSA_HEAD_STATIC, 0.3f, -1}, {VSA_HEAD_DENSE, 0.0f, -1}, {VSA_HEAD_STATIC, 0.1f, -1}};
  CHECK(mixed_sizes(&wan, st, VSA_EST_DSA2, &ps) == VSA_OK);
  CHECK(!ps.any_dynamic && ps.ws == 0 && !ps.bitmap);
  vsa_shape many = wan;
  many.heads = VSA_MAX_HEADS + 1;
  std::vector<vsa_head_option> mo(many.heads, o[0]);
  CHECK(mixed_sizes(&many, mo.data(), VSA_EST_MEAN, &ps) == VSA_ERR_UNSUPPORTED);
}

int main() {
  shapes();
  keep_rate_and_geometry();
  selection();
  mixed();
  std::printf("host checks ok: %d\n", g_checks);
  return 0;
}
