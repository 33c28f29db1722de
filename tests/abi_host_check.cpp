// Host-side checks of the C ABI (include/stca.h) for a build with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code: every call here either runs host-only code (workspace
// sizing, the stochastic-length and LITM planners, diagnostics) or must fail its argument checks
// before touching the device.  No GPU is needed; the process exits non-zero on the first wrong
// status, and the sanitizers abort it on any memory error or undefined behaviour they detect.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <random>
#include <vector>

#include "stca.h"

static int g_failures = 0;
#define EXPECT(cond)                                                        \
  do {                                                                      \
    if (!(cond)) {                                                          \
      fprintf(stderr, "FAILED %s:%d: %s (%s)\n", __FILE__, __LINE__, #cond, \
              stca_last_error());                                           \
      ++g_failures;                                                         \
    }                                                                       \
  } while (0)

static stca_dims dims(int d, int h, int M, int r, int dtype) {
  stca_dims dm;
  memset(&dm, 0, sizeof dm);
  dm.d = d;
  dm.h = h;
  dm.M = M;
  dm.r = r;
  dm.dtype = dtype;
  dm.ln_eps = 1e-5f;
  return dm;
}

// Device pointers are never dereferenced by the calls below (they fail before any device work);
// aligned, nonzero values stand in for them.
static void *fake(uintptr_t v) { return (void *)v; }

static void workspace_sizes() {
  // the five workloads' shapes
  struct W { int d, h, M, r, users; int64_t L, T, maxL, maxT; } ws[] = {
      {64, 4, 1, 2, 1, 256, 4, 256, 4},
      {128, 8, 2, 2, 256, 256 * 2048, 256 * 8, 2048, 8},
      {256, 8, 3, 4, 512, 1000161, 3110, 10000, 16},
      {256, 8, 3, 4, 1024, 10240000, 16384, 10000, 16},
      {512, 16, 4, 4, 256, 5120000, 8192, 20000, 32},
  };
  for (const W &w : ws) {
    for (int dt = 0; dt < 2; ++dt) {
      stca_dims dm = dims(w.d, w.h, w.M, w.r, dt);
      stca_batch b = {w.users, (const int64_t *)fake(256), (const int64_t *)fake(512), w.L, w.T, w.maxL, w.maxT};
      size_t e = 0, a = 0, f = 0, p = 0, bw = 0, bk = 0;
      EXPECT(stca_encode_workspace_size(&dm, w.L, &e) == STCA_OK);
      EXPECT(stca_attend_workspace_size(&dm, &b, &a) == STCA_OK);
      EXPECT(stca_forward_workspace_size(&dm, &b, &f) == STCA_OK);
      EXPECT(stca_predict_workspace_size(&dm, w.T, &p) == STCA_OK);
      EXPECT(stca_backward_workspace_size(&dm, &b, &bw) == STCA_OK);
      EXPECT(stca_backward_workspace_size_keep(&dm, &b, &bk) == STCA_OK);
      EXPECT(e > 0 && a > 0 && f >= a && p > 0 && bw > 0);
      // the fp32 path can keep the encode's intermediates; the mixed-precision (bf16) path recomputes
      EXPECT(dt == STCA_F32 ? bk > bw : bk == bw);
      EXPECT(f % 256 == 0 && a % 256 == 0);
    }
  }
}

static void argument_errors() {
  stca_dims good = dims(256, 8, 2, 4, STCA_BF16);
  size_t n = 0;
  stca_dims bad[] = {dims(100, 4, 1, 2, 1), dims(256, 3, 1, 2, 1), dims(256, 8, 0, 2, 1), dims(256, 8, 9, 2, 1),
                     dims(256, 8, 1, 0, 1), dims(256, 8, 1, 9, 1), dims(256, 8, 1, 2, 7)};
  for (stca_dims &dm : bad) EXPECT(stca_encode_workspace_size(&dm, 10, &n) == STCA_E_DIMS);
  stca_dims eps0 = good;
  eps0.ln_eps = 0.f;
  EXPECT(stca_encode_workspace_size(&eps0, 10, &n) == STCA_E_DIMS);
  stca_dims chunk = good;
  chunk.attn_chunk = 33;
  EXPECT(stca_encode_workspace_size(&chunk, 10, &n) == STCA_E_DIMS);
  stca_dims layers = good;
  layers.encode_layers = 3;
  EXPECT(stca_encode_workspace_size(&layers, 10, &n) == STCA_E_DIMS);
  EXPECT(stca_encode_workspace_size(nullptr, 10, &n) == STCA_E_ARG);
  EXPECT(stca_encode_workspace_size(&good, -1, &n) == STCA_E_ARG);
  EXPECT(stca_encode_workspace_size(&good, 10, nullptr) == STCA_E_ARG);

  // batch checks
  stca_batch b = {2, (const int64_t *)fake(256), (const int64_t *)fake(512), 100, 4, 60, 2};
  EXPECT(stca_attend_workspace_size(&good, &b, &n) == STCA_OK);
  stca_batch nb = b;
  nb.max_L = 40;  // 2 * 40 < 100: not an upper bound
  EXPECT(stca_attend_workspace_size(&good, &nb, &n) == STCA_E_ARG);
  nb = b;
  nb.hist_off = (const int64_t *)fake(258);
  EXPECT(stca_attend_workspace_size(&good, &nb, &n) == STCA_E_ALIGN);
  nb = b;
  nb.n_users = 0;
  EXPECT(stca_attend_workspace_size(&good, &nb, &n) == STCA_E_ARG);
  nb = b;
  nb.tgt_off = nullptr;
  EXPECT(stca_attend_workspace_size(&good, &nb, &n) == STCA_E_ARG);

  // weights / calls: every error is reported before device work
  stca_weights w;
  memset(&w, 0, sizeof w);
  EXPECT(stca_forward(&good, &w, &b, fake(4096), fake(8192), (float *)fake(12288), fake(16384), 1 << 30, nullptr) ==
         STCA_E_ARG);
  for (int i = 0; i < STCA_MAX_M; ++i) {
    stca_ffn f = {fake(4096), fake(4096), fake(4096), (const float *)fake(4096), (const float *)fake(4096)};
    w.hist[i] = w.query[i] = f;
    w.WQ[i] = w.WK[i] = w.WV[i] = w.WO[i] = w.WC[i] = fake(4096);
  }
  size_t need = 0;
  EXPECT(stca_forward_workspace_size(&good, &b, &need) == STCA_OK);
  EXPECT(stca_forward(&good, &w, &b, fake(4096), fake(8192), (float *)fake(12288), fake(16384), need - 1, nullptr) ==
         STCA_E_WORKSPACE);
  EXPECT(stca_forward(&good, &w, &b, fake(4097), fake(8192), (float *)fake(12288), fake(16384), need, nullptr) ==
         STCA_E_ALIGN);
  w.WC[1] = nullptr;
  EXPECT(stca_forward(&good, &w, &b, fake(4096), fake(8192), (float *)fake(12288), fake(16384), need, nullptr) ==
         STCA_E_ARG);
  w.WC[1] = fake(4096);
  EXPECT(stca_attend(&good, &w, 2, &b, fake(4096), (const float *)fake(4096), (float *)fake(4096), fake(4096), 1 << 30,
                     nullptr) == STCA_E_ARG);  // layer out of range
  EXPECT(stca_encode(&good, &w.hist[0], 10, nullptr, fake(4096), fake(4096), 1 << 30, nullptr) == STCA_E_ARG);
  EXPECT(stca_predict(&good, nullptr, &w.hist[0], 10, (const float *)fake(4096), fake(4096), (float *)fake(4096),
                      fake(4096), 1 << 30, nullptr) == STCA_E_ARG);
  EXPECT(stca_validate_batch(&b, nullptr, nullptr) == STCA_E_ARG);
  EXPECT(stca_validate_batch(&b, (int32_t *)fake(4098), nullptr) == STCA_E_ALIGN);

  // the allocation-free attention refuses a batch beyond its scratch before any device work
  stca_batch big = {1024, (const int64_t *)fake(256), (const int64_t *)fake(512), 10240000, 16384, 10000, 16};
  EXPECT(stca_attend_noalloc(&good, &w, 0, &big, fake(4096), (const float *)fake(4096), (float *)fake(4096), nullptr) ==
         STCA_E_WORKSPACE);

  // backward: NULL gradient pointers
  stca_grads g;
  memset(&g, 0, sizeof g);
  EXPECT(stca_backward(&good, &w, &b, fake(4096), fake(4096), (const float *)fake(4096), &g, fake(4096), 1 << 30,
                       nullptr) == STCA_E_ARG);

  // debug-build flags: the ordinary build checks nothing and touches no device
  uint32_t dflags = 123;
  int32_t denabled = 7;
  EXPECT(stca_debug_flags(&dflags, &denabled, 1) == STCA_OK && dflags == 0 && denabled == 0);
  EXPECT(stca_debug_flags(nullptr, &denabled, 0) == STCA_E_ARG);

  // diagnostics
  for (int s = -6; s <= 1; ++s) EXPECT(stca_status_string(s) != nullptr);
  EXPECT(strlen(stca_version()) > 0);
  EXPECT(stca_graph_destroy(nullptr) == STCA_OK);
}

static void stochastic_length_plans() {
  std::mt19937_64 rng(7);
  stca_sl_params p = {8, 10000, 2000, 10000};
  double beta = 0;
  EXPECT(stca_sl_beta(&p, 0.02, &beta) == STCA_OK && beta > 0);
  stca_sl_params badp = {8, 100, 200, 100};
  EXPECT(stca_sl_beta(&badp, 0.02, &beta) == STCA_E_ARG);
  for (int trial = 0; trial < 20; ++trial) {
    const int n = 1 + (int)(rng() % 300);
    std::vector<int64_t> full(n), len(n), off(n + 1);
    std::vector<double> s(n);
    std::vector<int32_t> order(n);
    for (int u = 0; u < n; ++u) {
      full[u] = (int64_t)(rng() % 12000);
      s[u] = (double)(rng() % 1000001) / 1e6;
      order[u] = u;
    }
    std::shuffle(order.begin(), order.end(), rng);
    EXPECT(stca_sl_plan(&p, n, full.data(), s.data(), order.data(), len.data(), off.data()) == STCA_OK);
    int64_t tot = 0;
    for (int u = 0; u < n; ++u) {
      EXPECT(len[u] >= 0 && len[u] <= full[u] && len[u] <= p.L_infer);
      EXPECT(off[u + 1] - off[u] == len[u]);
      tot += len[u];
    }
    EXPECT(off[0] == 0 && off[n] == tot && tot <= (int64_t)n * p.L_avg);
    order[0] = order[n > 1 ? 1 : 0] + (n > 1 ? 0 : n);  // not a permutation
    EXPECT(stca_sl_plan(&p, n, full.data(), s.data(), order.data(), len.data(), off.data()) == STCA_E_ARG);
  }
}

static void litm_plans() {
  std::mt19937_64 rng(11);
  for (int trial = 0; trial < 20; ++trial) {
    const int n = 1 + (int)(rng() % 50);
    std::vector<int64_t> off(n + 1, 0);
    for (int u = 0; u < n; ++u) off[u + 1] = off[u] + (int64_t)(rng() % 400);
    const int64_t total = off[n];
    std::vector<int64_t> ids(total > 0 ? total : 1);
    for (int64_t i = 0; i < total; ++i) ids[i] = (int64_t)(rng() % 40);
    std::vector<int64_t> merged(n + 1), group(total + 1), members(total > 0 ? total : 1);
    int64_t ng = -1;
    EXPECT(stca_litm_plan(n, off.data(), ids.data(), 3, merged.data(), group.data(), members.data(), &ng) == STCA_OK);
    EXPECT(ng >= 0 && ng <= total && merged[n] == ng && group[0] == 0 && group[ng] == total);
    std::vector<char> seen(total > 0 ? total : 1, 0);
    for (int64_t j = 0; j < total; ++j) {
      EXPECT(members[j] >= 0 && members[j] < total);
      if (members[j] >= 0 && members[j] < total) seen[members[j]]++;
    }
    for (int64_t j = 0; j < total; ++j) EXPECT(seen[j] == 1);
    EXPECT(stca_litm_plan(n, off.data(), ids.data(), -1, merged.data(), group.data(), members.data(), &ng) ==
           STCA_E_ARG);
  }
}

int main() {
  workspace_sizes();
  argument_errors();
  stochastic_length_plans();
  litm_plans();
  if (g_failures) {
    fprintf(stderr, "%d check(s) failed\n", g_failures);
    return 1;
  }
  printf("abi host checks passed\n");
  return 0;
}
