/*
 * Memory and undefined-behaviour check of the CPU oracle: built with the
 * address and undefined-behaviour sanitizers together with oracle/svref.c,
 * it calls every entry point of the oracle on many small random problems,
 * every optional output and diagnostic requested, with the awkward inputs
 * the entry points promise to handle (-inf and NaN logits, vectors with no
 * finite entry, ties, top-p at and past its ends, bad temperatures, k and
 * tokens out of range, forced positions and probe tokens, padded strides,
 * one and several threads).  The sanitizers abort on the first bad access;
 * the driver itself checks only the invariants every result must satisfy.
 *
 * Test infrastructure: tests/test_host_sanitizers.py builds and runs it.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "svref.h"

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;

static uint32_t rnd(void) { /* xorshift64* */
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return (uint32_t)((rng_state * 0x2545F4914F6CDD1Dull) >> 32);
}
static int rint_in(int lo, int hi) { return lo + (int)(rnd() % (uint32_t)(hi - lo + 1)); }
static double runif(void) { return (rnd() + 0.5) / 4294967296.0; }

static uint16_t to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

static int failures = 0;
#define CHECK(c)                                                      \
  do {                                                                \
    if (!(c)) {                                                       \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
      ++failures;                                                     \
    }                                                                 \
  } while (0)

/* A logit value of one of the kinds the oracle must take. */
static float logit(int kind) {
  switch (kind) {
    case 0: return (float)(4.0 * (runif() - 0.5));
    case 1: return -INFINITY;
    case 2: return 1.5f; /* ties */
    case 3: return NAN;
    case 4: return (float)(-1e4 * runif());
    default: return (float)(0.01 * (runif() - 0.5));
  }
}

static void fill(float* z, int n, int profile) {
  for (int j = 0; j < n; ++j) {
    int kind = 0;
    const uint32_t r = rnd() % 100;
    if (profile == 1 && r < 30) kind = 1;
    if (profile == 2 && r < 50) kind = 2;
    if (profile == 3 && r < 2) kind = 3;
    if (profile == 4) kind = 1; /* no finite entry */
    if (profile == 5 && r < 40) kind = 4;
    if (profile == 6) kind = 5;
    z[j] = logit(kind);
  }
}

static void one_sampled_case(int it) {
  const int B = rint_in(1, 6), K = rint_in(1, 4), V = rint_in(1, 40);
  const int dtype = rnd() & 1;
  const int pad = rint_in(0, 3);
  const int64_t ts = V + pad, ds = V + pad;
  const size_t nt = (size_t)B * (K + 1) * ts, nd = (size_t)B * K * ds;
  float* zt = malloc(nt * sizeof(float));
  float* zd = malloc(nd * sizeof(float));
  for (size_t v = 0; v < (size_t)B * (K + 1); ++v) fill(zt + v * ts, (int)ts, rint_in(0, 7));
  for (size_t v = 0; v < (size_t)B * K; ++v) fill(zd + v * ds, (int)ds, rint_in(0, 7));
  uint16_t *bt = NULL, *bd = NULL;
  if (dtype == SVREF_BF16) {
    bt = malloc(nt * 2);
    bd = malloc(nd * 2);
    for (size_t i = 0; i < nt; ++i) bt[i] = to_bf16(zt[i]);
    for (size_t i = 0; i < nd; ++i) bd[i] = to_bf16(zd[i]);
  }
  int32_t* toks = malloc(sizeof(int32_t) * B * K);
  int32_t* kpr = malloc(sizeof(int32_t) * B);
  float* T = malloc(sizeof(float) * B);
  float* P = malloc(sizeof(float) * B);
  int32_t* rows = malloc(sizeof(int32_t) * B);
  int32_t* forced = malloc(sizeof(int32_t) * B);
  int32_t* probe = malloc(sizeof(int32_t) * B * K);
  for (int b = 0; b < B; ++b) {
    kpr[b] = rint_in(0, K + 1);
    const uint32_t r = rnd() % 10;
    T[b] = r == 0 ? 0.0f : r == 1 ? -1.0f : r == 2 ? INFINITY : (float)(0.05 + 2 * runif());
    const uint32_t s = rnd() % 10;
    P[b] = s == 0 ? 0.0f : s == 1 ? NAN : s == 2 ? 1.0f : s == 3 ? 2.0f : s == 4 ? 1e-9f
                                                                         : (float)runif();
    rows[b] = rint_in(0, 1000);
    forced[b] = rint_in(-1, K + 1);
    for (int i = 0; i < K; ++i) {
      toks[b * K + i] = rint_in(-1, V);
      probe[b * K + i] = rint_in(-1, V);
    }
  }
  int32_t* out = malloc(sizeof(int32_t) * B * (K + 1));
  int32_t *acc = malloc(sizeof(int32_t) * B), *nem = malloc(sizeof(int32_t) * B);
  int32_t* st = malloc(sizeof(int32_t) * B);
  double* px = malloc(sizeof(double) * B * K);
  double* qx = malloc(sizeof(double) * B * K);
  double* rho = malloc(sizeof(double) * B * K);
  double* am = malloc(sizeof(double) * B * K);
  double* cm = malloc(sizeof(double) * B);
  double* tmt = malloc(sizeof(double) * B * (K + 1));
  double* tmd = malloc(sizeof(double) * B * K);
  double* rm = malloc(sizeof(double) * B);
  double* dp = malloc(sizeof(double) * B * K * 4);

  svref_verify_args a;
  memset(&a, 0, sizeof a);
  a.B = B;
  a.k_max = K;
  a.V = V;
  a.dtype = dtype;
  a.target = dtype == SVREF_BF16 ? (const void*)bt : (const void*)zt;
  a.target_vec_stride = ts;
  a.draft = dtype == SVREF_BF16 ? (const void*)bd : (const void*)zd;
  a.draft_vec_stride = ds;
  a.draft_tokens = toks;
  a.k_per_row = (rnd() & 1) ? kpr : NULL;
  a.temperature = T;
  a.top_p = (rnd() & 1) ? P : NULL;
  a.seed = rnd();
  a.offset = rnd();
  a.flags = (rnd() & 1) ? SVREF_TOPP_TARGET_ONLY : 0u;
  a.nthreads = it % 3 == 0 ? 3 : 1;
  a.row_ids = (rnd() & 1) ? rows : NULL;
  a.out_tokens = out;
  a.accepted = acc;
  a.num_emitted = nem;
  a.p_at_draft = px;
  a.q_at_draft = qx;
  a.row_status = st;
  a.diag_rho = rho;
  a.diag_acc_margin = am;
  a.diag_cdf_margin = cm;
  a.diag_topp_margin_t = tmt;
  a.diag_topp_margin_d = tmd;
  a.diag_residual_mass = rm;
  a.forced_accepted = (rnd() & 1) ? forced : NULL;
  a.probe_token = (rnd() & 1) ? probe : NULL;
  a.diag_probe = dp;

  CHECK(svref_verify_sample(&a) == 0);
  for (int b = 0; b < B; ++b) {
    CHECK(acc[b] >= -1 && acc[b] <= K);
    if (st[b] == 0) {
      const int kb = a.k_per_row ? kpr[b] : K;
      CHECK(acc[b] >= 0 && acc[b] <= kb);
      CHECK(out[b * (K + 1) + acc[b]] >= 0 && out[b * (K + 1) + acc[b]] < V);
    }
  }
  /* draft sampling over the same inputs (its probes are per position) */
  int32_t* dt = malloc(sizeof(int32_t) * B * K);
  a.probe_token = (rnd() & 1) ? probe : NULL;
  CHECK(svref_draft_sample(&a, dt) == 0);
  for (int b = 0; b < B * K; ++b) CHECK(dt[b] >= -1 && dt[b] < V);
  /* greedy, with and without draft logits */
  if (rnd() & 1) a.draft = NULL;
  CHECK(svref_verify_greedy(&a) == 0);
  for (int b = 0; b < B; ++b) CHECK(acc[b] >= -1 && acc[b] <= K);
  /* one distribution on its own */
  double* zz = malloc(sizeof(double) * V);
  double* pp = malloc(sizeof(double) * V);
  for (int j = 0; j < V; ++j) zz[j] = zt[j];
  double G = 0, M = 0;
  int64_t nk = 0;
  svref_softmax_topp(zz, V, T[0], P[0], pp, &G, &M, &nk);
  CHECK(nk >= 0 && nk <= V);

  free(zz); free(pp); free(dt);
  free(zt); free(zd); free(bt); free(bd); free(toks); free(kpr); free(T); free(P);
  free(rows); free(forced); free(probe); free(out); free(acc); free(nem); free(st);
  free(px); free(qx); free(rho); free(am); free(cm); free(tmt); free(tmd); free(rm); free(dp);
}

static void one_rollback_case(void) {
  const int B = rint_in(1, 8), K = rint_in(1, 5), ps = rint_in(1, 4), MP = rint_in(1, 12);
  const int pool_pages = B * MP + 8;
  int32_t* kv = malloc(sizeof(int32_t) * B);
  int32_t* kpr = malloc(sizeof(int32_t) * B);
  int32_t* acc = malloc(sizeof(int32_t) * B);
  int32_t* pt = malloc(sizeof(int32_t) * B * MP);
  int32_t* st = malloc(sizeof(int32_t) * B);
  int next = 0;
  for (int b = 0; b < B; ++b) {
    kv[b] = rint_in(-2, MP * ps + 2);
    kpr[b] = rint_in(0, K + 1);
    acc[b] = rint_in(-1, K + 1);
    for (int j = 0; j < MP; ++j) {
      const uint32_t r = rnd() % 20;
      pt[b * MP + j] = r == 0 ? -1 : r == 1 ? pool_pages + 3 : r == 2 ? -5 : next++ % pool_pages;
    }
  }
  const int cap = rint_in(0, B * MP + 4);
  int32_t* fp = malloc(sizeof(int32_t) * (cap + 1));
  int32_t top = rint_in(-1, cap);
  const int L = rint_in(1, 2), H = rint_in(1, 2), D = rint_in(1, 4);
  uint16_t* pool = malloc(sizeof(uint16_t) * (size_t)pool_pages * L * 2 * H * ps * D);
  memset(pool, 0, sizeof(uint16_t) * (size_t)pool_pages * L * 2 * H * ps * D);
  svref_rollback_args r;
  memset(&r, 0, sizeof r);
  r.B = B;
  r.k_max = K;
  r.page_size = ps;
  r.max_pages_per_seq = MP;
  r.kv_len = kv;
  r.k_per_row = (rnd() & 1) ? kpr : NULL;
  r.accepted = acc;
  r.page_table = pt;
  r.num_pages = pool_pages;
  r.free_pages = (rnd() & 1) ? fp : NULL;
  r.free_top = &top;
  r.free_capacity = cap;
  r.kv_pool = (rnd() & 1) ? pool : NULL;
  r.num_layers = L;
  r.kv_heads = H;
  r.head_dim = D;
  r.row_status = st;
  const int rc = svref_kv_rollback(&r);
  CHECK(rc == 0 || rc == -1);
  free(kv); free(kpr); free(acc); free(pt); free(st); free(fp); free(pool);
}

static void one_dynk_case(void) {
  const int B = rint_in(1, 8), W = rint_in(1, 6), cap = rint_in(1, 40);
  int32_t* acc = malloc(sizeof(int32_t) * B);
  int32_t* k = malloc(sizeof(int32_t) * B);
  int32_t* ha = malloc(sizeof(int32_t) * B * cap);
  int32_t* hp = malloc(sizeof(int32_t) * B * cap);
  int32_t* hl = calloc(B, sizeof(int32_t));
  for (int b = 0; b < B; ++b) k[b] = rint_in(1, 9);
  svref_dynk_args d;
  memset(&d, 0, sizeof d);
  d.B = B;
  d.window = W;
  d.k_min = 2;
  d.k_max = 8;
  d.up_num = 17;
  d.up_den = 20;
  d.down_num = 7;
  d.down_den = 10;
  d.accepted = acc;
  d.k_per_row = k;
  d.hist_accepted = ha;
  d.hist_proposed = hp;
  d.hist_len = hl;
  d.capacity = cap;
  for (int round = 0; round < cap + 2; ++round) {
    for (int b = 0; b < B; ++b) acc[b] = rint_in(-1, k[b] + 1);
    const int rc = svref_dynamic_k(&d);
    CHECK(rc == 0 || rc == -1);
    if (rc) break;
    for (int b = 0; b < B; ++b) CHECK(k[b] >= 1 && k[b] <= 9);
  }
  free(acc); free(k); free(ha); free(hp); free(hl);
}

int main(int argc, char** argv) {
  const int n = argc > 1 ? atoi(argv[1]) : 400;
  for (int it = 0; it < n; ++it) {
    one_sampled_case(it);
    one_rollback_case();
    one_dynk_case();
  }
  uint64_t c[4] = {1, 2, 3, 4}, k[2] = {5, 6}, o[4];
  svref_philox4x64_10(c, k, o);
  const double u = svref_uniform(1, 2, 3, 0, 4);
  CHECK(u >= 0.0 && u < 1.0);
  if (failures) {
    fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  printf("oracle fuzz ok: %d cases\n", n);
  return 0;
}
