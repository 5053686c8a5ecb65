/*
 * svref.c -- plain CPU oracle for the speculative-decoding verification step.
 *
 * TEST INFRASTRUCTURE ONLY (see svref.h).  Slow on purpose: every logit is
 * decoded to double, every probability is formed in fp64 with std exp(), and
 * every prefix is a left-to-right loop.  Compile without -ffast-math and
 * with -ffp-contract=off so the arithmetic is plain IEEE fp64.
 *
 * Page tags [SSD], [SD], [FS] are defined in svref.h.
 */
#define _GNU_SOURCE
#include "svref.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* ====================================================================== */
/* Philox4x64-10                                                           */
/* ====================================================================== */

/* Constants of Philox4x64 as published by Salmon et al. (SC'11): the two
 * round multipliers and the two Weyl key increments (golden ratio and
 * sqrt(3)-1, as 64-bit fractions). */
#define PHILOX_M0 0xD2E7470EE14C6C93ULL
#define PHILOX_M1 0xCA5A826395121157ULL
#define PHILOX_W0 0x9E3779B97F4A7C15ULL
#define PHILOX_W1 0xBB67AE8584CAA73BULL

void svref_philox4x64_10(const uint64_t ctr[4], const uint64_t key[2],
                         uint64_t out[4]) {
  uint64_t x0 = ctr[0], x1 = ctr[1], x2 = ctr[2], x3 = ctr[3];
  uint64_t k0 = key[0], k1 = key[1];
  for (int round = 0; round < 10; ++round) {
    /* one Philox round: two 64x64->128 products, the high halves mixed with
     * the other two words and the round key, the low halves passed on */
    unsigned __int128 p0 = (unsigned __int128)PHILOX_M0 * x0;
    unsigned __int128 p1 = (unsigned __int128)PHILOX_M1 * x2;
    uint64_t hi0 = (uint64_t)(p0 >> 64), lo0 = (uint64_t)p0;
    uint64_t hi1 = (uint64_t)(p1 >> 64), lo1 = (uint64_t)p1;
    uint64_t y0 = hi1 ^ x1 ^ k0;
    uint64_t y1 = lo1;
    uint64_t y2 = hi0 ^ x3 ^ k1;
    uint64_t y3 = lo0;
    x0 = y0; x1 = y1; x2 = y2; x3 = y3;
    /* key schedule: add the Weyl increments between rounds */
    k0 += PHILOX_W0;
    k1 += PHILOX_W1;
  }
  out[0] = x0; out[1] = x1; out[2] = x2; out[3] = x3;
}

/* The pages only ask that both sides share one seeded random state ([FS]
 * §5.1, [SSD] §5.2).  The counter layout is this library's choice. */
double svref_uniform(uint64_t seed, uint64_t row, uint64_t pos, uint64_t draw,
                     uint64_t offset) {
  uint64_t ctr[4] = {row, pos, draw, offset};
  uint64_t key[2] = {seed, 0};
  uint64_t out[4];
  svref_philox4x64_10(ctr, key, out);
  return (double)(out[0] >> 40) * (1.0 / 16777216.0);
}

/* ====================================================================== */
/* One distribution                                                        */
/* ====================================================================== */

static double decode_logit(const void* base, int32_t dtype, int64_t idx) {
  if (dtype == SVREF_BF16) {
    /* bf16 is the upper half of an IEEE binary32: widening is exact */
    uint16_t h = ((const uint16_t*)base)[idx];
    uint32_t bits = (uint32_t)h << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
  }
  return (double)((const float*)base)[idx];
}

static int cmp_desc(const void* a, const void* b) {
  double x = *(const double*)a, y = *(const double*)b;
  return (x < y) - (x > y);
}

/* Checks that do not need a temperature: NaN or +inf anywhere, or no finite
 * entry at all. */
static int vector_status(const double* z, int32_t V) {
  int st = 0, any_finite = 0;
  for (int32_t j = 0; j < V; ++j) {
    if (isnan(z[j]) || (isinf(z[j]) && z[j] > 0)) st |= SVREF_ROW_NONFINITE_LOGIT;
    else if (isfinite(z[j])) any_finite = 1;
  }
  if (!any_finite) st |= SVREF_ROW_NO_FINITE;
  return st;
}

int svref_softmax_topp(const double* z, int32_t V, double T, double top_p,
                       double* p_out, double* kept_mass, double* mass_above,
                       int64_t* n_kept) {
  int st = vector_status(z, V);
  if (!(T > 0.0) || !isfinite(T)) st |= SVREF_ROW_BAD_TEMPERATURE;
  if (isnan(top_p) || top_p <= 0.0) st |= SVREF_ROW_BAD_TOP_P;
  if (st) return st;

  /* Temperature softmax, the same T on both sides ([SSD] §2.4; [FS] §2.3):
   * p_j = exp(z_j/T - m) / S, m = max z/T. */
  double m = -INFINITY;
  for (int32_t j = 0; j < V; ++j) {
    double s = z[j] / T;
    if (s > m) m = s;
  }
  double S = 0.0;
  for (int32_t j = 0; j < V; ++j) {
    double w = exp(z[j] / T - m); /* exp(-inf) = 0 for masked entries */
    p_out[j] = w;
    S += w;
  }
  for (int32_t j = 0; j < V; ++j) p_out[j] /= S;

  if (!(top_p < 1.0)) { /* top-p off */
    if (kept_mass) *kept_mass = 1.0;
    if (mass_above) *mass_above = 0.0;
    if (n_kept) {
      int64_t n = 0;
      for (int32_t j = 0; j < V; ++j) n += p_out[j] > 0.0;
      *n_kept = n;
    }
    return 0;
  }

  /* Top-p ([FS] §3.2 sorts, takes the cumulative sum and drops a token when
   * the mass before it already exceeds top_p; [SSD] §3.4 truncates both
   * sides the same way, then renormalises).  Read tie-closed: keep j iff the
   * mass of tokens with a strictly larger logit is below top_p.  The kept set
   * is then {j : z_j >= tau} for the lowest kept value tau. */
  double* sorted = (double*)malloc(sizeof(double) * (size_t)V);
  memcpy(sorted, z, sizeof(double) * (size_t)V);
  qsort(sorted, (size_t)V, sizeof(double), cmp_desc);
  double before = 0.0; /* mass of values strictly above the current group */
  double tau = sorted[0], tau_before = 0.0;
  int32_t g = 0;
  while (g < V) {
    double v = sorted[g];
    int32_t e = g;
    double group = 0.0;
    while (e < V && sorted[e] == v) {
      group += exp(v / T - m) / S;
      ++e;
    }
    if (before < top_p) { tau = v; tau_before = before; }
    else break;
    before += group;
    g = e;
  }
  free(sorted);

  double G = 0.0;
  int64_t n = 0;
  for (int32_t j = 0; j < V; ++j) {
    if (z[j] >= tau) { G += p_out[j]; ++n; }
  }
  for (int32_t j = 0; j < V; ++j) p_out[j] = (z[j] >= tau) ? p_out[j] / G : 0.0;
  if (kept_mass) *kept_mass = G;
  if (mass_above) *mass_above = tau_before;
  if (n_kept) *n_kept = n;
  return 0;
}

/* ====================================================================== */
/* Row helpers                                                             */
/* ====================================================================== */

typedef struct {
  const svref_verify_args* a;
  int32_t k;
  double* z;   /* scratch: one decoded vector  */
  double* pa;  /* scratch: p' at one position   */
  double* qa;  /* scratch: q' at one position   */
} row_ctx;

static void load_target(const row_ctx* c, int32_t b, int32_t i) {
  const svref_verify_args* a = c->a;
  int64_t base = ((int64_t)b * (a->k_max + 1) + i) * a->target_vec_stride;
  for (int32_t j = 0; j < a->V; ++j)
    c->z[j] = decode_logit(a->target, a->dtype, base + j);
}

static void load_draft(const row_ctx* c, int32_t b, int32_t i) {
  const svref_verify_args* a = c->a;
  int64_t base = ((int64_t)b * a->k_max + i) * a->draft_vec_stride;
  for (int32_t j = 0; j < a->V; ++j)
    c->z[j] = decode_logit(a->draft, a->dtype, base + j);
}

static uint64_t row_id(const svref_verify_args* a, int32_t b) {
  return a->row_ids ? (uint64_t)a->row_ids[b] : (uint64_t)b;
}

static double row_top_p(const svref_verify_args* a, int32_t b) {
  return a->top_p ? (double)a->top_p[b] : 1.0;
}

/* Top-p margin of one distribution: how close the decisive masses are to P */
static double topp_margin(double P, double G, double above) {
  if (!(P < 1.0)) return INFINITY;
  double m1 = fabs(above - P), m2 = fabs(G - P);
  return m1 < m2 ? m1 : m2;
}

static void write_row_error(const svref_verify_args* a, int32_t b, int st,
                            int with_probs) {
  for (int32_t j = 0; j <= a->k_max; ++j)
    a->out_tokens[(int64_t)b * (a->k_max + 1) + j] = -1;
  a->accepted[b] = -1;
  if (a->num_emitted) a->num_emitted[b] = 0;
  if (with_probs) {
    for (int32_t i = 0; i < a->k_max; ++i) {
      if (a->p_at_draft) a->p_at_draft[(int64_t)b * a->k_max + i] = NAN;
      if (a->q_at_draft) a->q_at_draft[(int64_t)b * a->k_max + i] = NAN;
    }
  }
  if (a->row_status) a->row_status[b] = st;
}

/* Inverse CDF in token-index order: y = min{j : C_j > u * R} where C is the
 * left-to-right prefix of r and R = C_{V-1}.  Tokens with r_j = 0 can never
 * be chosen because the comparison is strict. */
static int32_t inverse_cdf(const double* r, int32_t V, double u, double* margin,
                           double* total) {
  double R = 0.0;
  for (int32_t j = 0; j < V; ++j) R += r[j];
  double target = u * R;
  double C = 0.0, prev = 0.0;
  int32_t y = -1;
  for (int32_t j = 0; j < V; ++j) {
    prev = C;
    C += r[j];
    if (C > target) { y = j; break; }
  }
  if (margin) {
    double lo = fabs(prev / R - u), hi = fabs(C / R - u);
    *margin = lo < hi ? lo : hi;
  }
  if (total) *total = R;
  return y;
}

/* Where token t lies in the inverse CDF over r: the prefix just below it and
 * at it, normalised by the total as inverse_cdf forms them (the same
 * left-to-right sums), its own share, and the uniform of the draw. */
static void probe_interval(const double* r, int32_t V, int32_t t, double u,
                           double out[4]) {
  out[3] = u;
  if (t < 0 || t >= V) { out[0] = out[1] = out[2] = NAN; return; }
  double C = 0.0, below = 0.0, at = 0.0;
  for (int32_t j = 0; j < V; ++j) {
    if (j == t) below = C;
    C += r[j];
    if (j == t) at = C;
  }
  out[0] = below / C;
  out[1] = at / C;
  out[2] = r[t] / C;
}

/* Basic per-row checks shared by all entry points. */
static int row_header_status(const svref_verify_args* a, int32_t b, int32_t* k_out,
                             int check_sampling) {
  int st = 0;
  int32_t k = a->k_per_row ? a->k_per_row[b] : a->k_max;
  if (k < 1 || k > a->k_max) st |= SVREF_ROW_BAD_K;
  if (check_sampling) {
    double T = (double)a->temperature[b];
    if (!(T > 0.0) || !isfinite(T)) st |= SVREF_ROW_BAD_TEMPERATURE;
    double P = row_top_p(a, b);
    if (isnan(P) || P <= 0.0) st |= SVREF_ROW_BAD_TOP_P;
  }
  *k_out = k;
  return st;
}

/* ====================================================================== */
/* Sampled verification                                                    */
/* ====================================================================== */

static void sample_row(row_ctx* c, int32_t b) {
  const svref_verify_args* a = c->a;
  const int32_t V = a->V, K = a->k_max;
  int32_t k;
  int st = row_header_status(a, b, &k, 1);
  if (st & SVREF_ROW_BAD_K) { write_row_error(a, b, st, 1); return; }
  for (int32_t i = 0; i < k; ++i) {
    int32_t x = a->draft_tokens[(int64_t)b * K + i];
    if (x < 0 || x >= V) st |= SVREF_ROW_BAD_TOKEN;
  }
  /* data checks on every vector the row uses */
  for (int32_t i = 0; i <= k; ++i) {
    load_target(c, b, i);
    st |= vector_status(c->z, V);
    if (i < k) {
      load_draft(c, b, i);
      st |= vector_status(c->z, V);
    }
  }
  if (st) { write_row_error(a, b, st, 1); return; }

  const double T = (double)a->temperature[b];
  const double P = row_top_p(a, b);
  const double Pq = (a->flags & SVREF_TOPP_TARGET_ONLY) ? 1.0 : P;

  /* p'_i(x_i), q'_i(x_i) at every draft position */
  double px[64], qx[64];
  for (int32_t i = 0; i < k; ++i) {
    int32_t x = a->draft_tokens[(int64_t)b * K + i];
    double G, above;
    load_target(c, b, i);
    svref_softmax_topp(c->z, V, T, P, c->pa, &G, &above, NULL);
    px[i] = c->pa[x];
    if (a->diag_topp_margin_t) a->diag_topp_margin_t[(int64_t)b * (K + 1) + i] = topp_margin(P, G, above);
    load_draft(c, b, i);
    svref_softmax_topp(c->z, V, T, Pq, c->qa, &G, &above, NULL);
    qx[i] = c->qa[x];
    if (a->diag_topp_margin_d) a->diag_topp_margin_d[(int64_t)b * K + i] = topp_margin(Pq, G, above);
  }
  if (a->diag_topp_margin_t) {
    double G, above;
    load_target(c, b, k);
    svref_softmax_topp(c->z, V, T, P, c->pa, &G, &above, NULL);
    a->diag_topp_margin_t[(int64_t)b * (K + 1) + k] = topp_margin(P, G, above);
  }

  /* Left-to-right chain: accept x_i with probability min(1, p'/q'), stop at
   * the first rejection and discard every later draft ([SD] §2.2; [SSD] §4.3).
   * Accept iff u < rho; rho = 0 when q'(x) = 0 ([SSD] §4.3 sets the ratio to
   * zero there).  Since u < 1, rho >= 1 always accepts. */
  int32_t acc = k;
  for (int32_t i = 0; i < k; ++i) {
    double rho = qx[i] > 0.0 ? px[i] / qx[i] : 0.0;
    double u = svref_uniform(a->seed, row_id(a, b), (uint64_t)i, 0, a->offset);
    if (a->diag_rho) a->diag_rho[(int64_t)b * K + i] = rho;
    if (a->diag_acc_margin) a->diag_acc_margin[(int64_t)b * K + i] = u - rho;
    if (!(u < rho)) { acc = i; break; }
  }
  for (int32_t i = acc + 1; i < k; ++i) {
    double rho = qx[i] > 0.0 ? px[i] / qx[i] : 0.0;
    if (a->diag_rho) a->diag_rho[(int64_t)b * K + i] = rho;
    if (a->diag_acc_margin) {
      double u = svref_uniform(a->seed, row_id(a, b), (uint64_t)i, 0, a->offset);
      a->diag_acc_margin[(int64_t)b * K + i] = u - rho;
    }
  }

  /* what-if: the draw the oracle makes when the scan stops at a given
   * position (used to check a result that stopped elsewhere) */
  if (a->forced_accepted) {
    int32_t f = a->forced_accepted[b];
    if (f >= 0 && f <= k) acc = f;
  }

  double u1 = svref_uniform(a->seed, row_id(a, b), (uint64_t)acc, 1, a->offset);
  int32_t y;
  double margin = INFINITY, R = -1.0;
  const double* drawn; /* the distribution the token is drawn from */
  if (acc < k) {
    /* First rejection: resample from norm(max(0, p' - q')) ([SSD] §2.4 and
     * §5.2 insist on the clamp; [SD] §2.1).  If that residual is all zero,
     * fall back to p' itself ([SSD] §4.3). */
    load_target(c, b, acc);
    svref_softmax_topp(c->z, V, T, P, c->pa, NULL, NULL, NULL);
    load_draft(c, b, acc);
    svref_softmax_topp(c->z, V, T, Pq, c->qa, NULL, NULL, NULL);
    double Rsum = 0.0;
    for (int32_t j = 0; j < V; ++j) {
      double d = c->pa[j] - c->qa[j];
      c->qa[j] = d > 0.0 ? d : 0.0; /* reuse qa as r */
      Rsum += c->qa[j];
    }
    drawn = Rsum == 0.0 ? c->pa : c->qa;
    y = inverse_cdf(drawn, V, u1, &margin, NULL);
    R = Rsum;
  } else {
    /* Every draft accepted: one bonus token from p' at position k
     * ([SD] §2.2; [SSD] §2.1 and §4.3). */
    load_target(c, b, k);
    svref_softmax_topp(c->z, V, T, P, c->pa, NULL, NULL, NULL);
    drawn = c->pa;
    y = inverse_cdf(drawn, V, u1, &margin, NULL);
  }
  if (a->probe_token && a->diag_probe)
    probe_interval(drawn, V, a->probe_token[b], u1, a->diag_probe + (int64_t)b * 4);

  int64_t ob = (int64_t)b * (K + 1);
  for (int32_t j = 0; j <= K; ++j) a->out_tokens[ob + j] = -1;
  for (int32_t i = 0; i < acc; ++i) a->out_tokens[ob + i] = a->draft_tokens[(int64_t)b * K + i];
  a->out_tokens[ob + acc] = y;
  a->accepted[b] = acc;
  if (a->num_emitted) a->num_emitted[b] = acc + 1;
  for (int32_t i = 0; i < K; ++i) {
    if (a->p_at_draft) a->p_at_draft[(int64_t)b * K + i] = i < k ? px[i] : 0.0;
    if (a->q_at_draft) a->q_at_draft[(int64_t)b * K + i] = i < k ? qx[i] : 0.0;
  }
  if (a->row_status) a->row_status[b] = 0;
  if (a->diag_cdf_margin) a->diag_cdf_margin[b] = margin;
  if (a->diag_residual_mass) a->diag_residual_mass[b] = R;
}

/* ====================================================================== */
/* Greedy verification                                                     */
/* ====================================================================== */

/* First index of the largest value. */
static int32_t argmax_first(const double* z, int32_t V) {
  int32_t best = 0;
  for (int32_t j = 1; j < V; ++j)
    if (z[j] > z[best]) best = j;
  return best;
}

static void greedy_row(row_ctx* c, int32_t b) {
  const svref_verify_args* a = c->a;
  const int32_t V = a->V, K = a->k_max;
  int32_t k;
  int st = row_header_status(a, b, &k, 0);
  if (st) { write_row_error(a, b, st, 0); return; }
  int32_t g[64], x[64];
  for (int32_t i = 0; i < k; ++i) {
    if (a->draft) {
      load_draft(c, b, i);
      st |= vector_status(c->z, V);
      x[i] = argmax_first(c->z, V);
    } else {
      x[i] = a->draft_tokens[(int64_t)b * K + i];
      if (x[i] < 0 || x[i] >= V) st |= SVREF_ROW_BAD_TOKEN;
    }
  }
  for (int32_t i = 0; i <= k; ++i) {
    load_target(c, b, i);
    st |= vector_status(c->z, V);
    g[i] = argmax_first(c->z, V);
  }
  if (st) { write_row_error(a, b, st, 0); return; }
  /* Greedy has no sampling: accept while the draft token equals the target
   * argmax; at the first difference emit the target argmax ([SSD] §2.4). */
  int32_t acc = k;
  for (int32_t i = 0; i < k; ++i)
    if (x[i] != g[i]) { acc = i; break; }
  int64_t ob = (int64_t)b * (K + 1);
  for (int32_t j = 0; j <= K; ++j) a->out_tokens[ob + j] = -1;
  for (int32_t i = 0; i < acc; ++i) a->out_tokens[ob + i] = x[i];
  a->out_tokens[ob + acc] = g[acc];
  a->accepted[b] = acc;
  if (a->num_emitted) a->num_emitted[b] = acc + 1;
  if (a->row_status) a->row_status[b] = 0;
}

/* ====================================================================== */
/* Draft sampling                                                          */
/* ====================================================================== */

typedef struct {
  row_ctx c;
  int32_t* out;
} draft_ctx;

static void draft_row(row_ctx* c, int32_t b, int32_t* out) {
  const svref_verify_args* a = c->a;
  const int32_t V = a->V, K = a->k_max;
  int32_t k;
  /* status bits follow the verify call: header checks, then the data
   * checks of every vector the row uses when k_b itself is valid */
  int st = row_header_status(a, b, &k, 1);
  for (int32_t i = 0; i < K; ++i) out[(int64_t)b * K + i] = -1;
  if (!(st & SVREF_ROW_BAD_K)) {
    for (int32_t i = 0; i < k; ++i) {
      load_draft(c, b, i);
      st |= vector_status(c->z, V);
    }
  }
  if (a->row_status) a->row_status[b] = st;
  if (st) return;
  const double T = (double)a->temperature[b];
  const double P = (a->flags & SVREF_TOPP_TARGET_ONLY) ? 1.0 : row_top_p(a, b);
  for (int32_t i = 0; i < k; ++i) {
    load_draft(c, b, i);
    double G, above, margin;
    svref_softmax_topp(c->z, V, T, P, c->qa, &G, &above, NULL);
    double u = svref_uniform(a->seed, row_id(a, b), (uint64_t)i, 2, a->offset);
    out[(int64_t)b * K + i] = inverse_cdf(c->qa, V, u, &margin, NULL);
    if (a->probe_token && a->diag_probe)
      probe_interval(c->qa, V, a->probe_token[(int64_t)b * K + i], u,
                     a->diag_probe + ((int64_t)b * K + i) * 4);
    if (a->diag_acc_margin) a->diag_acc_margin[(int64_t)b * K + i] = margin;
    if (a->diag_topp_margin_d) a->diag_topp_margin_d[(int64_t)b * K + i] = topp_margin(P, G, above);
  }
}

/* ====================================================================== */
/* Threads over rows                                                       */
/* ====================================================================== */

typedef struct {
  const svref_verify_args* a;
  int mode; /* 0 sample, 1 greedy, 2 draft */
  int32_t* draft_out;
  int tid, nthreads;
} worker_arg;

static void* worker(void* p) {
  worker_arg* w = (worker_arg*)p;
  const svref_verify_args* a = w->a;
  row_ctx c;
  c.a = a;
  c.k = 0;
  c.z = (double*)malloc(sizeof(double) * (size_t)a->V);
  c.pa = (double*)malloc(sizeof(double) * (size_t)a->V);
  c.qa = (double*)malloc(sizeof(double) * (size_t)a->V);
  for (int32_t b = w->tid; b < a->B; b += w->nthreads) {
    if (w->mode == 0) sample_row(&c, b);
    else if (w->mode == 1) greedy_row(&c, b);
    else draft_row(&c, b, w->draft_out);
  }
  free(c.z); free(c.pa); free(c.qa);
  return NULL;
}

static int run_rows(const svref_verify_args* a, int mode, int32_t* draft_out) {
  if (!a || a->B < 0 || a->V <= 0 || a->k_max < 1 || a->k_max > 64) return -1;
  if (a->dtype != SVREF_FP32 && a->dtype != SVREF_BF16) return -1;
  if (!a->target || !a->out_tokens || !a->accepted) {
    if (mode != 2) return -1;
  }
  int n = a->nthreads > 0 ? a->nthreads : 1;
  if (n > a->B) n = a->B > 0 ? a->B : 1;
  pthread_t th[256];
  worker_arg wa[256];
  if (n > 256) n = 256;
  for (int t = 0; t < n; ++t) {
    wa[t].a = a; wa[t].mode = mode; wa[t].draft_out = draft_out;
    wa[t].tid = t; wa[t].nthreads = n;
  }
  if (n == 1) { worker(&wa[0]); return 0; }
  for (int t = 0; t < n; ++t) pthread_create(&th[t], NULL, worker, &wa[t]);
  for (int t = 0; t < n; ++t) pthread_join(th[t], NULL);
  return 0;
}

int svref_verify_sample(const svref_verify_args* a) {
  if (!a || !a->draft || !a->draft_tokens || !a->temperature) return -1;
  return run_rows(a, 0, NULL);
}

int svref_verify_greedy(const svref_verify_args* a) {
  if (!a || (!a->draft && !a->draft_tokens)) return -1;
  return run_rows(a, 1, NULL);
}

int svref_draft_sample(const svref_verify_args* a, int32_t* tokens_out) {
  if (!a || !a->draft || !a->temperature || !tokens_out) return -1;
  return run_rows(a, 2, tokens_out);
}

/* ====================================================================== */
/* KV rollback                                                             */
/* ====================================================================== */

static int32_t ceil_div(int32_t x, int32_t d) { return (x + d - 1) / d; }

int svref_kv_rollback(const svref_rollback_args* a) {
  if (!a || a->B < 0 || a->k_max < 1 || a->page_size < 1 ||
      a->max_pages_per_seq < 1 || !a->kv_len || !a->accepted || !a->page_table)
    return -1;
  if (a->free_pages && (!a->free_top || a->free_capacity < 0)) return -1;
  if (a->kv_pool && a->num_pages <= 0) return -1;
  const int32_t ps = a->page_size, MP = a->max_pages_per_seq;
  int32_t* st = (int32_t*)calloc((size_t)(a->B > 0 ? a->B : 1), sizeof(int32_t));
  int32_t* newlen = (int32_t*)calloc((size_t)(a->B > 0 ? a->B : 1), sizeof(int32_t));
  int32_t* nrel = (int32_t*)calloc((size_t)(a->B > 0 ? a->B : 1), sizeof(int32_t));

  /* 1. Per-row checks and the new length.  After a round that wrote k_b + 1
   * slots, a_b accepted drafts leave old - (k_b - a_b) valid slots: the
   * caller's "write pointer = seq_len + i" of [SSD] §4.3, counted after the
   * writes.  The development-time assertion of [SSD] §3.3 (pointer equals
   * the committed length) becomes the page-table consistency check. */
  for (int32_t b = 0; b < a->B; ++b) {
    int32_t k = a->k_per_row ? a->k_per_row[b] : a->k_max;
    int32_t acc = a->accepted[b];
    int32_t old = a->kv_len[b];
    if (k < 1 || k > a->k_max) st[b] |= SVREF_ROW_BAD_K;
    else if (acc < 0 || acc > k || old - (k - acc) < 0) st[b] |= SVREF_ROW_BAD_ACCEPTED;
    if (old < 0 || ceil_div(old, ps) > MP) st[b] |= SVREF_ROW_BAD_PAGES;
    if (!st[b]) {
      /* The whole row of the page table must agree with the length: every
       * logical page below ceil(old/ps) maps a page of the pool, and, when
       * pages are released onto a free stack, every later entry is
       * unmapped, so the row maps exactly ceil(old/ps) pages and after the
       * rollback exactly ceil(new/ps).  Without a free stack, pages past the
       * length stay mapped by design ([SD] §4.3): those entries are free. */
      int32_t used = ceil_div(old, ps);
      for (int32_t pg = 0; pg < MP; ++pg) {
        int32_t e = a->page_table[(int64_t)b * MP + pg];
        if (pg < used) {
          if (e < 0 || (a->num_pages > 0 && e >= a->num_pages)) st[b] |= SVREF_ROW_BAD_PAGES;
        } else if (a->free_pages && e != -1) {
          st[b] |= SVREF_ROW_BAD_PAGES;
        }
      }
    }
    if (!st[b]) {
      newlen[b] = old - (k - acc);
      /* Paged cache: release whole logical pages beyond the new length
       * ([SSD] §3.3: page granularity) */
      nrel[b] = ceil_div(old, ps) - ceil_div(newlen[b], ps);
    }
  }

  /* 2. Free-stack pushes in (row, page) order.  A row's pages fit iff the
   * running total of releases over the valid rows up to and including it
   * stays within the stack capacity; a row that does not fit is flagged and
   * left untouched (and so is every later row that releases a page). */
  int32_t top0 = a->free_pages ? a->free_top[0] : 0;
  int64_t running = 0;
  int64_t pushed = 0;
  for (int32_t b = 0; b < a->B; ++b) {
    if (st[b]) continue;
    running += nrel[b];
    if (!a->free_pages || nrel[b] == 0) continue;
    if (top0 < 0 || (int64_t)top0 + running > a->free_capacity) {
      st[b] |= SVREF_ROW_FREE_OVERFLOW;
      continue;
    }
    int32_t first = ceil_div(newlen[b], ps);
    for (int32_t j = 0; j < nrel[b]; ++j)
      a->free_pages[top0 + (running - nrel[b]) + j] =
          a->page_table[(int64_t)b * MP + first + j];
    pushed = running;
  }

  /* 3. Optional poisoning of the rolled-back slots, then the commit. */
  for (int32_t b = 0; b < a->B; ++b) {
    if (st[b]) continue;
    int32_t old = a->kv_len[b];
    if (a->kv_pool) {
      for (int32_t pos = newlen[b]; pos < old; ++pos) {
        int32_t page = a->page_table[(int64_t)b * MP + pos / ps];
        int32_t slot = pos % ps;
        for (int32_t l = 0; l < a->num_layers; ++l)
          for (int32_t kv = 0; kv < 2; ++kv)
            for (int32_t h = 0; h < a->kv_heads; ++h) {
              /* pool layout [page][layer][K|V][head][slot][dim] */
              int64_t off = ((((int64_t)page * a->num_layers + l) * 2 + kv) * a->kv_heads + h);
              off = (off * ps + slot) * a->head_dim;
              for (int32_t d = 0; d < a->head_dim; ++d) a->kv_pool[off + d] = SVREF_POISON_BF16;
            }
      }
    }
    if (a->free_pages) {
      int32_t first = ceil_div(newlen[b], ps);
      for (int32_t j = 0; j < nrel[b]; ++j) a->page_table[(int64_t)b * MP + first + j] = -1;
    }
    a->kv_len[b] = newlen[b];
  }
  if (a->free_pages) a->free_top[0] = top0 + (int32_t)pushed;
  if (a->row_status)
    for (int32_t b = 0; b < a->B; ++b) a->row_status[b] = st[b];
  free(st); free(newlen); free(nrel);
  return 0;
}

/* ====================================================================== */
/* Dynamic draft length                                                    */
/* ====================================================================== */

int svref_dynamic_k(const svref_dynk_args* a) {
  if (!a || a->B < 0 || a->window < 1 || a->k_min < 1 || a->k_max < a->k_min ||
      a->up_den <= 0 || a->down_den <= 0 || a->capacity < 0)
    return -1;
  if (a->B > 0 && (!a->accepted || !a->k_per_row || !a->hist_accepted ||
                   !a->hist_proposed || !a->hist_len))
    return -1;
  for (int32_t b = 0; b < a->B; ++b)
    if (a->hist_len[b] < 0 || a->hist_len[b] > a->capacity) return -1;
  const int32_t W = a->window;
  for (int32_t b = 0; b < a->B; ++b) {
    const int32_t k = a->k_per_row[b];
    const int32_t acc = a->accepted[b];
    /* A round teaches the controller only if it verified a draft length the
     * controller could have chosen and its accepted count is possible: a
     * row error (accepted -1) or a k outside [k_min, k_max] leaves the row
     * as it is. */
    if (k < a->k_min || k > a->k_max || acc < 0 || acc > k) continue;
    int32_t* ha = a->hist_accepted + (int64_t)b * a->capacity;
    int32_t* hp = a->hist_proposed + (int64_t)b * a->capacity;
    int32_t n = a->hist_len[b];
    if (n == a->capacity) return -1; /* the caller's history is full */
    ha[n] = acc;
    hp[n] = k;
    a->hist_len[b] = ++n;
    /* [SSD] §3.2: the acceptance rate over the last W rounds, once W rounds
     * have been seen; above the upper threshold k grows by one, below the
     * lower one it shrinks by one, within [k_min, k_max] */
    int32_t next = k;
    if (n >= W) {
      int64_t sa = 0, sp = 0;
      for (int32_t r = n - W; r < n; ++r) { sa += ha[r]; sp += hp[r]; }
      if (sa * a->up_den > (int64_t)a->up_num * sp) next = k + 1;
      else if (sa * a->down_den < (int64_t)a->down_num * sp) next = k - 1;
    }
    if (next > a->k_max) next = a->k_max;
    if (next < a->k_min) next = a->k_min;
    a->k_per_row[b] = next;
  }
  return 0;
}
