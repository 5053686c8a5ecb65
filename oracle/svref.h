/*
 * svref.h -- plain CPU oracle for the speculative-decoding verification step.
 *
 * TEST INFRASTRUCTURE ONLY.  The tests, the smoke check and the CPU-baseline
 * leg of the benchmark are the only callers.  Nothing in the GPU library
 * includes, links or calls this code, and this code includes nothing of the
 * GPU library.  Everything is computed in IEEE fp64 with scalar loops, in the
 * order the pages describe, so that a reader can check it against them.
 *
 * Pages cited (title, then address):
 *   [SSD] "自投机解码：层跳过与KV复用实现大模型无损推理加速"  (xdnf.cn/news/378309)
 *   [SD]  "企业官网建设流程全解析" -- the HTML title of a page whose body is an
 *         explanation of the original draft-model speculative decoding
 *         (hotelren.com/news/5905390)
 *   [FS]  FlashSpec speculative-decoding practice write-up (nzsm.cn/news/47291)
 * Notation follows [SSD] and [SD]: p = target distribution, q = draft
 * distribution.  ([FS] swaps the two letters; its formulas are read with
 * them swapped back.)
 */
#ifndef SVREF_H
#define SVREF_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { SVREF_FP32 = 0, SVREF_BF16 = 1 };

/* Per-row status bits.  Same meaning as the GPU library's, defined here
 * independently. */
enum {
  SVREF_ROW_NONFINITE_LOGIT = 1 << 0, /* NaN or +inf in a logit vector used */
  SVREF_ROW_NO_FINITE       = 1 << 1, /* a vector with no finite entry     */
  SVREF_ROW_BAD_TOKEN       = 1 << 2, /* draft token outside [0, V)        */
  SVREF_ROW_BAD_K           = 1 << 3, /* k_b outside [1, k_max]            */
  SVREF_ROW_BAD_TEMPERATURE = 1 << 4, /* T <= 0 or not finite              */
  SVREF_ROW_BAD_TOP_P       = 1 << 5, /* top_p <= 0 or NaN                 */
  SVREF_ROW_BAD_PAGES       = 1 << 6, /* page table inconsistent           */
  SVREF_ROW_FREE_OVERFLOW   = 1 << 7, /* released pages do not fit         */
  SVREF_ROW_BAD_ACCEPTED    = 1 << 8  /* accepted outside [0, k_b], or a
                                          length that would go negative    */
};

/* verify flags */
enum {
  SVREF_TOPP_TARGET_ONLY = 1 << 0 /* truncate p only; q is left whole      */
};

/* ---------------------------------------------------------------------- */
/* Counter-based random numbers                                            */
/* ---------------------------------------------------------------------- */

/* Philox4x64-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As
 * Easy as 1, 2, 3", SC'11): the block for a 256-bit counter under a 128-bit
 * key. */
void svref_philox4x64_10(const uint64_t ctr[4], const uint64_t key[2],
                         uint64_t out[4]);

/* The uniform both sides draw: counter = (row, pos, draw, offset),
 * key = (seed, 0), the top 24 bits of output word 0 scaled by 2^-24, so the
 * value is exact in fp32 and lies in [0, 1).
 * draw 0 = acceptance test, 1 = residual / bonus draw, 2 = draft sampling. */
double svref_uniform(uint64_t seed, uint64_t row, uint64_t pos, uint64_t draw,
                     uint64_t offset);

/* ---------------------------------------------------------------------- */
/* One distribution: temperature softmax and tie-closed top-p              */
/* ---------------------------------------------------------------------- */

/* Computes p'_j for one logit vector z (already decoded to double):
 * p_j = exp(z_j/T - m) / S with m = max z/T and S = sum exp(z_j/T - m);
 * if 0 < top_p < 1, keep j iff sum_{i: z_i > z_j} p_i < top_p and renormalise
 * the kept mass to 1.  Returns a status bit set (0 = fine).
 * Optional outputs: *kept_mass = G (mass of the kept set before
 * renormalisation), *mass_above = mass strictly above the lowest kept value,
 * *n_kept = size of the kept set. */
int svref_softmax_topp(const double* z, int32_t V, double T, double top_p,
                       double* p_out, double* kept_mass, double* mass_above,
                       int64_t* n_kept);

/* ---------------------------------------------------------------------- */
/* Sampled verification, greedy verification, draft sampling               */
/* ---------------------------------------------------------------------- */

typedef struct {
  int32_t B, k_max, V, dtype;
  /* target vector (b, i), i in [0, k_max], starts at element
   * (b*(k_max+1) + i) * target_vec_stride; draft vector (b, i), i in
   * [0, k_max), at (b*k_max + i) * draft_vec_stride. */
  const void* target;
  int64_t target_vec_stride;
  const void* draft; /* greedy: may be NULL (then draft_tokens are used) */
  int64_t draft_vec_stride;
  const int32_t* draft_tokens; /* [B][k_max]                              */
  const int32_t* k_per_row;    /* [B] or NULL (then every row has k_max)  */
  const float* temperature;    /* [B]; unused by greedy                   */
  const float* top_p;          /* [B] or NULL; >= 1 means off             */
  uint64_t seed, offset;
  uint32_t flags;              /* SVREF_TOPP_TARGET_ONLY                  */
  int32_t nthreads;            /* worker threads over rows; <= 0 means 1  */
  const int32_t* row_ids;      /* [B] or NULL: the row index each row uses
                                  in the random counter (lets a subset of a
                                  batch be checked row by row)            */

  /* outputs (host memory) */
  int32_t* out_tokens;  /* [B][k_max+1], -1 padded                        */
  int32_t* accepted;    /* [B]; -1 on a row error                         */
  int32_t* num_emitted; /* [B] or NULL                                    */
  double* p_at_draft;   /* [B][k_max] or NULL: p'_i(x_i)                  */
  double* q_at_draft;   /* [B][k_max] or NULL: q'_i(x_i)                  */
  int32_t* row_status;  /* [B] or NULL                                    */

  /* diagnostics for the parity comparator (each NULL or as sized) */
  double* diag_rho;         /* [B][k_max]   rho_i = p'/q' (0 if q' = 0)   */
  double* diag_acc_margin;  /* [B][k_max]   u_i - rho_i                   */
  double* diag_cdf_margin;  /* [B]   distance of u to the nearest edge of
                               the chosen token's CDF interval (relative)  */
  double* diag_topp_margin_t; /* [B][k_max+1] min(|M_> - P|, |G - P|)     */
  double* diag_topp_margin_d; /* [B][k_max]                               */
  double* diag_residual_mass; /* [B]   R at the resampled position, or -1
                                 when the bonus path was taken            */
  /* draft sampling fills diag_acc_margin[b][i] with the CDF margin of its
   * draw at position i and diag_topp_margin_d with the top-p margins      */

  /* What-if inputs, so that a result that differs from the oracle's can be
   * checked against the oracle's own distributions (each NULL or as sized):
   * forced_accepted [B]: draw at this position instead of at the scan's
   *   first rejection (a value outside [0, k_b] is ignored); every
   *   diagnostic keeps its meaning, and the draw is the one the oracle makes
   *   when the scan stops there.
   * probe_token: verification [B], draft sampling [B][k_max]: a token whose
   *   interval in the drawn distribution is reported in diag_probe as
   *   {C_{t-1}/R, C_t/R, r_t/R, u}: the CDF just below and at t, the token's
   *   share of the mass and the uniform of the draw (NaN when t is not in
   *   [0, V)). */
  const int32_t* forced_accepted;
  const int32_t* probe_token;
  double* diag_probe;
} svref_verify_args;

/* Rejection-sampling verification, one row at a time ([SSD] §2.4, §4.3;
 * [SD] §2.1-§2.2).  Returns 0, or -1 on a malformed argument block. */
int svref_verify_sample(const svref_verify_args* a);

/* Greedy branch ([SSD] §2.4, §5.2): argmax compare, first index on ties. */
int svref_verify_greedy(const svref_verify_args* a);

/* Draft sampling from q' with draw 2 (the step before verification in
 * [SSD] §4.2 and [FS] §3.2): for i < k_b writes draft_tokens[b][i]
 * (the field is written through a cast), -1 beyond k_b or on a row error. */
int svref_draft_sample(const svref_verify_args* a, int32_t* tokens_out);

/* ---------------------------------------------------------------------- */
/* KV rollback                                                            */
/* ---------------------------------------------------------------------- */

typedef struct {
  int32_t B, k_max, page_size, max_pages_per_seq;
  int32_t* kv_len;             /* [B] in: after this round's writes; out  */
  const int32_t* k_per_row;    /* [B] or NULL -> k_max                     */
  const int32_t* accepted;     /* [B]                                      */
  int32_t* page_table;         /* [B][max_pages_per_seq], -1 = unmapped    */
  int32_t num_pages;           /* pool size; mapped entries must be below
                                  it (0 = unchecked, not allowed with a pool) */
  int32_t* free_pages;         /* stack storage, or NULL = keep pages      */
  int32_t* free_top;           /* [1] stack height                         */
  int32_t free_capacity;
  uint16_t* kv_pool;           /* NULL, or bf16 pool to poison             */
  int32_t num_layers, kv_heads, head_dim;
  int32_t* row_status;         /* [B] or NULL                              */
} svref_rollback_args;

/* Rolls each row's write pointer back to the accepted prefix and releases
 * whole pages beyond it ([SSD] §3.3, §4.3, §4.5; [SD] §4.3). */
int svref_kv_rollback(const svref_rollback_args* a);

#define SVREF_POISON_BF16 0xFFFFu

/* ---------------------------------------------------------------------- */
/* Dynamic draft length                                                   */
/* ---------------------------------------------------------------------- */

/* Per row, the history of the rounds seen so far: the accepted count and the
 * proposed draft length of each, oldest first.  Once `window` rounds have
 * been seen, every round: the draft length goes up by one when the
 * acceptance rate of the last `window` rounds, sum_acc / sum_prop, is above
 * up_num / up_den, down by one when it is below down_num / down_den, within
 * [k_min, k_max] ([SSD] §3.2: raise k above 85 %, lower it below 70 %).
 * Rates are compared as integer cross products, so the decision is exact.
 * A round whose k lies outside [k_min, k_max] or whose accepted count lies
 * outside [0, k] is not recorded and leaves k as it is. */
typedef struct {
  int32_t B, window, k_min, k_max;
  int32_t up_num, up_den, down_num, down_den;
  const int32_t* accepted;  /* [B] this round's accepted count             */
  int32_t* k_per_row;       /* [B] in: k used this round; out: next k      */
  int32_t* hist_accepted;   /* [B][capacity] accepted count of each round  */
  int32_t* hist_proposed;   /* [B][capacity] k of each round               */
  int32_t* hist_len;        /* [B] rounds recorded so far                  */
  int32_t capacity;         /* rounds each history row holds; a row that is
                               full when a round arrives makes the call
                               return -1                                    */
} svref_dynk_args;

int svref_dynamic_k(const svref_dynk_args* a);

#ifdef __cplusplus
}
#endif
#endif
