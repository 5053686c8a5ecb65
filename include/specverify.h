/*
 * specverify.h -- C ABI of the speculative-decoding verification step on
 * AMD Instinct MI355X (gfx950).
 *
 * Pages cited (title, then address):
 *   [SSD] "自投机解码：层跳过与KV复用实现大模型无损推理加速"  (xdnf.cn/news/378309)
 *   [SD]  "企业官网建设流程全解析" -- HTML title of a page explaining the
 *         original draft-model speculative decoding (hotelren.com/news/5905390)
 *   [FS]  FlashSpec speculative-decoding practice write-up (nzsm.cn/news/47291)
 * Notation: p = target distribution, q = draft distribution, x_i = draft token
 * at draft position i, k_b = draft length of row b, a_b = accepted count.
 *
 * Conventions for every entry point
 *   - Pointers in the argument blocks are DEVICE pointers unless the field
 *     says otherwise; the argument block itself lives in host memory and is
 *     read before the call returns.
 *   - The caller owns every buffer.  The library allocates no device memory;
 *     scratch comes from the caller's workspace, sized by the *_bytes calls.
 *   - Work is enqueued on the given stream and the call returns at once: no
 *     synchronisation, no device-to-host copy.  Outputs are valid once the
 *     stream has reached the call.
 *   - Host-detectable problems (NULL required pointer, sizes out of range,
 *     bad dtype, stride < V, workspace too small) return an error before any
 *     launch and touch no output.
 *   - Problems in the data itself are reported per row in row_status (bits
 *     below).  A flagged row gets out_tokens = -1, accepted = -1,
 *     num_emitted = 0 and NaN probabilities; other rows are unaffected.
 *   - A handle caches device properties only.  One handle per host thread,
 *     or lock around it.
 */
#ifndef SPECVERIFY_H
#define SPECVERIFY_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct sv_handle_s* sv_handle;

typedef enum {
  SV_OK = 0,
  SV_E_ARG = 1,       /* NULL required pointer or a size out of range     */
  SV_E_DTYPE = 2,     /* unknown dtype                                    */
  SV_E_WORKSPACE = 3, /* workspace missing or smaller than required       */
  SV_E_DEVICE = 4,    /* a HIP call or a launch failed                    */
  SV_E_INTERNAL = 5
} sv_status;

typedef enum { SV_FP32 = 0, SV_BF16 = 1 } sv_dtype;

/* Limits checked on the host. */
#define SV_MAX_K 32          /* k_max <= SV_MAX_K                          */
#define SV_MAX_V (1 << 30)   /* V <= SV_MAX_V (greedy)                     */
#define SV_MAX_V_SAMPLED (1 << 21) /* V bound of sampled verification and
                                      draft sampling                        */

/* row_status bits */
#define SV_ROW_NONFINITE_LOGIT (1u << 0) /* NaN or +inf in a vector the row uses */
#define SV_ROW_NO_FINITE       (1u << 1) /* a vector with no finite entry        */
#define SV_ROW_BAD_TOKEN       (1u << 2) /* draft token outside [0, V)           */
#define SV_ROW_BAD_K           (1u << 3) /* k_b outside [1, k_max]               */
#define SV_ROW_BAD_TEMPERATURE (1u << 4) /* T <= 0 or not finite                 */
#define SV_ROW_BAD_TOP_P       (1u << 5) /* top_p <= 0 or NaN                    */
#define SV_ROW_BAD_PAGES       (1u << 6) /* page table inconsistent with kv_len:
                                            a page holding a rolled-back
                                            position unmapped (or past the
                                            pool), or, when pages are
                                            released, the entry just past the
                                            old length mapped                 */
#define SV_ROW_FREE_OVERFLOW   (1u << 7) /* released pages do not fit the stack  */
#define SV_ROW_BAD_ACCEPTED    (1u << 8) /* accepted outside [0, k_b] (e.g. -1
                                            from a flagged verify) or a length
                                            that would go negative            */

/* verify flags */
#define SV_FLAG_TOPP_TARGET_ONLY (1u << 0) /* truncate p only, keep q whole
                                              ([SSD] §3.4, the author's
                                              preferred variant)              */
#define SV_FLAG_RECORDS_READY    (1u << 1) /* sv_verify_sample and
                                              sv_draft_sample: the workspace
                                              already holds this call's
                                              per-vector statistics (written
                                              by sv_shard_combine with the same
                                              sizes, slots, temperature, top-p
                                              and flags); skip their pass     */

/* Poison pattern written into rolled-back KV slots when a pool is given. */
#define SV_POISON_BF16 0xFFFFu

sv_status sv_create(int hip_device, sv_handle* out);
sv_status sv_destroy(sv_handle h);
const char* sv_status_string(sv_status s);

/* Kernel timing (diagnostics).  While enabled, every kernel this handle
 * launches is bracketed by two HIP events on the caller's stream: recorded
 * around the launch, or, for the bf16 statistics kernel, attached to its
 * dispatch so that they bound its execution alone (events are created on
 * first use and reused; at most 4096 launches are
 * kept between reads).  sv_timing_read waits for those events, writes up to
 * max_entries (kernel name, launch count, total milliseconds) triples
 * accumulated since the previous read, clears the record and returns the
 * number of distinct kernels.  Names point to static strings. */
sv_status sv_timing_enable(sv_handle h, int on);
int sv_timing_read(sv_handle h, int max_entries, const char** names,
                   int32_t* launches, double* total_ms);

/* ------------------------------------------------------------------------ */
/* Verification                                                             */
/* ------------------------------------------------------------------------ */

/* Argument block shared by the sampled and greedy entry points.
 *
 * Layout: target vector (b, i), i in [0, k_max], starts at element
 * (b*(k_max+1) + i) * target_vec_stride of target_logits; draft vector
 * (b, i), i in [0, k_max), at (b*k_max + i) * draft_vec_stride.  Elements
 * are fp32 or bf16 (dtype) and contiguous inside a vector; strides are in
 * elements and must be >= V.  A torch tensor of shape [B, k_max+1, V]
 * (contiguous) has target_vec_stride = V.  16-byte aligned vectors take the
 * wide-load path; any alignment is accepted.
 *
 * Positions beyond a row's k_b are ignored (their logits need not be valid).
 */
typedef struct {
  int32_t B, k_max, V;
  int32_t dtype;                     /* sv_dtype                               */
  const void* target_logits;         /* [B][k_max+1][vec_stride]               */
  int64_t target_vec_stride;
  const void* draft_logits;          /* [B][k_max][vec_stride]; greedy: NULL
                                        means use draft_tokens                 */
  int64_t draft_vec_stride;
  const int32_t* draft_tokens;       /* [B][k_max]; sampled: required          */
  const int32_t* k_per_row;          /* [B] in [1, k_max]; NULL -> k_max       */
  const float* temperature;          /* [B] > 0, one value for p AND q
                                        ([SSD] §2.4; [FS] §5.1); sampled only */
  const float* top_p;                /* [B] in (0, 1]; NULL or >= 1 -> off     */
  uint64_t seed, offset;             /* Philox key word 0 / round counter      */
  const uint64_t* offset_dev;        /* [1] device word, or NULL: when given,
                                        the kernels read the round counter
                                        from it as they run and `offset` is
                                        ignored, so a captured graph draws
                                        fresh numbers on every replay
                                        (8-byte aligned, else SV_E_ARG)       */
  uint32_t flags;                    /* SV_FLAG_*                              */

  int32_t* out_tokens;               /* [B][k_max+1], -1 padded                */
  int32_t* accepted;                 /* [B]                                    */
  int32_t* num_emitted;              /* [B] or NULL                            */
  float* p_at_draft;                 /* [B][k_max] or NULL: p'_i(x_i)          */
  float* q_at_draft;                 /* [B][k_max] or NULL: q'_i(x_i)          */
  int32_t* row_status;               /* [B] or NULL                            */

  void* workspace;                   /* device scratch, >= the *_bytes figure  */
  size_t workspace_bytes;
} sv_verify_args;

/* Workspace for sv_verify_sample / sv_verify_greedy / sv_draft_sample with
 * these sizes (the maximum over the three).  Pure host function. */
size_t sv_verify_workspace_bytes(int32_t B, int32_t k_max, int32_t V,
                                 int32_t dtype, uint32_t flags);

/* Host-side validation only (no HIP call).  mode: 0 sampled, 1 greedy,
 * 2 draft sampling.  Returns what the entry point would return before
 * launching anything. */
sv_status sv_check_verify_args(const sv_verify_args* a, int mode);

/* Rejection-sampling verification ([SSD] §2.4, §4.3; [SD] §2.1-§2.2; [FS]
 * §2.3 with its letters swapped back):
 *   p = softmax(target/T), q = softmax(draft/T), each optionally truncated
 *   to its tie-closed top-p set and renormalised (p', q');
 *   scanning i = 0..k_b-1, accept x_i iff u(b,i,0) < p'(x_i)/q'(x_i)
 *   (ratio 0 when q'(x_i) = 0);
 *   at the first rejection a, emit y ~ norm(max(0, p'_a - q'_a)) by inverse
 *   CDF in token order with u(b,a,1) (p'_a itself if that residual is zero);
 *   if all k_b accepted, emit a bonus y ~ p'_{k_b} with u(b,k_b,1).
 * u(b,pos,draw) is the top 24 bits of word 0 of Philox4x64-10 at counter
 * (b, pos, draw, offset) and key (seed, 0), times 2^-24.
 * Outputs: out_tokens[b] = x_0..x_{a-1}, y, -1...; accepted = a;
 * num_emitted = a + 1; p_at_draft/q_at_draft = p'_i(x_i), q'_i(x_i) for
 * i < k_b and 0 beyond. */
sv_status sv_verify_sample(sv_handle h, const sv_verify_args* a, hipStream_t s);

/* sv_verify_sample for callers that cannot allocate device memory or hand
 * in a workspace (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, kernels and results
 * as sv_verify_sample; a->workspace and a->workspace_bytes are ignored: the
 * per-vector records and work-queue counters live in a device array of the
 * library, sv_noalloc_scratch_bytes() (4 MiB) per GPU, held until the
 * process ends.  The call allocates nothing.  Every call on one GPU uses
 * that GPU's array: calls that overlap on one GPU (concurrent streams, or
 * two host threads) race and corrupt each other's results; serialise them.
 * Errors: as sv_verify_sample; SV_E_WORKSPACE when the records and counters
 * of B rows at k_max (sv_verify_workspace_bytes for the sampled path) need
 * more than the array holds; SV_E_ARG with SV_FLAG_RECORDS_READY (records
 * from a shard merge sit in a caller's workspace); SV_E_DEVICE when the
 * array's device address could not be looked up at sv_create. */
size_t sv_noalloc_scratch_bytes(void);
sv_status sv_verify_sample_noalloc(sv_handle h, const sv_verify_args* a, hipStream_t s);

/* Greedy branch ([SSD] §2.4, §5.2): g_i = argmax of the raw target logits at
 * position i (lowest index on ties; temperature and top-p ignored); x_i =
 * draft_tokens, or the argmax of draft_logits when those are given; a = first
 * i with x_i != g_i, else k_b; emits x_0..x_{a-1}, g_a.  p_at_draft and
 * q_at_draft are not written. */
sv_status sv_verify_greedy(sv_handle h, const sv_verify_args* a, hipStream_t s);

/* Greedy verification in one launch instead of two, for callers that keep a
 * small state buffer between calls: same arguments, checks and results as
 * sv_verify_greedy (the same decision, [SSD] §2.4 and §5.2), bit for bit.
 * Each chunk's maximum is published with a device-scope atomic into
 * `state` and the last chunk of a row decides the row, so no second kernel
 * folds the chunks.  `state`: device memory of at least
 * sv_greedy_state_bytes(B, k_max) bytes, 8-byte aligned, all zero before
 * its first call; every call leaves it zero again.  Two calls must not use
 * one state buffer at the same time.  Layouts other than the streaming one
 * (bf16, 16-byte aligned vectors and strides, V a multiple of 8) take
 * sv_verify_greedy's two launches and leave the state as it is.  Errors:
 * those of sv_verify_greedy; SV_E_WORKSPACE for a state that is NULL,
 * misaligned or too small; nothing is launched on an error. */
size_t sv_greedy_state_bytes(int32_t B, int32_t k_max);
sv_status sv_verify_greedy_one_launch(sv_handle h, const sv_verify_args* a, void* state,
                                      size_t state_bytes, hipStream_t s);

/* Draft sampling, the step before verification ([SSD] §4.2; [FS] §3.2):
 * writes draft_tokens[b][i] = inverse CDF of q'_i with u(b,i,2) for i < k_b
 * and -1 beyond (draft_tokens is an OUTPUT here, cast away from const).
 * Uses draft_logits, temperature, top_p, k_per_row, seed, offset, flags and
 * row_status; target_logits and the verify outputs are ignored. */
sv_status sv_draft_sample(sv_handle h, const sv_verify_args* a, hipStream_t s);

/* ------------------------------------------------------------------------ */
/* KV rollback                                                              */
/* ------------------------------------------------------------------------ */

/* Paged KV pool layout (only read when poisoning):
 *   bf16 [num_pages][num_layers][2 (K, V)][kv_heads][page_size][head_dim].
 */
typedef struct {
  int32_t B, k_max, page_size, max_pages_per_seq;
  int32_t* kv_len;          /* [B] in: length after this round's k_b + 1
                               speculative writes; out: committed length     */
  const int32_t* k_per_row; /* [B] or NULL -> k_max                          */
  const int32_t* accepted;  /* [B] from a verify call on the same stream     */
  int32_t* page_table;      /* [B][max_pages_per_seq]; -1 = unmapped         */
  int32_t num_pages;        /* physical pages in the pool: mapped entries
                               must be in [0, num_pages); required (> 0)
                               when kv_pool is given, 0 = unchecked otherwise */
  int32_t* free_pages;      /* free-page stack storage, or NULL to keep
                               pages mapped and only shrink lengths          */
  int32_t* free_top;        /* [1] stack height (device)                     */
  int32_t free_capacity;   /* a stack height outside [0, capacity] makes
                               every releasing row overflow                 */
  void* kv_pool;            /* NULL, or a bf16 pool whose rolled-back slots
                               are overwritten with SV_POISON_BF16           */
  int32_t num_layers, kv_heads, head_dim;
  int32_t* row_status;      /* [B] or NULL                                   */
  void* workspace;          /* per-row decisions and counters: at least
                               sv_rollback_workspace_bytes(B) bytes (also
                               when the call is fused into verification);
                               its contents need no initialisation          */
  size_t workspace_bytes;
} sv_rollback_args;

size_t sv_rollback_workspace_bytes(int32_t B);
sv_status sv_check_rollback_args(const sv_rollback_args* a);

/* Rolls each row's KV write pointer back to the accepted prefix ([SSD] §3.3,
 * §4.3: "reset the write pointer to seq_len + i"; §4.5: one offset per
 * sequence):
 *   new = kv_len - (k_b - a_b);
 * logical pages [ceil(new/ps), ceil(old/ps)) are released ([SSD] §3.3: paged
 * caches roll back at page granularity): their entries become -1 and the
 * physical pages are pushed on the free stack in (row, page) order.  A row's
 * pages are pushed iff the running total of releases over the valid rows up
 * to it fits the capacity; otherwise the row gets SV_ROW_FREE_OVERFLOW and is
 * left unchanged.  With free_pages = NULL nothing is released and only the
 * length shrinks ([SD] §4.3).  Rows failing a check (bad k, accepted, page
 * table) are left unchanged and flagged.  The page-table check covers the
 * whole row: the first ceil(old/ps) entries must map pages in
 * [0, num_pages) (any non-negative entry when num_pages is 0) and, with a
 * free stack, every later entry must be -1, so that a row maps exactly
 * ceil(new/ps) pages after its rollback ([SSD] §3.3 asserts that the write
 * pointer equals the committed length); without a free stack, entries past
 * the length are not constrained.  With kv_pool, the slots [new, old) of
 * committed rows are poisoned in every layer and head. */
sv_status sv_kv_rollback(sv_handle h, const sv_rollback_args* a, hipStream_t s);

/* Verification followed by the rollback of its rows, the two steps of one
 * round ([SSD] §3.3 and §4.3): sv_verify_sample(v), then sv_kv_rollback(r)
 * on the accepted counts it wrote, with the results of those two calls on
 * the same stream.  r->accepted must be v->accepted, and r must have the
 * same B, k_max and k_per_row as v.  Each verification workgroup takes its
 * row's rollback decision (checks, whole page-table row, new length) on the
 * accepted count it has just found.  When r has no free stack and no KV
 * pool, a row's rollback needs nothing from the other rows and the workgroup
 * commits it; otherwise it writes the decision to r's workspace and the
 * rollback's scan (and poisoning) kernels follow.  Results equal the two
 * calls'.
 * Errors: those of the two argument checks, SV_E_ARG for arguments that do
 * not match, nothing launched on an error. */
sv_status sv_check_verify_rollback_args(const sv_verify_args* v, const sv_rollback_args* r);
sv_status sv_verify_sample_rollback(sv_handle h, const sv_verify_args* v,
                                    const sv_rollback_args* r, hipStream_t s);

/* ------------------------------------------------------------------------ */
/* Dynamic draft length and the on-device round                            */
/* ------------------------------------------------------------------------ */

/* Per-row controller of the draft length ([SSD] §3.2: raise k when the
 * acceptance rate is above 85 %, lower it below 70 %).  Each row keeps the
 * last `window` rounds' (accepted, proposed) pairs in `state`; once the window
 * is full, every round k becomes k + 1 if sum_accepted * up_den > up_num *
 * sum_proposed, else k - 1 if sum_accepted * down_den < down_num *
 * sum_proposed, clamped to [k_min, k_max].  The comparisons are on integers,
 * so the decision is exact.  Defaults that match the page: window 64,
 * up 17/20, down 7/10, k in [2, 8], start at 5 (the caller's initial k). */
typedef struct {
  int32_t B, window, k_min, k_max;
  int32_t up_num, up_den, down_num, down_den;
  const int32_t* accepted;  /* [B] from a verify call; a value outside
                               [0, k] (a flagged row), or a k outside
                               [k_min, k_max], leaves the row as is (not
                               recorded, k unchanged)                       */
  int32_t* k_per_row;       /* [B] in: k used this round; out: next round's
                               k (usable directly as the next call's
                               k_per_row)                                    */
  int32_t* state;           /* [B][window + 4] int32, all zero before the
                               first round: filled count, oldest slot, sum of
                               accepted, sum of proposed, then one slot per
                               round (accepted | proposed << 16)            */
} sv_dynk_args;

/* Host checks only: window in [1, 4096], 1 <= k_min <= k_max <= SV_MAX_K,
 * positive denominators, non-NULL arrays when B > 0. */
sv_status sv_check_dynk_args(const sv_dynk_args* a);

/* One controller update for every row, on the stream (one thread per row). */
sv_status sv_dynamic_k(sv_handle h, const sv_dynk_args* a, hipStream_t s);

/* Adds delta to the device word *offset_dev on the stream (one thread): the
 * end of a round for callers that keep the Philox round counter on the
 * device (sv_verify_args.offset_dev), so that a captured round of draft
 * sampling, verification, rollback and controller update replays without
 * any host work.  Wraps modulo 2^64.  SV_E_ARG if offset_dev is NULL or not
 * 8-byte aligned. */
sv_status sv_advance_offset(sv_handle h, uint64_t* offset_dev, uint64_t delta, hipStream_t s);

/* The end of an on-device round in one launch: sv_dynamic_k(a), then
 * sv_advance_offset(offset_dev, delta), with the results of those two calls
 * on the same stream (the controller reads nothing the counter holds), for
 * one kernel launch per round instead of two.  With a->B == 0 only the
 * counter moves.  Errors: those of sv_check_dynk_args; SV_E_ARG for a NULL
 * handle or an offset_dev that is NULL or not 8-byte aligned; nothing is
 * launched on an error. */
sv_status sv_close_round(sv_handle h, const sv_dynk_args* a, uint64_t* offset_dev,
                         uint64_t delta, hipStream_t s);

/* ------------------------------------------------------------------------ */
/* Vocabulary-sharded statistics                                            */
/* ------------------------------------------------------------------------ */

/* When a tensor-parallel LM head leaves each of G GPUs with a contiguous
 * slice of the vocabulary, every per-vector statistic of the verification
 * (the largest logit, the softmax normaliser, the tie-closed top-p
 * threshold, p'(x) and q'(x); [SSD] §2.4 and §3.4) still needs all V
 * logits.  The work splits in two: each shard counts its own columns
 * (sv_shard_stats, the streaming pass over 1/G of the bytes), and the
 * partials -- exact value counts, so merging them loses nothing -- are
 * gathered and merged into the records of the whole vectors
 * (sv_shard_combine).  On one GPU the gather is the caller handing every
 * shard's partial buffer to sv_shard_combine.  bf16 logits only.  The
 * records then drive sv_verify_sample or sv_draft_sample with
 * SV_FLAG_RECORDS_READY. */
#define SV_MAX_SHARDS 16

/* One shard's pass.  Layout: the shard's target vector (b, i), i in
 * [0, k_max], starts at element (b*(k_max+1) + i) * target_vec_stride of
 * target_shard and holds columns [col_offset, col_offset + col_count) of the
 * full vector (bf16, contiguous); draft vector (b, i) at
 * (b*k_max + i) * draft_vec_stride of draft_shard.  Strides are in elements,
 * >= col_count.  The slots counted are those of sv_verify_sample (mode 0:
 * target positions 0..k_b, draft positions 0..k_b-1) or of sv_draft_sample
 * (mode 1: draft positions only; target_shard and draft_tokens unused). */
typedef struct {
  int32_t B, k_max, V;              /* V: the full vocabulary                 */
  int32_t col_offset, col_count;    /* this shard's columns, inside [0, V)    */
  int32_t mode;                     /* 0 verification, 1 draft sampling       */
  const void* target_shard;
  int64_t target_vec_stride;
  const void* draft_shard;
  int64_t draft_vec_stride;
  const int32_t* draft_tokens;      /* [B][k_max] ids in [0, V); mode 0       */
  const int32_t* k_per_row;         /* [B] or NULL -> k_max                   */
  void* partial;                    /* out: this shard's partials, at least
                                       sv_shard_partial_bytes                 */
  size_t partial_bytes;
  void* workspace;                  /* scratch (work queues, slot list), at
                                       least sv_shard_workspace_bytes         */
  size_t workspace_bytes;
} sv_shard_stats_args;

/* Sizes of a shard's partial buffer and of its scratch.  Pure host. */
size_t sv_shard_partial_bytes(int32_t B, int32_t k_max, int32_t col_count);
size_t sv_shard_workspace_bytes(int32_t B, int32_t k_max);
sv_status sv_check_shard_stats_args(const sv_shard_stats_args* a);

/* Counts the shard's logits of every used vector slot into its partial:
 * the count of each bf16 value in the window of magnitudes [2^-24, 2^16),
 * the zeros and -infs, up to 64 nonzero values below the window, NaN / +inf
 * and whether the shard holds a value the counts cannot (a finite magnitude
 * of 2^16 or more, more than 64 values below the window, or 65536 equal
 * values), and the logit of the slot's draft token when it is one of the
 * shard's columns. */
sv_status sv_shard_stats(sv_handle h, const sv_shard_stats_args* a, hipStream_t s);

/* The merge.  Shards g = 0..G-1 must tile [0, V) in order:
 * col_offset[0] = 0, col_offset[g+1] = col_offset[g] + col_count[g],
 * and the last ends at V.  partials[g] is shard g's partial buffer from
 * sv_shard_stats with the same B, k_max, V, mode, draft_tokens and
 * k_per_row (partial_bytes[g] its size, checked like sv_shard_stats
 * checks it).  target_shards / draft_shards (with their strides) are shard
 * g's logits, as passed to sv_shard_stats: they are read only for a vector
 * whose merged counts the table cannot hold, which is then redone from the
 * logits (the generic path of sv_verify_sample).  The records are written
 * into `workspace`, a verification workspace (sv_verify_workspace_bytes
 * for B, k_max, V), exactly as the statistics pass of sv_verify_sample
 * (mode 0) or sv_draft_sample (mode 1) would write them for the
 * concatenated vectors: pass that workspace, with SV_FLAG_RECORDS_READY set,
 * to that entry point. */
typedef struct {
  int32_t B, k_max, V, mode, G;
  const void* partials[SV_MAX_SHARDS];
  size_t partial_bytes[SV_MAX_SHARDS]; /* each at least sv_shard_partial_bytes */
  int32_t col_offset[SV_MAX_SHARDS], col_count[SV_MAX_SHARDS];
  const void* target_shards[SV_MAX_SHARDS];
  int64_t target_vec_stride[SV_MAX_SHARDS];
  const void* draft_shards[SV_MAX_SHARDS];
  int64_t draft_vec_stride[SV_MAX_SHARDS];
  const int32_t* draft_tokens;      /* [B][k_max]; mode 0                      */
  const int32_t* k_per_row;         /* [B] or NULL                             */
  const float* temperature;         /* [B]                                     */
  const float* top_p;               /* [B] or NULL                             */
  uint32_t flags;                   /* SV_FLAG_TOPP_TARGET_ONLY                */
  void* workspace;                  /* out: records (a verification workspace) */
  size_t workspace_bytes;
} sv_shard_combine_args;

sv_status sv_check_shard_combine_args(const sv_shard_combine_args* a);
sv_status sv_shard_combine(sv_handle h, const sv_shard_combine_args* a, hipStream_t s);

/* The draw of sampled verification over the same shards, in two steps per
 * shard with an exchange between them.  After the acceptance scan (computed
 * alike by every shard from the merged records), the drawn position a of
 * row b needs y = min{j : C_j > u(b,a,1) R} over the whole vocabulary in
 * token order ([SSD] §2.4, §4.3; [SD] §2.2):
 *   sv_shard_draw_mass:   shard g writes masses[g][b] = {R_g, P_g}, the
 *                         residual max(0, p'_a - q'_a) and p'_a summed over
 *                         its columns (R_g = 0 for a bonus row);
 *   (exchange: every shard needs every shard's masses -- an all-gather of
 *    G x B x 16 bytes; on one GPU, one buffer written by all shards)
 *   sv_shard_draw_locate: with R = sum of R_g (or of P_g for the bonus and
 *                         for a zero residual), the shard whose running mass
 *                         in shard order first passes u R draws the token
 *                         from its own columns; every shard writes the row's
 *                         other outputs, identically.
 * Both read the records that sv_shard_combine (mode 0) wrote into
 * `records`; outputs, seed, offset and flags are those of sv_verify_sample,
 * whose results this reproduces (on one GPU: after every shard's locate). */
typedef struct {
  int32_t B, k_max, V;
  int32_t col_offset, col_count;    /* this shard's columns                   */
  int32_t G, shard;                 /* shard index in [0, G), G <= SV_MAX_SHARDS */
  const void* target_shard;         /* bf16, layout as in sv_shard_stats_args */
  int64_t target_vec_stride;
  const void* draft_shard;
  int64_t draft_vec_stride;
  const int32_t* draft_tokens;      /* [B][k_max], global ids                 */
  const int32_t* k_per_row;         /* [B] or NULL                            */
  const float* temperature;         /* [B]                                    */
  const float* top_p;               /* [B] or NULL                            */
  uint64_t seed, offset;
  const uint64_t* offset_dev;       /* as in sv_verify_args                   */
  uint32_t flags;
  const void* records;              /* the merged records: the verification
                                       workspace sv_shard_combine wrote      */
  size_t records_bytes;
  double* masses;                   /* [G][B][2] exchange buffer              */
  size_t masses_bytes;              /* at least G * B * 16                    */
  int32_t* out_tokens;              /* outputs as in sv_verify_args           */
  int32_t* accepted;
  int32_t* num_emitted;
  float* p_at_draft;
  float* q_at_draft;
  int32_t* row_status;
} sv_shard_draw_args;

sv_status sv_check_shard_draw_args(const sv_shard_draw_args* a);
sv_status sv_shard_draw_mass(sv_handle h, const sv_shard_draw_args* a, hipStream_t s);
sv_status sv_shard_draw_locate(sv_handle h, const sv_shard_draw_args* a, hipStream_t s);

#ifdef __cplusplus
}
#endif
#endif /* SPECVERIFY_H */
