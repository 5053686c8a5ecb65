/*
 * Memory and undefined-behaviour check of the library's host side: built
 * with the address and undefined-behaviour sanitizers against a host-only
 * build of the library sources, it drives every pure-host entry point
 * (workspace sizes, argument checks, status strings) and every launching
 * entry point's checks before the device is touched (a NULL handle), with
 * valid argument blocks and with blocks whose fields are replaced, one or
 * several at a time, by extreme values: negative and huge sizes, NULL and
 * misaligned pointers, mismatched shapes.  Size arithmetic that overflowed
 * a signed type, or a read past an argument block, aborts the run.  The
 * driver also checks the documented outcome of the hand-built cases.
 *
 * Test infrastructure: tests/test_host_sanitizers.py builds and runs it.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "specverify.h"

static uint64_t rng_state = 0xD1B54A32D192ED03ull;
static uint32_t rnd(void) {
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return (uint32_t)((rng_state * 0x2545F4914F6CDD1Dull) >> 32);
}

static int failures = 0;
#define CHECK(c)                                                      \
  do {                                                                \
    if (!(c)) {                                                       \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
      ++failures;                                                     \
    }                                                                 \
  } while (0)

/* Stand-ins for device buffers: the checks compare and align them but never
 * dereference them. */
#define FAKE(off) ((void*)(uintptr_t)(0x100000u + (off)))

static int32_t extreme_i32(void) {
  static const int32_t v[] = {INT32_MIN, -65536, -2, -1, 0, 1, 2, 7, 8, 31, 32, 33,
                              65535, 65536, 1 << 21, (1 << 21) + 1, 1 << 30,
                              (1 << 30) + 1, INT32_MAX};
  return (rnd() & 3) ? v[rnd() % (sizeof v / sizeof v[0])] : (int32_t)rnd();
}
static int64_t extreme_i64(void) {
  static const int64_t v[] = {INT64_MIN, -1, 0, 1, 7, 8, 151936, (int64_t)1 << 31,
                              (int64_t)1 << 40, INT64_MAX};
  return (rnd() & 3) ? v[rnd() % (sizeof v / sizeof v[0])] : (int64_t)rnd();
}
static void* extreme_ptr(void) {
  switch (rnd() % 4) {
    case 0: return NULL;
    case 1: return FAKE(1);  /* misaligned */
    case 2: return FAKE(4);
    default: return FAKE(4096);
  }
}
static size_t extreme_size(void) {
  static const size_t v[] = {0, 1, 255, 256, 4096, (size_t)1 << 32, SIZE_MAX};
  return v[rnd() % (sizeof v / sizeof v[0])];
}

static sv_verify_args good_verify(int32_t B, int32_t K, int32_t V, int dtype) {
  sv_verify_args a;
  memset(&a, 0, sizeof a);
  a.B = B;
  a.k_max = K;
  a.V = V;
  a.dtype = dtype;
  a.target_logits = FAKE(0);
  a.target_vec_stride = V;
  a.draft_logits = FAKE(0x10000000u);
  a.draft_vec_stride = V;
  a.draft_tokens = (const int32_t*)FAKE(0x20000000u);
  a.temperature = (const float*)FAKE(0x21000000u);
  a.out_tokens = (int32_t*)FAKE(0x22000000u);
  a.accepted = (int32_t*)FAKE(0x23000000u);
  a.workspace = FAKE(0x24000000u);
  a.workspace_bytes = sv_verify_workspace_bytes(B, K, V, dtype, 0);
  return a;
}

static sv_rollback_args good_rollback(int32_t B, int32_t K) {
  sv_rollback_args r;
  memset(&r, 0, sizeof r);
  r.B = B;
  r.k_max = K;
  r.page_size = 16;
  r.max_pages_per_seq = 64;
  r.kv_len = (int32_t*)FAKE(0x30000000u);
  r.accepted = (const int32_t*)FAKE(0x23000000u);
  r.page_table = (int32_t*)FAKE(0x31000000u);
  r.workspace = FAKE(0x32000000u);
  r.workspace_bytes = sv_rollback_workspace_bytes(B);
  return r;
}

static void mutate_verify(sv_verify_args* a) {
  switch (rnd() % 16) {
    case 0: a->B = extreme_i32(); break;
    case 1: a->k_max = extreme_i32(); break;
    case 2: a->V = extreme_i32(); break;
    case 3: a->dtype = extreme_i32(); break;
    case 4: a->target_vec_stride = extreme_i64(); break;
    case 5: a->draft_vec_stride = extreme_i64(); break;
    case 6: a->target_logits = extreme_ptr(); break;
    case 7: a->draft_logits = extreme_ptr(); break;
    case 8: a->draft_tokens = (const int32_t*)extreme_ptr(); break;
    case 9: a->temperature = (const float*)extreme_ptr(); break;
    case 10: a->offset_dev = (const uint64_t*)extreme_ptr(); break;
    case 11: a->flags = rnd(); break;
    case 12: a->out_tokens = (int32_t*)extreme_ptr(); break;
    case 13: a->accepted = (int32_t*)extreme_ptr(); break;
    case 14: a->workspace = extreme_ptr(); break;
    default: a->workspace_bytes = extreme_size(); break;
  }
}

static void mutate_rollback(sv_rollback_args* r) {
  switch (rnd() % 14) {
    case 0: r->B = extreme_i32(); break;
    case 1: r->k_max = extreme_i32(); break;
    case 2: r->page_size = extreme_i32(); break;
    case 3: r->max_pages_per_seq = extreme_i32(); break;
    case 4: r->num_pages = extreme_i32(); break;
    case 5: r->free_pages = (int32_t*)extreme_ptr(); break;
    case 6: r->free_top = (int32_t*)extreme_ptr(); break;
    case 7: r->free_capacity = extreme_i32(); break;
    case 8: r->kv_pool = extreme_ptr(); break;
    case 9: r->num_layers = extreme_i32(); r->kv_heads = extreme_i32(); break;
    case 10: r->head_dim = extreme_i32(); break;
    case 11: r->kv_len = (int32_t*)extreme_ptr(); break;
    case 12: r->workspace = extreme_ptr(); break;
    default: r->workspace_bytes = extreme_size(); break;
  }
}

static void verify_checks(void) {
  /* hand-built cases */
  sv_verify_args a = good_verify(256, 6, 151936, SV_BF16);
  for (int mode = 0; mode < 3; ++mode) CHECK(sv_check_verify_args(&a, mode) == SV_OK);
  sv_verify_args b = a;
  b.B = 0;
  CHECK(sv_check_verify_args(&b, 0) == SV_OK); /* an empty batch is valid */
  b = a;
  b.k_max = SV_MAX_K + 1;
  CHECK(sv_check_verify_args(&b, 0) == SV_E_ARG);
  b = a;
  b.target_vec_stride = b.V - 1;
  CHECK(sv_check_verify_args(&b, 0) == SV_E_ARG);
  b = a;
  b.dtype = 7;
  CHECK(sv_check_verify_args(&b, 0) == SV_E_DTYPE);
  b = a;
  b.workspace_bytes = 16;
  CHECK(sv_check_verify_args(&b, 0) == SV_E_WORKSPACE);
  b = a;
  b.offset_dev = (const uint64_t*)FAKE(4);
  CHECK(sv_check_verify_args(&b, 0) == SV_E_ARG);
  /* launching entry points check before touching the device */
  CHECK(sv_verify_sample(NULL, &a, NULL) == SV_E_ARG);
  CHECK(sv_verify_greedy(NULL, &a, NULL) == SV_E_ARG);
  CHECK(sv_draft_sample(NULL, &a, NULL) == SV_E_ARG);
  CHECK(sv_verify_sample_noalloc(NULL, &a, NULL) == SV_E_ARG);
  CHECK(sv_verify_greedy_one_launch(NULL, &a, FAKE(0x50000000u), sv_greedy_state_bytes(256, 6),
                                    NULL) == SV_E_ARG);
  CHECK(sv_verify_sample(NULL, NULL, NULL) == SV_E_ARG);

  /* sizes over the whole range, and random mutations of valid blocks */
  for (int it = 0; it < 20000; ++it) {
    (void)sv_verify_workspace_bytes(extreme_i32(), extreme_i32(), extreme_i32(),
                                    extreme_i32(), rnd());
    const int32_t B = 1 + (int32_t)(rnd() % 512), K = 1 + (int32_t)(rnd() % SV_MAX_K);
    const int32_t V = 1 + (int32_t)(rnd() % 200000);
    sv_verify_args m = good_verify(B, K, V, (int)(rnd() & 1));
    const int n = 1 + (int)(rnd() % 3);
    for (int j = 0; j < n; ++j) mutate_verify(&m);
    const int mode = (int)(rnd() % 4) - (rnd() % 8 == 0 ? 2 : 0);
    const sv_status s = sv_check_verify_args(&m, mode);
    CHECK(s >= SV_OK && s <= SV_E_INTERNAL);
    CHECK(sv_verify_sample(NULL, &m, NULL) != SV_OK);
    (void)sv_greedy_state_bytes(extreme_i32(), extreme_i32());
    CHECK(sv_verify_greedy_one_launch(NULL, &m, extreme_ptr(), extreme_size(), NULL) != SV_OK);
    sv_rollback_args r = good_rollback(B, K);
    r.accepted = m.accepted;
    if (rnd() & 1) mutate_rollback(&r);
    const sv_status t = sv_check_verify_rollback_args(&m, &r);
    CHECK(t >= SV_OK && t <= SV_E_INTERNAL);
    CHECK(sv_verify_sample_rollback(NULL, &m, &r, NULL) != SV_OK);
  }
  (void)sv_noalloc_scratch_bytes();
}

static void rollback_checks(void) {
  sv_rollback_args r = good_rollback(64, 8);
  CHECK(sv_check_rollback_args(&r) == SV_OK);
  sv_rollback_args q = r;
  q.kv_pool = FAKE(0x40000000u);
  CHECK(sv_check_rollback_args(&q) == SV_E_ARG); /* a pool needs its sizes */
  q = r;
  q.free_pages = (int32_t*)FAKE(0x41000000u);
  CHECK(sv_check_rollback_args(&q) == SV_E_ARG); /* a stack needs its height */
  q = r;
  q.workspace_bytes -= 1;
  CHECK(sv_check_rollback_args(&q) == SV_E_WORKSPACE);
  CHECK(sv_kv_rollback(NULL, &r, NULL) == SV_E_ARG);
  for (int it = 0; it < 20000; ++it) {
    (void)sv_rollback_workspace_bytes(extreme_i32());
    sv_rollback_args m = good_rollback(1 + (int32_t)(rnd() % 4096), 1 + (int32_t)(rnd() % 32));
    const int n = 1 + (int)(rnd() % 3);
    for (int j = 0; j < n; ++j) mutate_rollback(&m);
    const sv_status s = sv_check_rollback_args(&m);
    CHECK(s >= SV_OK && s <= SV_E_INTERNAL);
  }
}

static void dynk_checks(void) {
  sv_dynk_args d;
  memset(&d, 0, sizeof d);
  d.B = 512;
  d.window = 64;
  d.k_min = 2;
  d.k_max = 8;
  d.up_num = 17;
  d.up_den = 20;
  d.down_num = 7;
  d.down_den = 10;
  d.accepted = (const int32_t*)FAKE(0x50000000u);
  d.k_per_row = (int32_t*)FAKE(0x51000000u);
  d.state = (int32_t*)FAKE(0x52000000u);
  CHECK(sv_check_dynk_args(&d) == SV_OK);
  CHECK(sv_dynamic_k(NULL, &d, NULL) == SV_E_ARG);
  CHECK(sv_advance_offset(NULL, (uint64_t*)FAKE(8), 1, NULL) == SV_E_ARG);
  CHECK(sv_close_round(NULL, &d, (uint64_t*)FAKE(8), 1, NULL) == SV_E_ARG);
  for (int it = 0; it < 20000; ++it) {
    sv_dynk_args m = d;
    switch (rnd() % 9) {
      case 0: m.B = extreme_i32(); break;
      case 1: m.window = extreme_i32(); break;
      case 2: m.k_min = extreme_i32(); break;
      case 3: m.k_max = extreme_i32(); break;
      case 4: m.up_num = extreme_i32(); m.up_den = extreme_i32(); break;
      case 5: m.down_num = extreme_i32(); m.down_den = extreme_i32(); break;
      case 6: m.accepted = (const int32_t*)extreme_ptr(); break;
      case 7: m.k_per_row = (int32_t*)extreme_ptr(); break;
      default: m.state = (int32_t*)extreme_ptr(); break;
    }
    const sv_status s = sv_check_dynk_args(&m);
    CHECK(s >= SV_OK && s <= SV_E_INTERNAL);
    CHECK(sv_close_round(NULL, &m, (uint64_t*)extreme_ptr(), rnd(), NULL) != SV_OK);
  }
}

static sv_shard_stats_args good_shard(int32_t B, int32_t K, int32_t V, int32_t off,
                                      int32_t cnt) {
  sv_shard_stats_args a;
  memset(&a, 0, sizeof a);
  a.B = B;
  a.k_max = K;
  a.V = V;
  a.col_offset = off;
  a.col_count = cnt;
  a.target_shard = FAKE(0);
  a.target_vec_stride = cnt;
  a.draft_shard = FAKE(0x10000000u);
  a.draft_vec_stride = cnt;
  a.draft_tokens = (const int32_t*)FAKE(0x20000000u);
  a.partial = FAKE(0x60000000u);
  a.partial_bytes = sv_shard_partial_bytes(B, K, cnt);
  a.workspace = FAKE(0x61000000u);
  a.workspace_bytes = sv_shard_workspace_bytes(B, K);
  return a;
}

static void shard_checks(void) {
  const int32_t B = 256, K = 6, V = 151936, G = 8;
  sv_shard_stats_args s = good_shard(B, K, V, 0, V / G);
  CHECK(sv_check_shard_stats_args(&s) == SV_OK);
  CHECK(sv_shard_stats(NULL, &s, NULL) == SV_E_ARG);
  sv_shard_combine_args c;
  memset(&c, 0, sizeof c);
  c.B = B;
  c.k_max = K;
  c.V = V;
  c.G = G;
  for (int g = 0; g < G; ++g) {
    c.partials[g] = FAKE(0x60000000u + 0x1000000u * (unsigned)g);
    c.partial_bytes[g] = sv_shard_partial_bytes(B, K, V / G);
    c.col_offset[g] = g * (V / G);
    c.col_count[g] = V / G;
    c.target_shards[g] = FAKE(0);
    c.target_vec_stride[g] = V / G;
    c.draft_shards[g] = FAKE(0x10000000u);
    c.draft_vec_stride[g] = V / G;
  }
  c.draft_tokens = (const int32_t*)FAKE(0x20000000u);
  c.temperature = (const float*)FAKE(0x21000000u);
  c.workspace = FAKE(0x24000000u);
  c.workspace_bytes = sv_verify_workspace_bytes(B, K, V, SV_BF16, 0);
  CHECK(sv_check_shard_combine_args(&c) == SV_OK);
  CHECK(sv_shard_combine(NULL, &c, NULL) == SV_E_ARG);
  sv_shard_draw_args d;
  memset(&d, 0, sizeof d);
  d.B = B;
  d.k_max = K;
  d.V = V;
  d.col_offset = 0;
  d.col_count = V / G;
  d.G = G;
  d.shard = 0;
  d.target_shard = FAKE(0);
  d.target_vec_stride = V / G;
  d.draft_shard = FAKE(0x10000000u);
  d.draft_vec_stride = V / G;
  d.draft_tokens = (const int32_t*)FAKE(0x20000000u);
  d.temperature = (const float*)FAKE(0x21000000u);
  d.records = FAKE(0x24000000u);
  d.records_bytes = c.workspace_bytes;
  d.masses = (double*)FAKE(0x70000000u);
  d.masses_bytes = (size_t)G * B * 16;
  d.out_tokens = (int32_t*)FAKE(0x22000000u);
  d.accepted = (int32_t*)FAKE(0x23000000u);
  const sv_status ds = sv_check_shard_draw_args(&d);
  CHECK(ds == SV_OK);
  CHECK(sv_shard_draw_mass(NULL, &d, NULL) == SV_E_ARG);
  CHECK(sv_shard_draw_locate(NULL, &d, NULL) == SV_E_ARG);
  for (int it = 0; it < 20000; ++it) {
    (void)sv_shard_partial_bytes(extreme_i32(), extreme_i32(), extreme_i32());
    (void)sv_shard_workspace_bytes(extreme_i32(), extreme_i32());
    sv_shard_stats_args m = s;
    switch (rnd() % 10) {
      case 0: m.B = extreme_i32(); break;
      case 1: m.k_max = extreme_i32(); break;
      case 2: m.V = extreme_i32(); break;
      case 3: m.col_offset = extreme_i32(); break;
      case 4: m.col_count = extreme_i32(); break;
      case 5: m.mode = extreme_i32(); break;
      case 6: m.target_vec_stride = extreme_i64(); break;
      case 7: m.partial_bytes = extreme_size(); break;
      case 8: m.partial = extreme_ptr(); break;
      default: m.workspace_bytes = extreme_size(); break;
    }
    const sv_status t = sv_check_shard_stats_args(&m);
    CHECK(t >= SV_OK && t <= SV_E_INTERNAL);
    sv_shard_combine_args n = c;
    switch (rnd() % 8) {
      case 0: n.G = extreme_i32(); break;
      case 1: n.col_offset[rnd() % SV_MAX_SHARDS] = extreme_i32(); break;
      case 2: n.col_count[rnd() % SV_MAX_SHARDS] = extreme_i32(); break;
      case 3: n.partial_bytes[rnd() % SV_MAX_SHARDS] = extreme_size(); break;
      case 4: n.V = extreme_i32(); break;
      case 5: n.mode = extreme_i32(); break;
      case 6: n.target_vec_stride[rnd() % SV_MAX_SHARDS] = extreme_i64(); break;
      default: n.workspace_bytes = extreme_size(); break;
    }
    const sv_status u = sv_check_shard_combine_args(&n);
    CHECK(u >= SV_OK && u <= SV_E_INTERNAL);
    sv_shard_draw_args e = d;
    switch (rnd() % 8) {
      case 0: e.G = extreme_i32(); break;
      case 1: e.shard = extreme_i32(); break;
      case 2: e.col_offset = extreme_i32(); break;
      case 3: e.col_count = extreme_i32(); break;
      case 4: e.masses_bytes = extreme_size(); break;
      case 5: e.records_bytes = extreme_size(); break;
      case 6: e.offset_dev = (const uint64_t*)extreme_ptr(); break;
      default: e.V = extreme_i32(); break;
    }
    const sv_status w = sv_check_shard_draw_args(&e);
    CHECK(w >= SV_OK && w <= SV_E_INTERNAL);
  }
}

int main(void) {
  for (int s = -2; s < 8; ++s) CHECK(sv_status_string((sv_status)s) != NULL);
  verify_checks();
  rollback_checks();
  dynk_checks();
  shard_checks();
  /* no handle, no timing */
  CHECK(sv_timing_enable(NULL, 1) == SV_E_ARG);
  CHECK(sv_destroy(NULL) == SV_E_ARG || sv_destroy(NULL) == SV_OK);
  if (failures) {
    fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  printf("host checks ok\n");
  return 0;
}
