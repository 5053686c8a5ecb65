// Internal definitions shared by the host library and the HIP kernels of
// specverify.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/specverify.h"

namespace sv {

// log2(e) / T, the factor that turns (z - m) into an exp2 argument, as fp32.
// A positive T so small that the factor overflows fp32 is given the largest
// finite float instead: (m - m) * c2 stays 0 (weight 1 for the maximum) and
// every smaller logit still gets weight 0, as in exact arithmetic.
__device__ __forceinline__ float log2e_over_T(float T) {
  const double c = 1.4426950408889634 / (double)T;
  return c < 3.4028234663852886e38 ? (float)c : 3.4028234663852886e38f;
}

// Per-vector statistics written by the stats kernels and read by the
// finalize kernel.  One record per (row, side, position) slot.
struct VecRec {
  float m;          // largest finite raw logit of the vector
  float tau;        // smallest kept raw logit (-inf when nothing is cut)
  double inv_kept;  // 1 / sum over kept j of exp((z_j - m) / T)
  double px;        // p'(x) (or q'(x)) of the vector's draft token, 0 if none
  uint32_t status;  // SV_ROW_* bits found in this vector
  uint32_t pad;
};
static_assert(sizeof(VecRec) == 32, "VecRec layout");

// Greedy argmax partial of one chunk of one vector.
struct ArgmaxPart {
  float value;
  int32_t index;    // -1 if the chunk held no comparable value
  uint32_t status;  // NONFINITE bit; bit 31 set if any finite entry was seen
  uint32_t pad;
};
static_assert(sizeof(ArgmaxPart) == 16, "ArgmaxPart layout");
constexpr uint32_t kSawFinite = 1u << 31;

// Rollback decision per row, used when the pool is poisoned.
struct RollRec {
  int32_t status;   // row status; 0 = the row is rolled back
  int32_t new_len;
  int32_t old_len;
  int32_t aux;      // pages released (after the check), then the index on
                    // the free stack of the row's first release (after the scan)
};
static_assert(sizeof(RollRec) == 16, "RollRec layout");

// Vector slots of one row: target positions 0..K, then draft positions 0..K-1.
inline __host__ __device__ int slots_per_row(int K) { return 2 * K + 1; }

// The one-launch greedy path's state: row counters, then the largest packed
// (order key, -index) of every vector, then every vector's flags, each
// entry on its own 128 or 64 bytes.
constexpr int kGreedyCntStride = 32;   // uint32 words per row counter
constexpr int kGreedyBestStride = 8;   // uint64 words per vector maximum
constexpr int kGreedyFlgStride = 16;   // uint32 words per vector's flags
inline size_t greedy_state_bytes(int B, int K) {  // for any draft-logits choice
  const size_t nvec = (size_t)B * (2 * (size_t)K + 1);
  return (size_t)B * kGreedyCntStride * 4 + nvec * (kGreedyBestStride * 8 + kGreedyFlgStride * 4);
}

// Greedy chunking of a vector over several workgroups.
constexpr int kGreedyChunk = 4096;
// (V >= 0; written so that it cannot overflow for any such V)
inline __host__ __device__ int greedy_chunks(int V) {
  return V / kGreedyChunk + (V % kGreedyChunk != 0 ? 1 : 0);
}

struct StatsParams {
  const void* target;
  const void* draft;
  int64_t t_stride, d_stride;
  const int32_t* tokens;
  const int32_t* k_per_row;
  const float* temperature;
  const float* top_p;
  int32_t B, K, V;
  uint32_t flags;
  int32_t mode;  // 0 verification (all slots), 1 draft sampling (draft slots only)
  VecRec* recs;
  uint32_t* tickets;     // queue counters of the bf16 kernel (workspace, after the records)
  int32_t* slot_count;   // with slot_list: the number of listed slots
  int32_t* slot_list;    // the slots the call uses, in order, when some rows
                         // use fewer than all of theirs (k_per_row given, or
                         // draft sampling); NULL: every slot, slot = item
  // vocabulary shard pass only (V is then the shard's column count): the
  // shard's first column, and where its per-vector partials go
  int32_t col_off;
  uint8_t* partial;
  int64_t part_stride;   // bytes per vector slot
};

// ---- vocabulary shards
// One vector's partial statistics from one shard of the vocabulary: exact
// value counts of the shard's logits, as a list of the nonzero words of the
// count table (window of magnitudes [2^-24, 2^16), 40 exponent rows x 128
// mantissas; a word holds the count of +v in its low half and of -v in its
// high half), the zeros and -infs, the nonzero values below the window, and
// the draft token's logit when the token is one of the shard's columns.
// Layout per vector slot: ShardHead, then kShardTinyCap tiny values (raw
// bf16 bits), then the list of (word, counts) pairs.
constexpr int kTableWords = 40 * 128;
constexpr int kShardTinyCap = 64;
constexpr uint32_t kShardFallback = 1u << 30;  // the count table cannot hold the shard's values
struct ShardHead {
  uint32_t status;   // SV_ROW_NONFINITE_LOGIT | kShardFallback
  int32_t maxpos;    // largest word with a +count, -1 if none
  int32_t minneg;    // smallest word with a -count, 0x7FFFFFFF if none
  uint32_t zeros, ninf;
  uint32_t ntiny;    // nonzero values below the window (more than the cap: fallback)
  uint32_t nlist;    // entries of the list
  uint32_t zx;       // bit 16: the draft token is a column of this shard; low 16: its bits
};
static_assert(sizeof(ShardHead) == 32, "ShardHead layout");
constexpr size_t kShardListOffset = sizeof(ShardHead) + 4 * kShardTinyCap;  // 288
inline __host__ __device__ int shard_list_cap(int32_t cols) {
  return cols < kTableWords ? cols : kTableWords;
}
// bytes per vector slot, a multiple of 16 (the header is read as 16-byte words)
inline __host__ __device__ int64_t shard_part_stride(int32_t cols) {
  return ((int64_t)kShardListOffset + 8 * (int64_t)shard_list_cap(cols) + 15) / 16 * 16;
}
constexpr int kMaxShards = SV_MAX_SHARDS;

// The merge of all shards' partials into the records of the full vectors.
struct CombineParams {
  StatsParams sp;  // the call over the whole vocabulary (B, K, V, tokens, ..., recs)
  int32_t G;
  const uint8_t* part[kMaxShards];
  int64_t part_stride[kMaxShards];
  int32_t col_off[kMaxShards], col_len[kMaxShards];
  // the shards' logits, read only for a vector the count table cannot hold
  const uint16_t* tgt[kMaxShards];
  const uint16_t* dft[kMaxShards];
  int64_t ts[kMaxShards], ds[kMaxShards];
};

// Bytes of workspace the bf16 stats kernel keeps its queue counters, slot
// count and slot list in (after the records).
size_t stats_plan_bytes(int32_t B, int32_t K);
size_t stats_ticket_bytes();

struct FinalizeParams {
  const void* target;
  const void* draft;
  int64_t t_stride, d_stride;
  const int32_t* tokens;
  const int32_t* k_per_row;
  const float* temperature;
  const float* top_p;
  int32_t B, K, V, dtype;
  uint32_t flags;
  uint64_t seed, offset;
  const uint64_t* offset_dev;  // when non-null, the round counter is read here
  const VecRec* recs;
  int32_t* out_tokens;
  int32_t* accepted;
  int32_t* num_emitted;
  float* p_at_draft;
  float* q_at_draft;
  int32_t* row_status;
  int32_t* draft_out;  // draft sampling mode: tokens written here
  // verification with the rollback of a cache that has no free stack and
  // no pool (kv_len non-null): each row also moves its own KV length back
  int32_t* kv_len;
  const int32_t* page_table;
  int32_t ps, MP, num_pages;
  int32_t* roll_status;
  // with a free stack or a pool, the rows' releases are placed by a scan over
  // all rows: each row then only writes its decision here (roll_recs
  // non-null), and the rollback's scan kernels commit; free_stack: entries
  // past the length must be unmapped
  RollRec* roll_recs;
  int32_t free_stack;
};

struct GreedyParams {
  const void* target;
  const void* draft;  // may be null
  int64_t t_stride, d_stride;
  const int32_t* tokens;
  const int32_t* k_per_row;
  int32_t B, K, V, dtype;
  ArgmaxPart* parts;
  void* state;  // NULL: two launches; else the one-launch path's zeroed state
  int32_t* out_tokens;
  int32_t* accepted;
  int32_t* num_emitted;
  int32_t* row_status;
};

struct RollbackParams {
  int32_t B, K, ps, MP;
  int32_t* kv_len;
  const int32_t* k_per_row;
  const int32_t* accepted;
  int32_t* page_table;
  int32_t num_pages;
  int32_t* free_pages;
  int32_t* free_top;
  int32_t free_capacity;
  uint16_t* kv_pool;
  int32_t L, H, D;
  int32_t* row_status;
  RollRec* recs;
  // per-row counters (kRollCntStride words apart) through which the last of
  // a row's poisoning workgroups commits the row
  uint32_t* row_cnt;
};
constexpr int kRollCntStride = 16;

// One shard's part of the draw: its columns of every vector, and the
// exchange buffer of all shards' per-row masses.
struct ShardDrawParams {
  const void* tgt;
  const void* dft;
  int64_t ts, ds;
  int32_t col_off, col_len, G, shard;
  double* masses;  // [G][B][2]: residual mass, p' mass of the drawn position
};

struct DynkParams {
  int32_t B, W, k_min, k_max, up_num, up_den, down_num, down_den;
  const int32_t* accepted;
  int32_t* k_per_row;
  int32_t* state;
  uint64_t* offset_dev;  // NULL, or the round counter to advance by offset_delta
  uint64_t offset_delta;
};

// Optional event bracketing of each launch (see sv_timing_enable).
class Timer {
 public:
  virtual ~Timer() {}
  virtual void begin(const char* name, hipStream_t s) = 0;
  virtual void end(hipStream_t s) = 0;
  // An unrecorded event pair for a launch that records them itself
  // (hipExtLaunchKernelGGL: the events then bound the kernel's execution,
  // not the launch); false if none is left.
  virtual bool pair(const char* name, hipEvent_t* start, hipEvent_t* stop) = 0;
};

struct TimedScope {
  Timer* t;
  hipStream_t s;
  TimedScope(Timer* t_, const char* name, hipStream_t s_) : t(t_), s(s_) {
    if (t) t->begin(name, s);
  }
  ~TimedScope() {
    if (t) t->end(s);
  }
};

// Launchers (each returns hipGetLastError() of its launch(es)).
hipError_t launch_stats(const StatsParams& p, int dtype, int num_cus, hipStream_t s, Timer* t);
hipError_t launch_shard_stats(const StatsParams& p, int num_cus, hipStream_t s, Timer* t);
hipError_t launch_shard_combine(const CombineParams& p, hipStream_t s, Timer* t);
hipError_t launch_finalize_sample(const FinalizeParams& p, int num_cus, hipStream_t s, Timer* t);
hipError_t launch_draft_sample(const FinalizeParams& p, int num_cus, hipStream_t s, Timer* t);
hipError_t launch_shard_draw(const FinalizeParams& p, const ShardDrawParams& d, bool locate,
                             int num_cus, hipStream_t s, Timer* t);
hipError_t launch_greedy(const GreedyParams& p, int num_cus, hipStream_t s, Timer* t);
hipError_t launch_rollback(const RollbackParams& p, hipStream_t s, Timer* t);
// The rollback's scan and commit (with a KV pool: the scan, then the
// poisoning, which commits) on decisions already in p.recs (written by the
// verification's finalize kernel).
hipError_t launch_rollback_decided(const RollbackParams& p, hipStream_t s, Timer* t);
hipError_t launch_dynk(const DynkParams& p, hipStream_t s, Timer* t);
hipError_t launch_advance_offset(uint64_t* offset_dev, uint64_t delta, hipStream_t s, Timer* t);

}  // namespace sv
