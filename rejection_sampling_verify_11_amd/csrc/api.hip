// Host side of the specverify C ABI: argument validation, workspace sizing
// and kernel launches on the caller's stream.  No device memory is
// allocated, no stream is synchronised and nothing is copied back.
#include <new>
#include <string.h>
#include <vector>

#include "sv_internal.h"

namespace {

// Event pairs around kernel launches, read back on request.
class EventTimer final : public sv::Timer {
 public:
  static constexpr size_t kMax = 4096;
  ~EventTimer() override {
    for (auto& e : pool_) {
      (void)hipEventDestroy(e.first);
      (void)hipEventDestroy(e.second);
    }
  }
  void begin(const char* name, hipStream_t s) override {
    cur_ = take(name);
    if (cur_ >= 0) (void)hipEventRecord(pool_[cur_].first, s);
  }
  bool pair(const char* name, hipEvent_t* start, hipEvent_t* stop) override {
    const long i = take(name);
    cur_ = -1;
    if (i < 0) return false;
    *start = pool_[i].first;
    *stop = pool_[i].second;
    return true;
  }
  void end(hipStream_t s) override {
    if (cur_ >= 0) (void)hipEventRecord(pool_[cur_].second, s);
    cur_ = -1;
  }
  int read(int max_entries, const char** names, int32_t* launches, double* total_ms) {
    std::vector<const char*> un;
    std::vector<int32_t> cnt;
    std::vector<double> ms;
    for (size_t i = 0; i < used_; ++i) {
      float t = 0.f;
      (void)hipEventSynchronize(pool_[i].second);
      if (hipEventElapsedTime(&t, pool_[i].first, pool_[i].second) != hipSuccess) t = 0.f;
      size_t k = 0;
      while (k < un.size() && strcmp(un[k], names_[i]) != 0) ++k;
      if (k == un.size()) { un.push_back(names_[i]); cnt.push_back(0); ms.push_back(0.0); }
      cnt[k] += 1;
      ms[k] += t;
    }
    used_ = 0;
    for (size_t k = 0; k < un.size() && (int)k < max_entries; ++k) {
      if (names) names[k] = un[k];
      if (launches) launches[k] = cnt[k];
      if (total_ms) total_ms[k] = ms[k];
    }
    return (int)un.size();
  }

 private:
  // the next entry's index (its events created on first use), -1 if full
  long take(const char* name) {
    if (used_ >= kMax) return -1;
    if (used_ == pool_.size()) {
      hipEvent_t a, b;
      if (hipEventCreate(&a) != hipSuccess) return -1;
      if (hipEventCreate(&b) != hipSuccess) { (void)hipEventDestroy(a); return -1; }
      pool_.push_back({a, b});
    }
    const long i = (long)used_++;
    names_.resize(used_);
    names_[i] = name;
    return i;
  }
  std::vector<std::pair<hipEvent_t, hipEvent_t>> pool_;
  std::vector<const char*> names_;
  size_t used_ = 0;
  long cur_ = -1;
};

}  // namespace

// Device memory of sv_verify_sample_noalloc: the records and work-queue
// counters that sv_verify_sample keeps in the caller's workspace.  Every GPU
// the library runs on holds its own copy for the life of the process.  In
// host code `scratch` names a host-side stand-in, never the device memory:
// the device address is looked up once per device (sv_create) and only that
// address is handed to kernels.
constexpr size_t kNoAllocScratchBytes = (size_t)4 << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

struct sv_handle_s {
  int device;
  int num_cus;
  char arch[64];
  bool timing;
  EventTimer* timer;
  void* scratch_dev;  // this device's copy of `scratch`, or NULL if the lookup failed
  sv::Timer* active() { return timing ? timer : nullptr; }
};

namespace {

constexpr int32_t kMaxVSampled = SV_MAX_V_SAMPLED;  // inverse-CDF segment table bound

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Per-vector records, then the queue counters, slot count and slot list of
// the bf16 stats kernel.
size_t recs_bytes(int32_t B, int32_t K) {
  return align_up((size_t)B * sv::slots_per_row(K) * sizeof(sv::VecRec), 256);
}

size_t sample_ws(int32_t B, int32_t K) {
  return recs_bytes(B, K) + sv::stats_plan_bytes(B, K);
}

size_t greedy_ws(int32_t B, int32_t K, int32_t V) {
  return align_up((size_t)B * (2 * (size_t)K + 1) * sv::greedy_chunks(V) * sizeof(sv::ArgmaxPart), 256);
}

// The controller update of every row, and the round counter advanced in the
// same launch when offset_dev is given.
sv_status dynk_launch(sv_handle h, const sv_dynk_args* a, uint64_t* offset_dev, uint64_t delta,
                      hipStream_t s) {
  sv::DynkParams p;
  p.B = a->B;
  p.W = a->window;
  p.k_min = a->k_min;
  p.k_max = a->k_max;
  p.up_num = a->up_num;
  p.up_den = a->up_den;
  p.down_num = a->down_num;
  p.down_den = a->down_den;
  p.accepted = a->accepted;
  p.k_per_row = a->k_per_row;
  p.state = a->state;
  p.offset_dev = offset_dev;
  p.offset_delta = delta;
  if (sv::launch_dynk(p, s, h->active()) != hipSuccess) return SV_E_DEVICE;
  return SV_OK;
}

}  // namespace

extern "C" {

const char* sv_status_string(sv_status s) {
  // a C caller may pass any int: read the argument's bits, not an enum value
  // the C++ type cannot hold
  static_assert(sizeof(sv_status) == sizeof(int), "sv_status is an int");
  int v;
  memcpy(&v, &s, sizeof v);
  switch (v) {
    case SV_OK: return "ok";
    case SV_E_ARG: return "invalid argument";
    case SV_E_DTYPE: return "unsupported dtype";
    case SV_E_WORKSPACE: return "workspace missing or too small";
    case SV_E_DEVICE: return "HIP device or launch error";
    case SV_E_INTERNAL: return "internal error";
  }
  return "unknown status";
}

sv_status sv_create(int hip_device, sv_handle* out) {
  if (!out) return SV_E_ARG;
  *out = nullptr;
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess || hip_device < 0 || hip_device >= n) return SV_E_DEVICE;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, hip_device) != hipSuccess) return SV_E_DEVICE;
  sv_handle h = new (std::nothrow) sv_handle_s;
  if (!h) return SV_E_INTERNAL;
  h->device = hip_device;
  h->timing = false;
  h->timer = nullptr;
  h->num_cus = prop.multiProcessorCount;
  strncpy(h->arch, prop.gcnArchName, sizeof(h->arch) - 1);
  h->arch[sizeof(h->arch) - 1] = 0;
  // the device address of this device's scratch array, with the device current
  h->scratch_dev = nullptr;
  int prev = -1;
  if (hipGetDevice(&prev) == hipSuccess && hipSetDevice(hip_device) == hipSuccess) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) == hipSuccess) h->scratch_dev = ptr;
    (void)hipSetDevice(prev);
  }
  (void)hipGetLastError();  // a failed lookup only disables sv_verify_sample_noalloc
  *out = h;
  return SV_OK;
}

sv_status sv_destroy(sv_handle h) {
  if (h) delete h->timer;
  delete h;
  return SV_OK;
}

sv_status sv_timing_enable(sv_handle h, int on) {
  if (!h) return SV_E_ARG;
  if (on && !h->timer) {
    h->timer = new (std::nothrow) EventTimer();
    if (!h->timer) return SV_E_INTERNAL;
  }
  h->timing = on != 0;
  return SV_OK;
}

int sv_timing_read(sv_handle h, int max_entries, const char** names, int32_t* launches,
                   double* total_ms) {
  if (!h || !h->timer) return 0;
  return h->timer->read(max_entries, names, launches, total_ms);
}

size_t sv_verify_workspace_bytes(int32_t B, int32_t k_max, int32_t V, int32_t dtype,
                                 uint32_t flags) {
  (void)dtype;
  (void)flags;
  if (B < 0 || k_max < 1 || k_max > SV_MAX_K || V < 1) return 0;
  const size_t a = sample_ws(B, k_max), g = greedy_ws(B, k_max, V);
  const size_t n = a > g ? a : g;
  return n > 0 ? n : 256;
}

sv_status sv_check_verify_args(const sv_verify_args* a, int mode) {
  if (!a || mode < 0 || mode > 2) return SV_E_ARG;
  if (a->B < 0 || a->k_max < 1 || a->k_max > SV_MAX_K || a->V < 1 || a->V > SV_MAX_V)
    return SV_E_ARG;
  if (a->dtype != SV_FP32 && a->dtype != SV_BF16) return SV_E_DTYPE;
  if ((int64_t)a->B * (2 * a->k_max + 1) * sv::greedy_chunks(a->V) > 0x7FFFFFFFLL) return SV_E_ARG;
  if (a->B == 0) return SV_OK;
  if (mode != 1 && a->V > kMaxVSampled) return SV_E_ARG;
  if ((uintptr_t)a->offset_dev & 7) return SV_E_ARG;
  if (mode == 0) {
    if (!a->target_logits || !a->draft_logits || !a->draft_tokens || !a->temperature ||
        !a->out_tokens || !a->accepted)
      return SV_E_ARG;
    if (a->target_vec_stride < a->V || a->draft_vec_stride < a->V) return SV_E_ARG;
  } else if (mode == 1) {
    if (!a->target_logits || !a->out_tokens || !a->accepted) return SV_E_ARG;
    if (!a->draft_logits && !a->draft_tokens) return SV_E_ARG;
    if (a->target_vec_stride < a->V) return SV_E_ARG;
    if (a->draft_logits && a->draft_vec_stride < a->V) return SV_E_ARG;
  } else {
    if (!a->draft_logits || !a->draft_tokens || !a->temperature) return SV_E_ARG;
    if (a->draft_vec_stride < a->V) return SV_E_ARG;
  }
  const size_t need = mode == 1 ? greedy_ws(a->B, a->k_max, a->V) : sample_ws(a->B, a->k_max);
  if (!a->workspace || a->workspace_bytes < need) return SV_E_WORKSPACE;
  return SV_OK;
}

static sv::StatsParams stats_params(const sv_verify_args* a, int mode) {
  sv::StatsParams p;
  p.target = a->target_logits;
  p.draft = a->draft_logits;
  p.t_stride = a->target_vec_stride;
  p.d_stride = a->draft_vec_stride;
  p.tokens = a->draft_tokens;
  p.k_per_row = a->k_per_row;
  p.temperature = a->temperature;
  p.top_p = a->top_p;
  p.B = a->B;
  p.K = a->k_max;
  p.V = a->V;
  p.flags = a->flags;
  p.mode = mode;
  p.recs = (sv::VecRec*)a->workspace;
  char* plan = (char*)a->workspace + recs_bytes(a->B, a->k_max);
  p.tickets = (uint32_t*)plan;
  p.slot_count = (int32_t*)(plan + align_up(sv::stats_ticket_bytes(), 256));
  // a list of the slots in use when rows differ in k; draft sampling with
  // one k maps its items to the draft slots arithmetically
  const bool listed = a->k_per_row != nullptr;
  p.slot_list = listed ? p.slot_count + 64 : nullptr;
  p.col_off = 0;
  p.partial = nullptr;
  p.part_stride = 0;
  return p;
}

static sv::FinalizeParams finalize_params(const sv_verify_args* a) {
  sv::FinalizeParams f;
  f.target = a->target_logits;
  f.draft = a->draft_logits;
  f.t_stride = a->target_vec_stride;
  f.d_stride = a->draft_vec_stride;
  f.tokens = a->draft_tokens;
  f.k_per_row = a->k_per_row;
  f.temperature = a->temperature;
  f.top_p = a->top_p;
  f.B = a->B;
  f.K = a->k_max;
  f.V = a->V;
  f.dtype = a->dtype;
  f.flags = a->flags;
  f.seed = a->seed;
  f.offset = a->offset;
  f.offset_dev = a->offset_dev;
  f.recs = (const sv::VecRec*)a->workspace;
  f.out_tokens = a->out_tokens;
  f.accepted = a->accepted;
  f.num_emitted = a->num_emitted;
  f.p_at_draft = a->p_at_draft;
  f.q_at_draft = a->q_at_draft;
  f.row_status = a->row_status;
  f.draft_out = const_cast<int32_t*>(a->draft_tokens);
  f.kv_len = nullptr;
  f.page_table = nullptr;
  f.ps = f.MP = f.num_pages = 0;
  f.roll_status = nullptr;
  f.roll_recs = nullptr;
  f.free_stack = 0;
  return f;
}

sv_status sv_verify_sample(sv_handle h, const sv_verify_args* a, hipStream_t s) {
  const sv_status st = sv_check_verify_args(a, 0);
  if (st != SV_OK) return st;
  if (!h) return SV_E_ARG;
  if (a->B == 0) return SV_OK;
  if (!(a->flags & SV_FLAG_RECORDS_READY) &&
      sv::launch_stats(stats_params(a, 0), a->dtype, h->num_cus, s, h->active()) != hipSuccess)
    return SV_E_DEVICE;
  if (sv::launch_finalize_sample(finalize_params(a), h->num_cus, s, h->active()) != hipSuccess)
    return SV_E_DEVICE;
  return SV_OK;
}

size_t sv_noalloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

sv_status sv_verify_sample_noalloc(sv_handle h, const sv_verify_args* a, hipStream_t s) {
  if (!a) return SV_E_ARG;
  sv_verify_args w = *a;
  w.workspace = nullptr;
  w.workspace_bytes = 0;
  // argument errors first (the missing workspace is this call's to supply)
  const sv_status st = sv_check_verify_args(&w, 0);
  if (st != SV_OK && st != SV_E_WORKSPACE) return st;
  if (w.flags & SV_FLAG_RECORDS_READY) return SV_E_ARG;  // records sit in a caller's workspace
  if (!h) return SV_E_ARG;
  if (w.B == 0) return SV_OK;
  if (sample_ws(w.B, w.k_max) > kNoAllocScratchBytes) return SV_E_WORKSPACE;
  if (!h->scratch_dev) return SV_E_DEVICE;
  w.workspace = h->scratch_dev;
  w.workspace_bytes = kNoAllocScratchBytes;
  return sv_verify_sample(h, &w, s);
}

sv_status sv_draft_sample(sv_handle h, const sv_verify_args* a, hipStream_t s) {
  const sv_status st = sv_check_verify_args(a, 2);
  if (st != SV_OK) return st;
  if (!h) return SV_E_ARG;
  if (a->B == 0) return SV_OK;
  if (!(a->flags & SV_FLAG_RECORDS_READY) &&
      sv::launch_stats(stats_params(a, 1), a->dtype, h->num_cus, s, h->active()) != hipSuccess)
    return SV_E_DEVICE;
  if (sv::launch_draft_sample(finalize_params(a), h->num_cus, s, h->active()) != hipSuccess)
    return SV_E_DEVICE;
  return SV_OK;
}

namespace {
sv_status greedy_launch(sv_handle h, const sv_verify_args* a, void* state, hipStream_t s) {
  sv::GreedyParams g;
  g.target = a->target_logits;
  g.draft = a->draft_logits;
  g.t_stride = a->target_vec_stride;
  g.d_stride = a->draft_vec_stride;
  g.tokens = a->draft_tokens;
  g.k_per_row = a->k_per_row;
  g.B = a->B;
  g.K = a->k_max;
  g.V = a->V;
  g.dtype = a->dtype;
  g.parts = (sv::ArgmaxPart*)a->workspace;
  g.state = state;
  g.out_tokens = a->out_tokens;
  g.accepted = a->accepted;
  g.num_emitted = a->num_emitted;
  g.row_status = a->row_status;
  if (sv::launch_greedy(g, h->num_cus, s, h->active()) != hipSuccess) return SV_E_DEVICE;
  return SV_OK;
}
}  // namespace

sv_status sv_verify_greedy(sv_handle h, const sv_verify_args* a, hipStream_t s) {
  const sv_status st = sv_check_verify_args(a, 1);
  if (st != SV_OK) return st;
  if (!h) return SV_E_ARG;
  if (a->B == 0) return SV_OK;
  return greedy_launch(h, a, nullptr, s);
}

size_t sv_greedy_state_bytes(int32_t B, int32_t k_max) {
  if (B < 0 || k_max < 1 || k_max > SV_MAX_K) return 0;
  const size_t n = align_up(sv::greedy_state_bytes(B, k_max), 256);
  return n > 0 ? n : 256;
}

sv_status sv_verify_greedy_one_launch(sv_handle h, const sv_verify_args* a, void* state,
                                      size_t state_bytes, hipStream_t s) {
  const sv_status st = sv_check_verify_args(a, 1);
  if (st != SV_OK) return st;
  if (!h) return SV_E_ARG;
  if (!state || ((uintptr_t)state & 7) || state_bytes < sv_greedy_state_bytes(a->B, a->k_max))
    return SV_E_WORKSPACE;
  if (a->B == 0) return SV_OK;
  return greedy_launch(h, a, state, s);
}

// the rows' decisions, then the per-row counters of the commit by the
// poisoning
static size_t rollback_recs_bytes(int32_t B) {
  return align_up((size_t)B * sizeof(sv::RollRec), 256);
}

size_t sv_rollback_workspace_bytes(int32_t B) {
  if (B < 0) return 0;
  const size_t n = rollback_recs_bytes(B) +
                   align_up((size_t)B * sv::kRollCntStride * sizeof(uint32_t), 256);
  return n > 0 ? n : 256;
}

sv_status sv_check_rollback_args(const sv_rollback_args* a) {
  if (!a) return SV_E_ARG;
  if (a->B < 0 || a->k_max < 1 || a->k_max > SV_MAX_K || a->page_size < 1 ||
      a->max_pages_per_seq < 1 || a->num_pages < 0)
    return SV_E_ARG;
  if ((int64_t)a->page_size * a->max_pages_per_seq > 0x7FFFFFFFLL) return SV_E_ARG;
  if (a->B == 0) return SV_OK;
  if (!a->kv_len || !a->accepted || !a->page_table) return SV_E_ARG;
  if (a->free_pages && (!a->free_top || a->free_capacity < 0)) return SV_E_ARG;
  if (a->kv_pool &&
      (a->num_pages < 1 || a->num_layers < 1 || a->kv_heads < 1 || a->head_dim < 1))
    return SV_E_ARG;
  if (!a->workspace || a->workspace_bytes < sv_rollback_workspace_bytes(a->B)) return SV_E_WORKSPACE;
  return SV_OK;
}

static sv::RollbackParams rollback_params(const sv_rollback_args* a) {
  sv::RollbackParams p;
  p.B = a->B;
  p.K = a->k_max;
  p.ps = a->page_size;
  p.MP = a->max_pages_per_seq;
  p.kv_len = a->kv_len;
  p.k_per_row = a->k_per_row;
  p.accepted = a->accepted;
  p.page_table = a->page_table;
  p.num_pages = a->num_pages;
  p.free_pages = a->free_pages;
  p.free_top = a->free_top;
  p.free_capacity = a->free_capacity;
  p.kv_pool = (uint16_t*)a->kv_pool;
  p.L = a->num_layers;
  p.H = a->kv_heads;
  p.D = a->head_dim;
  p.row_status = a->row_status;
  p.recs = (sv::RollRec*)a->workspace;
  p.row_cnt = (uint32_t*)((char*)a->workspace + rollback_recs_bytes(a->B));
  return p;
}

sv_status sv_kv_rollback(sv_handle h, const sv_rollback_args* a, hipStream_t s) {
  const sv_status st = sv_check_rollback_args(a);
  if (st != SV_OK) return st;
  if (!h) return SV_E_ARG;
  if (a->B == 0) return SV_OK;
  if (sv::launch_rollback(rollback_params(a), s, h->active()) != hipSuccess) return SV_E_DEVICE;
  return SV_OK;
}

sv_status sv_check_verify_rollback_args(const sv_verify_args* v, const sv_rollback_args* r) {
  sv_status st = sv_check_verify_args(v, 0);
  if (st != SV_OK) return st;
  st = sv_check_rollback_args(r);
  if (st != SV_OK) return st;
  if (r->B != v->B || r->k_max != v->k_max || r->k_per_row != v->k_per_row) return SV_E_ARG;
  if (v->B > 0 && r->accepted != v->accepted) return SV_E_ARG;
  return SV_OK;
}

sv_status sv_verify_sample_rollback(sv_handle h, const sv_verify_args* v,
                                    const sv_rollback_args* r, hipStream_t s) {
  const sv_status st = sv_check_verify_rollback_args(v, r);
  if (st != SV_OK) return st;
  if (!h) return SV_E_ARG;
  if (v->B == 0) return SV_OK;
  if (!(v->flags & SV_FLAG_RECORDS_READY) &&
      sv::launch_stats(stats_params(v, 0), v->dtype, h->num_cus, s, h->active()) != hipSuccess)
    return SV_E_DEVICE;
  sv::FinalizeParams f = finalize_params(v);
  f.kv_len = r->kv_len;
  f.page_table = r->page_table;
  f.ps = r->page_size;
  f.MP = r->max_pages_per_seq;
  f.num_pages = r->num_pages;
  // Without a free stack or pool each row commits its own rollback.  With
  // one, each row writes its decision, and a scan over all rows places the
  // releases on the stack (then poisons and commits).
  const bool scan = r->free_pages || r->kv_pool;
  f.roll_status = scan ? nullptr : r->row_status;
  f.roll_recs = scan ? (sv::RollRec*)r->workspace : nullptr;
  f.free_stack = r->free_pages ? 1 : 0;
  if (sv::launch_finalize_sample(f, h->num_cus, s, h->active()) != hipSuccess)
    return SV_E_DEVICE;
  if (scan && sv::launch_rollback_decided(rollback_params(r), s, h->active()) != hipSuccess)
    return SV_E_DEVICE;
  return SV_OK;
}

sv_status sv_check_dynk_args(const sv_dynk_args* a) {
  if (!a) return SV_E_ARG;
  if (a->B < 0 || a->window < 1 || a->window > 4096 || a->k_min < 1 || a->k_max < a->k_min ||
      a->k_max > SV_MAX_K || a->up_den <= 0 || a->down_den <= 0)
    return SV_E_ARG;
  if (a->B > 0 && (!a->accepted || !a->k_per_row || !a->state)) return SV_E_ARG;
  return SV_OK;
}


sv_status sv_dynamic_k(sv_handle h, const sv_dynk_args* a, hipStream_t s) {
  const sv_status st = sv_check_dynk_args(a);
  if (st != SV_OK) return st;
  if (!h) return SV_E_ARG;
  if (a->B == 0) return SV_OK;
  return dynk_launch(h, a, nullptr, 0, s);
}

sv_status sv_close_round(sv_handle h, const sv_dynk_args* a, uint64_t* offset_dev,
                         uint64_t delta, hipStream_t s) {
  const sv_status st = sv_check_dynk_args(a);
  if (st != SV_OK) return st;
  if (!h || !offset_dev || ((uintptr_t)offset_dev & 7)) return SV_E_ARG;
  return dynk_launch(h, a, offset_dev, delta, s);
}

sv_status sv_advance_offset(sv_handle h, uint64_t* offset_dev, uint64_t delta, hipStream_t s) {
  if (!h || !offset_dev || ((uintptr_t)offset_dev & 7)) return SV_E_ARG;
  if (sv::launch_advance_offset(offset_dev, delta, s, h->active()) != hipSuccess) return SV_E_DEVICE;
  return SV_OK;
}

}  // extern "C"

// ---------------------------------------------------------------- vocabulary shards

size_t sv_shard_partial_bytes(int32_t B, int32_t k_max, int32_t col_count) {
  if (B < 0 || k_max < 1 || k_max > SV_MAX_K || col_count < 1) return 0;
  const size_t n = (size_t)B * sv::slots_per_row(k_max) * (size_t)sv::shard_part_stride(col_count);
  return n > 0 ? n : 256;
}

size_t sv_shard_workspace_bytes(int32_t B, int32_t k_max) {
  if (B < 0 || k_max < 1 || k_max > SV_MAX_K) return 0;
  return sv::stats_plan_bytes(B, k_max);
}

sv_status sv_check_shard_stats_args(const sv_shard_stats_args* a) {
  if (!a) return SV_E_ARG;
  if (a->B < 0 || a->k_max < 1 || a->k_max > SV_MAX_K || a->V < 1 || a->V > kMaxVSampled)
    return SV_E_ARG;
  if (a->mode != 0 && a->mode != 1) return SV_E_ARG;
  if (a->col_offset < 0 || a->col_count < 1 || (int64_t)a->col_offset + a->col_count > a->V)
    return SV_E_ARG;
  if (a->B == 0) return SV_OK;
  if (!a->draft_shard || a->draft_vec_stride < a->col_count) return SV_E_ARG;
  if (a->mode == 0 &&
      (!a->target_shard || a->target_vec_stride < a->col_count || !a->draft_tokens))
    return SV_E_ARG;
  if (!a->partial || a->partial_bytes < sv_shard_partial_bytes(a->B, a->k_max, a->col_count))
    return SV_E_WORKSPACE;
  if (!a->workspace || a->workspace_bytes < sv_shard_workspace_bytes(a->B, a->k_max))
    return SV_E_WORKSPACE;
  return SV_OK;
}

sv_status sv_shard_stats(sv_handle h, const sv_shard_stats_args* a, hipStream_t s) {
  const sv_status st = sv_check_shard_stats_args(a);
  if (st != SV_OK) return st;
  if (!h) return SV_E_ARG;
  if (a->B == 0) return SV_OK;
  sv::StatsParams p;
  p.target = a->mode == 0 ? a->target_shard : a->draft_shard;
  p.draft = a->draft_shard;
  p.t_stride = a->mode == 0 ? a->target_vec_stride : a->draft_vec_stride;
  p.d_stride = a->draft_vec_stride;
  p.tokens = a->mode == 0 ? a->draft_tokens : nullptr;
  p.k_per_row = a->k_per_row;
  p.temperature = nullptr;  // the shard pass counts only
  p.top_p = nullptr;
  p.B = a->B;
  p.K = a->k_max;
  p.V = a->col_count;
  p.flags = 0;
  p.mode = a->mode;
  p.recs = nullptr;
  char* plan = (char*)a->workspace;
  p.tickets = (uint32_t*)plan;
  p.slot_count = (int32_t*)(plan + align_up(sv::stats_ticket_bytes(), 256));
  const bool listed = a->k_per_row != nullptr || a->mode == 1;
  p.slot_list = listed ? p.slot_count + 64 : nullptr;
  p.col_off = a->col_offset;
  p.partial = (uint8_t*)a->partial;
  p.part_stride = sv::shard_part_stride(a->col_count);
  if (sv::launch_shard_stats(p, h->num_cus, s, h->active()) != hipSuccess) return SV_E_DEVICE;
  return SV_OK;
}

sv_status sv_check_shard_combine_args(const sv_shard_combine_args* a) {
  if (!a) return SV_E_ARG;
  if (a->B < 0 || a->k_max < 1 || a->k_max > SV_MAX_K || a->V < 1 || a->V > kMaxVSampled)
    return SV_E_ARG;
  if (a->mode != 0 && a->mode != 1) return SV_E_ARG;
  if (a->G < 1 || a->G > SV_MAX_SHARDS) return SV_E_ARG;
  int64_t end = 0;
  for (int g = 0; g < a->G; ++g) {
    if (a->col_offset[g] != end || a->col_count[g] < 1) return SV_E_ARG;
    end += a->col_count[g];
  }
  if (end != a->V) return SV_E_ARG;
  if (a->B == 0) return SV_OK;
  for (int g = 0; g < a->G; ++g) {
    if (!a->partials[g] || !a->draft_shards[g] || a->draft_vec_stride[g] < a->col_count[g])
      return SV_E_ARG;
    if (a->mode == 0 && (!a->target_shards[g] || a->target_vec_stride[g] < a->col_count[g]))
      return SV_E_ARG;
    if (a->partial_bytes[g] < sv_shard_partial_bytes(a->B, a->k_max, a->col_count[g]))
      return SV_E_WORKSPACE;
  }
  if (!a->temperature || (a->mode == 0 && !a->draft_tokens)) return SV_E_ARG;
  if (!a->workspace || a->workspace_bytes < sample_ws(a->B, a->k_max)) return SV_E_WORKSPACE;
  return SV_OK;
}

sv_status sv_shard_combine(sv_handle h, const sv_shard_combine_args* a, hipStream_t s) {
  const sv_status st = sv_check_shard_combine_args(a);
  if (st != SV_OK) return st;
  if (!h) return SV_E_ARG;
  if (a->B == 0) return SV_OK;
  sv::CombineParams c;
  memset(&c, 0, sizeof(c));
  sv::StatsParams& p = c.sp;
  p.target = a->mode == 0 ? a->target_shards[0] : a->draft_shards[0];
  p.draft = a->draft_shards[0];
  p.t_stride = a->mode == 0 ? a->target_vec_stride[0] : a->draft_vec_stride[0];
  p.d_stride = a->draft_vec_stride[0];
  p.tokens = a->mode == 0 ? a->draft_tokens : nullptr;
  p.k_per_row = a->k_per_row;
  p.temperature = a->temperature;
  p.top_p = a->top_p;
  p.B = a->B;
  p.K = a->k_max;
  p.V = a->V;
  p.flags = a->flags;
  p.mode = a->mode;
  p.recs = (sv::VecRec*)a->workspace;
  p.tickets = nullptr;
  p.slot_count = nullptr;
  p.slot_list = nullptr;
  p.col_off = 0;
  p.partial = nullptr;
  p.part_stride = 0;
  c.G = a->G;
  for (int g = 0; g < a->G; ++g) {
    c.part[g] = (const uint8_t*)a->partials[g];
    c.part_stride[g] = sv::shard_part_stride(a->col_count[g]);
    c.col_off[g] = a->col_offset[g];
    c.col_len[g] = a->col_count[g];
    c.tgt[g] = (const uint16_t*)(a->mode == 0 ? a->target_shards[g] : a->draft_shards[g]);
    c.ts[g] = a->mode == 0 ? a->target_vec_stride[g] : a->draft_vec_stride[g];
    c.dft[g] = (const uint16_t*)a->draft_shards[g];
    c.ds[g] = a->draft_vec_stride[g];
  }
  if (sv::launch_shard_combine(c, s, h->active()) != hipSuccess) return SV_E_DEVICE;
  return SV_OK;
}

sv_status sv_check_shard_draw_args(const sv_shard_draw_args* a) {
  if (!a) return SV_E_ARG;
  if (a->B < 0 || a->k_max < 1 || a->k_max > SV_MAX_K || a->V < 1 || a->V > kMaxVSampled)
    return SV_E_ARG;
  if (a->G < 1 || a->G > SV_MAX_SHARDS || a->shard < 0 || a->shard >= a->G) return SV_E_ARG;
  if (a->col_offset < 0 || a->col_count < 1 || (int64_t)a->col_offset + a->col_count > a->V)
    return SV_E_ARG;
  if ((uintptr_t)a->offset_dev & 7) return SV_E_ARG;
  if (a->B == 0) return SV_OK;
  if (!a->target_shard || !a->draft_shard || !a->draft_tokens || !a->temperature ||
      !a->masses || !a->out_tokens || !a->accepted)
    return SV_E_ARG;
  if (a->target_vec_stride < a->col_count || a->draft_vec_stride < a->col_count) return SV_E_ARG;
  if (!a->records || a->records_bytes < sample_ws(a->B, a->k_max)) return SV_E_WORKSPACE;
  if (a->masses_bytes < (size_t)a->G * (size_t)a->B * 2 * sizeof(double)) return SV_E_WORKSPACE;
  return SV_OK;
}

static sv_status shard_draw(sv_handle h, const sv_shard_draw_args* a, bool locate, hipStream_t s) {
  const sv_status st = sv_check_shard_draw_args(a);
  if (st != SV_OK) return st;
  if (!h) return SV_E_ARG;
  if (a->B == 0) return SV_OK;
  sv::FinalizeParams f;
  memset(&f, 0, sizeof(f));
  f.tokens = a->draft_tokens;
  f.k_per_row = a->k_per_row;
  f.temperature = a->temperature;
  f.top_p = a->top_p;
  f.B = a->B;
  f.K = a->k_max;
  f.V = a->V;
  f.dtype = SV_BF16;
  f.flags = a->flags;
  f.seed = a->seed;
  f.offset = a->offset;
  f.offset_dev = a->offset_dev;
  f.recs = (const sv::VecRec*)a->records;
  f.out_tokens = a->out_tokens;
  f.accepted = a->accepted;
  f.num_emitted = a->num_emitted;
  f.p_at_draft = a->p_at_draft;
  f.q_at_draft = a->q_at_draft;
  f.row_status = a->row_status;
  sv::ShardDrawParams d;
  d.tgt = a->target_shard;
  d.dft = a->draft_shard;
  d.ts = a->target_vec_stride;
  d.ds = a->draft_vec_stride;
  d.col_off = a->col_offset;
  d.col_len = a->col_count;
  d.G = a->G;
  d.shard = a->shard;
  d.masses = a->masses;
  if (sv::launch_shard_draw(f, d, locate, h->num_cus, s, h->active()) != hipSuccess)
    return SV_E_DEVICE;
  return SV_OK;
}

sv_status sv_shard_draw_mass(sv_handle h, const sv_shard_draw_args* a, hipStream_t s) {
  return shard_draw(h, a, false, s);
}

sv_status sv_shard_draw_locate(sv_handle h, const sv_shard_draw_args* a, hipStream_t s) {
  return shard_draw(h, a, true, s);
}

