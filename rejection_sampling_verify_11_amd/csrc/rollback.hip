// KV write-pointer and page-table rollback after verification.
//
// [SSD] §3.3 and §4.3: the KV written for rejected drafts must be dropped by
// moving the write pointer back to the accepted prefix ("seq_len + i"), and
// the pointer must equal the sequence length after every rollback; with a
// paged cache the position -> page map is separate and rollback works at
// page granularity.  [SSD] §4.5: ragged acceptance needs one offset per
// sequence.  [SD] §4.3: with a preallocated slot per request only the valid
// length shrinks.
//
// The decision is taken by one wave per row: the row's checks, the new
// length, the number of whole pages released, and the check of the whole
// page-table row against the old length (every logical page below
// ceil(old/ps) maps a page of the pool; with a free stack every later entry
// is unmapped, so the row maps exactly ceil(new/ps) pages afterwards).  Then
// one workgroup walks the rows in tiles of 1024: an exclusive scan of the
// releases (valid rows only) gives every row its slots on the free stack in
// (row, page) order, and a row whose releases would pass the stack capacity
// is flagged and left unchanged.  With a KV pool the scan writes its
// decisions to the workspace first, then a kernel poisons the rolled-back
// slots while the page table still maps them, and the last of each row's
// poisoning workgroups commits the row.
#include "sv_internal.h"

namespace sv {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kCheckRows = 4;  // rows (waves) per check workgroup

__device__ __forceinline__ int ceil_div(int x, int d) { return (x + d - 1) / d; }

// One wave per row.  The record holds the status, the new and old lengths
// and the number of pages the row releases.
__global__ __launch_bounds__(64 * kCheckRows) void rollback_check_kernel(RollbackParams p) {
  const int b = blockIdx.x * kCheckRows + (threadIdx.x >> 6);
  const int l = threadIdx.x & 63;
  if (b >= p.B) return;
  const int k = p.k_per_row ? p.k_per_row[b] : p.K;
  const int acc = p.accepted[b];
  const int old = p.kv_len[b];
  uint32_t st = 0;
  if (k < 1 || k > p.K) st |= SV_ROW_BAD_K;
  else if (acc < 0 || acc > k || old - (k - acc) < 0) st |= SV_ROW_BAD_ACCEPTED;
  if (old < 0 || ceil_div(old, p.ps) > p.MP) st |= SV_ROW_BAD_PAGES;
  if (!st) {
    const int used = ceil_div(old, p.ps);
    const int32_t* row = p.page_table + (int64_t)b * p.MP;
    // past the length only a free stack constrains the entries
    const int span = p.free_pages ? p.MP : used;
    bool bad = false;
    for (int pg = l; pg < span; pg += 64) {
      const int32_t e = row[pg];
      bad = bad || (pg < used ? (e < 0 || (p.num_pages > 0 && e >= p.num_pages)) : e != -1);
    }
    if (__any(bad)) st |= SV_ROW_BAD_PAGES;
  }
  if (l == 0) {
    RollRec r;
    r.status = (int32_t)st;
    r.old_len = old;
    r.new_len = st ? old : old - (k - acc);
    r.aux = st ? 0 : ceil_div(old, p.ps) - ceil_div(r.new_len, p.ps);
    p.recs[b] = r;
  }
}

// phase 0: scan and commit; phase 1 (before the poisoning, which commits):
// scan into p.recs (aux becomes the row's first slot on the free stack,
// status the final status) and zero the rows' commit counters.  Both move
// the stack's top.
__global__ __launch_bounds__(kThreads) void rollback_kernel(RollbackParams p, int phase) {
  __shared__ int wsum[kWaves];
  __shared__ int wmax[kWaves];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int top0 = p.free_pages ? p.free_top[0] : 0;
  int carry = 0;     // releases of valid rows before this tile
  int pushed = 0;    // running total at the last committed row that released
  for (int t0 = 0; t0 < p.B; t0 += kThreads) {
    const int b = t0 + tid;
    RollRec d;
    d.status = 0; d.aux = 0; d.new_len = 0; d.old_len = 0;
    if (b < p.B) d = p.recs[b];
    uint32_t st = (uint32_t)d.status;
    const int rel = (b < p.B && !st) ? d.aux : 0;
    // inclusive scan of rel across the block
    int inc = rel;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(inc, o, 64);
      if (l >= o) inc += v;
    }
    if (l == 63) wsum[w] = inc;
    __syncthreads();
    int before = carry, tot = 0;
    for (int k = 0; k < kWaves; ++k) {
      if (k < w) before += wsum[k];
      tot += wsum[k];
    }
    __syncthreads();
    const int running = before + inc;  // inclusive, over valid rows
    if (b < p.B && !st && p.free_pages && rel > 0 &&
        (top0 < 0 || (int64_t)top0 + running > (int64_t)p.free_capacity))
      st |= SV_ROW_FREE_OVERFLOW;
    const bool commit = b < p.B && !st;
    const int push_base = top0 + running - rel;
    int my_pushed = (commit && p.free_pages && rel > 0) ? running : 0;
    if (phase == 1) {
      if (b < p.B) {
        RollRec r = d;
        r.status = (int32_t)st;
        r.aux = push_base;
        p.recs[b] = r;
        if (p.row_status) p.row_status[b] = (int32_t)st;
        p.row_cnt[(size_t)b * kRollCntStride] = 0u;
      }
    } else {
      if (commit) {
        int32_t* row = p.page_table + (int64_t)b * p.MP;
        if (p.free_pages) {
          const int first = ceil_div(d.new_len, p.ps);
          for (int j = 0; j < rel; ++j) {
            p.free_pages[push_base + j] = row[first + j];
            row[first + j] = -1;
          }
        }
        p.kv_len[b] = d.new_len;
      }
      if (b < p.B && p.row_status) p.row_status[b] = (int32_t)st;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) my_pushed = max(my_pushed, __shfl_xor(my_pushed, o, 64));
    if (l == 0) wmax[w] = my_pushed;
    __syncthreads();
    for (int k = 0; k < kWaves; ++k) pushed = max(pushed, wmax[k]);
    __syncthreads();
    carry += tot;
  }
  if (tid == 0 && p.free_pages) p.free_top[0] = top0 + pushed;
}

// One workgroup per (row, layer): overwrite the rolled-back slots with the
// poison pattern.  Pool layout [page][layer][K|V][head][slot][dim]: for one
// (page, layer, K|V, head) the page's slots are rows of D contiguous values,
// so consecutive slots of a row that share a page are contiguous too.  With
// D a multiple of 8 and the pool on a 16-byte boundary a thread writes 8
// values at once, consecutive threads along a slot row, then along the
// slots of one (K|V, head); otherwise one value at a time.  The rolled-back
// slots (at most k_max of them) lie on a few pages, whose numbers are read
// once into LDS.
//
// The rows are committed here too: each workgroup counts
// itself done for its row with a device-scope atomic once its page numbers
// are read, and the row's last one releases the row's pages onto the free
// stack (at the place the scan gave it) and sets the new length.  Only the
// row's own workgroups read its page-table row, so nothing reads an entry
// after the commit unmaps it.
constexpr int kPoisonPages = 64;
static_assert(kPoisonPages >= SV_MAX_K + 2, "rolled-back slots span at most k_max + 1 pages");

__global__ __launch_bounds__(256) void poison_kernel(RollbackParams p) {
  __shared__ int32_t pages[kPoisonPages];
  __shared__ int last;
  const int b = blockIdx.x / p.L, layer = blockIdx.x % p.L, tid = threadIdx.x;
  const RollRec r = p.recs[b];
  if (r.status != 0) return;
  const int nslots = r.old_len - r.new_len;
  if (nslots <= 0) return;  // nothing rolled back: nothing to release either
  int32_t* row = p.page_table + (int64_t)b * p.MP;
  const int lp0 = r.new_len / p.ps, npg = (r.old_len - 1) / p.ps - lp0 + 1;
  for (int j = tid; j < npg; j += blockDim.x) pages[j] = row[lp0 + j];
  __syncthreads();
  if ((p.D & 7) == 0 && ((uintptr_t)p.kv_pool & 15u) == 0) {
    const int dq = p.D >> 3;               // 16-byte pieces per slot row
    const int per_kvh = nslots * dq;       // pieces of one (K|V, head)
    const int n = 2 * p.H * per_kvh;
    const uint32_t w = (uint32_t)SV_POISON_BF16 * 0x10001u;
    for (int e = tid; e < n; e += blockDim.x) {
      const int kvh = e / per_kvh, rem = e - kvh * per_kvh;
      const int s = rem / dq, c = rem - s * dq;
      const int pos = r.new_len + s;
      const int page = pages[pos / p.ps - lp0];
      const int64_t off =
          ((((int64_t)page * p.L + layer) * 2 * p.H + kvh) * p.ps + pos % p.ps) * p.D + 8 * c;
      *reinterpret_cast<uint4*>(p.kv_pool + off) = make_uint4(w, w, w, w);
    }
  } else {
    const int per_slot = 2 * p.H * p.D;
    for (int e = tid; e < nslots * per_slot; e += blockDim.x) {
      const int s = e / per_slot, rem = e % per_slot;
      const int kvh = rem / p.D, dim = rem % p.D;  // kvh = kv * H + head
      const int pos = r.new_len + s;
      const int page = pages[pos / p.ps - lp0];
      const int64_t off =
          ((((int64_t)page * p.L + layer) * 2 * p.H + kvh) * p.ps + pos % p.ps) * p.D + dim;
      p.kv_pool[off] = (uint16_t)SV_POISON_BF16;
    }
  }
  if (tid == 0)
    last = __hip_atomic_fetch_add(&p.row_cnt[(size_t)b * kRollCntStride], 1u, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)(p.L - 1);
  __syncthreads();
  if (!last) return;
  if (p.free_pages) {
    const int first = ceil_div(r.new_len, p.ps);
    const int rel = ceil_div(r.old_len, p.ps) - first;
    for (int j = tid; j < rel; j += blockDim.x) {
      p.free_pages[r.aux + j] = row[first + j];
      row[first + j] = -1;
    }
  }
  if (tid == 0) p.kv_len[b] = r.new_len;
}

}  // namespace

hipError_t launch_rollback(const RollbackParams& p, hipStream_t s, Timer* t) {
  if (p.B == 0) return hipSuccess;
  {
    TimedScope ts(t, "rollback_check", s);
    hipLaunchKernelGGL(rollback_check_kernel, dim3((p.B + kCheckRows - 1) / kCheckRows),
                       dim3(64 * kCheckRows), 0, s, p);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_rollback_decided(p, s, t);
}

hipError_t launch_rollback_decided(const RollbackParams& p, hipStream_t s, Timer* t) {
  if (p.B == 0) return hipSuccess;
  hipError_t e = hipSuccess;
  if (!p.kv_pool) {
    TimedScope ts(t, "rollback", s);
    hipLaunchKernelGGL(rollback_kernel, dim3(1), dim3(kThreads), 0, s, p, 0);
    return hipGetLastError();
  }
  // decide, then poison; the poisoning commits the rows (the argument
  // checks give a pool at least one layer, head and dim)
  if (!p.row_cnt || p.L < 1 || p.H < 1 || p.D < 1) return hipErrorInvalidValue;
  {
    TimedScope ts(t, "rollback_decide", s);
    hipLaunchKernelGGL(rollback_kernel, dim3(1), dim3(kThreads), 0, s, p, 1);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  TimedScope ts(t, "rollback_poison", s);
  hipLaunchKernelGGL(poison_kernel, dim3((unsigned)p.B * (unsigned)p.L), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace sv
