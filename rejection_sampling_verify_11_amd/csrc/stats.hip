// Per-vector statistics of the verification step: the temperature softmax
// (largest logit m and the normaliser) and the tie-closed top-p threshold.
//
// The pages compute softmax(logits / T) for every verified position of both
// models, with the same T on both sides ([SSD] §2.4, §4.3 verify_stage;
// [FS] §2.3, §3.2), and truncate both to their top-p sets before taking
// ratios ([SSD] §3.4; [FS] §3.2 draft_sampling: sort, cumulative sum, drop a
// token once the mass before it exceeds top_p).  Here the top-p rule is read
// tie-closed: keep j iff the mass of strictly larger logits is below top_p,
// i.e. keep {j : z_j >= tau} for the lowest kept value tau.
//
// bf16 path.  A bf16 logit has only 2^16 possible values, so an exact count
// of each value determines everything: m is the largest value present, the
// normaliser is sum_v count(v) exp((v - m)/T), and the top-p threshold is
// found by walking values downwards until the mass reaches top_p * S.  The
// streaming loop therefore does integer work only (one LDS atomic per
// logit) and the exp()s are taken once per distinct value.  Two 16-bit
// counts share an LDS word: the low 15 bits of the value select the word,
// the sign bit the half.  A count can only wrap if 65536 or more logits of
// one vector are bit-identical; the sum of all stored counts then differs
// from V, which sends that vector down the generic path.
//
// The kernel is persistent: one 1024-thread workgroup per CU (the 132 KB
// count table fills the CU's LDS) walks its share of the vectors.  Per
// vector: stream the logits into the table; each thread reads and clears
// its 32 words (the table is then ready for the next vector); the distinct
// values are compacted into a list in ascending order; masses are formed
// per list entry (fp32 exp2, fp64 sums) and scanned; the thread whose run
// holds top_p * S resolves the threshold exactly.
//
// Generic path (fp32 logits, or a bf16 vector whose counts wrapped): passes
// over the vector in global memory: max, fp64 sum, then a 4-pass radix select
// on 32-bit order-preserving keys with fp64 mass histograms.
#include <math.h>

#include "sv_internal.h"
#include "wave_ops.h"

namespace sv {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kHistWords = 32768;
// Fixed-point scale of value masses: a mass is at most 65535 (count) and a
// vector's total at most V < 2^18, so sums stay below 2^63; one unit is
// 2^-45 of the largest value's weight.
constexpr double kFixScale = 35184372088832.0;  // 2^45
// Distinct finite values listed per vector; a vector with more (none of the
// workloads comes close: they hold 270..2900) takes the generic path.  Sized
// to what is left of the CU's 160 KB of LDS.
constexpr int kListCap = 7000;


// Rank order of bf16 values: rank r in [0, 65536).  r >= 32768 holds the
// non-negative key r - 32768; r < 32768 holds the negative key
// 0x8000 | (32767 - r).  Ranks [128, 65407] are finite, 127 is -inf, 65408 is
// +inf, the rest are NaN.
constexpr uint32_t kFlagWrap = 1u << 30;  // internal: a count passed 16 bits

__device__ __forceinline__ uint32_t rank_key(int r) {
  return r >= 32768 ? (uint32_t)(r - 32768) : (0x8000u | (uint32_t)(32767 - r));
}
__device__ __forceinline__ float bf16f(uint32_t key) { return __uint_as_float(key << 16); }

// ---------------------------------------------------------------- reductions

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ int wave_max_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_max_f(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ uint32_t wave_or(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v |= __shfl_xor(v, o, 64);
  return v;
}

struct Scratch {
  double d[kWaves];
  int i[kWaves];
  uint32_t u[kWaves];
  uint32_t u2[kWaves];
  uint32_t u3[kWaves];
  uint32_t u4[kWaves];
  float f[kWaves];
  double bd0, bd1;
  int bi0;
  uint32_t bu0;
};

__device__ double block_sum_d(double v, Scratch& s) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  if (l == 0) s.d[w] = v;
  __syncthreads();
  double t = 0.0;
  for (int i = 0; i < kWaves; ++i) t += s.d[i];
  __syncthreads();
  return t;
}

// ---------------------------------------------------------------- slot setup

struct Slot {
  bool needed;
  bool draft_side;
  const void* vec;
  int token;     // -1 when the slot verifies no draft token (bonus position)
  float T;
  bool T_ok;
  double P;      // top-p applied to this vector, >= 1 means none
};

__device__ Slot slot_of(const StatsParams& p, int dtype, int v) {
  Slot s;
  const int per = slots_per_row(p.K);
  const int b = v / per, j = v % per;
  const int kb = p.k_per_row ? p.k_per_row[b] : p.K;
  s.needed = false;
  if (kb < 1 || kb > p.K) return s;
  const size_t esz = dtype == SV_BF16 ? 2 : 4;
  if (j <= p.K) {
    if (j > kb || p.mode == 1) return s;
    s.draft_side = false;
    s.vec = (const char*)p.target + ((int64_t)b * (p.K + 1) + j) * p.t_stride * esz;
    s.token = j < kb ? p.tokens[(int64_t)b * p.K + j] : -1;
  } else {
    const int i = j - p.K - 1;
    if (i >= kb) return s;
    s.draft_side = true;
    s.vec = (const char*)p.draft + ((int64_t)b * p.K + i) * p.d_stride * esz;
    s.token = p.mode == 1 ? -1 : p.tokens[(int64_t)b * p.K + i];
  }
  s.needed = true;
  s.T = p.temperature[b];
  s.T_ok = s.T > 0.0f && isfinite(s.T);
  double P = p.top_p ? (double)p.top_p[b] : 1.0;
  if (!(P > 0.0)) P = 1.0;  // invalid top-p is flagged by the finalize kernel
  if (s.draft_side && (p.flags & SV_FLAG_TOPP_TARGET_ONLY)) P = 1.0;
  s.P = P;
  return s;
}

__device__ __forceinline__ float load_logit(const void* vec, int dtype, int64_t j) {
  if (dtype == SV_BF16) return __uint_as_float((uint32_t)((const uint16_t*)vec)[j] << 16);
  return ((const float*)vec)[j];
}

// The slot's draft-token logit (NaN when there is none or it is out of range).
__device__ __forceinline__ float token_logit(const Slot& s, int dtype, int V) {
  if (s.token < 0 || s.token >= V) return __uint_as_float(0x7FC00000u);
  return load_logit(s.vec, dtype, s.token);
}

// Weight exp((z - m) / T) of one value, formed as the finalize kernel forms
// it: exp2 of an fp32 argument, c2 = log2(e) / T.  (z - m) is exact for bf16.
__device__ __forceinline__ double weight(float z, float m, float c2) {
  return (double)__builtin_amdgcn_exp2f((z - m) * c2);
}

// Writes the record, including p'(x) of the slot's draft token (token -1:
// none; T_ok false: the temperature is invalid and no mass is formed).
__device__ void write_record(int token, float T, bool T_ok, int V, float m, float tau,
                             double kept, uint32_t status, float zx, VecRec* rec) {
  double px = 0.0;
  if (token >= 0) {
    if (token >= V) {
      status |= SV_ROW_BAD_TOKEN;
    } else if (!status && T_ok && kept > 0.0 && zx >= tau) {
      px = weight(zx, m, (float)(1.4426950408889634 / (double)T)) / kept;
    }
  } else if (token < -1) {
    status |= SV_ROW_BAD_TOKEN;
  }
  VecRec r;
  r.m = m;
  r.tau = tau;
  r.inv_kept = kept > 0.0 ? 1.0 / kept : 0.0;
  r.px = px;
  r.status = status;
  r.pad = 0;
  *rec = r;
}

// ---------------------------------------------------------------- generic path

__device__ __forceinline__ uint32_t order_key(float z) {
  uint32_t b = __float_as_uint(z == 0.0f ? 0.0f : z);  // -0 and +0 are one value
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k ^ 0x80000000u) : ~k);
}

// All threads of the block call this.  hist256 is LDS of 256 doubles.  Kept
// out of line: it is the rare path of the bf16 kernel and must not add to
// that kernel's register budget.  The slot arrives as plain values so that
// the caller keeps nothing in memory for the call.
__device__ __attribute__((noinline)) void generic_stats(const void* vec, int token, float T,
                                                        double P, int dtype, int V,
                                                        double* hist256, Scratch& sc,
                                                        VecRec* rec) {
  const int tid = threadIdx.x;
  const bool T_ok = T > 0.0f && isfinite(T);
  // pass 1: largest finite value, NaN / +inf, any finite entry
  float mx = -INFINITY;
  uint32_t fl = 0, nfin = 0;
  for (int64_t j = tid; j < V; j += kThreads) {
    const float z = load_logit(vec, dtype, j);
    if (isnan(z) || z == INFINITY) fl |= SV_ROW_NONFINITE_LOGIT;
    else if (z > -INFINITY) { nfin = 1; mx = fmaxf(mx, z); }
  }
  mx = wave_max_f(mx);
  fl = wave_or(fl | (nfin ? 0x80000000u : 0u));
  const int w = tid >> 6, l = tid & 63;
  if (l == 0) { sc.f[w] = mx; sc.u[w] = fl; }
  __syncthreads();
  float m = -INFINITY;
  uint32_t flags = 0;
  for (int i = 0; i < kWaves; ++i) { m = fmaxf(m, sc.f[i]); flags |= sc.u[i]; }
  __syncthreads();
  const float zx = (token >= 0 && token < V) ? load_logit(vec, dtype, token)
                                               : __uint_as_float(0x7FC00000u);
  uint32_t status = flags & SV_ROW_NONFINITE_LOGIT;
  if (!(flags & 0x80000000u)) status |= SV_ROW_NO_FINITE;
  if (status || !T_ok) {
    if (tid == 0) write_record(token, T, T_ok, V, m, -INFINITY, 0.0, status, zx, rec);
    return;
  }
  const float c2 = (float)(1.4426950408889634 / (double)T);
  // pass 2: normaliser S
  double acc = 0.0;
  for (int64_t j = tid; j < V; j += kThreads) acc += weight(load_logit(vec, dtype, j), m, c2);
  const double S = block_sum_d(acc, sc);
  if (!(P < 1.0)) {
    if (tid == 0) write_record(token, T, T_ok, V, m, -INFINITY, S, 0, zx, rec);
    return;
  }
  // passes 3-6: radix select of the threshold key, 8 bits at a time
  const double target = P * S;
  uint32_t prefix = 0;
  double kept = S;
  double above = 0.0;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    const uint32_t hmask = pass == 0 ? 0u : (0xFFFFFFFFu << (shift + 8));
    for (int i = tid; i < 256; i += kThreads) hist256[i] = 0.0;
    __syncthreads();
    for (int64_t j = tid; j < V; j += kThreads) {
      const float z = load_logit(vec, dtype, j);
      if (!(z > -INFINITY)) continue;
      const uint32_t k = order_key(z);
      if ((k & hmask) != (prefix & hmask)) continue;
      const double wgt = weight(z, m, c2);
      if (wgt > 0.0) atomicAdd(&hist256[(k >> shift) & 255u], wgt);
    }
    __syncthreads();
    if (tid == 0) {
      double cum = above;
      int sel = -1, last = -1;
      for (int bin = 255; bin >= 0; --bin) {
        const double h = hist256[bin];
        if (h == 0.0) continue;
        last = bin;
        if (cum + h >= target) { sel = bin; break; }
        cum += h;
      }
      if (sel < 0) { sel = last; cum -= hist256[last]; }  // rounding edge
      sc.bu0 = prefix | ((uint32_t)sel << shift);
      sc.bd0 = cum;
      sc.bd1 = cum + hist256[sel];
    }
    __syncthreads();
    prefix = sc.bu0;
    above = sc.bd0;
    kept = sc.bd1;
    __syncthreads();
  }
  if (tid == 0) write_record(token, T, T_ok, V, m, key_value(prefix), kept, 0, zx, rec);
}

__global__ __launch_bounds__(kThreads) void stats_generic_kernel(StatsParams p, int dtype) {
  __shared__ double hist256[256];
  __shared__ Scratch sc;
  const Slot s = slot_of(p, dtype, blockIdx.x);
  if (!s.needed) return;
  generic_stats(s.vec, s.token, s.T, s.P, dtype, p.V, hist256, sc, p.recs + blockIdx.x);
}

// ---------------------------------------------------------------- bf16 path

// Splits one table word into the counts of +key (lo) and -key (hi): -0 is
// folded into +0, -inf carries no mass, +inf and NaN are errors.  Returns
// flag bits.
__device__ __forceinline__ uint32_t split_counts(uint32_t x, uint32_t key, uint32_t* lo,
                                                 uint32_t* hi) {
  uint32_t l = x & 0xFFFFu, h = x >> 16, fl = 0;
  if (key == 0) {
    l += h;
    h = 0;
    if (l > 0xFFFFu) { fl |= kFlagWrap; l = 0; }
  }
  if (key >= 0x7F80u) {
    if (l) fl |= SV_ROW_NONFINITE_LOGIT;
    if (h && key > 0x7F80u) fl |= SV_ROW_NONFINITE_LOGIT;
    l = 0;
    h = 0;
  }
  *lo = l;
  *hi = h;
  return fl;
}

__device__ __forceinline__ void hist_add(uint32_t* hist, uint32_t key16) {
  const uint32_t word = key16 & 0x7FFFu;
  const uint32_t inc = 1u << ((key16 >> 11) & 16u);
  __hip_atomic_fetch_add(hist + word, inc, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void hist_add8(uint32_t* hist, const uint4& d) {
  hist_add(hist, d.x & 0xFFFFu); hist_add(hist, d.x >> 16);
  hist_add(hist, d.y & 0xFFFFu); hist_add(hist, d.y >> 16);
  hist_add(hist, d.z & 0xFFFFu); hist_add(hist, d.z >> 16);
  hist_add(hist, d.w & 0xFFFFu); hist_add(hist, d.w >> 16);
}

// Streams one vector into the count table.  Batches of 4 x 16 bytes per
// thread; the next batch is loaded before the current one is counted.  Every
// load is unconditional (indices past the end are clamped, their counts
// skipped) so the compiler's wait counts let the prefetch stay in flight.
__device__ __forceinline__ void count_values(const uint16_t* __restrict__ vec, int V,
                                             uint32_t* hist) {
  const int tid = threadIdx.x;
  const uintptr_t addr = (uintptr_t)vec;
  int head = (int)(((16u - (uint32_t)(addr & 15u)) & 15u) >> 1);
  if (head > V) head = V;
  if (tid < head) hist_add(hist, vec[tid]);
  const uint4* body = (const uint4*)(vec + head);
  const int nb = (V - head) >> 3;
  const int last = nb - 1;
  const int nbatch = (nb + 4 * kThreads - 1) / (4 * kThreads);
  if (nbatch > 0) {
    int i = tid;
    uint4 a0 = body[min(i, last)];
    uint4 a1 = body[min(i + kThreads, last)];
    uint4 a2 = body[min(i + 2 * kThreads, last)];
    uint4 a3 = body[min(i + 3 * kThreads, last)];
    for (int k = 0; k < nbatch; ++k) {
      const int j = (k + 1 < nbatch) ? i + 4 * kThreads : i;
      const uint4 b0 = body[min(j, last)];
      const uint4 b1 = body[min(j + kThreads, last)];
      const uint4 b2 = body[min(j + 2 * kThreads, last)];
      const uint4 b3 = body[min(j + 3 * kThreads, last)];
      if (i < nb) hist_add8(hist, a0);
      if (i + kThreads < nb) hist_add8(hist, a1);
      if (i + 2 * kThreads < nb) hist_add8(hist, a2);
      if (i + 3 * kThreads < nb) hist_add8(hist, a3);
      a0 = b0; a1 = b1; a2 = b2; a3 = b3;
      i += 4 * kThreads;
    }
  }
  const int t0 = head + (nb << 3);
  if (t0 + tid < V) hist_add(hist, vec[t0 + tid]);
}

__global__ __launch_bounds__(kThreads) void stats_bf16_kernel(StatsParams p) {
  __shared__ __align__(16) uint32_t hist[kHistWords];
  __shared__ uint32_t list[kListCap];
  __shared__ uint64_t bins1[256];   // fixed-point mass per (rank >> 8)
  __shared__ uint64_t bins2[256];   // fixed-point mass per rank inside the crossing bin
  __shared__ Scratch sc;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int V = p.V;
  const int nslots = p.B * slots_per_row(p.K);
  uint4* hist4 = reinterpret_cast<uint4*>(hist);

  for (int i = tid; i < kHistWords; i += kThreads) hist[i] = 0;
  if (tid < 256) { bins1[tid] = 0; bins2[tid] = 0; }
  __syncthreads();

  for (int v = blockIdx.x; v < nslots; v += gridDim.x) {
    const Slot s = slot_of(p, SV_BF16, v);
    if (!s.needed) continue;
    VecRec* rec = p.recs + v;
    const float zx = tid == 0 ? token_logit(s, SV_BF16, V) : 0.0f;

    count_values((const uint16_t*)s.vec, V, hist);
    __syncthreads();

    // ---- E1: thread t reads the 16-byte groups t + 1024 j (j < 8) of the
    // table: conflict-free, and a dense range of values spreads over many
    // threads.  Word w counts +w in its low half (rank 32768 + w) and -w in
    // its high half (rank 32767 - w).  Only groups holding a count are
    // looked at; jmask remembers them for the second pass.
    uint32_t fl = 0, total = 0, nfin = 0, nent = 0, jmask = 0;
    int maxr = -1;
#pragma unroll 1
    for (int j = 0; j < 8; ++j) {
      const uint4 g = hist4[tid + 1024 * j];
      if (!(g.x | g.y | g.z | g.w)) continue;
      jmask |= 1u << j;
      const uint32_t xs[4] = {g.x, g.y, g.z, g.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t x = xs[q];
        if (!x) continue;
        const uint32_t key = 4u * (tid + 1024u * j) + q;
        total += (x & 0xFFFFu) + (x >> 16);
        uint32_t lo, hi;
        fl |= split_counts(x, key, &lo, &hi);
        nfin += lo + hi;
        nent += (lo != 0) + (hi != 0);
        if (lo) maxr = max(maxr, 32768 + (int)key);
        if (hi) maxr = max(maxr, 32767 - (int)key);
      }
    }
    // block: exclusive scan of entry counts (thread order), flags, totals, max
    const uint32_t einc = wave_scan_u32<OpAddU32>(nent);
    {
      const uint32_t etot = wave_last_u32(einc);
      const int wmax = (int)wave_last_u32(wave_scan_u32<OpMaxI32>((uint32_t)maxr));
      const uint32_t wor = wave_last_u32(wave_scan_u32<OpOrU32>(fl));
      const uint32_t wtot = wave_last_u32(wave_scan_u32<OpAddU32>(total));
      const uint32_t wfin = wave_last_u32(wave_scan_u32<OpAddU32>(nfin));
      if (l == 0) {
        sc.i[w] = wmax;
        sc.u[w] = wor;
        sc.u2[w] = wtot;
        sc.u4[w] = wfin;
        sc.u3[w] = etot;
      }
    }
    __syncthreads();
    int MR = -1;
    uint32_t F = 0, TT = 0, N = 0, ebefore = 0, ND = 0;
    for (int k = 0; k < kWaves; ++k) {
      MR = max(MR, sc.i[k]);
      F |= sc.u[k];
      TT += sc.u2[k];
      N += sc.u4[k];
      if (k < w) ebefore += sc.u3[k];
      ND += sc.u3[k];
    }
    __syncthreads();
    if (TT != (uint32_t)V || (F & kFlagWrap) || ND > (uint32_t)kListCap) {
      // a 16-bit count wrapped (or too many distinct values to list): redo
      // the vector exactly on the generic path, borrowing the table
      generic_stats(s.vec, s.token, s.T, s.P, SV_BF16, V, reinterpret_cast<double*>(hist),
                    sc, rec);
      __syncthreads();
      for (int i = tid; i < kHistWords; i += kThreads) hist[i] = 0;
      __syncthreads();
      continue;
    }
    uint32_t status = F & SV_ROW_NONFINITE_LOGIT;
    if (N == 0) status |= SV_ROW_NO_FINITE;
    const float m = MR >= 0 ? bf16f(rank_key(MR)) : -INFINITY;
    const bool stats_ok = !status && s.T_ok;

    // ---- E2: second pass over the same groups: list entries (rank << 16 |
    // count) at this thread's scanned offset, and the table cleared for the
    // next vector.
    {
      uint32_t o = ebefore + (einc - nent);
#pragma unroll 1
      for (int j = 0; j < 8; ++j) {
        if (!((jmask >> j) & 1u)) continue;
        const uint4 g = hist4[tid + 1024 * j];
        hist4[tid + 1024 * j] = make_uint4(0u, 0u, 0u, 0u);
        if (!stats_ok) continue;
        const uint32_t xs[4] = {g.x, g.y, g.z, g.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (!xs[q]) continue;
          const uint32_t key = 4u * (tid + 1024u * j) + q;
          uint32_t lo, hi;
          split_counts(xs[q], key, &lo, &hi);
          if (lo) list[o++] = ((uint32_t)(32768 + (int)key) << 16) | lo;
          if (hi) list[o++] = ((uint32_t)(32767 - (int)key) << 16) | hi;
        }
      }
    }
    if (!stats_ok) {
      if (tid == 0) write_record(s.token, s.T, s.T_ok, V, m, -INFINITY, 0.0, status, zx, rec);
      __syncthreads();
      continue;
    }
    __syncthreads();

    // ---- E3: mass of each listed value, count * exp((v - m)/T), as a 64-bit
    // fixed-point number (scale 2^45; a vector's total stays below 2^63);
    // integer sums are exact in any order, so the results do not depend on
    // the schedule.  Coarse bins by rank >> 8 for the top-p search.
    const float c2 = (float)(1.4426950408889634 / (double)s.T);
    for (uint32_t e = tid; e < ND; e += kThreads) {
      const uint32_t ent = list[e];
      const uint32_t r = ent >> 16;
      const double mass = (double)(ent & 0xFFFFu) * weight(bf16f(rank_key((int)r)), m, c2);
      const uint64_t fx = (uint64_t)(mass * kFixScale + 0.5);
      if (fx) atomicAdd((unsigned long long*)&bins1[r >> 8], (unsigned long long)fx);
    }
    __syncthreads();

    // ---- E4: wave 0 walks the 256 coarse bins from the top: total S, and
    // the bin where the mass above reaches top_p * S.
    if (w == 0) {
      // lane l holds bins 255-4l .. 252-4l (descending)
      uint64_t b[4];
      double part = 0.0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        b[q] = bins1[255 - 4 * l - q];
        bins1[255 - 4 * l - q] = 0;
        part += (double)b[q];
      }
      const double incl = wave_scan_add_f64(part);   // lanes ascending = bins descending
      const double S_fix = wave_last_f64(incl);
      double above = incl - part;                    // mass of all higher bins
      if (l == 0) { sc.bd0 = S_fix; sc.bi0 = -1; }
      if (s.P < 1.0) {
        const double target = s.P * S_fix;
        if (above < target && above + part >= target) {
          double cum = above;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            if (cum + (double)b[q] >= target && b[q]) {
              sc.bi0 = 255 - 4 * l - q;
              sc.bd1 = cum;
              break;
            }
            cum += (double)b[q];
          }
        }
      }
    }
    __syncthreads();
    const double S_fix = sc.bd0;
    float tau = -INFINITY;
    double kept_fix = S_fix;
    if (s.P < 1.0 && sc.bi0 >= 0) {
      // level 2: the values of the crossing bin, each in its own slot
      const int b1 = sc.bi0;
      for (uint32_t e = tid; e < ND; e += kThreads) {
        const uint32_t ent = list[e];
        const uint32_t r = ent >> 16;
        if ((int)(r >> 8) != b1) continue;
        const double mass = (double)(ent & 0xFFFFu) * weight(bf16f(rank_key((int)r)), m, c2);
        bins2[r & 255u] = (uint64_t)(mass * kFixScale + 0.5);
      }
      __syncthreads();
      if (w == 0) {
        uint64_t b[4];
        double part = 0.0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          b[q] = bins2[255 - 4 * l - q];
          bins2[255 - 4 * l - q] = 0;
          part += (double)b[q];
        }
        const double incl = wave_scan_add_f64(part);
        const double above = sc.bd1 + (incl - part);
        const double target = s.P * S_fix;
        if (l == 0) sc.bu0 = 0xFFFFFFFFu;
        if (above < target && above + part >= target) {
          double cum = above;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            if (b[q] && cum + (double)b[q] >= target) {
              sc.bu0 = (uint32_t)(b1 << 8) | (uint32_t)(255 - 4 * l - q);
              sc.bd0 = cum + (double)b[q];
              break;
            }
            cum += (double)b[q];
          }
        }
      }
      __syncthreads();
      if (sc.bu0 != 0xFFFFFFFFu) {
        tau = bf16f(rank_key((int)sc.bu0));
        kept_fix = sc.bd0;
      }
    }
    if (tid == 0)
      write_record(s.token, s.T, s.T_ok, V, m, tau, kept_fix * (1.0 / kFixScale), 0, zx, rec);
    __syncthreads();  // scratch and list are reused by the next vector
  }
}

}  // namespace

hipError_t launch_stats(const StatsParams& p, int dtype, int num_cus, hipStream_t s, Timer* t) {
  const unsigned nslots = (unsigned)p.B * (unsigned)slots_per_row(p.K);
  if (nslots == 0) return hipSuccess;
  if (dtype == SV_BF16) {
    const unsigned cus = num_cus > 0 ? (unsigned)num_cus : 256u;
    const unsigned grid = nslots < cus ? nslots : cus;
    TimedScope ts(t, "stats_bf16", s);
    hipLaunchKernelGGL(stats_bf16_kernel, dim3(grid), dim3(kThreads), 0, s, p);
  } else {
    TimedScope ts(t, "stats_generic", s);
    hipLaunchKernelGGL(stats_generic_kernel, dim3(nslots), dim3(kThreads), 0, s, p, dtype);
  }
  return hipGetLastError();
}

}  // namespace sv
