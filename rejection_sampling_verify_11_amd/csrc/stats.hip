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
// bf16 path (one workgroup of 1024 threads per vector, one pass over HBM):
// a bf16 logit has only 2^16 possible values, so an exact count of each
// value determines everything: m is the largest value present, the
// normaliser is sum_v count(v) * exp((v - m)/T), and the top-p threshold is
// found by walking values downwards until the cumulative mass reaches
// top_p * S.  The streaming loop therefore does integer work only (one LDS
// atomic per logit); the exp()s are taken per distinct value afterwards, in
// fp64.  Two 16-bit counts share one LDS word: value bits & 0x7FFF select the
// word, the sign bit selects the half.  A count can only wrap if 65536 or
// more logits of one vector are bit-identical; the sum of all stored counts
// then differs from V, which sends the vector down the generic path.
//
// Generic path (fp32 logits, or a bf16 vector whose counts wrapped): passes
// over the vector in global memory: max, fp64 sum, then a 4-pass radix select
// on 32-bit order-preserving keys with fp64 mass histograms.
#include <math.h>

#include "sv_internal.h"

namespace sv {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kHistWords = 32768;
// One pad word per 64 words, so that 64 lanes reading word i of 64
// consecutive 64-word blocks hit 64 different banks.
constexpr int kHistPhys = kHistWords + kHistWords / 64;

__device__ __forceinline__ uint32_t hist_phys(uint32_t word) { return word + (word >> 6); }

// Rank order of bf16 values: rank r in [0, 65536).  r >= 32768 holds the
// non-negative key r - 32768; r < 32768 holds the negative key
// 0x8000 | (32767 - r).  Ranks [128, 65407] are finite, 127 is -inf, 65408 is
// +inf, the rest are NaN.
constexpr int kRankNegInf = 127;
constexpr int kRankPosInf = 65408;

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
  float f[kWaves];
  // broadcast slots
  double bd0, bd1;
  int bi0;
  uint32_t bu0;
  float bf0;
};

// Block-wide sums and maxima in a fixed order (deterministic).
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

__device__ Slot slot_of(const StatsParams& p, int dtype) {
  Slot s;
  const int per = slots_per_row(p.K);
  const int b = blockIdx.x / per, j = blockIdx.x % per;
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

// Writes the record, including p'(x) of the slot's draft token.
__device__ void write_record(const Slot& s, int dtype, int V, float m, float tau,
                             double kept, uint32_t status, VecRec* rec) {
  double px = 0.0;
  if (s.token >= 0) {
    if (s.token >= V) {
      status |= SV_ROW_BAD_TOKEN;
    } else if (!status && s.T_ok && kept > 0.0) {
      const float zx = load_logit(s.vec, dtype, s.token);
      if (zx >= tau) px = exp(((double)zx - (double)m) / (double)s.T) / kept;
    }
  } else if (s.token < -1) {
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

// All threads of the block call this.  hist256 is LDS of 256 doubles.
__device__ void generic_stats(const Slot& s, int dtype, int V, double* hist256,
                              Scratch& sc, VecRec* rec) {
  const int tid = threadIdx.x;
  // pass 1: largest finite value, NaN / +inf, any finite entry
  float mx = -INFINITY;
  uint32_t fl = 0, nfin = 0;
  for (int64_t j = tid; j < V; j += kThreads) {
    const float z = load_logit(s.vec, dtype, j);
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
  uint32_t status = flags & SV_ROW_NONFINITE_LOGIT;
  if (!(flags & 0x80000000u)) status |= SV_ROW_NO_FINITE;
  if (status || !s.T_ok) {
    if (tid == 0) write_record(s, dtype, V, m, -INFINITY, 0.0, status, rec);
    return;
  }
  const double T = (double)s.T, md = (double)m;
  // pass 2: normaliser S
  double acc = 0.0;
  for (int64_t j = tid; j < V; j += kThreads) {
    const float z = load_logit(s.vec, dtype, j);
    acc += exp(((double)z - md) / T);
  }
  const double S = block_sum_d(acc, sc);
  if (!(s.P < 1.0)) {
    if (tid == 0) write_record(s, dtype, V, m, -INFINITY, S, 0, rec);
    return;
  }
  // passes 3-6: radix select of the threshold key, 8 bits at a time
  const double target = s.P * S;
  uint32_t prefix = 0;
  double above = 0.0, kept = S;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    const uint32_t hmask = pass == 0 ? 0u : (0xFFFFFFFFu << (shift + 8));
    for (int i = tid; i < 256; i += kThreads) hist256[i] = 0.0;
    __syncthreads();
    for (int64_t j = tid; j < V; j += kThreads) {
      const float z = load_logit(s.vec, dtype, j);
      if (!(z > -INFINITY)) continue;
      const uint32_t k = order_key(z);
      if ((k & hmask) != (prefix & hmask)) continue;
      const double wgt = exp(((double)z - md) / T);
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
  if (tid == 0) write_record(s, dtype, V, m, key_value(prefix), kept, 0, rec);
}

// ---------------------------------------------------------------- kernels

__global__ __launch_bounds__(kThreads) void stats_generic_kernel(StatsParams p, int dtype) {
  __shared__ double hist256[256];
  __shared__ Scratch sc;
  const Slot s = slot_of(p, dtype);
  if (!s.needed) return;
  generic_stats(s, dtype, p.V, hist256, sc, p.recs + blockIdx.x);
}

__device__ __forceinline__ void hist_add(uint32_t* hist, uint32_t key16) {
  const uint32_t word = key16 & 0x7FFFu;
  const uint32_t inc = 1u << ((key16 >> 11) & 16u);
  __hip_atomic_fetch_add(hist + hist_phys(word), inc, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void hist_add8(uint32_t* hist, const uint4& d) {
  hist_add(hist, d.x & 0xFFFFu); hist_add(hist, d.x >> 16);
  hist_add(hist, d.y & 0xFFFFu); hist_add(hist, d.y >> 16);
  hist_add(hist, d.z & 0xFFFFu); hist_add(hist, d.z >> 16);
  hist_add(hist, d.w & 0xFFFFu); hist_add(hist, d.w >> 16);
}

// Count of rank (64*tid + i); -0 is folded into +0.
__device__ __forceinline__ uint32_t rank_count(const uint32_t* hist, int tid, int i) {
  if (tid >= 512) {
    const uint32_t word = 64u * (uint32_t)(tid - 512) + (uint32_t)i;
    uint32_t c = hist[hist_phys(word)] & 0xFFFFu;
    if (word == 0) c += hist[hist_phys(0)] >> 16;
    return c;
  }
  const uint32_t word = 64u * (uint32_t)(511 - tid) + (uint32_t)(63 - i);
  if (word == 0) return 0;  // -0, counted with +0
  return hist[hist_phys(word)] >> 16;
}

__global__ __launch_bounds__(kThreads) void stats_bf16_kernel(StatsParams p) {
  __shared__ __align__(16) uint32_t hist[kHistPhys];
  __shared__ Scratch sc;
  const Slot s = slot_of(p, SV_BF16);
  if (!s.needed) return;
  const int tid = threadIdx.x;
  const int V = p.V;

  for (int i = tid; i < kHistPhys; i += kThreads) hist[i] = 0;
  __syncthreads();

  // ---- one streaming pass: count every bf16 value
  {
    const uint16_t* vec = (const uint16_t*)s.vec;
    const uintptr_t addr = (uintptr_t)vec;
    int head = (int)(((16u - (uint32_t)(addr & 15u)) & 15u) >> 1);
    if (head > V) head = V;
    if (tid < head) hist_add(hist, vec[tid]);
    const uint4* body = (const uint4*)(vec + head);
    const int nb = (V - head) >> 3;
    int i = tid;
    for (; i + 3 * kThreads < nb; i += 4 * kThreads) {
      const uint4 d0 = body[i];
      const uint4 d1 = body[i + kThreads];
      const uint4 d2 = body[i + 2 * kThreads];
      const uint4 d3 = body[i + 3 * kThreads];
      hist_add8(hist, d0);
      hist_add8(hist, d1);
      hist_add8(hist, d2);
      hist_add8(hist, d3);
    }
    for (; i < nb; i += kThreads) hist_add8(hist, body[i]);
    const int t0 = head + (nb << 3);
    if (t0 + tid < V) hist_add(hist, vec[t0 + tid]);
  }
  __syncthreads();

  // ---- E1: largest finite rank, non-finite flags, totals
  int maxr = -1;
  uint32_t fl = 0, total = 0, nfin = 0;
  for (int i = 0; i < 64; ++i) {
    const uint32_t c = rank_count(hist, tid, i);
    if (!c) continue;
    const int r = 64 * tid + i;
    total += c;
    if (r < kRankNegInf || r >= kRankPosInf) fl |= SV_ROW_NONFINITE_LOGIT;
    else if (r > kRankNegInf) { maxr = r; nfin += c; }
  }
  {
    const int w = tid >> 6, l = tid & 63;
    const int mr = wave_max_i(maxr);
    const uint32_t f = wave_or(fl);
    const uint32_t t = wave_sum(total);
    const uint32_t n = wave_sum(nfin);
    if (l == 0) { sc.i[w] = mr; sc.u[w] = f; sc.u2[w] = t; sc.f[w] = __uint_as_float(n); }
    __syncthreads();
    int MR = -1;
    uint32_t F = 0, TT = 0, N = 0;
    for (int k = 0; k < kWaves; ++k) {
      MR = max(MR, sc.i[k]);
      F |= sc.u[k];
      TT += sc.u2[k];
      N += __float_as_uint(sc.f[k]);
    }
    __syncthreads();
    maxr = MR;
    fl = F;
    total = TT;
    nfin = N;
  }
  if (total != (uint32_t)V) {
    // a 16-bit count wrapped: redo this vector exactly on the generic path,
    // reusing the histogram memory for its 256 fp64 bins
    generic_stats(s, SV_BF16, V, reinterpret_cast<double*>(hist), sc, p.recs + blockIdx.x);
    return;
  }
  uint32_t status = fl;
  if (nfin == 0) status |= SV_ROW_NO_FINITE;
  const float m = maxr >= 0 ? bf16f(rank_key(maxr)) : -INFINITY;
  if (status || !s.T_ok) {
    if (tid == 0) write_record(s, SV_BF16, V, m, -INFINITY, 0.0, status, p.recs + blockIdx.x);
    return;
  }

  // ---- E2: per-thread mass of its 64 ranks, fp64, in descending rank order
  const double T = (double)s.T, md = (double)m;
  double mass = 0.0;
  for (int i = 63; i >= 0; --i) {
    const int r = 64 * tid + i;
    if (r <= kRankNegInf || r > maxr) continue;
    const uint32_t c = rank_count(hist, tid, i);
    if (!c) continue;
    mass += (double)c * exp(((double)bf16f(rank_key(r)) - md) / T);
  }
  // suffix scan over threads in descending order: excl = mass of higher ranks
  const int w = tid >> 6, l = tid & 63;
  double suf = mass;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double t = __shfl_down(suf, o, 64);
    if (l + o < 64) suf += t;
  }
  if (l == 0) sc.d[w] = suf;  // wave total
  __syncthreads();
  double higher = 0.0, S = 0.0;
  for (int k = kWaves - 1; k >= 0; --k) {
    if (k > w) higher += sc.d[k];
    S += sc.d[k];
  }
  const double excl = higher + (suf - mass);

  float tau = -INFINITY;
  double kept = S;
  if (s.P < 1.0) {
    const double target = s.P * S;
    if (tid == 0) { sc.bi0 = -1; sc.bd1 = S; }
    __syncthreads();
    if (mass > 0.0 && excl < target && excl + mass >= target) {
      double cum = excl;
      int tr = -1;
      double kz = S;
      for (int i = 63; i >= 0; --i) {
        const int r = 64 * tid + i;
        if (r <= kRankNegInf || r > maxr) continue;
        const uint32_t c = rank_count(hist, tid, i);
        if (!c) continue;
        const double g = (double)c * exp(((double)bf16f(rank_key(r)) - md) / T);
        if (!(cum < target)) break;
        tr = r;
        cum += g;
        kz = cum;
        if (cum >= target) break;
      }
      sc.bi0 = tr;
      sc.bd1 = kz;
    }
    __syncthreads();
    if (sc.bi0 >= 0) {
      tau = bf16f(rank_key(sc.bi0));
      kept = sc.bd1;
    }
  }
  if (tid == 0) write_record(s, SV_BF16, V, m, tau, kept, 0, p.recs + blockIdx.x);
}

}  // namespace

hipError_t launch_stats(const StatsParams& p, int dtype, hipStream_t s, Timer* t) {
  const unsigned grid = (unsigned)p.B * (unsigned)slots_per_row(p.K);
  if (grid == 0) return hipSuccess;
  if (dtype == SV_BF16) {
    TimedScope ts(t, "stats_bf16", s);
    hipLaunchKernelGGL(stats_bf16_kernel, dim3(grid), dim3(kThreads), 0, s, p);
  } else {
    TimedScope ts(t, "stats_generic", s);
    hipLaunchKernelGGL(stats_generic_kernel, dim3(grid), dim3(kThreads), 0, s, p, dtype);
  }
  return hipGetLastError();
}

}  // namespace sv
