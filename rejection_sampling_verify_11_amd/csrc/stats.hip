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
// bf16 path.  A bf16 logit takes few distinct values, so an exact count of
// each value determines everything: m is the largest value present, the
// normaliser is sum_v count(v) exp((v - m)/T), and the top-p threshold is
// found by walking values downwards until the mass reaches top_p * S.  The
// streaming loop does integer work only (one LDS atomic per logit) and the
// exp()s are taken once per distinct value.
//
// The count table covers a window of magnitudes, [2^-24, 2^16): 40 exponent
// rows of 128 mantissas, one 32-bit word per magnitude holding the count of
// +v in its low half and of -v in its high half (20 KB).  Zeros and -inf are
// counted in registers; NaN and +inf mark the row as an error.  Any other
// logit outside the window, or a count that wraps its 16 bits (65536 equal
// logits), sends the vector down the generic path.  The small table lets
// three workgroups share a CU, so one workgroup's epilogue (no memory traffic)
// overlaps the others' streaming; vectors are handed out from queues
// (below) so that the workgroups of a CU do not stay in step.
//
// Generic path (fp32 logits, or a bf16 vector the table cannot hold): passes
// over the vector in global memory: max, fp64 sum, then a 4-pass radix select
// on 32-bit order-preserving keys with fp64 mass histograms.
#include <hip/hip_ext.h>
#include <math.h>

#include "sv_internal.h"
#include "wave_ops.h"

namespace sv {
namespace {

constexpr int kGenThreads = 1024;  // generic kernel: one workgroup per vector

__device__ __forceinline__ float bf16f(uint32_t key) { return __uint_as_float(key << 16); }

// ---------------------------------------------------------------- reductions

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
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

template <int NW>
struct Scratch {
  double d[NW];
  uint32_t u[NW];
  float f[NW];
  double bd0, bd1;
  uint32_t bu0;
};

template <int NT>
__device__ double block_sum_d(double v, Scratch<NT / 64>& s) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  if (l == 0) s.d[w] = v;
  __syncthreads();
  double t = 0.0;
  for (int i = 0; i < NT / 64; ++i) t += s.d[i];
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

// The logits of one vector stored in one piece, for generic_stats.
struct VecLogits {
  const void* vec;
  int dtype;
  __device__ __forceinline__ float operator()(int64_t j) const { return load_logit(vec, dtype, j); }
};

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
      px = weight(zx, m, log2e_over_T(T)) / kept;
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

// The logits thread tid takes in the generic passes, j = tid, tid + NT, ...
// in increasing order.  Streamed: read again on every pass.
template <int NT, class Logits>
struct StreamedLogits {
  const Logits& logit;
  int V;
  template <class F>
  __device__ __forceinline__ void each(F&& f) const {
    for (int64_t j = threadIdx.x; j < V; j += NT) f(logit(j));
  }
};

// fp32 logits of a vector, streamed on every pass in 16-byte loads, kU of
// them in flight per thread: the logits before the first 16-byte boundary
// (at most three, threads 0..2), then thread tid takes the groups of four
// logits tid, tid + NT, ..., then the tail logits past the last whole group,
// in that order.
template <int NT>
struct StreamedF32 {
  const float* vec;
  int V;
  static constexpr int kU = 4;
  template <class F>
  __device__ __forceinline__ void each(F&& f) const {
    const int tid = threadIdx.x;
    const int head = min(V, (int)((((16u - (uint32_t)((uintptr_t)vec & 15u)) & 15u)) >> 2));
    if (tid < head) f(vec[tid]);
    const float* body = vec + head;
    const int nb = V - head;
    const int n4 = nb >> 2;
    const float4* v4 = reinterpret_cast<const float4*>(body);
    int g = tid;
    for (; g + (kU - 1) * NT < n4; g += kU * NT) {
      float4 a[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) a[u] = v4[g + u * NT];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        f(a[u].x);
        f(a[u].y);
        f(a[u].z);
        f(a[u].w);
      }
    }
    for (; g < n4; g += NT) {
      const float4 a = v4[g];
      f(a.x);
      f(a.y);
      f(a.z);
      f(a.w);
    }
    for (int j = 4 * n4 + tid; j < nb; j += NT) f(body[j]);
  }
};

// The same logits held in registers (V <= NT * R): read once, all loads in
// flight together, so a short vector costs one memory round trip instead of
// one per pass and per element.  The passes see the values in the same
// order, so the results are the streamed passes' bit for bit.
template <int NT, int R>
struct HeldLogits {
  float z[R];
  int V;
  template <class Logits>
  __device__ __forceinline__ void load(const Logits& logit, int n) {
    V = n;
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int64_t j = threadIdx.x + (int64_t)NT * i;
      z[i] = logit(j < n ? j : 0);
    }
  }
  template <class F>
  __device__ __forceinline__ void each(F&& f) const {
#pragma unroll
    for (int i = 0; i < R; ++i)
      if (threadIdx.x + (int64_t)NT * i < V) f(z[i]);
  }
};

// Doubles between the copies of the radix passes' 256-bin histogram: one
// more than the bins, so that copies of one bin lie in different banks.
constexpr int kHistStride = 257;

// All NT threads of the block call this.  hist256 is LDS of HC * kHistStride
// doubles (256 for one copy).
// The bf16 kernel reaches it only for a vector its count table cannot hold.
// `elems` yields this thread's logits (StreamedLogits or HeldLogits); zx is
// the draft token's logit (NaN when there is none).
template <int NT, class Elems, int HC = 1, int CAP = 0>
__device__ __forceinline__ void generic_stats(const Elems& elems, int token, float zx, float T,
                                              double P, int V, double* hist256,
                                              Scratch<NT / 64>& sc, VecRec* rec,
                                              float* cand = nullptr, uint32_t* ncand = nullptr) {
  const int tid = threadIdx.x;
  const bool T_ok = T > 0.0f && isfinite(T);
  // pass 1: largest finite value, NaN / +inf, any finite entry
  float mx = -INFINITY;
  uint32_t fl = 0, nfin = 0;
  elems.each([&](float z) {
    if (isnan(z) || z == INFINITY) fl |= SV_ROW_NONFINITE_LOGIT;
    else if (z > -INFINITY) { nfin = 1; mx = fmaxf(mx, z); }
  });
  mx = wave_max_f(mx);
  fl = wave_or(fl | (nfin ? 0x80000000u : 0u));
  const int w = tid >> 6, l = tid & 63;
  if (l == 0) { sc.f[w] = mx; sc.u[w] = fl; }
  __syncthreads();
  float m = -INFINITY;
  uint32_t flags = 0;
  for (int i = 0; i < NT / 64; ++i) { m = fmaxf(m, sc.f[i]); flags |= sc.u[i]; }
  __syncthreads();
  uint32_t status = flags & SV_ROW_NONFINITE_LOGIT;
  if (!(flags & 0x80000000u)) status |= SV_ROW_NO_FINITE;
  if (status || !T_ok) {
    if (tid == 0) write_record(token, T, T_ok, V, m, -INFINITY, 0.0, status, zx, rec);
    return;
  }
  const float c2 = log2e_over_T(T);
  // pass 2: normaliser S and, with a top-p cut, the masses of the radix
  // select's first digit; passes 3-5: the other three digits (8 bits each)
  const bool cut = P < 1.0;
  // with HC copies, lane l adds into copy l % HC: lanes of one wave that
  // land in one bin (few bins take most logits in the first passes) then
  // mostly hit different words
  double* hist = hist256 + (HC > 1 ? (tid & 63) % HC * kHistStride : 0);
  if (cut) {
    for (int i = tid; i < HC * kHistStride; i += NT) hist256[i] = 0.0;
    __syncthreads();
  }
  double acc = 0.0;
  elems.each([&](float z) {
    const double wgt = weight(z, m, c2);
    acc += wgt;
    if (cut && wgt > 0.0) atomicAdd(&hist[order_key(z) >> 24], wgt);
  });
  const double S = block_sum_d<NT>(acc, sc);
  if (!cut) {
    if (tid == 0) write_record(token, T, T_ok, V, m, -INFINITY, S, 0, zx, rec);
    return;
  }
  __syncthreads();
  const double target = P * S;
  uint32_t prefix = 0;
  double kept = S;
  double above = 0.0;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    if (pass > 0) {
      const uint32_t hmask = 0xFFFFFFFFu << (shift + 8);
      for (int i = tid; i < HC * kHistStride; i += NT) hist256[i] = 0.0;
      if (CAP > 0 && pass == 2 && tid == 0) *ncand = 0u;
      __syncthreads();
      const auto add = [&](float z, bool keep) {
        // held values would otherwise keep pass 2's weights alive (and
        // spill) instead of forming them again
        asm volatile("" : "+v"(z));
        if (!(z > -INFINITY)) return;
        const uint32_t k = order_key(z);
        if ((k & hmask) != (prefix & hmask)) return;
        // with CAP, the third digit's pass keeps the logits under its
        // 16-bit prefix (few: one bf16-wide bucket) for the last digit
        if (CAP > 0 && keep) {
          const uint32_t i = atomicAdd(ncand, 1u);
          if (i < (uint32_t)CAP) cand[i] = z;
        }
        const double wgt = weight(z, m, c2);
        if (wgt > 0.0) atomicAdd(&hist[(k >> shift) & 255u], wgt);
      };
      if (CAP > 0 && pass == 3 && *ncand <= (uint32_t)CAP) {
        const int n = (int)*ncand;
        for (int i = tid; i < n; i += NT) add(cand[i], false);
      } else {
        elems.each([&](float z) { add(z, pass == 2); });
      }
      __syncthreads();
    }
    if constexpr (HC > 1) {
      for (int bin = tid; bin < 256; bin += NT) {
        double t = 0.0;
#pragma unroll
        for (int c = 0; c < HC; ++c) t += hist256[c * kHistStride + bin];
        hist256[bin] = t;
      }
      __syncthreads();
    }
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

// The generic statistics over one stored vector: its draft token's logit
// is read with the first pass.
template <int NT, class Logits>
__device__ __forceinline__ void generic_stats(const Logits& logit, int token, float T, double P,
                                              int V, double* hist256, Scratch<NT / 64>& sc,
                                              VecRec* rec) {
  const float zx = (token >= 0 && token < V) ? logit(token) : __uint_as_float(0x7FC00000u);
  generic_stats<NT>(StreamedLogits<NT, Logits>{logit, V}, token, zx, T, P, V, hist256, sc, rec);
}

// Logits per thread that the generic kernel holds in registers.
constexpr int kGenHeld = 32;
// Copies of the radix histogram in the generic kernel.
constexpr int kGenHistCopies = 16;
// Logits under the threshold's 16-bit key prefix that the generic kernel
// keeps in LDS, so that the last radix digit needs no pass over the vector.
constexpr int kGenCand = 4096;

// fp32 logits of one stored vector (the generic kernel's dtype): a typed
// read, so that the held loads carry no dtype branch and all issue at once.
struct Fp32Logits {
  const float* vec;
  __device__ __forceinline__ float operator()(int64_t j) const { return vec[j]; }
};

// One workgroup per vector slot: HELD (fp32, V <= kGenThreads * kGenHeld)
// reads the vector once into registers, otherwise every pass streams it.
template <bool HELD>
__global__ __launch_bounds__(kGenThreads) void stats_generic_kernel(StatsParams p, int dtype) {
  __shared__ double hist256[kGenHistCopies * kHistStride];
  __shared__ Scratch<kGenThreads / 64> sc;
  __shared__ float cand[kGenCand];
  __shared__ uint32_t ncand;
  const Slot s = slot_of(p, dtype, blockIdx.x);
  if (!s.needed) return;
  const VecLogits logit{s.vec, dtype};
  if constexpr (HELD) {
    HeldLogits<kGenThreads, kGenHeld> held;
    held.load(Fp32Logits{(const float*)s.vec}, p.V);
    const float zx = (s.token >= 0 && s.token < p.V) ? logit(s.token)
                                                      : __uint_as_float(0x7FC00000u);
    generic_stats<kGenThreads, decltype(held), kGenHistCopies>(held, s.token, zx, s.T, s.P, p.V, hist256, sc,
                               p.recs + blockIdx.x);
  } else if (dtype == SV_FP32) {
    const float* vec = (const float*)s.vec;
    const float zx = (s.token >= 0 && s.token < p.V) ? vec[s.token] : __uint_as_float(0x7FC00000u);
    generic_stats<kGenThreads, StreamedF32<kGenThreads>, kGenHistCopies, kGenCand>(
        StreamedF32<kGenThreads>{vec, p.V}, s.token, zx, s.T, s.P, p.V, hist256, sc,
        p.recs + blockIdx.x, cand, &ncand);
  } else {
    const float zx = (s.token >= 0 && s.token < p.V) ? logit(s.token) : __uint_as_float(0x7FC00000u);
    generic_stats<kGenThreads, StreamedLogits<kGenThreads, VecLogits>, kGenHistCopies>(
        StreamedLogits<kGenThreads, VecLogits>{logit, p.V}, s.token, zx, s.T, s.P, p.V, hist256, sc,
        p.recs + blockIdx.x);
  }
}

// ---------------------------------------------------------------- bf16 path

constexpr int kT = 256;                  // threads per workgroup
constexpr int kWv = kT / 64;             // waves per workgroup
constexpr int kWgPerCu = 3;              // workgroups sharing a CU
constexpr int kBatch = 4;                // 16-byte loads per thread per batch
constexpr uint32_t kE0 = 103;            // lowest exponent field in the window (2^-24)
constexpr int kNE = 40;                  // exponent rows: magnitudes below 2^16
constexpr uint32_t kBase = kE0 << 7;     // magnitude bits of the window's first word
constexpr int kWords = kNE * 128;        // 5120 words, 20 KB
constexpr int kGroups = kWords / 4;      // 16-byte groups of the table
constexpr int kGpt = kGroups / kT;       // groups per thread
constexpr int kBins = kGroups / 64;      // bins of 256 magnitudes, per sign
// Rank bins, in value order: the -magnitude bins (largest magnitude first),
// the nonzero -values below the window, 0, the nonzero +values below the
// window, then the +magnitude bins.
constexpr int kRankBins = 2 * kBins + 3;
constexpr int kZeroBin = kBins + 1;      // rank bin of the value 0
constexpr int kTinyCap = 64;             // values below the window kept per vector
static_assert(kGroups % kT == 0 && kGpt * kWv <= kBins * 2, "table tiling");
static_assert(kBins == kWv * kGpt, "one (wave, row) per bin");

// The streaming loop counts into two copies of the table, lanes of even and
// odd index into copy 0 and 1.  The logits of one vector take few distinct
// values (a few hundred, a few dozen of them hot), and an LDS atomic
// instruction serialises its lanes that hit one address; two copies half as
// many bank rows apart halve that.  The first epilogue pass merges copy 1
// into copy 0 and clears copy 1.
constexpr int kCopies = 2;
constexpr int kCopyWords = kWords + 16;  // copy 1 starts 16 banks over
static_assert((kCopyWords * 4) % 16 == 0, "copies are 16-byte aligned");

constexpr uint32_t kFallback = 1u << 30;  // internal: the table cannot hold the vector

// Rank bin of magnitude bin b: +values above zero, -values below.
__device__ __forceinline__ int pos_bin(int b) { return kZeroBin + 2 + b; }
__device__ __forceinline__ int neg_bin(int b) { return kZeroBin - 2 - b; }

// Window test of both logits of a 32-bit word as arithmetic (no branches):
// the exponent bits less the window's first, unsigned, so that exponents
// below the window wrap high.  The word lies in the window iff the larger of
// the two is below kWords (the window is whole exponent rows).
__device__ __forceinline__ uint32_t window_excess(uint32_t x) {
  const uint32_t lo = (x & 0x7F80u) - kBase;
  const uint32_t hi = ((x >> 16) & 0x7F80u) - kBase;
  return max(lo, hi);
}

// Registers of the out-of-window logits seen by one thread.
struct Side {
  uint32_t nzero = 0, nninf = 0, flags = 0;
};

// Counts logit k when `valid`: in the window into the table, else into the
// thread's side counters (zero, -inf), the vector's list of nonzero values
// below the window (`tiny`: count, then up to kTinyCap raw values), or flags
// (NaN / +inf: error; a finite value above the window or a full list:
// fallback).  The table atomic always runs, adding 0 to a word of the
// thread's own (`spare`) when there is nothing to count.
__device__ __forceinline__ void count_slow(uint32_t* hist, uint32_t* tiny, uint32_t k, bool valid,
                                          uint32_t spare, Side& sd) {
  const uint32_t mag = k & 0x7FFFu;
  const uint32_t word = mag - kBase;
  const bool inw = valid && word < (uint32_t)kWords;
  const uint32_t inc = inw ? 1u << ((k >> 11) & 16u) : 0u;
  __hip_atomic_fetch_add(hist + (inw ? word : spare), inc, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_WORKGROUP);
  const bool out = valid && !inw;
  sd.nzero += (out && mag == 0u) ? 1u : 0u;
  sd.nninf += (out && k == 0xFF80u) ? 1u : 0u;
  sd.flags |= (out && mag >= 0x7F80u && k != 0xFF80u) ? (uint32_t)SV_ROW_NONFINITE_LOGIT : 0u;
  sd.flags |= (out && mag >= kBase + (uint32_t)kWords && mag < 0x7F80u) ? kFallback : 0u;
  if (out && mag != 0u && mag < kBase) {
    const uint32_t i = __hip_atomic_fetch_add(tiny, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    if (i < (uint32_t)kTinyCap) tiny[1 + i] = k;
    else sd.flags |= kFallback;
  }
}

// Counts both logits of a 32-bit word, known to lie in the window.  hbase
// is the table shifted down by the window's first word, so a logit's word
// is hbase + magnitude; the increment is 1 for a +value, 0x10000 for a
// -value (4 VALU instructions per logit).
__device__ __forceinline__ void count_word_fast(uint32_t* hbase, uint32_t w) {
  const uint32_t mlo = w & 0x7FFFu, mhi = __builtin_amdgcn_ubfe(w, 16, 15);
  const uint32_t slo = __builtin_amdgcn_ubfe(w, 15, 1), shi = w >> 31;
  __hip_atomic_fetch_add(hbase + mlo, slo * 0xFFFFu + 1u, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_WORKGROUP);
  __hip_atomic_fetch_add(hbase + mhi, shi * 0xFFFFu + 1u, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void count_group_fast(uint32_t* hbase, const uint4& d) {
  count_word_fast(hbase, d.x);
  count_word_fast(hbase, d.y);
  count_word_fast(hbase, d.z);
  count_word_fast(hbase, d.w);
}

// Window test of a batch with packed 16-bit arithmetic: per half, the
// exponent bits less the window's first, wrapping below it; the batch lies
// in the window iff the largest of them is below kWords.
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t batch_excess(const uint4 (&a)[kBatch]) {
  const u16x2 base = {(unsigned short)kBase, (unsigned short)kBase};
  u16x2 m = {0, 0};
#pragma unroll
  for (int q = 0; q < kBatch; ++q) {
    const uint32_t w[4] = {a[q].x, a[q].y, a[q].z, a[q].w};
#pragma unroll
    for (int t = 0; t < 4; ++t)
      m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, w[t] & 0x7F807F80u) - base);
  }
  return max((uint32_t)m.x, (uint32_t)m.y);
}

// Counts logit k, known to lie in the window, when `valid`; otherwise adds
// 0 to the thread's spare word (no branch).
__device__ __forceinline__ void hist_add_masked(uint32_t* hist, uint32_t k, bool valid,
                                                uint32_t spare) {
  const uint32_t word = (k & 0x7FFFu) - kBase;
  const uint32_t inc = valid ? 1u << ((k >> 11) & 16u) : 0u;
  __hip_atomic_fetch_add(hist + (valid ? word : spare), inc, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void count_group_masked(uint32_t* hist, const uint4& d, bool valid,
                                                  uint32_t spare) {
  const uint32_t w[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    hist_add_masked(hist, w[q] & 0xFFFFu, valid, spare);
    hist_add_masked(hist, w[q] >> 16, valid, spare);
  }
}
__device__ __forceinline__ void count_group_slow(uint32_t* hist, uint32_t* tiny, const uint4& d,
                                                bool valid, uint32_t spare, Side& sd) {
  const uint32_t w[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    count_slow(hist, tiny, w[q] & 0xFFFFu, valid, spare, sd);
    count_slow(hist, tiny, w[q] >> 16, valid, spare, sd);
  }
}

// A batch holding a logit outside the window (rare); group q counts when
// bit q of vmask is set.  Out of line, with everything passed by value, so
// that its register needs do not weigh on the streaming loop.
static_assert(kBatch == 4, "count_batch_slow takes four groups");
__device__ __attribute__((noinline)) Side count_batch_slow(uint32_t* hist, uint32_t* tiny,
                                                           uint4 d0, uint4 d1, uint4 d2, uint4 d3,
                                                           uint32_t vmask, uint32_t spare, Side sd) {
  count_group_slow(hist, tiny, d0, vmask & 1u, spare, sd);
  count_group_slow(hist, tiny, d1, (vmask >> 1) & 1u, spare, sd);
  count_group_slow(hist, tiny, d2, (vmask >> 2) & 1u, spare, sd);
  count_group_slow(hist, tiny, d3, (vmask >> 3) & 1u, spare, sd);
  return sd;
}

// The head and tail logits of a vector outside the window (rare), likewise.
__device__ __attribute__((noinline)) Side count_pair_slow(uint32_t* hist, uint32_t* tiny,
                                                          uint32_t xh, bool has_head, uint32_t xt,
                                                          bool has_tail, uint32_t spare, Side sd) {
  count_slow(hist, tiny, xh, has_head, spare, sd);
  count_slow(hist, tiny, xt, has_tail, spare, sd);
  return sd;
}

// Loads one batch: groups i, i + NTV, ... of a body with nb > 0 (NTV
// threads stream the vector); an index past the end is clamped to the last
// group (loaded, not counted).
template <int NTV>
__device__ __forceinline__ void load_batch(uint4 (&d)[kBatch], const uint4* body, int i, int nb) {
#pragma unroll
  for (int s = 0; s < kBatch; ++s) d[s] = body[min(i + s * NTV, nb - 1)];
}

// Streams one vector into the table.  Full batches go through the fast path
// unless a logit of the batch lies outside the window (a wave-uniform test);
// the last, partial batch and the unaligned head and tail always go through
// the slow path.  Batch k is counted while batch k + 1 loads.  NTV threads
// stream the vector; tid is this thread's index among them.
template <int NTV>
__device__ __forceinline__ void stream_vector(const uint16_t* vec, int V, uint32_t* hist,
                                              uint32_t* tiny, Side& sd, int tid) {
  const uint32_t spare = (uint32_t)tid % (uint32_t)kWords;
  uint32_t* hbase = hist - kBase;
  int head = (int)(((16u - (uint32_t)((uintptr_t)vec & 15u)) & 15u) >> 1);
  if (head > V) head = V;
  const uint4* body = (const uint4*)(vec + head);
  const int nb = (V - head) >> 3;
  const int t0 = head + (nb << 3);
  // head and tail logits (a lane without one loads logit 0 and counts nothing)
  const bool has_head = tid < head, has_tail = t0 + tid < V;
  const uint32_t xh = vec[has_head ? tid : 0];
  const uint32_t xt = vec[has_tail ? t0 + tid : 0];
  if (nb > 0) {
    const int step = kBatch * NTV;
    const int nfull = nb / step;
    const bool part = nfull * step < nb;
    uint4 a[kBatch];
    load_batch<NTV>(a, body, tid, nb);
    int i = tid;
    for (int k = 0; k < nfull; ++k) {
      uint4 n[kBatch];
      load_batch<NTV>(n, body, (k + 1 < nfull || part) ? i + step : i, nb);
      const uint32_t ex = batch_excess(a);
      if (!__any(ex >= (uint32_t)kWords)) {
#pragma unroll
        for (int q = 0; q < kBatch; ++q) count_group_fast(hbase, a[q]);
      } else {
        sd = count_batch_slow(hist, tiny, a[0], a[1], a[2], a[3], 0xFu, spare, sd);
      }
#pragma unroll
      for (int q = 0; q < kBatch; ++q) a[q] = n[q];
      i += step;
    }
    if (part) {
      uint32_t vmask = 0, ex = 0;
#pragma unroll
      for (int q = 0; q < kBatch; ++q) {
        const bool valid = i + q * NTV < nb;
        vmask |= valid ? 1u << q : 0u;
        const uint32_t e = max(max(window_excess(a[q].x), window_excess(a[q].y)),
                               max(window_excess(a[q].z), window_excess(a[q].w)));
        ex = max(ex, valid ? e : 0u);
      }
      if (!__any(ex >= (uint32_t)kWords)) {
#pragma unroll
        for (int q = 0; q < kBatch; ++q) count_group_masked(hist, a[q], (vmask >> q) & 1u, spare);
      } else {
        sd = count_batch_slow(hist, tiny, a[0], a[1], a[2], a[3], vmask, spare, sd);
      }
    }
  }
  const uint32_t exh = has_head ? ((xh & 0x7F80u) - kBase) : 0u;
  const uint32_t ext = has_tail ? ((xt & 0x7F80u) - kBase) : 0u;
  if (!__any(max(exh, ext) >= (uint32_t)kWords)) {
    hist_add_masked(hist, xh, has_head, spare);
    hist_add_masked(hist, xt, has_tail, spare);
  } else {
    sd = count_pair_slow(hist, tiny, xh, has_head, xt, has_tail, spare, sd);
  }
}

// Vectors are handed out dynamically: a workgroup that finishes early takes
// the next vector, so the workgroups of a CU drift apart and one's epilogue
// overlaps the others' streaming (a fixed schedule keeps them in step).  One
// counter for all would queue hundreds of device-scope atomics on a single
// address, so the work items are split into kQueues interleaved queues
// (queue q holds items q, q + kQueues, ...), each with its own counter 128
// bytes apart and served by the workgroups g with g % kQueues == q.  Ticket
// t of queue q is item q + kQueues t; workgroup g's first ticket is
// g / kQueues (no atomic) and each counter starts at its queue's number of
// workgroups.  Item i maps to a slot by item_slot, or is the i-th entry of
// the slot list when the call uses only some slots: a skipped slot costs no
// ticket.
constexpr int kQueues = 64;
constexpr int kQueueStride = 32;  // uint32 words between counters

__device__ __forceinline__ int queue_item(int q, uint32_t t) { return q + kQueues * (int)t; }

__device__ __forceinline__ int take_ticket(const StatsParams& p, int q) {
  return queue_item(q, atomicAdd(p.tickets + q * kQueueStride, 1u));
}

// Without a list, items run position-major: the bonus position of every
// row, then target and draft position K-1 of every row, ..., position 0
// last.  Vectors streamed side by side then belong to different rows, which
// measured ~3 % faster than the slot order (rows' vectors adjacent).  A
// list (in row order) is visited as item * stride mod n with a stride
// coprime to n, for the same effect.
__device__ __forceinline__ uint32_t list_stride(uint32_t n) {
  const uint32_t primes[4] = {1009u, 1013u, 1019u, 1021u};
  uint32_t s = 1u;
#pragma unroll
  for (int i = 3; i >= 0; --i) s = n % primes[i] ? primes[i] : s;
  return s;
}

// Items of a call without a slot list: every slot, or every draft slot when
// sampling drafts.
__host__ __device__ __forceinline__ int unlisted_items(const StatsParams& p) {
  return p.mode == 1 ? p.B * p.K : p.B * slots_per_row(p.K);
}

__device__ __forceinline__ int item_slot(const StatsParams& p, int item, uint32_t n, uint32_t stride) {
  if (p.slot_list) return p.slot_list[(uint32_t)(((uint64_t)item * stride) % n)];
  const int B = p.B, K = p.K, per = slots_per_row(K);
  if (p.mode == 1) {  // draft positions only, K-1 of every row first
    const int q = item / B, r = item - q * B;
    return r * per + K + 1 + (K - 1 - q);
  }
  if (item < B) return item * per + K;
  const int i = item - B, q = i / (2 * B), r = i - q * 2 * B;
  const int pos = K - 1 - q;
  return r < B ? r * per + pos : (r - B) * per + K + 1 + pos;
}

// A used slot's vector and parameters (the fields of slot_of).  The vector
// address is arithmetic; the loads are issued together and nothing branches
// on them.
struct SlotP {
  const uint16_t* vec;
  int token;
  float T;
  double P;
};

// The shard pass (SHARD) counts only: it reads no temperature or top-p.
template <bool SHARD>
__device__ __forceinline__ SlotP slot_params(const StatsParams& p, int v) {
  const int K = p.K, per = slots_per_row(K);
  const int b = v / per, j = v % per;
  const bool draft_side = j > K;
  const int i = draft_side ? j - K - 1 : j;
  SlotP s;
  s.vec = draft_side ? (const uint16_t*)p.draft + ((int64_t)b * K + i) * p.d_stride
                     : (const uint16_t*)p.target + ((int64_t)b * (K + 1) + i) * p.t_stride;
  // pointers that may be NULL are swapped for a valid dummy before loading
  const float* Tp = p.temperature + b;
  const int32_t* dummy = SHARD ? p.slot_count : (const int32_t*)Tp;
  const int32_t* tokp = p.tokens ? p.tokens + (int64_t)b * K + min(i, K - 1) : dummy;
  const int32_t* kbp = p.k_per_row ? p.k_per_row + b : dummy;
  const float* Pp = p.top_p ? p.top_p + b : Tp;
  const int tok = *tokp, kbl = *kbp;
  const float T = SHARD ? 1.0f : *Tp, Pl = SHARD ? 1.0f : *Pp;
  const int kb = p.k_per_row ? kbl : K;
  s.token = (p.mode == 1 || (!draft_side && i >= kb)) ? -1 : tok;
  s.T = T;
  double P = p.top_p ? (double)Pl : 1.0;
  if (!(P > 0.0)) P = 1.0;  // invalid top-p is flagged by the finalize kernel
  if (draft_side && (p.flags & SV_FLAG_TOPP_TARGET_ONLY)) P = 1.0;
  s.P = P;
  return s;
}

struct Bf16Shared {
  int wmaxpos[kWv], wminneg[kWv];
  uint32_t wtot[kWv], wzero[kWv], wninf[kWv], wflag[kWv], wwrap[kWv];
  int next;
};

// The count table as the streaming loop keeps it: one word per magnitude,
// the count of +v in the low half and of -v in the high half.
struct PackedTable {
  const uint4* hist4;
  // the counts of one sign at the four magnitudes of 16-byte group grp
  __device__ __forceinline__ uint4 counts(int grp, bool pos) const {
    const uint4 g = hist4[grp];
    return pos ? make_uint4(g.x & 0xFFFFu, g.y & 0xFFFFu, g.z & 0xFFFFu, g.w & 0xFFFFu)
               : make_uint4(g.x >> 16, g.y >> 16, g.z >> 16, g.w >> 16);
  }
};

// Level 2 of the top-p search, run by one wave: the 256 magnitudes of bin b
// of one sign, walked from the largest value down.  `above` is the mass of
// all larger values.  Returns the threshold value and the kept mass through
// it (wave-uniform).
template <class Table>
__device__ __forceinline__ void crossing_value(const Table& tab, int b, bool pos, double above,
                                               double target, float m, float c2, float* tau,
                                               double* kept) {
  const int l = threadIdx.x & 63;
  // lanes ascending = values descending: +values from the top magnitude
  // down, -values from the bottom magnitude up
  const int grp = b * 64 + (pos ? 63 - l : l);
  const uint4 g = tab.counts(grp, pos);
  const uint32_t xs[4] = {pos ? g.w : g.x, pos ? g.z : g.y, pos ? g.y : g.z, pos ? g.x : g.w};
  double mass[4];
  uint32_t keys[4];
  double part = 0.0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t word = 4u * (uint32_t)grp + (uint32_t)(pos ? 3 - i : i);
    const uint32_t c = xs[i];
    keys[i] = (word + kBase) | (pos ? 0u : 0x8000u);
    mass[i] = c ? (double)c * weight(bf16f(keys[i]), m, c2) : 0.0;
    part += mass[i];
  }
  const double incl = wave_scan_add_f64(part);
  const uint64_t hit = __ballot(part > 0.0 && above + incl >= target);
  const uint64_t any = __ballot(part > 0.0);
  // the caller's bin has mass, so some lane has; lane 0 if rounding says not
  const int L = hit ? __builtin_ctzll(hit) : any ? 63 - __builtin_clzll(any) : 0;
  // in lane L: the first value whose inclusive mass reaches the target (the
  // last present value if rounding left the target just out of reach)
  double cum = above + (incl - part);
  uint32_t sel = 0xFFFFFFFFu;
  double sel_kept = 0.0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (mass[i] > 0.0) {
      cum += mass[i];
      if (sel == 0xFFFFFFFFu && cum >= target) { sel = keys[i]; sel_kept = cum; }
    }
  }
  if (sel == 0xFFFFFFFFu) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (mass[i] > 0.0) sel = keys[i];
    sel_kept = cum;
  }
  const uint32_t key = (uint32_t)__builtin_amdgcn_readlane((int)sel, L);
  const uint64_t kb = (uint64_t)__double_as_longlong(sel_kept);
  const uint32_t klo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)kb, L);
  const uint32_t khi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(kb >> 32), L);
  *tau = bf16f(key);
  *kept = __longlong_as_double((long long)(((uint64_t)khi << 32) | klo));
}

__device__ __forceinline__ double readlane_f64(double x, int L) {
  const uint64_t b = (uint64_t)__double_as_longlong(x);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, L);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), L);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Level 2 of the top-p search when the crossing lies among the nonzero
// values below the window (one sign), run by one wave on the vector's list
// of them (n entries, n <= kTinyCap, one per lane).  Each lane forms the mass
// of the listed values of its sign that are >= its own (equal values are one
// value); the threshold is the largest value whose inclusive mass reaches
// the target (the smallest present if rounding leaves the target just out
// of reach), as in crossing_value.
__device__ __forceinline__ void tiny_crossing(const uint32_t* tiny, uint32_t n, bool pos,
                                              double above, double target, float m, float c2,
                                              float* tau, double* kept) {
  const int l = threadIdx.x & 63;
  const bool in = (uint32_t)l < n;
  const uint32_t k = tiny[1 + (in ? l : 0)];
  const bool valid = in && (((k & 0x8000u) == 0u) == pos);
  const float v = bf16f(k);
  const double wt = valid ? weight(v, m, c2) : 0.0;
  double ge = 0.0;
  for (int j = 0; j < 64; ++j) {
    const float vj = __shfl(v, j, 64);
    const double wj = __shfl(wt, j, 64);
    ge += vj >= v ? wj : 0.0;  // wj is 0 for lanes outside the bin
  }
  const uint64_t hit = __ballot(valid && above + ge >= target);
  const float cand = hit ? (((hit >> l) & 1u) ? v : -INFINITY) : (valid ? -v : -INFINITY);
  float best = wave_max_f(cand);
  if (!hit) best = -best;
  const uint64_t at = __ballot(valid && v == best);
  const int L = at ? __builtin_ctzll(at) : 0;
  *tau = best;
  *kept = readlane_f64(above + ge, L);
}

// E2 of the epilogue: the masses of the values of each (wave, row) bin --
// wave w with row j owns magnitude bin w + kWv j of both signs, thread t the
// 16-byte groups t + kT j (bit j of gmask: the group holds a count) -- then
// the zero bin and, by the last wave, the listed values below the window.
template <class Table>
__device__ __forceinline__ void bin_masses(const Table& tab, uint32_t gmask, float m, float c2,
                                           uint32_t Z, const uint32_t* tiny, uint32_t NT,
                                           double* bins) {
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
#pragma unroll 1
  for (int j = 0; j < kGpt; ++j) {
    const int g = tid + kT * j;
    const int b = w + kWv * j;
    double mp = 0.0, mn = 0.0;
    if ((gmask >> j) & 1u) {
      const uint4 cp = tab.counts(g, true), cn = tab.counts(g, false);
      const uint32_t ps[4] = {cp.x, cp.y, cp.z, cp.w}, ns[4] = {cn.x, cn.y, cn.z, cn.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t key = 4u * (uint32_t)g + (uint32_t)q + kBase;
        const uint32_t lo = ps[q], hi = ns[q];
        if (lo) mp += (double)lo * weight(bf16f(key), m, c2);
        if (hi) mn += (double)hi * weight(bf16f(key | 0x8000u), m, c2);
      }
    }
    if (__ballot((gmask >> j) & 1u)) {
      mp = wave_last_f64(wave_scan_add_f64(mp));
      mn = wave_last_f64(wave_scan_add_f64(mn));
    }
    if (l == 0) { bins[pos_bin(b)] = mp; bins[neg_bin(b)] = mn; }
  }
  if (tid == 0) bins[kZeroBin] = Z ? (double)Z * weight(0.0f, m, c2) : 0.0;
  if (w == kWv - 1) {  // the listed values below the window, by sign
    double tp = 0.0, tn = 0.0;
    if (NT) {
      const bool has = (uint32_t)l < NT;
      const uint32_t k = tiny[1 + (has ? l : 0)];
      const double wt = has ? weight(bf16f(k), m, c2) : 0.0;
      const bool neg = (k & 0x8000u) != 0u;
      tp = wave_last_f64(wave_scan_add_f64(neg ? 0.0 : wt));
      tn = wave_last_f64(wave_scan_add_f64(neg ? wt : 0.0));
    }
    if (l == 0) { bins[kZeroBin + 1] = tp; bins[kZeroBin - 1] = tn; }
  }
}

// The last step of the epilogue, run by wave 0: S and the top-p threshold in
// two levels (the rank bin holding the crossing, then the value inside it),
// then the record (written by thread 0).  zx is the draft token's logit
// (NaN when the slot verifies none).
template <class Table>
__device__ __forceinline__ void topp_record(const Table& tab, const double* bins,
                                            const uint32_t* tiny, uint32_t NT, bool stats_ok,
                                            double P, float m, float c2, int token, float T,
                                            bool T_ok, int V, uint32_t status, float zx,
                                            VecRec* rec) {
  const int l = threadIdx.x & 63;
  double S = 0.0, kept = 0.0;
  float tau = -INFINITY;
  if (stats_ok) {
    // lane l holds rank bin kRankBins - 1 - l (values descending)
    const int R = kRankBins - 1 - l;
    const double part = R >= 0 ? bins[R] : 0.0;
    const double incl = wave_scan_add_f64(part);
    S = wave_last_f64(incl);
    kept = S;
    if (P < 1.0) {
      const double target = P * S;
      const uint64_t hit = __ballot(part > 0.0 && incl >= target);
      const uint64_t any = __ballot(part > 0.0);
      // S > 0 (the maximum has weight 1), so some lane has mass
      const int L = hit ? __builtin_ctzll(hit) : any ? 63 - __builtin_clzll(any) : 0;
      const int RL = kRankBins - 1 - L;
      const double above = readlane_f64(incl - part, L);
      if (RL == kZeroBin) {
        tau = 0.0f;
        kept = above + readlane_f64(part, L);
      } else if (RL == kZeroBin + 1 || RL == kZeroBin - 1) {
        tiny_crossing(tiny, NT, RL > kZeroBin, above, target, m, c2, &tau, &kept);
      } else if (RL > kZeroBin) {
        crossing_value(tab, RL - kZeroBin - 2, true, above, target, m, c2, &tau, &kept);
      } else if (RL >= 0) {
        crossing_value(tab, kZeroBin - 2 - RL, false, above, target, m, c2, &tau, &kept);
      }
    }
  }
  if (threadIdx.x == 0) write_record(token, T, T_ok, V, m, tau, kept, status, zx, rec);
}


__global__ __launch_bounds__(kT, kWgPerCu) void stats_bf16_kernel(StatsParams p) {
  __shared__ __align__(16) uint32_t hist[kCopies * kCopyWords];
  __shared__ double bins[kRankBins];
  __shared__ Bf16Shared sh;
  __shared__ uint32_t tiny[1 + kTinyCap];  // values below the window: count, then values
  __shared__ double hist256[256];       // generic path
  __shared__ Scratch<kWv> sc;           // generic path
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int V = p.V;
  const int nitems = p.slot_list ? *p.slot_count : unlisted_items(p);
  uint4* hist4 = reinterpret_cast<uint4*>(hist);

  // the first item; a workgroup without one has none later either
  const int queue = (int)(blockIdx.x % kQueues);
  if (queue_item(queue, blockIdx.x / kQueues) >= nitems) return;
  const uint32_t stride = list_stride((uint32_t)nitems);
  int v = item_slot(p, queue_item(queue, blockIdx.x / kQueues), (uint32_t)nitems, stride);
  for (int i = tid; i < kCopies * kCopyWords; i += kT) hist[i] = 0;
  if (tid == 0) tiny[0] = 0u;
  uint32_t* hcopy = hist + (l & 1) * kCopyWords;  // this lane's copy
  const uint4* copy1 = reinterpret_cast<const uint4*>(hist + kCopyWords);
  SlotP cur = slot_params<false>(p, v);

  for (;;) {
    __syncthreads();  // every thread has read sh.next
    // no counters (one vector per workgroup, see launch_stats): no next item
    if (tid == 0) sh.next = p.tickets ? take_ticket(p, queue) : nitems;
    const bool T_ok = cur.T > 0.0f && isfinite(cur.T);
    VecRec* rec = p.recs + v;
    // the draft token's logit, loaded by every thread from one address
    const bool has_zx = cur.token >= 0 && cur.token < V;
    const uint32_t zbits = cur.vec[has_zx ? cur.token : 0];

    Side sd;
    stream_vector<kT>(cur.vec, V, hcopy, tiny, sd, tid);
    {
      const uint32_t z = wave_last_u32(wave_scan_u32<OpAddU32>(sd.nzero));
      const uint32_t n = wave_last_u32(wave_scan_u32<OpAddU32>(sd.nninf));
      const uint32_t f = wave_last_u32(wave_scan_u32<OpOrU32>(sd.flags));
      if (l == 0) { sh.wzero[w] = z; sh.wninf[w] = n; sh.wflag[w] = f; }
    }
    __syncthreads();  // B1: table complete
    const int in = sh.next;
    const bool has_next = in < nitems;
    const int vn = has_next ? item_slot(p, in, (uint32_t)nitems, stride) : v;
    const SlotP nxt = slot_params<false>(p, vn);  // loads in flight meanwhile

    // ---- E1: thread t merges groups t + kT j of the two copies into copy 0
    // and clears copy 1; largest +magnitude, smallest -magnitude present,
    // total count, and whether a merged count passed 16 bits
    uint32_t gmask = 0, total = 0, wrap = 0;
    int maxpos = -1, minneg = 0x7FFFFFFF;
#pragma unroll 1
    for (int j = 0; j < kGpt; ++j) {
      const int g = tid + kT * j;
      const uint4 d0 = hist4[g], d1 = copy1[g];
      // most groups are empty and come in runs: a wave whose groups are
      // all empty has nothing to merge, count or clear
      if (!__any((d0.x | d0.y | d0.z | d0.w | d1.x | d1.y | d1.z | d1.w) != 0u)) continue;
      const uint32_t a0[4] = {d0.x, d0.y, d0.z, d0.w};
      const uint32_t a1[4] = {d1.x, d1.y, d1.z, d1.w};
      uint32_t xs[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t lo = (a0[q] & 0xFFFFu) + (a1[q] & 0xFFFFu);
        const uint32_t hi = (a0[q] >> 16) + (a1[q] >> 16);
        wrap |= (lo | hi) >> 16;
        xs[q] = (hi << 16) | (lo & 0xFFFFu);
        const int word = 4 * g + q;
        total += lo + hi;
        if (lo) maxpos = max(maxpos, word);
        if (hi) minneg = min(minneg, word);
      }
      if (d1.x | d1.y | d1.z | d1.w) {
        hist4[g] = make_uint4(xs[0], xs[1], xs[2], xs[3]);
        reinterpret_cast<uint4*>(hist + kCopyWords)[g] = make_uint4(0u, 0u, 0u, 0u);
      }
      if (xs[0] | xs[1] | xs[2] | xs[3]) gmask |= 1u << j;
    }
    {
      const int a = (int)wave_last_u32(wave_scan_u32<OpMaxI32>((uint32_t)maxpos));
      const int b = (int)wave_last_u32(wave_scan_u32<OpMinI32>((uint32_t)minneg));
      const uint32_t t = wave_last_u32(wave_scan_u32<OpAddU32>(total));
      const uint32_t x = wave_last_u32(wave_scan_u32<OpOrU32>(wrap));
      if (l == 0) { sh.wmaxpos[w] = a; sh.wminneg[w] = b; sh.wtot[w] = t; sh.wwrap[w] = x; }
    }
    __syncthreads();  // B2
    int MP = -1, MN = 0x7FFFFFFF;
    uint32_t TT = 0, Z = 0, NI = 0, FL = 0, WR = 0;
#pragma unroll
    for (int k = 0; k < kWv; ++k) {
      MP = max(MP, sh.wmaxpos[k]);
      MN = min(MN, sh.wminneg[k]);
      TT += sh.wtot[k];
      Z += sh.wzero[k];
      NI += sh.wninf[k];
      FL |= sh.wflag[k];
      WR |= sh.wwrap[k];
    }
    uint32_t status = FL & SV_ROW_NONFINITE_LOGIT;
    const uint32_t NT = tiny[0];
    // a count wrapped 16 bits (65536 equal logits in one copy, or a merged
    // count past 65535), a logit above the window, more values below it than
    // the list holds, or no positive value in the window while some lie
    // below it (the largest logit would be one of them): the generic path
    // redoes the vector
    const bool fallback =
        !status && ((FL & kFallback) || WR || TT + Z + NI + NT != (uint32_t)V ||
                    (MP < 0 && NT > 0));
    if (!fallback && TT + Z == 0) status |= SV_ROW_NO_FINITE;
    const float m = MP >= 0 ? bf16f((uint32_t)MP + kBase)
                  : Z > 0   ? 0.0f
                  : MN < 0x7FFFFFFF ? bf16f(((uint32_t)MN + kBase) | 0x8000u)
                                    : -INFINITY;
    const bool stats_ok = !fallback && !status && T_ok;
    const float c2 = log2e_over_T(cur.T);

    if (stats_ok) bin_masses(PackedTable{hist4}, gmask, m, c2, Z, tiny, NT, bins);
    __syncthreads();  // B3: bins written
    if (w == 0 && !fallback)
      topp_record(PackedTable{hist4}, bins, tiny, NT, stats_ok, cur.P, m, c2, cur.token, cur.T,
                  T_ok, V, status, has_zx ? bf16f(zbits) : __uint_as_float(0x7FC00000u), rec);
    if (fallback) {
      generic_stats<kT>(VecLogits{cur.vec, SV_BF16}, cur.token, cur.T, cur.P, V, hist256, sc,
                        rec);
    }
    __syncthreads();  // B4: the table is no longer read
    if (tid == 0) tiny[0] = 0u;
#pragma unroll 1
    for (int j = 0; j < kGpt; ++j)
      if ((gmask >> j) & 1u) hist4[tid + kT * j] = make_uint4(0u, 0u, 0u, 0u);
    if (!has_next) break;
    v = vn;
    cur = nxt;
  }
}

// ---------------------------------------------------------------- shard pass

// A vocabulary shard is a short vector (V/G columns: 38 KB of bf16 at
// V = 151936 over 8 shards), so a workgroup's per-vector costs -- the first
// loads' latency, the scan of the table, the list and the header -- weigh
// about as much as its streaming.  The shard pass therefore takes two
// vectors per workgroup pass: lanes of even index stream the pair's first
// vector into table 0, lanes of odd index its second into table 1, one copy
// each (so there is no merge; each table gets the lanes of one parity, as
// the two copies of the unsharded kernel do), and waves 0-1 then scan and
// list table 0 while waves 2-3 do table 1.  Work items are pairs of
// consecutive items (the last one may be alone).
constexpr int kHalfT = kT / 2;              // threads per vector while streaming / listing
constexpr int kHalfGpt = kGroups / kHalfT;  // table groups per listing thread
static_assert(kGroups % kHalfT == 0 && kHalfGpt <= 32 && kWv == 4, "pair tiling");

struct PairShared {
  uint32_t wzero[2][kWv], wninf[2][kWv], wflag[2][kWv];  // [vector][wave]: streaming side counts
  int wmaxpos[kWv], wminneg[kWv];                         // [wave]: the table its wave scanned
  uint32_t wtot[kWv], wlist[kWv];
  int slot[2];       // the pair's vectors (slot), -1 for none
  uint32_t zx[2];    // bit 16: the draft token is one of the shard's columns; low 16: its bits
  int next;
};

// The list of one table's nonzero words, its below-window values and its
// header, written by the kHalfT threads (two waves) of that table; the
// block barrier inside is reached by every thread of the workgroup.
__device__ __forceinline__ void pair_emit(const StatsParams& p, int v, const uint4* hist4,
                                          uint32_t gmask, const uint32_t* tiny, uint32_t NT,
                                          uint32_t status, int MP, int MN, uint32_t Z,
                                          uint32_t NI, uint32_t zx, PairShared& sh) {
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int te = tid & (kHalfT - 1), wp = w & ~1;  // index within the pair of waves; its first wave
  uint32_t mine = 0;
#pragma unroll 1
  for (int j = 0; j < kHalfGpt; ++j) {
    if ((gmask >> j) & 1u) {
      const uint4 d = hist4[te + kHalfT * j];
      mine += (d.x != 0u ? 1u : 0u) + (d.y != 0u ? 1u : 0u) + (d.z != 0u ? 1u : 0u) +
              (d.w != 0u ? 1u : 0u);
    }
  }
  const uint32_t incl = wave_scan_u32<OpAddU32>(mine);
  if (l == 63) sh.wlist[w] = incl;
  __syncthreads();
  const uint32_t o0 = incl - mine + (w & 1 ? sh.wlist[wp] : 0u);
  const uint32_t total = sh.wlist[wp] + sh.wlist[wp + 1];
  if (v < 0) return;
  uint8_t* base = p.partial + (int64_t)v * p.part_stride;
  uint2* list = reinterpret_cast<uint2*>(base + kShardListOffset);
  uint32_t o = o0;
#pragma unroll 1
  for (int j = 0; j < kHalfGpt; ++j) {
    if ((gmask >> j) & 1u) {
      const int g = te + kHalfT * j;
      const uint4 d = hist4[g];
      const uint32_t xs[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (xs[q]) list[o++] = make_uint2(4u * (uint32_t)g + (uint32_t)q, xs[q]);
    }
  }
  uint32_t* tl = reinterpret_cast<uint32_t*>(base + sizeof(ShardHead));
  if ((uint32_t)te < min(NT, (uint32_t)kShardTinyCap)) tl[te] = tiny[1 + te];
  if (te == 0) {
    ShardHead hd;
    hd.status = status;
    hd.maxpos = MP;
    hd.minneg = MN;
    hd.zeros = Z;
    hd.ninf = NI;
    hd.ntiny = NT;
    hd.nlist = total;
    hd.zx = zx;
    *reinterpret_cast<ShardHead*>(base) = hd;
  }
}

__global__ __launch_bounds__(kT, kWgPerCu) void shard_pair_kernel(StatsParams p) {
  __shared__ __align__(16) uint32_t hist[kCopies * kCopyWords];  // table h at h * kCopyWords
  __shared__ uint32_t tiny[2][1 + kTinyCap];
  __shared__ PairShared sh;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int h = l & 1;          // the vector this lane streams
  const int tv = tid >> 1;      // its index among that vector's threads
  const int eh = w >> 1;        // the table this thread scans and lists
  const int te = tid & (kHalfT - 1);
  const int V = p.V;
  const int nitems = p.slot_list ? *p.slot_count : unlisted_items(p);
  const int npairs = (nitems + 1) >> 1;
  const int queue = (int)(blockIdx.x % kQueues);
  int pr = queue_item(queue, blockIdx.x / kQueues);
  if (pr >= npairs) return;
  const uint32_t stride = list_stride((uint32_t)nitems);
  for (int i = tid; i < kCopies * kCopyWords; i += kT) hist[i] = 0;
  if (tid < 2) tiny[tid][0] = 0u;
  uint32_t* const ht = hist + h * kCopyWords;           // streamed by this lane
  const uint4* const et = reinterpret_cast<const uint4*>(hist + eh * kCopyWords);  // scanned
  // this lane's vector of pair pr: slot, logits (slot 0's when the pair has
  // no second vector, which is then not streamed) and the draft token
  auto lane_vec = [&](int pair, int& slot, SlotP& sp) {
    const int item = 2 * pair + h;
    slot = item < nitems ? item_slot(p, item, (uint32_t)nitems, stride) : -1;
    sp = slot_params<true>(p, slot >= 0 ? slot : 0);
  };
  int slot;
  SlotP cur;
  lane_vec(pr, slot, cur);

  for (;;) {
    __syncthreads();  // every thread has read the previous pass's shared figures
    if (tid == 0) sh.next = take_ticket(p, queue);
    if (tid < 2) {  // lanes 0 and 1 of wave 0: the pair's two vectors
      const int tokl = cur.token - p.col_off;
      const bool has_zx = slot >= 0 && cur.token >= 0 && tokl >= 0 && tokl < V;
      sh.slot[h] = slot;
      sh.zx[h] = has_zx ? (1u << 16) | (uint32_t)cur.vec[tokl] : 0u;
    }
    Side sd;
    stream_vector<kHalfT>(cur.vec, slot >= 0 ? V : 0, ht, tiny[h], sd, tv);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const uint32_t z = wave_last_u32(wave_scan_u32<OpAddU32>(h == q ? sd.nzero : 0u));
      const uint32_t n = wave_last_u32(wave_scan_u32<OpAddU32>(h == q ? sd.nninf : 0u));
      const uint32_t f = wave_last_u32(wave_scan_u32<OpOrU32>(h == q ? sd.flags : 0u));
      if (l == 0) { sh.wzero[q][w] = z; sh.wninf[q][w] = n; sh.wflag[q][w] = f; }
    }
    __syncthreads();  // B1: both tables complete
    const int in = sh.next;
    const bool has_next = in < npairs;
    int nslot = slot;
    SlotP nxt = cur;
    if (has_next) lane_vec(in, nslot, nxt);  // loads in flight meanwhile

    // scan of table eh by its two waves: groups te + kHalfT j
    uint32_t gmask = 0, total = 0;
    int maxpos = -1, minneg = 0x7FFFFFFF;
#pragma unroll 1
    for (int j = 0; j < kHalfGpt; ++j) {
      const uint4 d = et[te + kHalfT * j];
      if (!__any((d.x | d.y | d.z | d.w) != 0u)) continue;
      const uint32_t a[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t lo = a[q] & 0xFFFFu, hi = a[q] >> 16;
        const int word = 4 * (te + kHalfT * j) + q;
        total += lo + hi;
        if (lo) maxpos = max(maxpos, word);
        if (hi) minneg = min(minneg, word);
      }
      if (d.x | d.y | d.z | d.w) gmask |= 1u << j;
    }
    {
      const int a = (int)wave_last_u32(wave_scan_u32<OpMaxI32>((uint32_t)maxpos));
      const int b = (int)wave_last_u32(wave_scan_u32<OpMinI32>((uint32_t)minneg));
      const uint32_t t = wave_last_u32(wave_scan_u32<OpAddU32>(total));
      if (l == 0) { sh.wmaxpos[w] = a; sh.wminneg[w] = b; sh.wtot[w] = t; }
    }
    __syncthreads();  // B2
    const int wp = 2 * eh;
    const int MP = max(sh.wmaxpos[wp], sh.wmaxpos[wp + 1]);
    const int MN = min(sh.wminneg[wp], sh.wminneg[wp + 1]);
    const uint32_t TT = sh.wtot[wp] + sh.wtot[wp + 1];
    uint32_t Z = 0, NI = 0, FL = 0;
#pragma unroll
    for (int k = 0; k < kWv; ++k) {
      Z += sh.wzero[eh][k];
      NI += sh.wninf[eh][k];
      FL |= sh.wflag[eh][k];
    }
    const uint32_t NT = tiny[eh][0];
    // a count that wrapped 16 bits, a logit above the window, or more values
    // below it than the list holds: the merge redoes the vector
    const bool over = (FL & kFallback) || TT + Z + NI + NT != (uint32_t)V;
    const uint32_t status = (FL & SV_ROW_NONFINITE_LOGIT) | (over ? kShardFallback : 0u);
    pair_emit(p, sh.slot[eh], et, gmask, tiny[eh], NT, status, MP, MN, Z, NI, sh.zx[eh], sh);
    __syncthreads();  // B3: the tables are no longer read
    if (te == 0) tiny[eh][0] = 0u;
    uint4* const et_w = reinterpret_cast<uint4*>(hist + eh * kCopyWords);
#pragma unroll 1
    for (int j = 0; j < kHalfGpt; ++j)
      if ((gmask >> j) & 1u) et_w[te + kHalfT * j] = make_uint4(0u, 0u, 0u, 0u);
    if (!has_next) break;
    pr = in;
    slot = nslot;
    cur = nxt;
  }
}

// ---------------------------------------------------------------- shards

static_assert(kWords == kTableWords && kTinyCap == kShardTinyCap, "shard partial layout");

// The merged table of the combine: one 32-bit count per magnitude and sign
// (a merged count may pass 16 bits).
struct SplitTable {
  const uint4* pos4;
  const uint4* neg4;
  __device__ __forceinline__ uint4 counts(int grp, bool pos) const {
    return pos ? pos4[grp] : neg4[grp];
  }
};

// The logits of one vector held as the shards' column slices, for
// generic_stats (a vector the merged table cannot hold).
struct SliceLogits {
  const CombineParams& cp;
  int64_t idx;  // vector index: b (k+1) + i on the target side, b k + i on the draft side
  bool draft;
  __device__ __forceinline__ float operator()(int64_t j) const {
    int g = 0;
    while (g + 1 < cp.G && j >= cp.col_off[g + 1]) ++g;
    const uint16_t* vec = draft ? cp.dft[g] + idx * cp.ds[g] : cp.tgt[g] + idx * cp.ts[g];
    return __uint_as_float((uint32_t)vec[j - cp.col_off[g]] << 16);
  }
};

// One workgroup per vector slot: the G shards' partials merged into one
// count table (integer adds, exact), the zeros, -infs and values below the
// window gathered in shard order, then the same epilogue as the unsharded
// pass -- bin masses, S, the tie-closed top-p threshold, p'(x) -- so the
// record is the one the unsharded pass writes for the concatenated vector.
// A vector whose counts the table cannot hold is redone from the shards'
// logits by the generic path.
__global__ __launch_bounds__(kT, kWgPerCu) void shard_combine_kernel(CombineParams cp) {
  __shared__ __align__(16) uint32_t cpos[kWords];
  __shared__ __align__(16) uint32_t cneg[kWords];
  __shared__ double bins[kRankBins];
  __shared__ uint32_t tiny[1 + kTinyCap];
  __shared__ __align__(16) ShardHead heads[kMaxShards];
  __shared__ uint32_t lstart[kMaxShards + 1], tstart[kMaxShards + 1];
  __shared__ const uint2* lbase[kMaxShards];
  __shared__ double hist256[256];
  __shared__ Scratch<kWv> sc;
  const StatsParams& p = cp.sp;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int v = blockIdx.x;
  const int G = cp.G;
  // the shards' headers load while the slot's parameters do (a slot the
  // call does not use has no partial: its header is read, not used)
  uint4 h0 = make_uint4(0u, 0u, 0u, 0u), h1 = h0;  // ShardHead as two 16-byte words
  if (tid < G) {
    const uint4* hp = reinterpret_cast<const uint4*>(cp.part[tid] + (int64_t)v * cp.part_stride[tid]);
    h0 = hp[0];
    h1 = hp[1];
  }
  const Slot s = slot_of(p, SV_BF16, v);
  if (!s.needed) return;
  uint4* pos4 = reinterpret_cast<uint4*>(cpos);
  uint4* neg4 = reinterpret_cast<uint4*>(cneg);
  for (int i = tid; i < kGroups; i += kT) {
    pos4[i] = make_uint4(0u, 0u, 0u, 0u);
    neg4[i] = make_uint4(0u, 0u, 0u, 0u);
  }
  if (tid < G) {
    reinterpret_cast<uint4*>(heads + tid)[0] = h0;
    reinterpret_cast<uint4*>(heads + tid)[1] = h1;
    lstart[tid + 1] = min(h1.z, (uint32_t)shard_list_cap(cp.col_len[tid]));  // nlist
    tstart[tid + 1] = min(h1.y, (uint32_t)kShardTinyCap);                    // ntiny
    lbase[tid] = reinterpret_cast<const uint2*>(cp.part[tid] + (int64_t)v * cp.part_stride[tid] +
                                                kShardListOffset);
  }
  if (tid == 0) lstart[0] = tstart[0] = 0u;
  __syncthreads();
  if (tid == 0)
    for (int g = 0; g < G; ++g) {
      lstart[g + 1] += lstart[g];
      tstart[g + 1] += tstart[g];
    }
  __syncthreads();
  // all shards' lists as one range of entries, eight per thread in flight
  // before their adds (entry e is entry e - lstart[g] of shard g)
  const uint32_t nent = lstart[G];
  constexpr int kUnroll = 8;
  for (uint32_t e0 = (uint32_t)tid; e0 < nent; e0 += kUnroll * kT) {
    uint2 x[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint32_t e = e0 + (uint32_t)(u * kT);
      x[u] = make_uint2((uint32_t)kWords, 0u);
      if (e < nent) {
        int g = 0;
        while (g + 1 < G && e >= lstart[g + 1]) ++g;
        x[u] = lbase[g][e - lstart[g]];
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (x[u].x < (uint32_t)kWords) {
        const uint32_t lo = x[u].y & 0xFFFFu, hi = x[u].y >> 16;
        if (lo)
          __hip_atomic_fetch_add(cpos + x[u].x, lo, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        if (hi)
          __hip_atomic_fetch_add(cneg + x[u].x, hi, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      }
    }
  }
  uint32_t st = 0, Z = 0, NT = 0;
  int MP = -1, MN = 0x7FFFFFFF;
  for (int g = 0; g < G; ++g) {
    const ShardHead& hg = heads[g];
    st |= hg.status;
    Z += hg.zeros;
    NT += hg.ntiny;
    MP = max(MP, hg.maxpos);
    MN = min(MN, hg.minneg);
  }
  // the values below the window, in shard order: lane l takes entry l of
  // the concatenated lists (one load each)
  const uint32_t ntl = tstart[G];
  if (w == 0 && ntl > 0 && (uint32_t)l < min(ntl, (uint32_t)kTinyCap)) {
    int g = 0;
    while (g + 1 < G && (uint32_t)l >= tstart[g + 1]) ++g;
    const uint32_t* t = reinterpret_cast<const uint32_t*>(
        cp.part[g] + (int64_t)v * cp.part_stride[g] + sizeof(ShardHead));
    tiny[1 + l] = t[l - tstart[g]];
  }
  __syncthreads();
  uint32_t gmask = 0;
#pragma unroll 1
  for (int j = 0; j < kGpt; ++j) {
    const uint4 a = pos4[tid + kT * j], b = neg4[tid + kT * j];
    if (a.x | a.y | a.z | a.w | b.x | b.y | b.z | b.w) gmask |= 1u << j;
  }
  uint32_t status = st & SV_ROW_NONFINITE_LOGIT;
  // a shard the table could not hold, more values below the window than
  // the list holds, or no positive value in the window while some lie
  // below it: the generic path over the shards' logits
  const bool fallback = !status && ((st & kShardFallback) || NT > (uint32_t)kTinyCap ||
                                    (MP < 0 && NT > 0));
  if (!fallback && MP < 0 && MN == 0x7FFFFFFF && Z == 0) status |= SV_ROW_NO_FINITE;
  const float m = MP >= 0 ? bf16f((uint32_t)MP + kBase)
                : Z > 0   ? 0.0f
                : MN < 0x7FFFFFFF ? bf16f(((uint32_t)MN + kBase) | 0x8000u)
                                  : -INFINITY;
  const bool stats_ok = !fallback && !status && s.T_ok;
  const float c2 = log2e_over_T(s.T);
  const SplitTable tab{pos4, neg4};
  if (stats_ok) bin_masses(tab, gmask, m, c2, Z, tiny, NT, bins);
  __syncthreads();
  VecRec* rec = p.recs + v;
  if (w == 0 && !fallback) {
    // the draft token's logit, from the shard that holds its column
    float zx = __uint_as_float(0x7FC00000u);
    if (s.token >= 0 && s.token < p.V) {
      int g = 0;
      while (g + 1 < G && s.token >= cp.col_off[g + 1]) ++g;
      if ((heads[g].zx >> 16) & 1u) zx = bf16f(heads[g].zx & 0xFFFFu);
    }
    topp_record(tab, bins, tiny, NT, stats_ok, s.P, m, c2, s.token, s.T, s.T_ok, p.V, status, zx,
                rec);
  }
  if (fallback) {
    const int per = slots_per_row(p.K), b = v / per, j = v % per;
    const bool draft = j > p.K;
    const int64_t idx = draft ? (int64_t)b * p.K + (j - p.K - 1) : (int64_t)b * (p.K + 1) + j;
    generic_stats<kT>(SliceLogits{cp, idx, draft}, s.token, s.T, s.P, p.V, hist256, sc, rec);
  }
}

// Runs before the bf16 stats kernel, one workgroup.  Counter q starts at the
// number of workgroups serving queue q (their first tickets are taken
// without it).  With a slot list, rows are numbered in tiles of kPlanT: a
// block-wide exclusive scan of each row's slot count gives its place in the
// list, and the row writes its slots there in slot order (target positions
// 0..k_b, then draft positions 0..k_b - 1; draft positions only when
// sampling drafts).  A row with k_b outside [1, K] lists nothing.
constexpr int kPlanT = 1024;

__global__ __launch_bounds__(kPlanT) void stats_plan_kernel(StatsParams p, uint32_t grid) {
  __shared__ uint32_t wsum[kPlanT / 64];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  if (tid < kQueues)
    p.tickets[tid * kQueueStride] = grid > (uint32_t)tid ? (grid - tid + kQueues - 1) / kQueues : 0u;
  if (!p.slot_list) return;
  const int K = p.K, per = slots_per_row(K);
  uint32_t carry = 0;
  for (int b0 = 0; b0 < p.B; b0 += kPlanT) {
    const int b = b0 + tid;
    const int kb = b < p.B ? (p.k_per_row ? p.k_per_row[b] : K) : 0;
    const bool ok = b < p.B && kb >= 1 && kb <= K;
    const uint32_t n = ok ? (p.mode == 1 ? (uint32_t)kb : 2u * (uint32_t)kb + 1u) : 0u;
    const uint32_t incl = wave_scan_u32<OpAddU32>(n);
    if (l == 63) wsum[w] = incl;
    __syncthreads();
    uint32_t before = carry, total = carry;
#pragma unroll
    for (int k = 0; k < kPlanT / 64; ++k) {
      before += k < w ? wsum[k] : 0u;
      total += wsum[k];
    }
    __syncthreads();  // wsum is rewritten by the next tile
    int32_t* out = p.slot_list + before + (incl - n);
    const int s0 = b * per;
    if (ok) {
      int o = 0;
      if (p.mode != 1)
        for (int j = 0; j <= kb; ++j) out[o++] = s0 + j;
      for (int i = 0; i < kb; ++i) out[o++] = s0 + K + 1 + i;
    }
    carry = total;
  }
  if (tid == 0) *p.slot_count = (int32_t)carry;
}

}  // namespace

size_t stats_ticket_bytes() { return (size_t)kQueues * kQueueStride * sizeof(uint32_t); }

size_t stats_plan_bytes(int32_t B, int32_t K) {
  const size_t nslots = (size_t)(B > 0 ? B : 0) * (size_t)slots_per_row(K);
  const size_t tickets = (stats_ticket_bytes() + 255) / 256 * 256;
  const size_t list = (64 * sizeof(int32_t) + nslots * sizeof(int32_t) + 255) / 256 * 256;
  return tickets + list;
}

hipError_t launch_stats(const StatsParams& p, int dtype, int num_cus, hipStream_t s, Timer* t) {
  const unsigned nslots = (unsigned)p.B * (unsigned)slots_per_row(p.K);
  if (nslots == 0) return hipSuccess;
  if (dtype == SV_BF16) {
    const unsigned cus = num_cus > 0 ? (unsigned)num_cus : 256u;
    // every queue needs a workgroup: at least kQueues of them (or one per
    // vector); extra workgroups simply wait for a free CU
    unsigned want = cus * (unsigned)kWgPerCu;
    if (want < (unsigned)kQueues) want = (unsigned)kQueues;
    const unsigned items = p.slot_list ? nslots : (unsigned)unlisted_items(p);
    if (items == 0) return hipSuccess;
    const unsigned grid = items < want ? items : want;
    // With every slot in use and no more slots than workgroups, each
    // workgroup's first vector (its own index) is the whole schedule: no
    // queue counters to arm, no plan launch.
    StatsParams q = p;
    if (!p.slot_list && items <= want) {
      q.tickets = nullptr;
    } else {
      TimedScope ts(t, "stats_plan", s);
      hipLaunchKernelGGL(stats_plan_kernel, dim3(1), dim3(kPlanT), 0, s, p, grid);
    }
    // timed by events attached to the dispatch, which bound the kernel's
    // execution as a kernel trace does
    hipEvent_t e0, e1;
    if (t && t->pair("stats_bf16", &e0, &e1))
      hipExtLaunchKernelGGL(stats_bf16_kernel, dim3(grid), dim3(kT), 0, s, e0, e1, 0u, q);
    else
      hipLaunchKernelGGL(stats_bf16_kernel, dim3(grid), dim3(kT), 0, s, q);
  } else {
    TimedScope ts(t, "stats_generic", s);
    if (dtype == SV_FP32 && p.V <= kGenThreads * kGenHeld)
      hipLaunchKernelGGL(stats_generic_kernel<true>, dim3(nslots), dim3(kGenThreads), 0, s, p,
                         dtype);
    else
      hipLaunchKernelGGL(stats_generic_kernel<false>, dim3(nslots), dim3(kGenThreads), 0, s, p,
                         dtype);
  }
  return hipGetLastError();
}

hipError_t launch_shard_stats(const StatsParams& p, int num_cus, hipStream_t s, Timer* t) {
  const unsigned nslots = (unsigned)p.B * (unsigned)slots_per_row(p.K);
  if (nslots == 0) return hipSuccess;
  const unsigned cus = num_cus > 0 ? (unsigned)num_cus : 256u;
  unsigned want = cus * (unsigned)kWgPerCu;
  if (want < (unsigned)kQueues) want = (unsigned)kQueues;
  // work items are pairs of vectors (of the listed slots when there is a
  // list, which holds at most nslots)
  const unsigned npairs = (nslots + 1) / 2;
  const unsigned grid = npairs < want ? npairs : want;
  {
    TimedScope ts(t, "stats_plan", s);
    hipLaunchKernelGGL(stats_plan_kernel, dim3(1), dim3(kPlanT), 0, s, p, grid);
  }
  TimedScope ts(t, "shard_stats", s);
  hipLaunchKernelGGL(shard_pair_kernel, dim3(grid), dim3(kT), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_shard_combine(const CombineParams& p, hipStream_t s, Timer* t) {
  const unsigned nslots = (unsigned)p.sp.B * (unsigned)slots_per_row(p.sp.K);
  if (nslots == 0) return hipSuccess;
  TimedScope ts(t, "shard_combine", s);
  hipLaunchKernelGGL(shard_combine_kernel, dim3(nslots), dim3(kT), 0, s, p);
  return hipGetLastError();
}

}  // namespace sv
