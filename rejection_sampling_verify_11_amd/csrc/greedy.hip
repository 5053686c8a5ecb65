// Greedy branch of the verification step ([SSD] §2.4, §5.2): with no
// sampling, a draft token is accepted iff it equals the target's argmax at
// that position, and the first mismatch emits the target's argmax.  The
// page asks for this to be its own code path, and here it is: raw logits,
// no temperature, no top-p, lowest index on ties.
//
// Kernel 1 splits every vector into chunks of kGreedyChunk logits and writes
// (max value, first index, flags) per chunk.  For bf16 vectors on 16-byte
// boundaries with V a multiple of 8 (the usual case) a persistent grid of
// waves streams the chunks, a whole chunk per wave -- each lane issues its
// eight 16-byte loads, then the wave reduces with shuffles alone (no LDS, no
// barrier) -- and takes the next chunk; other layouts take a workgroup of
// 256 threads per chunk.  Kernel 2 runs one wave per row: lane i folds the
// chunks of position i (target, and draft when draft logits are given), and
// a ballot finds the first mismatch.
//
// One launch instead of two, for callers that keep a zeroed state buffer
// (argmax_fused_kernel): the streaming grid publishes each chunk's maximum
// into its vector's slot with a device-scope atomic max on a packed
// (order key, -index) word, then counts the chunk for its row; the row's
// last chunk reads the row's slots, decides the row and zeroes its state.
// Device-scope atomics are performed where every XCD sees them, and a
// chunk counts only once its maximum's atomic has returned, so the last
// chunk finds every maximum in place without a cache write-back.  Items are
// taken chunk-major (every vector's chunk 0, then chunk 1, ...) so that the
// chunks in flight at once belong to many vectors and rows: their atomics
// do not queue on one address.
#include <math.h>

#include "sv_internal.h"

namespace sv {
namespace {

constexpr int kThreads = 256;
constexpr int kPerThread = kGreedyChunk / kThreads;  // 16 logits
constexpr int kLoads = kPerThread / 8;               // 16-byte loads per thread
constexpr int kLaneLoads = kGreedyChunk / 8 / 64;    // 8: a wave's loads per lane and chunk
constexpr int kStreamWgPerCu = 4;                    // workgroups of the streaming grid per CU
constexpr int kFusedWgPerCu = 5;                     // workgroups of the one-launch grid per CU

// (v, i) beats (bv, bi): larger value, or equal value with a lower index.
__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return i >= 0 && (bi < 0 || v > bv || (v == bv && i < bi));
}

// Order keys of the two bf16 logits of a 32-bit word, per 16-bit half:
// h | 0x8000 for a +value, ~h for a -value, so that a larger float has a
// larger unsigned key (-inf 0x007F, -0 0x7FFF, +0 0x8000, +inf 0xFF80; a
// +NaN lies above +inf, a -NaN below -inf).
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef short s16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ u16x2 order_keys(uint32_t w) {
  const s16x2 h = __builtin_bit_cast(s16x2, w);
  const s16x2 neg = h >> (short)15;  // all ones in a half that holds a -value
  const uint32_t m = __builtin_bit_cast(uint32_t, neg) & 0x7FFF7FFFu;
  return __builtin_bit_cast(u16x2, w ^ m ^ 0x80008000u);
}
__device__ __forceinline__ uint32_t key_of(uint32_t h) {  // one half
  return (h & 0x8000u) ? (~h & 0xFFFFu) : (h | 0x8000u);
}
__device__ __forceinline__ float value_of_key(uint32_t k) {
  const uint32_t h = (k & 0x8000u) ? (k & 0x7FFFu) : (~k & 0xFFFFu);
  return __uint_as_float(h << 16);
}
// Keys of equal floats: the two zeros are one value.
__device__ __forceinline__ bool same_value(uint32_t k, uint32_t kmax) {
  const bool zero = kmax == 0x8000u || kmax == 0x7FFFu;
  return zero ? (k == 0x8000u || k == 0x7FFFu) : k == kmax;
}
constexpr uint32_t kKeyNegInf = 0x007Fu, kKeyPosInf = 0xFF80u;

__global__ __launch_bounds__(kThreads) void argmax_chunks_kernel(GreedyParams p) {
  const int nch = greedy_chunks(p.V);
  const int nvec_t = p.B * (p.K + 1);
  const int v = blockIdx.x / nch, c = blockIdx.x % nch;
  int b, pos;
  bool draft_side;
  if (v < nvec_t) { b = v / (p.K + 1); pos = v % (p.K + 1); draft_side = false; }
  else { b = (v - nvec_t) / p.K; pos = (v - nvec_t) % p.K; draft_side = true; }
  const int kb = p.k_per_row ? p.k_per_row[b] : p.K;
  if (kb < 1 || kb > p.K) return;
  if (draft_side ? pos >= kb : pos > kb) return;
  const size_t esz = p.dtype == SV_BF16 ? 2 : 4;
  const char* vec = draft_side
      ? (const char*)p.draft + ((int64_t)b * p.K + pos) * p.d_stride * esz
      : (const char*)p.target + ((int64_t)b * (p.K + 1) + pos) * p.t_stride * esz;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int64_t c0 = (int64_t)c * kGreedyChunk;
  const int n = (int)min((int64_t)kGreedyChunk, (int64_t)p.V - c0);
  __shared__ float sv_[kThreads / 64];
  __shared__ int si_[kThreads / 64];
  __shared__ uint32_t sf_[kThreads / 64];

  float bv = -INFINITY;
  int bi = -1;
  uint32_t fl = 0;
  const bool aligned = ((((uintptr_t)vec) + c0 * esz) & 15u) == 0;
  if (p.dtype == SV_BF16 && aligned && n == kGreedyChunk) {
    // Full bf16 chunk: the largest order key with packed 16-bit max/min over
    // the thread's 64 logits, the chunk's largest key by a block max, then
    // the first index holding it, searched only by the threads that hold it.
    const uint16_t* base = (const uint16_t*)vec + c0;
    uint4 d[kLoads];
#pragma unroll
    for (int j = 0; j < kLoads; ++j) d[j] = *(const uint4*)(base + 8 * (tid + kThreads * j));
    u16x2 kmax = {0, 0}, kmin = {0xFFFF, 0xFFFF};
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
      const uint32_t ws[4] = {d[j].x, d[j].y, d[j].z, d[j].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const u16x2 k = order_keys(ws[q]);
        kmax = __builtin_elementwise_max(kmax, k);
        kmin = __builtin_elementwise_min(kmin, k);
      }
    }
    uint32_t tmax = max((uint32_t)kmax.x, (uint32_t)kmax.y);
    uint32_t tmin = min((uint32_t)kmin.x, (uint32_t)kmin.y);
    const uint32_t t0 = tmax;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      tmax = max(tmax, (uint32_t)__shfl_xor((int)tmax, o, 64));
      tmin = min(tmin, (uint32_t)__shfl_xor((int)tmin, o, 64));
    }
    if (l == 0) { si_[w] = (int)tmax; sf_[w] = tmin; }
    __syncthreads();
    uint32_t cmax = 0, cmin = 0xFFFFu;
#pragma unroll
    for (int k = 0; k < kThreads / 64; ++k) {
      cmax = max(cmax, (uint32_t)si_[k]);
      cmin = min(cmin, sf_[k]);
    }
    __syncthreads();  // si_ and sf_ are reused below
    // flags: +inf or a NaN above +inf, a NaN below -inf; a finite value
    // exists if the largest key is finite
    if (cmax >= kKeyPosInf || cmin < kKeyNegInf) fl |= SV_ROW_NONFINITE_LOGIT;
    if (cmax > kKeyNegInf && cmax < kKeyPosInf) fl |= kSawFinite;
    if (same_value(t0, cmax)) {  // this thread holds the chunk's largest value
      int first = 0x7FFFFFFF;
#pragma unroll
      for (int j = 0; j < kLoads; ++j) {
        const uint32_t ws[4] = {d[j].x, d[j].y, d[j].z, d[j].w};
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const uint32_t h = t & 1 ? ws[t >> 1] >> 16 : ws[t >> 1] & 0xFFFFu;
          const int idx = (int)(c0 + 8 * (tid + kThreads * j) + t);
          first = same_value(key_of(h), cmax) ? min(first, idx) : first;
        }
      }
      bi = first;
      bv = value_of_key(cmax);
    }
  } else if (p.dtype == SV_BF16 && aligned) {
    const uint16_t* base = (const uint16_t*)vec + c0;
    const int n8 = n >> 3;
    // thread t reads 16-byte groups t, t+256, ... : increasing index order;
    // all loads first (indices past the end clamp to group 0 and are skipped)
    uint4 d[kLoads];
#pragma unroll
    for (int j = 0; j < kLoads; ++j) d[j] = make_uint4(0u, 0u, 0u, 0u);
    if (n8 > 0) {  // a chunk shorter than one group has only its tail loop
#pragma unroll
      for (int j = 0; j < kLoads; ++j) {
        const int g = tid + kThreads * j;
        d[j] = *(const uint4*)(base + 8 * (g < n8 ? g : 0));
      }
    }
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
      const int g = tid + kThreads * j;
      const bool valid = g < n8;
      const uint32_t w4[4] = {d[j].x, d[j].y, d[j].z, d[j].w};
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const float z = __uint_as_float(t & 1 ? (w4[t >> 1] & 0xFFFF0000u) : (w4[t >> 1] << 16));
        const bool bad = isnan(z) || z == INFINITY;
        fl |= valid && bad ? (uint32_t)SV_ROW_NONFINITE_LOGIT : 0u;
        fl |= valid && !bad && z > -INFINITY ? kSawFinite : 0u;
        const bool take = valid && (z > bv || (bi < 0 && z == -INFINITY));
        bv = take ? z : bv;
        bi = take ? (int)(c0 + 8 * g + t) : bi;
      }
    }
    for (int j = (n8 << 3) + tid; j < n; j += kThreads) {
      const float z = __uint_as_float((uint32_t)base[j] << 16);
      if (isnan(z) || z == INFINITY) fl |= SV_ROW_NONFINITE_LOGIT;
      else if (z > -INFINITY) fl |= kSawFinite;
      if (z > bv || (bi < 0 && z == -INFINITY)) { bv = z; bi = (int)(c0 + j); }
    }
  } else {
    for (int j = tid; j < n; j += kThreads) {
      const float z = p.dtype == SV_BF16
          ? __uint_as_float((uint32_t)((const uint16_t*)vec)[c0 + j] << 16)
          : ((const float*)vec)[c0 + j];
      if (isnan(z) || z == INFINITY) fl |= SV_ROW_NONFINITE_LOGIT;
      else if (z > -INFINITY) fl |= kSawFinite;
      if (z > bv || (bi < 0 && z == -INFINITY)) { bv = z; bi = (int)(c0 + j); }
    }
  }
  // wave then block reduction on (value desc, index asc)
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(bv, o, 64);
    const int oi = __shfl_xor(bi, o, 64);
    fl |= __shfl_xor(fl, o, 64);
    if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
  }
  if (l == 0) { sv_[w] = bv; si_[w] = bi; sf_[w] = fl; }
  __syncthreads();
  if (tid == 0) {
    for (int k = 1; k < kThreads / 64; ++k) {
      if (better(sv_[k], si_[k], bv, bi)) { bv = sv_[k]; bi = si_[k]; }
      fl |= sf_[k];
    }
    ArgmaxPart r;
    r.value = bv;
    r.index = bi;
    r.status = fl;
    r.pad = 0;
    p.parts[blockIdx.x] = r;
  }
}

// The vector a chunk item belongs to: target vectors (b, pos) first, then
// draft vectors; false when the row does not use it (k_b invalid, or a
// position past k_b).
__device__ __forceinline__ bool chunk_vector(const GreedyParams& p, int v, const uint16_t** vec) {
  const int nvec_t = p.B * (p.K + 1);
  int b, pos;
  bool draft_side;
  if (v < nvec_t) { b = v / (p.K + 1); pos = v % (p.K + 1); draft_side = false; }
  else { b = (v - nvec_t) / p.K; pos = (v - nvec_t) % p.K; draft_side = true; }
  const int kb = p.k_per_row ? p.k_per_row[b] : p.K;
  if (kb < 1 || kb > p.K || (draft_side ? pos >= kb : pos > kb)) return false;
  *vec = draft_side ? (const uint16_t*)p.draft + ((int64_t)b * p.K + pos) * p.d_stride
                    : (const uint16_t*)p.target + ((int64_t)b * (p.K + 1) + pos) * p.t_stride;
  return true;
}

// Streams chunk items (vector-major), one wave per chunk at a time; items
// wave, wave + waves, ... of the persistent grid.  bf16, every vector on a
// 16-byte boundary, V a multiple of 8.  Lane l holds the 16-byte groups
// l + 64 j of the chunk (j < 8), so each load instruction reads 1 KB of
// consecutive logits; a group past the chunk's end (last chunk of a vector)
// is loaded clamped and left out.
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, kStreamWgPerCu)))
void argmax_stream_kernel(GreedyParams p, int nitems) {
  const int l = threadIdx.x & 63;
  const int waves = gridDim.x * (kThreads / 64);
  const int nch = greedy_chunks(p.V);
  const int n8v = p.V >> 3;  // 16-byte groups per vector
  for (int item = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6); item < nitems; item += waves) {
    const int v = item / nch, c = item % nch;
    const uint16_t* vec;
    if (!chunk_vector(p, v, &vec)) continue;  // wave-uniform
    const int g0 = c * (kGreedyChunk / 8);
    const int n8 = min(kGreedyChunk / 8, n8v - g0);
    const uint4* body = (const uint4*)vec + g0;
    uint4 d[kLaneLoads];
#pragma unroll
    for (int j = 0; j < kLaneLoads; ++j) d[j] = body[min(l + 64 * j, n8 - 1)];
    // the largest and smallest order key of each load's eight logits
    uint32_t jmax[kLaneLoads];
    u16x2 kmin = {0xFFFF, 0xFFFF};
#pragma unroll
    for (int j = 0; j < kLaneLoads; ++j) {
      const bool valid = l + 64 * j < n8;
      const uint32_t ws[4] = {d[j].x, d[j].y, d[j].z, d[j].w};
      u16x2 m = {0, 0};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const u16x2 k = order_keys(ws[q]);
        m = __builtin_elementwise_max(m, k);
        kmin = __builtin_elementwise_min(kmin, k);
      }
      // a clamped load repeats the chunk's last group: harmless for the
      // minimum, and kept out of the maximum (and so of the search)
      jmax[j] = valid ? max((uint32_t)m.x, (uint32_t)m.y) : 0u;
    }
    uint32_t cmax = 0;
#pragma unroll
    for (int j = 0; j < kLaneLoads; ++j) cmax = max(cmax, jmax[j]);
    uint32_t cmin = min((uint32_t)kmin.x, (uint32_t)kmin.y);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      cmax = max(cmax, (uint32_t)__shfl_xor((int)cmax, o, 64));
      cmin = min(cmin, (uint32_t)__shfl_xor((int)cmin, o, 64));
    }
    // The first index holding the chunk's largest value.  Indices grow with
    // the load j, then the lane, then the logit within the group: the first
    // load any lane of which holds the value, its lowest such lane, and that
    // lane's first logit in the group (the branches on j are wave-uniform).
    int jstar = 0;
    uint64_t bal = 0;
#pragma unroll
    for (int j = kLaneLoads - 1; j >= 0; --j) {
      const uint64_t bj = __ballot(same_value(jmax[j], cmax));
      if (bj) { jstar = j; bal = bj; }
    }
    const int L = bal ? __builtin_ctzll(bal) : 0;
    int first = 0x7FFFFFFF;
#pragma unroll
    for (int j = 0; j < kLaneLoads; ++j) {
      if (j == jstar && l == L) {
        const uint32_t ws[4] = {d[j].x, d[j].y, d[j].z, d[j].w};
#pragma unroll
        for (int t = 7; t >= 0; --t) {
          const uint32_t h = t & 1 ? ws[t >> 1] >> 16 : ws[t >> 1] & 0xFFFFu;
          first = same_value(key_of(h), cmax) ? 8 * (g0 + l + 64 * j) + t : first;
        }
      }
    }
    first = __shfl(first, L, 64);
    if (l == 0) {
      uint32_t fl = 0;
      if (cmax >= kKeyPosInf || cmin < kKeyNegInf) fl |= SV_ROW_NONFINITE_LOGIT;
      if (cmax > kKeyNegInf && cmax < kKeyPosInf) fl |= kSawFinite;
      ArgmaxPart r;
      r.value = value_of_key(cmax);
      r.index = first;
      r.status = fl;
      r.pad = 0;
      p.parts[item] = r;
    }
  }
}

// Folds the chunk results of vector v: (value, first index) and flags.  The
// kernel runs a wave per row, so registers are plentiful: up to kFoldBatch
// chunk results load at once (every one of them for V <= 131072).
constexpr int kFoldBatch = 32;
__device__ __forceinline__ int fold_argmax(const GreedyParams& p, int v, int nch, uint32_t* fl) {
  float bv = -INFINITY;
  int bi = -1;
  const ArgmaxPart* r = p.parts + (int64_t)v * nch;
  for (int c0 = 0; c0 < nch; c0 += kFoldBatch) {
    ArgmaxPart q[kFoldBatch];
#pragma unroll
    for (int u = 0; u < kFoldBatch; ++u) q[u] = r[min(c0 + u, nch - 1)];
#pragma unroll
    for (int u = 0; u < kFoldBatch; ++u) {
      if (c0 + u < nch) {
        *fl |= q[u].status;
        if (better(q[u].value, q[u].index, bv, bi)) { bv = q[u].value; bi = q[u].index; }
      }
    }
  }
  return bi;
}

// One wave per row; lane i owns position i.
__global__ __launch_bounds__(256) void greedy_finalize_kernel(GreedyParams p) {
  const int b = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int l = threadIdx.x & 63;
  if (b >= p.B) return;
  const int K = p.K, nch = greedy_chunks(p.V);
  // every load of the row is issued before anything waits on one: k_b, the
  // lane's draft token and its position's chunk results (the latter two
  // for any lane that could need them, masked by k_b afterwards)
  const int kb = p.k_per_row ? p.k_per_row[b] : K;
  const int xt = (!p.draft && l < K) ? p.tokens[(int64_t)b * K + l] : -1;
  uint32_t ft = 0, fd = 0;
  const int gt = l <= K ? fold_argmax(p, b * (K + 1) + l, nch, &ft) : -1;
  const int gd = (p.draft && l < K) ? fold_argmax(p, p.B * (K + 1) + b * K + l, nch, &fd) : -1;
  const bool kok = kb >= 1 && kb <= K;
  uint32_t st = kok ? 0u : (uint32_t)SV_ROW_BAD_K;
  int g = -1, x = -1;
  if (kok) {
    uint32_t fl = 0;
    if (l <= kb) {
      g = gt;
      fl |= ft & SV_ROW_NONFINITE_LOGIT;
      if (!(ft & kSawFinite)) fl |= SV_ROW_NO_FINITE;
    }
    if (l < kb) {
      if (p.draft) {
        x = gd;
        fl |= fd & SV_ROW_NONFINITE_LOGIT;
        if (!(fd & kSawFinite)) fl |= SV_ROW_NO_FINITE;
      } else {
        x = xt;
        if (x < 0 || x >= p.V) fl |= SV_ROW_BAD_TOKEN;
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) fl |= __shfl_xor(fl, o, 64);
    st = fl;
  }
  const uint64_t miss = __ballot(kok && l < kb && x != g);
  const int acc = miss ? __builtin_ctzll(miss) : kb;
  const int y = __shfl(g, (acc >= 0 && acc < 64) ? acc : 0, 64);
  int32_t* out = p.out_tokens + (int64_t)b * (K + 1);
  if (l <= K) out[l] = st ? -1 : l < acc ? x : l == acc ? y : -1;
  if (l == 0) {
    p.accepted[b] = st ? -1 : acc;
    if (p.num_emitted) p.num_emitted[b] = st ? 0 : acc + 1;
    if (p.row_status) p.row_status[b] = (int32_t)st;
  }
}


// ---- one launch (argmax_fused_kernel)

// Chunk item `item` taken chunk-major (item = c * nvec + v): its vector's
// address (valid whether or not the row uses the vector), row and chunk.
struct FusedItem {
  const uint16_t* vec;
  int b, v, g0, n8;
  bool used;
};
__device__ __forceinline__ FusedItem fused_item(const GreedyParams& p, int item, int nvec,
                                                int n8v) {
  FusedItem f;
  const int c = item / nvec;
  f.v = item % nvec;
  const int nvec_t = p.B * (p.K + 1);
  bool draft_side;
  int pos;
  if (f.v < nvec_t) { f.b = f.v / (p.K + 1); pos = f.v % (p.K + 1); draft_side = false; }
  else { f.b = (f.v - nvec_t) / p.K; pos = (f.v - nvec_t) % p.K; draft_side = true; }
  const int kb = p.k_per_row ? p.k_per_row[f.b] : p.K;
  f.used = kb >= 1 && kb <= p.K && (draft_side ? pos < kb : pos <= kb);
  f.vec = draft_side ? (const uint16_t*)p.draft + ((int64_t)f.b * p.K + pos) * p.d_stride
                     : (const uint16_t*)p.target + ((int64_t)f.b * (p.K + 1) + pos) * p.t_stride;
  f.g0 = c * (kGreedyChunk / 8);
  f.n8 = min(kGreedyChunk / 8, n8v - f.g0);
  return f;
}

// The chunk's largest and smallest order keys and the first index holding
// the largest value, as argmax_stream_kernel finds them.
__device__ __forceinline__ void fused_chunk(const FusedItem& f, uint32_t& cmax, uint32_t& cmin,
                                            int& first) {
  const int l = threadIdx.x & 63;
  const uint4* body = (const uint4*)f.vec + f.g0;
  uint4 d[kLaneLoads];
#pragma unroll
  for (int j = 0; j < kLaneLoads; ++j) d[j] = body[min(l + 64 * j, f.n8 - 1)];
  uint32_t jmax[kLaneLoads];
  u16x2 kmin = {0xFFFF, 0xFFFF};
#pragma unroll
  for (int j = 0; j < kLaneLoads; ++j) {
    const bool valid = l + 64 * j < f.n8;
    const uint32_t ws[4] = {d[j].x, d[j].y, d[j].z, d[j].w};
    u16x2 m = {0, 0};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const u16x2 k = order_keys(ws[q]);
      m = __builtin_elementwise_max(m, k);
      kmin = __builtin_elementwise_min(kmin, k);
    }
    jmax[j] = valid ? max((uint32_t)m.x, (uint32_t)m.y) : 0u;
  }
  cmax = 0;
#pragma unroll
  for (int j = 0; j < kLaneLoads; ++j) cmax = max(cmax, jmax[j]);
  cmin = min((uint32_t)kmin.x, (uint32_t)kmin.y);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    cmax = max(cmax, (uint32_t)__shfl_xor((int)cmax, o, 64));
    cmin = min(cmin, (uint32_t)__shfl_xor((int)cmin, o, 64));
  }
  int jstar = 0;
  uint64_t bal = 0;
#pragma unroll
  for (int j = kLaneLoads - 1; j >= 0; --j) {
    const uint64_t bj = __ballot(same_value(jmax[j], cmax));
    if (bj) { jstar = j; bal = bj; }
  }
  const int L = bal ? __builtin_ctzll(bal) : 0;
  first = 0x7FFFFFFF;
#pragma unroll
  for (int j = 0; j < kLaneLoads; ++j) {
    if (j == jstar && l == L) {
      const uint32_t ws[4] = {d[j].x, d[j].y, d[j].z, d[j].w};
#pragma unroll
      for (int t = 7; t >= 0; --t) {
        const uint32_t h = t & 1 ? ws[t >> 1] >> 16 : ws[t >> 1] & 0xFFFFu;
        first = same_value(key_of(h), cmax) ? 8 * (f.g0 + l + 64 * j) + t : first;
      }
    }
  }
  first = __shfl(first, L, 64);
}

struct FusedState {
  uint32_t* cnt;              // per row: chunks counted so far
  unsigned long long* best;   // per vector: largest (order key << 32 | ~index)
  uint32_t* flg;              // per vector: SV_ROW_NONFINITE_LOGIT if seen
};

// The decision of row b by one wave, as greedy_finalize_kernel takes it,
// from the row's published maxima; then the row's state is zeroed.  A
// vector's maximum holds only chunks whose largest value is below +inf (a
// chunk holding +inf or a NaN flags the vector instead), so the vector has
// a finite value iff its maximum is finite, the rule the chunk records
// follow.
__device__ __forceinline__ void fused_decide_row(const GreedyParams& p, int b,
                                                 const FusedState& s) {
  const int l = threadIdx.x & 63, K = p.K;
  const int kb = p.k_per_row ? p.k_per_row[b] : K;
  const int xt = (!p.draft && l < K) ? p.tokens[(int64_t)b * K + l] : -1;
  const int vt = b * (K + 1) + min(l, K);
  const int vd = p.B * (K + 1) + b * K + min(l, K - 1);
  const unsigned long long kt = __hip_atomic_load(&s.best[(size_t)vt * kGreedyBestStride],
                                                  __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint32_t ftv = __hip_atomic_load(&s.flg[(size_t)vt * kGreedyFlgStride], __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
  unsigned long long kd = 0;
  uint32_t fdv = 0;
  if (p.draft) {
    kd = __hip_atomic_load(&s.best[(size_t)vd * kGreedyBestStride], __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    fdv = __hip_atomic_load(&s.flg[(size_t)vd * kGreedyFlgStride], __ATOMIC_RELAXED,
                            __HIP_MEMORY_SCOPE_AGENT);
  }
  auto flags_of = [](unsigned long long k, uint32_t f) {
    const uint32_t key = (uint32_t)(k >> 32);
    return f | (key > kKeyNegInf && key < kKeyPosInf ? kSawFinite : 0u);
  };
  const uint32_t ft = flags_of(kt, ftv), fd = flags_of(kd, fdv);
  const int gt = (int)(0xFFFFFFFFu - (uint32_t)kt), gd = (int)(0xFFFFFFFFu - (uint32_t)kd);
  const bool kok = kb >= 1 && kb <= K;
  uint32_t st = kok ? 0u : (uint32_t)SV_ROW_BAD_K;
  int g = -1, x = -1;
  if (kok) {
    uint32_t fl = 0;
    if (l <= kb) {
      g = gt;
      fl |= ft & SV_ROW_NONFINITE_LOGIT;
      if (!(ft & kSawFinite)) fl |= SV_ROW_NO_FINITE;
    }
    if (l < kb) {
      if (p.draft) {
        x = gd;
        fl |= fd & SV_ROW_NONFINITE_LOGIT;
        if (!(fd & kSawFinite)) fl |= SV_ROW_NO_FINITE;
      } else {
        x = xt;
        if (x < 0 || x >= p.V) fl |= SV_ROW_BAD_TOKEN;
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) fl |= __shfl_xor(fl, o, 64);
    st = fl;
  }
  const uint64_t miss = __ballot(kok && l < kb && x != g);
  const int acc = miss ? __builtin_ctzll(miss) : kb;
  const int y = __shfl(g, (acc >= 0 && acc < 64) ? acc : 0, 64);
  int32_t* out = p.out_tokens + (int64_t)b * (K + 1);
  if (l <= K) out[l] = st ? -1 : l < acc ? x : l == acc ? y : -1;
  if (l == 0) {
    p.accepted[b] = st ? -1 : acc;
    if (p.num_emitted) p.num_emitted[b] = st ? 0 : acc + 1;
    if (p.row_status) p.row_status[b] = (int32_t)st;
  }
  // every chunk of the row has been counted: nothing else touches its state
  if (l <= K) {
    s.best[(size_t)vt * kGreedyBestStride] = 0ull;
    s.flg[(size_t)vt * kGreedyFlgStride] = 0u;
  }
  if (p.draft && l < K) {
    s.best[(size_t)vd * kGreedyBestStride] = 0ull;
    s.flg[(size_t)vd * kGreedyFlgStride] = 0u;
  }
  if (l == 0) s.cnt[(size_t)b * kGreedyCntStride] = 0u;
}

// The streaming grid of argmax_stream_kernel, chunk-major, with the fold and
// the decision of each row done by the row's last chunk.  Every item counts
// for its row, used or not (a row with an invalid k_b uses none), so every
// row is decided once.
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, kFusedWgPerCu)))
void argmax_fused_kernel(GreedyParams p, int nitems, int nvec) {
  const int l = threadIdx.x & 63;
  const int waves = gridDim.x * (kThreads / 64);
  const int n8v = p.V >> 3;
  FusedState s;
  s.cnt = (uint32_t*)p.state;
  s.best = (unsigned long long*)(s.cnt + (size_t)p.B * kGreedyCntStride);
  s.flg = (uint32_t*)(s.best + (size_t)nvec * kGreedyBestStride);
  const uint32_t per_row =
      (uint32_t)greedy_chunks(p.V) * (uint32_t)(p.K + 1 + (p.draft ? p.K : 0));
  for (int item = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6); item < nitems; item += waves) {
    const FusedItem f = fused_item(p, item, nvec, n8v);
    unsigned long long ret = 0;
    if (f.used) {  // wave-uniform
      uint32_t cmax, cmin;
      int first;
      fused_chunk(f, cmax, cmin, first);
      if (l == 0) {
        if (cmax >= kKeyPosInf || cmin < kKeyNegInf)  // +inf or a NaN
          ret = __hip_atomic_fetch_or(&s.flg[(size_t)f.v * kGreedyFlgStride],
                                      (uint32_t)SV_ROW_NONFINITE_LOGIT, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
        if (cmax < kKeyPosInf) {
          const uint32_t key = cmax == 0x7FFFu ? 0x8000u : cmax;  // the two zeros are one value
          const unsigned long long packed =
              ((unsigned long long)key << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)first);
          ret |= __hip_atomic_fetch_max(&s.best[(size_t)f.v * kGreedyBestStride], packed,
                                        __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
    // the chunk counts for its row once its atomics have returned: the
    // increment depends on their result (it is never 2, but the compiler
    // cannot know that, so it waits for them)
    uint32_t prev = 0;
    if (l == 0) {
      const uint32_t inc = ret == ~0ull ? 2u : 1u;
      prev = __hip_atomic_fetch_add(&s.cnt[(size_t)f.b * kGreedyCntStride], inc, __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT);
    }
    prev = (uint32_t)__shfl((int)prev, 0, 64);
    if (prev == per_row - 1) fused_decide_row(p, f.b, s);
  }
}
}  // namespace

hipError_t launch_greedy(const GreedyParams& p, int num_cus, hipStream_t s, Timer* t) {
  if (p.B == 0) return hipSuccess;
  const int nvec = p.B * (p.K + 1) + (p.draft ? p.B * p.K : 0);
  const unsigned nitems = (unsigned)nvec * (unsigned)greedy_chunks(p.V);
  const bool stream = p.dtype == SV_BF16 && (p.V & 7) == 0 &&
                      ((uintptr_t)p.target & 15u) == 0 && (p.t_stride & 7) == 0 &&
                      (!p.draft || (((uintptr_t)p.draft & 15u) == 0 && (p.d_stride & 7) == 0));
  if (stream) {
    const unsigned cus = num_cus > 0 ? (unsigned)num_cus : 256u;
    const unsigned wgs_needed = (nitems + kThreads / 64 - 1) / (kThreads / 64);
    if (p.state) {
      const unsigned grid = min(cus * (unsigned)kFusedWgPerCu, wgs_needed);
      TimedScope ts(t, "greedy_fused", s);
      hipLaunchKernelGGL(argmax_fused_kernel, dim3(grid), dim3(kThreads), 0, s, p, (int)nitems,
                         nvec);
      return hipGetLastError();
    }
    const unsigned grid = min(cus * (unsigned)kStreamWgPerCu, wgs_needed);
    TimedScope ts(t, "greedy_argmax", s);
    hipLaunchKernelGGL(argmax_stream_kernel, dim3(grid), dim3(kThreads), 0, s, p, (int)nitems);
  } else {
    TimedScope ts(t, "greedy_argmax", s);
    hipLaunchKernelGGL(argmax_chunks_kernel, dim3(nitems), dim3(kThreads), 0, s, p);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    TimedScope ts(t, "greedy_finalize", s);
    hipLaunchKernelGGL(greedy_finalize_kernel, dim3((p.B + 3) / 4), dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace sv
