// Greedy branch of the verification step ([SSD] §2.4, §5.2): with no
// sampling, a draft token is accepted iff it equals the target's argmax at
// that position, and the first mismatch emits the target's argmax.  The
// page asks for this to be its own code path, and here it is: raw logits,
// no temperature, no top-p, lowest index on ties.
//
// Kernel 1 splits every vector into chunks of kGreedyChunk logits, one
// workgroup of 256 threads per chunk, and writes (max value, first index,
// flags) per chunk.  Kernel 2 (one workgroup per row) folds the chunks of
// each position and makes the row's decision.
#include <math.h>

#include "sv_internal.h"

namespace sv {
namespace {

constexpr int kThreads = 256;
constexpr int kPerThread = kGreedyChunk / kThreads;  // 64 logits

// (v, i) beats (bv, bi): larger value, or equal value with a lower index.
__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return i >= 0 && (bi < 0 || v > bv || (v == bv && i < bi));
}

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
  const int tid = threadIdx.x;
  const int64_t c0 = (int64_t)c * kGreedyChunk;
  const int n = (int)min((int64_t)kGreedyChunk, (int64_t)p.V - c0);

  float bv = -INFINITY;
  int bi = -1;
  uint32_t fl = 0;
  const bool aligned = ((((uintptr_t)vec) + c0 * esz) & 15u) == 0;
  if (p.dtype == SV_BF16 && aligned) {
    const uint16_t* base = (const uint16_t*)vec + c0;
    const int n8 = n >> 3;
    // thread t reads 16-byte groups t, t+256, ... : increasing index order
    for (int g = tid; g < n8; g += kThreads) {
      const uint4 d = *(const uint4*)(base + 8 * g);
      const uint32_t w[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const float z = __uint_as_float(t & 1 ? (w[t >> 1] & 0xFFFF0000u) : (w[t >> 1] << 16));
        if (isnan(z) || z == INFINITY) fl |= SV_ROW_NONFINITE_LOGIT;
        else if (z > -INFINITY) fl |= kSawFinite;
        if (z > bv || (bi < 0 && z == -INFINITY)) { bv = z; bi = (int)(c0 + 8 * g + t); }
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
  __shared__ float sv_[kThreads / 64];
  __shared__ int si_[kThreads / 64];
  __shared__ uint32_t sf_[kThreads / 64];
  const int w = tid >> 6, l = tid & 63;
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

__device__ int fold_argmax(const GreedyParams& p, int v, uint32_t* status) {
  const int nch = greedy_chunks(p.V);
  float bv = -INFINITY;
  int bi = -1;
  uint32_t fl = 0;
  for (int c = 0; c < nch; ++c) {
    const ArgmaxPart r = p.parts[(int64_t)v * nch + c];
    fl |= r.status;
    if (better(r.value, r.index, bv, bi)) { bv = r.value; bi = r.index; }
  }
  uint32_t st = fl & SV_ROW_NONFINITE_LOGIT;
  if (!(fl & kSawFinite)) st |= SV_ROW_NO_FINITE;
  *status |= st;
  return bi;
}

__global__ void greedy_finalize_kernel(GreedyParams p) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= p.B) return;
  const int K = p.K;
  const int kb = p.k_per_row ? p.k_per_row[b] : K;
  uint32_t st = 0;
  int32_t* out = p.out_tokens + (int64_t)b * (K + 1);
  if (kb < 1 || kb > K) st |= SV_ROW_BAD_K;
  int acc = 0, y = -1;
  if (!st) {
    const int nvec_t = p.B * (K + 1);
    // first pass: status of every vector the row uses
    for (int i = 0; i < kb; ++i) {
      if (p.draft) {
        fold_argmax(p, nvec_t + b * K + i, &st);
      } else {
        const int x = p.tokens[(int64_t)b * K + i];
        if (x < 0 || x >= p.V) st |= SV_ROW_BAD_TOKEN;
      }
    }
    for (int i = 0; i <= kb; ++i) fold_argmax(p, b * (K + 1) + i, &st);
    if (!st) {
      acc = kb;
      for (int i = 0; i < kb; ++i) {
        uint32_t dummy = 0;
        const int x = p.draft ? fold_argmax(p, nvec_t + b * K + i, &dummy)
                              : p.tokens[(int64_t)b * K + i];
        const int g = fold_argmax(p, b * (K + 1) + i, &dummy);
        if (x != g) { acc = i; y = g; break; }
        out[i] = x;
      }
      if (acc == kb) {
        uint32_t dummy = 0;
        y = fold_argmax(p, b * (K + 1) + kb, &dummy);
      }
    }
  }
  if (st) {
    for (int j = 0; j <= K; ++j) out[j] = -1;
    p.accepted[b] = -1;
    if (p.num_emitted) p.num_emitted[b] = 0;
  } else {
    out[acc] = y;
    for (int j = acc + 1; j <= K; ++j) out[j] = -1;
    p.accepted[b] = acc;
    if (p.num_emitted) p.num_emitted[b] = acc + 1;
  }
  if (p.row_status) p.row_status[b] = (int32_t)st;
}

}  // namespace

hipError_t launch_greedy(const GreedyParams& p, hipStream_t s, Timer* t) {
  if (p.B == 0) return hipSuccess;
  const int nvec = p.B * (p.K + 1) + (p.draft ? p.B * p.K : 0);
  const unsigned grid = (unsigned)nvec * (unsigned)greedy_chunks(p.V);
  {
    TimedScope ts(t, "greedy_argmax", s);
    hipLaunchKernelGGL(argmax_chunks_kernel, dim3(grid), dim3(kThreads), 0, s, p);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    TimedScope ts(t, "greedy_finalize", s);
    hipLaunchKernelGGL(greedy_finalize_kernel, dim3((p.B + 63) / 64), dim3(64), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace sv
