// Inverse-CDF draws over one vector, shared by the verification's finalize
// kernel and the draft sampler's fused statistics-and-draw kernel.  The
// method (token-index order, segment sums, the p'-only early stop) is
// described at the top of finalize.hip.
#pragma once

#include <math.h>

#include "philox.h"
#include "sv_internal.h"
#include "wave_ops.h"

namespace sv {
namespace {

// Workgroups have NT = 1024, 512 or 256 threads (a template parameter): 1024
// when the launch has about one workgroup per CU, 512 when it has two or
// more per CU, so that two fit a CU (registers and LDS) and one's serial
// steps (row header, scan, located segment) overlap the other's streaming;
// the draft sampler takes 256 from four per CU on.
constexpr int kSeg = 512;             // logits per (tile, wave) segment
constexpr int kMaxSeg = 4096;         // V <= 2^21 on this path

struct Dist {
  const void* vec;
  float m, tau, c2;  // c2 = log2(e) / T
  float invf;        // 1 / G, the kept mass's normaliser, in fp32
};

// Loads 8 consecutive logits starting at j0 (elements >= V read as -inf).
__device__ __forceinline__ void load8(const void* vec, int dtype, int64_t j0, int V,
                                      bool aligned, float z[8]) {
  if (aligned && j0 + 8 <= V) {
    if (dtype == SV_BF16) {
      const uint4 d = *(const uint4*)((const uint16_t*)vec + j0);
      const uint32_t w[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        z[2 * t] = __uint_as_float(w[t] << 16);
        z[2 * t + 1] = __uint_as_float(w[t] & 0xFFFF0000u);
      }
    } else {
      const float4 a = *(const float4*)((const float*)vec + j0);
      const float4 b = *(const float4*)((const float*)vec + j0 + 4);
      z[0] = a.x; z[1] = a.y; z[2] = a.z; z[3] = a.w;
      z[4] = b.x; z[5] = b.y; z[6] = b.z; z[7] = b.w;
    }
    return;
  }
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const int64_t j = j0 + t;
    if (j >= V) { z[t] = -INFINITY; continue; }
    z[t] = dtype == SV_BF16 ? __uint_as_float((uint32_t)((const uint16_t*)vec)[j] << 16)
                            : ((const float*)vec)[j];
  }
}

// The probability of logit z under d, in fp32: exp2 is an fp32 operation
// anyway, and the residual max(0, p' - q') of two such values is within a
// few ulp of p' and q'; sums are taken in fp64.
__device__ __forceinline__ float prob_f(const Dist& d, float z) {
  return z >= d.tau ? __builtin_amdgcn_exp2f((z - d.m) * d.c2) * d.invf : 0.0f;
}

// r_j for the 8 logits at j0: residual max(0, p' - q') (mode 0) or p' (mode
// 1), from fp32 probabilities as on the bf16 path (the sums are fp64).
__device__ __forceinline__ void r8(const Dist& P, const Dist& Q, int mode, int dtype,
                                   int64_t j0, int V, bool aligned, float r[8]) {
  float zp[8], zq[8];
  load8(P.vec, dtype, j0, V, aligned, zp);
  if (mode == 0) load8(Q.vec, dtype, j0, V, aligned, zq);
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const float pp = prob_f(P, zp[t]);
    r[t] = mode == 0 ? fmaxf(pp - prob_f(Q, zq[t]), 0.0f) : pp;
  }
}

// Capacity of a wave's token list on the bf16 path: two 8-token chunks per
// lane (the path is defined below).
constexpr int kListTok = 2 * 512;

template <int NT, int MS = kMaxSeg>
struct CdfScratch {
  double seg[MS];
  // bf16 path with a top-p cut: each wave's list of the tokens of its
  // segment that can carry mass, plus one spare slot per lane
  uint32_t list[NT / 64][kListTok + 64];
  double wsum[NT / 64];
  double R;
  int sstar;
  int y;
  double base;
};

// The Philox round counter of this call: the device word when one is given
// (read as the kernel runs, for captured rounds), else the host value.
__device__ __forceinline__ uint64_t round_offset(const FinalizeParams& p) {
  return p.offset_dev ? *p.offset_dev : p.offset;
}

__device__ __forceinline__ bool is_aligned16(const void* p) {
  return (((uintptr_t)p) & 15u) == 0;
}

// ---- bf16 fast path: 16-byte aligned vectors with V a multiple of 8.
// Groups of (NT / 64) segments of Seg<MODE>::tok tokens; in group G wave w
// owns segment G (NT / 64) + w, the tok contiguous tokens from
// (G (NT / 64) + w) tok, and lane l the 8-token chunks at 512 s + 8 l of it
// (s < Seg<MODE>::cps), so every wave load is 1 KB contiguous.  Pass 1 loads
// group G + 1 while it sums group G.  The residual (MODE 0) reads two
// vectors and takes two chunks per lane; p' alone (MODE 1) takes four, so
// that a wave has as many bytes in flight either way.
template <int MODE>
struct Seg {
  static constexpr int cps = MODE == 1 ? 4 : 2;  // chunks per lane per segment
  static constexpr int tok = 512 * cps;          // tokens per segment
};

// MODE 0: residual max(0, p' - q'); MODE 1: p' alone.
template <int MODE>
struct Chunks {
  uint4 p[Seg<MODE>::cps];
  uint4 q[MODE == 0 ? Seg<MODE>::cps : 1];
};

// Loads the chunks of this lane in segment `seg` (chunk indices past the last
// clamp to it; their values are masked by the caller).
template <int MODE>
__device__ __forceinline__ void load_segment(Chunks<MODE>& c, const uint16_t* P, const uint16_t* Q,
                                             int seg, int nchunks) {
  const int l = threadIdx.x & 63;
  const int c0 = seg * (Seg<MODE>::tok / 8) + l;
#pragma unroll
  for (int s = 0; s < Seg<MODE>::cps; ++s) {
    const int ci = min(c0 + 64 * s, nchunks - 1);
    c.p[s] = *(const uint4*)(P + 8 * (int64_t)ci);
    if (MODE == 0) c.q[s] = *(const uint4*)(Q + 8 * (int64_t)ci);
  }
}

// r of the 8 tokens of chunk s (0 where the chunk lies past the end).
template <int MODE>
__device__ __forceinline__ void chunk_r(const Dist& Pd, const Dist& Qd, const Chunks<MODE>& c,
                                        int s, bool valid, double r[8]) {
  const uint32_t pw[4] = {c.p[s].x, c.p[s].y, c.p[s].z, c.p[s].w};
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const float zp = __uint_as_float(t & 1 ? (pw[t >> 1] & 0xFFFF0000u) : (pw[t >> 1] << 16));
    float v = prob_f(Pd, zp);
    if (MODE == 0) {
      const uint32_t qw = t < 2 ? c.q[s].x : t < 4 ? c.q[s].y : t < 6 ? c.q[s].z : c.q[s].w;
      const float zq = __uint_as_float(t & 1 ? (qw & 0xFFFF0000u) : (qw << 16));
      v = fmaxf(v - prob_f(Qd, zq), 0.0f);
    }
    r[t] = valid ? (double)v : 0.0;
  }
}

// Pass 1 of one segment: the sum of r over the chunks of this lane, summed
// over the wave and stored as the segment's mass.  Every token's p' (and q')
// is formed; the tau test on the p side is taken only when CP (p' has a
// top-p cut), on the q side only when CQ.  A lane sums its tokens in fp32
// before the fp64 wave sum: the token probabilities are fp32 values anyway,
// and the located segment is re-derived token by token in fp64.
template <int MODE, bool CP, bool CQ>
__device__ __forceinline__ void segment_sum_direct(const Dist& P, const Dist& Q,
                                                  const Chunks<MODE>& c, int seg, int nchunks,
                                                  double* segs) {
  const int l = threadIdx.x & 63;
  float lf = 0.0f;
#pragma unroll
  for (int s = 0; s < Seg<MODE>::cps; ++s) {
    const bool valid = seg * (Seg<MODE>::tok / 8) + l + 64 * s < nchunks;
    const uint32_t pw[4] = {c.p[s].x, c.p[s].y, c.p[s].z, c.p[s].w};
    float cs = 0.0f;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const float zp = __uint_as_float(t & 1 ? (pw[t >> 1] & 0xFFFF0000u) : (pw[t >> 1] << 16));
      float v = CP ? prob_f(P, zp) : __builtin_amdgcn_exp2f((zp - P.m) * P.c2) * P.invf;
      if (MODE == 0) {
        const uint32_t qw = t < 2 ? c.q[s].x : t < 4 ? c.q[s].y : t < 6 ? c.q[s].z : c.q[s].w;
        const float zq = __uint_as_float(t & 1 ? (qw & 0xFFFF0000u) : (qw << 16));
        const float qv = CQ ? prob_f(Q, zq) : __builtin_amdgcn_exp2f((zq - Q.m) * Q.c2) * Q.invf;
        v = fmaxf(v - qv, 0.0f);
      }
      cs += v;
    }
    lf += valid ? cs : 0.0f;
  }
  const double ls = wave_last_f64(wave_scan_add_f64((double)lf));
  if (l == 0) segs[seg] = ls;
}

// The same sum when p' has a top-p cut.  r is zero at every token below
// tau_p (p' is zero there, so is max(0, p' - q')), and with a cut that is
// most tokens.  Two chunks at a time, the wave first lists the tokens at or
// above tau_p in LDS -- the raw p bits in the low half of an entry, q's in
// the high half -- by a ballot and a lane prefix count (branch-free: a lane
// with nothing to list writes its spare slot), then forms r on the list
// only.  The sum is over the same fp32 values as segment_sum's, in another
// order.
template <int MODE>
__device__ __forceinline__ void segment_sum_listed(const Dist& P, const Dist& Q,
                                                   const Chunks<MODE>& c, int seg, int nchunks,
                                                   double* segs, uint32_t* list) {
  static_assert(Seg<MODE>::cps % 2 == 0 && 2 * 512 == kListTok, "two chunks fill the list");
  const int l = threadIdx.x & 63;
  double ls = 0.0;
#pragma unroll
  for (int h = 0; h < Seg<MODE>::cps; h += 2) {
    uint32_t n = 0;  // list length (wave-uniform)
#pragma unroll
    for (int s = h; s < h + 2; ++s) {
      const bool valid = seg * (Seg<MODE>::tok / 8) + l + 64 * s < nchunks;
      const uint32_t pw[4] = {c.p[s].x, c.p[s].y, c.p[s].z, c.p[s].w};
      uint32_t qw[4] = {0u, 0u, 0u, 0u};
      if (MODE == 0) {
        qw[0] = c.q[s].x; qw[1] = c.q[s].y; qw[2] = c.q[s].z; qw[3] = c.q[s].w;
      }
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const uint32_t word = pw[t >> 1];
        const uint32_t hi = t & 1 ? word & 0xFFFF0000u : word << 16;  // p as fp32 bits
        const bool keep = valid && __uint_as_float(hi) >= P.tau;
        const uint64_t m = __ballot(keep);
        const uint32_t pre = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                       __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        uint32_t e = hi >> 16;
        if (MODE == 0) e |= t & 1 ? qw[t >> 1] & 0xFFFF0000u : qw[t >> 1] << 16;
        list[keep ? n + pre : (uint32_t)(kListTok + l)] = e;
        n += (uint32_t)__builtin_popcountll(m);
      }
    }
    for (uint32_t i0 = 0; i0 < n; i0 += 64) {
      const uint32_t i = i0 + (uint32_t)l;
      const uint32_t e = list[i < n ? i : 0u];
      float v = prob_f(P, __uint_as_float(e << 16));
      if (MODE == 0) v = fmaxf(v - prob_f(Q, __uint_as_float(e & 0xFFFF0000u)), 0.0f);
      ls += i < n ? (double)v : 0.0;
    }
  }
  ls = wave_last_f64(wave_scan_add_f64(ls));
  if (l == 0) segs[seg] = ls;
}

// Pass-1 variants: 0 listed tokens (the residual when p' has a top-p cut:
// most tokens then carry no mass, and listing spares their two exp2s),
// 1 no cut on either side, 2 a cut on q' only, 3 p' alone with a cut (one
// exp2 per token costs less than listing).
enum { kPassListed = 0, kPassUncut = 1, kPassCutQ = 2, kPassCutP = 3 };

template <int MODE, int PASS>
__device__ __forceinline__ void pass1_segment(const Dist& P, const Dist& Q, const Chunks<MODE>& c,
                                              int seg, int nchunks, double* segs, uint32_t* list) {
  if (PASS == kPassListed) segment_sum_listed<MODE>(P, Q, c, seg, nchunks, segs, list);
  else segment_sum_direct<MODE, PASS == kPassCutP, PASS == kPassCutQ>(P, Q, c, seg, nchunks, segs);
}

// Pass 2 by one wave over the segment `seg` held in c: its tokens in order
// (s, then lane, then t) in fp64, `before` the mass of every token ahead of
// the segment.  Returns the first token whose inclusive prefix exceeds
// `target`, else (a rounding edge) the last token with mass, -1 if none has
// any.  The result is the same in every lane.
template <int MODE>
__device__ __forceinline__ int locate_in_segment(const Dist& P, const Dist& Q,
                                                 const Chunks<MODE>& c, int seg, int nchunks,
                                                 double before, double target) {
  const int l = threadIdx.x & 63;
  double running = before;
  int hit = 0x7FFFFFFF, lastpos = -1;
#pragma unroll
  for (int s = 0; s < Seg<MODE>::cps; ++s) {
    const int ci = seg * (Seg<MODE>::tok / 8) + l + 64 * s;
    double r[8];
    chunk_r<MODE>(P, Q, c, s, ci < nchunks, r);
    double ls = 0.0;
#pragma unroll
    for (int t = 0; t < 8; ++t) ls += r[t];
    const double incl = wave_scan_add_f64(ls);
    double cum = running + (incl - ls);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      cum += r[t];
      if (r[t] > 0.0) {
        lastpos = 8 * ci + t;
        if (hit == 0x7FFFFFFF && cum > target) hit = 8 * ci + t;
      }
    }
    running += wave_last_f64(incl);
  }
  hit = (int)wave_last_u32(wave_scan_u32<OpMinI32>((uint32_t)hit));
  lastpos = (int)wave_last_u32(wave_scan_u32<OpMaxI32>((uint32_t)lastpos));
  return hit != 0x7FFFFFFF ? hit : lastpos;
}

// The early stop of a draw from a normalised distribution (MODE 1: p' alone,
// whose mass is 1 by construction, so the crossing point u is known before
// any token is read).  Called by every thread once the kWaves segment sums
// of a group are in `seg`: adds them to `cum` in token order and returns the
// wave whose segment holds the first prefix above `target` (-1 if the group
// ends at or below it), with the mass before that segment in `before`.
// Every thread reads the same values and adds them in the same order, so
// all take the same decision.
template <int kWaves>
__device__ __forceinline__ int group_crossing(const double* seg, double target, double& cum,
                                              double& before) {
  int hw = -1;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const double nx = cum + seg[w];
    if (hw < 0 && nx > cum && nx > target) {
      hw = w;
      before = cum;
    }
    cum = nx;
  }
  return hw;
}

// One inverse-CDF draw with this layout: returns y, -1 if R is 0 (the
// caller then retries on p' alone, for MODE 0) or the distribution is empty.
//
// MODE 0 reads the whole vector: R, the residual's mass, is known only at
// the end.  MODE 1 knows its mass before it starts -- `scale`: 1 for a
// whole normalised p', a shard's own mass for the part of p' it holds -- and
// stops after the group in which the running mass passes u * scale; the wave
// that holds the crossing segment in its registers locates the token without
// reading it again.  At a rounding edge (the running mass never passes
// u * scale) it falls back to the scan over all segment sums with R their
// total, as MODE 0 does.
template <int MODE, int PASS, int NT, int MS = kMaxSeg>
__device__ __forceinline__ int inverse_cdf_bf16(const Dist& P, const Dist& Q, int V, double u,
                                              double scale, CdfScratch<NT, MS>& sc) {
  constexpr int kWaves = NT / 64, kGroupTok = kWaves * Seg<MODE>::tok;
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const uint16_t* Pv = (const uint16_t*)P.vec;
  const uint16_t* Qv = (const uint16_t*)Q.vec;
  const int nchunks = V / 8;
  const int ngroups = (V + kGroupTok - 1) / kGroupTok;
  const int nseg = ngroups * kWaves;
  // pass 1: segment sums; group G + 1 loads while group G is summed, in two
  // register sets taken in turn (a copy would wait for the loads)
  {
    Chunks<MODE> ca, cb;
    uint32_t* list = sc.list[w];
    double cum = 0.0, before = 0.0;
    int hw = -1, gx = 0;  // MODE 1: the crossing's wave and group
    load_segment<MODE>(ca, Pv, Qv, w, nchunks);
    for (int G = 0; G < ngroups; G += 2) {
      load_segment<MODE>(cb, Pv, Qv, min(G + 1, ngroups - 1) * kWaves + w, nchunks);
      pass1_segment<MODE, PASS>(P, Q, ca, G * kWaves + w, nchunks, sc.seg, list);
      if (MODE == 1) {
        __syncthreads();
        hw = group_crossing<kWaves>(sc.seg + G * kWaves, u * scale, cum, before);
        gx = G;
        if (hw >= 0) break;
      }
      if (G + 1 >= ngroups) break;
      load_segment<MODE>(ca, Pv, Qv, min(G + 2, ngroups - 1) * kWaves + w, nchunks);
      pass1_segment<MODE, PASS>(P, Q, cb, (G + 1) * kWaves + w, nchunks, sc.seg, list);
      if (MODE == 1) {
        __syncthreads();
        hw = group_crossing<kWaves>(sc.seg + (G + 1) * kWaves, u * scale, cum, before);
        gx = G + 1;
        if (hw >= 0) break;
      }
    }
    if (MODE == 1 && hw >= 0) {  // the same in every thread
      if (w == hw) {
        // the crossing group's chunks are in ca (even group) or cb (odd)
        Chunks<MODE> c;
        const bool odd = (gx & 1) != 0;
#pragma unroll
        for (int i = 0; i < Seg<MODE>::cps; ++i) c.p[i] = odd ? cb.p[i] : ca.p[i];
        const int y =
            locate_in_segment<MODE>(P, Q, c, gx * kWaves + w, nchunks, before, u * scale);
        if (l == 0) sc.y = y;
      }
      __syncthreads();
      const int y = sc.y;
      __syncthreads();  // sc is reused by the next call
      return y;
    }
  }
  __syncthreads();
  // exclusive scan over segments (token order), by wave 0
  if (w == 0) {
    double carry = 0.0;
    for (int s0 = 0; s0 < nseg; s0 += 64) {
      const int i = s0 + l;
      const double v = i < nseg ? sc.seg[i] : 0.0;
      const double inc = wave_scan_add_f64(v);
      if (i < nseg) sc.seg[i] = carry + (inc - v);
      carry += wave_last_f64(inc);
    }
    if (l == 0) sc.R = carry;
  }
  __syncthreads();
  const double R = sc.R;
  if (!(R > 0.0)) {
    __syncthreads();  // sc is reused by a retry
    return -1;
  }
  const double target = u * R;
  // the segment holding the crossing: the last segment whose exclusive prefix
  // is <= target and whose mass is positive (or, at a rounding edge, the last
  // segment with mass); then its tokens in order
  if (w == 0) {
    int best = -1, lastm = -1;
    for (int s0 = 0; s0 < nseg; s0 += 64) {
      const int i = s0 + l;
      const double ex = i < nseg ? sc.seg[i] : 0.0;
      const double nx = i + 1 < nseg ? sc.seg[i + 1] : R;
      const bool has = i < nseg && nx > ex;
      if (has && ex <= target && nx > target) best = max(best, i);
      if (has) lastm = max(lastm, i);
    }
    best = (int)wave_last_u32(wave_scan_u32<OpMaxI32>((uint32_t)best));
    lastm = (int)wave_last_u32(wave_scan_u32<OpMaxI32>((uint32_t)lastm));
    const int ss = best >= 0 ? best : lastm >= 0 ? lastm : 0;
    Chunks<MODE> c;
    load_segment<MODE>(c, Pv, Qv, ss, nchunks);
    const int y = locate_in_segment<MODE>(P, Q, c, ss, nchunks, sc.seg[ss], target);
    if (l == 0) sc.y = y;
  }
  __syncthreads();
  const int y = sc.y;
  __syncthreads();  // sc is reused by the next call
  return y;
}

// Inverse CDF over one position, all threads of the block participate.
// mode 0: residual of (P, Q), falling back to P if it is identically zero;
// mode 1: P alone.  Returns y (same value in every thread), or -1 if the
// distribution is empty.  *zero_residual reports the fallback.
template <int NT>
__device__ __forceinline__ int inverse_cdf(const Dist& P, const Dist& Q, int mode, int dtype, int V,
                                           double u, CdfScratch<NT>& sc, bool* zero_residual,
                                           double scale = 1.0) {
  constexpr int kThreads = NT, kWaves = NT / 64, kTile = NT * 8;
  if (dtype == SV_BF16 && (V & 7) == 0 && is_aligned16(P.vec) &&
      (mode == 1 || is_aligned16(Q.vec))) {
    *zero_residual = false;
    // the same in every thread
    const bool cutp = P.tau > -INFINITY, cutq = Q.tau > -INFINITY;
    if (mode == 0) {
      const int y = cutp ? inverse_cdf_bf16<0, kPassListed, NT>(P, Q, V, u, 1.0, sc)
                  : cutq ? inverse_cdf_bf16<0, kPassCutQ, NT>(P, Q, V, u, 1.0, sc)
                         : inverse_cdf_bf16<0, kPassUncut, NT>(P, Q, V, u, 1.0, sc);
      if (y >= 0) return y;
      // R == 0: the residual vanishes identically; draw from p' instead
      *zero_residual = true;
    }
    return cutp ? inverse_cdf_bf16<1, kPassCutP, NT>(P, P, V, u, scale, sc)
                : inverse_cdf_bf16<1, kPassUncut, NT>(P, P, V, u, scale, sc);
  }
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int ntiles = (V + kTile - 1) / kTile;
  const int nseg = ntiles * kWaves;
  const bool aligned = is_aligned16(P.vec) && (mode == 1 || is_aligned16(Q.vec));
  *zero_residual = false;
  for (int attempt = 0; attempt < 2; ++attempt) {
    // pass 1: per-segment sums
    for (int s = 0; s < ntiles; ++s) {
      const int64_t j0 = (int64_t)s * kTile + 8 * tid;
      float r[8];
      r8(P, Q, mode, dtype, j0, V, aligned, r);
      float lf = 0.0f;  // a lane's 8 tokens in fp32, the wave's sum in fp64
#pragma unroll
      for (int t = 0; t < 8; ++t) lf += r[t];
      double ls = (double)lf;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) ls += __shfl_xor(ls, o, 64);
      if (l == 0) sc.seg[s * kWaves + w] = ls;
    }
    __syncthreads();
    // exclusive scan over segments (in token order), one pass of 1024 at a time
    double carry = 0.0;
    for (int s0 = 0; s0 < nseg; s0 += kThreads) {
      const int i = s0 + tid;
      const double v = i < nseg ? sc.seg[i] : 0.0;
      double inc = v;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const double t = __shfl_up(inc, o, 64);
        if (l >= o) inc += t;
      }
      if (l == 63) sc.wsum[w] = inc;
      __syncthreads();
      double before = carry;
      double tot = 0.0;
      for (int k = 0; k < kWaves; ++k) {
        if (k < w) before += sc.wsum[k];
        tot += sc.wsum[k];
      }
      __syncthreads();
      if (i < nseg) sc.seg[i] = before + (inc - v);  // exclusive prefix
      carry += tot;
    }
    if (tid == 0) sc.R = carry;
    __syncthreads();
    const double R = sc.R;
    if (mode == 0 && R == 0.0 && attempt == 0) {
      mode = 1;
      *zero_residual = true;
      __syncthreads();
      continue;
    }
    if (!(R > 0.0)) return -1;
    const double target = u * R;
    // segment holding the crossing: the last segment whose exclusive prefix
    // is <= target and whose mass is positive
    if (tid == 0) sc.sstar = -1;
    __syncthreads();
    for (int i = tid; i < nseg; i += kThreads) {
      const double ex = sc.seg[i];
      const double nx = i + 1 < nseg ? sc.seg[i + 1] : R;
      if (ex <= target && nx > ex && nx > target) atomicMax(&sc.sstar, i);
    }
    __syncthreads();
    int ss = sc.sstar;
    if (ss < 0) {  // rounding edge: take the last segment with mass
      if (tid == 0) {
        for (int i = nseg - 1; i >= 0; --i) {
          const double nx = i + 1 < nseg ? sc.seg[i + 1] : R;
          if (nx > sc.seg[i]) { ss = i; break; }
        }
        sc.sstar = ss;
      }
      __syncthreads();
      ss = sc.sstar;
    }
    if (ss < 0) ss = 0;  // R > 0 guarantees a segment with mass; stay in bounds regardless
    // pass 2: wave 0 re-derives segment ss and finds the token
    if (w == 0) {
      const int st = ss / kWaves, sw = ss % kWaves;
      const int64_t j0 = (int64_t)st * kTile + (int64_t)sw * kSeg + 8 * l;
      float rf[8];
      r8(P, Q, mode, dtype, j0, V, aligned, rf);
      double r[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) r[t] = (double)rf[t];
      double ls = 0.0;
#pragma unroll
      for (int t = 0; t < 8; ++t) ls += r[t];
      double inc = ls;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const double t = __shfl_up(inc, o, 64);
        if (l >= o) inc += t;
      }
      double exl = __shfl_up(inc, 1, 64);
      if (l == 0) exl = 0.0;
      const double base = sc.seg[ss] + exl;
      int hit = 0x7FFFFFFF, lastpos = -1;
      double loc = 0.0;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        loc += r[t];
        if (r[t] > 0.0) {
          lastpos = (int)(j0 + t);
          if (hit == 0x7FFFFFFF && base + loc > target) hit = (int)(j0 + t);
        }
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        hit = min(hit, __shfl_xor(hit, o, 64));
        lastpos = max(lastpos, __shfl_xor(lastpos, o, 64));
      }
      if (l == 0) sc.y = hit != 0x7FFFFFFF ? hit : lastpos;
    }
    __syncthreads();
    return sc.y;
  }
  return -1;
}

__device__ __forceinline__ Dist make_dist(const void* base, int64_t vec_index, int64_t stride,
                                          int dtype, float m, float tau, double inv_kept, float T) {
  Dist d;
  d.vec = (const char*)base + vec_index * stride * (dtype == SV_BF16 ? 2 : 4);
  d.m = m;
  d.tau = tau;
  d.c2 = log2e_over_T(T);
  d.invf = (float)inv_kept;
  return d;
}

}  // namespace
}  // namespace sv
