// Per-row decision of the sampled verification, and the inverse-CDF draws.
//
// One workgroup per row ([SD] §2.2, [SSD] §4.3 accept_or_reject):
//   rho_i = p'_i(x_i) / q'_i(x_i) (0 when q'_i(x_i) = 0), taken from the
//   per-vector records; accept while u(b,i,0) < rho_i; the first rejection a
//   is followed by one draw from norm(max(0, p'_a - q'_a)) ([SSD] §2.4,
//   §5.2; [SD] §2.1), or from p'_a when that residual is identically zero
//   ([SSD] §4.3); if nothing is rejected the bonus comes from p'_{k_b}
//   ([SD] §2.2).
//
// The draw is an inverse CDF in token-index order: y = min{j : C_j > u R},
// C the inclusive prefix of r, R its total.  Pass 1 sums r per segment of
// consecutive tokens; a scan over the segments finds the one holding u R;
// pass 2 re-derives that segment's values token by token, scans them across
// lanes in fp64 and picks the token.  bf16 vectors that are 16-byte
// aligned with V a multiple of 8 are read in groups of NT / 64 segments,
// one per wave (1024 tokens of both vectors for the residual, 2048 for p'
// alone), with the next group's loads in flight; under a top-p cut on p'
// the residual's pass 1 works on the listed tokens at or above tau_p only.
// On this path a draw from p' alone (the bonus, the zero-residual fallback,
// the draft sampler's q') knows its mass before it starts (R = 1), so pass 1
// stops after the group in which the running sum passes u -- about half
// the vector on average -- and the wave holding that segment locates the
// token from its registers.  Other vectors (fp32, unaligned, ragged V) are
// read in tiles of 1024 x 8 logits with 512-token segments.  Probabilities
// are fp32 on both paths (exp2 of an fp32 argument, v_exp_f32, times the
// fp32 1/G normaliser); a lane sums its tokens in fp32, and segment and
// prefix sums are fp64.
//
// With a KV rollback that keeps pages mapped (no free stack, no pool), the
// row's workgroup also rolls the row back on the accepted count it found
// (finalize_sample_kernel<NT, true>, below).
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

template <int NT>
struct CdfScratch {
  double seg[kMaxSeg];
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
template <int MODE, int PASS, int NT>
__device__ __forceinline__ int inverse_cdf_bf16(const Dist& P, const Dist& Q, int V, double u,
                                              double scale, CdfScratch<NT>& sc) {
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

__device__ Dist make_dist(const void* base, int64_t vec_index, int64_t stride, int dtype, float m,
                          float tau, double inv_kept, float T) {
  Dist d;
  d.vec = (const char*)base + vec_index * stride * (dtype == SV_BF16 ? 2 : 4);
  d.m = m;
  d.tau = tau;
  d.c2 = log2e_over_T(T);
  d.invf = (float)inv_kept;
  return d;
}

// The fields of a record the kernels use, loaded field by field (a whole
// VecRec copied under a lane condition stays a private array).
struct RecFields {
  float m, tau;
  double inv_kept, px;
  uint32_t status;
};

__device__ __forceinline__ RecFields load_rec(const VecRec* r, bool valid) {
  RecFields f;
  f.m = valid ? r->m : 0.0f;
  f.tau = valid ? r->tau : 0.0f;
  f.inv_kept = valid ? r->inv_kept : 0.0;
  f.px = valid ? r->px : 0.0;
  f.status = valid ? r->status : 0u;
  return f;
}

struct RowShared {
  int kb, acc, mode, go;
  uint32_t status;
  float T;
  double u1;
  float pm, ptau, qm, qtau;  // records of the drawn position (target, draft)
  double pinv, qinv;
};

// Row header by wave 0 (every thread calls it), one lane per position:
// checks, ratios, uniforms; the first rejection is the lowest lane that
// rejects.  Every load is issued up front -- lane l reads the draft token and
// the target and draft records of position l whatever k_b is, and k_b masks
// them afterwards -- so the header waits for memory once.  Fills rs; with
// OUT, also writes p'(x_i), q'(x_i) and a flagged row's outputs.  Returns the
// lane's draft token (lanes of wave 0), for the output row.
template <bool OUT>
__device__ __forceinline__ int row_header(const FinalizeParams& p, int b, RowShared& rs) {
  int x = 0;
  if (threadIdx.x < 64) {
    const int K = p.K, V = p.V;
    const VecRec* recs = p.recs + (int64_t)b * slots_per_row(K);
    const int l = threadIdx.x;
    const int kb = p.k_per_row ? p.k_per_row[b] : K;
    const float T = p.temperature[b];
    const float P = p.top_p ? p.top_p[b] : 1.0f;
    const uint64_t off = round_offset(p);
    if (l < K) x = p.tokens[(int64_t)b * K + l];
    const RecFields rt = load_rec(recs + min(l, K), l <= K);
    const RecFields rd = load_rec(recs + K + 1 + min(l, K - 1), l < K);
    uint32_t st = 0;
    if (kb < 1 || kb > K) st |= SV_ROW_BAD_K;
    if (!(T > 0.0f) || !isfinite(T)) st |= SV_ROW_BAD_TEMPERATURE;
    if (isnan(P) || P <= 0.0f) st |= SV_ROW_BAD_TOP_P;
    double px = 0.0, qx = 0.0;
    uint32_t lst = 0;
    if (!(st & SV_ROW_BAD_K)) {
      if (l < kb) {
        if (x < 0 || x >= V) lst |= SV_ROW_BAD_TOKEN;
        px = rt.px;
        qx = rd.px;
        lst |= rt.status | rd.status;
      } else if (l == kb) {
        lst |= rt.status;
      }
    }
    st |= wave_last_u32(wave_scan_u32<OpOrU32>(lst));
    int acc = 0;
    if (!st) {
      bool rej = false;
      if (l < kb) {
        const double rho = qx > 0.0 ? px / qx : 0.0;
        const double u = uniform24(p.seed, (uint64_t)b, (uint64_t)l, 0, off);
        rej = !(u < rho);
      }
      const uint64_t rm = __ballot(rej);
      acc = rm ? __builtin_ctzll(rm) : kb;
      if (OUT && l < K) {
        if (p.p_at_draft) p.p_at_draft[(int64_t)b * K + l] = l < kb ? (float)px : 0.0f;
        if (p.q_at_draft) p.q_at_draft[(int64_t)b * K + l] = l < kb ? (float)qx : 0.0f;
      }
      // lane acc (<= k_b <= K) holds the drawn position's records
      if (l == acc) {
        rs.pm = rt.m;
        rs.ptau = rt.tau;
        rs.pinv = rt.inv_kept;
        rs.qm = rd.m;
        rs.qtau = rd.tau;
        rs.qinv = rd.inv_kept;
      }
    } else if (OUT) {
      if (l <= K) p.out_tokens[(int64_t)b * (K + 1) + l] = -1;
      if (l < K) {
        if (p.p_at_draft) p.p_at_draft[(int64_t)b * K + l] = NAN;
        if (p.q_at_draft) p.q_at_draft[(int64_t)b * K + l] = NAN;
      }
      if (l == 0) {
        p.accepted[b] = -1;
        if (p.num_emitted) p.num_emitted[b] = 0;
        if (p.row_status) p.row_status[b] = (int32_t)st;
      }
    }
    if (l == 0) {
      rs.kb = kb;
      rs.acc = acc;
      rs.go = st == 0;
      rs.status = st;
      rs.T = T;
      rs.mode = acc < kb ? 0 : 1;
      rs.u1 = uniform24(p.seed, (uint64_t)b, (uint64_t)acc, 1, off);
    }
  }
  return x;
}

// ---- the rollback of a row, fused into its verification
// The rollback kernel's decision for the row ([SSD] §3.3: the write pointer
// moves back to the accepted prefix, and the page table must agree with the
// length: the first ceil(old/ps) entries map pages of the pool and, with a
// free stack, every later entry is unmapped), taken on the accepted count
// the row's verification just found (-1 for a flagged row).  Without a free
// stack or pool the row's rollback needs nothing from the others and is
// committed here; otherwise the decision goes to the rollback's records and
// its scan over all rows places the releases.  Every thread loads one page
// entry after the header, so that the loads overlap the draw; the entries
// are tested, and the result written, at the end.
struct RollCheck {
  uint32_t st;
  int old_len, new_len, used, span;
  int32_t e;  // page entry threadIdx.x (when below span)
};

__device__ __forceinline__ int ceil_div_i(int x, int d) { return (x + d - 1) / d; }

__device__ __forceinline__ RollCheck roll_begin(const FinalizeParams& p, int b, const RowShared& rs,
                                                int old) {
  RollCheck r;
  const int k = rs.kb, acc = rs.go ? rs.acc : -1;
  r.st = 0;
  if (k < 1 || k > p.K) r.st |= SV_ROW_BAD_K;
  else if (acc < 0 || acc > k || old - (k - acc) < 0) r.st |= SV_ROW_BAD_ACCEPTED;
  if (old < 0 || ceil_div_i(old, p.ps) > p.MP) r.st |= SV_ROW_BAD_PAGES;
  r.old_len = old;
  r.new_len = r.st ? old : old - (k - acc);
  r.used = r.st ? 0 : ceil_div_i(old, p.ps);
  // past the length only a free stack constrains the entries
  r.span = r.st ? 0 : (p.free_stack ? p.MP : r.used);
  // clamped into the row, loaded whether or not it is tested
  const int pg = min((int)threadIdx.x, p.MP - 1);
  r.e = p.page_table[(int64_t)b * p.MP + pg];
  return r;
}

// Called by every thread of the workgroup.
template <int NT>
__device__ __forceinline__ void roll_end(const FinalizeParams& p, int b, const RollCheck& r) {
  const int tid = threadIdx.x;
  auto bad_entry = [&](int pg, int32_t e) {
    return pg < r.used ? (e < 0 || (p.num_pages > 0 && e >= p.num_pages)) : e != -1;
  };
  bool bad = tid < r.span && bad_entry(tid, r.e);
  for (int pg = tid + NT; pg < r.span; pg += NT)  // tables longer than NT pages
    bad = bad || bad_entry(pg, p.page_table[(int64_t)b * p.MP + pg]);
  const uint32_t st = r.st | (__syncthreads_or(bad) ? (uint32_t)SV_ROW_BAD_PAGES : 0u);
  if (tid == 0) {
    if (p.roll_recs) {
      // the rollback's record: status, lengths and the pages released
      RollRec rec;
      rec.status = (int32_t)st;
      rec.old_len = r.old_len;
      rec.new_len = st ? r.old_len : r.new_len;
      rec.aux = st ? 0 : r.used - ceil_div_i(r.new_len, p.ps);
      p.roll_recs[b] = rec;
    } else {
      if (!st) p.kv_len[b] = r.new_len;
      if (p.roll_status) p.roll_status[b] = (int32_t)st;
    }
  }
}

template <int NT, bool ROLL>
__global__ __launch_bounds__(NT) void finalize_sample_kernel(FinalizeParams p) {
  __shared__ CdfScratch<NT> sc;
  __shared__ RowShared rs;
  const int b = blockIdx.x, K = p.K, V = p.V, tid = threadIdx.x;
  // the KV length loads with the header's loads
  const int old = ROLL ? p.kv_len[b] : 0;
  const int x = row_header<true>(p, b, rs);
  __syncthreads();
  RollCheck rc;
  if (ROLL) rc = roll_begin(p, b, rs, old);
  if (!rs.go) {
    if (ROLL) roll_end<NT>(p, b, rc);
    return;
  }
  const int acc = rs.acc, mode = rs.mode;
  const Dist P = make_dist(p.target, (int64_t)b * (K + 1) + acc, p.t_stride, p.dtype, rs.pm,
                           rs.ptau, rs.pinv, rs.T);
  Dist Q = P;
  if (mode == 0)
    Q = make_dist(p.draft, (int64_t)b * K + acc, p.d_stride, p.dtype, rs.qm, rs.qtau, rs.qinv,
                  rs.T);
  bool zero = false;
  const int y = inverse_cdf(P, Q, mode, p.dtype, V, rs.u1, sc, &zero);
  if (tid < 64) {
    const int l = tid;
    if (l <= K) {
      const int32_t v = l < acc ? x : l == acc ? y : -1;
      p.out_tokens[(int64_t)b * (K + 1) + l] = v;
    }
    if (l == 0) {
      p.accepted[b] = acc;
      if (p.num_emitted) p.num_emitted[b] = acc + 1;
      if (p.row_status) p.row_status[b] = 0;
    }
  }
  if (ROLL) roll_end<NT>(p, b, rc);
}

// Draft sampling: one workgroup per (row, draft position).  The header
// issues every load at once, as the verification header does: k_b, T,
// top-p, the round counter and the status words of all K draft records
// (masked by k_b afterwards), and this position's record.
template <int NT>
__global__ __launch_bounds__(NT) void draft_sample_kernel(FinalizeParams p) {
  __shared__ CdfScratch<NT> sc;
  __shared__ int go;
  __shared__ float Ts;
  __shared__ double us;
  __shared__ float qm, qtau;
  __shared__ double qinv;
  const int b = blockIdx.x / p.K, i = blockIdx.x % p.K, K = p.K, tid = threadIdx.x;
  const int per = slots_per_row(K);
  const VecRec* recs = p.recs + (int64_t)b * per;
  if (tid < 64) {
    const int l = tid;
    const int kb = p.k_per_row ? p.k_per_row[b] : K;
    const float T = p.temperature[b];
    const float P = p.top_p ? p.top_p[b] : 1.0f;
    const uint64_t off = round_offset(p);
    const RecFields rd = load_rec(recs + K + 1 + min(l, K - 1), l < K);
    uint32_t st = 0;
    if (kb < 1 || kb > K) st |= SV_ROW_BAD_K;
    if (!(T > 0.0f) || !isfinite(T)) st |= SV_ROW_BAD_TEMPERATURE;
    if (isnan(P) || P <= 0.0f) st |= SV_ROW_BAD_TOP_P;
    const uint32_t lst = !(st & SV_ROW_BAD_K) && l < kb ? rd.status : 0u;
    st |= wave_last_u32(wave_scan_u32<OpOrU32>(lst));
    if (l == i) {
      qm = rd.m;
      qtau = rd.tau;
      qinv = rd.inv_kept;
    }
    if (l == 0) {
      // every workgroup of the row sees the same status; position 0 reports it
      if (i == 0 && p.row_status) p.row_status[b] = (int32_t)st;
      go = (st == 0 && i < kb) ? 1 : 0;
      if (!go) p.draft_out[(int64_t)b * K + i] = -1;
      Ts = T;
      us = uniform24(p.seed, (uint64_t)b, (uint64_t)i, 2, off);
    }
  }
  __syncthreads();
  if (!go) return;
  const Dist Q = make_dist(p.draft, (int64_t)b * K + i, p.d_stride, p.dtype, qm, qtau, qinv, Ts);
  bool zero = false;
  const int y = inverse_cdf(Q, Q, 1, p.dtype, p.V, us, sc, &zero);
  if (tid == 0) p.draft_out[(int64_t)b * K + i] = y;
}

// ---- vocabulary-sharded draw
// Shard g holds columns [col_off, col_off + col_len) of every vector, and the
// records are the merged ones.  The draw takes two launches per shard with an
// exchange between them:
//   mass:   over its own columns of the drawn position, each shard sums the
//           residual max(0, p' - q') and p' (masses[g][b] = {R_g, P_g});
//   locate: with every shard's masses, each finds the shard whose running
//           mass, in shard order, first passes u R -- R the sum of the R_g,
//           or of the P_g for the bonus and for a zero residual ([SSD] §4.3)
//           -- and that shard alone draws the token from its columns, with
//           the target u R less the mass of the shards before it.
// Every shard writes the same row outputs; the drawn token comes from the
// shard that holds it.

// Sums over n columns of the residual (mode 0) and of p', four 8-token chunks
// per thread in flight; fp32 within a chunk, fp64 across chunks and threads.
template <int NT>
__device__ __forceinline__ void column_masses(const Dist& P, const Dist& Q, int mode, int dtype,
                                              int n, double* red, double* rsum, double* psum) {
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const bool aligned = is_aligned16(P.vec) && (mode == 1 || is_aligned16(Q.vec));
  double r = 0.0, q = 0.0;
  constexpr int kU = 4;
  for (int64_t j0 = 8 * (int64_t)tid; j0 < n; j0 += 8 * (int64_t)NT * kU) {
    float zp[kU][8], zq[kU][8];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t j = j0 + 8 * (int64_t)NT * u;
      load8(P.vec, dtype, j, n, aligned, zp[u]);  // past n: -inf, mass 0
      if (mode == 0) load8(Q.vec, dtype, j, n, aligned, zq[u]);
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      float cr = 0.0f, cp = 0.0f;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const float pp = prob_f(P, zp[u][t]);
        cp += pp;
        if (mode == 0) cr += fmaxf(pp - prob_f(Q, zq[u][t]), 0.0f);
      }
      r += cr;
      q += cp;
    }
  }
  r = wave_last_f64(wave_scan_add_f64(r));
  q = wave_last_f64(wave_scan_add_f64(q));
  if (l == 0) {
    red[2 * w] = r;
    red[2 * w + 1] = q;
  }
  __syncthreads();
  double a = 0.0, c = 0.0;
#pragma unroll
  for (int k = 0; k < NT / 64; ++k) {
    a += red[2 * k];
    c += red[2 * k + 1];
  }
  *rsum = a;
  *psum = c;
}

template <int NT>
__global__ __launch_bounds__(NT) void shard_mass_kernel(FinalizeParams p, ShardDrawParams d) {
  __shared__ RowShared rs;
  __shared__ double red[2 * (NT / 64)];
  const int b = blockIdx.x, K = p.K;
  row_header<false>(p, b, rs);
  __syncthreads();
  double* out = d.masses + ((int64_t)d.shard * p.B + b) * 2;
  if (!rs.go) {
    if (threadIdx.x == 0) out[0] = out[1] = 0.0;
    return;
  }
  const int acc = rs.acc, mode = rs.mode;
  const Dist P = make_dist(d.tgt, (int64_t)b * (K + 1) + acc, d.ts, p.dtype, rs.pm, rs.ptau,
                           rs.pinv, rs.T);
  Dist Q = P;
  if (mode == 0)
    Q = make_dist(d.dft, (int64_t)b * K + acc, d.ds, p.dtype, rs.qm, rs.qtau, rs.qinv, rs.T);
  double rsum, psum;
  column_masses<NT>(P, Q, mode, p.dtype, d.col_len, red, &rsum, &psum);
  if (threadIdx.x == 0) {
    out[0] = mode == 0 ? rsum : 0.0;
    out[1] = psum;
  }
}

template <int NT>
__global__ __launch_bounds__(NT) void shard_locate_kernel(FinalizeParams p, ShardDrawParams d) {
  __shared__ CdfScratch<NT> sc;
  __shared__ RowShared rs;
  __shared__ double ms[kMaxShards][2];
  const int b = blockIdx.x, K = p.K, tid = threadIdx.x;
  if (tid < d.G) {
    const double* m = d.masses + ((int64_t)tid * p.B + b) * 2;
    ms[tid][0] = m[0];
    ms[tid][1] = m[1];
  }
  const int x = row_header<true>(p, b, rs);
  __syncthreads();
  if (!rs.go) return;
  const int acc = rs.acc;
  // the total and the owner, the same in every thread (LDS, shard order)
  double R = 0.0;
  for (int g = 0; g < d.G; ++g) R += ms[g][0];
  int mode = rs.mode;
  if (mode == 0 && !(R > 0.0)) mode = 1;  // a zero residual: draw from p'
  const int side = mode == 0 ? 0 : 1;
  if (side == 1) {
    R = 0.0;
    for (int g = 0; g < d.G; ++g) R += ms[g][1];
  }
  const double target = rs.u1 * R;
  int owner = -1, lastm = -1;
  double before = 0.0, before_last = 0.0, run = 0.0;
  for (int g = 0; g < d.G; ++g) {
    const double m = ms[g][side];
    if (m > 0.0) {
      if (owner < 0 && run + m > target) {
        owner = g;
        before = run;
      }
      lastm = g;
      before_last = run;
    }
    run += m;
  }
  if (owner < 0) {  // rounding edge: the last shard with mass
    owner = lastm;
    before = before_last;
  }
  int y = -1;  // no mass at all: an empty distribution
  if (owner == d.shard) {
    const Dist P = make_dist(d.tgt, (int64_t)b * (K + 1) + acc, d.ts, p.dtype, rs.pm, rs.ptau,
                             rs.pinv, rs.T);
    Dist Q = P;
    if (mode == 0)
      Q = make_dist(d.dft, (int64_t)b * K + acc, d.ds, p.dtype, rs.qm, rs.qtau, rs.qinv, rs.T);
    const double m = ms[owner][side];
    bool zero = false;
    // u' m is the target less the mass of the shards before this one
    const int yl = inverse_cdf(P, Q, mode, p.dtype, d.col_len, (target - before) / m, sc, &zero, m);
    y = yl >= 0 ? d.col_off + yl : -1;
  }
  const bool writes_y = owner == d.shard || (owner < 0 && d.shard == 0);
  if (tid < 64) {
    const int l = tid;
    if (l <= K && (l != acc || writes_y)) {
      const int32_t v = l < acc ? x : l == acc ? y : -1;
      p.out_tokens[(int64_t)b * (K + 1) + l] = v;
    }
    if (l == 0) {
      p.accepted[b] = acc;
      if (p.num_emitted) p.num_emitted[b] = acc + 1;
      if (p.row_status) p.row_status[b] = 0;
    }
  }
}

}  // namespace

// 512-thread workgroups when there are at least two per CU.
static bool use_half_blocks(unsigned nblocks, int num_cus) {
  const unsigned cus = num_cus > 0 ? (unsigned)num_cus : 256u;
  return nblocks >= 2u * cus;
}

hipError_t launch_finalize_sample(const FinalizeParams& p, int num_cus, hipStream_t s, Timer* t) {
  if (p.B == 0) return hipSuccess;
  TimedScope ts(t, "finalize_sample", s);
  const bool half = use_half_blocks((unsigned)p.B, num_cus);
  if (half && p.kv_len)
    hipLaunchKernelGGL((finalize_sample_kernel<512, true>), dim3(p.B), dim3(512), 0, s, p);
  else if (half)
    hipLaunchKernelGGL((finalize_sample_kernel<512, false>), dim3(p.B), dim3(512), 0, s, p);
  else if (p.kv_len)
    hipLaunchKernelGGL((finalize_sample_kernel<1024, true>), dim3(p.B), dim3(1024), 0, s, p);
  else
    hipLaunchKernelGGL((finalize_sample_kernel<1024, false>), dim3(p.B), dim3(1024), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_draft_sample(const FinalizeParams& p, int num_cus, hipStream_t s, Timer* t) {
  if (p.B == 0) return hipSuccess;
  TimedScope ts(t, "draft_sample", s);
  const unsigned n = (unsigned)p.B * (unsigned)p.K;
  // with many vectors, smaller workgroups: more of them share a CU, so one's
  // header and locate overlap the others' streaming
  const unsigned cus = num_cus > 0 ? (unsigned)num_cus : 256u;
  if (n >= 4u * cus)
    hipLaunchKernelGGL(draft_sample_kernel<256>, dim3(n), dim3(256), 0, s, p);
  else if (use_half_blocks(n, num_cus))
    hipLaunchKernelGGL(draft_sample_kernel<512>, dim3(n), dim3(512), 0, s, p);
  else
    hipLaunchKernelGGL(draft_sample_kernel<1024>, dim3(n), dim3(1024), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_shard_draw(const FinalizeParams& p, const ShardDrawParams& d, bool locate,
                             int num_cus, hipStream_t s, Timer* t) {
  if (p.B == 0) return hipSuccess;
  const bool half = use_half_blocks((unsigned)p.B, num_cus);
  if (locate) {
    TimedScope ts(t, "shard_locate", s);
    if (half)
      hipLaunchKernelGGL(shard_locate_kernel<512>, dim3(p.B), dim3(512), 0, s, p, d);
    else
      hipLaunchKernelGGL(shard_locate_kernel<1024>, dim3(p.B), dim3(1024), 0, s, p, d);
  } else {
    TimedScope ts(t, "shard_mass", s);
    if (half)
      hipLaunchKernelGGL(shard_mass_kernel<512>, dim3(p.B), dim3(512), 0, s, p, d);
    else
      hipLaunchKernelGGL(shard_mass_kernel<1024>, dim3(p.B), dim3(1024), 0, s, p, d);
  }
  return hipGetLastError();
}

}  // namespace sv
