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

#include "draw.h"
#include "philox.h"
#include "sv_internal.h"
#include "wave_ops.h"

namespace sv {
namespace {

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
