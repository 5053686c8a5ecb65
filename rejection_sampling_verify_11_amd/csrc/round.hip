// The two small kernels that close a round on the device.
//
// Dynamic draft length ([SSD] §3.2): per row, the acceptance rate over a
// window of recent rounds moves the next round's k up above one threshold
// and down below another.  One thread per row; the state row holds the
// filled count, the oldest slot, the two window sums and one packed slot
// (accepted | proposed << 16) per round.
//
// Round counter: the Philox offset of the next round, kept in device memory
// so that a captured round needs no host update between replays.  A round
// that ends with both steps takes them in one launch (the controller kernel
// also advances the counter).
#include "sv_internal.h"

namespace sv {
namespace {

__global__ void dynk_kernel(DynkParams p) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  // closing a round: the counter is read by no other thread of this launch
  if (b == 0 && p.offset_dev) *p.offset_dev += p.offset_delta;
  if (b >= p.B) return;
  const int W = p.W;
  int32_t* st = p.state + (int64_t)b * (W + 4);
  const int32_t k = p.k_per_row[b];
  const int32_t acc = p.accepted[b];
  // A flagged row (accepted outside [0, k]) teaches nothing; neither does a
  // k the controller could not have chosen (outside [k_min, k_max]).  The
  // host keeps k_max <= SV_MAX_K, so a slot's 16-bit fields always suffice.
  if (k < p.k_min || k > p.k_max || acc < 0 || acc > k) return;
  int32_t filled = st[0], oldest = st[1], sa = st[2], sp = st[3];
  if (filled < W) {
    st[4 + (oldest + filled) % W] = acc | (k << 16);
    ++filled;
  } else {
    const int32_t gone = st[4 + oldest];
    sa -= gone & 0xFFFF;
    sp -= gone >> 16;
    st[4 + oldest] = acc | (k << 16);
    oldest = (oldest + 1) % W;
  }
  sa += acc;
  sp += k;
  int32_t next = k;
  if (filled == W) {
    if ((int64_t)sa * p.up_den > (int64_t)p.up_num * sp) next = k + 1;
    else if ((int64_t)sa * p.down_den < (int64_t)p.down_num * sp) next = k - 1;
  }
  next = max(p.k_min, min(p.k_max, next));
  st[0] = filled;
  st[1] = oldest;
  st[2] = sa;
  st[3] = sp;
  p.k_per_row[b] = next;
}

__global__ void advance_offset_kernel(uint64_t* offset_dev, uint64_t delta) {
  if (threadIdx.x == 0) *offset_dev += delta;
}

}  // namespace

hipError_t launch_dynk(const DynkParams& p, hipStream_t s, Timer* t) {
  if (p.B == 0 && !p.offset_dev) return hipSuccess;
  TimedScope ts(t, p.offset_dev ? "close_round" : "dynamic_k", s);
  hipLaunchKernelGGL(dynk_kernel, dim3(p.B > 0 ? (p.B + 255) / 256 : 1), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_advance_offset(uint64_t* offset_dev, uint64_t delta, hipStream_t s, Timer* t) {
  TimedScope ts(t, "advance_offset", s);
  hipLaunchKernelGGL(advance_offset_kernel, dim3(1), dim3(64), 0, s, offset_dev, delta);
  return hipGetLastError();
}

}  // namespace sv
