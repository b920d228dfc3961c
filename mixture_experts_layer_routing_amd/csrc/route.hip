// Top-k routing: one 64-lane wavefront per token, four tokens per workgroup.
//
// Lane l holds logits l, l+64, l+128, ... of its token in registers.  Each of
// the top_k rounds is a wave-wide argmax (largest logit, ties to the lower
// expert index) by butterfly shuffles; the winner is retired and lane j keeps
// slot j.  The choice is made on the fp32 logits themselves, so ids are exact
// and independent of exp/sigmoid rounding.  Weights follow in fp32 from the
// selected logits (and, for softmax without renormalisation, from the
// wave-reduced max and sum over all E).
#include "moe_device.h"
#include "launch.h"

namespace moe {
namespace {

template <int VPL>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits, int T, int E,
                                                    int top_k, int scoring, int renorm,
                                                    int32_t* __restrict__ ids,
                                                    float* __restrict__ weights) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* row = logits + static_cast<size_t>(t) * E;
  float v[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = lane + 64 * i;
    v[i] = e < E ? row[e] : -__builtin_inff();
  }
  uint32_t taken = 0;
  float my_v = 0.f, top_v = 0.f;
  int my_e = 0;
  for (int j = 0; j < top_k; ++j) {
    float bv = -__builtin_inff();
    int be = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int e = lane + 64 * i;
      const bool ok = e < E && !((taken >> i) & 1u);
      if (ok && (v[i] > bv || (v[i] == bv && e < be))) { bv = v[i]; be = e; }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oe = __shfl_xor(be, o, 64);
      if (ov > bv || (ov == bv && oe < be)) { bv = ov; be = oe; }
    }
    if (j == 0) top_v = bv;
    if (lane == j) { my_v = bv; my_e = be; }
    if ((be & 63) == lane) taken |= 1u << (be >> 6);
  }
  const bool active = lane < top_k;
  float w;
  if (scoring == 0) {  // softmax
    if (renorm) {
      const float ex = active ? expf(my_v - top_v) : 0.f;
      w = ex / wave_sum(ex);
    } else {
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < VPL; ++i)
        if (lane + 64 * i < E) s += expf(v[i] - top_v);
      w = expf(my_v - top_v) / wave_sum(s);
    }
  } else {  // sigmoid
    const float sg = active ? 1.0f / (1.0f + expf(-my_v)) : 0.f;
    w = renorm ? sg / wave_sum(sg) : sg;
  }
  if (active) {
    ids[static_cast<size_t>(t) * top_k + lane] = my_e;
    weights[static_cast<size_t>(t) * top_k + lane] = w;
  }
}

template <int VPL>
void launch_route_vpl(const float* logits, int T, int E, int top_k, int scoring, int renorm,
                      int32_t* ids, float* w, hipStream_t s) {
  const int blocks = (T + 3) / 4;
  route_kernel<VPL><<<blocks, 256, 0, s>>>(logits, T, E, top_k, scoring, renorm, ids, w);
}

}  // namespace

void launch_route(const float* logits, int T, int E, int top_k, int scoring, int renorm,
                  int32_t* ids, float* w, hipStream_t s) {
  if (E <= 64) launch_route_vpl<1>(logits, T, E, top_k, scoring, renorm, ids, w, s);
  else if (E <= 128) launch_route_vpl<2>(logits, T, E, top_k, scoring, renorm, ids, w, s);
  else if (E <= 256) launch_route_vpl<4>(logits, T, E, top_k, scoring, renorm, ids, w, s);
  else if (E <= 512) launch_route_vpl<8>(logits, T, E, top_k, scoring, renorm, ids, w, s);
  else launch_route_vpl<16>(logits, T, E, top_k, scoring, renorm, ids, w, s);
}

}  // namespace moe
