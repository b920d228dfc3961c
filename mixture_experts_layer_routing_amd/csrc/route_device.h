// Top-k routing of one token by one 64-lane wavefront (device side, shared
// by the routing kernel and the decode prologue).
//
// Lane l holds logits l, l+64, l+128, ... of the token in registers.  Each of
// the top_k rounds is a wave-wide argmax (largest logit, ties to the lower
// expert index) by butterfly shuffles; the winner is retired and lane j keeps
// slot j.  The choice is made on the fp32 logits themselves, so ids are exact
// and independent of exp/sigmoid rounding.  Weights follow in fp32 from the
// selected logits (and, for softmax without renormalisation, from the
// wave-reduced max and sum over all E).
#pragma once
#include "moe_device.h"

namespace moe {

// Every lane of the wave calls it; lanes j < top_k get slot j's expert in
// *e_out and its weight in *w_out.
template <int VPL>
__device__ __forceinline__ void route_token(const float* __restrict__ row, int E, int top_k,
                                            int scoring, int renorm, int* e_out, float* w_out) {
  const int lane = threadIdx.x & 63;
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
  *e_out = my_e;
  *w_out = w;
}

}  // namespace moe
