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

// Lane l's logits l, l+64, ... of one token (-inf past E).
template <int VPL>
__device__ __forceinline__ void load_logits(const float* __restrict__ row, int E, float (&v)[VPL]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = lane + 64 * i;
    v[i] = e < E ? row[e] : -__builtin_inff();
  }
}

// Top-k of TB tokens whose logits the lanes hold (load_logits), the
// tokens' rounds interleaved so that their cross-lane steps overlap; each
// token's operations and their order are those of a single token.  Every
// lane of the wave calls it; lanes j < top_k get slot j's expert in
// e_out[b] and its weight in w_out[b].
template <int VPL, int TB>
__device__ __forceinline__ void route_logits(const float (&v)[TB][VPL], int E, int top_k,
                                             int scoring, int renorm, int (&e_out)[TB],
                                             float (&w_out)[TB]) {
  const int lane = threadIdx.x & 63;
  uint32_t taken[TB];
  float my_v[TB], top_v[TB];
  int my_e[TB];
#pragma unroll
  for (int b = 0; b < TB; ++b) { taken[b] = 0; my_v[b] = 0.f; top_v[b] = 0.f; my_e[b] = 0; }
  for (int j = 0; j < top_k; ++j) {
    float bv[TB];
    int be[TB];
#pragma unroll
    for (int b = 0; b < TB; ++b) {
      bv[b] = -__builtin_inff();
      be[b] = 0x7fffffff;
#pragma unroll
      for (int i = 0; i < VPL; ++i) {
        const int e = lane + 64 * i;
        const bool ok = (e < E) & !((taken[b] >> i) & 1u);
        const bool better = ok & ((v[b][i] > bv[b]) | ((v[b][i] == bv[b]) & (e < be[b])));
        bv[b] = better ? v[b][i] : bv[b];
        be[b] = better ? e : be[b];
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
#pragma unroll
      for (int b = 0; b < TB; ++b) {
        const float ov = __shfl_xor(bv[b], o, 64);
        const int oe = __shfl_xor(be[b], o, 64);
        // branch-free, so the tokens' shuffles can overlap
        const bool better = (ov > bv[b]) | ((ov == bv[b]) & (oe < be[b]));
        bv[b] = better ? ov : bv[b];
        be[b] = better ? oe : be[b];
      }
    }
#pragma unroll
    for (int b = 0; b < TB; ++b) {
      top_v[b] = j == 0 ? bv[b] : top_v[b];
      my_v[b] = lane == j ? bv[b] : my_v[b];
      my_e[b] = lane == j ? be[b] : my_e[b];
      taken[b] |= ((be[b] & 63) == lane ? 1u : 0u) << (be[b] >> 6);
    }
  }
  const bool active = lane < top_k;
#pragma unroll
  for (int b = 0; b < TB; ++b) {
    float w;
    if (scoring == 0) {  // softmax
      if (renorm) {
        const float ex = active ? expf(my_v[b] - top_v[b]) : 0.f;
        w = ex / wave_sum(ex);
      } else {
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < VPL; ++i)
          if (lane + 64 * i < E) s += expf(v[b][i] - top_v[b]);
        w = expf(my_v[b] - top_v[b]) / wave_sum(s);
      }
    } else {  // sigmoid
      const float sg = active ? 1.0f / (1.0f + expf(-my_v[b])) : 0.f;
      w = renorm ? sg / wave_sum(sg) : sg;
    }
    e_out[b] = my_e[b];
    w_out[b] = w;
  }
}

template <int VPL>
__device__ __forceinline__ void route_token(const float* __restrict__ row, int E, int top_k,
                                            int scoring, int renorm, int* e_out, float* w_out) {
  float v[1][VPL];
  load_logits<VPL>(row, E, v[0]);
  int e[1];
  float w[1];
  route_logits<VPL, 1>(v, E, top_k, scoring, renorm, e, w);
  *e_out = e[0];
  *w_out = w[0];
}

}  // namespace moe
