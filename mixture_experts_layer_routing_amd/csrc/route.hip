// Top-k routing: one 64-lane wavefront per token (route_token), four tokens
// per workgroup.
#include "moe_device.h"
#include "route_device.h"
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
  int e;
  float w;
  route_token<VPL>(logits + static_cast<size_t>(t) * E, E, top_k, scoring, renorm, &e, &w);
  if (lane < top_k) {
    ids[static_cast<size_t>(t) * top_k + lane] = e;
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
