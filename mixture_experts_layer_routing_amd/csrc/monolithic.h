// Host side of the one-launch layer (monolithic.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace moe {

// The whole layer in one launch (monolithic.hip): bf16 or fp8 weights (E4M3
// with 128 x 128 blocks, activations quantised to E4M3 G(128)), T <= 512,
// T*top_k <= 512.  Pointers as moe_forward's; ws holds
// monolithic_workspace_bytes.  Returns -1 (nothing launched) when the kernel
// cannot have one workgroup resident on every CU of the stream.
struct MonoLaunch {
  const uint16_t* x;
  const float* logits;
  int T, H, E, top_k, scoring, renorm, woi, act, gated, fp8;
  const uint16_t* w13;
  const uint16_t* w2;
  int I;
  const uint16_t* sw13;
  const uint16_t* sw2;
  int Is;
  const float* w13s;
  const float* w2s;
  const float* sw13s;
  const float* sw2s;
  const uint16_t* residual;
  const uint16_t* gamma;
  float eps;
  int out_fp8;
  void* out;
  float* out_scale;
  uint16_t* residual_out;
  void* ws;
};
bool monolithic_fits(int T, int top_k);
size_t monolithic_workspace_bytes(int T, int H, int top_k, int I, int Is, bool fp8);
int launch_monolithic(const MonoLaunch& m, hipStream_t s);

}  // namespace moe
