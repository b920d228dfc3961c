// prepare: optional top-1 router weight on the input, then the activation
// quantiser ("[vLLM] MoE Oracle & Prepare/Finalize", no-DP/EP prepare code;
// G(128) from the quant-format key of "Fused MoE Kernel Features").
//
// HBM-bound streaming kernel: every thread owns one 16-byte chunk of 8 bf16
// values.  On the fp8 path 16 consecutive lanes own one 128-value group, so
// the group amax is a 4-step butterfly inside the wave; each lane writes its
// 8 codes as one 8-byte store and the group's first lane writes the scale.
#include "moe_device.h"
#include "launch.h"

namespace moe {
namespace {

__device__ __forceinline__ void unpack8(const u32x4& r, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_to_f32(r[i]);
    f[2 * i + 1] = bf16_to_f32(r[i] >> 16);
  }
}

// Weighted input: a = bf16(x * bf16(w)).  The product of two bf16 values is
// exact in fp32, so this is one rounding.
__device__ __forceinline__ void weight8(float* f, float wq) {
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = bf16_to_f32(f32_to_bf16(f[i] * wq));
}

__global__ __launch_bounds__(256) void prepare_bf16_weight_kernel(
    const uint16_t* __restrict__ a1, int chunks_per_row, int64_t total_chunks,
    const float* __restrict__ w, uint16_t* __restrict__ out) {
  const int64_t c = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (c >= total_chunks) return;
  const u32x4 r = *reinterpret_cast<const u32x4*>(a1 + c * 8);
  float f[8];
  unpack8(r, f);
  const float wq = bf16_to_f32(f32_to_bf16(w[c / chunks_per_row]));
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(f[2 * i] * wq, f[2 * i + 1] * wq);
  *reinterpret_cast<u32x4*>(out + c * 8) = o;
}

__global__ __launch_bounds__(256) void prepare_fp8_kernel(
    const uint16_t* __restrict__ a1, int chunks_per_row, int64_t total_chunks,
    const float* __restrict__ w, int apply_weight, uint8_t* __restrict__ q,
    float* __restrict__ scale) {
  const int64_t c = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  // total_chunks is a multiple of 16 (H % 128 == 0), so a 16-lane group is
  // either wholly valid or wholly past the end: the shuffles stay uniform.
  const bool valid = c < total_chunks;
  float f[8];
  if (valid) {
    unpack8(*reinterpret_cast<const u32x4*>(a1 + c * 8), f);
    if (apply_weight) weight8(f, bf16_to_f32(f32_to_bf16(w[c / chunks_per_row])));
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = 0.f;
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, __builtin_fabsf(f[i]));
  amax = group_max<16>(amax);
  const float s = fmaxf(amax, kQuantEps) / kFp8Max;
  u32x2 o;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t word = pack4_e4m3(f[4 * h] / s, f[4 * h + 1] / s, f[4 * h + 2] / s,
                                   f[4 * h + 3] / s);
    o[h] = word;
  }
  if (valid) {
    *reinterpret_cast<u32x2*>(q + c * 8) = o;
    if ((threadIdx.x & 15) == 0) scale[c >> 4] = s;
  }
}

}  // namespace

void launch_prepare(const uint16_t* a1, int T, int H, const float* w, int apply_weight,
                    int quant, void* a1q, float* a1q_scale, hipStream_t s) {
  const int cpr = H / 8;
  const int64_t total = static_cast<int64_t>(T) * cpr;
  const unsigned blocks = static_cast<unsigned>((total + 255) / 256);
  if (quant == 1) {
    prepare_fp8_kernel<<<blocks, 256, 0, s>>>(a1, cpr, total, w, apply_weight,
                                              static_cast<uint8_t*>(a1q), a1q_scale);
  } else if (apply_weight) {
    prepare_bf16_weight_kernel<<<blocks, 256, 0, s>>>(a1, cpr, total, w,
                                                      static_cast<uint16_t*>(a1q));
  } else if (static_cast<const void*>(a1) != a1q) {
    (void)hipMemcpyAsync(a1q, a1, static_cast<size_t>(total) * 16, hipMemcpyDeviceToDevice, s);
  }
}

}  // namespace moe
