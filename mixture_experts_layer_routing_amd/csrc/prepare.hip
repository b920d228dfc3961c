// prepare: optional top-1 router weight on the input, then the activation
// quantiser ("[vLLM] MoE Oracle & Prepare/Finalize", no-DP/EP prepare code;
// G(128), A (per token) and T (per tensor) from the quant-format key of
// "Fused MoE Kernel Features").
//
// HBM-bound streaming kernel: every thread owns one 16-byte chunk of 8 bf16
// values.  On the fp8 path 16 consecutive lanes own one 128-value group, so
// the group amax is a 4-step butterfly inside the wave; each lane writes its
// 8 codes as one 8-byte store and the group's first lane writes the scale.
#include <algorithm>

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

// Per-token ("A") fp8: one 256-thread workgroup per row; the row's chunks
// (at most MAXC per thread) stay in registers between the row amax (wave
// butterfly, then 4 partials in LDS) and the quantised store.
template <int MAXC>
__global__ __launch_bounds__(256) void prepare_fp8_token_kernel(
    const uint16_t* __restrict__ a1, int cpr, const float* __restrict__ w, int apply_weight,
    uint8_t* __restrict__ q, float* __restrict__ scale) {
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t row = static_cast<int64_t>(t) * cpr;
  const float wq = apply_weight ? bf16_to_f32(f32_to_bf16(w[t])) : 1.f;
  float f[MAXC][8];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int c = tid + 256 * i;
    if (c < cpr) {
      unpack8(*reinterpret_cast<const u32x4*>(a1 + (row + c) * 8), f[i]);
      if (apply_weight) weight8(f[i], wq);
#pragma unroll
      for (int v = 0; v < 8; ++v) amax = fmaxf(amax, __builtin_fabsf(f[i][v]));
    }
  }
  __shared__ float part[4];
  amax = wave_max(amax);
  if ((tid & 63) == 0) part[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3]));
  const float s = fmaxf(amax, kQuantEps) / kFp8Max;
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int c = tid + 256 * i;
    if (c < cpr) {
      u32x2 o;
      o[0] = pack4_e4m3(f[i][0] / s, f[i][1] / s, f[i][2] / s, f[i][3] / s);
      o[1] = pack4_e4m3(f[i][4] / s, f[i][5] / s, f[i][6] / s, f[i][7] / s);
      *reinterpret_cast<u32x2*>(q + (row + c) * 8) = o;
    }
  }
  if (tid == 0) scale[t] = s;
}

// Per-tensor ("T") fp8, in four launches that need no memset: zero the
// amax slot, fold every chunk's amax into it (float bits of non-negative
// values order like integers, so an integer atomic max is exact and the
// result independent of order), quantise with the tensor scale, and turn
// the amax slot into the scale.
__global__ void prepare_tensor_init_kernel(float* __restrict__ scale) { scale[0] = 0.f; }

__global__ __launch_bounds__(256) void prepare_tensor_amax_kernel(
    const uint16_t* __restrict__ a1, int chunks_per_row, int64_t total_chunks,
    const float* __restrict__ w, int apply_weight, float* __restrict__ amax_slot) {
  float amax = 0.f;
  for (int64_t c = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; c < total_chunks;
       c += static_cast<int64_t>(gridDim.x) * 256) {
    float f[8];
    unpack8(*reinterpret_cast<const u32x4*>(a1 + c * 8), f);
    if (apply_weight) weight8(f, bf16_to_f32(f32_to_bf16(w[c / chunks_per_row])));
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, __builtin_fabsf(f[i]));
  }
  amax = wave_max(amax);
  if ((threadIdx.x & 63) == 0)
    atomicMax(reinterpret_cast<int*>(amax_slot), __float_as_int(amax));
}

__global__ __launch_bounds__(256) void prepare_tensor_quant_kernel(
    const uint16_t* __restrict__ a1, int chunks_per_row, int64_t total_chunks,
    const float* __restrict__ w, int apply_weight, const float* __restrict__ amax_slot,
    uint8_t* __restrict__ q) {
  const int64_t c = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (c >= total_chunks) return;
  const float s = fmaxf(amax_slot[0], kQuantEps) / kFp8Max;
  float f[8];
  unpack8(*reinterpret_cast<const u32x4*>(a1 + c * 8), f);
  if (apply_weight) weight8(f, bf16_to_f32(f32_to_bf16(w[c / chunks_per_row])));
  u32x2 o;
  o[0] = pack4_e4m3(f[0] / s, f[1] / s, f[2] / s, f[3] / s);
  o[1] = pack4_e4m3(f[4] / s, f[5] / s, f[6] / s, f[7] / s);
  *reinterpret_cast<u32x2*>(q + c * 8) = o;
}

__global__ void prepare_tensor_scale_kernel(float* __restrict__ scale) {
  scale[0] = fmaxf(scale[0], kQuantEps) / kFp8Max;
}

template <int MAXC>
void launch_token(const uint16_t* a1, int T, int cpr, const float* w, int apply_weight,
                  uint8_t* q, float* scale, hipStream_t s) {
  prepare_fp8_token_kernel<MAXC><<<T, 256, 0, s>>>(a1, cpr, w, apply_weight, q, scale);
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
  } else if (quant == 2) {
    uint8_t* q = static_cast<uint8_t*>(a1q);
    if (cpr <= 256) launch_token<1>(a1, T, cpr, w, apply_weight, q, a1q_scale, s);
    else if (cpr <= 512) launch_token<2>(a1, T, cpr, w, apply_weight, q, a1q_scale, s);
    else if (cpr <= 1024) launch_token<4>(a1, T, cpr, w, apply_weight, q, a1q_scale, s);
    else launch_token<8>(a1, T, cpr, w, apply_weight, q, a1q_scale, s);
  } else if (quant == 3) {
    prepare_tensor_init_kernel<<<1, 1, 0, s>>>(a1q_scale);
    const unsigned ablocks = static_cast<unsigned>(std::min<int64_t>((total + 255) / 256, 2048));
    prepare_tensor_amax_kernel<<<ablocks, 256, 0, s>>>(a1, cpr, total, w, apply_weight, a1q_scale);
    prepare_tensor_quant_kernel<<<blocks, 256, 0, s>>>(a1, cpr, total, w, apply_weight, a1q_scale,
                                                       static_cast<uint8_t*>(a1q));
    prepare_tensor_scale_kernel<<<1, 1, 0, s>>>(a1q_scale);
  } else if (apply_weight) {
    prepare_bf16_weight_kernel<<<blocks, 256, 0, s>>>(a1, cpr, total, w,
                                                      static_cast<uint16_t*>(a1q));
  } else if (static_cast<const void*>(a1) != a1q) {
    (void)hipMemcpyAsync(a1q, a1, static_cast<size_t>(total) * 16, hipMemcpyDeviceToDevice, s);
  }
}

}  // namespace moe
