// Device helpers shared by the HIP kernels of the fused-MoE layer (gfx950).
//
// Number formats: bf16 travels as raw uint16 bit patterns; fp8 is OCP E4M3
// (bias 7, no infinities, 0x7F/0xFF NaN, largest finite 448), the format of
// the G(128) activation quantisation listed for fp8 on "Fused MoE Kernel
// Features" (quant-format key).  Both encoders below round to nearest, ties
// to even; the fp8 one saturates at +-448.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr float kFp8Max = 448.0f;
constexpr float kQuantEps = 1e-10f;

__device__ __forceinline__ float bf16_to_f32(uint32_t b) {
  return __uint_as_float((b & 0xffffu) << 16);
}

// float32 -> bf16, round to nearest even; NaN -> 0x7FC0, overflow -> inf.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Hardware float32 -> bf16 (v_cvt_pk_bf16_f32, round to nearest even).
__device__ __forceinline__ uint32_t f32_to_bf16_hw(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}

// float32 -> OCP E4M3 code, round to nearest even, saturating to +-448.
__device__ __forceinline__ uint32_t f32_to_e4m3(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t sign = (u >> 24) & 0x80u;
  const float a = __builtin_fabsf(f);
  if (!(a == a)) return sign | 0x7fu;
  if (a >= kFp8Max) return sign | 0x7eu;
  if (a >= 0x1p-6f) {
    // Normal: keep 3 of the 23 mantissa bits, ties to even, then rebias 127 -> 7.
    uint32_t ua = __float_as_uint(a);
    ua += 0x7ffffu + ((ua >> 20) & 1u);
    const uint32_t e = (ua >> 23) - 120u;
    const uint32_t m = (ua >> 20) & 7u;
    return sign | (e << 3) | m;
  }
  // Subnormal (quantum 2^-9); a result of 8 is the smallest normal, code 0x08.
  return sign | static_cast<uint32_t>(__builtin_rintf(a * 512.0f));
}

// Four floats -> four OCP E4M3 codes (byte i holds value i), round to
// nearest even, on the gfx950 packed conversion.  For every finite input
// within +-448 -- all the quantisers here produce, since they divide by
// amax/448 -- it returns exactly f32_to_e4m3's codes: checked on the GPU on
// every code, every midpoint between neighbouring codes and the floats
// either side of it, and 2^20 random values.
__device__ __forceinline__ uint32_t pack4_e4m3(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return static_cast<uint32_t>(w);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Max over aligned groups of `width` lanes (width a power of two <= 64).
template <int width>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int o = width / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ uint64_t lanemask_lt() {
  const uint32_t lane = __lane_id();
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// silu(v) = v / (1 + exp(-v)) with the accurate expf (finalize-side users).
__device__ __forceinline__ float silu(float v) {
  return v / (1.0f + expf(-v));
}

// GEMM-epilogue silu: v * rcp(1 + 2^(-v*log2 e)) on the hardware exp2/rcp
// (about 1 ulp each; the epilogue runs it on every element of a tile).
__device__ __forceinline__ float silu_fast(float v) {
  const float e = __builtin_amdgcn_exp2f(-v * 1.4426950408889634f);
  return v * __builtin_amdgcn_rcpf(1.0f + e);
}

// Exact GELU, v * Phi(v) = v/2 * (1 + erf(v / sqrt 2)), with the device erf.
__device__ __forceinline__ float gelu_erf(float v) {
  return 0.5f * v * (1.0f + erff(v * 0.70710678118654752f));
}

// The first GEMM's activation of the gate value (ACT_SILU or ACT_GELU).
__device__ __forceinline__ float act_apply(int act, float v) {
  return act == 1 ? gelu_erf(v) : silu_fast(v);
}

}  // namespace moe
