// finalize: the weight-and-reduce over each token's top-k expert rows
// ("[vLLM] MoE Oracle & Prepare/Finalize", no-DP/EP finalize) fused with the
// shared-expert row, residual add, RMSNorm and an optional fp8 G(128) output
// (the single-GPU part of the flashinfer finalize program, "[flashinfer] MoE
// Finalize + AllReduce fusion ...", introduction).
//
// Inside the whole-layer forward, a second GEMM that split its K may leave
// its fp32 partials to finalize (finalize_part_kernel, without RMSNorm): a
// token's expert row is then the sum of its partials in split order,
// rounded to bf16 -- the value the split-K reduction kernel would have
// stored -- before it is weighted, so the output bits do not change and one
// launch is saved.
//
// HBM-bound: one 256-thread workgroup per token; thread tid owns the 16-byte
// chunks c = tid + 256*i of the row (8 bf16 each), so every load and store is
// a coalesced 16-byte access and each operand is read exactly once.  The
// accumulated row stays in registers between the sum-of-squares reduction
// (wave butterfly, then 4 partials in LDS) and the normalised store.  With an
// fp8 output, 16 consecutive lanes own one 128-column group.
#include "moe_device.h"
#include "launch.h"

namespace moe {
namespace {

// The per-token rows are touched exactly once: they are loaded and stored
// with the non-temporal hint, so they do not displace what the caches hold
// for other workgroups (measured on MI355X: 5.1 -> 5.8 TB/s at T=16384).
// gamma, read by every token, uses ordinary loads.
__device__ __forceinline__ u32x4 load16_stream(const uint16_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ void unpack8(const u32x4 r, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_to_f32(r[i]);
    f[2 * i + 1] = bf16_to_f32(r[i] >> 16);
  }
}

__device__ __forceinline__ void load8_stream(const uint16_t* p, float* f) {
  unpack8(load16_stream(p), f);
}

__device__ __forceinline__ void load8(const uint16_t* p, float* f) {
  unpack8(*reinterpret_cast<const u32x4*>(p), f);
}

__device__ __forceinline__ void store8_bf16(uint16_t* p, const float* f) {
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
  __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(p));
}

// The bf16 value of a split row's chunk: its ksplit fp32 partials (slice
// floats apart) summed in split order, rounded to bf16.
// (ksplit <= kMaxSplit; the loads of all splits are issued before the adds)
constexpr int kMaxSplit = 8;
__device__ __forceinline__ void load8_partials(const float* p, int ksplit, int64_t slice, float* f) {
  f32x4 x[kMaxSplit], z[kMaxSplit];
#pragma unroll
  for (int s = 0; s < kMaxSplit; ++s) {
    if (s < ksplit) {
      x[s] = *reinterpret_cast<const f32x4*>(p + s * slice);
      z[s] = *reinterpret_cast<const f32x4*>(p + s * slice + 4);
    }
  }
  float a[8];
#pragma unroll
  for (int v = 0; v < 8; ++v) a[v] = 0.f;
#pragma unroll
  for (int s = 0; s < kMaxSplit; ++s) {
    if (s < ksplit) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        a[v] += x[s][v];
        a[4 + v] += z[s][v];
      }
    }
  }
#pragma unroll
  for (int v = 0; v < 8; ++v) f[v] = bf16_to_f32(f32_to_bf16_hw(a[v]));
}

// Split partials handed to finalize: the routed rows' [ysplit][T*top_k][H]
// and the shared expert's [shsplit][T][H] (either may be null).
struct FinParts {
  const float* y;
  int ysplit;
  const float* sh;
  int shsplit;
};

// KT: top_k when it is one of the common 1, 2, 4, 8 (the row loads are then
// unrolled and all issued before the first add), 0 for any other value.
template <int MAXC, bool FP8OUT, int KT>
__global__ __launch_bounds__(256) void finalize_kernel(
    void* __restrict__ output, float* __restrict__ out_scale,
    const uint16_t* __restrict__ y, const float* __restrict__ w, int top_k, int H,
    int weight_on_input, const uint16_t* __restrict__ shared, const uint16_t* __restrict__ residual,
    uint16_t* __restrict__ residual_out, const uint16_t* __restrict__ gamma, float eps) {
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const int nch = H / 8;
  const size_t row = static_cast<size_t>(t) * H;
  float acc[MAXC][8];
  float sumsq = 0.f;
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int c = tid + 256 * i;
#pragma unroll
    for (int v = 0; v < 8; ++v) acc[i][v] = 0.f;
    if (c < nch) {
      if constexpr (KT > 0) {
        u32x4 r[KT];
#pragma unroll
        for (int j = 0; j < KT; ++j)
          r[j] = load16_stream(y + (static_cast<size_t>(t) * KT + j) * H + c * 8);
#pragma unroll
        for (int j = 0; j < KT; ++j) {
          const float wj = weight_on_input ? 1.0f : w[static_cast<size_t>(t) * KT + j];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            acc[i][2 * q] += wj * bf16_to_f32(r[j][q]);
            acc[i][2 * q + 1] += wj * bf16_to_f32(r[j][q] >> 16);
          }
        }
      } else {
        for (int j = 0; j < top_k; ++j) {
          const float wj = weight_on_input ? 1.0f : w[static_cast<size_t>(t) * top_k + j];
          float f[8];
          load8_stream(y + (static_cast<size_t>(t) * top_k + j) * H + c * 8, f);
#pragma unroll
          for (int v = 0; v < 8; ++v) acc[i][v] += wj * f[v];
        }
      }
      if (shared) {
        float f[8];
        load8_stream(shared + row + c * 8, f);
#pragma unroll
        for (int v = 0; v < 8; ++v) acc[i][v] += f[v];
      }
      if (residual) {
        float f[8];
        load8_stream(residual + row + c * 8, f);
#pragma unroll
        for (int v = 0; v < 8; ++v) acc[i][v] += f[v];
      }
      if (residual_out) store8_bf16(residual_out + row + c * 8, acc[i]);
#pragma unroll
      for (int v = 0; v < 8; ++v) sumsq += acc[i][v] * acc[i][v];
    }
  }
  float r = 1.0f;
  if (gamma) {
    __shared__ float part[4];
    const float ws = wave_sum(sumsq);
    if ((tid & 63) == 0) part[tid >> 6] = ws;
    __syncthreads();
    const float tot = (part[0] + part[1]) + (part[2] + part[3]);
    r = 1.0f / sqrtf(tot / static_cast<float>(H) + eps);
  }
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int c = tid + 256 * i;
    float o[8];
    if (c < nch) {
      float g[8];
      if (gamma) {
        load8(gamma + c * 8, g);
#pragma unroll
        for (int v = 0; v < 8; ++v) o[v] = acc[i][v] * r * g[v];
      } else {
#pragma unroll
        for (int v = 0; v < 8; ++v) o[v] = acc[i][v];
      }
    } else {
#pragma unroll
      for (int v = 0; v < 8; ++v) o[v] = 0.f;
    }
    if constexpr (FP8OUT) {
      // nch is a multiple of 16 (H % 128 == 0): 16-lane groups are uniform.
      if (256 * i < nch) {
        float amax = 0.f;
#pragma unroll
        for (int v = 0; v < 8; ++v) amax = fmaxf(amax, __builtin_fabsf(o[v]));
        amax = group_max<16>(amax);
        const float s = fmaxf(amax, kQuantEps) / kFp8Max;
        if (c < nch) {
          u32x2 q;
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const uint32_t word = pack4_e4m3(o[4 * h] / s, o[4 * h + 1] / s, o[4 * h + 2] / s,
                                   o[4 * h + 3] / s);
            q[h] = word;
          }
          __builtin_nontemporal_store(q, reinterpret_cast<u32x2*>(static_cast<uint8_t*>(output) + row + c * 8));
          if ((tid & 15) == 0) out_scale[static_cast<size_t>(t) * (H / 128) + (c >> 4)] = s;
        }
      }
    } else {
      if (c < nch) store8_bf16(static_cast<uint16_t*>(output) + row + c * 8, o);
    }
  }
}

// Split partials without RMSNorm: nothing needs a whole row, so the
// workgroups tile (token, 2048-column block) and each thread owns one
// 8-column chunk -- at decode sizes the partials are then read by many
// workgroups at once instead of one per token.
template <bool FP8OUT>
__global__ __launch_bounds__(256) void finalize_part_kernel(
    void* __restrict__ output, float* __restrict__ out_scale, const uint16_t* __restrict__ y,
    const float* __restrict__ w, int top_k, int H, int weight_on_input,
    const uint16_t* __restrict__ shared, const uint16_t* __restrict__ residual,
    uint16_t* __restrict__ residual_out, FinParts fp) {
  const int t = blockIdx.x;
  const int c = blockIdx.y * 256 + threadIdx.x;
  const int nch = H / 8;
  const size_t row = static_cast<size_t>(t) * H;
  float acc[8];
#pragma unroll
  for (int v = 0; v < 8; ++v) acc[v] = 0.f;
  if (c < nch) {
    for (int j = 0; j < top_k; ++j) {
      const float wj = weight_on_input ? 1.0f : w[static_cast<size_t>(t) * top_k + j];
      const size_t yrow = (static_cast<size_t>(t) * top_k + j) * H + c * 8;
      float f[8];
      if (fp.y)
        load8_partials(fp.y + yrow, fp.ysplit, static_cast<int64_t>(gridDim.x) * top_k * H, f);
      else
        load8_stream(y + yrow, f);
#pragma unroll
      for (int v = 0; v < 8; ++v) acc[v] += wj * f[v];
    }
    if (fp.sh || shared) {
      float f[8];
      if (fp.sh) load8_partials(fp.sh + row + c * 8, fp.shsplit, static_cast<int64_t>(gridDim.x) * H, f);
      else load8_stream(shared + row + c * 8, f);
#pragma unroll
      for (int v = 0; v < 8; ++v) acc[v] += f[v];
    }
    if (residual) {
      float f[8];
      load8_stream(residual + row + c * 8, f);
#pragma unroll
      for (int v = 0; v < 8; ++v) acc[v] += f[v];
    }
    if (residual_out) store8_bf16(residual_out + row + c * 8, acc);
  }
  if constexpr (FP8OUT) {
    // nch is a multiple of 16 (H % 128 == 0): 16-lane groups are uniform.
    if (blockIdx.y * 256 + (threadIdx.x & ~15) < nch) {
      float amax = 0.f;
#pragma unroll
      for (int v = 0; v < 8; ++v) amax = fmaxf(amax, __builtin_fabsf(acc[v]));
      amax = group_max<16>(amax);
      const float sc = fmaxf(amax, kQuantEps) / kFp8Max;
      u32x2 q;
#pragma unroll
      for (int h = 0; h < 2; ++h)
        q[h] = pack4_e4m3(acc[4 * h] / sc, acc[4 * h + 1] / sc, acc[4 * h + 2] / sc, acc[4 * h + 3] / sc);
      __builtin_nontemporal_store(q, reinterpret_cast<u32x2*>(static_cast<uint8_t*>(output) + row + c * 8));
      if ((threadIdx.x & 15) == 0) out_scale[static_cast<size_t>(t) * (H / 128) + (c >> 4)] = sc;
    }
  } else {
    if (c < nch) store8_bf16(static_cast<uint16_t*>(output) + row + c * 8, acc);
  }
}

template <int MAXC, int KT>
void launch_fin_k(void* out, float* out_scale, int out_quant, const uint16_t* y, const float* w,
                  int T, int k, int H, int woi, const uint16_t* sh, const uint16_t* res,
                  uint16_t* res_out, const uint16_t* gamma, float eps, hipStream_t s) {
  if (out_quant == 1)
    finalize_kernel<MAXC, true, KT><<<T, 256, 0, s>>>(out, out_scale, y, w, k, H, woi, sh, res,
                                                      res_out, gamma, eps);
  else
    finalize_kernel<MAXC, false, KT><<<T, 256, 0, s>>>(out, out_scale, y, w, k, H, woi, sh, res,
                                                       res_out, gamma, eps);
}

template <int MAXC>
void launch_fin(void* out, float* out_scale, int out_quant, const uint16_t* y, const float* w,
                int T, int k, int H, int woi, const uint16_t* sh, const uint16_t* res,
                uint16_t* res_out, const uint16_t* gamma, float eps, hipStream_t s) {
  switch (k) {
    case 1: launch_fin_k<MAXC, 1>(out, out_scale, out_quant, y, w, T, k, H, woi, sh, res, res_out, gamma, eps, s); break;
    case 2: launch_fin_k<MAXC, 2>(out, out_scale, out_quant, y, w, T, k, H, woi, sh, res, res_out, gamma, eps, s); break;
    case 4: launch_fin_k<MAXC, 4>(out, out_scale, out_quant, y, w, T, k, H, woi, sh, res, res_out, gamma, eps, s); break;
    case 8: launch_fin_k<MAXC, 8>(out, out_scale, out_quant, y, w, T, k, H, woi, sh, res, res_out, gamma, eps, s); break;
    default: launch_fin_k<MAXC, 0>(out, out_scale, out_quant, y, w, T, k, H, woi, sh, res, res_out, gamma, eps, s); break;
  }
}

}  // namespace

void launch_finalize(void* out, float* out_scale, int out_quant, const uint16_t* y,
                     const float* w, int T, int k, int H, int woi, const uint16_t* sh,
                     const uint16_t* res, uint16_t* res_out, const uint16_t* gamma, float eps,
                     hipStream_t s, const float* ypart, int ysplit, const float* shpart,
                     int shsplit) {
  const int nch = H / 8;
  if (ypart || shpart) {   // (never with gamma: the forward then reduces the splits first)
    const FinParts fp{ypart, ysplit, shpart, shsplit};
    const dim3 grid(static_cast<unsigned>(T), (nch + 255) / 256);
    if (out_quant == 1)
      finalize_part_kernel<true><<<grid, 256, 0, s>>>(out, out_scale, y, w, k, H, woi, sh, res,
                                                     res_out, fp);
    else
      finalize_part_kernel<false><<<grid, 256, 0, s>>>(out, out_scale, y, w, k, H, woi, sh, res,
                                                      res_out, fp);
    return;
  }
  if (nch <= 256) launch_fin<1>(out, out_scale, out_quant, y, w, T, k, H, woi, sh, res, res_out, gamma, eps, s);
  else if (nch <= 512) launch_fin<2>(out, out_scale, out_quant, y, w, T, k, H, woi, sh, res, res_out, gamma, eps, s);
  else if (nch <= 1024) launch_fin<4>(out, out_scale, out_quant, y, w, T, k, H, woi, sh, res, res_out, gamma, eps, s);
  else launch_fin<8>(out, out_scale, out_quant, y, w, T, k, H, woi, sh, res, res_out, gamma, eps, s);
}

}  // namespace moe
