// Split-K reductions for the grouped GEMM.
//
// When a launch has too few output tiles to fill the GPU (decode-sized T:
// a few expert blocks, or the shared expert over a handful of tokens), the
// GEMM cuts K into ksplit ranges and every workgroup writes an fp32 partial
// tile.  These kernels sum the partials in split order (so the result does
// not depend on scheduling) and apply the epilogue the GEMM would have
// applied: the activation (SiLU or GELU, times up when gated) and the bf16 /
// fp8 G(128) store of z for the first GEMM,
// the bf16 store of y to its fused_expert_output (or shared_out) row for
// the second.  The arithmetic matches the GEMM epilogue (act_apply,
// hardware bf16 rounding, the same fp8 quantiser).
//
// One workgroup covers 2048 columns of one row, 8 per thread, so each
// partial read is two 16-byte loads per thread and every store is 16 bytes
// (bf16) or 8 bytes (fp8), coalesced along the row.
#include "moe_device.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kCols = 2048;   // columns per workgroup: 256 threads x 8

__device__ __forceinline__ void sum8(const float* p, int ksplit, int64_t slice, float* f) {
#pragma unroll
  for (int v = 0; v < 8; ++v) f[v] = 0.f;
  for (int s = 0; s < ksplit; ++s) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p + s * slice);
    const f32x4 b = *reinterpret_cast<const f32x4*>(p + s * slice + 4);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      f[v] += a[v];
      f[4 + v] += b[v];
    }
  }
}

__global__ __launch_bounds__(256) void splitk_z_kernel(
    const float* __restrict__ partial, int ksplit, int64_t slice, int ldp,
    const int32_t* __restrict__ ntp, const int32_t* __restrict__ sorted, int nflat, int T,
    int inter, int gated, int act, int fp8, void* __restrict__ z, float* __restrict__ z_scale,
    int ldz) {
  const int r = blockIdx.x;
  const int rows = sorted ? ntp[0] : T;
  if (r >= rows) return;   // whole workgroup
  const int c = blockIdx.y * kCols + threadIdx.x * 8;
  const bool live = c < inter;   // uniform over 16-lane groups: inter % 128 == 0 with fp8
  const bool pad = sorted != nullptr && sorted[r] >= nflat;
  float zv[8];
#pragma unroll
  for (int v = 0; v < 8; ++v) zv[v] = 0.f;
  if (live && !pad) {
    const float* row = partial + static_cast<int64_t>(r) * ldp;
    float g[8];
    sum8(row + c, ksplit, slice, g);
    if (gated) {
      float u[8];
      sum8(row + inter + c, ksplit, slice, u);
#pragma unroll
      for (int v = 0; v < 8; ++v) zv[v] = act_apply(act, g[v]) * u[v];
    } else {
#pragma unroll
      for (int v = 0; v < 8; ++v) zv[v] = act_apply(act, g[v]);
    }
  }
  if (!fp8) {
    if (live) {
      u32x4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        o[i] = f32_to_bf16_hw(zv[2 * i]) | (f32_to_bf16_hw(zv[2 * i + 1]) << 16);
      *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(z) + static_cast<int64_t>(r) * ldz + c) = o;
    }
    return;
  }
  if (!live) return;   // whole 16-lane groups
  float amax = 0.f;
#pragma unroll
  for (int v = 0; v < 8; ++v) amax = fmaxf(amax, __builtin_fabsf(zv[v]));
  amax = group_max<16>(amax);
  const float s = fmaxf(amax, kQuantEps) / kFp8Max;
  u32x2 q;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t word = pack4_e4m3(zv[4 * h] / s, zv[4 * h + 1] / s, zv[4 * h + 2] / s,
                                   zv[4 * h + 3] / s);
    q[h] = word;
  }
  *reinterpret_cast<u32x2*>(static_cast<uint8_t*>(z) + static_cast<int64_t>(r) * ldz + c) = q;
  if ((threadIdx.x & 15) == 0) z_scale[static_cast<int64_t>(r) * (ldz / 128) + c / 128] = s;
}

__global__ __launch_bounds__(256) void splitk_y_kernel(
    const float* __restrict__ partial, int ksplit, int64_t slice, int ldp,
    const int32_t* __restrict__ ntp, const int32_t* __restrict__ sorted, int nflat, int T, int n,
    uint16_t* __restrict__ out, int ldo) {
  const int r = blockIdx.x;
  const int rows = sorted ? ntp[0] : T;
  if (r >= rows) return;
  int orow = r;
  if (sorted) {
    orow = sorted[r];
    if (orow >= nflat) return;   // pad row
  }
  const int c = blockIdx.y * kCols + threadIdx.x * 8;
  if (c >= n) return;
  float y[8];
  sum8(partial + static_cast<int64_t>(r) * ldp + c, ksplit, slice, y);
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = f32_to_bf16_hw(y[2 * i]) | (f32_to_bf16_hw(y[2 * i + 1]) << 16);
  *reinterpret_cast<u32x4*>(out + static_cast<int64_t>(orow) * ldo + c) = o;
}

}  // namespace

void launch_splitk_z(const float* partial, int ksplit, int64_t part_rows, int ldp,
                     int64_t max_rows, const int32_t* ntp, const int32_t* sorted, int nflat,
                     int T, int inter, bool gated, int act, bool fp8, void* z, float* z_scale,
                     int ldz, hipStream_t s) {
  if (max_rows <= 0) return;
  const dim3 grid(static_cast<unsigned>(max_rows), (inter + kCols - 1) / kCols);
  splitk_z_kernel<<<grid, 256, 0, s>>>(partial, ksplit, part_rows * ldp, ldp, ntp, sorted, nflat,
                                       T, inter, gated ? 1 : 0, act, fp8 ? 1 : 0, z, z_scale, ldz);
}

void launch_splitk_y(const float* partial, int ksplit, int64_t part_rows, int ldp,
                     int64_t max_rows, const int32_t* ntp, const int32_t* sorted, int nflat,
                     int T, int n, uint16_t* out, int ldo, hipStream_t s) {
  if (max_rows <= 0) return;
  const dim3 grid(static_cast<unsigned>(max_rows), (n + kCols - 1) / kCols);
  splitk_y_kernel<<<grid, 256, 0, s>>>(partial, ksplit, part_rows * ldp, ldp, ntp, sorted, nflat,
                                       T, n, out, ldo);
}

}  // namespace moe
