// The whole layer in one launch for decode-sized batches: the monolithic
// mode of "[vLLM] MoE Oracle & Prepare/Finalize" (section on modular vs
// monolithic kernels: the monolithic mode fuses routing, the experts and
// finalize into a single kernel), for T <= 512 and T*top_k <= 512, bf16
// weights or fp8 weights (E4M3, 128 x 128 block scales) with G(128)
// activations.
//
// One persistent launch, one 512-thread workgroup per CU the stream may use
// (all resident at once), phases with a grid barrier between each two
// (grid_sync.h: per-workgroup arrival flags tagged with a per-call epoch,
// bounded waits):
//   A  routing: wave t routes token t (route_token, as the routing kernel),
//      ids and weights to the workspace; fp8: x to E4M3 G(128) as prepare
//      quantises.
//   B  first GEMMs: every workgroup sorts the T*top_k routed rows by expert
//      in LDS (flat-index order within an expert, as align orders them) and
//      cuts each expert's rows into 16-row groups.  Work items, one wave
//      each: (routed group, 16 z columns) and (16 tokens, 16 shared z
//      columns).  fp8: z stays fp32, and a phase of its own quantises it to
//      E4M3 G(128) once whole 128-column groups exist.
//   C  second GEMMs: (routed group, 16 H columns, K slice), (16 tokens, 16
//      H columns, K slice), fp32 partials.
//   D  finalize: workgroup g finalizes tokens g, g+G, ... (the slices
//      summed, the weighted sum of the token's rows, shared row, residual,
//      optional RMSNorm, bf16 or fp8 G(128) output), as the finalize kernel.
// A wave computes its 16 output columns for 16 rows at a time with
// 16x16x32 bf16 MFMAs (fp8: 16x16x128, one per k-tile, promoted with the
// block scales), the weight rows as first operand, both operands loaded
// from global memory straight into registers several batches of k-steps
// ahead: at decode sizes each weight byte is read about once and the
// activation rows come from the L2, so nothing is staged in LDS.  Each
// output is a plain fp32 sum over K of the products, rounded once (z after
// the activation, y) -- the modular path's arithmetic in another summation
// order.
#include "moe_device.h"
#include "launch.h"
#include "monolithic.h"
#include "route_device.h"
#include "grid_sync.h"

#include <algorithm>
#include <type_traits>

namespace moe {
namespace {

constexpr int kMonoThreads = 512, kMonoWaves = kMonoThreads / 64;
constexpr int kMonoMaxRows = 512;     // T * top_k (and T)
constexpr int kMonoMaxGroups = kMonoMaxRows + kMonoMaxRows / 16;   // 16-row groups, routed
constexpr int kMonoMaxGrid = kMonoThreads;   // arrival flags (workgroup 0 polls one a thread)
constexpr int kMonoMaxSplit = 8;     // K split of the second GEMMs

struct MonoArgs {
  const uint16_t* x;
  const float* logits;
  int T, H, E, top_k, scoring, renorm, woi, act, gated, fp8;
  const uint16_t* w13;    // [E][G*I][H]  (fp8: the same layout in bytes)
  const uint16_t* w2;     // [E][H][I]
  int I;
  const uint16_t* sw13;   // shared expert [G*Is][H], or null
  const uint16_t* sw2;    // [H][Is]
  int Is;
  // fp8 weights: one fp32 scale per 128 x 128 block, [E][G*I/128][H/128],
  // [E][H/128][I/128], and the shared expert's
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
  // workspace
  int32_t* ids;           // [T*top_k]
  float* wts;             // [T*top_k]
  uint16_t* z;            // [T*top_k][I] bf16 (fp8 weights: E4M3 codes, [T*top_k][I] bytes)
  uint16_t* zsh;          // [T][Is]
  // fp8 weights: x as E4M3 G(128) codes and scales, z before its
  // quantisation (fp32), and the scales of z
  uint8_t* xq;            // [T][H]
  float* xs;              // [T][H/128]
  float* zf;              // [T*top_k][I]
  float* zshf;            // [T][Is]
  float* zs;              // [T*top_k][I/128]
  float* zshs;            // [T][Is/128]
  float* yp;              // second-GEMM partials [S][T*top_k][H]
  float* yshp;            // [S][T][H]
  uint64_t* flags;        // [kMonoMaxGrid] arrival flags, then the go word
  uint64_t epoch;
  int max_split;          // bound on the second GEMMs' K split (the workspace's partials)
};

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ u32x4 ld16(const uint16_t* p) { return *reinterpret_cast<const u32x4*>(p); }

// bf16(f32(v) * s) of 8 packed bf16 values (weight on the input: the
// product of two bf16 numbers is exact in f32, one rounding).
__device__ __forceinline__ u32x4 scale8(u32x4 v, float s) {
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    o[i] = f32_to_bf16(bf16_to_f32(v[i]) * s) | (f32_to_bf16(bf16_to_f32(v[i] >> 16) * s) << 16);
  return o;
}

// One wave: acc[g][v] += sum over k in [k0, k0 + K) of a[row r16][k] *
// w_g[4q + v][k] for the lane's activation row arow and G weight rows (the
// lane's row r16 of each 16-row fragment).  Output column r16 depends on
// activation row r16 alone, so lanes without a row of their own read any
// valid row and leave their column unstored.  K a
// multiple of 32 * U.  WOI: the activation row is first multiplied by aw
// and rounded to bf16 (weight on the input).  Batches of U k-steps in a ring
// of three: two batches load while one feeds the MFMAs.  Inside the main
// loop every batch issues its loads (past the last batch they fetch the
// last one again, into a slot that is not read), so the compiler's count of
// the loads in flight stays exact across the loop and its waits cover only
// the batch about to be used.
template <int G, int U, bool WOI>
__device__ __forceinline__ void wave_gemm(const uint16_t* arow, float aw,
                                          const uint16_t* const (&wrow)[G], int k0, int K, int q,
                                          f32x4 (&acc)[G]) {
  u32x4 A[3][U], W[3][U][G];
  const int nb = K / (32 * U);
  auto load = [&](int b, int buf) {
    b = min(b, nb - 1);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = k0 + (b * U + u) * 32 + 8 * q;
      A[buf][u] = ld16(arow + k);
#pragma unroll
      for (int g = 0; g < G; ++g) W[buf][u][g] = ld16(wrow[g] + k);
    }
  };
  auto comp = [&](int buf) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const u32x4 a = WOI ? scale8(A[buf][u], aw) : A[buf][u];
#pragma unroll
      for (int g = 0; g < G; ++g)
        acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, W[buf][u][g]),
                                                         __builtin_bit_cast(bf16x8_t, a), acc[g], 0, 0, 0);
    }
  };
  load(0, 0);
  load(1, 1);
  int b = 0;
  for (; b + 3 <= nb; b += 3) {
    load(b + 2, 2);
    comp(0);
    load(b + 3, 0);
    comp(1);
    load(b + 4, 1);
    comp(2);
  }
  // the last nb mod 3 batches: b in slot 0, b+1 in slot 1
  if (b < nb) comp(0);
  if (b + 1 < nb) comp(1);
}

template <int G, bool WOI>
__device__ __forceinline__ void wave_gemm_k(const uint16_t* arow, float aw,
                                            const uint16_t* const (&wrow)[G], int k0, int K, int q,
                                            f32x4 (&acc)[G]) {
  if (K % 128 == 0) wave_gemm<G, 4, WOI>(arow, aw, wrow, k0, K, q, acc);
  else wave_gemm<G, 2, WOI>(arow, aw, wrow, k0, K, q, acc);
}

// The routed rows sorted by expert (LDS): rows[p] is the p-th flat row
// t*top_k+j in expert order, flat order within an expert; the touched
// experts' rows cut into groups of up to 16 (a group never spans two
// experts): group g < n_groups belongs to expert slot_e[grp_slot[g]] and
// holds rows rows[grp_row0[g] .. grp_row1[g]).  The shared expert's groups
// follow (tokens 16 j ..), n_sgroups of them.
struct RowTable {
  int ids[kMonoMaxRows];
  int rows[kMonoMaxRows];
  int slot_e[kMonoMaxRows];
  int slot_off[kMonoMaxRows + 1];
  int grp_slot[kMonoMaxGroups];
  int grp_row0[kMonoMaxGroups];
  int grp_row1[kMonoMaxGroups];
  int wsum[kMonoWaves];
  int n_slots, n_groups, n_sgroups;
  int ksplit;           // the second GEMMs' K split (see phase_gemm2)
};

// Exclusive prefix sum of v over the workgroup's threads (thread order);
// *total gets the sum.  Every thread calls it.
__device__ int block_scan(int v, int* wsum, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kMonoWaves; ++w) {
    before += w < wave ? wsum[w] : 0;
    all += wsum[w];
  }
  __syncthreads();
  *total = all;
  return before + x - v;
}

__device__ void build_rows(const MonoArgs& a, RowTable& tb, int nw) {
  const int tid = threadIdx.x;
  const int n = a.T * a.top_k;
  static_assert(kMonoThreads >= kMonoMaxRows, "a thread per routed row");
  if (tid < n) tb.ids[tid] = a.ids[tid];
  __syncthreads();
  // row tid's place: rows of smaller experts, then earlier rows of its own
  if (tid < n) {
    const int my = tb.ids[tid];
    int pos = 0;
    for (int j = 0; j < n; ++j) {
      const int o = tb.ids[j];
      pos += (o < my) | ((o == my) & (j < tid));
    }
    tb.rows[pos] = tid;
  }
  __syncthreads();
  // touched experts: a slot where the expert changes along rows[]
  int e = -1;
  bool first = false;
  if (tid < n) {
    e = tb.ids[tb.rows[tid]];
    first = tid == 0 || e != tb.ids[tb.rows[tid - 1]];
  }
  int ns = 0;
  const int slot = block_scan(first ? 1 : 0, tb.wsum, &ns);
  if (first) {
    tb.slot_e[slot] = e;
    tb.slot_off[slot] = tid;
  }
  if (tid == 0) tb.slot_off[ns] = n;
  __syncthreads();
  // 16-row groups of each slot
  int ng = 0;
  if (tid < ns) ng = (tb.slot_off[tid + 1] - tb.slot_off[tid] + 15) / 16;
  int total = 0;
  const int g0 = block_scan(ng, tb.wsum, &total);
  if (tid < ns)
    for (int j = 0; j < ng; ++j) {
      tb.grp_slot[g0 + j] = tid;
      tb.grp_row0[g0 + j] = tb.slot_off[tid] + 16 * j;
      tb.grp_row1[g0 + j] = min(tb.slot_off[tid] + 16 * j + 16, tb.slot_off[tid + 1]);
    }
  if (tid == 0) {
    tb.n_slots = ns;
    tb.n_groups = total;
    tb.n_sgroups = a.sw13 ? (a.T + 15) / 16 : 0;
    // Second GEMMs: split K in S (a power of two up to a.max_split) while the
    // items still fit the waves twice over and every slice stays whole 64-deep
    // batches -- at T = 1 the H/16 column items of one or two experts leave
    // most waves idle otherwise.
    const int items = (total + tb.n_sgroups) * (a.H / 16);
    int S = 1;
    const int kq = a.fp8 ? 128 : 64;     // slices of whole batches (fp8: k-tiles)
    while (S < a.max_split && items * S * 2 <= nw && a.I % (2 * S * kq) == 0 &&
           (!a.sw2 || a.Is % (2 * S * kq) == 0))
      S *= 2;
    tb.ksplit = S;
  }
  __syncthreads();
}

// Phase B: first GEMMs.  Item i < n_groups * I/16: routed row group
// i / (I/16), z columns 16 (i mod I/16) ..; then the shared expert's row
// groups times Is/16 columns.
template <int G>
__device__ void phase_gemm1(const MonoArgs& a, const RowTable& tb, int gw, int nw) {
  const int lane = threadIdx.x & 63, q = lane >> 4, r16 = lane & 15;
  const int cw = a.I / 16, cs = a.Is / 16;
  const int routed = tb.n_groups * cw;
  const int total = routed + tb.n_sgroups * cs;
  for (int it = gw; it < total; it += nw) {
    const bool shared = it >= routed;
    const int j = shared ? it - routed : it;
    const int grp = shared ? j / cs : j / cw;
    const int c = shared ? j % cs : j % cw;
    const int In = shared ? a.Is : a.I;
    const uint16_t* wb = shared ? a.sw13
                                : a.w13 + static_cast<int64_t>(tb.slot_e[tb.grp_slot[grp]]) * G * a.I * a.H;
    const uint16_t* wrow[G];
    wrow[0] = wb + static_cast<int64_t>(16 * c + r16) * a.H;
    if constexpr (G == 2) wrow[1] = wb + static_cast<int64_t>(In + 16 * c + r16) * a.H;
    // this lane's row of the group: a token (shared) or a flat routed row
    int flat = -1, tok = -1;
    if (shared) {
      if (16 * grp + r16 < a.T) tok = flat = 16 * grp + r16;
    } else if (tb.grp_row0[grp] + r16 < tb.grp_row1[grp]) {
      flat = tb.rows[tb.grp_row0[grp] + r16];
      tok = flat / a.top_k;
    }
    const bool woi = a.woi && !shared;   // the shared expert reads the unweighted input
    float aw = 1.0f;
    if (woi && flat >= 0) aw = bf16_to_f32(f32_to_bf16(a.wts[flat]));
    f32x4 acc[G];
#pragma unroll
    for (int g = 0; g < G; ++g) acc[g] = f32x4{0.f, 0.f, 0.f, 0.f};
    // (lanes without a row read token 0; their column is not stored)
    const uint16_t* arow = a.x + static_cast<int64_t>(tok >= 0 ? tok : 0) * a.H;
    if (woi) wave_gemm_k<G, true>(arow, aw, wrow, 0, a.H, q, acc);
    else wave_gemm_k<G, false>(arow, aw, wrow, 0, a.H, q, acc);
    if (flat >= 0) {
      uint16_t* zr = (shared ? a.zsh + static_cast<int64_t>(flat) * a.Is
                             : a.z + static_cast<int64_t>(flat) * a.I) + 16 * c + 4 * q;
      float zv[4];
#pragma unroll
      for (int v = 0; v < 4; ++v)
        zv[v] = G == 2 ? act_apply(a.act, acc[0][v]) * acc[G - 1][v] : act_apply(a.act, acc[0][v]);
      u32x2 pk;
      pk[0] = f32_to_bf16_hw(zv[0]) | (f32_to_bf16_hw(zv[1]) << 16);
      pk[1] = f32_to_bf16_hw(zv[2]) | (f32_to_bf16_hw(zv[3]) << 16);
      *reinterpret_cast<u32x2*>(zr) = pk;
    }
  }
}

// Phase C: second GEMMs in fp32 partials over S slices of K (S =
// tb.ksplit).  Item i < n_groups * H/16 * S: slice i mod S of routed row
// group (i / S) / (H/16), H columns 16 ((i / S) mod H/16) ..; then the
// shared expert's groups likewise.  Finalize sums the slices in order and
// rounds once to bf16, the value of an unsplit sum up to its order.
__device__ void phase_gemm2(const MonoArgs& a, const RowTable& tb, int gw, int nw) {
  const int lane = threadIdx.x & 63, q = lane >> 4, r16 = lane & 15;
  const int ch = a.H / 16, S = tb.ksplit;
  const int n = a.T * a.top_k;
  const int routed = tb.n_groups * ch * S;
  const int total = routed + tb.n_sgroups * ch * S;
  for (int it = gw; it < total; it += nw) {
    const bool shared = it >= routed;
    const int j = shared ? it - routed : it;
    const int sp = j % S, rest = j / S;
    const int grp = rest / ch, c = rest % ch;
    const int K = shared ? a.Is : a.I;
    const int Ks = K / S;
    const uint16_t* wb = shared ? a.sw2
                                : a.w2 + static_cast<int64_t>(tb.slot_e[tb.grp_slot[grp]]) * a.H * a.I;
    const uint16_t* wrow[1] = {wb + static_cast<int64_t>(16 * c + r16) * K};
    int flat = -1, src;
    if (shared) {
      if (16 * grp + r16 < a.T) flat = 16 * grp + r16;
      src = flat >= 0 ? flat : 16 * grp;
    } else {
      if (tb.grp_row0[grp] + r16 < tb.grp_row1[grp]) flat = tb.rows[tb.grp_row0[grp] + r16];
      src = flat >= 0 ? flat : tb.rows[tb.grp_row0[grp]];
    }
    // (lanes without a row read the group's first row; not stored)
    const uint16_t* arow = shared ? a.zsh + static_cast<int64_t>(src) * a.Is
                                  : a.z + static_cast<int64_t>(src) * a.I;
    f32x4 acc[1] = {f32x4{0.f, 0.f, 0.f, 0.f}};
    wave_gemm_k<1, false>(arow, 1.0f, wrow, sp * Ks, Ks, q, acc);
    if (flat >= 0) {
      float* yr = shared ? a.yshp + (static_cast<int64_t>(sp) * a.T + flat) * a.H
                         : a.yp + (static_cast<int64_t>(sp) * n + flat) * a.H;
      *reinterpret_cast<f32x4*>(yr + 16 * c + 4 * q) = acc[0];
    }
  }
}

// 8 columns of a second-GEMM output row from its S fp32 slices: summed in
// slice order, rounded to bf16 (the layer's y), returned as floats.
__device__ __forceinline__ void y8(const float* p, int64_t slice_stride, int S, float* f) {
  f32x4 lo = *reinterpret_cast<const f32x4*>(p), hi = *reinterpret_cast<const f32x4*>(p + 4);
  for (int sp = 1; sp < S; ++sp) {
    lo += *reinterpret_cast<const f32x4*>(p + sp * slice_stride);
    hi += *reinterpret_cast<const f32x4*>(p + sp * slice_stride + 4);
  }
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    f[v] = bf16_to_f32(f32_to_bf16_hw(lo[v]));
    f[4 + v] = bf16_to_f32(f32_to_bf16_hw(hi[v]));
  }
}

__device__ __forceinline__ void unpack8f(u32x4 r, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_to_f32(r[i]);
    f[2 * i + 1] = bf16_to_f32(r[i] >> 16);
  }
}

// Phase D: finalize of token t by the workgroup; thread tid owns the
// 8-column chunks tid + 512 i.  acc = sum_j w'_j y[t, j] (slot order; w' = 1
// with the weight on the input) + shared row + residual; residual_out =
// bf16(acc); with gamma, out = acc * (1 / sqrt(mean(acc^2) + eps)) * gamma;
// bf16 out, or E4M3 with one scale per 128 columns.
__device__ void finalize_token(const MonoArgs& a, int t, int S, float* part) {
  constexpr int MAXC = 4;                   // H <= 16384
  const int tid = threadIdx.x;
  const int nch = a.H / 8;
  const int64_t row = static_cast<int64_t>(t) * a.H;
  float acc[MAXC][8];
  float sumsq = 0.f;
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int c = tid + kMonoThreads * i;
#pragma unroll
    for (int v = 0; v < 8; ++v) acc[i][v] = 0.f;
    if (c < nch) {
      for (int j = 0; j < a.top_k; ++j) {
        const int f = t * a.top_k + j;
        const float wj = a.woi ? 1.0f : a.wts[f];
        float yv[8];
        y8(a.yp + static_cast<int64_t>(f) * a.H + c * 8, static_cast<int64_t>(a.T) * a.top_k * a.H, S,
           yv);
#pragma unroll
        for (int v = 0; v < 8; ++v) acc[i][v] += wj * yv[v];
      }
      if (a.sw2) {
        float sv[8];
        y8(a.yshp + row + c * 8, static_cast<int64_t>(a.T) * a.H, S, sv);
#pragma unroll
        for (int v = 0; v < 8; ++v) acc[i][v] += sv[v];
      }
      if (a.residual) {
        float rv[8];
        unpack8f(ld16(a.residual + row + c * 8), rv);
#pragma unroll
        for (int v = 0; v < 8; ++v) acc[i][v] += rv[v];
      }
      if (a.residual_out) {
        u32x4 o;
#pragma unroll
        for (int h = 0; h < 4; ++h) o[h] = pack_bf16x2(acc[i][2 * h], acc[i][2 * h + 1]);
        *reinterpret_cast<u32x4*>(a.residual_out + row + c * 8) = o;
      }
#pragma unroll
      for (int v = 0; v < 8; ++v) sumsq += acc[i][v] * acc[i][v];
    }
  }
  float r = 1.0f;
  if (a.gamma) {
    const float ws = wave_sum(sumsq);
    if ((tid & 63) == 0) part[tid >> 6] = ws;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < kMonoWaves; ++w) tot += part[w];
    __syncthreads();                        // part is reused by the next token
    r = 1.0f / sqrtf(tot / static_cast<float>(a.H) + a.eps);
  }
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int c = tid + kMonoThreads * i;
    float o[8];
    if (c < nch && a.gamma) {
      float g[8];
      unpack8f(ld16(a.gamma + c * 8), g);
#pragma unroll
      for (int v = 0; v < 8; ++v) o[v] = acc[i][v] * r * g[v];
    } else {
#pragma unroll
      for (int v = 0; v < 8; ++v) o[v] = acc[i][v];
    }
    if (a.out_fp8) {
      // nch is a multiple of 16 (H % 128 == 0): 16-lane groups are uniform
      if (kMonoThreads * i < nch) {
        float amax = 0.f;
#pragma unroll
        for (int v = 0; v < 8; ++v) amax = fmaxf(amax, __builtin_fabsf(o[v]));
        amax = group_max<16>(amax);
        const float s = fmaxf(amax, kQuantEps) / kFp8Max;
        if (c < nch) {
          u32x2 qv;
          qv[0] = pack4_e4m3(o[0] / s, o[1] / s, o[2] / s, o[3] / s);
          qv[1] = pack4_e4m3(o[4] / s, o[5] / s, o[6] / s, o[7] / s);
          *reinterpret_cast<u32x2*>(static_cast<uint8_t*>(a.out) + row + c * 8) = qv;
          if ((tid & 15) == 0) a.out_scale[static_cast<int64_t>(t) * (a.H / 128) + (c >> 4)] = s;
        }
      }
    } else if (c < nch) {
      u32x4 ov;
#pragma unroll
      for (int h = 0; h < 4; ++h) ov[h] = pack_bf16x2(o[2 * h], o[2 * h + 1]);
      *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(a.out) + row + c * 8) = ov;
    }
  }
}

// ---- fp8 weights ----------------------------------------------------------

// Rows of width W (a multiple of 128) to E4M3 G(128) codes and one scale per
// 128 columns, as prepare and the first GEMM's epilogue quantise: s =
// max(amax, 1e-10) / 448, code = RNE(v / s).  Item = (row, 512 columns),
// one wave each: lane l holds 8 columns, 16 lanes a 128-column group.
template <class SRC>
__device__ void quant_rows(const SRC* src, int rows, int W, uint8_t* q, float* sc, int gw, int nw) {
  const int lane = threadIdx.x & 63;
  const int per = (W + 511) / 512;
  for (int it = gw; it < rows * per; it += nw) {
    const int r = it / per, c0 = (it % per) * 512 + 8 * lane;
    // lanes past the row (whole 16-lane groups: W % 128 == 0) take zeros
    // through the group maximum and store nothing
    const bool valid = c0 < W;
    float f[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (!valid) {
    } else if constexpr (sizeof(SRC) == 2) {
      const u32x4 v = ld16(reinterpret_cast<const uint16_t*>(src) + static_cast<int64_t>(r) * W + c0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f[2 * i] = bf16_to_f32(v[i]);
        f[2 * i + 1] = bf16_to_f32(v[i] >> 16);
      }
    } else {
      const float* p = reinterpret_cast<const float*>(src) + static_cast<int64_t>(r) * W + c0;
      const f32x4 lo = *reinterpret_cast<const f32x4*>(p), hi = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f[i] = lo[i];
        f[4 + i] = hi[i];
      }
    }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, __builtin_fabsf(f[i]));
    amax = group_max<16>(amax);
    const float s = fmaxf(amax, kQuantEps) / kFp8Max;
    u32x2 o;
    o[0] = pack4_e4m3(f[0] / s, f[1] / s, f[2] / s, f[3] / s);
    o[1] = pack4_e4m3(f[4] / s, f[5] / s, f[6] / s, f[7] / s);
    if (valid) {
      *reinterpret_cast<u32x2*>(q + static_cast<int64_t>(r) * W + c0) = o;
      if ((lane & 15) == 0) sc[static_cast<int64_t>(r) * (W / 128) + c0 / 128] = s;
    }
  }
}

// One wave, fp8: acc[g][v] += sum over k-tiles kt in [kt0, kt0 + nkt) of
// (sum over the k-tile of a[row r16][k] * w_g[4q + v][k]) * sa[kt] * sw_g[kt]:
// one 16x16x128 MFMA per k-tile and fragment from zero, promoted with the
// row's activation scale and the fragment's weight-block scale (the 16 rows
// lie in one 128-row block) -- the fp8 tiles' arithmetic.  Lane group q
// holds bytes [32q, 32q+32) of each k-tile row.  One k-tile per batch, a
// ring of four: three load while one feeds the MFMAs; every batch issues its
// loads (clamped to the last k-tile) so the compiler's count stays exact.
template <int G>
__device__ __forceinline__ void wave_gemm_fp8(const uint8_t* arow, const float* asc,
                                              const uint8_t* const (&wrow)[G],
                                              const float* const (&wsc)[G], int kt0, int nkt, int q,
                                              f32x4 (&acc)[G]) {
  i32x8 A[4], W[4][G];
  float SA[4], SW[4][G];
  auto load = [&](int b, int buf) {
    const int kt = kt0 + min(b, nkt - 1);
    const int64_t k = static_cast<int64_t>(kt) * 128 + 32 * q;
    const u32x4 a0 = *reinterpret_cast<const u32x4*>(arow + k);
    const u32x4 a1 = *reinterpret_cast<const u32x4*>(arow + k + 16);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      A[buf][i] = a0[i];
      A[buf][4 + i] = a1[i];
    }
    SA[buf] = asc[kt];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const u32x4 w0 = *reinterpret_cast<const u32x4*>(wrow[g] + k);
      const u32x4 w1 = *reinterpret_cast<const u32x4*>(wrow[g] + k + 16);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        W[buf][g][i] = w0[i];
        W[buf][g][4 + i] = w1[i];
      }
      SW[buf][g] = wsc[g][kt];
    }
  };
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  auto comp = [&](int buf) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const f32x4 p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(W[buf][g], A[buf], zero, 0, 0, 0,
                                                                       0, 0, 0);
      const float sc = SA[buf] * SW[buf][g];
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[g][v] += p[v] * sc;
    }
  };
  load(0, 0);
  load(1, 1);
  load(2, 2);
  int b = 0;
  for (; b + 4 <= nkt; b += 4) {
    load(b + 3, 3);
    comp(0);
    load(b + 4, 0);
    comp(1);
    load(b + 5, 1);
    comp(2);
    load(b + 6, 2);
    comp(3);
  }
  // the last nkt mod 4 k-tiles: b, b+1, b+2 in slots 0, 1, 2
  if (b < nkt) comp(0);
  if (b + 1 < nkt) comp(1);
  if (b + 2 < nkt) comp(2);
}

// Phase B, fp8: as phase_gemm1, z = act(gate) * up in fp32 (quantised by
// the next phase, which sees whole 128-column groups).
template <int G>
__device__ void phase_gemm1_fp8(const MonoArgs& a, const RowTable& tb, int gw, int nw) {
  const int lane = threadIdx.x & 63, q = lane >> 4, r16 = lane & 15;
  const int cw = a.I / 16, cs = a.Is / 16;
  const int routed = tb.n_groups * cw;
  const int total = routed + tb.n_sgroups * cs;
  const int kb = a.H / 128;
  for (int it = gw; it < total; it += nw) {
    const bool shared = it >= routed;
    const int j = shared ? it - routed : it;
    const int grp = shared ? j / cs : j / cw;
    const int c = shared ? j % cs : j % cw;
    const int In = shared ? a.Is : a.I;
    const int e = shared ? 0 : tb.slot_e[tb.grp_slot[grp]];
    const uint8_t* wb = reinterpret_cast<const uint8_t*>(shared ? a.sw13 : a.w13) +
                        static_cast<int64_t>(e) * G * a.I * a.H;
    const float* sb = (shared ? a.sw13s : a.w13s) + static_cast<int64_t>(e) * (G * a.I / 128) * kb;
    const uint8_t* wrow[G];
    const float* wsc[G];
    wrow[0] = wb + static_cast<int64_t>(16 * c + r16) * a.H;
    wsc[0] = sb + static_cast<int64_t>((16 * c) / 128) * kb;
    if constexpr (G == 2) {
      wrow[1] = wb + static_cast<int64_t>(In + 16 * c + r16) * a.H;
      wsc[1] = sb + static_cast<int64_t>((In + 16 * c) / 128) * kb;
    }
    int flat = -1, tok = -1;
    if (shared) {
      if (16 * grp + r16 < a.T) tok = flat = 16 * grp + r16;
    } else if (tb.grp_row0[grp] + r16 < tb.grp_row1[grp]) {
      flat = tb.rows[tb.grp_row0[grp] + r16];
      tok = flat / a.top_k;
    }
    // (lanes without a row read token 0; their column is not stored)
    const int t0 = tok >= 0 ? tok : 0;
    f32x4 acc[G];
#pragma unroll
    for (int g = 0; g < G; ++g) acc[g] = f32x4{0.f, 0.f, 0.f, 0.f};
    wave_gemm_fp8<G>(a.xq + static_cast<int64_t>(t0) * a.H, a.xs + static_cast<int64_t>(t0) * kb,
                     wrow, wsc, 0, kb, q, acc);
    if (flat >= 0) {
      float* zr = (shared ? a.zshf + static_cast<int64_t>(flat) * a.Is
                          : a.zf + static_cast<int64_t>(flat) * a.I) + 16 * c + 4 * q;
      f32x4 zv;
#pragma unroll
      for (int v = 0; v < 4; ++v)
        zv[v] = G == 2 ? act_apply(a.act, acc[0][v]) * acc[G - 1][v] : act_apply(a.act, acc[0][v]);
      *reinterpret_cast<f32x4*>(zr) = zv;
    }
  }
}

// Phase C, fp8: as phase_gemm2, on the E4M3 z rows and their scales.
__device__ void phase_gemm2_fp8(const MonoArgs& a, const RowTable& tb, int gw, int nw) {
  const int lane = threadIdx.x & 63, q = lane >> 4, r16 = lane & 15;
  const int ch = a.H / 16, S = tb.ksplit;
  const int n = a.T * a.top_k;
  const int routed = tb.n_groups * ch * S;
  const int total = routed + tb.n_sgroups * ch * S;
  for (int it = gw; it < total; it += nw) {
    const bool shared = it >= routed;
    const int j = shared ? it - routed : it;
    const int sp = j % S, rest = j / S;
    const int grp = rest / ch, c = rest % ch;
    const int K = shared ? a.Is : a.I;
    const int kb = K / 128, nkt = kb / S;
    const int e = shared ? 0 : tb.slot_e[tb.grp_slot[grp]];
    const uint8_t* wb = reinterpret_cast<const uint8_t*>(shared ? a.sw2 : a.w2) +
                        static_cast<int64_t>(e) * a.H * a.I;
    const float* sb = (shared ? a.sw2s : a.w2s) + static_cast<int64_t>(e) * (a.H / 128) * (a.I / 128);
    const uint8_t* wrow[1] = {wb + static_cast<int64_t>(16 * c + r16) * K};
    const float* wsc[1] = {sb + static_cast<int64_t>((16 * c) / 128) * kb};
    int flat = -1, src;
    if (shared) {
      if (16 * grp + r16 < a.T) flat = 16 * grp + r16;
      src = flat >= 0 ? flat : 16 * grp;
    } else {
      if (tb.grp_row0[grp] + r16 < tb.grp_row1[grp]) flat = tb.rows[tb.grp_row0[grp] + r16];
      src = flat >= 0 ? flat : tb.rows[tb.grp_row0[grp]];
    }
    const uint8_t* arow = reinterpret_cast<const uint8_t*>(shared ? a.zsh : a.z) +
                          static_cast<int64_t>(src) * K;
    const float* asc = (shared ? a.zshs : a.zs) + static_cast<int64_t>(src) * kb;
    f32x4 acc[1] = {f32x4{0.f, 0.f, 0.f, 0.f}};
    wave_gemm_fp8<1>(arow, asc, wrow, wsc, sp * nkt, nkt, q, acc);
    if (flat >= 0) {
      float* yr = shared ? a.yshp + (static_cast<int64_t>(sp) * a.T + flat) * a.H
                         : a.yp + (static_cast<int64_t>(sp) * n + flat) * a.H;
      *reinterpret_cast<f32x4*>(yr + 16 * c + 4 * q) = acc[0];
    }
  }
}

template <int VPL, int G, bool FP8>
__global__ __launch_bounds__(kMonoThreads) void moe_monolithic_kernel(MonoArgs a) {
  __shared__ RowTable tb;
  __shared__ float part[kMonoWaves];
  __shared__ int okf;
  const int g = blockIdx.x, G_ = gridDim.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int gw = g * kMonoWaves + wave, nw = G_ * kMonoWaves;
  uint64_t* flags = a.flags;
  uint64_t* go = a.flags + kMonoMaxGrid;
  uint64_t ep = a.epoch;
  auto barrier = [&]() {
    __syncthreads();
    ++ep;
    grid_arrive(flags, ep, g);
    return grid_await(flags, go, ep, g, G_, &okf);
  };

  // A: routing, one wave per token (fp8: and x to E4M3 G(128))
  for (int t = gw; t < a.T; t += nw) {
    int e;
    float w;
    route_token<VPL>(a.logits + static_cast<int64_t>(t) * a.E, a.E, a.top_k, a.scoring, a.renorm,
                     &e, &w);
    if (lane < a.top_k) {
      a.ids[t * a.top_k + lane] = e;
      a.wts[t * a.top_k + lane] = w;
    }
  }
  if constexpr (FP8) quant_rows(a.x, a.T, a.H, a.xq, a.xs, gw, nw);
  if (!barrier()) return;

  // B: first GEMMs
  build_rows(a, tb, nw);
  if constexpr (FP8) {
    phase_gemm1_fp8<G>(a, tb, gw, nw);
    if (!barrier()) return;
    // z to E4M3 G(128): the routed rows, then the shared expert's
    quant_rows(a.zf, a.T * a.top_k, a.I, reinterpret_cast<uint8_t*>(a.z), a.zs, gw, nw);
    if (a.sw13) quant_rows(a.zshf, a.T, a.Is, reinterpret_cast<uint8_t*>(a.zsh), a.zshs, gw, nw);
  } else {
    phase_gemm1<G>(a, tb, gw, nw);
  }
  if (!barrier()) return;

  // C: second GEMMs
  if constexpr (FP8) phase_gemm2_fp8(a, tb, gw, nw);
  else phase_gemm2(a, tb, gw, nw);
  if (!barrier()) return;

  // D: finalize
  for (int t = g; t < a.T; t += G_) finalize_token(a, t, tb.ksplit, part);
}

template <int VPL, bool FP8>
void launch_vpl(const MonoArgs& a, int grid, hipStream_t s) {
  if (a.gated) moe_monolithic_kernel<VPL, 2, FP8><<<grid, kMonoThreads, 0, s>>>(a);
  else moe_monolithic_kernel<VPL, 1, FP8><<<grid, kMonoThreads, 0, s>>>(a);
}

size_t align_up(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }

}  // namespace

bool monolithic_fits(int T, int top_k) {
  return T >= 1 && T <= kMonoMaxRows && static_cast<int64_t>(T) * top_k <= kMonoMaxRows;
}

// The second GEMMs split K only while the items fit the waves twice over;
// with at least H/16 items, and at most kMonoMaxGrid workgroups of
// kMonoWaves waves, S stays below this bound.
static int max_split(int H) {
  const int items = std::max(H / 16, 1);
  int S = 1;
  while (S < kMonoMaxSplit && items * S * 2 <= kMonoMaxGrid * kMonoWaves) S *= 2;
  return S;
}

// Workspace: arrival flags, go word and spare words; ids and weights; z of
// the routed rows and of the shared expert (bf16, or E4M3 bytes in the same
// room); the second GEMMs' fp32 partials; with fp8 weights also x's codes
// and scales, fp32 z before its quantisation, and z's scales.
struct MonoLayout {
  size_t flags, ids, wts, z, zsh, yp, yshp, xq, xs, zf, zshf, zs, zshs, bytes;
};

MonoLayout mono_layout(int T, int H, int top_k, int I, int Is, bool fp8) {
  const size_t n = static_cast<size_t>(T) * top_k, t = static_cast<size_t>(T);
  const size_t ms = static_cast<size_t>(max_split(H));
  MonoLayout L{};
  size_t o = 0;
  auto take = [&](size_t bytes) { const size_t at = o; o += align_up(bytes); return at; };
  L.flags = take((kMonoMaxGrid + 3) * sizeof(uint64_t));
  L.ids = take(n * 4);
  L.wts = take(n * 4);
  L.z = take(n * I * 2);
  L.zsh = take(t * Is * 2);
  L.yp = take(ms * n * H * 4);
  L.yshp = take(ms * t * H * 4);
  if (fp8) {
    L.xq = take(t * H);
    L.xs = take(t * (H / 128) * 4);
    L.zf = take(n * I * 4);
    L.zshf = take(t * Is * 4);
    L.zs = take(n * (I / 128) * 4);
    L.zshs = take(t * (Is / 128) * 4);
  }
  L.bytes = o;
  return L;
}

size_t monolithic_workspace_bytes(int T, int H, int top_k, int I, int Is, bool fp8) {
  return mono_layout(T, H, top_k, I, Is, fp8).bytes;
}

// Workgroups the launch may use: one per CU of the stream's CU mask (the
// kernel fits a CU), 0 if it does not fit at all.
int monolithic_grid(hipStream_t s, bool fp8, bool gated) {
  int nb = 0;
  const void* k = fp8 ? (gated ? reinterpret_cast<const void*>(moe_monolithic_kernel<16, 2, true>)
                               : reinterpret_cast<const void*>(moe_monolithic_kernel<16, 1, true>))
                      : (gated ? reinterpret_cast<const void*>(moe_monolithic_kernel<16, 2, false>)
                               : reinterpret_cast<const void*>(moe_monolithic_kernel<16, 1, false>));
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, k, kMonoThreads, 0) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  if (nb < 1) return 0;
  uint32_t mask[32] = {};
  if (hipExtStreamGetCUMask(s, 32, mask) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  int cus = 0;
  for (uint32_t mk : mask) cus += __builtin_popcount(mk);
  return std::min(cus, kMonoMaxGrid);
}

int launch_monolithic(const MonoLaunch& m, hipStream_t s) {
  const int grid = monolithic_grid(s, m.fp8 != 0, m.gated != 0);
  if (grid <= 0) return -1;
  MonoArgs a{};
  a.x = m.x;
  a.logits = m.logits;
  a.T = m.T;
  a.H = m.H;
  a.E = m.E;
  a.top_k = m.top_k;
  a.scoring = m.scoring;
  a.renorm = m.renorm;
  a.woi = m.woi;
  a.act = m.act;
  a.gated = m.gated;
  a.fp8 = m.fp8;
  a.w13 = m.w13;
  a.w2 = m.w2;
  a.I = m.I;
  a.sw13 = m.Is > 0 ? m.sw13 : nullptr;
  a.sw2 = m.Is > 0 ? m.sw2 : nullptr;
  a.Is = m.Is;
  a.w13s = m.w13s;
  a.w2s = m.w2s;
  a.sw13s = m.Is > 0 ? m.sw13s : nullptr;
  a.sw2s = m.Is > 0 ? m.sw2s : nullptr;
  a.residual = m.residual;
  a.gamma = m.gamma;
  a.eps = m.eps;
  a.out_fp8 = m.out_fp8;
  a.out = m.out;
  a.out_scale = m.out_scale;
  a.residual_out = m.residual_out;
  const MonoLayout L = mono_layout(m.T, m.H, m.top_k, m.I, m.Is, m.fp8 != 0);
  uint8_t* p = static_cast<uint8_t*>(m.ws);
  a.flags = reinterpret_cast<uint64_t*>(p + L.flags);
  a.ids = reinterpret_cast<int32_t*>(p + L.ids);
  a.wts = reinterpret_cast<float*>(p + L.wts);
  a.z = reinterpret_cast<uint16_t*>(p + L.z);
  a.zsh = reinterpret_cast<uint16_t*>(p + L.zsh);
  a.yp = reinterpret_cast<float*>(p + L.yp);
  a.yshp = reinterpret_cast<float*>(p + L.yshp);
  if (m.fp8) {
    a.xq = p + L.xq;
    a.xs = reinterpret_cast<float*>(p + L.xs);
    a.zf = reinterpret_cast<float*>(p + L.zf);
    a.zshf = reinterpret_cast<float*>(p + L.zshf);
    a.zs = reinterpret_cast<float*>(p + L.zs);
    a.zshs = reinterpret_cast<float*>(p + L.zshs);
  }
  a.max_split = max_split(m.H);
  // barriers take epoch + 1, + 2, ...: the low bits start at zero
  a.epoch = next_epoch() & ~static_cast<uint64_t>(7);
  auto go = [&](auto fp8) {
    constexpr bool F = decltype(fp8)::value;
    if (m.E <= 64) launch_vpl<1, F>(a, grid, s);
    else if (m.E <= 128) launch_vpl<2, F>(a, grid, s);
    else if (m.E <= 256) launch_vpl<4, F>(a, grid, s);
    else if (m.E <= 512) launch_vpl<8, F>(a, grid, s);
    else launch_vpl<16, F>(a, grid, s);
  };
  if (m.fp8) go(std::true_type{});
  else go(std::false_type{});
  return 0;
}

}  // namespace moe
