// Grouped GEMM for the experts stage on gfx950 MFMA.
//
// C[m, n] = sum_k A[m, k] * W[n, k] for the rows of one expert at a time: A is
// the activation rows of an M-tile (gathered through sorted_token_ids for the
// first GEMM, contiguous for the second), W the expert's weight matrix stored
// [N, K] row-major, so both operands stream along K.  The experts and their
// block-padded row groups come from align; the shared expert runs the same
// kernel in "dense" mode over all T rows.
//
// Tiling: 256 threads = 4 waves, tile BM x NB (NB = 2*BNZ when gated: BNZ
// gate rows n0.. and the matching BNZ up rows I+n0.., so SiLU-mul is
// elementwise in registers).  Each k-tile is 128 bytes of K per row (64 bf16
// or 128 fp8 elements), staged global -> registers -> LDS, double-buffered
// with one barrier per k-tile; the next tile's global loads are in flight
// while the current one feeds the MFMAs.  LDS rows are 128 B with the 16-byte
// chunk index XOR-swizzled by (row & 7), so the fragment reads (8 lanes = 8
// rows at one chunk column) hit all 32 banks.
//
// MFMA: bf16 v_mfma_f32_32x32x16_bf16 / 16x16x32_bf16; fp8 E4M3
// v_mfma_f32_32x32x64_f8f6f4 / 16x16x128_f8f6f4.  Operand lane layout: lane l
// holds row (l mod MF) and a contiguous run of K (8 bf16 or 32 fp8 values) at
// offset (l div MF) * run; A and B use the same K placement, so the product
// is independent of how the unit orders K internally.
//
// fp8 scales: one fp32 scale per (activation row, 128 of K) and per 128x128
// weight block.  A k-tile is exactly one scale block along K, so each
// fragment's k-tile partial sum is formed from zero and promoted into the
// fp32 accumulator as acc += partial * s_a[row] * s_w[block].
//
// Tile order: workgroups are dealt to the 8 XCDs round-robin; each XCD gets
// a contiguous range of tiles in a grouped order (8 M-blocks down, then the
// next N-tile), so the workgroups resident on one XCD share activation rows
// and weight tiles through that XCD's L2.
#pragma once

#include "moe_device.h"
#include "launch.h"

namespace moe {

enum { A_GATHER = 0, A_ROWS = 1, A_DENSE = 2 };
enum { EPI_Z = 0, EPI_OUT_ROUTED = 1, EPI_OUT_DENSE = 2 };

template <int BM_, int BNZ_, int WAVES_M_, int WAVES_N_, int MF_, bool FP8_, bool GATED_,
          int AMODE_, int EPI_>
struct GemmCfg {
  static constexpr int BM = BM_, BNZ = BNZ_, WAVES_M = WAVES_M_, WAVES_N = WAVES_N_, MF = MF_;
  static constexpr bool FP8 = FP8_, GATED = GATED_;
  static constexpr int AMODE = AMODE_, EPI = EPI_;
};

__device__ __forceinline__ int swz(int row, int chunk) {
  return row * 128 + ((chunk ^ (row & 7)) << 4);
}

template <int MF, bool FP8>
struct Mfma;

template <>
struct Mfma<32, false> {
  typedef f32x16 acc_t;
  typedef u32x4 frag_t;
  static constexpr int NSUB = 4, NACC = 16;
  __device__ static frag_t read(const uint8_t* base, int row, int s, int lane) {
    return *reinterpret_cast<const u32x4*>(base + swz(row, 2 * s + (lane >> 5)));
  }
  __device__ static acc_t mma(const frag_t& a, const frag_t& b, const acc_t& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};

template <>
struct Mfma<16, false> {
  typedef f32x4 acc_t;
  typedef u32x4 frag_t;
  static constexpr int NSUB = 2, NACC = 4;
  __device__ static frag_t read(const uint8_t* base, int row, int s, int lane) {
    return *reinterpret_cast<const u32x4*>(base + swz(row, 4 * s + (lane >> 4)));
  }
  __device__ static acc_t mma(const frag_t& a, const frag_t& b, const acc_t& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};

template <>
struct Mfma<32, true> {
  typedef f32x16 acc_t;
  typedef i32x8 frag_t;
  static constexpr int NSUB = 2, NACC = 16;
  __device__ static frag_t read(const uint8_t* base, int row, int s, int lane) {
    const int c0 = 4 * s + 2 * (lane >> 5);
    const u32x4 lo = *reinterpret_cast<const u32x4*>(base + swz(row, c0));
    const u32x4 hi = *reinterpret_cast<const u32x4*>(base + swz(row, c0 + 1));
    frag_t f;
    f[0] = lo[0]; f[1] = lo[1]; f[2] = lo[2]; f[3] = lo[3];
    f[4] = hi[0]; f[5] = hi[1]; f[6] = hi[2]; f[7] = hi[3];
    return f;
  }
  __device__ static acc_t mma(const frag_t& a, const frag_t& b, const acc_t& c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
  }
};

template <>
struct Mfma<16, true> {
  typedef f32x4 acc_t;
  typedef i32x8 frag_t;
  static constexpr int NSUB = 1, NACC = 4;
  __device__ static frag_t read(const uint8_t* base, int row, int s, int lane) {
    const int c0 = 2 * (lane >> 4);
    const u32x4 lo = *reinterpret_cast<const u32x4*>(base + swz(row, c0));
    const u32x4 hi = *reinterpret_cast<const u32x4*>(base + swz(row, c0 + 1));
    frag_t f;
    f[0] = lo[0]; f[1] = lo[1]; f[2] = lo[2]; f[3] = lo[3];
    f[4] = hi[0]; f[5] = hi[1]; f[6] = hi[2]; f[7] = hi[3];
    (void)s;
    return f;
  }
  __device__ static acc_t mma(const frag_t& a, const frag_t& b, const acc_t& c) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
  }
};

// Row / column of accumulator element v of lane `lane` inside an MF x MF tile.
template <int MF>
__device__ __forceinline__ int acc_row(int v, int lane) {
  if constexpr (MF == 32) return (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
  else return (lane >> 4) * 4 + v;
}
template <int MF>
__device__ __forceinline__ int acc_col(int lane) {
  return lane & (MF - 1);
}

constexpr int cmax(int a, int b) { return a > b ? a : b; }

template <class C>
__global__ __launch_bounds__(256) void grouped_gemm_kernel(GemmParams p) {
  constexpr int BM = C::BM, BNZ = C::BNZ, MF = C::MF;
  constexpr bool FP8 = C::FP8;
  constexpr int G = C::GATED ? 2 : 1;
  constexpr int NB = G * BNZ;
  constexpr int WM = BM / C::WAVES_M, WN = BNZ / C::WAVES_N;
  constexpr int FM = WM / MF, FN = WN / MF;
  static_assert(C::WAVES_M * C::WAVES_N == 4, "4 waves");
  static_assert(FM >= 1 && FN >= 1 && WM % MF == 0 && WN % MF == 0, "wave tile");
  constexpr int A_BYTES = BM * 128, B_BYTES = NB * 128, STAGE = A_BYTES + B_BYTES;
  constexpr int A_CH = (BM * 8 + 255) / 256;
  constexpr int B_CH = NB * 8 / 256;
  static_assert(NB * 8 % 256 == 0, "B tile");
  constexpr int EB = FP8 ? 1 : 2;
  typedef Mfma<MF, FP8> M;
  typedef typename M::acc_t acc_t;
  typedef typename M::frag_t frag_t;
  constexpr int NSUB = M::NSUB, NACC = M::NACC;
  constexpr int SA_BYTES = FP8 ? 2 * BM * 4 : 0;
  constexpr int EPI_BYTES = (C::EPI == EPI_Z && FP8) ? BM * BNZ * 4 : BM * BNZ * 2;
  constexpr int SMEM = cmax(2 * STAGE + SA_BYTES, EPI_BYTES);
  __shared__ __attribute__((aligned(16))) uint8_t smem[SMEM];
  float* sA = reinterpret_cast<float*>(smem + 2 * STAGE);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;

  // ---- tile decode (XCD-aware grouped order) ----
  const int rows_total = (C::AMODE == A_DENSE) ? p.T : p.ntp[0];
  const int n_mblk = (rows_total + BM - 1) / BM;
  const int total = n_mblk * p.n_tiles;
  const int per = (total + 7) >> 3;
  const int jj = blockIdx.x >> 3;
  if (jj >= per) return;
  const int logical = (blockIdx.x & 7) * per + jj;
  if (logical >= total) return;
  constexpr int GM = 8;
  const int grp = logical / (GM * p.n_tiles);
  const int first_m = grp * GM;
  const int gm = min(n_mblk - first_m, GM);
  const int rem = logical - grp * GM * p.n_tiles;
  const int mblk = first_m + rem % gm;
  const int ntile = rem / gm;
  const int m0 = mblk * BM, n0 = ntile * BNZ;

  const uint8_t* wbase = p.w;
  const float* wsbase = p.w_scale;
  if constexpr (C::AMODE != A_DENSE) {
    const int e = p.block_expert[mblk];
    wbase += static_cast<int64_t>(e) * p.w_stride;
    if constexpr (FP8) wsbase += static_cast<int64_t>(e) * p.ws_stride;
  }
  const int nflat = p.T * p.top_k;
  const int kc = tid & 7;
  const int64_t krow_bytes = static_cast<int64_t>(p.K) * EB;
  const int kblocks = p.K / 128;  // fp8: scale blocks along K (= k-tiles)

  // ---- A rows for this thread's chunks ----
  const uint8_t* a_ptr[A_CH];
  bool a_ok[A_CH];
  int a_src[A_CH];
#pragma unroll
  for (int i = 0; i < A_CH; ++i) {
    const int c = tid + 256 * i;
    const int row = c >> 3;
    const bool in = c < BM * 8;
    int src = 0;
    bool ok = false;
    if (in) {
      if constexpr (C::AMODE == A_GATHER) {
        const int sid = p.sorted[m0 + row];
        ok = sid < nflat;
        src = ok ? sid / p.top_k : 0;
      } else if constexpr (C::AMODE == A_ROWS) {
        ok = true;
        src = m0 + row;
      } else {
        ok = m0 + row < p.T;
        src = ok ? m0 + row : 0;
      }
    }
    a_ok[i] = ok;
    a_src[i] = src;
    a_ptr[i] = p.a + static_cast<int64_t>(src) * krow_bytes + kc * 16;
  }
  const uint8_t* b_ptr[B_CH];
#pragma unroll
  for (int i = 0; i < B_CH; ++i) {
    const int brow = (tid + 256 * i) >> 3;
    int wrow;
    if constexpr (C::GATED) wrow = brow < BNZ ? n0 + brow : p.inter + n0 + (brow - BNZ);
    else wrow = n0 + brow;
    b_ptr[i] = wbase + static_cast<int64_t>(wrow) * krow_bytes + kc * 16;
  }
  // fp8 weight-scale rows (gate block, up block) for this N-tile
  const float* sw_row0 = nullptr;
  const float* sw_row1 = nullptr;
  if constexpr (FP8) {
    sw_row0 = wsbase + static_cast<int64_t>(n0 / 128) * kblocks;
    if constexpr (C::GATED) sw_row1 = wsbase + static_cast<int64_t>((p.inter + n0) / 128) * kblocks;
  }

  u32x4 ra[A_CH], rb[B_CH];
  float rsa[A_CH];
  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      if (a_ok[i]) ra[i] = *reinterpret_cast<const u32x4*>(a_ptr[i] + kt * 128);
      else ra[i] = u32x4{0u, 0u, 0u, 0u};
      if constexpr (FP8)
        rsa[i] = (a_ok[i] && kc == 0) ? p.a_scale[static_cast<int64_t>(a_src[i]) * kblocks + kt] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < B_CH; ++i) rb[i] = *reinterpret_cast<const u32x4*>(b_ptr[i] + kt * 128);
  };
  auto sstore = [&](int buf) {
    uint8_t* As = smem + buf * STAGE;
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int c = tid + 256 * i;
      if (c < BM * 8) {
        *reinterpret_cast<u32x4*>(As + swz(c >> 3, kc)) = ra[i];
        if constexpr (FP8) if (kc == 0) sA[buf * BM + (c >> 3)] = rsa[i];
      }
    }
#pragma unroll
    for (int i = 0; i < B_CH; ++i)
      *reinterpret_cast<u32x4*>(As + A_BYTES + swz((tid + 256 * i) >> 3, kc)) = rb[i];
  };

  acc_t acc[G][FM][FN];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int v = 0; v < NACC; ++v) acc[g][fm][fn][v] = 0.f;

  const int nk = p.K / (128 / EB);
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    const uint8_t* As = smem + buf * STAGE;
    const uint8_t* Bs = As + A_BYTES;
    frag_t fa[NSUB][FM], fb[NSUB][G][FN];
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
        fa[s][fm] = M::read(As, wm * WM + fm * MF + (lane & (MF - 1)), s, lane);
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
          fb[s][g][fn] = M::read(Bs, g * BNZ + wn * WN + fn * MF + (lane & (MF - 1)), s, lane);
    }
    if constexpr (!FP8) {
#pragma unroll
      for (int s = 0; s < NSUB; ++s)
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
              acc[g][fm][fn] = M::mma(fa[s][fm], fb[s][g][fn], acc[g][fm][fn]);
    } else {
      const float swg[2] = {sw_row0[kt], C::GATED ? sw_row1[kt] : 0.f};
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) {
        // activation scales of this lane's accumulator rows
        float sa[NACC];
#pragma unroll
        for (int v = 0; v < NACC; ++v) sa[v] = sA[buf * BM + wm * WM + fm * MF + acc_row<MF>(v, lane)];
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int fn = 0; fn < FN; ++fn) {
            acc_t part;
#pragma unroll
            for (int v = 0; v < NACC; ++v) part[v] = 0.f;
#pragma unroll
            for (int s = 0; s < NSUB; ++s) part = M::mma(fa[s][fm], fb[s][g][fn], part);
#pragma unroll
            for (int v = 0; v < NACC; ++v) acc[g][fm][fn][v] += part[v] * (sa[v] * swg[g]);
          }
      }
    }
    if (kt + 1 < nk) sstore(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue ----
  if constexpr (C::EPI == EPI_Z) {
    // z = silu(gate) * up (gated) or silu(h); staged in LDS, then written as
    // whole rows: bf16, or fp8 E4M3 G(128) along I with one scale per row.
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int v = 0; v < NACC; ++v) {
          const int r = wm * WM + fm * MF + acc_row<MF>(v, lane);
          const int cc = wn * WN + fn * MF + acc_col<MF>(lane);
          float z;
          if constexpr (C::GATED) z = silu(acc[0][fm][fn][v]) * acc[G - 1][fm][fn][v];
          else z = silu(acc[0][fm][fn][v]);
          if constexpr (FP8) reinterpret_cast<float*>(smem)[r * BNZ + cc] = z;
          else reinterpret_cast<uint16_t*>(smem)[r * BNZ + cc] = static_cast<uint16_t>(f32_to_bf16(z));
        }
    __syncthreads();
    if constexpr (FP8) {
      static_assert(BNZ == 128, "fp8 z tile is one 128-column group");
      const int ch = tid & 15;
#pragma unroll
      for (int i = 0; i < (BM + 15) / 16; ++i) {
        const int r = (tid >> 4) + 16 * i;
        if (r < BM) {  // uniform per 16-lane group
          const float* zr = reinterpret_cast<const float*>(smem) + r * BNZ + ch * 8;
          float f[8];
          float amax = 0.f;
#pragma unroll
          for (int v = 0; v < 8; ++v) { f[v] = zr[v]; amax = fmaxf(amax, __builtin_fabsf(f[v])); }
          amax = group_max<16>(amax);
          const float s = fmaxf(amax, kQuantEps) / kFp8Max;
          const int grow = m0 + r;
          if (C::AMODE != A_DENSE || grow < p.T) {
            u32x2 q;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              uint32_t word = 0;
#pragma unroll
              for (int v = 0; v < 4; ++v) word |= f32_to_e4m3(f[4 * h + v] / s) << (8 * v);
              q[h] = word;
            }
            *reinterpret_cast<u32x2*>(static_cast<uint8_t*>(p.out) +
                                      static_cast<int64_t>(grow) * p.ldo + n0 + ch * 8) = q;
            if (ch == 0) p.out_scale[static_cast<int64_t>(grow) * (p.ldo / 128) + n0 / 128] = s;
          }
        }
      }
    } else {
      constexpr int CPR = BNZ / 8;  // 16-byte chunks per tile row
      for (int c = tid; c < BM * CPR; c += 256) {
        const int r = c / CPR, ch = c % CPR;
        const int grow = m0 + r;
        if (C::AMODE == A_DENSE && grow >= p.T) continue;
        const u32x4 v = *reinterpret_cast<const u32x4*>(smem + (r * BNZ + ch * 8) * 2);
        *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(p.out) +
                                  static_cast<int64_t>(grow) * p.ldo + n0 + ch * 8) = v;
      }
    }
  } else {
    // y -> bf16 rows of fused_expert_output (row = flat index sorted[m0+r])
    // or of shared_out (row = token m0+r).
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int v = 0; v < NACC; ++v) {
          const int r = wm * WM + fm * MF + acc_row<MF>(v, lane);
          const int cc = wn * WN + fn * MF + acc_col<MF>(lane);
          reinterpret_cast<uint16_t*>(smem)[r * BNZ + cc] =
              static_cast<uint16_t>(f32_to_bf16(acc[0][fm][fn][v]));
        }
    __syncthreads();
    constexpr int CPR = BNZ / 8;
    for (int c = tid; c < BM * CPR; c += 256) {
      const int r = c / CPR, ch = c % CPR;
      int orow;
      if constexpr (C::EPI == EPI_OUT_ROUTED) {
        orow = p.sorted[m0 + r];
        if (orow >= nflat) continue;
      } else {
        orow = m0 + r;
        if (orow >= p.T) continue;
      }
      const u32x4 v = *reinterpret_cast<const u32x4*>(smem + (r * BNZ + ch * 8) * 2);
      *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(p.out) + static_cast<int64_t>(orow) * p.ldo +
                                n0 + ch * 8) = v;
    }
  }
}

template <class C>
void launch_gemm(const GemmParams& p, int64_t max_mblk, hipStream_t s) {
  const int64_t tiles = max_mblk * p.n_tiles;
  const int64_t grid = (tiles + 7) / 8 * 8;
  if (grid == 0) return;
  grouped_gemm_kernel<C><<<static_cast<unsigned>(grid), 256, 0, s>>>(p);
}

}  // namespace moe
