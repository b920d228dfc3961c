// Grouped GEMM for the experts stage on gfx950 MFMA.
//
// C[m, n] = sum_k A[m, k] * W[n, k] for the rows of one expert at a time: A is
// the activation rows of an M-tile (gathered through sorted_token_ids for the
// first GEMM, contiguous for the second), W the expert's weight matrix stored
// [N, K] row-major, so both operands stream along K.  The experts and their
// block-padded row groups come from align; the shared expert runs the same
// kernel in "dense" mode over all T rows.
//
// Tiling: 4 or 8 waves, tile BM x NB (NB = 2*BNZ when gated: BNZ
// gate rows n0.. and the matching BNZ up rows I+n0.., so SiLU-mul is
// elementwise in registers).  Each k-tile is RB bytes of K per row (128: 64
// bf16 or 128 fp8 elements; 64: 32 bf16), moved global -> LDS by
// direct-to-LDS loads (global_load_lds_dwordx4: no staging registers, no
// ds_write) into a ring of NSTAGE LDS stages with one barrier per k-tile:
// NSTAGE-1 k-tiles of loads are in flight while one feeds the MFMAs.  The
// barrier is a bare s_barrier (lds_barrier): __syncthreads() would also wait
// for the loads still in flight.  The 16-byte
// chunk index of each LDS row is XOR-swizzled so that the fragment reads
// (16 lanes = 16 rows at one chunk column) hit all 64 banks; a direct load
// writes 64 lanes x 16 B contiguously, so each lane fetches the global chunk
// that belongs in its slot.  Fragments whose rows are all padding skip their
// MFMAs.
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
// a contiguous range of tiles in a grouped order -- expert-major (one
// expert's M-blocks down, then the next N-tile) when the align offsets are
// given, else 8 M-blocks down, then the next N-tile -- so the workgroups
// resident on one XCD share activation rows and weight tiles through that
// XCD's L2.
#pragma once

#include <type_traits>

#include "moe_device.h"
#include "launch.h"

namespace moe {

enum { A_GATHER = 0, A_ROWS = 1, A_DENSE = 2 };
enum { EPI_Z = 0, EPI_OUT_ROUTED = 1, EPI_OUT_DENSE = 2 };

// f(integral_constant<int, i>) for i = 0 .. N-1, unrolled at compile time
template <int I, int N, class F>
__device__ __forceinline__ void static_for_from(F& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for_from<I + 1, N>(f);
  }
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_from<0, N>(f);
}

template <int BM_, int BNZ_, int WAVES_M_, int WAVES_N_, int MF_, bool FP8_, bool GATED_,
          int AMODE_, int EPI_, int NSTAGE_ = 2, int RB_ = 128, bool SPLIT_ = false,
          bool SWAP_ = false>
struct GemmCfg {
  static constexpr int BM = BM_, BNZ = BNZ_, WAVES_M = WAVES_M_, WAVES_N = WAVES_N_, MF = MF_;
  static constexpr bool FP8 = FP8_, GATED = GATED_;
  static constexpr int AMODE = AMODE_, EPI = EPI_;
  // LDS stages: NSTAGE-1 k-tiles of direct-to-LDS loads in flight while
  // one is consumed (one barrier per k-tile either way).
  static constexpr int NSTAGE = NSTAGE_;
  // Bytes of K per row in one k-tile: 128, or 64 (bf16 only).
  static constexpr int RB = RB_;
  // Split rings: the activation rows (A) in a ring of 2 k-tiles, the weight
  // rows (B) in a ring of 3, so two k-tiles of weight loads are in flight
  // while one is consumed (weights stream from HBM; activation rows are
  // re-read by every column tile and mostly come from L2).  NSTAGE is
  // unused then.
  static constexpr bool SPLIT = SPLIT_;
  // fp8 tiles: the weight fragment is the matrix instruction's first
  // operand, so the accumulator tile is transposed -- each lane holds one
  // activation row and 16 output columns of one fragment, and the k-tile's
  // promotion needs one scale product per fragment instead of one per
  // accumulator (the products and their rounding are the same).
  static constexpr bool SWAP = SWAP_;
  // Epilogue staging rows: fp32 z of the fp8 first GEMM (floats), one more
  // than the tile's columns when lanes write down columns (SWAP), which
  // keeps a wave's stores on distinct banks; bf16 y (elements), eight more
  // (a 16-byte row shift) for the same reason, rows staying 16-byte aligned.
  static constexpr int ZSTRIDE = SWAP_ ? BNZ_ + 1 : BNZ_;
  static constexpr int YSTRIDE = SWAP_ ? BNZ_ + 8 : BNZ_;
};

// gfx950 LDS: 64 banks of 4 bytes; a 16-byte read serves 16 lanes per
// cycle (256 B).  128-byte rows: rows r and r+2 share banks, and XOR-ing the
// chunk with (row >> 1) & 7 gives the 8 rows of each parity among 16
// consecutive rows 8 distinct chunks.  64-byte rows: rows r and r+4 share
// banks, and XOR-ing with (row >> 2) & 3 gives the 4 rows of each residue
// mod 4 distinct chunks.  Either way a fragment read (16 lanes = 16
// consecutive rows at one chunk column) touches all 64 banks once.
template <int RB>
__device__ __forceinline__ int swz_key(int row) {
  static_assert(RB == 128 || RB == 64, "row bytes");
  return RB == 128 ? (row >> 1) & 7 : (row >> 2) & 3;
}
template <int RB>
__device__ __forceinline__ int swz(int row, int chunk) {
  return row * RB + ((chunk ^ swz_key<RB>(row)) << 4);
}

template <int MF, bool FP8>
struct Mfma;

template <>
struct Mfma<32, false> {
  typedef f32x16 acc_t;
  typedef u32x4 frag_t;
  static constexpr int KSTEP = 32, NACC = 16;  // bytes of K per MFMA
  template <int RB>
  __device__ static frag_t read(const uint8_t* base, int row, int s, int lane) {
    return *reinterpret_cast<const u32x4*>(base + swz<RB>(row, 2 * s + (lane >> 5)));
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
  static constexpr int KSTEP = 64, NACC = 4;
  template <int RB>
  __device__ static frag_t read(const uint8_t* base, int row, int s, int lane) {
    return *reinterpret_cast<const u32x4*>(base + swz<RB>(row, 4 * s + (lane >> 4)));
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
  static constexpr int KSTEP = 64, NACC = 16;
  template <int RB>
  __device__ static frag_t read(const uint8_t* base, int row, int s, int lane) {
    const int c0 = 4 * s + 2 * (lane >> 5);
    const u32x4 lo = *reinterpret_cast<const u32x4*>(base + swz<RB>(row, c0));
    const u32x4 hi = *reinterpret_cast<const u32x4*>(base + swz<RB>(row, c0 + 1));
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
  static constexpr int KSTEP = 128, NACC = 4;
  template <int RB>
  __device__ static frag_t read(const uint8_t* base, int row, int s, int lane) {
    const int c0 = 2 * (lane >> 4);
    const u32x4 lo = *reinterpret_cast<const u32x4*>(base + swz<RB>(row, c0));
    const u32x4 hi = *reinterpret_cast<const u32x4*>(base + swz<RB>(row, c0 + 1));
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

// Tile row and column of accumulator element v of lane `lane` in fragment
// (fm, fn) of a wave whose rows start at row_w and columns at col_w; with
// swapped operands the fragment is transposed.
template <int MF, bool SWAP>
__device__ __forceinline__ int acc_tile_row(int row_w, int fm, int v, int lane) {
  return row_w + fm * MF + (SWAP ? acc_col<MF>(lane) : acc_row<MF>(v, lane));
}
template <int MF, bool SWAP>
__device__ __forceinline__ int acc_tile_col(int col_w, int fn, int v, int lane) {
  return col_w + fn * MF + (SWAP ? acc_row<MF>(v, lane) : acc_col<MF>(lane));
}

// 64 lanes x 16 bytes from per-lane global addresses into 1 KB of LDS,
// lane i landing at lds + 16*i (global_load_lds_dwordx4).
__device__ __forceinline__ void lds_dma16(const uint8_t* g, uint8_t* lds) {
  typedef __attribute__((address_space(3))) void lds_void;
  __builtin_amdgcn_global_load_lds(g, (lds_void*)lds, 16, 0, 0);
}

// Workgroup barrier for the k-loop.  __syncthreads() (and a workgroup
// fence, even one restricted to LDS) makes every wave wait for all of its
// outstanding global loads (vmcnt(0)) before arriving; that includes the
// direct-to-LDS loads of the later stages and would cut the pipeline to one
// k-tile in flight.  Here the caller has already waited for its own loads of
// the stage about to be read (s_waitcnt vmcnt(N)); lgkmcnt(0) completes this
// wave's LDS reads and writes, and the "memory" clobbers keep the compiler
// from moving LDS accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Wait for every outstanding global (and direct-to-LDS) load of this wave.
__device__ __forceinline__ void wait_vm_loads() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Wait until at most N of this wave's global loads are outstanding.
template <int N>
__device__ __forceinline__ void wait_vm_loads_but() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// LDS of one tile: the k-tile stages (or split rings), reused by the
// epilogue's staging, then (fp8 only) the activation-scale table and the
// tile's weight-block scales along K (sW: gate row, then up row).  bf16
// tiles use every byte of the 160 KB for stages.
template <class C>
struct GemmLds {
  static constexpr int G = C::GATED ? 2 : 1;
  static constexpr int NB = G * C::BNZ;
  static constexpr int A_BYTES = C::BM * C::RB, B_BYTES = NB * C::RB;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int EPI_BYTES = (C::EPI == EPI_Z && C::FP8) ? C::BM * C::ZSTRIDE * 4 : C::BM * C::YSTRIDE * 2;
  static constexpr int ARING = 2, BRING = 3;
  static constexpr int RING_BYTES = C::SPLIT ? ARING * A_BYTES + BRING * B_BYTES : C::NSTAGE * STAGE;
  static constexpr int SMEM_TILE = cmax(RING_BYTES, EPI_BYTES);
  static constexpr int kMaxKB = 128;  // K <= 16384
  // Activation scales: the tile's whole table [k-tile][row] when its
  // k-tiles fit SA_KB (loaded once before the k-loop), else two k-tiles in
  // turn.  SA_KB (2..64) takes what the LDS leaves without lowering the
  // number of workgroups per CU that the tile had with two k-tiles of
  // scales.
  static constexpr int kLds = 163840;
  static constexpr int BASE_BYTES = SMEM_TILE + (C::FP8 ? (2 * C::BM + 2 * kMaxKB) * 4 : 0);
  static constexpr int PER_WG = BASE_BYTES > kLds ? kLds : kLds / (kLds / BASE_BYTES);
  static constexpr int SA_FIT = (PER_WG - SMEM_TILE - 2 * kMaxKB * 4) / (C::BM * 4);
  static constexpr int SA_KB = !C::FP8 ? 2 : (SA_FIT < 2 ? 2 : (SA_FIT > 64 ? 64 : SA_FIT));
  static constexpr int SCALE_BYTES = C::FP8 ? (SA_KB * C::BM + 2 * kMaxKB) * 4 : 0;
  static_assert(SMEM_TILE + SCALE_BYTES <= kLds, "tile exceeds the LDS");
};

// Occupancy hint: the fp8 second-GEMM tile of 128 rows (64 KB of LDS) is
// held to 128 VGPRs so that two workgroups share a CU, one's prologue and
// epilogue overlapping the other's k-loop (its k-loop is only K/128 = 16
// tiles long at the DeepSeek shape, so those fixed costs weigh ~20 %).
template <class C>
constexpr int gemm_min_waves_per_eu() {
  return (C::FP8 && C::EPI != EPI_Z && C::BM == 128) ? 4 : 1;
}

template <class C>
__global__ __launch_bounds__(64 * C::WAVES_M * C::WAVES_N, gemm_min_waves_per_eu<C>()) void grouped_gemm_kernel(GemmParams p) {
  constexpr int BM = C::BM, BNZ = C::BNZ, MF = C::MF;
  constexpr bool FP8 = C::FP8;
  constexpr int G = C::GATED ? 2 : 1;
  constexpr int NB = G * BNZ;
  constexpr int WM = BM / C::WAVES_M, WN = BNZ / C::WAVES_N;
  constexpr int FM = WM / MF, FN = WN / MF;
  constexpr int NW = C::WAVES_M * C::WAVES_N;   // waves per workgroup
  constexpr int NT = 64 * NW;                     // threads per workgroup
  static_assert(NW == 4 || NW == 8, "4 or 8 waves");
  static_assert(FM >= 1 && FN >= 1 && WM % MF == 0 && WN % MF == 0, "wave tile");
  constexpr int RB = C::RB;
  static_assert(RB == 128 || (RB == 64 && !FP8), "fp8 k-tiles are one 128-wide scale block");
  constexpr int A_BYTES = BM * RB, B_BYTES = NB * RB, STAGE = A_BYTES + B_BYTES;
  constexpr int ROWS = BM + NB;           // LDS rows per stage: A rows, then B rows
  constexpr int LPR = RB / 16;            // lanes per row in one 1 KB direct load
  constexpr int RPG = 64 / LPR;           // rows per load group
  static_assert(ROWS % RPG == 0, "whole load groups");
  constexpr int NI = ROWS / RPG;          // 1 KB direct-to-LDS loads per k-tile
  constexpr int NIW = (NI + NW - 1) / NW; // ... per wave (at most)
  constexpr int EB = FP8 ? 1 : 2;
  typedef Mfma<MF, FP8> M;
  typedef typename M::acc_t acc_t;
  typedef typename M::frag_t frag_t;
  constexpr int NSUB = RB / M::KSTEP, NACC = M::NACC;
  static_assert(NSUB >= 1, "k-tile holds at least one MFMA step");
  constexpr int EPI_BYTES = (C::EPI == EPI_Z && FP8) ? BM * C::ZSTRIDE * 4 : BM * C::YSTRIDE * 2;
  constexpr bool SWAP = C::SWAP;
  static_assert(!SWAP || FP8, "swapped operands: fp8 tiles");
  constexpr int NSTAGE = C::NSTAGE;
  static_assert(NSTAGE == 2 || NI % NW == 0, "deeper pipelines: whole load groups");
  constexpr bool SPLIT = C::SPLIT;
  static_assert(!SPLIT || NSTAGE == 2, "split rings replace the stage count");
  constexpr int A_G = BM / RPG, B_G = NB / RPG;          // 1 KB load groups of A and of B rows
  constexpr int NIA = (A_G + NW - 1) / NW, NIB = (B_G + NW - 1) / NW;
  static_assert(!SPLIT || (B_G % NW == 0 && BM % RPG == 0),
                "split rings: every wave issues the same number of weight loads");
  typedef GemmLds<C> LDS;
  constexpr int ARING = LDS::ARING, BRING = LDS::BRING;
  constexpr int SMEM_TILE = LDS::SMEM_TILE;
  static_assert(SMEM_TILE >= cmax(LDS::RING_BYTES, EPI_BYTES), "LDS layout");
  constexpr int kMaxKB = LDS::kMaxKB;
  constexpr int SA_KB = LDS::SA_KB;
  constexpr int SCALE_BYTES = LDS::SCALE_BYTES;
  static_assert(!FP8 || SA_KB >= NSTAGE, "a ring slot of activation scales per stage");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[SMEM_TILE + SCALE_BYTES];
  float* const sA = reinterpret_cast<float*>(smem + SMEM_TILE);
  float* const sW = sA + SA_KB * BM;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  // fp8, ungated, 256 columns: each wave's columns lie in one of the tile's
  // two 128-row weight-scale blocks, wblk
  constexpr bool WIDE = FP8 && !C::GATED && BNZ > 128;
  static_assert(!FP8 || (C::GATED ? BNZ == 128 : (BNZ == 128 || (BNZ == 256 && 128 % WN == 0))),
                "fp8 tiles: 128 columns, or 256 ungated with each wave inside one scale block");
  const int wblk = WIDE ? (wn * WN) / 128 : 0;

  // ---- tile decode (XCD-aware grouped order) ----
  // split K: the grid holds ksplit copies of the tile grid, split-major
  const int grid1 = static_cast<int>(gridDim.x) / p.ksplit;
  const int ks = static_cast<int>(blockIdx.x) / grid1;
  const int bid = static_cast<int>(blockIdx.x) - ks * grid1;
  const int rows_total = (C::AMODE == A_DENSE) ? p.T : p.ntp[0];
  const int n_mblk = (rows_total + BM - 1) / BM;
  const int total = n_mblk * p.n_tiles;
  const int per = (total + 7) >> 3;
  const int jj = bid >> 3;
  if (jj >= per) return;
  const int logical = (bid & 7) * per + jj;
  if (logical >= total) return;
  int mblk, ntile;
  if (C::AMODE != A_DENSE && p.expert_offsets != nullptr) {
    // Expert-major order: the tiles of one expert are consecutive, its
    // M-blocks fastest, so the tiles resident on an XCD at once share the
    // expert's weight tiles (and its activation rows) in that XCD's L2.
    // Expert e owns tiles [b0 * n_tiles, b1 * n_tiles) with b0, b1 its first
    // and end M-block, so M-block logical / n_tiles is one of e's blocks.
    const int e = p.block_expert[(logical / p.n_tiles) * BM / p.align_bm];
    const int b0 = p.expert_offsets[e] / BM, nb = p.expert_offsets[e + 1] / BM - b0;
    const int rem = logical - b0 * p.n_tiles;
    mblk = b0 + rem % nb;
    ntile = rem / nb;
  } else {
    // groups of GM M-blocks (8 down, then the next N-tile)
    constexpr int GM = 8;
    const int grp = logical / (GM * p.n_tiles);
    const int first_m = grp * GM;
    const int gm = min(n_mblk - first_m, GM);
    const int rem = logical - grp * GM * p.n_tiles;
    mblk = first_m + rem % gm;
    ntile = rem / gm;
  }
  const int m0 = mblk * BM, n0 = ntile * BNZ;

  const uint8_t* wbase = p.w;
  const float* wsbase = p.w_scale;
  if constexpr (C::AMODE != A_DENSE) {
    // the tile may be a fraction of the align block (GEMM-2 at BM/2)
    const int e = p.block_expert[m0 / p.align_bm];
    wbase += static_cast<int64_t>(e) * p.w_stride;
    if constexpr (FP8) wsbase += static_cast<int64_t>(e) * p.ws_stride;
  }
  const int nflat = p.T * p.top_k;
  const int64_t krow_bytes = static_cast<int64_t>(p.K) * EB;
  const int kblocks = p.K / 128;  // fp8: scale blocks along K (= k-tiles)

  // Rows of this block that carry data: pad rows sit at the end of an
  // expert's segment (and past T in dense mode), so a count is enough.
  int valid_rows;
  if constexpr (C::AMODE == A_DENSE) {
    valid_rows = min(BM, p.T - m0);
  } else {
    // one row per thread; the per-wave counts meet in the first bytes of
    // smem, which the stage loads only overwrite after the second barrier
    static_assert(BM <= NT, "one row per thread");
    const bool live = tid < BM && p.sorted[m0 + tid] < nflat;
    int* const red = reinterpret_cast<int*>(smem);
    const int wcount = __builtin_popcountll(__ballot(live));
    if (lane == 0) red[wave] = wcount;
    __syncthreads();
    int v = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) v += red[w];
    __syncthreads();
    valid_rows = v;
    if (valid_rows == 0) return;  // a tile past its expert's rows (block-uniform)
  }

  // ---- direct-to-LDS source pointers ----
  // Row r of a stage (A rows 0..BM-1, then B rows) and where it starts in
  // global memory.
  auto row_src = [&](int r) -> const uint8_t* {
    if (r < BM) {
      int srow = 0;
      if constexpr (C::AMODE == A_GATHER) {
        const int sid = p.sorted[m0 + r];
        srow = sid < nflat ? sid / p.top_k : 0;   // pad rows read token 0 (discarded)
      } else if constexpr (C::AMODE == A_ROWS) {
        srow = m0 + r;
      } else {
        srow = min(m0 + r, p.T - 1);
      }
      return p.a + static_cast<int64_t>(srow) * krow_bytes;
    }
    const int b = r - BM;
    int wrow;
    if constexpr (C::GATED) wrow = b < BNZ ? n0 + b : p.inter + n0 + (b - BNZ);
    else wrow = n0 + b;
    return wbase + static_cast<int64_t>(wrow) * krow_bytes;
  };
  // Load group j covers LDS rows RPG*j.. of a stage; lane i fills the
  // 16-byte slot i of the group, i.e. row RPG*j + i/LPR at physical chunk
  // i%LPR, which holds logical chunk (i%LPR) ^ swz_key(row).  (The key of
  // a row depends on its index mod 16 only, and BM is a multiple of 16, so
  // B rows have the same key whether counted from the stage or from B.)
  const uint8_t* src[SPLIT ? 1 : NIW];
  const uint8_t* srcA[SPLIT ? NIA : 1];
  const uint8_t* srcB[SPLIT ? NIB : 1];
  if constexpr (!SPLIT) {
#pragma unroll
    for (int s = 0; s < NIW; ++s) {
      const int j = wave + NW * s;
      const int r = RPG * j + lane / LPR;
      const int lchunk = (lane % LPR) ^ swz_key<RB>(r);
      src[s] = (j < NI ? row_src(r) : p.a) + lchunk * 16;   // p.a: any valid row, unused
    }
  } else {
#pragma unroll
    for (int s = 0; s < NIA; ++s) {
      const int a = wave + NW * s;
      const int r = RPG * a + lane / LPR;
      srcA[s] = (a < A_G ? row_src(r) : p.a) + ((lane % LPR) ^ swz_key<RB>(r)) * 16;
    }
#pragma unroll
    for (int s = 0; s < NIB; ++s) {
      const int rb = RPG * (wave + NW * s) + lane / LPR;
      srcB[s] = row_src(BM + rb) + ((lane % LPR) ^ swz_key<RB>(rb)) * 16;
    }
  }
  // fp8: this thread's activation-scale row (threads < BM) and the weight-scale rows
  static_assert(!FP8 || BM <= NT, "one activation-scale row per thread");
  int a_srow = 0;
  const float* sw_row0 = nullptr;
  const float* sw_row1 = nullptr;
  if constexpr (FP8) {
    if (tid < BM) {
      if constexpr (C::AMODE == A_GATHER) {
        const int sid = p.sorted[m0 + tid];
        a_srow = sid < nflat ? sid / p.top_k : 0;
      } else if constexpr (C::AMODE == A_ROWS) {
        a_srow = m0 + tid;
      } else {
        a_srow = min(m0 + tid, p.T - 1);
      }
    }
    sw_row0 = wsbase + static_cast<int64_t>(n0 / 128) * kblocks;
    if constexpr (C::GATED) sw_row1 = wsbase + static_cast<int64_t>((p.inter + n0) / 128) * kblocks;
    // an ungated tile 256 columns wide spans two 128-row weight blocks: the
    // second one's scales take the slot the up half uses in a gated tile
    if constexpr (WIDE) sw_row1 = wsbase + static_cast<int64_t>(n0 / 128 + 1) * kblocks;
    for (int i = tid; i < kblocks; i += NT) {
      sW[i] = sw_row0[i];
      if constexpr (C::GATED || WIDE) sW[kMaxKB + i] = sw_row1[i];
    }
    // made visible by the first k-tile's barrier
  }

  // this workgroup's k-tiles: [kbase, kbase + nk)
  const int nk = p.K / (RB / EB) / p.ksplit;
  const int kbase = ks * nk;
  // In the k-loop of tiles with padding rows (not FULL), load groups of A
  // rows that lie wholly past the block's data rows (the padding at the end
  // of an expert's segment, or past T) are not loaded: their LDS rows keep
  // stale values, which only ever reach the outputs of pad rows (MFMA rows
  // are independent), and those are never stored or read.  A half-filled
  // 256-row block saves a quarter of its loads.  The count of loads in
  // flight then varies by wave, so this needs the two-stage loop, which
  // waits for all of them (vmcnt(0)).  Full tiles keep branch-free loads.
  // With split rings the weight loads alone are counted by the waits, so
  // the activation loads may be skipped as well.
  const int a_groups = (NSTAGE == 2) ? (valid_rows + RPG - 1) / RPG : BM / RPG;
  auto dma = [&](int kt, int buf, auto full_tag) {
    constexpr bool FULL = decltype(full_tag)::value;
    kt += kbase;
#pragma unroll
    for (int s = 0; s < NIW; ++s) {
      const int j = wave + NW * s;
      if ((NI % NW == 0 || j < NI) && (FULL || j >= BM / RPG || j < a_groups))
        lds_dma16(src[s] + static_cast<int64_t>(kt) * RB, smem + buf * STAGE + j * 1024);
    }
  };
  // split rings: A k-tile kt into A buffer buf, B k-tile kt into B buffer buf
  auto dma_a = [&](int kt, int buf, auto full_tag) {
    constexpr bool FULL = decltype(full_tag)::value;
    kt += kbase;
#pragma unroll
    for (int s = 0; s < NIA; ++s) {
      const int a = wave + NW * s;
      if ((A_G % NW == 0 || a < A_G) && (FULL || a < a_groups))
        lds_dma16(srcA[s] + static_cast<int64_t>(kt) * RB, smem + buf * A_BYTES + a * 1024);
    }
  };
  auto dma_b = [&](int kt, int buf) {
    kt += kbase;
#pragma unroll
    for (int s = 0; s < NIB; ++s)
      lds_dma16(srcB[s] + static_cast<int64_t>(kt) * RB,
                smem + ARING * A_BYTES + buf * B_BYTES + (wave + NW * s) * 1024);
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

  const int row_w = wm * WM;
  // fragments of this wave that hold at least one data row (wave-uniform)
  const int fm_live = __builtin_amdgcn_readfirstlane(
      valid_rows > row_w ? min(FM, (valid_rows - row_w + MF - 1) / MF) : 0);

  // fp8 tiles below 256 rows (whole partial sets fit beside the
  // accumulators; not the tile held to 128 registers, where this spilled):
  // k-tile kt's partials and their scale products are promoted into acc at
  // the start of k-tile kt+1, once its fragment reads are issued, and after
  // the last k-tile -- in k-tile order, so the sums are the same.  A wave
  // then goes on to the next barrier while its MFMAs still run, and the
  // promotion's vector work covers the fragment reads.
  constexpr bool DEFER = FP8 && SWAP && BM < 256 && gemm_min_waves_per_eu<C>() == 1;
  acc_t dpart[DEFER ? G : 1][DEFER ? FM : 1][DEFER ? FN : 1];
  float dsc[DEFER ? G : 1][DEFER ? FM : 1];
  // fp8 tiles of 256 rows (one row fragment's partial set at a time): each
  // fragment's partial and scale products wait in lpend / lsc until the next
  // fragment's MFMAs are issued -- the k-tile's last fragment until the next
  // k-tile's first, or the end -- and are then promoted into row fragment fm
  // of acc (same products, same order per accumulator).
  constexpr bool LAG = FP8 && SWAP && BM >= 256;
  acc_t lpend[LAG ? G : 1][LAG ? FN : 1];
  float lsc[LAG ? G : 1];
  auto promote_lag = [&](auto fm_c) {
    constexpr int fm = decltype(fm_c)::value;
    if constexpr (LAG) {
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
          for (int v = 0; v < NACC; ++v) acc[g][fm][fn][v] += lpend[g][fn][v] * lsc[g];
    }
  };
  auto promote_deferred = [&](auto full_tag) {
    constexpr bool FULL = decltype(full_tag)::value;
    if constexpr (DEFER) {
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) {
        if (!(FULL || fm < fm_live)) continue;
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int fn = 0; fn < FN; ++fn)
#pragma unroll
            for (int v = 0; v < NACC; ++v) acc[g][fm][fn][v] += dpart[g][fm][fn][v] * dsc[g][fm];
      }
    }
  };

  // fp8 k-tiles.  A k-tile is one 128-deep scale block: its MFMAs sum into a
  // fresh partial, which is promoted into the fp32 accumulator as
  // acc += partial * s_a[row] * s_w.  The k-tile's activation scales are
  // read from LDS (16-byte reads: an accumulator's rows come in runs of 4)
  // right after the barrier, so their latency hides behind the MFMAs.
  // The rows' scales reach LDS as one [k-tile][row] table per tile, loaded
  // before the loop; when the table does not fit (two-stage ring only), by
  // a direct-to-LDS load per k-tile issued with the stage loads.  Either way
  // no load into a register is in flight inside the loop.  (Loaded into a
  // register and stored to LDS at the end of each iteration, the scale made
  // the compiler wait for vmcnt(0) inside the iteration -- loads complete in
  // order -- which also drained the next k-tile's stage loads: 12 % of the
  // gated first GEMM's time at DeepSeek-V3 T=8192.)
  // (Deferring each promotion by one k-tile with two partial sets was
  // measured slower: the extra registers cost occupancy.)
  // Whole table when it fits; split rings always fit it (the host only
  // picks a split-ring tile when K / 128 / ksplit <= its capacity).
  const bool whole = SPLIT || nk <= SA_KB;
  // Row r's scale of k-tile kt straight to sA[b][r] (ring slot b) by a 4-byte
  // direct-to-LDS load (threads r < BM; lane i of a wave writes 4*i bytes
  // past the wave's base), issued with the k-tile's stage loads.
  auto dma_sa = [&](int kt, int b) {
    if (tid < BM) {
      typedef __attribute__((address_space(3))) void lds_void;
      const float* g = p.a_scale + static_cast<int64_t>(a_srow) * p.sa_row +
                       static_cast<int64_t>(kbase + kt) * p.sa_k;
      __builtin_amdgcn_global_load_lds(g, (lds_void*)(sA + b * BM + (tid & ~63)), 4, 0, 0);
    }
  };
  // Chunked (swapped tiles whose table does not fit, G(128) scales, whole
  // 16-byte chunks): row r's scales of k-tiles 4c..4c+3 are contiguous, so
  // one 16-byte direct load per row brings four k-tiles -- a quarter of the
  // line requests of the per-k-tile loads.  Chunk c goes to ring slot
  // c % NCH, laid out [row][4]; at the top of k-tile 4c (c >= 1) the slot of
  // chunk c-1 is free and chunk c-1+NCH is loaded into it, NCH-1 chunks
  // ahead of its use.
  constexpr int NCH = (SA_KB / 4) < 8 ? (SA_KB / 4) : 8;
  const int nchunks = nk / 4;
  const bool chunked = SWAP && !whole && NCH >= 2 && p.sa_k == 1 && (nk & 3) == 0 &&
                       (kbase & 3) == 0 && (p.sa_row & 3) == 0 &&
                       (reinterpret_cast<uintptr_t>(p.a_scale) & 15) == 0;
  auto dma_chunk = [&](int c) {
    if (tid < BM) {
      typedef __attribute__((address_space(3))) void lds_void;
      const float* g = p.a_scale + static_cast<int64_t>(a_srow) * p.sa_row + kbase + 4 * c;
      __builtin_amdgcn_global_load_lds(g, (lds_void*)(sA + (c % NCH) * BM * 4 + (tid & ~63) * 4), 16, 0, 0);
    }
  };
  // the chunk (if any) issued at the top of k-tile kt
  auto chunk_at = [&](int kt) { return (kt > 0 && (kt & 3) == 0) ? kt / 4 - 1 + NCH : -1; };
  // Whole table: thread r < BM loads its row's scales of this tile's
  // k-tiles (16-byte loads where the row's G(128) scales are contiguous and
  // aligned) and stores them to sA[kt][r]; the first barrier publishes them.
  // The loads are consumed here, before the loop, so none is in flight into
  // a register when it starts.
  auto load_scale_table = [&]() {
    if (!(whole && tid < BM)) return;
    // batches of up to 8 loads in flight before their stores (the first
    // k-tiles' stage loads are already under way)
    const float* g = p.a_scale + static_cast<int64_t>(a_srow) * p.sa_row +
                     static_cast<int64_t>(kbase) * p.sa_k;
    int kv = 0;   // scales taken by whole 16-byte loads (never past k-tile nk-1)
    if (p.sa_k == 1 && (reinterpret_cast<uintptr_t>(g) & 15) == 0) {
      kv = nk & ~3;
      for (int k0 = 0; k0 < kv; k0 += 32) {
        f32x4 v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (k0 + 4 * j < kv) v[j] = *reinterpret_cast<const f32x4*>(g + k0 + 4 * j);
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (k0 + 4 * j < kv) {
#pragma unroll
            for (int i = 0; i < 4; ++i) sA[(k0 + 4 * j + i) * BM + tid] = v[j][i];
          }
      }
    }
    for (int k0 = kv; k0 < nk; k0 += 8) {
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (k0 + j < nk) v[j] = g[static_cast<int64_t>(k0 + j) * p.sa_k];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (k0 + j < nk) sA[(k0 + j) * BM + tid] = v[j];
    }
  };

  // One fp8 k-tile (kt, tile-local) from stage buffers As / Bs.
  auto compute_fp8 = [&](int kt, int slot, const uint8_t* As, const uint8_t* Bs, auto full_tag) {
    constexpr bool FULL = decltype(full_tag)::value;
    // this k-tile's scales: weight blocks (gate, up) and the rows' activation
    // scales; the latter are read ahead of the MFMAs unless registers are
    // held to 128 for occupancy (LEAN), then inside the promotion
    constexpr bool LEAN = gemm_min_waves_per_eu<C>() > 1;
    constexpr bool PER_FRAGMENT = BM >= 256;
    const float swg[2] = {sW[wblk * kMaxKB + kbase + kt], C::GATED ? sW[kMaxKB + kbase + kt] : 0.f};
    const float* sAb = sA + (whole ? kt : slot) * BM;
    auto read_sa = [&](int fm, float (&out)[NACC]) {
#pragma unroll
      for (int q = 0; q < NACC / 4; ++q) {
        const f32x4 t = *reinterpret_cast<const f32x4*>(sAb + row_w + fm * MF + acc_row<MF>(4 * q, lane));
#pragma unroll
        for (int r = 0; r < 4; ++r) out[4 * q + r] = t[r];
      }
    };
    if constexpr (PER_FRAGMENT) {
      // 256-row tiles: each row fragment's partial is summed, then promoted
      // once the next fragment's MFMAs are issued (LAG), so at most two
      // fragments' partials are live beside the accumulators (a full
      // partial set would double them).
      frag_t fb[NSUB][G][FN];
#pragma unroll
      for (int s = 0; s < NSUB; ++s)
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int fn = 0; fn < FN; ++fn)
            fb[s][g][fn] = M::template read<RB>(Bs, g * BNZ + wn * WN + fn * MF + (lane & (MF - 1)), s, lane);
      if constexpr (LAG) {
        static_for<FM>([&](auto fm_c) {
          constexpr int fm = decltype(fm_c)::value;
          constexpr int pfm = fm == 0 ? FM - 1 : fm - 1;
          const bool live = FULL || fm < fm_live;
          acc_t pf[G][FN];
          if (live) {
#pragma unroll
            for (int s = 0; s < NSUB; ++s) {
              const frag_t fa = M::template read<RB>(As, row_w + fm * MF + (lane & (MF - 1)), s, lane);
#pragma unroll
              for (int g = 0; g < G; ++g)
#pragma unroll
                for (int fn = 0; fn < FN; ++fn) {
                  if (s == 0) {
#pragma unroll
                    for (int v = 0; v < NACC; ++v) pf[g][fn][v] = 0.f;
                  }
                  pf[g][fn] = M::mma(fb[s][g][fn], fa, pf[g][fn]);
                }
            }
          }
          // the pending fragment: fm-1, or the previous k-tile's last
          if ((fm > 0 || kt > 0) && (FULL || pfm < fm_live)) promote_lag(std::integral_constant<int, pfm>{});
          if (live) {
            const int r = row_w + fm * MF + (lane & (MF - 1));
            const float sa1 = chunked ? sA[((kt >> 2) % NCH) * BM * 4 + r * 4 + (kt & 3)] : sAb[r];
#pragma unroll
            for (int g = 0; g < G; ++g) {
              lsc[g] = sa1 * swg[g];
#pragma unroll
              for (int fn = 0; fn < FN; ++fn) lpend[g][fn] = pf[g][fn];
            }
          }
        });
        return;
      }
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) {
        if (!(FULL || fm < fm_live)) continue;
        acc_t pf[G][FN];
#pragma unroll
        for (int s = 0; s < NSUB; ++s) {
          const frag_t fa = M::template read<RB>(As, row_w + fm * MF + (lane & (MF - 1)), s, lane);
#pragma unroll
          for (int g = 0; g < G; ++g)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
              if (s == 0) {
#pragma unroll
                for (int v = 0; v < NACC; ++v) pf[g][fn][v] = 0.f;
              }
              pf[g][fn] = SWAP ? M::mma(fb[s][g][fn], fa, pf[g][fn]) : M::mma(fa, fb[s][g][fn], pf[g][fn]);
            }
        }
        if constexpr (SWAP) {
          // this lane's activation row of the fragment: one scale product
          const int r = row_w + fm * MF + (lane & (MF - 1));
          const float sa1 = chunked ? sA[((kt >> 2) % NCH) * BM * 4 + r * 4 + (kt & 3)] : sAb[r];
#pragma unroll
          for (int g = 0; g < G; ++g) {
            const float sc = sa1 * swg[g];
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
#pragma unroll
              for (int v = 0; v < NACC; ++v) acc[g][fm][fn][v] += pf[g][fn][v] * sc;
          }
          continue;
        }
        float sr[NACC];
        read_sa(fm, sr);
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int fn = 0; fn < FN; ++fn)
#pragma unroll
            for (int v = 0; v < NACC; ++v)
              acc[g][fm][fn][v] += pf[g][fn][v] * (sr[v] * swg[g]);
      }
      return;
    }
    float sa[(LEAN || PER_FRAGMENT || SWAP) ? 1 : FM][NACC];
    if constexpr (!LEAN && !PER_FRAGMENT && !SWAP) {
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) read_sa(fm, sa[fm]);
    }
    // swapped operands: this lane's activation row of each row fragment
    float sa_row[SWAP ? FM : 1];
    if constexpr (SWAP) {
      const float* sAc = sA + ((kt >> 2) % NCH) * BM * 4 + (kt & 3);
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) {
        const int r = row_w + fm * MF + (lane & (MF - 1));
        sa_row[fm] = chunked ? sAc[r * 4] : sAb[r];
      }
    }
    if constexpr (DEFER) {
      // both substeps' fragments, then the previous k-tile's promotion, then
      // this k-tile's MFMAs into the partials it has just read
      frag_t fa[NSUB][FM], fb[NSUB][G][FN];
#pragma unroll
      for (int s = 0; s < NSUB; ++s) {
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
          if (FULL || fm < fm_live) fa[s][fm] = M::template read<RB>(As, row_w + fm * MF + (lane & (MF - 1)), s, lane);
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int fn = 0; fn < FN; ++fn)
            fb[s][g][fn] = M::template read<RB>(Bs, g * BNZ + wn * WN + fn * MF + (lane & (MF - 1)), s, lane);
      }
      if (kt > 0) promote_deferred(full_tag);
#pragma unroll
      for (int s = 0; s < NSUB; ++s)
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
          if (FULL || fm < fm_live)
#pragma unroll
            for (int g = 0; g < G; ++g)
#pragma unroll
              for (int fn = 0; fn < FN; ++fn) {
                if (s == 0) {
#pragma unroll
                  for (int v = 0; v < NACC; ++v) dpart[g][fm][fn][v] = 0.f;
                }
                dpart[g][fm][fn] = M::mma(fb[s][g][fn], fa[s][fm], dpart[g][fm][fn]);
              }
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int g = 0; g < G; ++g) dsc[g][fm] = sa_row[fm] * swg[g];
      return;
    }
    acc_t part[G][FM][FN];
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
      frag_t fa[FM], fb[G][FN];
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
        if (FULL || fm < fm_live) fa[fm] = M::template read<RB>(As, row_w + fm * MF + (lane & (MF - 1)), s, lane);
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
          fb[g][fn] = M::template read<RB>(Bs, g * BNZ + wn * WN + fn * MF + (lane & (MF - 1)), s, lane);
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
        if (FULL || fm < fm_live)
#pragma unroll
          for (int g = 0; g < G; ++g)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
              if (s == 0) {
#pragma unroll
                for (int v = 0; v < NACC; ++v) part[g][fm][fn][v] = 0.f;
              }
              part[g][fm][fn] = SWAP ? M::mma(fb[g][fn], fa[fm], part[g][fm][fn])
                                     : M::mma(fa[fm], fb[g][fn], part[g][fm][fn]);
            }
    }
    if constexpr (SWAP) {
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) {
        if (!(FULL || fm < fm_live)) continue;
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const float sc = sa_row[fm] * swg[g];
#pragma unroll
          for (int fn = 0; fn < FN; ++fn)
#pragma unroll
            for (int v = 0; v < NACC; ++v) acc[g][fm][fn][v] += part[g][fm][fn][v] * sc;
        }
      }
      return;
    }
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      if (!(FULL || fm < fm_live)) continue;
      const float* sr = sa[0];
      float lean[NACC];
      if constexpr (LEAN) {
        read_sa(fm, lean);
        sr = lean;
      } else {
        sr = sa[fm];
      }
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
          for (int v = 0; v < NACC; ++v)
            acc[g][fm][fn][v] += part[g][fm][fn][v] * (sr[v] * swg[g]);
    }
  };

  // One bf16 k-tile from stage buffers As / Bs.  Two fragment sets:
  // substep s+1's LDS reads are in flight while substep s's MFMAs issue
  // (interleaved by sched_group_barrier).
  auto compute_bf16 = [&](const uint8_t* As, const uint8_t* Bs, auto full_tag) {
    constexpr bool FULL = decltype(full_tag)::value;
    frag_t fa[2][FM], fb[2][G][FN];
    auto rd = [&](int s, int set) {
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
        if (FULL || fm < fm_live)
          fa[set][fm] = M::template read<RB>(As, row_w + fm * MF + (lane & (MF - 1)), s, lane);
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
          fb[set][g][fn] = M::template read<RB>(Bs, g * BNZ + wn * WN + fn * MF + (lane & (MF - 1)), s, lane);
    };
    rd(0, 0);
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
      const int cur = s & 1;
      if (s + 1 < NSUB) rd(s + 1, cur ^ 1);
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
        if (FULL || fm < fm_live)
#pragma unroll
          for (int g = 0; g < G; ++g)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
              acc[g][fm][fn] = M::mma(fa[cur][fm], fb[cur][g][fn], acc[g][fm][fn]);
      if constexpr (FULL) {
        if (s + 1 < NSUB) {
          constexpr int NR = FM + G * FN, NMM = G * FM * FN;
          constexpr int PER = NMM / NR > 0 ? NMM / NR : 1;
#pragma unroll
          for (int i = 0; i < NR; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, PER, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);    // DS read
          }
          __builtin_amdgcn_sched_group_barrier(0x008, NMM - PER * NR > 0 ? NMM - PER * NR : 0, 0);
        }
      }
    }
  };

  auto compute = [&](int kt, int slot, const uint8_t* As, const uint8_t* Bs, auto full_tag) {
    if constexpr (FP8) compute_fp8(kt, slot, As, Bs, full_tag);
    else compute_bf16(As, Bs, full_tag);
  };

  // The k-loop, instantiated twice: branch-free when every fragment row
  // block holds data (all but an expert's last block), and with uniform
  // per-fragment guards otherwise.
  auto kloop = [&](auto full_tag) {
    if constexpr (SPLIT) {
      // Loads issue in the order B(0) A(0) B(1) | A(1) B(2) | A(2) B(3) ...
      // (iteration kt issues A(kt+1), then B(kt+2)).  At the top of
      // iteration kt the only loads of this wave that may still be in flight
      // are B(kt+1)'s NIB (issued after A(kt) and B(kt)), and loads complete
      // in order, so vmcnt(NIB) means A(kt) and B(kt) have landed.  The
      // barrier then also guarantees that every wave has finished reading
      // A buffer (kt+1)&1 and B buffer (kt+2)%3, last read in iteration kt-1.
      if (nk > 0) {
        dma_b(0, 0);
        dma_a(0, 0, full_tag);
      }
      if (nk > 1) dma_b(1, 1);
      if constexpr (FP8) load_scale_table();
      int bb = 0;
      for (int kt = 0; kt < nk; ++kt) {
        if (kt + 1 < nk) wait_vm_loads_but<NIB>();
        else wait_vm_loads();
        lds_barrier();
        const int bn2 = bb + 2 >= BRING ? bb + 2 - BRING : bb + 2;
        if (kt + 1 < nk) dma_a(kt + 1, (kt + 1) & 1, full_tag);
        if (kt + 2 < nk) dma_b(kt + 2, bn2);
        compute(kt, kt & 1, smem + (kt & 1) * A_BYTES, smem + ARING * A_BYTES + bb * B_BYTES, full_tag);
        bb = bb + 1 == BRING ? 0 : bb + 1;
      }
      return;
    }
    if constexpr (FP8) {
      // As the generic loop below, plus the activation scales: the whole
      // table before the loop, or one 4-byte direct load per row and k-tile
      // into ring slot kt % NSTAGE, issued with the k-tile's stage loads by
      // the waves that hold rows (< BM), which then count one load more per
      // k-tile.
      if (chunked)
        for (int c = 0; c < NCH && c < nchunks; ++c) dma_chunk(c);
#pragma unroll
      for (int st = 0; st < NSTAGE - 1; ++st)
        if (st < nk) {
          if (!whole && !chunked) dma_sa(st, st);
          dma(st, st, full_tag);
        }
      load_scale_table();
      const bool row_wave = wave * 64 < BM;
      const bool sa_wave = !whole && !chunked && row_wave;
      int buf = 0, nbuf = NSTAGE - 1;
      for (int kt = 0; kt < nk; ++kt) {
        // k-tile kt's loads (stage and scales) have landed: at most the
        // loads issued after them are still in flight -- the later stages',
        // and a chunk issued at the top of k-tile kt-1 (NSTAGE 3)
        if constexpr (NSTAGE > 2) {
          static_assert(NSTAGE == 3 || !SWAP, "chunk accounting assumes three stages");
          const bool chunk_prev = chunked && row_wave && chunk_at(kt - 1) >= 0 &&
                                  chunk_at(kt - 1) < nchunks;
          if (kt + NSTAGE - 2 < nk) {
            if (sa_wave || chunk_prev) wait_vm_loads_but<(NIW + 1) * (NSTAGE - 2)>();
            else wait_vm_loads_but<NIW * (NSTAGE - 2)>();
          } else {
            wait_vm_loads();
          }
        } else {
          wait_vm_loads();
        }
        lds_barrier();
        if (chunked) {
          // chunk kt/4 - 1 (k-tiles up to kt-1) was last read before this barrier
          const int c = chunk_at(kt);
          if (c >= 0 && c < nchunks) dma_chunk(c);
        }
        if (kt + NSTAGE - 1 < nk) {
          // slot nbuf was last read in iteration kt-1, before this barrier
          if (!whole && !chunked) dma_sa(kt + NSTAGE - 1, nbuf);
          dma(kt + NSTAGE - 1, nbuf, full_tag);
        }
        compute(kt, buf, smem + buf * STAGE, smem + buf * STAGE + A_BYTES, full_tag);
        buf = buf + 1 == NSTAGE ? 0 : buf + 1;
        nbuf = nbuf + 1 == NSTAGE ? 0 : nbuf + 1;
      }
      return;
    }
#pragma unroll
    for (int st = 0; st < NSTAGE - 1; ++st)
      if (st < nk) dma(st, st, full_tag);
    int buf = 0;                       // kt % NSTAGE
    int nbuf = NSTAGE - 1;             // (kt + NSTAGE - 1) % NSTAGE
    for (int kt = 0; kt < nk; ++kt) {
      // k-tile kt has landed once at most the loads of the NSTAGE-2 later
      // k-tiles (NIW per wave each) are still outstanding.
      if constexpr (NSTAGE > 2) {
        if (kt + NSTAGE - 2 < nk) wait_vm_loads_but<NIW * (NSTAGE - 2)>();
        else wait_vm_loads();
      } else {
        wait_vm_loads();
      }
      lds_barrier();
      if (kt + NSTAGE - 1 < nk) dma(kt + NSTAGE - 1, nbuf, full_tag);
      compute(kt, buf, smem + buf * STAGE, smem + buf * STAGE + A_BYTES, full_tag);
      buf = buf + 1 == NSTAGE ? 0 : buf + 1;
      nbuf = nbuf + 1 == NSTAGE ? 0 : nbuf + 1;
    }
  };
  if (fm_live == FM) {
    kloop(std::true_type{});
    if (nk > 0) promote_deferred(std::true_type{});
    if (nk > 0) promote_lag(std::integral_constant<int, FM - 1>{});
  } else {
    kloop(std::false_type{});
    if (nk > 0) promote_deferred(std::false_type{});
    if (nk > 0 && FM - 1 < fm_live) promote_lag(std::integral_constant<int, FM - 1>{});
  }
  __syncthreads();

  // ---- epilogue ----
  if (p.ksplit > 1) {
    // fp32 partial tile; the reduction kernel applies the real epilogue
    float* part = p.partial + static_cast<int64_t>(ks) * p.part_rows * p.ldp;
    const int row_end = (C::AMODE == A_DENSE) ? min(BM, p.T - m0) : valid_rows;
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
          for (int v = 0; v < NACC; ++v) {
            const int r = acc_tile_row<MF, SWAP>(row_w, fm, v, lane);
            if (r < row_end) {
              const int cc = acc_tile_col<MF, SWAP>(wn * WN, fn, v, lane);
              const int prow = p.part_flat ? p.sorted[m0 + r] : m0 + r;
              part[static_cast<int64_t>(prow) * p.ldp + g * p.inter + n0 + cc] =
                  acc[g][fm][fn][v];
            }
          }
    return;
  }
  if constexpr (C::EPI == EPI_Z) {
    // z = act(gate) * up (gated) or act(h), act = SiLU or GELU; staged in LDS, then written as
    // whole rows: bf16, or fp8 E4M3 G(128) along I with one scale per row.
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int v = 0; v < NACC; ++v) {
          const int r = acc_tile_row<MF, SWAP>(row_w, fm, v, lane);
          const int cc = acc_tile_col<MF, SWAP>(wn * WN, fn, v, lane);
          float z;
          if constexpr (C::GATED) z = act_apply(p.act, acc[0][fm][fn][v]) * acc[G - 1][fm][fn][v];
          else z = act_apply(p.act, acc[0][fm][fn][v]);
          if constexpr (FP8) reinterpret_cast<float*>(smem)[r * C::ZSTRIDE + cc] = z;
          else reinterpret_cast<uint16_t*>(smem)[r * BNZ + cc] = static_cast<uint16_t>(f32_to_bf16_hw(z));
        }
    __syncthreads();
    if constexpr (FP8) {
      static_assert(BNZ == 128, "fp8 z tile is one 128-column group");
      const int ch = tid & 15;
      constexpr int RPP = NT / 16;  // rows per pass
#pragma unroll
      for (int i = 0; i < (BM + RPP - 1) / RPP; ++i) {
        const int r = (tid >> 4) + RPP * i;
        if (r < BM) {  // uniform per 16-lane group
          const float* zr = reinterpret_cast<const float*>(smem) + r * C::ZSTRIDE + ch * 8;
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
              const uint32_t word = pack4_e4m3(f[4 * h] / s, f[4 * h + 1] / s, f[4 * h + 2] / s,
                                   f[4 * h + 3] / s);
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
      for (int c = tid; c < BM * CPR; c += NT) {
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
          const int r = acc_tile_row<MF, SWAP>(row_w, fm, v, lane);
          const int cc = acc_tile_col<MF, SWAP>(wn * WN, fn, v, lane);
          reinterpret_cast<uint16_t*>(smem)[r * C::YSTRIDE + cc] =
              static_cast<uint16_t>(f32_to_bf16_hw(acc[0][fm][fn][v]));
        }
    __syncthreads();
    constexpr int CPR = BNZ / 8;
    for (int c = tid; c < BM * CPR; c += NT) {
      const int r = c / CPR, ch = c % CPR;
      if (r >= valid_rows) continue;
      int orow;
      if constexpr (C::EPI == EPI_OUT_ROUTED) orow = p.sorted[m0 + r];
      else orow = m0 + r;
      const u32x4 v = *reinterpret_cast<const u32x4*>(smem + (r * C::YSTRIDE + ch * 8) * 2);
      *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(p.out) + static_cast<int64_t>(orow) * p.ldo +
                                n0 + ch * 8) = v;
    }
  }
}

template <class C>
void launch_gemm(const GemmParams& p, int64_t max_mblk, hipStream_t s) {
  const int64_t tiles = max_mblk * p.n_tiles;
  const int64_t grid = (tiles + 7) / 8 * 8 * p.ksplit;
  if (grid == 0) return;
  grouped_gemm_kernel<C><<<static_cast<unsigned>(grid), 64 * C::WAVES_M * C::WAVES_N, 0, s>>>(p);
}

}  // namespace moe
