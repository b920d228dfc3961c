// bf16 grouped-GEMM instantiations (see gemm_impl.h for the kernel).
//
// Tile shapes by align block size BM (rows per expert block) and output
// tile width BNZ (z columns for the gated first GEMM, whose weight tile is
// 2*BNZ rows):
//   BM 16/32  -- 16x16x32 MFMA, the 4 waves split N (skinny, weight-streaming)
//   BM 64     -- 32x32x16 MFMA, 2x2 waves of 32 x BNZ/2
//   BM 128    -- 32x32x16 MFMA, 2x4 waves of 64 x BNZ/4 (BNZ 64: 2x2 waves)
//   BM 256    -- 32x32x16 MFMA, 2x4 waves (two per SIMD) of 128 x BNZ/4
//                (gated: x2), 128 fp32 accumulators per lane
#include "gemm_impl.h"

namespace moe {

// k-tile geometry: 128-byte k-tiles (64 bf16) in two LDS stages for every
// tile.  Measured on MI355X with Mixtral-shaped GEMMs: 64-byte k-tiles in
// four or five stages (twice the bytes in flight in the same LDS) run
// 10-35 % slower than two 128-byte stages -- the half-line requests cost
// more than the deeper pipeline gains -- and a third 128-byte stage does not
// fit beside a 256 x 512-row tile, or costs a resident workgroup at 128 rows.
constexpr int bf16_rb(int bm) { return (void)bm, 128; }
constexpr int bf16_stages(int bm, int nb) { return (void)bm, (void)nb, 2; }

// Wave grid of the 256-row tiles: 8 waves (2 per SIMD), each 128 rows x a
// quarter of the tile's columns; two waves per SIMD let one issue MFMAs
// while the other waits on LDS or the barrier.  Same for 128 x 128 tiles.
constexpr int kW256M = 2, kW256N = 4;
constexpr int kW128M = 2, kW128N = 4;

template <int BM, int BNZ, int WM, int WN, int MF, bool GATED, int AM, int EP>
using Bf16Cfg = GemmCfg<BM, BNZ, WM, WN, MF, false, GATED, AM, EP,
                        bf16_stages(BM, GATED ? 2 * BNZ : BNZ), bf16_rb(BM)>;
// 256 x 256 tiles with split rings (GemmCfg::SPLIT): 2 A + 3 B k-tiles of
// 32 KB, the whole 160 KB of LDS.  Measured on MI355X against the two-stage
// tile: routed GEMMs at Llama-4 T=2048 and Mixtral T=512 (one 256-row block
// or less per expert, weights streamed) 9-10 % faster; Mixtral T=4096 (four
// blocks per expert) 2 % slower; the dense shared-expert GEMMs of Llama-4
// T=2048 3-8 % slower, so launches choose (GemmParams::split_ring).
constexpr bool kBf16Split = true;
template <int BM, int BNZ, int WM, int WN, int MF, bool GATED, int AM, int EP>
using Bf16Split = GemmCfg<BM, BNZ, WM, WN, MF, false, GATED, AM, EP, 2, 128, kBf16Split>;

// Launches the tile for (block_m, bnz) and returns 0, or returns -1
// without launching when no such tile exists; with p == nullptr it only
// answers whether the tile exists.
template <class C>
static int run(const GemmParams* p, int64_t max_mblk, hipStream_t s) {
  if (p) launch_gemm<C>(*p, max_mblk, s);
  return 0;
}

template <int AM, int EP, bool GATED>
static int dispatch_bm(int block_m, int bnz, const GemmParams* p, int64_t max_mblk,
                       hipStream_t s) {
  if (bnz != 64 && bnz != 128 && !(bnz == 256 && !GATED && block_m == 256)) return -1;
  switch (block_m) {
    case 16:
      return bnz == 64 ? run<Bf16Cfg<16, 64, 1, 4, 16, GATED, AM, EP>>(p, max_mblk, s)
                       : run<Bf16Cfg<16, 128, 1, 4, 16, GATED, AM, EP>>(p, max_mblk, s);
    case 32:
      return bnz == 64 ? run<Bf16Cfg<32, 64, 1, 4, 16, GATED, AM, EP>>(p, max_mblk, s)
                       : run<Bf16Cfg<32, 128, 1, 4, 16, GATED, AM, EP>>(p, max_mblk, s);
    case 64:
      return bnz == 64 ? run<Bf16Cfg<64, 64, 2, 2, 32, GATED, AM, EP>>(p, max_mblk, s)
                       : run<Bf16Cfg<64, 128, 2, 2, 32, GATED, AM, EP>>(p, max_mblk, s);
    case 128:
      return bnz == 64 ? run<Bf16Cfg<128, 64, 2, 2, 32, GATED, AM, EP>>(p, max_mblk, s)
                       : run<Bf16Cfg<128, 128, kW128M, kW128N, 32, GATED, AM, EP>>(p, max_mblk, s);
    case 256:
      if (bnz == 64) return run<Bf16Cfg<256, 64, 2, 2, 32, GATED, AM, EP>>(p, max_mblk, s);
      if (bnz == 128) {
        if (p && p->split_ring)
          return run<Bf16Split<256, 128, kW256M, kW256N, 32, GATED, AM, EP>>(p, max_mblk, s);
        return run<Bf16Cfg<256, 128, kW256M, kW256N, 32, GATED, AM, EP>>(p, max_mblk, s);
      }
      if constexpr (!GATED) {
        if (p && p->split_ring)
          return run<Bf16Split<256, 256, kW256M, kW256N, 32, false, AM, EP>>(p, max_mblk, s);
        return run<Bf16Cfg<256, 256, kW256M, kW256N, 32, false, AM, EP>>(p, max_mblk, s);
      }
      return -1;
    default:
      return -1;
  }
}

int launch_gemm_bf16(int kind, bool gated, int block_m, int bnz, const GemmParams* p,
                     int64_t max_mblk, hipStream_t s) {
  switch (kind) {
    case GEMM_Z_ROUTED:
      return gated ? dispatch_bm<A_GATHER, EPI_Z, true>(block_m, bnz, p, max_mblk, s)
                   : dispatch_bm<A_GATHER, EPI_Z, false>(block_m, bnz, p, max_mblk, s);
    case GEMM_Y_ROUTED:
      return dispatch_bm<A_ROWS, EPI_OUT_ROUTED, false>(block_m, bnz, p, max_mblk, s);
    case GEMM_Z_DENSE:
      return gated ? dispatch_bm<A_DENSE, EPI_Z, true>(block_m, bnz, p, max_mblk, s)
                   : dispatch_bm<A_DENSE, EPI_Z, false>(block_m, bnz, p, max_mblk, s);
    case GEMM_Y_DENSE:
      return dispatch_bm<A_DENSE, EPI_OUT_DENSE, false>(block_m, bnz, p, max_mblk, s);
    default:
      return -1;
  }
}

int gemm_tile_n(int kind, bool fp8, bool gated, int block_m, int n) {
  const bool first = kind == GEMM_Z_ROUTED || kind == GEMM_Z_DENSE;
  // fp8: 128 columns (a z group on the first GEMM); second GEMMs of 16 or 32
  // rows take 256 (half the tiles, each re-reading its z rows half as often;
  // still two workgroups per CU -- at 64 rows the wider tile would hold a CU
  // alone, and measured slower)
  if (fp8) return (!first && block_m <= 32 && n % 256 == 0) ? 256 : 128;
  if (first && gated) return (block_m >= 128 && n % 128 == 0) ? 128 : 64;
  if (first) return 128;
  return (block_m == 256 && n % 256 == 0) ? 256 : 128;
}

}  // namespace moe
