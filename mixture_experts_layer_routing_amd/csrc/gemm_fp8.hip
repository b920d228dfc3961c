// fp8 E4M3 grouped-GEMM instantiations (see gemm_impl.h for the kernel).
//
// First-GEMM tiles are 128 output columns wide: one 128-column group of z,
// so the fused re-quantisation of z to E4M3 G(128) finds each group's amax
// inside the tile.  Second GEMMs of 16 or 32 rows are 256 columns wide.  BM 16/32 use 16x16x128 MFMA with
// 4 waves split along N, BM 64/128/256 use 32x32x64 MFMA on 2x4 waves (two
// per SIMD).  256-row tiles serve the second GEMM (and ungated first GEMMs):
// the gated first GEMM would need a partial set beside 2 x 128 accumulators
// per lane, which spills, so it runs two 128-row tiles per 256-row block.
#include "gemm_impl.h"

namespace moe {

template <int AM, int EP, bool GATED>
static void dispatch_bm(int block_m, const GemmParams& p, int64_t max_mblk, hipStream_t s) {
  switch (block_m) {
    case 16: launch_gemm<GemmCfg<16, 128, 1, 4, 16, true, GATED, AM, EP>>(p, max_mblk, s); break;
    case 32: launch_gemm<GemmCfg<32, 128, 1, 4, 16, true, GATED, AM, EP>>(p, max_mblk, s); break;
    case 64: launch_gemm<GemmCfg<64, 128, 2, 4, 32, true, GATED, AM, EP>>(p, max_mblk, s); break;
    case 128: launch_gemm<GemmCfg<128, 128, 2, 4, 32, true, GATED, AM, EP>>(p, max_mblk, s); break;
    default:
      // 256-row tiles exist for the ungated GEMMs only (a gated 256-row
      // tile does not fit the registers); the host never asks for one
      if constexpr (!GATED) launch_gemm<GemmCfg<256, 128, 2, 4, 32, true, false, AM, EP>>(p, max_mblk, s);
      break;
  }
}

// Second GEMMs of 16 or 32 rows on 256-column tiles (gemm_tile_n): each
// wave's 64 columns stay inside one 128-row weight-scale block.
template <int AM, int EP>
static void dispatch_wide(int block_m, const GemmParams& p, int64_t max_mblk, hipStream_t s) {
  if (block_m == 16) launch_gemm<GemmCfg<16, 256, 1, 4, 16, true, false, AM, EP>>(p, max_mblk, s);
  else launch_gemm<GemmCfg<32, 256, 1, 4, 16, true, false, AM, EP>>(p, max_mblk, s);
}

void launch_gemm_fp8(int kind, bool gated, int block_m, int bnz, const GemmParams& p,
                     int64_t max_mblk, hipStream_t s) {
  switch (kind) {
    case GEMM_Z_ROUTED:
      if (gated) dispatch_bm<A_GATHER, EPI_Z, true>(block_m, p, max_mblk, s);
      else dispatch_bm<A_GATHER, EPI_Z, false>(block_m, p, max_mblk, s);
      break;
    case GEMM_Y_ROUTED:
      if (bnz == 256) dispatch_wide<A_ROWS, EPI_OUT_ROUTED>(block_m, p, max_mblk, s);
      else dispatch_bm<A_ROWS, EPI_OUT_ROUTED, false>(block_m, p, max_mblk, s);
      break;
    case GEMM_Z_DENSE:
      if (gated) dispatch_bm<A_DENSE, EPI_Z, true>(block_m, p, max_mblk, s);
      else dispatch_bm<A_DENSE, EPI_Z, false>(block_m, p, max_mblk, s);
      break;
    default:
      if (bnz == 256) dispatch_wide<A_DENSE, EPI_OUT_DENSE>(block_m, p, max_mblk, s);
      else dispatch_bm<A_DENSE, EPI_OUT_DENSE, false>(block_m, p, max_mblk, s);
      break;
  }
}

}  // namespace moe
