// fp8 E4M3 grouped-GEMM instantiations (see gemm_impl.h for the kernel).
//
// Every tile is 128 output columns wide: on the first GEMM that is one
// 128-column group of z, so the fused re-quantisation of z to E4M3 G(128)
// finds each group's amax inside the tile.  BM 16/32 use 16x16x128 MFMA with
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

void launch_gemm_fp8(int kind, bool gated, int block_m, int bnz, const GemmParams& p,
                     int64_t max_mblk, hipStream_t s) {
  (void)bnz;  // always 128
  switch (kind) {
    case GEMM_Z_ROUTED:
      if (gated) dispatch_bm<A_GATHER, EPI_Z, true>(block_m, p, max_mblk, s);
      else dispatch_bm<A_GATHER, EPI_Z, false>(block_m, p, max_mblk, s);
      break;
    case GEMM_Y_ROUTED:
      dispatch_bm<A_ROWS, EPI_OUT_ROUTED, false>(block_m, p, max_mblk, s);
      break;
    case GEMM_Z_DENSE:
      if (gated) dispatch_bm<A_DENSE, EPI_Z, true>(block_m, p, max_mblk, s);
      else dispatch_bm<A_DENSE, EPI_Z, false>(block_m, p, max_mblk, s);
      break;
    default:
      dispatch_bm<A_DENSE, EPI_OUT_DENSE, false>(block_m, p, max_mblk, s);
      break;
  }
}

}  // namespace moe
