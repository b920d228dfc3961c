// bf16 grouped-GEMM instantiations (see gemm_impl.h for the kernel).
//
// Tile shapes by align block size BM (rows per expert block):
//   BM 16/32  -- 16x16x32 MFMA, the 4 waves split N (skinny, weight-streaming)
//   BM 64/128 -- 32x32x16 MFMA, 2x2 waves
//   BM 256    -- 32x32x16 MFMA, 4x1 waves, 64x64 (gated: x2) per wave
// Gated first GEMM: 64 z columns per tile (64 gate + 64 up weight rows);
// everything else 128 output columns per tile.
#include "gemm_impl.h"

namespace moe {

template <int AM, int EP, bool GATED, int BNZ>
static void dispatch_bm(int block_m, const GemmParams& p, int64_t max_mblk, hipStream_t s) {
  switch (block_m) {
    case 16: launch_gemm<GemmCfg<16, BNZ, 1, 4, 16, false, GATED, AM, EP>>(p, max_mblk, s); break;
    case 32: launch_gemm<GemmCfg<32, BNZ, 1, 4, 16, false, GATED, AM, EP>>(p, max_mblk, s); break;
    case 64: launch_gemm<GemmCfg<64, BNZ, 2, 2, 32, false, GATED, AM, EP>>(p, max_mblk, s); break;
    case 128: launch_gemm<GemmCfg<128, BNZ, 2, 2, 32, false, GATED, AM, EP>>(p, max_mblk, s); break;
    default: launch_gemm<GemmCfg<256, BNZ, 4, 1, 32, false, GATED, AM, EP>>(p, max_mblk, s); break;
  }
}

void launch_gemm_bf16(int kind, bool gated, int block_m, const GemmParams& p, int64_t max_mblk,
                      hipStream_t s) {
  switch (kind) {
    case GEMM_Z_ROUTED:
      if (gated) dispatch_bm<A_GATHER, EPI_Z, true, 64>(block_m, p, max_mblk, s);
      else dispatch_bm<A_GATHER, EPI_Z, false, 128>(block_m, p, max_mblk, s);
      break;
    case GEMM_Y_ROUTED:
      dispatch_bm<A_ROWS, EPI_OUT_ROUTED, false, 128>(block_m, p, max_mblk, s);
      break;
    case GEMM_Z_DENSE:
      if (gated) dispatch_bm<A_DENSE, EPI_Z, true, 64>(block_m, p, max_mblk, s);
      else dispatch_bm<A_DENSE, EPI_Z, false, 128>(block_m, p, max_mblk, s);
      break;
    default:
      dispatch_bm<A_DENSE, EPI_OUT_DENSE, false, 128>(block_m, p, max_mblk, s);
      break;
  }
}

int gemm_tile_n(int kind, bool fp8, bool gated, int block_m) {
  (void)block_m;
  if (!fp8 && gated && (kind == GEMM_Z_ROUTED || kind == GEMM_Z_DENSE)) return 64;
  return 128;
}

}  // namespace moe
