// fp8 E4M3 grouped-GEMM instantiations (see gemm_impl.h for the kernel).
//
// First-GEMM tiles are 128 output columns wide: one 128-column group of z,
// so the fused re-quantisation of z to E4M3 G(128) finds each group's amax
// inside the tile.  Second GEMMs of 16 or 32 rows are 256 columns wide.  BM 16/32 use 16x16x128 MFMA with
// 4 waves split along N, BM 64/128/256 use 32x32x64 MFMA on 2x4 waves (two
// per SIMD).  256-row tiles serve the second GEMM (and ungated first GEMMs):
// the gated first GEMM would need a partial set beside 2 x 128 accumulators
// per lane, which spills (swapped and promoted fragment by fragment too), so
// it runs two 128-row tiles per 256-row block.
#include "gemm_impl.h"

namespace moe {

// Each dispatcher launches the tile for (block_m, width) and returns 0, or
// returns -1 without launching when no such tile exists.  With p == nullptr
// it only answers whether the tile exists (the host asks before it
// enqueues anything).
template <class C>
static int run(const GemmParams* p, int64_t max_mblk, hipStream_t s) {
  if (p) launch_gemm<C>(*p, max_mblk, s);
  return 0;
}

// LDS stages: three for the 128-row first-GEMM tiles (two k-tiles of loads
// in flight, 144 KB; the activation scales then come by a direct load per
// k-tile into a ring unless the tile's whole table fits beside), two for the
// rest (a third stage made the 256-row second GEMM slower: DeepSeek-V3
// T=8192 2.03 -> 2.15 ms).
constexpr int fp8_stages(int bm, int ep) { return bm == 128 && ep == EPI_Z ? 3 : 2; }

// Every fp8 tile runs with swapped operands (GemmCfg::SWAP).
template <int BM, int BNZ, int WM, int WN, int MF, bool GATED, int AM, int EP>
using Fp8Cfg = GemmCfg<BM, BNZ, WM, WN, MF, true, GATED, AM, EP, fp8_stages(BM, EP), 128, false, true>;

template <int AM, int EP, bool GATED>
static int dispatch_bm(int block_m, const GemmParams* p, int64_t max_mblk, hipStream_t s) {
  switch (block_m) {
    case 16: return run<Fp8Cfg<16, 128, 1, 4, 16, GATED, AM, EP>>(p, max_mblk, s);
    case 32: return run<Fp8Cfg<32, 128, 1, 4, 16, GATED, AM, EP>>(p, max_mblk, s);
    case 64: return run<Fp8Cfg<64, 128, 2, 4, 32, GATED, AM, EP>>(p, max_mblk, s);
    case 128:
      // first GEMMs only: the 128-row second-GEMM tile keeps two workgroups
      // per CU on two stages (gemm_min_waves_per_eu)
      return run<Fp8Cfg<128, 128, 2, 4, 32, GATED, AM, EP>>(p, max_mblk, s);
    case 256:
      // 256-row tiles exist for the ungated GEMMs only (a gated 256-row
      // tile does not fit the registers)
      if constexpr (!GATED) return run<Fp8Cfg<256, 128, 2, 4, 32, false, AM, EP>>(p, max_mblk, s);
      return -1;
    default:
      return -1;
  }
}

// Second GEMMs of 16 or 32 rows on 256-column tiles (gemm_tile_n): each
// wave's 64 columns stay inside one 128-row weight-scale block.
template <int AM, int EP>
static int dispatch_wide(int block_m, const GemmParams* p, int64_t max_mblk, hipStream_t s) {
  if (block_m == 16) return run<Fp8Cfg<16, 256, 1, 4, 16, false, AM, EP>>(p, max_mblk, s);
  if (block_m == 32) return run<Fp8Cfg<32, 256, 1, 4, 16, false, AM, EP>>(p, max_mblk, s);
  return -1;
}

int launch_gemm_fp8(int kind, bool gated, int block_m, int bnz, const GemmParams* p,
                    int64_t max_mblk, hipStream_t s) {
  const bool first = kind == GEMM_Z_ROUTED || kind == GEMM_Z_DENSE;
  if (bnz != 128 && !(bnz == 256 && !first)) return -1;
  switch (kind) {
    case GEMM_Z_ROUTED:
      return gated ? dispatch_bm<A_GATHER, EPI_Z, true>(block_m, p, max_mblk, s)
                   : dispatch_bm<A_GATHER, EPI_Z, false>(block_m, p, max_mblk, s);
    case GEMM_Y_ROUTED:
      return bnz == 256 ? dispatch_wide<A_ROWS, EPI_OUT_ROUTED>(block_m, p, max_mblk, s)
                        : dispatch_bm<A_ROWS, EPI_OUT_ROUTED, false>(block_m, p, max_mblk, s);
    case GEMM_Z_DENSE:
      return gated ? dispatch_bm<A_DENSE, EPI_Z, true>(block_m, p, max_mblk, s)
                   : dispatch_bm<A_DENSE, EPI_Z, false>(block_m, p, max_mblk, s);
    case GEMM_Y_DENSE:
      return bnz == 256 ? dispatch_wide<A_DENSE, EPI_OUT_DENSE>(block_m, p, max_mblk, s)
                        : dispatch_bm<A_DENSE, EPI_OUT_DENSE, false>(block_m, p, max_mblk, s);
    default:
      return -1;
  }
}

}  // namespace moe
