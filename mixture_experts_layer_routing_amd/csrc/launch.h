// Internal launchers (host side) of the HIP kernels.  Arguments are checked
// by the C-ABI layer before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace moe {

void launch_route(const float* logits, int T, int E, int top_k, int scoring, int renorm,
                  int32_t* ids, float* w, hipStream_t s);

void launch_prepare(const uint16_t* a1, int T, int H, const float* w, int apply_weight,
                    int quant, void* a1q, float* a1q_scale, hipStream_t s);

size_t align_workspace_bytes(int64_t n, int E);
// Routing and align of a decode-sized batch in one launch (one wave), with
// the outputs of launch_route and launch_align; only where
// decode_prologue_fits (T <= 8, T*top_k <= 64, E <= 1024, sorted capacity <= 16384).
bool decode_prologue_fits(int T, int top_k, int E, int64_t sorted_cap);
void launch_decode_prologue(const float* logits, int T, int E, int top_k, int scoring,
                            int renorm, int32_t* ids, float* weights, int BM, int32_t* counts,
                            int32_t* offsets, int32_t* sorted, int64_t sorted_cap,
                            int32_t* block_ids, int64_t block_cap, int32_t* ntp, hipStream_t s);
void launch_align(const int32_t* ids, int64_t n, int E, int BM, int32_t* counts,
                  int32_t* offsets, int32_t* sorted, int64_t sorted_cap, int32_t* block_ids,
                  int64_t block_cap, int32_t* ntp, void* ws, hipStream_t s);

// Block schedule of the batched format (counts [E] -> sorted rows e*M + m,
// block owners, padded row total), block_cap = E * ceil(M / bm).
void launch_batched_schedule(const int32_t* counts, int E, int M, int bm, int64_t block_cap,
                             int32_t* sorted, int32_t* block_expert, int32_t* ntp, hipStream_t s);

// ypart / shpart (optional, only without gamma): split-K partials of the
// routed rows [ysplit][T*k][H] and of the shared expert [shsplit][T][H],
// summed here in split order and rounded to bf16 in place of y / sh.
void launch_finalize(void* out, float* out_scale, int out_quant, const uint16_t* y,
                     const float* w, int T, int k, int H, int woi, const uint16_t* sh,
                     const uint16_t* res, uint16_t* res_out, const uint16_t* gamma, float eps,
                     hipStream_t s, const float* ypart = nullptr, int ysplit = 1,
                     const float* shpart = nullptr, int shsplit = 1);

// One grouped-GEMM launch (see gemm_impl.h).
struct GemmParams {
  const uint8_t* a;        // activation rows: bf16 or fp8 bytes, row length K
  const float* a_scale;    // fp8: scale of (row, k-block kb) at a_scale[row*sa_row + kb*sa_k]
  int64_t sa_row;          //   G(128): (K/128, 1); per token: (1, 0); per tensor: (0, 0)
  int sa_k;
  const uint8_t* w;        // expert 0's (or the shared expert's) weight matrix [n_w][K]
  const float* w_scale;    // fp8: [n_w/128][K/128] per expert
  int64_t w_stride;        // bytes between consecutive experts' matrices
  int64_t ws_stride;       // floats between consecutive experts' scale grids
  int K;                   // reduction length in elements
  int inter;               // gated: row offset of the up half (I)
  int n_tiles;             // output column tiles
  const int32_t* sorted;   // align outputs (routed launches)
  const int32_t* block_expert;
  const int32_t* ntp;
  const int32_t* expert_offsets;   // align's padded offsets [E+1] (rows), or null:
                                   // then the tile order ignores expert boundaries
  int T, top_k;
  int align_bm;            // align block size (routed launches); a multiple of the tile BM
  void* out;               // z / fused_expert_output / shared_out
  float* out_scale;        // fp8 z scales [rows][ldo/128]
  int ldo;                 // output row length in elements
  int act;                 // first GEMM's activation: ACT_SILU or ACT_GELU
  // Split K: ksplit > 1 cuts the k-tiles into ksplit equal ranges, one
  // workgroup each; every workgroup then writes its fp32 partial tile to
  // partial[split][row][col] (rows as in the output, part_rows per split,
  // ldp columns: gate then up for the gated first GEMM) and a reduction
  // kernel finishes the epilogue.
  int ksplit;
  float* partial;
  int64_t part_rows;
  int ldp;
  // Routed second GEMM only: index the partial rows by the flat row
  // t*top_k + j (sorted[row]) instead of the sorted row, pad rows skipped,
  // so that finalize can sum a token's partials itself.
  int part_flat;
  // Weight rows through a 3-deep ring where a tile exists for it
  // (GemmCfg::SPLIT): set for the routed bf16 GEMMs, whose 256-row tiles
  // stream weights with little reuse at medium T.
  int split_ring;
};

enum ActFn { ACT_SILU = 0, ACT_GELU = 1 };

// Finish a split first GEMM: z[r] = act(sum of partials) -> bf16 or fp8
// G(128) (+ scales).  Rows: the padded routed rows up to *ntp (pad rows get
// zeros), or the T dense rows when sorted == nullptr.
void launch_splitk_z(const float* partial, int ksplit, int64_t part_rows, int ldp,
                     int64_t max_rows, const int32_t* ntp, const int32_t* sorted, int nflat,
                     int T, int inter, bool gated, int act, bool fp8, void* z, float* z_scale,
                     int ldz, hipStream_t s);
// Finish a split second GEMM: y = bf16(sum of partials) written to
// out[sorted[r]] (routed; pad rows skipped) or out[r] (dense rows < T).
void launch_splitk_y(const float* partial, int ksplit, int64_t part_rows, int ldp,
                     int64_t max_rows, const int32_t* ntp, const int32_t* sorted, int nflat,
                     int T, int n, uint16_t* out, int ldo, hipStream_t s);

enum GemmKind {
  GEMM_Z_ROUTED = 0,   // first GEMM of the routed experts (gather), activation, z out
  GEMM_Y_ROUTED = 1,   // second GEMM of the routed experts, scatter to [T, k, H]
  GEMM_Z_DENSE = 2,    // first GEMM of the shared expert over all T rows
  GEMM_Y_DENSE = 3     // second GEMM of the shared expert
};

// Output column tile of a launch (BNZ: z columns for the first GEMM, H
// columns for the second) for an output of n columns.
int gemm_tile_n(int kind, bool fp8, bool gated, int block_m, int n);
// Launch one grouped GEMM with output tile bnz; max_mblk bounds the M-blocks
// (grid sizing).  Returns 0, or -1 (nothing launched) when no tile of that
// (kind, gated, block_m, bnz) exists.  p == nullptr only asks the question.
int launch_gemm_bf16(int kind, bool gated, int block_m, int bnz, const GemmParams* p,
                     int64_t max_mblk, hipStream_t s);
int launch_gemm_fp8(int kind, bool gated, int block_m, int bnz, const GemmParams* p,
                    int64_t max_mblk, hipStream_t s);

}  // namespace moe
