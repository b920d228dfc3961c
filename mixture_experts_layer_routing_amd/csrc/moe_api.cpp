// C ABI of libmoe.so: argument checks, workspace sizing and kernel launches.
// The declarations and the contract of every entry point are in moe.h.
#include "../../include/moe.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>

#include "launch.h"
#include "monolithic.h"

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

int check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return MOE_OK;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Bump allocator over the caller's workspace (sizes only when base is null);
// `last` is the byte offset of the most recent piece.
struct Carve {
  char* base;
  size_t used = 0;
  size_t last = 0;
  explicit Carve(void* b) : base(static_cast<char*>(b)) {}
  void* take(size_t bytes) {
    void* p = base ? base + used : nullptr;
    last = used;
    used += align_up(bytes);
    return p;
  }
};

bool quant_fp8(int quant) {
  return quant == MOE_QUANT_FP8_G128 || quant == MOE_QUANT_FP8_TOKEN ||
         quant == MOE_QUANT_FP8_TENSOR;
}
// The prepare quant_config: a known format with the one group and weight
// block size the kernels implement (128; the per-token and per-tensor
// formats have no channel group).
int check_quant_config(const moe_quant_config* qc) {
  if (!qc) return fail(MOE_ERR_INVALID_ARG, "quant_config is NULL");
  if (qc->quant == MOE_QUANT_NONE) return MOE_OK;
  if (!quant_fp8(qc->quant)) return fail(MOE_ERR_UNSUPPORTED, "quant %d not supported", qc->quant);
  const int group = qc->quant == MOE_QUANT_FP8_G128 ? 128 : 0;
  if (qc->act_group != group)
    return fail(MOE_ERR_UNSUPPORTED, "act_group %d: quant %d takes %d", qc->act_group, qc->quant,
                group);
  if (qc->w_block_n != 128 || qc->w_block_k != 128)
    return fail(MOE_ERR_UNSUPPORTED, "weight blocks %dx%d: only 128x128", qc->w_block_n,
                qc->w_block_k);
  return MOE_OK;
}

// fp32 scales of an fp8 [rows, K] activation in the given format
size_t act_scale_count(int quant, int64_t rows, int K) {
  if (quant == MOE_QUANT_FP8_G128) return static_cast<size_t>(rows) * (K / 128);
  if (quant == MOE_QUANT_FP8_TOKEN) return static_cast<size_t>(rows);
  if (quant == MOE_QUANT_FP8_TENSOR) return 1;
  return 0;
}
// GEMM strides of those scales: (row, 128-deep k-block)
void act_scale_strides(int quant, int K, int64_t* sa_row, int* sa_k) {
  *sa_row = quant == MOE_QUANT_FP8_G128 ? K / 128 : (quant == MOE_QUANT_FP8_TOKEN ? 1 : 0);
  *sa_k = quant == MOE_QUANT_FP8_G128 ? 1 : 0;
}

// Gated activations read the gate and up halves of W13; GELU or SiLU.
bool act_gated(int activation) {
  return activation == MOE_ACT_SILU_MUL || activation == MOE_ACT_GELU_MUL;
}
int act_fn(int activation) {
  return (activation == MOE_ACT_GELU_MUL || activation == MOE_ACT_GELU_NO_MUL) ? moe::ACT_GELU
                                                                               : moe::ACT_SILU;
}

bool valid_block_m(int bm) { return bm == 16 || bm == 32 || bm == 64 || bm == 128 || bm == 256; }

struct Caps {
  int64_t sorted_cap, block_cap;
};

Caps capacities(int T, int top_k, int E, int bm) {
  const int64_t n = static_cast<int64_t>(T) * top_k;
  const int64_t cap = n + std::min<int64_t>(E, n) * (bm - 1);
  return {cap, (cap + bm - 1) / bm};
}

// The rows the routed GEMMs walk.  Standard format: align's schedule over
// the T*top_k flat rows of a [T, H] activation (top_k rows per token).
// Batched format: the schedule built from per-expert counts over the E*M
// rows of an [E, M, H] activation, each its own "token" (top_k 1).
struct Routed {
  int T, top_k;
  Caps cp;
};

Routed standard_rows(int T, int top_k, int E, int bm) { return {T, top_k, capacities(T, top_k, E, bm)}; }

Routed batched_rows(int E, int M, int bm) {
  const int64_t nb = (static_cast<int64_t>(M) + bm - 1) / bm;
  return {E * M, 1, {E * nb * bm, E * nb}};
}

int dense_block_m(int T) {
  if (T <= 16) return 16;
  if (T <= 32) return 32;
  if (T <= 64) return 64;
  return 128;
}

// Row tiles of the shared expert's two dense GEMMs (first: W13, second: W2):
// from 1024 tokens the bf16 GEMMs take the 256-row tiles of the routed
// path (Llama-4 shared expert at T=2048 on MI355X: 0.64 -> 0.54 ms).
int dense_block_m(int T, bool fp8, bool first) {
  (void)first;
  if (!fp8 && T >= 1024) return 256;
  return dense_block_m(T);
}

int check_weights(const moe_weights* w, int H, int activation, bool need_ptrs) {
  if (!w) return fail(MOE_ERR_INVALID_ARG, "weights is NULL");
  if (w->num_experts < 1 || w->num_experts > 1024)
    return fail(MOE_ERR_INVALID_ARG, "num_experts %d outside [1, 1024]", w->num_experts);
  if (w->quant != MOE_QUANT_NONE && !quant_fp8(w->quant))
    return fail(MOE_ERR_UNSUPPORTED, "weight quant %d not supported", w->quant);
  if (activation < MOE_ACT_SILU_MUL || activation > MOE_ACT_GELU_NO_MUL)
    return fail(MOE_ERR_UNSUPPORTED, "activation %d not supported", activation);
  if (H <= 0 || H % 128) return fail(MOE_ERR_UNSUPPORTED, "H=%d must be a positive multiple of 128", H);
  if (H > 16384 || w->inter > 16384 || w->shared_inter > 16384)
    return fail(MOE_ERR_UNSUPPORTED, "H and I are limited to 16384 (fp8 scale staging, K > 16384)");
  const bool fp8 = quant_fp8(w->quant);
  const bool gated = act_gated(activation);
  const int step = (!fp8 && gated) ? 64 : 128;
  if (w->inter <= 0 || w->inter % step)
    return fail(MOE_ERR_UNSUPPORTED, "I=%d must be a positive multiple of %d", w->inter, step);
  if (w->shared_inter < 0 || (w->shared_inter > 0 && w->shared_inter % step))
    return fail(MOE_ERR_UNSUPPORTED, "shared I=%d must be a multiple of %d", w->shared_inter, step);
  if (need_ptrs) {
    if (!w->w13 || !w->w2) return fail(MOE_ERR_INVALID_ARG, "w13/w2 is NULL");
    if (fp8 && (!w->w13_scale || !w->w2_scale))
      return fail(MOE_ERR_INVALID_ARG, "fp8 weights need w13_scale and w2_scale");
    if (w->shared_inter > 0) {
      if (!w->shared_w13 || !w->shared_w2) return fail(MOE_ERR_INVALID_ARG, "shared weights are NULL");
      if (fp8 && (!w->shared_w13_scale || !w->shared_w2_scale))
        return fail(MOE_ERR_INVALID_ARG, "fp8 shared weights need scales");
    }
  }
  return MOE_OK;
}

// Tile height of the routed second GEMM: the align block (z is read
// row-contiguously, so a tile could also be half a block).  256-row bf16
// tiles over H read half the bytes per flop of 128-row ones; the K split
// below keeps their smaller grid balanced.
int second_gemm_bm(bool fp8, int bm) { return (void)fp8, bm; }

// Tile height of the routed first GEMM: the align block, except that a gated
// fp8 tile stops at 128 rows (two per 256-row block).
int first_gemm_bm(bool fp8, bool gated, int bm) { return (fp8 && gated) ? std::min(bm, 128) : bm; }

// Output width of the routed first GEMM's tile.  A bf16 gated tile of fewer
// than 128 rows has 64 z columns by default (gemm_tile_n); it takes 128 (half
// the tiles, each streaming twice the weight rows against the same gathered
// rows) while the launch still holds at least two such tiles per CU, by the
// same block estimate as the K split (n = T*top_k ids, min(E, n) experts
// touched).  Measured on MI355X: Llama-4 T=128 GEMM-1 0.471 -> 0.457 ms,
// Mixtral T=32 0.354 -> 0.351 ms; Mixtral T=1 (224 such tiles) 0.083 -> 0.092.
int first_gemm_bn(bool fp8, bool gated, int bm1, int I, int64_t n, int E) {
  int bn = moe::gemm_tile_n(moe::GEMM_Z_ROUTED, fp8, gated, bm1, I);
  if (!fp8 && gated && bn == 64 && I % 128 == 0) {
    const int64_t touched = std::min<int64_t>(E, n);
    if ((touched + (n - touched) / bm1) * (I / 128) >= 2 * 256) bn = 128;
  }
  return bn;
}

// The bf16 second GEMM on 256 x 256 tiles runs one workgroup per CU; with
// fewer than four rounds of tiles (1024) the last round leaves CUs idle, so
// its K is cut in exactly two (measured on MI355X, Mixtral/Llama-4 shapes:
// 7-19 % faster than 128-row tiles without a split, the fp32 partials
// included; four ways lose to two once the partials approach half the
// weight bytes).
int balance_split(bool fp8, int bm2, int64_t tiles, int K, int ktile, int S) {
  const int nk = K / ktile;
  if (fp8 || bm2 != 256 || tiles >= 1024 || nk % 2 || nk / 2 < 8) return S;
  return 2;
}

// Split K (see GemmParams::ksplit): a launch with fewer than 384 output
// tiles (1.5 per CU; decode-sized T, or the shared expert over a few
// tokens) cuts its k-tiles into 2, 4 or 8 ranges.  S doubles while the grid
// stays within 1024 workgroups, every range keeps at least 8 k-tiles, and
// the fp32 partials (written and read once: 8*S*rows*ldp bytes) stay within
// half the weight bytes the launch streams.  The routed tile count and the
// touched experts are estimated from n = T*k alone (min(E, n) experts, each
// starting a block, the other rows filling further blocks), since the real
// ones are known only on the device.
int pick_ksplit(int64_t tiles, int K, int ktile, int64_t rows, int64_t ldp, double wbytes) {
  if (tiles >= 384) return 1;
  const int nk = K / ktile;
  int S = 1;
  while (S < 8 && tiles * S * 2 <= 1024 && nk % (2 * S) == 0 && nk / (2 * S) >= 8 &&
         8.0 * (2 * S) * rows * ldp <= 0.5 * wbytes)
    S *= 2;
  return S;
}

struct SplitPlan {
  int s1, s2, s3, s4;   // routed GEMM-1, routed GEMM-2, shared GEMM-1, shared GEMM-2
  size_t partial_bytes;
};

SplitPlan split_plan(const Routed& rt, int T, int H, const moe_weights* w, int activation,
                     int bm) {
  using namespace moe;
  const bool fp8 = quant_fp8(w->quant);
  const bool gated = act_gated(activation);
  const int ktile = fp8 ? 128 : 64;
  const int E = w->num_experts, I = w->inter;
  const int64_t n = static_cast<int64_t>(rt.T) * rt.top_k;
  const double eb = fp8 ? 1.0 : 2.0;
  const int64_t touched = std::min<int64_t>(E, n);
  auto est_blocks = [&](int b) { return touched + (n - touched) / b; };
  SplitPlan sp{1, 1, 1, 1, 0};
  const int64_t rows = rt.cp.block_cap * bm;
  const int64_t R = gated ? 2 * I : I;
  const int bm1 = first_gemm_bm(fp8, gated, bm);
  const int bn1 = first_gemm_bn(fp8, gated, bm1, I, n, E);
  sp.s1 = pick_ksplit(est_blocks(bm1) * (I / bn1), H, ktile, rows, R,
                      static_cast<double>(touched) * R * H * eb);
  const int bm2 = second_gemm_bm(fp8, bm);
  const int bn2 = gemm_tile_n(GEMM_Y_ROUTED, fp8, gated, bm2, H);
  sp.s2 = pick_ksplit(est_blocks(bm2) * (H / bn2), I, ktile, rows, H,
                      static_cast<double>(touched) * H * I * eb);
  sp.s2 = balance_split(fp8, bm2, est_blocks(bm2) * (H / bn2), I, ktile, sp.s2);
  size_t b = 0;
  if (sp.s1 > 1) b = std::max<size_t>(b, static_cast<size_t>(sp.s1) * rows * R * 4);
  if (sp.s2 > 1) b = std::max<size_t>(b, static_cast<size_t>(sp.s2) * rows * H * 4);
  if (w->shared_inter > 0) {
    const int Is = w->shared_inter;
    const int dbm3 = dense_block_m(T, fp8, true), dbm4 = dense_block_m(T, fp8, false);
    const int64_t mblk3 = (T + dbm3 - 1) / dbm3, mblk4 = (T + dbm4 - 1) / dbm4;
    const int64_t Rs = gated ? 2 * Is : Is;
    const int bn3 = gemm_tile_n(GEMM_Z_DENSE, fp8, gated, dbm3, Is);
    sp.s3 = pick_ksplit(mblk3 * (Is / bn3), H, ktile, T, Rs, static_cast<double>(Rs) * H * eb);
    const int bn4 = gemm_tile_n(GEMM_Y_DENSE, fp8, gated, dbm4, H);
    sp.s4 = pick_ksplit(mblk4 * (H / bn4), Is, ktile, T, H, static_cast<double>(H) * Is * eb);
    if (sp.s3 > 1) b = std::max<size_t>(b, static_cast<size_t>(sp.s3) * T * Rs * 4);
    if (sp.s4 > 1) b = std::max<size_t>(b, static_cast<size_t>(sp.s4) * T * H * 4);
  }
  sp.partial_bytes = b;
  return sp;
}

// Workspace of the experts stage: z for the routed rows and for the shared
// expert, in the GEMM input format of the second GEMM, then the split-K
// partial sums (shared by the launches, which run in stream order).
size_t experts_ws(const Routed& rt, int T, int H, const moe_weights* w, int activation, int bm,
                  Carve& c, void** z, float** zs, void** zsh, float** zshs, float** part,
                  size_t* offs = nullptr) {
  const bool fp8 = quant_fp8(w->quant);
  const size_t eb = fp8 ? 1 : 2;
  const int64_t rows = rt.cp.block_cap * bm;
  const size_t start = c.used;
  const size_t none = static_cast<size_t>(-1);
  size_t o[5] = {none, none, none, none, static_cast<size_t>(rows)};
  *z = c.take(static_cast<size_t>(rows) * w->inter * eb);
  o[0] = c.last - start;
  *zs = nullptr;
  if (fp8) {
    *zs = static_cast<float*>(c.take(static_cast<size_t>(rows) * (w->inter / 128) * 4));
    o[1] = c.last - start;
  }
  *zsh = nullptr;
  *zshs = nullptr;
  if (w->shared_inter > 0) {
    *zsh = c.take(static_cast<size_t>(T) * w->shared_inter * eb);
    o[2] = c.last - start;
    if (fp8) {
      *zshs = static_cast<float*>(c.take(static_cast<size_t>(T) * (w->shared_inter / 128) * 4));
      o[3] = c.last - start;
    }
  }
  const SplitPlan sp = split_plan(rt, T, H, w, activation, bm);
  *part = sp.partial_bytes ? static_cast<float*>(c.take(sp.partial_bytes)) : nullptr;
  if (offs) for (int i = 0; i < 5; ++i) offs[i] = o[i];
  return c.used - start;
}

struct StageEvents {
  hipEvent_t* ev;
  hipStream_t s;
  void mark(int i) const {
    if (ev) (void)hipEventRecord(ev[i], s);
  }
};

// Whether a GEMM tile exists for each of the four launches the experts
// stage would make (routed first and second GEMM, shared expert's two):
// asked before anything is enqueued, so an unsupported request leaves no
// partial work behind.
int tiles_exist(int T, int H, const moe_weights* w, int activation, int bm) {
  using namespace moe;
  const bool fp8 = quant_fp8(w->quant);
  const bool gated = act_gated(activation);
  auto has = [&](int kind, int blk_m, int bnz) {
    return (fp8 ? launch_gemm_fp8(kind, gated, blk_m, bnz, nullptr, 0, nullptr)
                : launch_gemm_bf16(kind, gated, blk_m, bnz, nullptr, 0, nullptr)) == 0;
  };
  const int bm1 = first_gemm_bm(fp8, gated, bm);
  const int bm2 = second_gemm_bm(fp8, bm);
  struct Q { int kind, bm, bn; } q[4] = {
      {GEMM_Z_ROUTED, bm1, gemm_tile_n(GEMM_Z_ROUTED, fp8, gated, bm1, w->inter)},
      {GEMM_Y_ROUTED, bm2, gemm_tile_n(GEMM_Y_ROUTED, fp8, gated, bm2, H)}, {0, 0, 0}, {0, 0, 0}};
  int nq = 2;
  if (w->shared_inter > 0) {
    const int dbm3 = dense_block_m(T, fp8, true), dbm4 = dense_block_m(T, fp8, false);
    q[nq++] = {GEMM_Z_DENSE, dbm3, gemm_tile_n(GEMM_Z_DENSE, fp8, gated, dbm3, w->shared_inter)};
    q[nq++] = {GEMM_Y_DENSE, dbm4, gemm_tile_n(GEMM_Y_DENSE, fp8, gated, dbm4, H)};
  }
  for (int i = 0; i < nq; ++i)
    if (!has(q[i].kind, q[i].bm, q[i].bn))
      return fail(MOE_ERR_UNSUPPORTED, "no %s GEMM tile for kind %d, %d rows x %d columns%s",
                  fp8 ? "fp8" : "bf16", q[i].kind, q[i].bm, q[i].bn, gated ? " (gated)" : "");
  return MOE_OK;
}

// Second-GEMM partials left to finalize (whole-layer forward only): when a
// second GEMM splits its K and the region is given, the GEMM writes its
// partials there and the split-K reduction launch is skipped; ysplit /
// shsplit report the split (1: fused_expert_output / shared_out written).
struct Deferred {
  float* ypart;    // [s2][T*top_k][H]
  float* shpart;   // [s4][T][H]
  int ysplit = 1, shsplit = 1;
};

int run_experts(const void* a1q, const float* a1q_scale, const void* shared_in,
                const float* shared_in_scale, const Routed& rt, int T, int H, const moe_weights* w,
                int activation, const int32_t* sorted, const int32_t* block_expert,
                const int32_t* ntp, const int32_t* offsets, int bm, uint16_t* feo,
                uint16_t* shared_out, void* ws, const StageEvents& se, hipStream_t s,
                Deferred* defer = nullptr) {
  using namespace moe;
  const bool fp8 = quant_fp8(w->quant);
  const bool gated = act_gated(activation);
  const size_t eb = fp8 ? 1 : 2;
  const int I = w->inter;
  const int R = gated ? 2 * I : I;
  Carve c(ws);
  void *z, *zsh;
  float *zs, *zshs, *part;
  experts_ws(rt, T, H, w, activation, bm, c, &z, &zs, &zsh, &zshs, &part);
  const SplitPlan sp = split_plan(rt, T, H, w, activation, bm);
  const Caps& cp = rt.cp;
  const int64_t rows = cp.block_cap * bm;
  const int nflat = rt.T * rt.top_k;
  // every tile was checked to exist before anything was enqueued (tiles_exist)
  auto launch = [&](int kind, int blk_m, int bnz, const GemmParams& p, int64_t max_mblk) {
    if (fp8) (void)launch_gemm_fp8(kind, gated, blk_m, bnz, &p, max_mblk, s);
    else (void)launch_gemm_bf16(kind, gated, blk_m, bnz, &p, max_mblk, s);
  };
  const int act = act_fn(activation);
  // Weight rows through the 3-deep ring (routed launches whose experts
  // average at most one block of rows: each weight tile then serves one
  // block and its loads stream from HBM; measured 9-10 % faster there,
  // 2 % slower at Mixtral T=4096 with four blocks per expert).
  const int64_t touched_e = std::min<int64_t>(w->num_experts, std::max<int64_t>(nflat, 1));
  const bool stream_rows = nflat <= touched_e * bm;
  auto split = [&](GemmParams& g, int S, int64_t part_rows, int ldp) {
    g.act = act;
    g.split_ring = (g.sorted != nullptr && stream_rows) ? 1 : 0;
    g.ksplit = S;
    g.partial = S > 1 ? part : nullptr;
    g.part_rows = part_rows;
    g.ldp = ldp;
  };
  // routed first GEMM: gather a1q rows, activation, z [rows, I]
  GemmParams p{};
  p.a = static_cast<const uint8_t*>(a1q);
  p.a_scale = a1q_scale;
  act_scale_strides(w->quant, H, &p.sa_row, &p.sa_k);
  p.w = static_cast<const uint8_t*>(w->w13);
  p.w_scale = w->w13_scale;
  p.w_stride = static_cast<int64_t>(R) * H * eb;
  p.ws_stride = static_cast<int64_t>(R / 128) * (H / 128);
  p.K = H;
  p.inter = I;
  const int bm1 = first_gemm_bm(fp8, gated, bm);
  const int bn1 = first_gemm_bn(fp8, gated, bm1, I, static_cast<int64_t>(rt.T) * rt.top_k,
                                w->num_experts);
  p.n_tiles = I / bn1;
  p.sorted = sorted;
  p.block_expert = block_expert;
  p.ntp = ntp;
  p.expert_offsets = offsets;
  p.T = rt.T;
  p.top_k = rt.top_k;
  p.align_bm = bm;
  p.out = z;
  p.out_scale = zs;
  p.ldo = I;
  split(p, sp.s1, rows, R);
  launch(GEMM_Z_ROUTED, bm1, bn1, p, cp.block_cap * (bm / bm1));
  if (sp.s1 > 1)
    launch_splitk_z(part, sp.s1, rows, R, rows, ntp, sorted, nflat, rt.T, I, gated, act, fp8, z,
                    zs, I, s);
  se.mark(4);
  // routed second GEMM: z rows -> fused_expert_output[sorted row]
  const int bm2 = second_gemm_bm(fp8, bm);
  GemmParams q{};
  q.a = static_cast<const uint8_t*>(z);
  q.a_scale = zs;
  act_scale_strides(MOE_QUANT_FP8_G128, I, &q.sa_row, &q.sa_k);   // z: G(128) along I
  q.w = static_cast<const uint8_t*>(w->w2);
  q.w_scale = w->w2_scale;
  q.w_stride = static_cast<int64_t>(H) * I * eb;
  q.ws_stride = static_cast<int64_t>(H / 128) * (I / 128);
  q.K = I;
  q.inter = 0;
  const int bn2 = gemm_tile_n(GEMM_Y_ROUTED, fp8, gated, bm2, H);
  q.n_tiles = H / bn2;
  q.sorted = sorted;
  q.block_expert = block_expert;
  q.ntp = ntp;
  q.expert_offsets = offsets;
  q.T = rt.T;
  q.top_k = rt.top_k;
  q.align_bm = bm;
  q.out = feo;
  q.ldo = H;
  split(q, sp.s2, rows, H);
  const bool defer_y = defer && defer->ypart && sp.s2 > 1;
  if (defer_y) {
    q.partial = defer->ypart;
    q.part_rows = nflat;
    q.part_flat = 1;
    defer->ysplit = sp.s2;
  }
  launch(GEMM_Y_ROUTED, bm2, bn2, q, cp.block_cap * (bm / bm2));
  if (sp.s2 > 1 && !defer_y)
    launch_splitk_y(part, sp.s2, rows, H, rows, ntp, sorted, nflat, rt.T, H, feo, H, s);
  se.mark(5);
  if (w->shared_inter > 0) {
    const int Is = w->shared_inter;
    const int Rs = gated ? 2 * Is : Is;
    const int dbm3 = dense_block_m(T, fp8, true), dbm4 = dense_block_m(T, fp8, false);
    const int64_t mblk3 = (T + dbm3 - 1) / dbm3, mblk4 = (T + dbm4 - 1) / dbm4;
    GemmParams d{};
    d.a = static_cast<const uint8_t*>(shared_in);
    d.a_scale = shared_in_scale;
    act_scale_strides(w->quant, H, &d.sa_row, &d.sa_k);
    d.w = static_cast<const uint8_t*>(w->shared_w13);
    d.w_scale = w->shared_w13_scale;
    d.K = H;
    d.inter = Is;
    const int bn3 = gemm_tile_n(GEMM_Z_DENSE, fp8, gated, dbm3, Is);
    d.n_tiles = Is / bn3;
    d.T = T;
    d.top_k = 1;
    d.align_bm = dbm3;
    d.out = zsh;
    d.out_scale = zshs;
    d.ldo = Is;
    split(d, sp.s3, T, Rs);
    launch(GEMM_Z_DENSE, dbm3, bn3, d, mblk3);
    if (sp.s3 > 1)
      launch_splitk_z(part, sp.s3, T, Rs, T, nullptr, nullptr, 0, T, Is, gated, act, fp8, zsh, zshs,
                      Is, s);
    GemmParams e{};
    e.a = static_cast<const uint8_t*>(zsh);
    e.a_scale = zshs;
    act_scale_strides(MOE_QUANT_FP8_G128, Is, &e.sa_row, &e.sa_k);
    e.w = static_cast<const uint8_t*>(w->shared_w2);
    e.w_scale = w->shared_w2_scale;
    e.K = Is;
    const int bn4 = gemm_tile_n(GEMM_Y_DENSE, fp8, gated, dbm4, H);
    e.n_tiles = H / bn4;
    e.T = T;
    e.top_k = 1;
    e.align_bm = dbm4;
    e.out = shared_out;
    e.ldo = H;
    split(e, sp.s4, T, H);
    const bool defer_sh = defer && defer->shpart && sp.s4 > 1;
    if (defer_sh) {
      e.partial = defer->shpart;
      defer->shsplit = sp.s4;
    }
    launch(GEMM_Y_DENSE, dbm4, bn4, e, mblk4);
    if (sp.s4 > 1 && !defer_sh)
      launch_splitk_y(part, sp.s4, T, H, T, nullptr, nullptr, 0, T, H, shared_out, H, s);
  }
  se.mark(6);
  return check_launch("moe_experts");
}

}  // namespace

extern "C" {

const char* moe_status_str(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
    default: return "MOE_ERR_UNKNOWN";
  }
}

const char* moe_last_error(void) { return g_err; }

// Block size by average rows per expert, from sweeps on MI355X over the
// Mixtral/DeepSeek/Llama-4 shapes: skinny experts want short tiles (weight
// streaming, more workgroups); from ~100 rows the 8-wave 256-row bf16 tile
// wins even with padding.  fp8 takes 256-row blocks only from ~200 rows per
// expert (DeepSeek-V3 T=8192: the second GEMM gains 15 %, the gated first
// GEMM, which runs 128-row tiles, loses 6 % to the extra padding).
int moe_pick_block_m(int T, int top_k, int num_experts, int quant) {
  if (T <= 0 || top_k <= 0 || num_experts <= 0) return 16;
  const int64_t avg = (static_cast<int64_t>(T) * top_k + num_experts - 1) / num_experts;
  if (avg <= 16) return 16;
  if (avg <= 32) return 32;
  if (quant_fp8(quant)) return avg <= 96 ? 64 : (avg <= 192 ? 128 : 256);
  return avg <= 64 ? 64 : 256;
}

int moe_route(const float* logits, int T, int E, int top_k, int scoring, int renormalize,
              int32_t* topk_ids, float* topk_weights, hipStream_t stream) {
  g_err[0] = 0;
  if (T < 0) return fail(MOE_ERR_INVALID_ARG, "T=%d < 0", T);
  if (E < 1 || E > 1024) return fail(MOE_ERR_INVALID_ARG, "E=%d outside [1, 1024]", E);
  if (top_k < 1 || top_k > std::min(E, 64))
    return fail(MOE_ERR_INVALID_ARG, "top_k=%d outside [1, min(E, 64)]", top_k);
  if (scoring != MOE_SCORING_SOFTMAX && scoring != MOE_SCORING_SIGMOID)
    return fail(MOE_ERR_INVALID_ARG, "scoring=%d", scoring);
  if (T == 0) return MOE_OK;
  if (!logits || !topk_ids || !topk_weights) return fail(MOE_ERR_INVALID_ARG, "NULL pointer");
  moe::launch_route(logits, T, E, top_k, scoring, renormalize ? 1 : 0, topk_ids, topk_weights,
                    stream);
  return check_launch("moe_route");
}

int moe_prepare(const uint16_t* a1, int T, int H, const float* topk_weights,
                const int32_t* topk_ids, int top_k, int apply_router_weight_on_input,
                const moe_quant_config* qc, void* a1q, float* a1q_scale, hipStream_t stream) {
  g_err[0] = 0;
  (void)topk_ids;   // no dispatch without expert parallelism: the ids pass through
  if (int st = check_quant_config(qc)) return st;
  const int quant = qc->quant;
  if (T < 0 || H <= 0 || H % 8) return fail(MOE_ERR_INVALID_ARG, "T=%d H=%d", T, H);
  if (quant_fp8(quant) && H % 128)
    return fail(MOE_ERR_INVALID_ARG, "fp8 needs H %% 128 == 0 (H=%d)", H);
  if (quant == MOE_QUANT_FP8_TOKEN && H > 16384)
    return fail(MOE_ERR_UNSUPPORTED, "per-token fp8 holds a row in registers: H=%d > 16384", H);
  if (top_k < 1) return fail(MOE_ERR_INVALID_ARG, "top_k=%d < 1", top_k);
  if (apply_router_weight_on_input && top_k != 1)
    return fail(MOE_ERR_INVALID_ARG, "router weight on the input needs top_k == 1 (got %d)", top_k);
  if (T == 0) return MOE_OK;
  if (!a1 || !a1q || (apply_router_weight_on_input && !topk_weights) ||
      (quant_fp8(quant) && !a1q_scale))
    return fail(MOE_ERR_INVALID_ARG, "NULL pointer");
  if (quant_fp8(quant) && static_cast<const void*>(a1) == a1q)
    return fail(MOE_ERR_INVALID_ARG, "a1q may not alias a1 for fp8");
  moe::launch_prepare(a1, T, H, topk_weights, apply_router_weight_on_input ? 1 : 0, quant, a1q,
                      a1q_scale, stream);
  return check_launch("moe_prepare");
}

int moe_align_capacity(int T, int top_k, int E, int block_m, int64_t* sorted_capacity,
                       int64_t* block_capacity) {
  g_err[0] = 0;
  if (T < 0 || top_k < 1 || E < 1 || !valid_block_m(block_m))
    return fail(MOE_ERR_INVALID_ARG, "T=%d top_k=%d E=%d block_m=%d", T, top_k, E, block_m);
  const Caps c = capacities(T, top_k, E, block_m);
  if (sorted_capacity) *sorted_capacity = c.sorted_cap;
  if (block_capacity) *block_capacity = c.block_cap;
  return MOE_OK;
}

size_t moe_align_workspace_bytes(int T, int top_k, int E, int block_m) {
  (void)block_m;
  if (T <= 0 || top_k <= 0 || E <= 0) return 0;
  return moe::align_workspace_bytes(static_cast<int64_t>(T) * top_k, E);
}

int moe_align(const int32_t* topk_ids, int T, int top_k, int E, int block_m,
              int32_t* expert_counts, int32_t* expert_offsets, int32_t* sorted_token_ids,
              int32_t* block_expert_ids, int32_t* num_tokens_post_padded, void* workspace,
              size_t workspace_bytes, hipStream_t stream) {
  g_err[0] = 0;
  if (T < 0 || top_k < 1 || E < 1 || E > 1024)
    return fail(MOE_ERR_INVALID_ARG, "T=%d top_k=%d E=%d", T, top_k, E);
  if (!valid_block_m(block_m)) return fail(MOE_ERR_INVALID_ARG, "block_m=%d", block_m);
  if (static_cast<int64_t>(T) * top_k > (1 << 30)) return fail(MOE_ERR_INVALID_ARG, "T*top_k too large");
  if (!expert_counts || !expert_offsets || !num_tokens_post_padded || (T > 0 && !topk_ids) ||
      (T > 0 && (!sorted_token_ids || !block_expert_ids)))
    return fail(MOE_ERR_INVALID_ARG, "NULL pointer");
  const size_t need = moe_align_workspace_bytes(T, top_k, E, block_m);
  if (need && (!workspace || workspace_bytes < need))
    return fail(MOE_ERR_WORKSPACE, "align workspace %zu < %zu", workspace_bytes, need);
  const Caps c = capacities(T, top_k, E, block_m);
  moe::launch_align(topk_ids, static_cast<int64_t>(T) * top_k, E, block_m, expert_counts,
                    expert_offsets, sorted_token_ids, c.sorted_cap, block_expert_ids, c.block_cap,
                    num_tokens_post_padded, workspace, stream);
  return check_launch("moe_align");
}

size_t moe_experts_workspace_bytes(int T, int H, int top_k, const moe_weights* weights,
                                   int activation, int block_m) {
  if (!weights || T < 0 || top_k < 1 || !valid_block_m(block_m)) return 0;
  if (check_weights(weights, H, activation, false) != MOE_OK) return 0;
  Carve c(nullptr);
  void *z, *zsh;
  float *zs, *zshs, *part;
  return experts_ws(standard_rows(T, top_k, weights->num_experts, block_m), T, H, weights,
                    activation, block_m, c, &z, &zs, &zsh, &zshs, &part);
}

int moe_experts_workspace_layout(int T, int H, int top_k, const moe_weights* weights,
                                 int activation, int block_m, size_t* out) {
  g_err[0] = 0;
  if (!out || T < 0 || top_k < 1 || !valid_block_m(block_m))
    return fail(MOE_ERR_INVALID_ARG, "bad arguments");
  if (int st = check_weights(weights, H, activation, false)) return st;
  Carve c(nullptr);
  void *z, *zsh;
  float *zs, *zshs, *part;
  experts_ws(standard_rows(T, top_k, weights->num_experts, block_m), T, H, weights, activation,
             block_m, c, &z, &zs, &zsh, &zshs, &part, out);
  return MOE_OK;
}

int moe_experts(const void* a1q, const float* a1q_scale, const void* shared_in,
                const float* shared_in_scale, int T, int H, int top_k,
                const moe_weights* weights, int activation, const int32_t* sorted_token_ids,
                const int32_t* block_expert_ids, const int32_t* num_tokens_post_padded,
                int block_m, uint16_t* fused_expert_output, uint16_t* shared_out,
                void* workspace, size_t workspace_bytes, hipStream_t stream) {
  g_err[0] = 0;
  if (T < 0 || top_k < 1) return fail(MOE_ERR_INVALID_ARG, "T=%d top_k=%d", T, top_k);
  if (!valid_block_m(block_m)) return fail(MOE_ERR_INVALID_ARG, "block_m=%d", block_m);
  if (int st = check_weights(weights, H, activation, true)) return st;
  if (top_k > weights->num_experts) return fail(MOE_ERR_INVALID_ARG, "top_k > E");
  const bool fp8 = quant_fp8(weights->quant);
  if (static_cast<int64_t>(T) * top_k > (1 << 30)) return fail(MOE_ERR_INVALID_ARG, "T*top_k too large");
  if (T == 0) return MOE_OK;
  if (!a1q || !sorted_token_ids || !block_expert_ids || !num_tokens_post_padded ||
      !fused_expert_output || (fp8 && !a1q_scale))
    return fail(MOE_ERR_INVALID_ARG, "NULL pointer");
  if (weights->shared_inter > 0 && (!shared_in || !shared_out || (fp8 && !shared_in_scale)))
    return fail(MOE_ERR_INVALID_ARG, "shared expert needs shared_in (+scale) and shared_out");
  const size_t need = moe_experts_workspace_bytes(T, H, top_k, weights, activation, block_m);
  if (!workspace || workspace_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "experts workspace %zu < %zu", workspace_bytes, need);
  if (int st = tiles_exist(T, H, weights, activation, block_m)) return st;
  return run_experts(a1q, a1q_scale, shared_in, shared_in_scale,
                     standard_rows(T, top_k, weights->num_experts, block_m), T, H, weights,
                     activation, sorted_token_ids, block_expert_ids, num_tokens_post_padded,
                     nullptr, block_m, fused_expert_output, shared_out, workspace,
                     StageEvents{nullptr, stream}, stream);
}

namespace {

// Workspace of the batched experts: the block schedule, then the experts
// stage's own pieces.  The shared expert is not part of this stage.
struct BatchedLayout {
  int32_t *sorted, *blocks, *ntp;
  void* experts_ws;
  size_t experts_ws_bytes;
  size_t offs[5];   // experts_ws pieces, from the workspace start (SIZE_MAX = absent)
};

moe_weights routed_only(const moe_weights* w) {
  moe_weights r = *w;
  r.shared_inter = 0;
  r.shared_w13 = r.shared_w2 = nullptr;
  r.shared_w13_scale = r.shared_w2_scale = nullptr;
  return r;
}

int batched_block_m(int M, int block_m, int quant) {
  return block_m ? block_m : moe_pick_block_m(M, 1, 1, quant);
}

size_t batched_layout(int M, int H, const moe_weights* w, int activation, int bm, void* base,
                      BatchedLayout* L) {
  const Routed rt = batched_rows(w->num_experts, M, bm);
  Carve c(base);
  L->sorted = static_cast<int32_t*>(c.take(static_cast<size_t>(rt.cp.sorted_cap) * 4));
  L->blocks = static_cast<int32_t*>(c.take(static_cast<size_t>(rt.cp.block_cap) * 4));
  L->ntp = static_cast<int32_t*>(c.take(4));
  Carve sub(nullptr);
  void *z, *zsh;
  float *zs, *zshs, *part;
  L->experts_ws_bytes =
      experts_ws(rt, 0, H, w, activation, bm, sub, &z, &zs, &zsh, &zshs, &part, L->offs);
  L->experts_ws = c.take(L->experts_ws_bytes);
  for (int i = 0; i < 4; ++i)
    if (L->offs[i] != static_cast<size_t>(-1)) L->offs[i] += c.last;
  return c.used;
}

}  // namespace

size_t moe_experts_batched_workspace_bytes(int max_tokens, int H, const moe_weights* weights,
                                           int activation, int block_m) {
  if (!weights || max_tokens < 0) return 0;
  if (check_weights(weights, H, activation, false) != MOE_OK) return 0;
  const moe_weights w = routed_only(weights);
  const int bm = batched_block_m(max_tokens, block_m, w.quant);
  if (!valid_block_m(bm)) return 0;
  if (static_cast<int64_t>(w.num_experts) * (max_tokens + bm) > (1 << 30)) return 0;
  BatchedLayout L;
  return batched_layout(max_tokens, H, &w, activation, bm, nullptr, &L);
}

int moe_experts_batched_workspace_layout(int max_tokens, int H, const moe_weights* weights,
                                         int activation, int block_m, size_t* out) {
  g_err[0] = 0;
  if (!out || max_tokens < 0) return fail(MOE_ERR_INVALID_ARG, "bad arguments");
  if (int st = check_weights(weights, H, activation, false)) return st;
  const moe_weights w = routed_only(weights);
  const int bm = batched_block_m(max_tokens, block_m, w.quant);
  if (!valid_block_m(bm)) return fail(MOE_ERR_INVALID_ARG, "block_m=%d", bm);
  BatchedLayout L;
  batched_layout(max_tokens, H, &w, activation, bm, nullptr, &L);
  out[0] = 0;   // the schedule is the first piece
  out[1] = L.offs[0];
  out[2] = L.offs[1];
  out[3] = L.offs[4];
  return MOE_OK;
}

int moe_experts_batched(const void* a, const float* a_scale, const int32_t* expert_num_tokens,
                        int max_tokens, int H, const moe_weights* weights, int activation,
                        int block_m, uint16_t* out, void* workspace, size_t workspace_bytes,
                        hipStream_t stream) {
  g_err[0] = 0;
  if (max_tokens < 0) return fail(MOE_ERR_INVALID_ARG, "max_tokens=%d < 0", max_tokens);
  if (int st = check_weights(weights, H, activation, true)) return st;
  const moe_weights w = routed_only(weights);
  const int bm = batched_block_m(max_tokens, block_m, w.quant);
  if (!valid_block_m(bm)) return fail(MOE_ERR_INVALID_ARG, "block_m=%d", bm);
  const bool fp8 = quant_fp8(w.quant);
  const int E = w.num_experts;
  if (static_cast<int64_t>(E) * (max_tokens + bm) > (1 << 30))
    return fail(MOE_ERR_INVALID_ARG, "E*(max_tokens+block_m) too large");
  if (max_tokens == 0) return MOE_OK;
  if (!a || !expert_num_tokens || !out || (fp8 && !a_scale))
    return fail(MOE_ERR_INVALID_ARG, "NULL pointer");
  BatchedLayout L;
  const size_t need = batched_layout(max_tokens, H, &w, activation, bm, nullptr, &L);
  if (!workspace || workspace_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "batched experts workspace %zu < %zu", workspace_bytes, need);
  if (int st = tiles_exist(0, H, &w, activation, bm)) return st;
  batched_layout(max_tokens, H, &w, activation, bm, workspace, &L);
  const Routed rt = batched_rows(E, max_tokens, bm);
  moe::launch_batched_schedule(expert_num_tokens, E, max_tokens, bm, rt.cp.block_cap, L.sorted,
                               L.blocks, L.ntp, stream);
  if (int st = check_launch("moe_experts_batched schedule")) return st;
  return run_experts(a, a_scale, nullptr, nullptr, rt, 0, H, &w, activation, L.sorted, L.blocks,
                     L.ntp, nullptr, bm, out, nullptr, L.experts_ws, StageEvents{nullptr, stream},
                     stream);
}

int moe_finalize(void* output, float* output_scale, int out_quant,
                 const uint16_t* fused_expert_output, const float* topk_weights,
                 const int32_t* topk_ids, int T, int top_k, int H,
                 int apply_router_weight_on_input, const uint16_t* shared,
                 const uint16_t* residual, uint16_t* residual_out, const uint16_t* gamma,
                 float eps, hipStream_t stream) {
  g_err[0] = 0;
  (void)topk_ids;
  if (T < 0 || top_k < 1 || top_k > 64) return fail(MOE_ERR_INVALID_ARG, "T=%d top_k=%d", T, top_k);
  if (H <= 0 || H % 8 || H > 16384) return fail(MOE_ERR_INVALID_ARG, "H=%d", H);
  if (out_quant != MOE_QUANT_NONE && out_quant != MOE_QUANT_FP8_G128)
    return fail(MOE_ERR_UNSUPPORTED, "out_quant %d", out_quant);
  if (out_quant == MOE_QUANT_FP8_G128 && H % 128)
    return fail(MOE_ERR_INVALID_ARG, "fp8 output needs H %% 128 == 0");
  if (!(eps >= 0.0f)) return fail(MOE_ERR_INVALID_ARG, "eps must be >= 0");
  if (T == 0) return MOE_OK;
  if (!output || !fused_expert_output || (!apply_router_weight_on_input && !topk_weights) ||
      (out_quant == MOE_QUANT_FP8_G128 && !output_scale))
    return fail(MOE_ERR_INVALID_ARG, "NULL pointer");
  moe::launch_finalize(output, output_scale, out_quant, fused_expert_output, topk_weights, T, top_k,
                       H, apply_router_weight_on_input ? 1 : 0, shared, residual, residual_out,
                       gamma, eps, stream);
  return check_launch("moe_finalize");
}

namespace {

struct ForwardLayout {
  int32_t* ids;
  float* tw;
  void* a1q;
  float* a1q_scale;
  void* shin;
  float* shin_scale;
  int32_t *counts, *offsets, *sorted, *blocks, *ntp;
  void* align_ws;
  void* experts_ws;
  size_t experts_ws_bytes;
  uint16_t* feo;
  uint16_t* shared_out;
  float* ypart;    // split second GEMMs' partials, summed by finalize (or null)
  float* shpart;
};

size_t forward_layout(int T, int H, int top_k, const moe_weights* w, int activation, int bm,
                      int woi, void* base, ForwardLayout* L) {
  Carve c(base);
  const bool fp8 = quant_fp8(w->quant);
  const size_t eb = fp8 ? 1 : 2;
  const int E = w->num_experts;
  const int64_t n = static_cast<int64_t>(T) * top_k;
  const Caps cp = capacities(T, top_k, E, bm);
  L->ids = static_cast<int32_t*>(c.take(n * 4));
  L->tw = static_cast<float*>(c.take(n * 4));
  L->a1q = c.take(static_cast<size_t>(T) * H * eb);
  L->a1q_scale = fp8 ? static_cast<float*>(c.take(act_scale_count(w->quant, T, H) * 4)) : nullptr;
  L->shin = nullptr;
  L->shin_scale = nullptr;
  if (w->shared_inter > 0 && woi && fp8) {
    L->shin = c.take(static_cast<size_t>(T) * H);
    L->shin_scale = static_cast<float*>(c.take(act_scale_count(w->quant, T, H) * 4));
  }
  L->counts = static_cast<int32_t*>(c.take(E * 4));
  L->offsets = static_cast<int32_t*>(c.take((E + 1) * 4));
  L->sorted = static_cast<int32_t*>(c.take(cp.sorted_cap * 4));
  L->blocks = static_cast<int32_t*>(c.take(cp.block_cap * 4));
  L->ntp = static_cast<int32_t*>(c.take(4));
  L->align_ws = c.take(moe::align_workspace_bytes(n, E));
  Carve sub(nullptr);
  void *z, *zsh;
  float *zs, *zshs, *part;
  L->experts_ws_bytes = experts_ws(standard_rows(T, top_k, E, bm), T, H, w, activation, bm, sub, &z,
                                   &zs, &zsh, &zshs, &part);
  L->experts_ws = c.take(L->experts_ws_bytes);
  L->feo = static_cast<uint16_t*>(c.take(static_cast<size_t>(n) * H * 2));
  L->shared_out = w->shared_inter > 0 ? static_cast<uint16_t*>(c.take(static_cast<size_t>(T) * H * 2))
                                      : nullptr;
  const SplitPlan sp = split_plan(standard_rows(T, top_k, E, bm), T, H, w, activation, bm);
  L->ypart = sp.s2 > 1 ? static_cast<float*>(c.take(static_cast<size_t>(sp.s2) * n * H * 4)) : nullptr;
  L->shpart = (w->shared_inter > 0 && sp.s4 > 1)
                  ? static_cast<float*>(c.take(static_cast<size_t>(sp.s4) * T * H * 4))
                  : nullptr;
  return c.used;
}

}  // namespace

size_t moe_forward_workspace_bytes(int T, int H, int top_k, const moe_weights* weights,
                                   int activation, int block_m, int apply_router_weight_on_input) {
  if (!weights || T < 0 || top_k < 1) return 0;
  if (check_weights(weights, H, activation, false) != MOE_OK) return 0;
  const int bm = block_m ? block_m : moe_pick_block_m(T, top_k, weights->num_experts, weights->quant);
  if (!valid_block_m(bm)) return 0;
  ForwardLayout L;
  return forward_layout(T, H, top_k, weights, activation, bm, apply_router_weight_on_input, nullptr,
                        &L);
}

// The forward's argument checks (host only, nothing enqueued); *bm gets
// the block size the call uses.  MOE_OK with T == 0 means a no-op.
static int forward_args(const uint16_t* x, const float* logits, int T, int H, int top_k,
                        int scoring, int apply_router_weight_on_input,
                        const moe_weights* weights, int activation, int block_m, float eps,
                        int out_quant, const void* output, const float* output_scale, int* bm) {
  if (T < 0) return fail(MOE_ERR_INVALID_ARG, "T=%d < 0", T);
  if (int st = check_weights(weights, H, activation, true)) return st;
  const int E = weights->num_experts;
  if (top_k < 1 || top_k > std::min(E, 64)) return fail(MOE_ERR_INVALID_ARG, "top_k=%d", top_k);
  if (scoring != MOE_SCORING_SOFTMAX && scoring != MOE_SCORING_SIGMOID)
    return fail(MOE_ERR_INVALID_ARG, "scoring=%d", scoring);
  if (apply_router_weight_on_input && top_k != 1)
    return fail(MOE_ERR_INVALID_ARG, "router weight on the input needs top_k == 1");
  if (out_quant != MOE_QUANT_NONE && out_quant != MOE_QUANT_FP8_G128)
    return fail(MOE_ERR_UNSUPPORTED, "out_quant %d", out_quant);
  if (H > 16384) return fail(MOE_ERR_INVALID_ARG, "H=%d > 16384", H);
  if (!(eps >= 0.0f)) return fail(MOE_ERR_INVALID_ARG, "eps must be >= 0");
  if (static_cast<int64_t>(T) * top_k > (1 << 30)) return fail(MOE_ERR_INVALID_ARG, "T*top_k too large");
  *bm = block_m ? block_m : moe_pick_block_m(T, top_k, E, weights->quant);
  if (!valid_block_m(*bm)) return fail(MOE_ERR_INVALID_ARG, "block_m=%d", *bm);
  if (T == 0) return MOE_OK;
  if (!x || !logits || !output || (out_quant == MOE_QUANT_FP8_G128 && !output_scale))
    return fail(MOE_ERR_INVALID_ARG, "NULL pointer");
  return MOE_OK;
}

int moe_forward(const uint16_t* x, const float* logits, int T, int H, int top_k, int scoring,
                int renormalize, int apply_router_weight_on_input, const moe_weights* weights,
                int activation, int block_m, const uint16_t* residual, const uint16_t* gamma,
                float eps, int out_quant, void* output, float* output_scale,
                uint16_t* residual_out, void* workspace, size_t workspace_bytes,
                hipEvent_t* stage_events, hipStream_t stream) {
  g_err[0] = 0;
  int bm = 0;
  if (int st = forward_args(x, logits, T, H, top_k, scoring, apply_router_weight_on_input,
                            weights, activation, block_m, eps, out_quant, output, output_scale,
                            &bm))
    return st;
  if (T == 0) return MOE_OK;
  const int E = weights->num_experts;
  const bool fp8 = quant_fp8(weights->quant);
  ForwardLayout L;
  const size_t need = forward_layout(T, H, top_k, weights, activation, bm,
                                     apply_router_weight_on_input, nullptr, &L);
  if (!workspace || workspace_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "forward workspace %zu < %zu", workspace_bytes, need);
  if (int st = tiles_exist(T, H, weights, activation, bm)) return st;
  forward_layout(T, H, top_k, weights, activation, bm, apply_router_weight_on_input, workspace,
                 &L);
  const StageEvents se{stage_events, stream};
  const int quant = weights->quant;
  const int64_t n = static_cast<int64_t>(T) * top_k;
  const Caps cp = capacities(T, top_k, E, bm);

  // decode-sized batches: routing and align in one launch (stage 1 then
  // covers both, and the align stage is empty)
  const bool prologue = moe::decode_prologue_fits(T, top_k, E, cp.sorted_cap);
  se.mark(0);
  if (prologue)
    moe::launch_decode_prologue(logits, T, E, top_k, scoring, renormalize ? 1 : 0, L.ids, L.tw, bm,
                                L.counts, L.offsets, L.sorted, cp.sorted_cap, L.blocks,
                                cp.block_cap, L.ntp, stream);
  else
    moe::launch_route(logits, T, E, top_k, scoring, renormalize ? 1 : 0, L.ids, L.tw, stream);
  se.mark(1);
  const void* a1q = x;
  if (quant_fp8(quant) || apply_router_weight_on_input) {
    moe::launch_prepare(x, T, H, L.tw, apply_router_weight_on_input ? 1 : 0, quant, L.a1q,
                        L.a1q_scale, stream);
    a1q = L.a1q;
  }
  // The shared expert reads the unweighted input in a1q's format.
  const void* shin = a1q;
  const float* shin_scale = L.a1q_scale;
  if (weights->shared_inter > 0 && apply_router_weight_on_input) {
    if (fp8) {
      moe::launch_prepare(x, T, H, nullptr, 0, quant, L.shin, L.shin_scale, stream);
      shin = L.shin;
      shin_scale = L.shin_scale;
    } else {
      shin = x;
      shin_scale = nullptr;
    }
  }
  se.mark(2);
  if (!prologue)
    moe::launch_align(L.ids, n, E, bm, L.counts, L.offsets, L.sorted, cp.sorted_cap, L.blocks,
                      cp.block_cap, L.ntp, L.align_ws, stream);
  se.mark(3);
  // (with RMSNorm finalize needs whole rows in one workgroup, too few at
  // decode sizes to read split partials quickly: reduce the splits first)
  Deferred df{gamma ? nullptr : L.ypart, gamma ? nullptr : L.shpart};
  int st = run_experts(a1q, L.a1q_scale, shin, shin_scale, standard_rows(T, top_k, E, bm), T, H,
                       weights, activation, L.sorted, L.blocks, L.ntp, L.offsets, bm, L.feo,
                       L.shared_out, L.experts_ws, se, stream, &df);
  if (st) return st;
  moe::launch_finalize(output, output_scale, out_quant, L.feo, L.tw, T, top_k, H,
                       apply_router_weight_on_input ? 1 : 0, L.shared_out, residual, residual_out,
                       gamma, eps, stream, df.ysplit > 1 ? L.ypart : nullptr, df.ysplit,
                       df.shsplit > 1 ? L.shpart : nullptr, df.shsplit);
  se.mark(7);
  return check_launch("moe_forward");
}

struct moe_graph {
  hipGraph_t graph;
  hipGraphExec_t exec;
};

int moe_forward_graph_create(const uint16_t* x, const float* logits, int T, int H, int top_k,
                             int scoring, int renormalize, int apply_router_weight_on_input,
                             const moe_weights* weights, int activation, int block_m,
                             const uint16_t* residual, const uint16_t* gamma, float eps,
                             int out_quant, void* output, float* output_scale,
                             uint16_t* residual_out, void* workspace, size_t workspace_bytes,
                             hipStream_t stream, moe_graph** graph) {
  g_err[0] = 0;
  if (!graph) return fail(MOE_ERR_INVALID_ARG, "graph is NULL");
  *graph = nullptr;
  if (!stream) return fail(MOE_ERR_INVALID_ARG, "capture needs a created stream, not the null stream");
  hipError_t e = hipStreamBeginCapture(stream, hipStreamCaptureModeThreadLocal);
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "hipStreamBeginCapture: %s", hipGetErrorString(e));
  const int st = moe_forward(x, logits, T, H, top_k, scoring, renormalize,
                             apply_router_weight_on_input, weights, activation, block_m, residual,
                             gamma, eps, out_quant, output, output_scale, residual_out, workspace,
                             workspace_bytes, nullptr, stream);
  hipGraph_t g = nullptr;
  e = hipStreamEndCapture(stream, &g);
  if (st != MOE_OK) {
    if (g) (void)hipGraphDestroy(g);
    return st;   // moe_forward's own message
  }
  if (e != hipSuccess || !g)
    return fail(MOE_ERR_HIP, "hipStreamEndCapture: %s", hipGetErrorString(e));
  hipGraphExec_t ex = nullptr;
  e = hipGraphInstantiate(&ex, g, nullptr, nullptr, 0);
  if (e != hipSuccess) {
    (void)hipGraphDestroy(g);
    return fail(MOE_ERR_HIP, "hipGraphInstantiate: %s", hipGetErrorString(e));
  }
  moe_graph* h = new (std::nothrow) moe_graph{g, ex};
  if (!h) {
    (void)hipGraphExecDestroy(ex);
    (void)hipGraphDestroy(g);
    return fail(MOE_ERR_INVALID_ARG, "out of host memory");
  }
  *graph = h;
  return MOE_OK;
}

int moe_forward_graph_launch(moe_graph* graph, hipStream_t stream) {
  g_err[0] = 0;
  if (!graph) return fail(MOE_ERR_INVALID_ARG, "graph is NULL");
  const hipError_t e = hipGraphLaunch(graph->exec, stream);
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "hipGraphLaunch: %s", hipGetErrorString(e));
  return MOE_OK;
}

int moe_forward_graph_destroy(moe_graph* graph) {
  g_err[0] = 0;
  if (!graph) return MOE_OK;
  const hipError_t a = hipGraphExecDestroy(graph->exec);
  const hipError_t b = hipGraphDestroy(graph->graph);
  delete graph;
  if (a != hipSuccess || b != hipSuccess)
    return fail(MOE_ERR_HIP, "graph destroy: %s", hipGetErrorString(a != hipSuccess ? a : b));
  return MOE_OK;
}

}  // extern "C"

// ---- moe_forward_monolithic: the layer in one launch ----

size_t moe_forward_monolithic_workspace_bytes(int T, int H, int top_k, const moe_weights* weights,
                                              int activation) {
  if (!weights || T <= 0 || top_k <= 0 || H <= 0) return 0;
  (void)activation;
  return moe::monolithic_workspace_bytes(T, H, top_k, weights->inter,
                                         std::max(weights->shared_inter, 0),
                                         quant_fp8(weights->quant));
}

int moe_forward_monolithic(const uint16_t* x, const float* logits, int T, int H, int top_k,
                           int scoring, int renormalize, int apply_router_weight_on_input,
                           const moe_weights* weights, int activation, const uint16_t* residual,
                           const uint16_t* gamma, float eps, int out_quant, void* output,
                           float* output_scale, uint16_t* residual_out, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  g_err[0] = 0;
  int bm = 0;
  if (int st = forward_args(x, logits, T, H, top_k, scoring, apply_router_weight_on_input,
                            weights, activation, 0, eps, out_quant, output, output_scale, &bm))
    return st;
  if (T == 0) return MOE_OK;
  if (weights->quant != MOE_QUANT_NONE && weights->quant != MOE_QUANT_FP8_G128)
    return fail(MOE_ERR_UNSUPPORTED,
                "the one-launch layer takes bf16 weights or fp8 with G(128) activations");
  if (weights->quant == MOE_QUANT_FP8_G128 && apply_router_weight_on_input)
    return fail(MOE_ERR_UNSUPPORTED, "the one-launch layer's fp8 path has no weight on the input");
  if (!moe::monolithic_fits(T, top_k))
    return fail(MOE_ERR_UNSUPPORTED, "the one-launch layer needs T <= 512 and T*top_k <= 512 (T=%d, top_k=%d)",
                T, top_k);
  const size_t need = moe_forward_monolithic_workspace_bytes(T, H, top_k, weights, activation);
  if (!workspace || workspace_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "one-launch workspace %zu < %zu", workspace_bytes, need);
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cs) != hipSuccess) {
    (void)hipGetLastError();
    return fail(MOE_ERR_HIP, "hipStreamIsCapturing failed");
  }
  if (cs != hipStreamCaptureStatusNone)
    return fail(MOE_ERR_UNSUPPORTED, "the one-launch layer cannot be captured into a graph");
  moe::MonoLaunch m{};
  m.x = x;
  m.logits = logits;
  m.T = T;
  m.H = H;
  m.E = weights->num_experts;
  m.top_k = top_k;
  m.scoring = scoring;
  m.renorm = renormalize ? 1 : 0;
  m.woi = apply_router_weight_on_input ? 1 : 0;
  m.act = act_fn(activation);
  m.gated = act_gated(activation) ? 1 : 0;
  m.w13 = static_cast<const uint16_t*>(weights->w13);
  m.w2 = static_cast<const uint16_t*>(weights->w2);
  m.I = weights->inter;
  m.sw13 = static_cast<const uint16_t*>(weights->shared_w13);
  m.sw2 = static_cast<const uint16_t*>(weights->shared_w2);
  m.Is = std::max(weights->shared_inter, 0);
  m.fp8 = weights->quant == MOE_QUANT_FP8_G128 ? 1 : 0;
  m.w13s = weights->w13_scale;
  m.w2s = weights->w2_scale;
  m.sw13s = weights->shared_w13_scale;
  m.sw2s = weights->shared_w2_scale;
  m.residual = residual;
  m.gamma = gamma;
  m.eps = eps;
  m.out_fp8 = out_quant == MOE_QUANT_FP8_G128 ? 1 : 0;
  m.out = output;
  m.out_scale = output_scale;
  m.residual_out = residual_out;
  m.ws = workspace;
  if (moe::launch_monolithic(m, stream) != 0)
    return fail(MOE_ERR_UNSUPPORTED, "the one-launch kernel does not fit the stream's CUs");
  return check_launch("moe_forward_monolithic");
}

// ---- moe_forward_noalloc: the forward on a fixed scratch array ----
//
// One array per GPU, defined here, held by each GPU the library runs on
// until the process ends.  Host code never passes `scratch` itself (its
// host-side name is a stand-in, not a device address): the device address
// comes from hipGetSymbolAddress, once per device, and is kept per device.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the device that owns `stream` (the
// current device for the null stream).
int scratch_for(hipStream_t stream, void** out) {
  int dev = 0;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "device of the stream: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MOE_ERR_UNSUPPORTED, "device %d beyond the %d the scratch table holds", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = 0;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return fail(MOE_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess)
      return fail(MOE_ERR_HIP, "hipSetDevice(%d): %s", dev, hipGetErrorString(e));
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    const hipError_t back = cur != dev ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess || !p)
      return fail(MOE_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                  hipGetErrorString(e));
    if (back != hipSuccess)
      return fail(MOE_ERR_HIP, "hipSetDevice(%d): %s", cur, hipGetErrorString(back));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_forward_noalloc(const uint16_t* x, const float* logits, int T, int H, int top_k,
                        int scoring, int renormalize, int apply_router_weight_on_input,
                        const moe_weights* weights, int activation, int block_m,
                        const uint16_t* residual, const uint16_t* gamma, float eps, int out_quant,
                        void* output, float* output_scale, uint16_t* residual_out,
                        hipStream_t stream) {
  g_err[0] = 0;
  int bm = 0;
  if (int st = forward_args(x, logits, T, H, top_k, scoring, apply_router_weight_on_input,
                            weights, activation, block_m, eps, out_quant, output, output_scale,
                            &bm))
    return st;
  if (T == 0) return MOE_OK;
  const size_t need = moe_forward_workspace_bytes(T, H, top_k, weights, activation, bm,
                                                  apply_router_weight_on_input);
  if (need > MOE_NOALLOC_SCRATCH_BYTES)
    return fail(MOE_ERR_WORKSPACE,
                "moe_forward_noalloc: these sizes need %zu bytes of scratch, above the fixed "
                "%zu (use moe_forward with a workspace)",
                need, static_cast<size_t>(MOE_NOALLOC_SCRATCH_BYTES));
  void* ws = nullptr;
  if (int st = scratch_for(stream, &ws)) return st;
  // Every piece of the forward's workspace is written before it is read
  // (align and the per-tensor scale clear their own counters with kernels),
  // so stale contents from an earlier call do not matter.
  return moe_forward(x, logits, T, H, top_k, scoring, renormalize, apply_router_weight_on_input,
                     weights, activation, block_m, residual, gamma, eps, out_quant, output,
                     output_scale, residual_out, ws, MOE_NOALLOC_SCRATCH_BYTES, nullptr, stream);
}

}  // extern "C"
