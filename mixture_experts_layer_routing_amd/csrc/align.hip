// align: sort the flat rows i = t*top_k + j by expert into block_m-padded
// groups, deterministically (ascending i inside every expert).
//
// Stable ranks.  A wave takes 64 ids at a time (one per lane) and needs,
// for every lane, the lanes holding the same expert id (its peers): the
// lane's rank is the number of peers below it, and the lowest peer (the
// leader) is the only lane that advances the expert's cursor.  Ways to find
// peers:
//   * ballots, one per bit of the id (AND over the bits of the lanes that
//     agree on that bit): ceil(log2 E) ballots and about six vector
//     instructions per bit (the tiled path's scatter);
//   * a per-wave table of 64-bit lane masks in LDS, one per expert: every lane
//     ORs its lane bit into its expert's entry, reads the entry back (the
//     wave's LDS operations complete in issue order, so the read sees every
//     OR of the instruction) and the leader clears it.  The OR is
//     commutative, so the mask does not depend on the order in which the LDS
//     serves the lanes.  A few LDS operations, whatever E is.
//   * for E <= 8, no peers at all: one-hot counts in 8-bit fields, summed
//     over the lanes by a DPP prefix scan.
// (Counting alone is order-free: per-id LDS atomic adds.)
//
// n <= 32768 ids: one 1024-thread workgroup does everything (count, padded
// offsets, block owners, scatter), re-reading the ids from the L2.
//
// Larger n with E <= 256, up to 65536 ids per CU the stream may use, and the
// stream not capturing a graph: the resident path, one launch that reads
// every id once.  One 1024-thread workgroup per CU holds a tile of up to
// 65536 consecutive ids (64 per lane, ranked as they land and kept as packed
// expert/rank pairs), publishes the tile's expert counts and places its ids
// into a 16-bit LDS stage in tile-slot order; after one grid barrier
// (per-workgroup arrival flags that workgroup 0 collects before it raises a
// go word, all tagged with a per-call epoch) each workgroup reads every
// tile's counts, takes the padded offsets and its own global slots, and
// copies each expert's run out with consecutive lanes on consecutive slots.
// The waits are bounded: a workgroup that waits too long gives up, and the
// call then leaves num_tokens_post_padded at -1.
//
// Otherwise (E > 256, n beyond what the grid can hold, or a stream under
// graph capture): tiles of 2048-8192 ids (see plan()), each split into 8
// wave sub-ranges, in three launches:
//   count   -- one workgroup per tile: per-(wave, expert) counts, and the
//              tile's per-expert totals in expert-major columns.  Tiles are
//              dealt to the XCDs in contiguous ranges (xcd_tile).
//   colscan -- one workgroup per expert: exclusive prefix of its column
//              over the tiles, and the expert's total
//   scatter -- one workgroup per tile: padded offsets from the totals; the
//              tile is sorted into its slots in LDS, then each expert's run
//              is copied to the global slots with consecutive lanes on
//              consecutive slots (whole lines, not one 4-byte store per
//              lane scattered over up to 64 lines); the workgroups also
//              share the block-owner and pad-sentinel fills.
// No atomics carry data to global memory on any path (the resident path's
// only global atomics are its flags), so the result is bit-exact and
// run-to-run identical.
#include "moe_device.h"
#include "launch.h"
#include "route_device.h"
#include "grid_sync.h"

#include <algorithm>
#include <atomic>
#include <chrono>
#include <cstdlib>
#include <random>
#include <type_traits>

namespace moe {
namespace {

constexpr int kMaxE = 1024;
constexpr int kSmallN = 32768;      // one-workgroup path up to this many ids
constexpr int kSmallThreads = 1024;
constexpr int kTileThreads = 512;   // multi-tile count and scatter: 8 waves
constexpr int kTileWaves = kTileThreads / 64;
constexpr int kMaxTile = 8192;      // ids per tile: its slots fill 32 KB of LDS
constexpr int kMidE = 256;          // scatter LDS sizing for E <= 256
constexpr int kScanThreads = 256;   // column scan: one workgroup per expert
constexpr int kLoads = 16;          // ids in flight per lane

int ceil_log2(int E) {
  int b = 0;
  while ((1 << b) < E) ++b;
  return b;
}

// Lanes of the wave whose key equals this lane's (among lanes with valid
// keys); every lane of the wave must call it (the ballots are wave-wide).
__device__ __forceinline__ uint64_t peer_mask(int key, bool valid, int nbits) {
  uint64_t m = __ballot(valid);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (key >> b) & 1;
    const uint64_t bal = __ballot(bit);
    m &= bit ? bal : ~bal;
  }
  return m;
}

// Adds the counts of the valid ids in [lo, hi) to h (this wave's E LDS
// ints).  Order does not matter here, so every lane adds its own ids with
// LDS atomics (no return value: nothing waits on them).  Measured faster
// than one add per group of equal ids found by ballots (peer_mask): the
// ballots cost more vector instructions than the atomics' conflicts.
__device__ void wave_count(const int32_t* __restrict__ ids, int lo, int hi, int E, int nbits,
                           int* h) {
  const int lane = threadIdx.x & 63;
  for (int c = lo; c < hi; c += 64 * kLoads) {
    int key[kLoads];
#pragma unroll
    for (int s = 0; s < kLoads; ++s) {
      const int i = c + 64 * s + lane;
      key[s] = i < hi ? ids[i] : -1;
    }
#pragma unroll
    for (int s = 0; s < kLoads; ++s) {
      if (static_cast<unsigned>(key[s]) < static_cast<unsigned>(E)) atomicAdd(&h[key[s]], 1);
    }
  }
}

// Stable slots of NK groups of 64 ids held in registers: key[s] is the
// expert of id c + 64*s + lane (-1 if none); out[cur[e]++] = id, in index
// order (out is the global slots, or a tile's slots in LDS).
template <int NK>
__device__ __forceinline__ void scatter_keys(const int (&key)[NK], int c, int E, int nbits,
                                             int* cur, int32_t* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const uint64_t below = lanemask_lt();
#pragma unroll
  for (int s = 0; s < NK; ++s) {
    const bool valid = static_cast<unsigned>(key[s]) < static_cast<unsigned>(E);
    const uint64_t m = peer_mask(key[s], valid, nbits);
    if (valid) {
      const int base = cur[key[s]];
      out[base + __builtin_popcountll(m & below)] = c + 64 * s + lane;
      if (lane == __builtin_ctzll(m)) cur[key[s]] = base + __builtin_popcountll(m);
    }
  }
}

// Writes the valid ids of [lo, hi) in index order: out[cur[e]++] = i.
__device__ void wave_scatter(const int32_t* __restrict__ ids, int lo, int hi, int E, int nbits,
                             int* cur, int32_t* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  for (int c = lo; c < hi; c += 64 * kLoads) {
    int key[kLoads];
#pragma unroll
    for (int s = 0; s < kLoads; ++s) {
      const int i = c + 64 * s + lane;
      key[s] = i < hi ? ids[i] : -1;
    }
    scatter_keys(key, c, E, nbits, cur, out);
  }
}

// Exclusive scan of v[0..count) in LDS by all NT threads of the block;
// returns the total.  `partial` needs NT/64 + 1 ints of LDS.
template <int NT>
__device__ int block_exclusive_scan(int* v, int count, int* partial) {
  const int tid = threadIdx.x;
  const int per = (count + NT - 1) / NT;
  const int lo = min(tid * per, count), hi = min(lo + per, count);
  int local = 0;
  for (int i = lo; i < hi; ++i) local += v[i];
  const int lane = tid & 63, wave = tid >> 6;
  int incl = local;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int up = __shfl_up(incl, o, 64);
    if (lane >= o) incl += up;
  }
  if (lane == 63) partial[wave] = incl;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int w = 0; w < NT / 64; ++w) { const int x = partial[w]; partial[w] = run; run += x; }
    partial[NT / 64] = run;
  }
  __syncthreads();
  int run = partial[wave] + incl - local;
  for (int i = lo; i < hi; ++i) { const int x = v[i]; v[i] = run; run += x; }
  const int total = partial[NT / 64];
  __syncthreads();
  return total;
}

// block_ids[b] for b in [b0, b1) by the NT threads of the block: the owner
// of block b is the last expert whose padded offset is <= b*BM (binary
// search over the E offsets in LDS; an empty expert shares its offset with
// the next one and owns no block), -1 at or past the padded total.
template <int NT>
__device__ void fill_block_owners(const int* off, int E, int BM, int total, int64_t b0,
                                  int64_t b1, int32_t* __restrict__ block_ids) {
  const int nblk = total / BM;
  for (int64_t b = b0 + threadIdx.x; b < b1; b += NT) {
    int owner = -1;
    if (b < nblk) {
      const int row = static_cast<int>(b) * BM;
      int lo = 0, hi = E - 1;   // off[lo] <= row (off[0] == 0)
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (off[mid] <= row) lo = mid;
        else hi = mid - 1;
      }
      owner = lo;
    }
    block_ids[b] = owner;
  }
}

// Per-expert totals -> counts, padded offsets, num_tokens_post_padded;
// returns the padded total.  `cnt` (LDS, E) holds totals on entry and the
// exclusive padded offsets on exit; `tot` (LDS, E) receives the totals.
template <int NT>
__device__ int finish_offsets(int* cnt, int E, int BM, int* partial,
                              int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                              int32_t* __restrict__ ntp, int* tot) {
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += NT) {
    const int c = cnt[e];
    counts[e] = c;
    tot[e] = c;
    cnt[e] = (c + BM - 1) / BM * BM;
  }
  __syncthreads();
  const int total = block_exclusive_scan<NT>(cnt, E, partial);
  for (int e = tid; e < E; e += NT) offsets[e] = cnt[e];
  if (tid == 0) { offsets[E] = total; ntp[0] = total; }
  return total;
}

// Pad sentinel n in the slots [off[e] + cnt[e], off[e + 1]) of the experts
// e = w0, w0 + wstep, ... (one wave per expert: fewer than BM <= 256 slots,
// so at most 4 stores per lane) and in [p0, p1) of the tail past the padded
// total (all threads, step pstep).
__device__ __forceinline__ void fill_sentinels(const int* off, const int32_t* cnt, int E, int n,
                                               int w0, int wstep, int64_t p0, int64_t p1,
                                               int pstep, int32_t* __restrict__ sorted) {
  const int lane = threadIdx.x & 63;
  for (int e = w0; e < E; e += wstep)
    for (int p = off[e] + cnt[e] + lane; p < off[e + 1]; p += 64) sorted[p] = n;
  for (int64_t p = p0; p < p1; p += pstep) sorted[p] = n;
}

// ---- n <= kSmallN: one workgroup of 16 waves ------------------------------
__global__ __launch_bounds__(kSmallThreads) void align_small_kernel(
    const int32_t* __restrict__ ids, int n, int E, int nbits, int BM,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ sorted,
    int64_t sorted_cap, int32_t* __restrict__ block_ids, int64_t block_cap,
    int32_t* __restrict__ ntp) {
  constexpr int NW = kSmallThreads / 64;
  __shared__ int hist[NW * kMaxE];   // per wave: counts, then cursors
  __shared__ int cnt[kMaxE + 1];
  __shared__ int tot[kMaxE];
  __shared__ int partial[NW + 1];
  const int tid = threadIdx.x, wave = tid >> 6;
  for (int x = tid; x < NW * E; x += kSmallThreads) hist[x] = 0;
  __syncthreads();
  const int per = (n + NW - 1) / NW;
  const int lo = min(wave * per, n), hi = min(lo + per, n);
  wave_count(ids, lo, hi, E, nbits, hist + wave * E);
  __syncthreads();
  // per expert: exclusive prefix over the waves (in place), total
  for (int e = tid; e < E; e += kSmallThreads) {
    int run = 0;
    for (int w = 0; w < NW; ++w) { const int x = hist[w * E + e]; hist[w * E + e] = run; run += x; }
    cnt[e] = run;
  }
  __syncthreads();
  const int total = finish_offsets<kSmallThreads>(cnt, E, BM, partial, counts, offsets, ntp, tot);
  if (tid == 0) cnt[E] = total;
  __syncthreads();
  fill_block_owners<kSmallThreads>(cnt, E, BM, total, 0, block_cap, block_ids);
  fill_sentinels(cnt, tot, E, n, wave, NW, total + tid, sorted_cap, kSmallThreads, sorted);
  for (int x = tid; x < NW * E; x += kSmallThreads) hist[x] += cnt[x % E];
  __syncthreads();
  wave_scatter(ids, lo, hi, E, nbits, hist + wave * E, sorted);
}

// ---- multi-tile path ------------------------------------------------------
// Workgroup b runs on XCD b % 8; give each XCD a contiguous range of tiles
// so that neighbouring tiles (whose runs of one expert meet inside a line)
// share that XCD's L2.
__device__ __forceinline__ int xcd_tile(int b, int ntiles) {
  const int q = ntiles >> 3, r = ntiles & 7, x = b & 7;
  return x * q + min(x, r) + (b >> 3);
}

// Each of the 8 waves of a tile's workgroup owns an eighth of the tile.
__device__ __forceinline__ void tile_wave_range(int tile, int tile_ids, int n, int& lo, int& hi) {
  const int wave = threadIdx.x >> 6;
  const int t0 = tile * tile_ids;
  const int t1 = min(t0 + tile_ids, n);
  const int per = tile_ids / kTileWaves;
  lo = min(t0 + wave * per, t1);
  hi = min(lo + per, t1);
}

// Per tile: the counts of every wave's sub-range, sub[tile][wave][e], and the
// tile's totals in expert-major order, tcol[e][tile] (one column per expert
// for the scan).
__global__ __launch_bounds__(kTileThreads) void align_count_kernel(
    const int32_t* __restrict__ ids, int n, int E, int nbits, int tile_ids, int ntiles,
    int32_t* __restrict__ sub, int32_t* __restrict__ tcol) {
  constexpr int NW = kTileWaves;
  __shared__ int hist[NW * kMaxE];
  const int tid = threadIdx.x, wave = tid >> 6;
  for (int x = tid; x < NW * E; x += kTileThreads) hist[x] = 0;
  __syncthreads();
  int lo, hi;
  const int tile = xcd_tile(blockIdx.x, ntiles);
  tile_wave_range(tile, tile_ids, n, lo, hi);
  wave_count(ids, lo, hi, E, nbits, hist + wave * E);
  __syncthreads();
  int32_t* out = sub + static_cast<int64_t>(tile) * NW * E;
  for (int x = tid; x < NW * E; x += kTileThreads) out[x] = hist[x];
  for (int e = tid; e < E; e += kTileThreads) {
    int t = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) t += hist[w * E + e];
    tcol[static_cast<int64_t>(e) * ntiles + tile] = t;
  }
}

// One workgroup per expert: exclusive prefix of its column of tile totals
// (in place) and the expert's total.
__global__ __launch_bounds__(kScanThreads) void align_colscan_kernel(
    int32_t* __restrict__ tcol, int ntiles, int32_t* __restrict__ tot) {
  constexpr int NW = kScanThreads / 64, PER = 8;
  __shared__ int partial[NW + 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int32_t* col = tcol + static_cast<int64_t>(blockIdx.x) * ntiles;
  int run = 0;
  for (int base = 0; base < ntiles; base += kScanThreads * PER) {
    const int lo = base + tid * PER;
    int x[PER];
    int local = 0;
#pragma unroll
    for (int v = 0; v < PER; ++v) {
      x[v] = lo + v < ntiles ? col[lo + v] : 0;
      local += x[v];
    }
    int incl = local;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int up = __shfl_up(incl, o, 64);
      if (lane >= o) incl += up;
    }
    if (lane == 63) partial[wave] = incl;
    __syncthreads();
    if (tid == 0) {
      int r = 0;
      for (int w = 0; w < NW; ++w) { const int y = partial[w]; partial[w] = r; r += y; }
      partial[NW] = r;
    }
    __syncthreads();
    int r = run + partial[wave] + incl - local;
#pragma unroll
    for (int v = 0; v < PER; ++v) {
      if (lo + v < ntiles) col[lo + v] = r;
      r += x[v];
    }
    run += partial[NW];
    __syncthreads();
  }
  if (tid == 0) tot[blockIdx.x] = run;
}

// Per tile: padded offsets from the expert totals; the tile's slots are
// sorted in LDS first (each wave walks its sub-range in index order with
// cursors starting at the tile-local prefix of its expert and its earlier
// waves), then each expert's run is copied out to its global slots with
// consecutive lanes on consecutive slots.  The workgroups also share the
// block-owner and pad-sentinel fills; workgroup 0 writes counts, offsets and
// the padded total.  MAXE bounds E (LDS sizing).
template <int MAXE>
__global__ __launch_bounds__(kTileThreads) void align_scatter_kernel(
    const int32_t* __restrict__ ids, int n, int E, int nbits, int BM, int tile_ids, int ntiles,
    const int32_t* __restrict__ sub, const int32_t* __restrict__ tcol,
    const int32_t* __restrict__ tot, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ ntp, int32_t* __restrict__ block_ids,
    int64_t block_cap, int32_t* __restrict__ sorted, int64_t sorted_cap) {
  constexpr int NW = kTileWaves;
  __shared__ int stage[kMaxTile];   // the tile's flat indices in slot order
  __shared__ int cur[NW * MAXE];    // per-wave cursors into stage
  __shared__ int off[MAXE + 1];     // padded offsets
  __shared__ int tt[MAXE];          // expert totals
  __shared__ int lb[MAXE + 1];      // tile-local counts, then their exclusive prefix
  __shared__ int gb[MAXE];          // global slot of the tile's first id of each expert
  __shared__ int partial[NW + 1];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  int lo, hi;
  const int tile = xcd_tile(blockIdx.x, ntiles);
  tile_wave_range(tile, tile_ids, n, lo, hi);
  // the wave's whole sub-range, loaded before the prologue so that the
  // loads overlap it
  constexpr int KPL = kMaxTile / kTileThreads;
  int key[KPL];
#pragma unroll
  for (int s = 0; s < KPL; ++s) {
    const int i = lo + 64 * s + lane;
    key[s] = i < hi ? ids[i] : -1;
  }
  const int32_t* sp = sub + static_cast<int64_t>(tile) * NW * E;
  for (int e = tid; e < E; e += kTileThreads) {
    const int t = tot[e];
    tt[e] = t;
    off[e] = (t + BM - 1) / BM * BM;
    int run = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) { const int x = sp[w * E + e]; cur[w * E + e] = run; run += x; }
    lb[e] = run;
  }
  __syncthreads();
  const int total = block_exclusive_scan<kTileThreads>(off, E, partial);
  const int tile_total = block_exclusive_scan<kTileThreads>(lb, E, partial);
  if (tid == 0) { off[E] = total; lb[E] = tile_total; }
  for (int e = tid; e < E; e += kTileThreads)
    gb[e] = off[e] + tcol[static_cast<int64_t>(e) * ntiles + tile];
  if (blockIdx.x == 0) {
    for (int e = tid; e < E; e += kTileThreads) { counts[e] = tt[e]; offsets[e] = off[e]; }
    if (tid == 0) { offsets[E] = total; ntp[0] = total; }
  }
  for (int x = tid; x < NW * E; x += kTileThreads) cur[x] += lb[x % E];
  __syncthreads();
  scatter_keys(key, lo, E, nbits, cur + wave * E, stage);
  __syncthreads();
  for (int e = wave; e < E; e += NW) {
    const int s0 = lb[e], c = lb[e + 1] - s0;
    int32_t* dst = sorted + gb[e];
    for (int j = lane; j < c; j += 64) dst[j] = stage[s0 + j];
  }
  const int64_t per = (block_cap + gridDim.x - 1) / gridDim.x;
  const int64_t b0 = min<int64_t>(static_cast<int64_t>(blockIdx.x) * per, block_cap);
  fill_block_owners<kTileThreads>(off, E, BM, total, b0, min(b0 + per, block_cap), block_ids);
  const int64_t tail = sorted_cap - total;
  const int64_t tper = (tail + gridDim.x - 1) / gridDim.x;
  const int64_t p0 = total + min<int64_t>(static_cast<int64_t>(blockIdx.x) * tper, tail);
  const int64_t p1 = min<int64_t>(p0 + tper, sorted_cap);
  fill_sentinels(off, tt, E, n, blockIdx.x * NW + wave, gridDim.x * NW, p0 + tid, p1,
                 kTileThreads, sorted);
}

// ---- resident path: one launch, every id read once ------------------------
constexpr int kResThreads = 1024;
constexpr int kResWaves = kResThreads / 64;
constexpr int kResMaxRows = 16;                          // 256-id rows per wave
constexpr int kResMaxSlots = 4 * kResMaxRows;            // ids per lane
constexpr int kResMaxTile = kResThreads * kResMaxSlots;  // 65536: 16-bit local index
constexpr int kResMaxE = 256;
constexpr int kResMaxGrid = 256;
constexpr uint32_t kNoRank = 0xFFFF;
// LDS bytes.  The 16-bit stage holds the tile in slot order from placement
// on; before that it holds each wave's lane masks (E entries of 8 B) and its
// 1 KB transpose buffer.
constexpr int kStageBytes = kResMaxTile * 2 + 16;   // + a spare entry
constexpr int kTableBytes = kResMaxE * 8;
constexpr int kXposeOff = kResWaves * kTableBytes;
constexpr int kCurOff = kStageBytes;                     // int [wave][kResMaxE]
constexpr int kArrOff = kCurOff + kResWaves * kResMaxE * 4;
constexpr int kChunks = kResMaxTile / 64;
constexpr int kResLdsBytes = kArrOff + 5 * (kResMaxE + 1) * 4 + kChunks * 2 + (kResWaves + 2) * 4;
static_assert(kXposeOff + kResWaves * 1024 <= kStageBytes, "tables exceed the stage");
static_assert(kResLdsBytes <= 160 * 1024, "resident tile exceeds the LDS");

// Exclusive prefix over the wave's lanes (lane 0 gets 0) of four 8-bit
// fields packed in x, by DPP steps: a shift of the whole wave by one lane,
// then an inclusive scan (rows of 16, then the row broadcasts).  No field's
// sum over lanes 0..62 may reach 256 (nothing carries between fields).
__device__ __forceinline__ uint32_t wave_excl_scan_u8x4(uint32_t x) {
  constexpr int kWaveShr1 = 0x138, kRowShr = 0x110, kRowBcast15 = 0x142, kRowBcast31 = 0x143;
  int v = __builtin_amdgcn_update_dpp(0, static_cast<int>(x), kWaveShr1, 0xF, 0xF, true);
  v += __builtin_amdgcn_update_dpp(0, v, kRowShr + 1, 0xF, 0xF, true);
  v += __builtin_amdgcn_update_dpp(0, v, kRowShr + 2, 0xF, 0xF, true);
  v += __builtin_amdgcn_update_dpp(0, v, kRowShr + 4, 0xF, 0xF, true);
  v += __builtin_amdgcn_update_dpp(0, v, kRowShr + 8, 0xF, 0xF, true);
  v += __builtin_amdgcn_update_dpp(0, v, kRowBcast15, 0xA, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, kRowBcast31, 0xC, 0xF, false);
  return static_cast<uint32_t>(v);
}

// One wave's share of the ranking: its 256*ROWS ids (wids[0..), m of them
// valid when !FULL, m <= 0 allowed), read as rows of 256 with 16 B a lane,
// RING rows in flight.  Row r of the wave holds ids 256r + 4l + q in lane l
// (lane-major); in index order, id 256r + 4l + q precedes every id of a
// later lane.  Results: the expert of slot (r, q) in byte q of kv[r], its
// rank in 16-bit half (q & 1) of rv[2r + q/2] (kNoRank: out of range).
//
// ONEHOT (E <= 8): the rank is within the row (counts of the lane's own
// four ids in 8-bit fields, scanned over the lanes); rowoff[r*8 + k] gets
// the wave's count of expert k before row r, and cnt[k] the wave's counts
// (lanes k < E).  No LDS in the ranking itself.
//
// Table (E <= 256): the rank is within the wave, by the lane masks msk and
// the cursors cnt (E entries each, zero on entry; the cursors end as the
// wave's counts).  A row whose lanes each hold four distinct experts
// ranks in one pass: every lane ORs its bit into the entries of its four
// experts, reads them back, and the leader of each expert (its lowest lane)
// advances the cursor.  Any other row goes through the wave's transpose
// buffer xb so that lane l ranks ids 64j + l (j = 0..3) one slot at a
// time; bit r of the returned mask marks such a row (its slot (r, j) then
// holds id 256r + 64j + l).
template <bool ONEHOT, int ROWS, bool FULL>
__device__ __forceinline__ uint32_t rank_rows(const int32_t* __restrict__ wids, int m, int E,
                                              uint64_t* msk, int* xb, int* rowoff, int* cnt,
                                              uint32_t (&kv)[ROWS], uint32_t (&rv)[2 * ROWS]) {
  constexpr int RING = ROWS < 8 ? ROWS : 8;
  const int lane = threadIdx.x & 63;
  auto load = [&](int r) {
    const int i = 256 * r + 4 * lane;
    if constexpr (FULL) {
      return *reinterpret_cast<const int4*>(wids + i);
    } else {
      int4 x;
      x.x = i < m ? wids[i] : -1;
      x.y = i + 1 < m ? wids[i + 1] : -1;
      x.z = i + 2 < m ? wids[i + 2] : -1;
      x.w = i + 3 < m ? wids[i + 3] : -1;
      return x;
    }
  };
  int4 raw[RING];
#pragma unroll
  for (int r = 0; r < RING; ++r) raw[r] = load(r);
  const uint64_t bit = 1ull << lane;
  uint32_t transposed = 0;
  int mycur = 0;   // ONEHOT: lane k < 8 keeps the wave's count of expert k
#pragma unroll
  for (int r = 0; r < ROWS; ++r) {
    const int4 x = raw[r % RING];
    if (r + RING < ROWS) raw[r % RING] = load(r + RING);
    const int k[4] = {x.x, x.y, x.z, x.w};
    bool valid[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) valid[q] = static_cast<unsigned>(k[q]) < static_cast<unsigned>(E);
    kv[r] = 0;
    rv[2 * r] = 0;
    rv[2 * r + 1] = 0;
    if constexpr (ONEHOT) {
      // keys 0-3 count in lo, 4-7 in hi, one byte each
      uint32_t lo = 0, hi = 0, plo[4], phi[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        plo[q] = lo;
        phi[q] = hi;
        const uint32_t one = valid[q] ? 1u << (8 * (k[q] & 3)) : 0u;
        lo += (k[q] & 4) ? 0u : one;
        hi += (k[q] & 4) ? one : 0u;
      }
      const uint32_t elo = wave_excl_scan_u8x4(lo), ehi = wave_excl_scan_u8x4(hi);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t b = (k[q] & 4) ? ehi + phi[q] : elo + plo[q];
        const uint32_t rank = (b >> (8 * (k[q] & 3))) & 0xFF;
        kv[r] |= static_cast<uint32_t>(valid[q] ? k[q] : 0) << (8 * q);
        rv[2 * r + (q >> 1)] |= (valid[q] ? rank : kNoRank) << (16 * (q & 1));
      }
      // the row's counts: lane 63's exclusive prefix plus its own four
      const uint32_t e63 = (lane & 4) ? __builtin_amdgcn_readlane(static_cast<int>(ehi), 63)
                                      : __builtin_amdgcn_readlane(static_cast<int>(elo), 63);
      const uint32_t o63 = (lane & 4) ? __builtin_amdgcn_readlane(static_cast<int>(hi), 63)
                                      : __builtin_amdgcn_readlane(static_cast<int>(lo), 63);
      if (lane < 8) rowoff[r * 8 + lane] = mycur;
      mycur += static_cast<int>(((e63 >> (8 * (lane & 3))) & 0xFF) + ((o63 >> (8 * (lane & 3))) & 0xFF));
    } else {
      const bool dup = (k[0] == k[1]) | (k[0] == k[2]) | (k[0] == k[3]) | (k[1] == k[2]) |
                       (k[1] == k[3]) | (k[2] == k[3]);
      if (__ballot(dup) == 0) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (valid[q])
            __hip_atomic_fetch_or(msk + k[q], bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        uint64_t mk[4];
        int base[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          mk[q] = valid[q] ? msk[k[q]] : 0ull;
          base[q] = valid[q] ? cnt[k[q]] : 0;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int below = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mk[q] >> 32),
                                                     __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mk[q]), 0));
          kv[r] |= static_cast<uint32_t>(valid[q] ? k[q] : 0) << (8 * q);
          rv[2 * r + (q >> 1)] |=
              static_cast<uint32_t>(valid[q] ? base[q] + below : kNoRank) << (16 * (q & 1));
          if (valid[q] && below == 0) {
            msk[k[q]] = 0ull;
            cnt[k[q]] = base[q] + __builtin_popcountll(mk[q]);
          }
        }
      } else {
        transposed |= 1u << r;
        *reinterpret_cast<int4*>(xb + 4 * lane) = x;
        int keys[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) keys[j] = xb[64 * j + lane];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int key = keys[j];
          const bool ok = static_cast<unsigned>(key) < static_cast<unsigned>(E);
          if (ok) __hip_atomic_fetch_or(msk + key, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
          const uint64_t mk = ok ? msk[key] : 0ull;
          const int b = ok ? cnt[key] : 0;
          const int below = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mk >> 32),
                                                     __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mk), 0));
          kv[r] |= static_cast<uint32_t>(ok ? key : 0) << (8 * j);
          rv[2 * r + (j >> 1)] |= static_cast<uint32_t>(ok ? b + below : kNoRank) << (16 * (j & 1));
          if (ok && below == 0) {
            msk[key] = 0ull;
            cnt[key] = b + __builtin_popcountll(mk);
          }
        }
      }
    }
    // materialise the row's packed results here: otherwise the compiler
    // sinks their arithmetic into the placement loop and keeps every slot's
    // operands alive until then
    asm volatile("" : "+v"(kv[r]), "+v"(rv[2 * r]), "+v"(rv[2 * r + 1]));
  }
  if constexpr (ONEHOT) {
    if (lane < E) cnt[lane] = mycur;
  }
  return transposed;
}

// Workgroup g owns the ids [g*tile, (g+1)*tile), tile = 4096*rows: wave w
// owns 256*rows consecutive ids and reads them as rows of 256 (16 B a lane),
// each row transposed through LDS so that lane l ranks ids 64j + l of it
// (j = 0..3) in index order.  ws: the 64-bit arrival flags [kResMaxGrid],
// the 64-bit go word, then the tiles' expert counts [G][E].  A flag or go
// word counts only when it equals this call's epoch, so nothing has to be
// cleared before the launch.  The grid must be resident at once: at most one
// 1024-thread workgroup fits a CU (the LDS), and the grid is no larger than
// the CUs the stream may use; the waits are bounded all the same.
template <bool ONEHOT, int ROWS>
__global__ __launch_bounds__(kResThreads) void align_resident_kernel(
    const int32_t* __restrict__ ids, int n, int E, int nbits, int BM, uint64_t epoch,
    uint64_t* flags, int32_t* cnt, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* ntp, int32_t* __restrict__ block_ids, int64_t block_cap,
    int32_t* __restrict__ sorted, int64_t sorted_cap) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kResLdsBytes];
  uint16_t* stage = reinterpret_cast<uint16_t*>(lds);
  int* cur = reinterpret_cast<int*>(lds + kCurOff);
  int* lb = reinterpret_cast<int*>(lds + kArrOff);   // tile counts -> exclusive prefix [E+1]
  int* off = lb + kResMaxE + 1;                      // padded offsets [E+1]
  int* tt = off + kResMaxE + 1;                      // expert totals
  int* gpre = tt + kResMaxE + 1;                     // earlier tiles' counts
  int* dl = gpre + kResMaxE + 1;                     // global slot - tile slot, per expert
  uint16_t* ce = reinterpret_cast<uint16_t*>(dl + kResMaxE + 1);   // expert of slot 64c
  int* partial = reinterpret_cast<int*>(ce + kChunks);
  int* okf = partial + kResWaves + 1;
  // the wave index as a scalar: the wave's pointers stay in scalar registers
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // tile g: the tiles are dealt to the XCDs in contiguous ranges, so that
  // the line where one tile's run of an expert meets the next tile's is
  // written in one L2
  const int G = gridDim.x, g = xcd_tile(blockIdx.x, G);
  constexpr int tile = kResThreads * 4 * ROWS;
  const int t0 = g * tile;
  const int lbase = wave * 256 * ROWS;   // the wave's first id, local to the tile
  uint64_t* go = flags + kResMaxGrid;

  uint64_t* msk = reinterpret_cast<uint64_t*>(lds + wave * kTableBytes);   // lane masks
  int* xb = reinterpret_cast<int*>(lds + kXposeOff + wave * 1024);
  int* cw = cur + wave * kResMaxE;    // the wave's cursors/counts, then its slot bases
  int* rowoff = cw + 8;               // ONEHOT: [row][8] counts before each row
  if (!ONEHOT)
    for (int x = lane; x < kResMaxE; x += 64) { msk[x] = 0ull; cw[x] = 0; }
  uint32_t kv[ROWS], rv[2 * ROWS];
  const int* wids = ids + t0 + lbase;
  const uint32_t transposed =
      t0 + tile <= n
          ? rank_rows<ONEHOT, ROWS, true>(wids, n - t0 - lbase, E, msk, xb, rowoff, cw, kv, rv)
          : rank_rows<ONEHOT, ROWS, false>(wids, n - t0 - lbase, E, msk, xb, rowoff, cw, kv, rv);
  __syncthreads();
  // ---- the tile's counts: published, then turned into slot bases ---------
  int32_t* row = cnt + static_cast<int64_t>(g) * E;
  for (int e = tid; e < E; e += kResThreads) {
    int run = 0;
#pragma unroll
    for (int w = 0; w < kResWaves; ++w) {
      const int x = cur[w * kResMaxE + e];
      cur[w * kResMaxE + e] = run;
      run += x;
    }
    lb[e] = run;
    row[e] = run;
  }
  __syncthreads();
  const int tile_total = block_exclusive_scan<kResThreads>(lb, E, partial);
  if (tid == 0) lb[E] = tile_total;
  grid_arrive(flags, epoch, g);
  for (int e = tid; e < E; e += kResThreads)
    for (int w = 0; w < kResWaves; ++w) cur[w * kResMaxE + e] += lb[e];
  __syncthreads();
  if (ONEHOT) {   // fold the slot bases into the per-row offsets
    for (int x = tid; x < kResWaves * ROWS * 8; x += kResThreads) {
      const int w = x / (ROWS * 8), rk = x % (ROWS * 8);
      if ((rk & 7) < E) cur[w * kResMaxE + 8 + rk] += cur[w * kResMaxE + (rk & 7)];
    }
    __syncthreads();
  }
  // (slot (r, q): local id 256r + 4*lane + q of the wave, or 256r + 64q +
  // lane in a transposed row; an id out of range writes the spare entry
  // past the stage, so the loop has no branch)
#pragma unroll
  for (int r = 0; r < ROWS; ++r) {
    int at[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int key = (kv[r] >> (8 * q)) & 0xFF;
      at[q] = ONEHOT ? rowoff[r * 8 + key] : cw[key];
    }
    const bool tr = (transposed >> r) & 1;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t rank = (rv[2 * r + (q >> 1)] >> (16 * (q & 1))) & 0xFFFF;
      stage[rank != kNoRank ? at[q] + static_cast<int>(rank) : kResMaxTile] =
          static_cast<uint16_t>(lbase + 256 * r + (tr ? 64 * q + lane : 4 * lane + q));
    }
  }
  // ---- barrier: every tile's counts are published ------------------------
  if (!grid_await(flags, go, epoch, g, G, okf)) {
    if (tid == 0) __hip_atomic_store(ntp, -1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  // ---- expert totals tt and the earlier tiles' counts gpre, from the rows --
  for (int e = tid; e < E; e += kResThreads) { tt[e] = 0; gpre[e] = 0; }
  __syncthreads();
  {
    const int S = kResThreads / E;   // slices of the rows, one thread per (slice, expert)
    if (tid < S * E) {
      const int e = tid % E, sl = tid / E;
      const int per = (G + S - 1) / S;
      const int r0 = min(sl * per, G), r1 = min(r0 + per, G);
      int all = 0, pre = 0;
      for (int r = r0; r < r1; r += 8) {   // 8 loads in flight
        int x[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) x[u] = r + u < r1 ? cnt[static_cast<int64_t>(r + u) * E + e] : 0;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          all += x[u];
          pre += r + u < g ? x[u] : 0;
        }
      }
      atomicAdd(&tt[e], all);
      atomicAdd(&gpre[e], pre);
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += kResThreads) off[e] = (tt[e] + BM - 1) / BM * BM;
  __syncthreads();
  const int total = block_exclusive_scan<kResThreads>(off, E, partial);
  if (tid == 0) off[E] = total;
  for (int e = tid; e < E; e += kResThreads) dl[e] = off[e] + gpre[e] - lb[e];
  if (g == 0) {
    for (int e = tid; e < E; e += kResThreads) { counts[e] = tt[e]; offsets[e] = off[e]; }
    if (tid == 0) { offsets[E] = total; ntp[0] = total; }
  }
  // the expert owning slot 64c: the last e with lb[e] <= 64c
  const int nch = (tile_total + 63) >> 6;
  for (int c = tid; c < nch; c += kResThreads) {
    const int p = c << 6;
    int lo = 0, hi = E - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (lb[mid] <= p) lo = mid;
      else hi = mid - 1;
    }
    ce[c] = static_cast<uint16_t>(lo);
  }
  __syncthreads();
  // ---- copy-out: consecutive lanes on consecutive slots ------------------
  for (int c = wave; c < nch; c += kResWaves) {
    const int p = (c << 6) + lane;
    if (p < tile_total) {
      int e = ce[c];
      while (lb[e + 1] <= p) ++e;
      sorted[dl[e] + p] = t0 + stage[p];
    }
  }
  const int64_t per = (block_cap + G - 1) / G;
  const int64_t b0 = min<int64_t>(static_cast<int64_t>(g) * per, block_cap);
  fill_block_owners<kResThreads>(off, E, BM, total, b0, min(b0 + per, block_cap), block_ids);
  const int64_t tail = sorted_cap - total;
  const int64_t tper = (tail + G - 1) / G;
  const int64_t p0 = total + min<int64_t>(static_cast<int64_t>(g) * tper, tail);
  const int64_t p1 = min<int64_t>(p0 + tper, sorted_cap);
  fill_sentinels(off, tt, E, n, g * kResWaves + wave, G * kResWaves, p0 + tid, p1, kResThreads,
                 sorted);
}

// ---- decode prologue: routing and align in one wave (T <= 8, T*top_k <= 64)
// Decode-sized batches spend more time launching the routing and align
// kernels than computing them; this one wave does both.  It routes its
// tokens in batches of TB with their cross-lane steps interleaved, but a
// wave still spends about a microsecond per token on them, so past 8
// tokens the two launches (one wave per token) are faster.  Lane l of the wave
// then holds flat row l's expert: one peer mask per lane gives the counts
// (its leader's popcount) and the stable slots (peers below); the padded
// offsets are a wave scan over the experts; pad slots and the tail get the
// sentinel from loops over the touched experts (at most 64) and the tail.
// The wave's LDS operations complete in issue order, so no barrier is
// needed between its LDS writes and reads.
constexpr int kPrologueMaxIds = 64;
constexpr int kPrologueMaxE = 1024;
constexpr int kPrologueMaxTokens = 8;

template <int VPL, int TB>
__global__ __launch_bounds__(64) void decode_prologue_kernel(
    const float* __restrict__ logits, int T, int E, int top_k, int scoring, int renorm,
    int32_t* __restrict__ ids, float* __restrict__ weights, int nbits, int BM,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ sorted,
    int64_t sorted_cap, int32_t* __restrict__ block_ids, int64_t block_cap,
    int32_t* __restrict__ ntp) {
  __shared__ int flat[kPrologueMaxIds];
  __shared__ int cnt[kPrologueMaxE];
  __shared__ int off[kPrologueMaxE + 1];
  const int lane = threadIdx.x;
  const int n = T * top_k;
  // the tokens' logits in batches of TB (one round trip per batch), then the
  // batch's top-k with the tokens' cross-lane steps interleaved (padding
  // tokens of the last batch hold -inf and are not stored)
  for (int t0 = 0; t0 < T; t0 += TB) {
    float v[TB][VPL];
#pragma unroll
    for (int b = 0; b < TB; ++b) {
      if (t0 + b < T) {
        load_logits<VPL>(logits + static_cast<size_t>(t0 + b) * E, E, v[b]);
      } else {
#pragma unroll
        for (int i = 0; i < VPL; ++i) v[b][i] = -__builtin_inff();
      }
    }
    int e[TB];
    float w[TB];
    route_logits<VPL, TB>(v, E, top_k, scoring, renorm, e, w);
#pragma unroll
    for (int b = 0; b < TB; ++b) {
      const int t = t0 + b;
      if (t < T && lane < top_k) {
        ids[t * top_k + lane] = e[b];
        weights[t * top_k + lane] = w[b];
        flat[t * top_k + lane] = e[b];
      }
    }
  }
  for (int e = lane; e < E; e += 64) cnt[e] = 0;
  const int key = lane < n ? flat[lane] : -1;
  const bool valid = static_cast<unsigned>(key) < static_cast<unsigned>(E);
  const uint64_t m = peer_mask(key, valid, nbits);
  const uint64_t below = lanemask_lt();
  const bool leader = valid && (m & below) == 0;
  if (leader) cnt[key] = __builtin_popcountll(m);
  // padded offsets: lane l scans experts [l*per, (l+1)*per)
  const int per = (E + 63) / 64;
  const int e0 = min(lane * per, E), e1 = min(e0 + per, E);
  int local = 0;
  for (int e = e0; e < e1; ++e) local += (cnt[e] + BM - 1) / BM * BM;
  int incl = local;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int up = __shfl_up(incl, o, 64);
    if (lane >= o) incl += up;
  }
  int run = incl - local;
  for (int e = e0; e < e1; ++e) {
    const int c = cnt[e];
    off[e] = run;
    counts[e] = c;
    offsets[e] = run;
    run += (c + BM - 1) / BM * BM;
  }
  const int total = __shfl(incl, 63, 64);
  if (lane == 0) {
    off[E] = total;
    offsets[E] = total;
    ntp[0] = total;
  }
  // stable slots: the peers below, after the expert's offset
  if (valid) sorted[off[key] + __builtin_popcountll(m & below)] = lane;
  // the sentinel in each touched expert's pad slots, one expert at a time
  uint64_t lead = __ballot(leader);
  while (lead) {
    const int src = __builtin_ctzll(lead);
    lead &= lead - 1;
    const int e = __shfl(key, src, 64);
    const int c = __shfl(cnt[key > 0 ? key : 0], src, 64);
    for (int p = off[e] + c + lane; p < off[e + 1]; p += 64) sorted[p] = n;
  }
  for (int64_t p = total + lane; p < sorted_cap; p += 64) sorted[p] = n;
  for (int64_t b = lane; b < block_cap; b += 64) {
    int owner = -1;
    if (b * BM < total) {
      const int row = static_cast<int>(b) * BM;
      int lo = 0, hi = E - 1;   // the last expert whose offset is <= row
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (off[mid] <= row) lo = mid;
        else hi = mid - 1;
      }
      owner = lo;
    }
    block_ids[b] = owner;
  }
}

struct AlignPlan {
  int tile_ids, ntiles;
};

// Tiles of 2048..8192 ids (a power of two): the smallest that gives at most
// about 1024 tiles, capped at the 8192 slots (32 KB) that the scatter sorts
// in LDS (so that several scatter workgroups share a CU).
AlignPlan plan(int64_t n, int E) {
  (void)E;
  AlignPlan p{0, 0};
  if (n <= kSmallN) return p;
  int t = 2048;
  while (t < kMaxTile && static_cast<int64_t>(t) * 1024 < n) t *= 2;
  p.tile_ids = t;
  p.ntiles = static_cast<int>((n + t - 1) / t);
  return p;
}

// Resident path: at most one workgroup per CU (the LDS) and one per CU the
// stream may use; 0 if the kernel does not fit a CU at all.
int resident_grid_capacity(hipStream_t s) {
  static std::atomic<int> occ[64];   // per device: 0 unknown, -1 none, else 1
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int o = occ[dev].load(std::memory_order_relaxed);
  if (o == 0) {
    int nb_t = 0, nb_b = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb_t, align_resident_kernel<true, 16>,
                                                     kResThreads, 0) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb_b, align_resident_kernel<false, 16>,
                                                     kResThreads, 0) != hipSuccess)
      (void)hipGetLastError();
    o = (nb_t >= 1 && nb_b >= 1) ? 1 : -1;
    occ[dev].store(o, std::memory_order_relaxed);
  }
  if (o < 0) return 0;
  uint32_t mask[32] = {};
  if (hipExtStreamGetCUMask(s, 32, mask) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  int cus = 0;
  for (uint32_t m : mask) cus += __builtin_popcount(m);
  return std::min(cus, kResMaxGrid);
}

// A bound on the resident grid for n ids: a tile holds at least 4096 ids.
int64_t resident_grid_bound(int64_t n) {
  return std::min<int64_t>(kResMaxGrid, (n + kResThreads * 4 - 1) / (kResThreads * 4));
}

// the arrival flags and the go word; the count rows [G][E]
size_t resident_workspace_bytes(int64_t n, int E) {
  return (kResMaxGrid + 1) * sizeof(uint64_t) +
         static_cast<size_t>(resident_grid_bound(n)) * E * sizeof(int32_t);
}

// Launches the resident path if it applies; false if the caller must take
// the tiled path (nothing was enqueued).
bool launch_resident(const int32_t* ids, int n, int E, int nbits, int BM, int32_t* counts,
                     int32_t* offsets, int32_t* sorted, int64_t sorted_cap, int32_t* block_ids,
                     int64_t block_cap, int32_t* ntp, void* ws, hipStream_t s) {
  if (n <= kSmallN || E > kResMaxE || (reinterpret_cast<uintptr_t>(ids) & 15)) return false;
  const char* env = std::getenv("MOE_ALIGN_RESIDENT");
  if (env && env[0] == '0') return false;
  // a captured graph would replay this call's epoch
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cs) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  if (cs != hipStreamCaptureStatusNone) return false;
  const int cap = resident_grid_capacity(s);
  if (cap <= 0 || static_cast<int64_t>(n) > static_cast<int64_t>(cap) * kResMaxTile) return false;
  // rows of 256 ids per wave: the smallest power of two that fits n on the grid
  const int64_t per_row = static_cast<int64_t>(cap) * kResWaves * 256;
  int rows = 1;
  while (static_cast<int64_t>(rows) * per_row < n) rows *= 2;
  const int tile = kResThreads * 4 * rows;
  const int grid = (n + tile - 1) / tile;
  uint64_t* flags = static_cast<uint64_t*>(ws);
  int32_t* cnt = reinterpret_cast<int32_t*>(flags + kResMaxGrid + 1);
  const uint64_t epoch = next_epoch();
  auto go = [&](auto table, auto rows_c) {
    align_resident_kernel<decltype(table)::value, decltype(rows_c)::value>
        <<<grid, kResThreads, 0, s>>>(ids, n, E, nbits, BM, epoch, flags, cnt, counts, offsets,
                                      ntp, block_ids, block_cap, sorted, sorted_cap);
  };
  auto pick = [&](auto table) {
    switch (rows) {
      case 1: go(table, std::integral_constant<int, 1>{}); break;
      case 2: go(table, std::integral_constant<int, 2>{}); break;
      case 4: go(table, std::integral_constant<int, 4>{}); break;
      case 8: go(table, std::integral_constant<int, 8>{}); break;
      default: go(table, std::integral_constant<int, 16>{}); break;
    }
  };
  if (E <= 8) pick(std::true_type{});    // one-hot counts
  else pick(std::false_type{});
  return true;
}

}  // namespace

size_t align_workspace_bytes(int64_t n, int E) {
  const AlignPlan p = plan(n, E);
  if (p.ntiles == 0) return 0;
  const size_t tiled = (static_cast<size_t>(p.ntiles) * (kTileWaves + 1) + 1) * E * sizeof(int32_t);
  return std::max(tiled, resident_workspace_bytes(n, E));
}

void launch_align(const int32_t* ids, int64_t n, int E, int BM, int32_t* counts,
                  int32_t* offsets, int32_t* sorted, int64_t sorted_cap, int32_t* block_ids,
                  int64_t block_cap, int32_t* ntp, void* ws, hipStream_t s) {
  const int nbits = ceil_log2(E);
  const int nn = static_cast<int>(n);
  const AlignPlan p = plan(n, E);
  if (p.ntiles == 0) {
    align_small_kernel<<<1, kSmallThreads, 0, s>>>(ids, nn, E, nbits, BM, counts, offsets, sorted,
                                                   sorted_cap, block_ids, block_cap, ntp);
    return;
  }
  if (launch_resident(ids, nn, E, nbits, BM, counts, offsets, sorted, sorted_cap, block_ids,
                      block_cap, ntp, ws, s))
    return;
  int32_t* sub = static_cast<int32_t*>(ws);
  int32_t* tcol = sub + static_cast<int64_t>(p.ntiles) * kTileWaves * E;
  int32_t* tot = tcol + static_cast<int64_t>(p.ntiles) * E;
  align_count_kernel<<<p.ntiles, kTileThreads, 0, s>>>(ids, nn, E, nbits, p.tile_ids, p.ntiles,
                                                       sub, tcol);
  align_colscan_kernel<<<E, kScanThreads, 0, s>>>(tcol, p.ntiles, tot);
  if (E <= kMidE)
    align_scatter_kernel<kMidE><<<p.ntiles, kTileThreads, 0, s>>>(
        ids, nn, E, nbits, BM, p.tile_ids, p.ntiles, sub, tcol, tot, counts, offsets, ntp,
        block_ids, block_cap, sorted, sorted_cap);
  else
    align_scatter_kernel<kMaxE><<<p.ntiles, kTileThreads, 0, s>>>(
        ids, nn, E, nbits, BM, p.tile_ids, p.ntiles, sub, tcol, tot, counts, offsets, ntp,
        block_ids, block_cap, sorted, sorted_cap);
}

bool decode_prologue_fits(int T, int top_k, int E, int64_t sorted_cap) {
  return T <= kPrologueMaxTokens && static_cast<int64_t>(T) * top_k <= kPrologueMaxIds &&
         E <= kPrologueMaxE && sorted_cap <= 16384;
}

void launch_decode_prologue(const float* logits, int T, int E, int top_k, int scoring,
                            int renorm, int32_t* ids, float* weights, int BM, int32_t* counts,
                            int32_t* offsets, int32_t* sorted, int64_t sorted_cap,
                            int32_t* block_ids, int64_t block_cap, int32_t* ntp, hipStream_t s) {
  const int nbits = ceil_log2(E);
  // batch: the tokens' count rounded up to a power of two, at most 8/VPL
  // logits registers' worth (8 for E <= 64)
  auto go = [&](auto vpl) {
    constexpr int V = decltype(vpl)::value;
    auto run = [&](auto tb) {
      decode_prologue_kernel<V, decltype(tb)::value><<<1, 64, 0, s>>>(
          logits, T, E, top_k, scoring, renorm, ids, weights, nbits, BM, counts, offsets, sorted,
          sorted_cap, block_ids, block_cap, ntp);
    };
    constexpr int cap = V >= 8 ? 1 : 8 / V;
    if (T <= 1 || cap == 1) run(std::integral_constant<int, 1>{});
    else if (T <= 2 || cap == 2) run(std::integral_constant<int, (cap >= 2 ? 2 : 1)>{});
    else if (T <= 4 || cap == 4) run(std::integral_constant<int, (cap >= 4 ? 4 : 1)>{});
    else run(std::integral_constant<int, (cap >= 8 ? 8 : 1)>{});
  };
  if (E <= 64) go(std::integral_constant<int, 1>{});
  else if (E <= 128) go(std::integral_constant<int, 2>{});
  else if (E <= 256) go(std::integral_constant<int, 4>{});
  else if (E <= 512) go(std::integral_constant<int, 8>{});
  else go(std::integral_constant<int, 16>{});
}

}  // namespace moe
