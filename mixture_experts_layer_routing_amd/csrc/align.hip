// align: sort the flat rows i = t*top_k + j by expert into block_m-padded
// groups, deterministically (ascending i inside every expert).
//
// A wave takes 64 consecutive ids at a time and finds, for every lane, the
// lanes holding the same expert id with one ballot per bit of the id (peer
// mask = AND over the bits of the lanes that agree on that bit, ceil(log2 E)
// ballots).  The lowest peer is the group's leader and is the only lane that
// advances the expert's LDS cursor, so no two lanes of an instruction hit the
// same address.  A lane's rank among its peers is the popcount of the peers
// below it.  (Counting is order-free: per-id LDS atomic adds.)  Each wave owns a contiguous sub-range of its workgroup's ids and
// walks it in index order with a private per-expert cursor, so ranks need no
// exchange between waves beyond one prefix over the waves' counts.  Every
// lane keeps 16 ids in flight (strided by 64, so each load is a coalesced
// 256-byte row and the processing order is the index order).
//
// n <= 32768 ids: one 1024-thread workgroup does everything (count, padded
// offsets, block owners, scatter).  Larger n: tiles of 2048-8192 ids (see
// plan()), each split into 8 wave sub-ranges, in three launches:
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
// No global atomics anywhere, so the result is bit-exact and run-to-run
// identical.
#include "moe_device.h"
#include "launch.h"

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

}  // namespace

size_t align_workspace_bytes(int64_t n, int E) {
  const AlignPlan p = plan(n, E);
  if (p.ntiles == 0) return 0;
  return (static_cast<size_t>(p.ntiles) * (kTileWaves + 1) + 1) * E * sizeof(int32_t);
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

}  // namespace moe
