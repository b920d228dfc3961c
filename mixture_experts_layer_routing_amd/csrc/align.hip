// align: sort the flat rows i = t*top_k + j by expert into block_m-padded
// groups, deterministically (ascending i inside every expert).
//
// Counting is order-free (LDS atomic adds per id).  Stable ranks need no
// atomics: a wave takes 64 consecutive ids at a time
// and finds, for every lane, the lanes holding the same expert id with one
// ballot per bit of the id (peer mask = AND over the bits of the lanes that
// agree on that bit, ceil(log2 E) ballots).  The lane's rank among its peers
// is the popcount of the peers below it; the lowest peer is the group's
// leader and is the only lane that touches the expert's LDS counter, so no
// two lanes of an instruction hit the same address.  Each wave owns a
// contiguous sub-range of its workgroup's ids and walks it in index order
// with a private per-expert cursor, so ranks need no exchange between waves
// beyond one prefix over the waves' counts.  Every lane keeps 16 ids in
// flight (strided by 64, so each load is a coalesced 256-byte row and the
// processing order is the index order).
//
// n <= 32768 ids: one 1024-thread workgroup does everything (count, padded
// offsets, block owners, scatter).  Larger n: tiles of 2048-65536 ids (see
// plan()), each split into 4 wave sub-ranges:
//   count   -- one workgroup per tile: per-(sub-range, expert) counts
//   scan    -- blocks of 64 sub-ranges: exclusive prefix per expert within
//              the block, block totals
//   top     -- one workgroup: prefix over the block totals, expert totals,
//              padded offsets
//   scatter -- one workgroup per tile: each wave starts its cursors at
//              offset + block prefix + sub-range prefix and walks; the
//              workgroups also share the block-owner and pad-sentinel fills.
// No global atomics anywhere, so the result is bit-exact and run-to-run
// identical.
#include "moe_device.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kMaxE = 1024;
constexpr int kSmallN = 32768;      // one-workgroup path up to this many ids
constexpr int kSmallThreads = 1024;
constexpr int kTileThreads = 256;   // multi-tile kernels: 4 waves
constexpr int kScanBlock = 64;      // tiles per first-level scan block
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
// LDS atomics (no return value: nothing waits on them).
__device__ void wave_count(const int32_t* __restrict__ ids, int lo, int hi, int E, int* h) {
  const int lane = threadIdx.x & 63;
  for (int c = lo; c < hi; c += 64 * kLoads) {
    int key[kLoads];
#pragma unroll
    for (int s = 0; s < kLoads; ++s) {
      const int i = c + 64 * s + lane;
      key[s] = i < hi ? ids[i] : -1;
    }
#pragma unroll
    for (int s = 0; s < kLoads; ++s)
      if (static_cast<unsigned>(key[s]) < static_cast<unsigned>(E)) atomicAdd(&h[key[s]], 1);
  }
}

// Writes the valid ids of [lo, hi) in index order: sorted[cur[e]++] = i.
__device__ void wave_scatter(const int32_t* __restrict__ ids, int lo, int hi, int E, int nbits,
                             int* cur, int32_t* __restrict__ sorted) {
  const int lane = threadIdx.x & 63;
  const uint64_t below = lanemask_lt();
  for (int c = lo; c < hi; c += 64 * kLoads) {
    int key[kLoads];
#pragma unroll
    for (int s = 0; s < kLoads; ++s) {
      const int i = c + 64 * s + lane;
      key[s] = i < hi ? ids[i] : -1;
    }
#pragma unroll
    for (int s = 0; s < kLoads; ++s) {
      const bool valid = static_cast<unsigned>(key[s]) < static_cast<unsigned>(E);
      const uint64_t m = peer_mask(key[s], valid, nbits);
      if (valid) {
        const int base = cur[key[s]];
        sorted[base + __builtin_popcountll(m & below)] = c + 64 * s + lane;
        if (lane == __builtin_ctzll(m)) cur[key[s]] = base + __builtin_popcountll(m);
      }
    }
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
  wave_count(ids, lo, hi, E, hist + wave * E);
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
// Each of the 4 waves of a tile's workgroup owns a quarter of the tile.
__device__ __forceinline__ void tile_wave_range(int tile, int tile_ids, int n, int& lo, int& hi) {
  const int wave = threadIdx.x >> 6;
  const int t0 = tile * tile_ids;
  const int t1 = min(t0 + tile_ids, n);
  const int per = tile_ids / (kTileThreads / 64);
  lo = min(t0 + wave * per, t1);
  hi = min(lo + per, t1);
}

// Counts of every wave's sub-range: sub_counts[4*tile + wave][e].
__global__ __launch_bounds__(kTileThreads) void align_count_kernel(
    const int32_t* __restrict__ ids, int n, int E, int tile_ids, int32_t* __restrict__ sub_counts) {
  constexpr int NW = kTileThreads / 64;
  __shared__ int hist[NW * kMaxE];
  const int tid = threadIdx.x, wave = tid >> 6;
  for (int x = tid; x < NW * E; x += kTileThreads) hist[x] = 0;
  __syncthreads();
  int lo, hi;
  tile_wave_range(blockIdx.x, tile_ids, n, lo, hi);
  wave_count(ids, lo, hi, E, hist + wave * E);
  __syncthreads();
  int32_t* out = sub_counts + static_cast<int64_t>(blockIdx.x) * NW * E;
  for (int x = tid; x < NW * E; x += kTileThreads) out[x] = hist[x];
}

// In-place exclusive prefix of the column v[0], v[stride], ... v[(len-1)*
// stride] (len <= 64 per call) plus `run` carried in; returns the new run.
// All loads are issued before the first store, so a call costs one round
// trip to memory rather than one per element.
__device__ __forceinline__ int column_prefix64(int32_t* v, int64_t stride, int len, int run) {
  int x[64];
#pragma unroll
  for (int t = 0; t < 64; ++t) x[t] = t < len ? v[t * stride] : 0;
#pragma unroll
  for (int t = 0; t < 64; ++t) {
    if (t < len) v[t * stride] = run;
    run += x[t];
  }
  return run;
}

// Block b of kScanBlock sub-ranges: sub_counts -> exclusive prefix per
// expert inside the block (in place); block_sums[b][e] = the block's total.
__global__ __launch_bounds__(kTileThreads) void align_scan_kernel(
    int32_t* __restrict__ sub_counts, int nsub, int E, int32_t* __restrict__ block_sums) {
  static_assert(kScanBlock == 64, "one column_prefix64 per block");
  const int s0 = blockIdx.x * kScanBlock;
  const int len = min(kScanBlock, nsub - s0);
  for (int e = threadIdx.x; e < E; e += kTileThreads) {
    const int run = column_prefix64(sub_counts + static_cast<int64_t>(s0) * E + e, E, len, 0);
    block_sums[static_cast<int64_t>(blockIdx.x) * E + e] = run;
  }
}

// One workgroup of 4 waves (one per SIMD, so column_prefix64's 64 loads in
// flight per thread fit in registers).
__global__ __launch_bounds__(kTileThreads) void align_top_kernel(
    int32_t* __restrict__ block_sums, int nblocks, int E, int BM, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ ntp) {
  __shared__ int cnt[kMaxE];
  __shared__ int tot[kMaxE];
  __shared__ int partial[kTileThreads / 64 + 1];
  for (int e = threadIdx.x; e < E; e += kTileThreads) {
    int run = 0;
    for (int b0 = 0; b0 < nblocks; b0 += 64)
      run = column_prefix64(block_sums + static_cast<int64_t>(b0) * E + e, E,
                            min(64, nblocks - b0), run);
    cnt[e] = run;
  }
  __syncthreads();
  finish_offsets<kTileThreads>(cnt, E, BM, partial, counts, offsets, ntp, tot);
}

// Each wave starts its cursors at expert offset + block prefix + its
// sub-range's prefix and walks; the workgroup also fills its share of
// block_ids (the owner search needs the offsets, known only after top).
__global__ __launch_bounds__(kTileThreads) void align_scatter_kernel(
    const int32_t* __restrict__ ids, int n, int E, int nbits, int BM, int tile_ids,
    const int32_t* __restrict__ sub_prefix, const int32_t* __restrict__ block_base,
    const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets,
    int32_t* __restrict__ block_ids, int64_t block_cap, int32_t* __restrict__ sorted,
    int64_t sorted_cap) {
  constexpr int NW = kTileThreads / 64;
  __shared__ int cur[NW * kMaxE];
  __shared__ int off[kMaxE + 1];
  const int tid = threadIdx.x, wave = tid >> 6;
  const int64_t sub0 = static_cast<int64_t>(blockIdx.x) * NW;
  const int32_t* sp = sub_prefix + sub0 * E;
  for (int x = tid; x < NW * E; x += kTileThreads) {
    const int64_t sub = sub0 + x / E;
    cur[x] = sp[x] + block_base[(sub / kScanBlock) * E + x % E];
  }
  for (int e = tid; e <= E; e += kTileThreads) off[e] = offsets[e];
  __syncthreads();
  for (int x = tid; x < NW * E; x += kTileThreads) cur[x] += off[x % E];
  __syncthreads();
  int lo, hi;
  tile_wave_range(blockIdx.x, tile_ids, n, lo, hi);
  wave_scatter(ids, lo, hi, E, nbits, cur + wave * E, sorted);
  const int64_t per = (block_cap + gridDim.x - 1) / gridDim.x;
  const int64_t b0 = min<int64_t>(static_cast<int64_t>(blockIdx.x) * per, block_cap);
  fill_block_owners<kTileThreads>(off, E, BM, off[E], b0, min(b0 + per, block_cap), block_ids);
  const int64_t tail = sorted_cap - off[E];
  const int64_t tper = (tail + gridDim.x - 1) / gridDim.x;
  const int64_t p0 = off[E] + min<int64_t>(static_cast<int64_t>(blockIdx.x) * tper, tail);
  const int64_t p1 = min<int64_t>(p0 + tper, sorted_cap);
  fill_sentinels(off, counts, E, n, blockIdx.x * NW + wave, gridDim.x * NW, p0 + tid, p1,
                 kTileThreads, sorted);
}

struct AlignPlan {
  int tile_ids, ntiles, nsub, nblocks;
};

// Tiles: at most 2048 of them (several per CU at the largest sizes); and,
// while at least 512 tiles remain, at least 128 ids per expert on average,
// so that each expert's run of slots written by one tile spans several
// 128-byte lines (a line shared with the neighbouring tile, possibly on
// another XCD, is written back partially).
AlignPlan plan(int64_t n, int E) {
  AlignPlan p{0, 0, 0, 0};
  if (n <= kSmallN) return p;
  int t = 2048;
  while (t < 65536) {
    const bool too_many = static_cast<int64_t>(t) * 2048 < n;
    const bool short_runs = t < 128 * E && n / (2 * static_cast<int64_t>(t)) >= 512;
    if (!too_many && !short_runs) break;
    t *= 2;
  }
  p.tile_ids = t;
  p.ntiles = static_cast<int>((n + t - 1) / t);
  p.nsub = p.ntiles * (kTileThreads / 64);
  p.nblocks = (p.nsub + kScanBlock - 1) / kScanBlock;
  return p;
}

}  // namespace

size_t align_workspace_bytes(int64_t n, int E) {
  const AlignPlan p = plan(n, E);
  return static_cast<size_t>(p.nsub + p.nblocks) * E * sizeof(int32_t);
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
  int32_t* sc = static_cast<int32_t*>(ws);
  int32_t* bs = sc + static_cast<int64_t>(p.nsub) * E;
  align_count_kernel<<<p.ntiles, kTileThreads, 0, s>>>(ids, nn, E, p.tile_ids, sc);
  align_scan_kernel<<<p.nblocks, kTileThreads, 0, s>>>(sc, p.nsub, E, bs);
  align_top_kernel<<<1, kTileThreads, 0, s>>>(bs, p.nblocks, E, BM, counts, offsets, ntp);
  align_scatter_kernel<<<p.ntiles, kTileThreads, 0, s>>>(ids, nn, E, nbits, BM, p.tile_ids, sc,
                                                         bs, counts, offsets, block_ids,
                                                         block_cap, sorted, sorted_cap);
}

}  // namespace moe
