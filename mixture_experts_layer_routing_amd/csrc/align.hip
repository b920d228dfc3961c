// align: sort the flat rows i = t*top_k + j by expert into block_m-padded
// groups, deterministically (ascending i inside every expert).
//
// The ids are cut into tiles of 1024 (four 256-id steps per workgroup: the
// ballot grouping costs one pass per distinct id in a wave, so short tiles
// spread it over many workgroups).  count: one workgroup per tile builds
// the tile's expert histogram with LDS atomics (order-free).  scan: one
// workgroup turns the [tile][expert] counts into per-expert totals, padded
// offsets (exclusive scan), per-(tile, expert) write bases, block owners and
// the pad sentinels.  scatter: one workgroup per tile walks its ids in order,
// 256 at a time; inside a wave, lanes with equal ids are grouped with ballots
// (stable rank = lanes below with the same id), waves of the same step are
// ordered through a small LDS table, and a per-expert LDS cursor carries the
// position across steps.  No global atomics, so the result is bit-exact.
// A single-tile input (T*k <= 1024) runs all three phases in one launch.
#include "moe_device.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kTile = 1024;
constexpr int kMaxE = 1024;

// Exclusive scan of v[0..count) in LDS by all NT threads of the block;
// returns the total.  `partial` needs NT/64 + 1 ints of LDS.
template <int NT>
__device__ int block_exclusive_scan(int* v, int count, int* partial) {
  const int tid = threadIdx.x;
  const int per = (count + NT - 1) / NT;
  const int lo = min(tid * per, count), hi = min(lo + per, count);
  int local = 0;
  for (int i = lo; i < hi; ++i) local += v[i];
  // inclusive scan of `local` across the wave
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

// Histogram of one tile into hist (LDS, E entries, zeroed by the caller).
__device__ void tile_histogram(const int32_t* __restrict__ ids, int n, int E, int tile, int* hist) {
  const int base = tile * kTile;
  for (int r = 0; r < kTile / 256; ++r) {
    const int i = base + r * 256 + threadIdx.x;
    if (i < n) {
      const int id = ids[i];
      if (static_cast<unsigned>(id) < static_cast<unsigned>(E)) atomicAdd(&hist[id], 1);
    }
  }
}

// Stable scatter of one tile: cursor[e] (LDS) starts at the tile's first slot
// for expert e.  wcnt: LDS [4][E] scratch.  256 threads.
__device__ void tile_scatter(const int32_t* __restrict__ ids, int n, int E, int tile,
                             int* cursor, uint32_t* wcnt, int32_t* __restrict__ sorted) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int x = tid; x < 4 * E; x += 256) wcnt[x] = 0xffffffffu;
  __syncthreads();
  const int base = tile * kTile;
  const uint64_t below = lanemask_lt();
  for (int r = 0; r < kTile / 256; ++r) {
    const int i = base + r * 256 + tid;
    int id = -1;
    if (i < n) id = ids[i];
    const bool valid = static_cast<unsigned>(id) < static_cast<unsigned>(E);
    uint64_t pending = __ballot(valid);
    int rank = 0, grp = 0;
    bool leader = false;
    while (pending) {
      const int src = __builtin_ctzll(pending);
      const int v = __shfl(id, src, 64);
      const uint64_t m = __ballot(valid && id == v);
      if (valid && id == v) {
        rank = __builtin_popcountll(m & below);
        grp = __builtin_popcountll(m);
        leader = lane == src;
      }
      pending &= ~m;
    }
    if (leader) wcnt[wave * E + id] = (static_cast<uint32_t>(r) << 8) | static_cast<uint32_t>(grp);
    __syncthreads();
    if (valid) {
      int prefix = 0;
      for (int w = 0; w < wave; ++w) {
        const uint32_t c = wcnt[w * E + id];
        if ((c >> 8) == static_cast<uint32_t>(r)) prefix += static_cast<int>(c & 0xffu);
      }
      sorted[cursor[id] + prefix + rank] = i;
    }
    __syncthreads();
    if (leader) atomicAdd(&cursor[id], grp);
    __syncthreads();
  }
}

// Per-expert totals -> counts, padded offsets, block owners, pad sentinels.
// `cnt` (LDS, E) holds totals on entry and the exclusive padded offsets on
// exit.  Returns num_tokens_post_padded.
template <int NT>
__device__ int finish_offsets(int* cnt, int E, int BM, int n, int* partial,
                              int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                              int32_t* __restrict__ sorted, int64_t sorted_cap,
                              int32_t* __restrict__ block_ids, int64_t block_cap,
                              int32_t* __restrict__ ntp, int* total_lds) {
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += NT) {
    const int c = cnt[e];
    counts[e] = c;
    total_lds[e] = c;
    cnt[e] = (c + BM - 1) / BM * BM;
  }
  __syncthreads();
  const int total = block_exclusive_scan<NT>(cnt, E, partial);
  for (int e = tid; e < E; e += NT) {
    const int off = cnt[e];
    const int c = total_lds[e];
    const int end = (e + 1 < E) ? cnt[e + 1] : total;
    offsets[e] = off;
    for (int b = off / BM; b < end / BM; ++b) block_ids[b] = e;
    for (int p = off + c; p < end; ++p) sorted[p] = n;
  }
  if (tid == 0) { offsets[E] = total; ntp[0] = total; }
  for (int64_t b = total / BM + tid; b < block_cap; b += NT) block_ids[b] = -1;
  for (int64_t p = total + tid; p < sorted_cap; p += NT) sorted[p] = n;
  return total;
}

__global__ __launch_bounds__(256) void align_single_kernel(
    const int32_t* __restrict__ ids, int n, int E, int BM, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted, int64_t sorted_cap,
    int32_t* __restrict__ block_ids, int64_t block_cap, int32_t* __restrict__ ntp) {
  __shared__ int cnt[kMaxE];
  __shared__ int tot[kMaxE];
  __shared__ uint32_t wcnt[4 * kMaxE];
  __shared__ int partial[8];
  for (int e = threadIdx.x; e < E; e += 256) cnt[e] = 0;
  __syncthreads();
  tile_histogram(ids, n, E, 0, cnt);
  __syncthreads();
  finish_offsets<256>(cnt, E, BM, n, partial, counts, offsets, sorted, sorted_cap, block_ids,
                      block_cap, ntp, tot);
  __syncthreads();
  tile_scatter(ids, n, E, 0, cnt, wcnt, sorted);
}

__global__ __launch_bounds__(256) void align_count_kernel(const int32_t* __restrict__ ids, int n,
                                                          int E, int32_t* __restrict__ tile_counts) {
  __shared__ int hist[kMaxE];
  for (int e = threadIdx.x; e < E; e += 256) hist[e] = 0;
  __syncthreads();
  tile_histogram(ids, n, E, blockIdx.x, hist);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256)
    tile_counts[static_cast<int64_t>(blockIdx.x) * E + e] = hist[e];
}

__global__ __launch_bounds__(1024) void align_scan_kernel(
    int32_t* __restrict__ tile_counts, int ntiles, int n, int E, int BM,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ sorted,
    int64_t sorted_cap, int32_t* __restrict__ block_ids, int64_t block_cap,
    int32_t* __restrict__ ntp) {
  __shared__ int cnt[kMaxE];
  __shared__ int tot[kMaxE];
  __shared__ int partial[17];
  // per expert: exclusive prefix over tiles (in place), total
  for (int e = threadIdx.x; e < E; e += 1024) {
    int run = 0;
    for (int t = 0; t < ntiles; ++t) {
      int32_t* p = tile_counts + static_cast<int64_t>(t) * E + e;
      const int c = *p;
      *p = run;
      run += c;
    }
    cnt[e] = run;
  }
  __syncthreads();
  finish_offsets<1024>(cnt, E, BM, n, partial, counts, offsets, sorted, sorted_cap, block_ids,
                       block_cap, ntp, tot);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 1024) {
    const int off = cnt[e];
    for (int t = 0; t < ntiles; ++t) tile_counts[static_cast<int64_t>(t) * E + e] += off;
  }
}

__global__ __launch_bounds__(256) void align_scatter_kernel(const int32_t* __restrict__ ids, int n,
                                                            int E,
                                                            const int32_t* __restrict__ tile_base,
                                                            int32_t* __restrict__ sorted) {
  __shared__ int cursor[kMaxE];
  __shared__ uint32_t wcnt[4 * kMaxE];
  for (int e = threadIdx.x; e < E; e += 256)
    cursor[e] = tile_base[static_cast<int64_t>(blockIdx.x) * E + e];
  __syncthreads();
  tile_scatter(ids, n, E, blockIdx.x, cursor, wcnt, sorted);
}

}  // namespace

size_t align_workspace_bytes(int64_t n, int E) {
  const int64_t ntiles = (n + kTile - 1) / kTile;
  return ntiles <= 1 ? 0 : static_cast<size_t>(ntiles) * E * sizeof(int32_t);
}

void launch_align(const int32_t* ids, int64_t n, int E, int BM, int32_t* counts,
                  int32_t* offsets, int32_t* sorted, int64_t sorted_cap, int32_t* block_ids,
                  int64_t block_cap, int32_t* ntp, void* ws, hipStream_t s) {
  const int64_t ntiles = (n + kTile - 1) / kTile;
  if (ntiles <= 1) {
    align_single_kernel<<<1, 256, 0, s>>>(ids, static_cast<int>(n), E, BM, counts, offsets, sorted,
                                          sorted_cap, block_ids, block_cap, ntp);
    return;
  }
  int32_t* tc = static_cast<int32_t*>(ws);
  const int nn = static_cast<int>(n);
  align_count_kernel<<<static_cast<unsigned>(ntiles), 256, 0, s>>>(ids, nn, E, tc);
  align_scan_kernel<<<1, 1024, 0, s>>>(tc, static_cast<int>(ntiles), nn, E, BM, counts, offsets,
                                       sorted, sorted_cap, block_ids, block_cap, ntp);
  align_scatter_kernel<<<static_cast<unsigned>(ntiles), 256, 0, s>>>(ids, nn, E, tc, sorted);
}

}  // namespace moe
