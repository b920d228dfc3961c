// Block schedule of the batched activation format.
//
// The batched format hands the experts one batch per expert: rows
// [0, count[e]) of an [E, M, H] activation belong to expert e, the rest of
// its M rows carry nothing.  The grouped GEMMs walk the same kind of
// schedule align produces for the standard format -- a sorted row list cut
// into block_m-row blocks, each owned by one expert -- so this kernel writes
// that schedule straight from the counts:
//   block_expert[b] = e for the ceil(count[e] / bm) blocks of expert e
//                     (experts in index order), -1 past the last one
//   sorted[b*bm + r] = e*M + m with m = (b - first block of e)*bm + r when
//                     m < count[e], else the sentinel E*M
//   ntp[0]          = bm * (number of owned blocks)
// Row e*M + m is then both the activation row the first GEMM reads (the
// "token" with top_k 1) and the output row the second GEMM writes, so the
// batch rows are used in place: no gather, no scatter.
//
// Every workgroup rebuilds the padded block offsets of all experts in LDS
// (a few KB of counts from L2) and then fills its share of positions, one
// binary search over the offsets per position.  Counts are clamped to
// [0, M] so no schedule entry can point outside the caller's batches.
#include <algorithm>

#include "moe_device.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kMaxE = 1024;
constexpr int kThreads = 256;
constexpr int kMaxGrid = 2048;

__global__ __launch_bounds__(kThreads) void batched_schedule_kernel(
    const int32_t* __restrict__ counts, int E, int M, int bm_log2, int64_t positions,
    int32_t* __restrict__ sorted, int32_t* __restrict__ block_expert, int32_t* __restrict__ ntp) {
  __shared__ int cnt[kMaxE];
  __shared__ int boff[kMaxE + 1];
  __shared__ int wsum[kThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int bm = 1 << bm_log2;

  for (int e = tid; e < E; e += kThreads) {
    const int c = min(max(counts[e], 0), M);
    cnt[e] = c;
    boff[e] = (c + bm - 1) >> bm_log2;
  }
  __syncthreads();

  // exclusive scan of the per-expert block counts: each thread owns a run
  // of consecutive experts, a wave scan of the run sums, then the waves
  const int per = (E + kThreads - 1) / kThreads;
  const int lo = min(tid * per, E), hi = min(lo + per, E);
  int local = 0;
  for (int i = lo; i < hi; ++i) local += boff[i];
  int incl = local;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int up = __shfl_up(incl, o, 64);
    if (lane >= o) incl += up;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int run = incl - local;
  for (int w = 0; w < wave; ++w) run += wsum[w];
  for (int i = lo; i < hi; ++i) {
    const int x = boff[i];
    boff[i] = run;
    run += x;
  }
  if (tid == kThreads - 1) boff[E] = run;   // the last run ends at the total
  __syncthreads();

  const int total = boff[E];
  if (blockIdx.x == 0 && tid == 0) ntp[0] = total << bm_log2;
  const int sentinel = E * M;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
  for (int64_t p = static_cast<int64_t>(blockIdx.x) * kThreads + tid; p < positions; p += stride) {
    const int b = static_cast<int>(p >> bm_log2);
    const int r = static_cast<int>(p & (bm - 1));
    int val = sentinel, owner = -1;
    if (b < total) {
      // the owner is the last expert whose first block is <= b (an empty
      // expert shares its offset with the next one and owns nothing)
      int l = 0, h = E - 1;
      while (l < h) {
        const int mid = (l + h + 1) >> 1;
        if (boff[mid] <= b) l = mid;
        else h = mid - 1;
      }
      owner = l;
      const int m = ((b - boff[l]) << bm_log2) + r;
      if (m < cnt[l]) val = l * M + m;
    }
    sorted[p] = val;
    if (r == 0) block_expert[b] = owner;
  }
}

}  // namespace

void launch_batched_schedule(const int32_t* counts, int E, int M, int bm, int64_t block_cap,
                             int32_t* sorted, int32_t* block_expert, int32_t* ntp, hipStream_t s) {
  int bm_log2 = 0;
  while ((1 << bm_log2) < bm) ++bm_log2;
  const int64_t positions = block_cap * bm;
  const int64_t want = (positions + kThreads - 1) / kThreads;
  const unsigned grid = static_cast<unsigned>(std::max<int64_t>(1, std::min<int64_t>(want, kMaxGrid)));
  batched_schedule_kernel<<<grid, kThreads, 0, s>>>(counts, E, M, bm_log2, positions, sorted,
                                                     block_expert, ntp);
}

}  // namespace moe
