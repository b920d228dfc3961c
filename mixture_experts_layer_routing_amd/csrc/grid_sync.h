// Grid-wide synchronisation of a launch whose workgroups are all resident
// at once (the align kernel's one-launch path, the one-launch layer).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <chrono>
#include <random>

namespace moe {
// (internal linkage: each including source keeps its own copy, as when the
// functions lived in it)
namespace {

constexpr uint32_t kMaxSpins = 1u << 20;                 // about a second of polling

// Grid barrier over resident workgroups, in two halves.  arrive: thread 0
// publishes (release) flag[g] = epoch after the workgroup's stores (the
// caller synchronises the workgroup first).  await: workgroup 0 waits for
// every flag, then raises go = epoch; the others wait for go.  Afterwards
// each workgroup's loads see what every workgroup stored before arriving.
// The waits give up after kMaxSpins polls; await then returns false in
// every thread of the workgroup.
__device__ __forceinline__ void grid_arrive(uint64_t* flag, uint64_t epoch, int g) {
  if (threadIdx.x == 0) __hip_atomic_store(flag + g, epoch, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ bool grid_await(uint64_t* flag, uint64_t* go, uint64_t epoch, int g, int G, int* okf) {
  const int tid = threadIdx.x;
  if (g == 0) {
    int ok = 1;
    if (tid < G) {
      uint32_t spins = 0;
      while (__hip_atomic_load(flag + tid, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != epoch) {
        __builtin_amdgcn_s_sleep(2);
        if (++spins == kMaxSpins) { ok = 0; break; }
      }
    }
    ok = __syncthreads_and(ok);
    if (tid == 0) {
      *okf = ok;
      if (ok) {
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        __hip_atomic_store(go, epoch, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  } else if (tid == 0) {
    int ok = 1;
    uint32_t spins = 0;
    while (__hip_atomic_load(go, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != epoch) {
      __builtin_amdgcn_s_sleep(2);
      if (++spins == kMaxSpins) { ok = 0; break; }
    }
    *okf = ok;
  }
  if (tid == 0) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  __syncthreads();
  return *okf != 0;
}

// A new epoch per call: flags and the go word from earlier calls (or from
// whatever the workspace held) differ from it.  64 random bits to start.
uint64_t next_epoch() {
  static std::atomic<uint64_t> ctr{0};
  static const uint64_t seed = [] {
    std::random_device rd;
    return (static_cast<uint64_t>(rd()) << 32) ^ rd() ^
           static_cast<uint64_t>(std::chrono::steady_clock::now().time_since_epoch().count());
  }();
  return seed + 0x9E3779B97F4A7C15ull * (ctr.fetch_add(1, std::memory_order_relaxed) + 1);
}

}  // namespace
}  // namespace moe
