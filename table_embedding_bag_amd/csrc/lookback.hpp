// lookback.hpp -- decoupled look-back helpers shared by the radix passes and
// the bucket-local sort (sort.hip) and by the linearize step that scatters on
// the high digit (linearize.hpp).  Internal; the public interface is tbe.h.
//
// A status word holds a 2-bit flag and a 30-bit count: kFlagAgg for a tile's
// own count, kFlagIncl for the count up to and including the tile.  Words are
// read and written with agent-scope atomics, so they are coherent across the
// XCDs' L2 caches.
#pragma once

#include "common.hpp"

namespace tbe {

constexpr uint32_t kFlagAgg = 1u << 30;     // status word: this tile's own count
constexpr uint32_t kFlagIncl = 2u << 30;    // status word: count up to and including this tile
constexpr uint32_t kValueMask = (1u << 30) - 1u;

__device__ __forceinline__ uint32_t ld_status(uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_status(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Counts of digits d0 .. d0 + DPT - 1 in all tiles before `tile` (decoupled
// look-back; every digit keeps DEPTH status words in flight per round).
// status rows have `slots` words per tile.  A wait that gives up leaves excl
// at most the true count, so every position derived from it stays in range.
template <int DPT, int DEPTH>
__device__ void lookback_digits(uint32_t* status, int slots, int tile, int d0, WaitCtl wait,
                                uint32_t (&excl)[DPT]) {
  int j[DPT];
  bool done[DPT];
#pragma unroll
  for (int q = 0; q < DPT; ++q) excl[q] = 0u, j[q] = tile - 1, done[q] = false;
  if (wait.limit == 0u) {
    atomicOr(wait.err, 1u);
    return;
  }
  uint32_t spins = 0;
  while (true) {
    uint32_t w[DPT][DEPTH];
#pragma unroll
    for (int q = 0; q < DPT; ++q)
#pragma unroll
      for (int k = 0; k < DEPTH; ++k)
        w[q][k] = (!done[q] && j[q] - k >= 0)
                      ? ld_status(status + static_cast<int64_t>(j[q] - k) * slots + d0 + q)
                      : kFlagIncl;
    bool all_done = true, moved = false;
#pragma unroll
    for (int q = 0; q < DPT; ++q) {
      if (done[q]) continue;
      bool stop = false;
      int used = 0;
#pragma unroll
      for (int k = 0; k < DEPTH; ++k) {
        if (!stop) {
          const uint32_t f = w[q][k] & ~kValueMask;
          if (f == 0) {
            stop = true;  // not published yet: poll again from here
          } else {
            excl[q] += w[q][k] & kValueMask;
            ++used;
            if (f == kFlagIncl) stop = done[q] = true;
          }
        }
      }
      j[q] -= used;
      moved |= used > 0;
      all_done &= done[q];
    }
    if (all_done) return;
    if (!moved) {
      if (++spins > wait.limit) {
        atomicOr(wait.err, 1u);
        return;
      }
      __builtin_amdgcn_s_sleep(2);
    }
  }
}

// Window range records of the bucket-local sort: bucket d of the high digit
// (sorted positions [start, start + count)) belongs to window start /
// kBucketWindow.  A record is {~first start, end, ~first bucket, last bucket +
// 1}, built with atomic maxima on a zeroed record, so 0 in the last word
// means the window starts no bucket.
__device__ __forceinline__ void record_window(uint32_t* wtable, uint32_t start, uint32_t count,
                                              uint32_t d) {
  uint32_t* w = wtable + 4 * (start / kBucketWindow);
  atomicMax(w + 0, ~start);
  atomicMax(w + 1, start + count);
  atomicMax(w + 2, ~d);
  atomicMax(w + 3, d + 1u);
}

// Exclusive prefix sum over a block of NW waves; *total receives the sum.
template <int NW>
__device__ __forceinline__ uint32_t block_excl_n(uint32_t x, uint32_t* scratch, uint32_t* total) {
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const uint32_t incl = wave_inclusive_sum(x);
  if (lane == kWave - 1) scratch[wave] = incl;
  __syncthreads();
  uint32_t base = 0, sum = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint32_t s = scratch[w];
    base += (w < wave) ? s : 0u;
    sum += s;
  }
  __syncthreads();
  *total = sum;
  return base + incl - x;
}

}  // namespace tbe
