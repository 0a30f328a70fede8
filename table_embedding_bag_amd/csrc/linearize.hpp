// linearize.hpp -- the linearize step of the TBE backward's grouping, shared
// by the stand-alone linearize kernel (sort.hip) and the forward kernel that
// also linearizes the batch it pools (forward.hip).
//
// kimbodo.com/?p=28372, "Kimbodo Engineering Perspective": the grouping starts
// with a transpose of the batch into (table, row) ids.  Here
//   key_i = roff_t + x_i (one 32-bit id space over all tables),
//   value_i = bag id k (plain sums), or lookup id i with a side record
//             {k, p_i * s_k} when lookups carry a coefficient,
// and the digits of every radix pass are counted on the way (the counts do not
// depend on the order of the keys, so no pass needs a counting kernel).
#pragma once

#include "common.hpp"

namespace tbe {

constexpr int kLinBags = 128;               // bags per linearize tile
// Bags per tile of the stand-alone linearize kernel when a batch has more
// tiles of kLinBags than its grid holds: fewer, longer tiles then amortise
// each tile's offset staging (16.8 M lookups in bags of 8: 141 -> 121 us).
// The launch that pools and linearizes together keeps kLinBags (512 doubled
// its time).
constexpr int kLinBagsLarge = 512;
constexpr int64_t kLinMaxBlocks = 1024;     // linearize grid bound
constexpr int kLinThreads = 1024;           // threads per linearize workgroup

// Workgroups of the linearize step: one per tile of bags, at most kLinMaxBlocks.
inline int64_t linearize_blocks(int64_t num_bags, int bags = kLinBags) {
  const int64_t b = (num_bags + bags - 1) / bags;
  return b < 1 ? 1 : (b < kLinMaxBlocks ? b : kLinMaxBlocks);
}

template <typename IT>
__device__ __forceinline__ int64_t lin_index(const void* p, int64_t i) {
  return static_cast<int64_t>(static_cast<const IT*>(p)[i]);
}

// A workgroup of NT threads takes tiles first, first + stride, ... of
// BAGS consecutive bags.  A tile's offsets are staged in LDS; the
// workgroup then walks the tile's lookups NT * K at a time, each thread
// taking K positions (consecutive threads on consecutive lookups): the bags
// are found by binary search in LDS and all K row ids are loaded before any
// is used, so a thread keeps K loads in flight.  Digit counts are kept in LDS
// across the workgroup's tiles and added to the global counts once at the end
// (a bounded grid keeps those global atomics, all on the same few hundred
// words, few).  The global digit counts must be zero before the first
// workgroup starts.
template <typename IT, int NT, int K, int BAGS = kLinBags>
__device__ __forceinline__ void linearize_tiles(const BackwardLaunch& a, int64_t first,
                                                int64_t stride) {
  static_assert(NT >= BAGS, "one thread per bag stages the offsets");
  __shared__ int64_t s_off[BAGS + 1];
  __shared__ uint32_t s_roff[BAGS];
  __shared__ float s_scale[BAGS];
  __shared__ uint32_t s_hist[kMaxRadixPasses << kMaxRadixBits];

  const int tid = threadIdx.x;
  const int passes = radix_passes(a.key_bits, a.num_indices);
  const int bits = radix_digit_bits(a.key_bits, a.num_indices);
  const int slots = radix_slots(bits);
  const uint32_t dmask = (1u << bits) - 1u;
  for (int i = tid; i < passes * slots; i += NT) s_hist[i] = 0u;
  const int64_t ntiles = (a.num_bags + BAGS - 1) / BAGS;
  for (int64_t tile = first; tile < ntiles; tile += stride) {
    const int64_t k0 = tile * BAGS;
    const int nb = static_cast<int>(min(static_cast<int64_t>(BAGS), a.num_bags - k0));
    __syncthreads();  // the previous tile's offsets are no longer read
    if (tid < nb) {
      const int64_t k = k0 + tid;
      const int64_t lo = lin_index<IT>(a.offsets, k);
      const int64_t hi = lin_index<IT>(a.offsets, k + 1);
      s_off[tid] = lo;
      if (tid == nb - 1) s_off[nb] = hi;
      const int t = static_cast<int>(k / a.B);
      s_roff[tid] = static_cast<uint32_t>(a.meta[t].roff);
      s_scale[tid] = a.mean ? ((hi > lo) ? 1.0f / static_cast<float>(hi - lo) : 0.0f) : 1.0f;
    }
    __syncthreads();

    const int64_t p0 = s_off[0], p1 = s_off[nb];
    // A tile whose lookups are nb times its first bag's length most likely
    // has equally long bags: there the slot interpolated from the position is
    // exact (it is checked before it is used) and the binary search is
    // skipped.  Bags of 8 lookups: 121 -> 107 us on 16.8 M lookups; trying it
    // on every tile cost 4 us on 5.2 M lookups of Poisson lengths.
    const bool even = p1 - p0 == static_cast<int64_t>(nb) * (s_off[1] - p0);
    const float per = even && p1 > p0 ? static_cast<float>(nb) / static_cast<float>(p1 - p0) : 0.0f;
    for (int64_t base = p0; base < p1; base += static_cast<int64_t>(NT) * K) {
      int slot[K];
      bool ok[K];
      int64_t x[K];
      float pw[K];
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const int64_t p = base + tid + static_cast<int64_t>(NT) * k;
        ok[k] = p < p1;
        // bag slot s with s_off[s] <= p < s_off[s + 1]
        int g = static_cast<int>(static_cast<float>(p - p0) * per);
        g = g < 0 ? 0 : (g > nb - 1 ? nb - 1 : g);
        if (even && s_off[g] <= p && p < s_off[g + 1]) {
          slot[k] = g;
        } else {
          int lo = 0, hi = nb;
          while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (s_off[mid] <= p)
              lo = mid;
            else
              hi = mid;
          }
          slot[k] = lo;
        }
      }
      // every load of the batch is issued before any is used (positions past
      // the tile read its last lookup instead)
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const int64_t p = ok[k] ? base + tid + static_cast<int64_t>(NT) * k : p1 - 1;
        x[k] = lin_index<IT>(a.indices, p);
        pw[k] = a.psw ? a.psw[p] : 1.0f;
      }
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const int64_t p = base + tid + static_cast<int64_t>(NT) * k;
        const uint32_t key = s_roff[slot[k]] + static_cast<uint32_t>(x[k]);
        const uint32_t bag = static_cast<uint32_t>(k0 + slot[k]);
        if (ok[k]) {
          a.buf.keys[0][p] = key;
          if (a.use_rec) {
            a.buf.vals[0][p] = static_cast<uint32_t>(p);
            a.buf.rec[p] = make_uint2(bag, __float_as_uint(pw[k] * s_scale[slot[k]]));
          } else {
            a.buf.vals[0][p] = bag;
          }
        }
        // digit counts: lanes holding the same digit are matched through one
        // ballot per digit bit and only the lowest of them adds their number
        // (the high digits of one table's keys take few values, so per-lane
        // atomics would queue on a handful of LDS words)
        const uint64_t active = __ballot(ok[k]);
        if (active == 0) continue;
        for (int q = 0; q < passes; ++q) {
          const uint32_t d = (key >> (q * bits)) & dmask;
          uint64_t peers = active;
          for (int bit = 0; bit < bits; ++bit) {
            const bool set = (d >> bit) & 1u;
            const uint64_t bal = __ballot(set);
            peers &= set ? bal : ~bal;
          }
          if (ok[k] && popc_below(peers) == 0) atomicAdd(&s_hist[q * slots + d], __popcll(peers));
        }
      }
    }
  }
  __syncthreads();
  for (int i = tid; i < passes * slots; i += NT)
    if (s_hist[i]) atomicAdd(&a.buf.digit_hist[i], s_hist[i]);
}

}  // namespace tbe
