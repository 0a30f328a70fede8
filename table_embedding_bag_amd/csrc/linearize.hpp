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
#include "lookback.hpp"

namespace tbe {

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

// Bag slot s of a tile with s_off[s] <= p < s_off[s + 1] (s_off: the tile's
// nb + 1 offsets in LDS).  A tile whose lookups are nb times its first bag's
// length most likely has equally long bags: there the slot interpolated from
// the position (per = nb / lookups) is exact -- it is checked before it is
// used -- and the binary search is skipped.  Bags of 8 lookups: 121 -> 107 us
// on 16.8 M lookups; trying it on every tile cost 4 us on 5.2 M lookups of
// Poisson lengths.
__device__ __forceinline__ int tile_bag_slot(const int64_t* s_off, int nb, int64_t p, int64_t p0,
                                             bool even, float per) {
  int g = static_cast<int>(static_cast<float>(p - p0) * per);
  g = g < 0 ? 0 : (g > nb - 1 ? nb - 1 : g);
  if (even && s_off[g] <= p && p < s_off[g + 1]) return g;
  int lo = 0, hi = nb;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (s_off[mid] <= p)
      lo = mid;
    else
      hi = mid;
  }
  return lo;
}

// Lanes among `active` whose digit d (of `bits` bits) equals this lane's: one
// ballot per digit bit.  Call with the whole wave.
__device__ __forceinline__ uint64_t match_bits(uint64_t active, uint32_t d, int bits) {
  return match_low_bits(active, d, bits);
}

// A workgroup of NT threads takes tiles first, first + stride, ... of
// BAGS consecutive bags.  A tile's offsets are staged in LDS; the
// workgroup then walks the tile's lookups NT * K at a time, each thread
// taking K positions (consecutive threads on consecutive lookups): the bags
// are found by binary search in LDS and all K row ids are loaded before any
// is used, so a thread keeps K loads in flight.  On batches of up to 2^20
// lookups the radix digits are counted too: the counts are kept in LDS across
// the workgroup's tiles and added to the global counts once at the end (a
// bounded grid keeps those global atomics, all on the same few hundred words,
// few), which must be zero before the first workgroup starts.
template <typename IT, int NT, int K, int BAGS = kLinBags>
__device__ __forceinline__ void linearize_tiles(const BackwardLaunch& a, int64_t first,
                                                int64_t stride) {
  static_assert(NT >= BAGS, "one thread per bag stages the offsets");
  __shared__ int64_t s_off[BAGS + 1];
  __shared__ uint32_t s_roff[BAGS];
  __shared__ float s_scale[BAGS];
  __shared__ uint32_t s_hist[kMaxRadixPasses << kMaxRadixBits];

  const int tid = threadIdx.x;
  // (counted passes take their digit counts themselves)
  const int passes = counted_passes(a.num_indices) ? 0 : radix_passes(a.key_bits, a.num_indices);
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
        slot[k] = tile_bag_slot(s_off, nb, p, p0, even, per);
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
          const uint64_t peers = match_bits(active, d, bits);
          if (ok[k] && popc_below(peers) == 0) atomicAdd(&s_hist[q * slots + d], __popcll(peers));
        }
      }
    }
  }
  __syncthreads();
  for (int i = tid; i < passes * slots; i += NT)
    if (s_hist[i]) atomicAdd(&a.buf.digit_hist[i], s_hist[i]);
}

// The linearize step for batches whose grouping takes the bucket-local sort
// (ids of two digits; the high digit is key >> lbits), with the tile's lookups
// also sorted by the high digit inside the tile's own positions.  Tile `tile`
// of kLinBags bags, lookups [p0, p1); wave w owns the consecutive positions
// [p0 + w*C, p0 + (w+1)*C) (C a multiple of 64), walked in steps of 64:
//   1. count: keys are computed (the first kStash steps' keys stay in
//      registers, their loads all issued at once) and each wave counts the
//      high digits of its positions in its own LDS counters (lanes with equal
//      digits matched by ballots, the lowest adds their number);
//   2. the tile's row of segment bounds goes out: row[d] = p0 + the number of
//      the tile's keys with a high digit below d (row[2^kMaxRadixBits] = p1),
//      and every wave's counter becomes its first position for that digit
//      (digits in order, waves in order within a digit);
//   3. place: each wave walks its positions again and writes every key to
//      buf.keys[1] / buf.vals[1] at its counter plus its rank among equal
//      digits in the step, which keeps lookup order within a digit (the
//      stashed steps keep their ranks from the count, so only later steps
//      match their digits again).
// Two barriers per tile; no workgroup waits for another, and nothing here
// needs cleared memory: tile 0 clears the counters and status words of the
// kernels that follow.  The bucket-local sort gathers a bucket's keys from the
// tiles' segments [row_i[d], row_i[d+1]) in tile order, which is lookup order.
template <typename IT, int NT>
__device__ __forceinline__ void linearize_bucket(const BackwardLaunch& a, int tile) {
  constexpr int NW = NT / kWave;
  constexpr int DIG = 1 << kMaxRadixBits;
  constexpr int DPT = DIG / NT;  // digits owned per thread
  constexpr int kStash = 8;      // steps whose keys stay in registers
  static_assert(DPT >= 1 && DPT * NT == DIG, "threads own whole digits");
  __shared__ int64_t s_off[kLinBags + 1];
  __shared__ uint32_t s_roff[kLinBags];
  __shared__ float s_scale[kLinBags];
  __shared__ __align__(16) uint32_t s_wc[NW][DIG];  // per-wave digit counts, then next positions
  __shared__ uint32_t scratch[NW];

  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const int lbits = radix_digit_bits(a.key_bits, a.num_indices);
  const int hbits = a.key_bits - lbits;
  const uint32_t hmask = (1u << hbits) - 1u;
  const int64_t k0 = static_cast<int64_t>(tile) * kLinBags;
  if (tile == 0) {
    // the counters and look-back status words of the later kernels (this
    // launch uses none of them, so no separate clearing launch is needed)
    const int64_t nvec = (static_cast<int64_t>(a.buf.sort_status - a.buf.counters) + 3) / 4;
    uint4* const z = reinterpret_cast<uint4*>(a.buf.counters);
    for (int64_t i = tid; i < nvec; i += NT) z[i] = make_uint4(0u, 0u, 0u, 0u);
  }
  const int nb = static_cast<int>(min(static_cast<int64_t>(kLinBags), a.num_bags - k0));
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
  {
    uint4* z = reinterpret_cast<uint4*>(&s_wc[0][0]);
    constexpr int NZ = static_cast<int>(sizeof(s_wc) / sizeof(uint4));
    for (int i = tid; i < NZ; i += NT) z[i] = make_uint4(0u, 0u, 0u, 0u);
  }
  __syncthreads();
  const int64_t p0 = s_off[0], p1 = s_off[nb];
  const bool even = p1 - p0 == static_cast<int64_t>(nb) * (s_off[1] - p0);
  const float per = even && p1 > p0 ? static_cast<float>(nb) / static_cast<float>(p1 - p0) : 0.0f;
  const int64_t C = ((p1 - p0 + NW - 1) / NW + kWave - 1) / kWave * kWave;
  const int64_t c0 = p0 + wave * C;                   // this wave's positions [c0, c1)
  const int64_t c1 = c0 + C < p1 ? c0 + C : p1;
  const int steps = c1 > c0 ? static_cast<int>((c1 - c0 + kWave - 1) / kWave) : 0;
  uint32_t* const wc = s_wc[wave];

  // key, bag slot and (with side records) the record of the lookup at p
  const auto lookup = [&](int64_t p, bool ok, uint32_t* key, int* slot) {
    *slot = ok ? tile_bag_slot(s_off, nb, p, p0, even, per) : 0;
    const int64_t x = ok ? lin_index<IT>(a.indices, p) : 0;
    *key = s_roff[*slot] + static_cast<uint32_t>(x);
  };
  const auto record = [&](int64_t p, int slot) {
    const float pw = a.psw ? a.psw[p] : 1.0f;
    a.buf.rec[p] = make_uint2(static_cast<uint32_t>(k0 + slot),
                              __float_as_uint(pw * s_scale[slot]));
  };
  // returns the lane's rank among equal digits in the step and their number
  // (rank | number << 8), which the place step of a stashed key reuses
  const auto count = [&](uint32_t key, bool ok) {
    const uint32_t d = (key >> lbits) & hmask;
    const uint64_t peers = match_bits(__ballot(ok), d, hbits);
    const uint32_t below = popc_below(peers), n = __popcll(peers);
    if (ok && below == 0) wc[d] += n;
    return below | (n << 8);
  };

  // 1. count (steps past kStash are read again when placed)
  // stashed steps: the key, and the bag slot (< kLinBags, bits 0-7) packed
  // with the rank and number that count returns (bits 8-23)
  uint32_t key[kStash], sr[kStash];
#pragma unroll
  for (int s = 0; s < kStash; ++s) {
    const int64_t p = c0 + s * kWave + lane;
    int sl;
    lookup(p, s < steps && p < c1, &key[s], &sl);
    sr[s] = static_cast<uint32_t>(sl);
  }
#pragma unroll
  for (int s = 0; s < kStash; ++s) {
    if (s >= steps) break;
    const int64_t p = c0 + s * kWave + lane;
    const bool ok = p < c1;
    if (a.use_rec && ok) record(p, static_cast<int>(sr[s]));
    sr[s] |= count(key[s], ok) << 8;
  }
  for (int s = kStash; s < steps; ++s) {
    const int64_t p = c0 + s * kWave + lane;
    const bool ok = p < c1;
    uint32_t kk;
    int sl;
    lookup(p, ok, &kk, &sl);
    if (a.use_rec && ok) record(p, sl);
    count(kk, ok);
  }
  __syncthreads();

  // 2. the tile's row of segment bounds, the global counts, each wave's first
  // position per digit
  const int d0 = tid * DPT;
  uint32_t c[DPT][NW], tot[DPT], tsum = 0;
#pragma unroll
  for (int q = 0; q < DPT; ++q) {
    tot[q] = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      c[q][w] = s_wc[w][d0 + q];
      tot[q] += c[q][w];
    }
    tsum += tot[q];
  }
  {
    uint32_t all;
    uint32_t st = static_cast<uint32_t>(p0) + block_excl_n<NW>(tsum, scratch, &all);
    uint32_t* const row = a.buf.tile_rows + static_cast<int64_t>(tile) * kTileRowWords;
#pragma unroll
    for (int q = 0; q < DPT; ++q) {
      row[d0 + q] = st;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        s_wc[w][d0 + q] = st;
        st += c[q][w];
      }
    }
    if (tid == 0) row[DIG] = static_cast<uint32_t>(p1);
  }
  __syncthreads();

  // 3. place
  uint32_t* const kout = a.buf.keys[1];
  uint32_t* const vout = a.buf.vals[1];
  // r: the lane's rank among equal digits in the step and their number, as
  // count returns them
  const auto place = [&](int64_t p, bool ok, uint32_t k, int sl, uint32_t r) {
    const uint32_t d = (k >> lbits) & hmask;
    const uint32_t below = r & 0xFFu;
    const uint32_t pre = ok ? wc[d] : 0u;
    if (ok && below == 0) wc[d] = pre + (r >> 8);
    if (ok) {
      // pre + below lies in [p0, p1): a digit's positions never pass its count
      kout[pre + below] = k;
      vout[pre + below] = a.use_rec ? static_cast<uint32_t>(p) : static_cast<uint32_t>(k0 + sl);
    }
  };
#pragma unroll
  for (int s = 0; s < kStash; ++s) {
    if (s >= steps) break;
    const int64_t p = c0 + s * kWave + lane;
    place(p, p < c1, key[s], static_cast<int>(sr[s] & 0xFFu), sr[s] >> 8);
  }
  for (int s = kStash; s < steps; ++s) {
    const int64_t p = c0 + s * kWave + lane;
    const bool ok = p < c1;
    uint32_t kk;
    int sl;
    lookup(p, ok, &kk, &sl);
    const uint32_t d = (kk >> lbits) & hmask;
    const uint64_t peers = match_bits(__ballot(ok), d, hbits);
    place(p, ok, kk, sl, popc_below(peers) | (static_cast<uint32_t>(__popcll(peers)) << 8));
  }
}

}  // namespace tbe
