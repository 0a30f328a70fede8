// sort.hip -- the grouping front of the TBE backward on gfx950: linearize the
// lookups to (table, row) ids, sort them with an LDS radix sort and
// run-length encode the sorted ids.
//
// kimbodo.com/?p=28372, "What Happened": updates are grouped by table and row
// so that each row gets one optimizer update; "Kimbodo Engineering
// Perspective": the grouping is a transpose, a sort and a run-length encoding.
//
//   init        zeroes the device counters, digit histograms and the status
//               words the passes below chain through.
//   linearize   key_i = roff_t + x_i (one 32-bit id space over all tables),
//               value_i = bag id k (plain sums) or lookup id i with a side
//               record {k, p_i * s_k} when lookups carry a coefficient.  On
//               batches of up to 2^20 lookups it also counts the digits of
//               every radix pass (these counts do not depend on the order of
//               the keys), so no look-back pass needs a counting kernel.
//   radix pass  one kernel per digit of a stable LSD radix sort on
//               ceil(log2(sum E_t)) bits, split evenly into the fewest digits
//               of at most 10 bits (20-bit ids: two 10-bit passes).  A tile
//               of keys is ranked in LDS (equal digits matched within a wave
//               through one ballot per digit bit, per-wave digit counters),
//               its digit counts are published and the tile's offset within
//               every digit bucket is found by a decoupled look-back over the
//               tiles before it; the tile is then written bucket by bucket so
//               global stores are coalesced.  Up to 8-bit digits: 256 threads
//               per tile; 9-10 bits: 1024 threads, so that every thread still
//               looks back for one digit.  Batches of more than 2^20 lookups
//               take counted passes instead: a kernel counts every tile's
//               digits, a second scans the counts over the tiles, and the pass
//               places each tile at its scanned offsets without a look-back.
//   RLE         one kernel: run heads of an 8192-key tile, a look-back over
//               the head counts of earlier tiles, then unique ids and run
//               starts.  The number of runs U stays on the device.
//
// A tile only waits for tiles numbered before it, which publish their counts
// before they wait themselves.  When the grid is small enough to be resident
// all at once, tiles are numbered by workgroup id; otherwise by an atomic
// ticket taken when a workgroup starts, so every tile waited for is running.
// Every wait is bounded: past a spin limit (set per handle) the workgroup
// raises an error flag and stops waiting, so no wave can hang; the segment
// kernels then update nothing and the handle is marked.
#include "common.hpp"
#include "linearize.hpp"
#include "lookback.hpp"

namespace tbe {
namespace {

constexpr int kResidentTiles = 256;         // grids this small are resident all at once
// keys per thread of a counted pass: 4096-key tiles, 36 KB of LDS, four
// workgroups per CU (8192-key tiles fit two per CU: passes 15-40% slower)
constexpr int kCountedKpt = 16;

template <typename IT>
__device__ __forceinline__ int64_t ld_index(const void* p, int64_t i) {
  return static_cast<int64_t>(static_cast<const IT*>(p)[i]);
}

// 16-byte stores: the zeroed region starts 256-byte aligned and its carve is
// rounded up to 256 bytes, so nvec = ceil(words / 4) stays inside it.
__global__ __launch_bounds__(kBlock) void init_workspace(uint4* words, int64_t nvec) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; i < nvec;
       i += static_cast<int64_t>(gridDim.x) * kBlock)
    words[i] = make_uint4(0u, 0u, 0u, 0u);
}

// K lookups in flight per thread: 2 when a tile holds more lookups than the
// workgroup has threads, else 1 (short bags would leave half the slots idle).
template <typename IT, int K, int BAGS>
__global__ __launch_bounds__(kLinThreads) void linearize_kernel(BackwardLaunch a) {
  linearize_tiles<IT, kLinThreads, K, BAGS>(a, blockIdx.x, gridDim.x);
}

// The same with each tile's lookups sorted by the high digit: one workgroup per tile.
template <typename IT>
__global__ __launch_bounds__(kLinThreads) void linearize_bucket_kernel(BackwardLaunch a) {
  linearize_bucket<IT, kLinThreads>(a, blockIdx.x);
}

// Lanes of the wave (among those with ok) whose digit d equals this lane's.
// Each lane sets its bit in the LDS slot chosen by the low 8 bits of d and
// reads the slot back; lanes that share the slot but differ in the digit's
// higher bits (at most RB - 8 of them) are removed with one ballot per bit.
// The slot is cleared again for the next round.  Replaces RB ballots per
// round by one LDS atomic, one read and RB - 8 ballots: used for 9- and
// 10-bit digits (for 8-bit digits the LDS round trip costs more than the
// ballots it saves).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int RB>
__device__ __forceinline__ uint64_t match_digit(uint64_t* s_slots, uint32_t d, bool ok) {
  // Lanes holding the first active lane's digit are matched by one ballot: a
  // hot row fills whole rounds with one digit, and atomics of all of its
  // lanes on one slot would be serialised.  The other lanes use the slots.
  const uint64_t act = __ballot(ok);
  if (act == 0) return 0;
  const uint32_t d0 = static_cast<uint32_t>(
      __builtin_amdgcn_readlane(static_cast<int>(d), __builtin_ctzll(act)));
  const bool same = ok && d == d0;
  const uint64_t m0 = __ballot(same);
  if (m0 == act) return same ? m0 : 0u;
  const bool rest = ok && !same;
  uint64_t* slot = s_slots + (d & 255u);
  if (rest)
    __hip_atomic_fetch_or(slot, uint64_t{1} << lane_id(), __ATOMIC_RELAXED,
                          __HIP_MEMORY_SCOPE_WAVEFRONT);
  wave_lds_sync();
  uint64_t peers = rest ? __hip_atomic_load(slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT) : 0u;
  wave_lds_sync();
  if (rest) __hip_atomic_store(slot, uint64_t{0}, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
  if constexpr (RB > 8) peers = match_low_bits(peers, d >> 8, RB - 8);
  return same ? m0 : peers;
}

// One LSD pass on the digit (key >> shift) & (2^bits - 1), bits <= RB.  A
// tile of 256*KPT keys; thread tid owns the DPT = 2^RB / 256 consecutive
// digits tid*DPT .. tid*DPT + DPT - 1 for counting, look-back and offsets.
// COUNTED: the tile's offset inside every digit bucket is read from
// status[d * ntiles + tile] (the exclusive prefix over earlier tiles that
// radix_count and radix_scan left there) instead of being found by a
// look-back, so no tile waits for another.
template <int KPT, int RB, bool COUNTED = false>
__global__ __launch_bounds__(kBlock) void radix_pass(
    const uint32_t* __restrict__ kin, const uint32_t* __restrict__ vin, uint32_t* __restrict__ kout,
    uint32_t* __restrict__ vout, int64_t n, int shift, int bits, const uint32_t* __restrict__ totals,
    uint32_t* status, uint32_t* ticket, WaitCtl wait, uint32_t* wtable) {
  constexpr int TS = kBlock * KPT;
  constexpr int RMAX = 1 << RB;
  constexpr int DPT = RMAX / kBlock;
  constexpr int DEPTH = DPT == 1 ? 16 : (DPT == 2 ? 8 : 4);
  __shared__ uint32_t s_k[TS];
  __shared__ uint32_t s_v[TS];
  __shared__ uint32_t s_cnt[kWavesPerBlock][RMAX];
  __shared__ uint32_t s_dstart[RMAX];
  __shared__ uint32_t s_gbase[RMAX];
  __shared__ uint32_t scratch[kWavesPerBlock];
  __shared__ uint32_t s_tile;

  // (no early exit on an earlier failure: every write below is clamped in range,
  // and a failed call is reported by the kernels after the sort)
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const int d0 = tid * DPT;
  const int ntiles = static_cast<int>((n + TS - 1) / TS);
  uint32_t my_total[DPT], before[DPT];  // issued with the key loads below
#pragma unroll
  for (int q = 0; q < DPT; ++q) {
    my_total[q] = totals[d0 + q];
    before[q] = 0u;
    if constexpr (COUNTED) before[q] = status[static_cast<int64_t>(d0 + q) * ntiles + blockIdx.x];
  }
  if (tid == 0) s_tile = (ticket && !COUNTED) ? atomicAdd(ticket, 1u) : blockIdx.x;
  for (int i = tid; i < kWavesPerBlock * RMAX; i += kBlock) (&s_cnt[0][0])[i] = 0u;
  __syncthreads();
  const int tile = static_cast<int>(s_tile);
  const int64_t base = static_cast<int64_t>(tile) * TS;
  const uint32_t dmask = (1u << bits) - 1u;

  // rank: wave w owns tile positions [w*64*KPT, (w+1)*64*KPT), ranked in KPT
  // rounds of 64 consecutive keys, so equal digits keep their input order
  const int64_t seg = base + static_cast<int64_t>(wave) * (kWave * KPT);
  uint32_t key[KPT], val[KPT], rank[KPT];
#pragma unroll
  for (int r = 0; r < KPT; ++r) {
    const int64_t p = seg + r * kWave + lane;
    const bool ok = p < n;
    key[r] = ok ? kin[p] : 0u;
    val[r] = ok ? vin[p] : 0u;
  }
#pragma unroll
  for (int r = 0; r < KPT; ++r) {
    const bool ok = (seg + r * kWave + lane) < n;
    const uint32_t d = (key[r] >> shift) & dmask;
    // (bits above `bits` are 0 everywhere: matching them changes nothing)
    const uint64_t peers = match_low_bits(__ballot(ok), d, RB);
    const uint32_t below = popc_below(peers);
    const uint32_t cnt = __popcll(peers);
    const uint32_t pre = ok ? s_cnt[wave][d] : 0u;
    rank[r] = pre + below;
    if (ok && below == 0) s_cnt[wave][d] = pre + cnt;
  }
  __syncthreads();

  // per owned digit: wave offsets, tile-local bucket starts, and the tile's
  // offset inside the global bucket
  uint32_t mine[DPT], loc[DPT], tsum = 0;
#pragma unroll
  for (int q = 0; q < DPT; ++q) {
    const int d = d0 + q;
    const uint32_t c0 = s_cnt[0][d], c1 = s_cnt[1][d], c2 = s_cnt[2][d], c3 = s_cnt[3][d];
    mine[q] = c0 + c1 + c2 + c3;
    s_cnt[0][d] = 0u;
    s_cnt[1][d] = c0;
    s_cnt[2][d] = c0 + c1;
    s_cnt[3][d] = c0 + c1 + c2;
    loc[q] = tsum;
    tsum += mine[q];
  }
  uint32_t total;
  const uint32_t tbase = block_exclusive_sum(tsum, scratch, &total);
  uint32_t* my_status = status + static_cast<int64_t>(tile) * RMAX + d0;
#pragma unroll
  for (int q = 0; q < DPT; ++q) {
    s_dstart[d0 + q] = tbase + loc[q];
    if constexpr (!COUNTED) st_status(my_status + q, (tile == 0 ? kFlagIncl : kFlagAgg) | mine[q]);
  }
  if (!COUNTED && tile > 0) {
    lookback_digits<DPT, DEPTH>(status, RMAX, tile, d0, wait, before);
#pragma unroll
    for (int q = 0; q < DPT; ++q)
      st_status(my_status + q, kFlagIncl | ((before[q] + mine[q]) & kValueMask));
  }
  uint32_t gsum = 0, gloc[DPT];
#pragma unroll
  for (int q = 0; q < DPT; ++q) gloc[q] = gsum, gsum += my_total[q];
  const uint32_t gbase = block_exclusive_sum(gsum, scratch, &total);
#pragma unroll
  for (int q = 0; q < DPT; ++q) s_gbase[d0 + q] = gbase + gloc[q] + before[q];
  if (wtable) {  // every tile knows all bucket starts; digit d is recorded by tile d % tiles
#pragma unroll
    for (int q = 0; q < DPT; ++q)
      if (my_total[q] > 0 && (d0 + q) % ntiles == tile)
        record_window(wtable, gbase + gloc[q], my_total[q], d0 + q);
  }
  __syncthreads();

#pragma unroll
  for (int r = 0; r < KPT; ++r) {
    const bool ok = (seg + r * kWave + lane) < n;
    if (ok) {
      const uint32_t d = (key[r] >> shift) & dmask;
      const uint32_t lp = s_dstart[d] + s_cnt[wave][d] + rank[r];
      s_k[lp] = key[r];
      s_v[lp] = val[r];
    }
  }
  __syncthreads();
  const int tile_n = static_cast<int>(min(static_cast<int64_t>(TS), n - base));
  for (int i = tid; i < tile_n; i += kBlock) {
    const uint32_t k = s_k[i];
    const uint32_t d = (k >> shift) & dmask;
    const uint32_t gp = s_gbase[d] + (static_cast<uint32_t>(i) - s_dstart[d]);
    if (gp < static_cast<uint64_t>(n)) {  // always true unless a look-back gave up
      kout[gp] = k;
      vout[gp] = s_v[i];
    }
  }
}

// Counted passes (batches of more than 2^20 lookups, digits of at most 8
// bits): every tile's digit counts are taken by radix_count, scanned over the
// tiles by radix_scan, and radix_pass<.., COUNTED> then places each tile at
// its scanned offsets.  The counts cost one more read of the keys (4 bytes a
// lookup); in exchange no tile waits for the tiles before it (with 512 tiles
// resident at once, the look-back's chain of status words took a third of a
// tile's time).
//
// radix_count: tile `tile` (kBlock*KPT keys, the tiles of radix_pass) counts
// the digits of its keys into cnt[d * ntiles + tile].  Lanes holding the
// first active lane's digit add their number once (a hot row fills whole
// rounds with one digit); the others add one each.  Workgroups are renumbered
// XCD by XCD so that the counts of neighbouring tiles are written from one L2.
template <int KPT>
__global__ __launch_bounds__(kBlock) void radix_count(const uint32_t* __restrict__ kin, int64_t n,
                                                      int shift, int bits,
                                                      uint32_t* __restrict__ cnt, int ntiles) {
  __shared__ uint32_t s_c[kBlock];
  const int tid = threadIdx.x;
  const int tile = xcd_contiguous_block(blockIdx.x, gridDim.x);
  s_c[tid] = 0u;
  const int64_t base = static_cast<int64_t>(tile) * (kBlock * KPT);
  const uint32_t dmask = (1u << bits) - 1u;
  uint32_t key[KPT];
#pragma unroll
  for (int r = 0; r < KPT; ++r) {
    const int64_t p = base + r * kBlock + tid;
    key[r] = p < n ? kin[p] : 0u;
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < KPT; ++r) {
    const bool ok = base + r * kBlock + tid < n;
    const uint32_t d = (key[r] >> shift) & dmask;
    const uint64_t act = __ballot(ok);
    if (act == 0) continue;  // the same on the whole wave
    const uint32_t dl = static_cast<uint32_t>(
        __builtin_amdgcn_readlane(static_cast<int>(d), __builtin_ctzll(act)));
    const bool same = ok && d == dl;
    const uint64_t m = __ballot(same);
    if (same && popc_below(m) == 0) atomicAdd(&s_c[dl], static_cast<uint32_t>(__popcll(m)));
    if (ok && !same) atomicAdd(&s_c[d], 1u);
  }
  __syncthreads();
  cnt[static_cast<int64_t>(tid) * ntiles + tile] = s_c[tid];
}

// radix_scan: workgroup d turns cnt[d * ntiles + t] into the exclusive prefix
// over tiles t' < t and writes the digit's total to totals[d].
__global__ __launch_bounds__(kBlock) void radix_scan(uint32_t* __restrict__ cnt, int ntiles,
                                                     uint32_t* __restrict__ totals) {
  __shared__ uint32_t scratch[kWavesPerBlock];
  uint32_t* col = cnt + static_cast<int64_t>(blockIdx.x) * ntiles;
  uint32_t carry = 0;
  for (int t0 = 0; t0 < ntiles; t0 += kBlock * 4) {
    uint32_t c[4], s = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = t0 + threadIdx.x * 4 + j;
      c[j] = t < ntiles ? col[t] : 0u;
      s += c[j];
    }
    uint32_t total;
    uint32_t run = carry + block_exclusive_sum(s, scratch, &total);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = t0 + threadIdx.x * 4 + j;
      if (t < ntiles) col[t] = run;
      run += c[j];
    }
    carry += total;
  }
  if (threadIdx.x == 0) totals[blockIdx.x] = carry;
}

// A pass on digits wider than 8 bits: 1024 threads, one digit per thread
// (2^RB = 1024 digits), so the look-back keeps 16 status words in flight per
// digit as in the 8-bit pass.
template <int KPT, int RB>
__global__ __launch_bounds__(1024) void radix_pass_wide(
    const uint32_t* __restrict__ kin, const uint32_t* __restrict__ vin, uint32_t* __restrict__ kout,
    uint32_t* __restrict__ vout, int64_t n, int shift, int bits, const uint32_t* __restrict__ totals,
    uint32_t* status, uint32_t* ticket, WaitCtl wait, uint32_t* wtable) {
  constexpr int NT = 1024, NW = NT / kWave;
  constexpr int TS = NT * KPT;
  constexpr int RMAX = 1 << RB;
  static_assert(RMAX == NT, "one digit per thread");
  __shared__ uint32_t s_k[TS];
  __shared__ uint32_t s_v[TS];
  __shared__ uint32_t s_cnt[NW][RMAX];
  __shared__ uint64_t s_slots[NW][256];
  __shared__ uint32_t s_dstart[RMAX];
  __shared__ uint32_t s_gbase[RMAX];
  __shared__ uint32_t scratch[NW];
  __shared__ uint32_t s_tile;

  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const uint32_t my_total = totals[tid];
  if (tid == 0) s_tile = ticket ? atomicAdd(ticket, 1u) : blockIdx.x;
  for (int i = tid; i < NW * RMAX; i += NT) (&s_cnt[0][0])[i] = 0u;
  for (int i = tid; i < NW * 256; i += NT) (&s_slots[0][0])[i] = 0u;
  __syncthreads();
  const int tile = static_cast<int>(s_tile);
  const int64_t base = static_cast<int64_t>(tile) * TS;
  const uint32_t dmask = (1u << bits) - 1u;
  const int64_t seg = base + static_cast<int64_t>(wave) * (kWave * KPT);
  uint32_t key[KPT], val[KPT], rank[KPT];
#pragma unroll
  for (int r = 0; r < KPT; ++r) {
    const int64_t p = seg + r * kWave + lane;
    const bool ok = p < n;
    key[r] = ok ? kin[p] : 0u;
    val[r] = ok ? vin[p] : 0u;
  }
#pragma unroll
  for (int r = 0; r < KPT; ++r) {
    const bool ok = (seg + r * kWave + lane) < n;
    const uint32_t d = (key[r] >> shift) & dmask;
    const uint64_t peers = match_digit<RB>(s_slots[wave], d, ok);
    const uint32_t below = popc_below(peers);
    const uint32_t cnt = __popcll(peers);
    const uint32_t pre = ok ? s_cnt[wave][d] : 0u;
    rank[r] = pre + below;
    if (ok && below == 0) s_cnt[wave][d] = pre + cnt;
  }
  __syncthreads();
  // this digit's count per wave (all read before any is rewritten: one LDS
  // round trip), then the waves' offsets inside the tile's bucket
  uint32_t c[NW];
#pragma unroll
  for (int w = 0; w < NW; ++w) c[w] = s_cnt[w][tid];
  uint32_t mine = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    s_cnt[w][tid] = mine;
    mine += c[w];
  }
  uint32_t total;
  s_dstart[tid] = block_excl_n<NW>(mine, scratch, &total);
  uint32_t* my_status = status + static_cast<int64_t>(tile) * RMAX + tid;
  st_status(my_status, (tile == 0 ? kFlagIncl : kFlagAgg) | mine);
  // the bucket's global start does not depend on the look-back
  const uint32_t gb = block_excl_n<NW>(my_total, scratch, &total);
  // every tile knows all bucket starts; digit d is recorded by tile d % tiles
  if (wtable && my_total > 0 && tid % static_cast<int>((n + TS - 1) / TS) == tile)
    record_window(wtable, gb, my_total, tid);
  uint32_t before[1] = {0u};
  if (tile > 0) {
    lookback_digits<1, 16>(status, RMAX, tile, tid, wait, before);
    st_status(my_status, kFlagIncl | ((before[0] + mine) & kValueMask));
  }
  s_gbase[tid] = gb + before[0];
  __syncthreads();
#pragma unroll
  for (int r = 0; r < KPT; ++r) {
    const bool ok = (seg + r * kWave + lane) < n;
    if (ok) {
      const uint32_t d = (key[r] >> shift) & dmask;
      const uint32_t lp = s_dstart[d] + s_cnt[wave][d] + rank[r];
      s_k[lp] = key[r];
      s_v[lp] = val[r];
    }
  }
  __syncthreads();
  const int tile_n = static_cast<int>(min(static_cast<int64_t>(TS), n - base));
  for (int i = tid; i < tile_n; i += NT) {
    const uint32_t k = s_k[i];
    const uint32_t d = (k >> shift) & dmask;
    const uint32_t gp = s_gbase[d] + (static_cast<uint32_t>(i) - s_dstart[d]);
    if (gp < static_cast<uint64_t>(n)) {
      kout[gp] = k;
      vout[gp] = s_v[i];
    }
  }
}

__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
#pragma unroll
  for (int o = kWave >> 1; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Sum of the values of all tiles before `tile` (one status word per tile; a
// whole wave reads 64 predecessors at once).  A wait that gives up returns at
// most the true sum.
__device__ uint32_t lookback_wave(uint32_t* status, int tile, WaitCtl wait) {
  const int lane = lane_id();
  uint32_t excl = 0;
  int j = tile - 1;
  if (wait.limit == 0u) {
    if (lane == 0) atomicOr(wait.err, 1u);
    return 0u;
  }
  uint32_t spins = 0;
  while (true) {
    const int idx = j - lane;
    const uint32_t w = idx >= 0 ? ld_status(status + idx) : kFlagIncl;
    const uint32_t f = w & ~kValueMask;
    const uint64_t not_ready = __ballot(f == 0);
    const uint64_t incl = __ballot(f == kFlagIncl);
    const int first_nr = not_ready ? __builtin_ctzll(not_ready) : kWave;
    const int first_in = incl ? __builtin_ctzll(incl) : kWave;
    const int take = first_in < first_nr ? first_in + 1 : first_nr;
    excl += wave_sum_u32(lane < take ? (w & kValueMask) : 0u);
    if (first_in < first_nr) return excl;
    j -= take;
    if (take == 0) {
      if (++spins > wait.limit) {
        if (lane == 0) atomicOr(wait.err, 1u);
        return excl;
      }
      __builtin_amdgcn_s_sleep(2);
    }
  }
}

// Counted run-length encoding (batches of more than 2^20 lookups): the run
// heads of every 8192-key tile are counted first (rle_count), the counts are
// scanned over the tiles (radix_scan on one column), and rle_kernel<true>
// then writes each tile's runs at its scanned run id, with no look-back.
//
// rle_count: heads of tile blockIdx.x (p == 0 or keys[p] != keys[p - 1]);
// each thread owns 8 consecutive positions.
__global__ __launch_bounds__(1024) void rle_count(const uint32_t* __restrict__ keys, int64_t n,
                                                  uint32_t* __restrict__ cnt) {
  constexpr int NT = 1024;
  constexpr int PER = kRleTile / NT;
  __shared__ uint32_t scratch[NT / kWave];
  const int tid = threadIdx.x;
  const int64_t p0 = static_cast<int64_t>(blockIdx.x) * kRleTile + tid * PER;
  uint32_t k[PER + 1];
  k[0] = (p0 > 0 && p0 - 1 < n) ? keys[p0 - 1] : 0u;
  if (p0 + PER <= n) {
    const uint4 a = *reinterpret_cast<const uint4*>(keys + p0);
    const uint4 b = *reinterpret_cast<const uint4*>(keys + p0 + 4);
    k[1] = a.x, k[2] = a.y, k[3] = a.z, k[4] = a.w, k[5] = b.x, k[6] = b.y, k[7] = b.z, k[8] = b.w;
  } else {
#pragma unroll
    for (int j = 0; j < PER; ++j) k[j + 1] = p0 + j < n ? keys[p0 + j] : 0u;
  }
  uint32_t c = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int64_t p = p0 + j;
    if (p < n && (p == 0 || k[j + 1] != k[j])) ++c;
  }
  uint32_t total;
  (void)block_excl_n<NT / kWave>(c, scratch, &total);
  if (tid == 0) cnt[blockIdx.x] = total;
}

// Run heads of an 8192-key tile (staged in LDS with the key before it), 1024
// threads per tile; each thread owns 8 consecutive positions so run ids
// follow position order.  The tile's first run id comes from a look-back over
// the earlier tiles' head counts, or (COUNTED) from cnt[tile], their scan.
template <bool COUNTED>
__global__ __launch_bounds__(1024) void rle_kernel(const uint32_t* __restrict__ keys,
                                                     const uint32_t* __restrict__ vals, int64_t n,
                                                     int ntiles, uint32_t* status, uint32_t* ticket,
                                                     uint32_t* counters, uint32_t* unique_keys,
                                                     uint32_t* run_start, uint32_t* run_first,
                                                     int fstride, uint32_t spin_limit) {
  constexpr int NT = 1024;
  constexpr int PER = kRleTile / NT;
  __shared__ uint32_t s_k[kRleTile + 1];
  __shared__ uint32_t scratch[NT / kWave];
  __shared__ uint32_t s_tile, s_base;
  const int tid = threadIdx.x;  // every write below is clamped in range
  if (tid == 0) s_tile = (ticket && !COUNTED) ? atomicAdd(ticket, 1u) : blockIdx.x;
  __syncthreads();
  const int tile = static_cast<int>(s_tile);
  const int64_t base = static_cast<int64_t>(tile) * kRleTile;
  {
    // s_k[i] = keys[base - 1 + i]; the PER loads of a thread are all issued
    // before any is stored
    uint32_t v[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int64_t p = base + j * NT + tid;
      v[j] = p < n ? keys[p] : 0u;
    }
    if (tid == 0) s_k[0] = (base > 0 && base - 1 < n) ? keys[base - 1] : 0u;
#pragma unroll
    for (int j = 0; j < PER; ++j) s_k[1 + j * NT + tid] = v[j];
  }
  __syncthreads();
  uint32_t c = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = tid * PER + j;
    const int64_t p = base + i;
    if (p < n && (p == 0 || s_k[i + 1] != s_k[i])) ++c;
  }
  uint32_t total;
  uint32_t r = block_excl_n<NT / kWave>(c, scratch, &total);
  if (tid < kWave) {
    uint32_t before = 0;
    if constexpr (COUNTED) {
      before = status[tile];
    } else {
      if (tid == 0) st_status(status + tile, (tile == 0 ? kFlagIncl : kFlagAgg) | total);
      if (tile > 0) before = lookback_wave(status, tile, WaitCtl{counters + kCntError, spin_limit});
    }
    if (tid == 0) {
      if (!COUNTED && tile > 0) st_status(status + tile, kFlagIncl | ((before + total) & kValueMask));
      s_base = before;
      if (tile == ntiles - 1) {
        // U <= n always, unless a look-back gave up; keep every index in range regardless
        const uint32_t U = min(before + total, static_cast<uint32_t>(n));
        counters[kCntUnique] = U;
        run_start[U] = static_cast<uint32_t>(n);
      }
    }
  }
  __syncthreads();
  r += s_base;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = tid * PER + j;
    const int64_t p = base + i;
    if (p < n && (p == 0 || s_k[i + 1] != s_k[i])) {
      if (r < static_cast<uint64_t>(n)) {
        unique_keys[r] = s_k[i + 1];
        run_start[r] = static_cast<uint32_t>(p);
        for (int q = 0; q < fstride; ++q)
          run_first[static_cast<int64_t>(r) * fstride + q] = p + q < n ? vals[p + q] : 0u;
      }
      ++r;
    }
  }
}


// ---------------------------------------------------------------------------
// Ids of two digits: one look-back pass on the HIGH digit, then a
// bucket-local sort and run-length encoding.
//
// After a stable pass on the high digit every bucket holds whole runs (equal
// ids share their high digit), so the rest of the sort and the run heads are
// local to a bucket.  A window of kBucketWindow sorted positions takes the
// buckets that start inside it (each bucket belongs to exactly one window);
// its range of whole buckets is sorted in LDS by two stable counting passes
// (low digit, then bucket), which leaves the ids in the order of the two LSD
// passes (stable on the full id).  The range's run heads are counted, the
// range's first run id comes from a look-back over the earlier windows' run
// counts, and unique ids and run starts are written.  This replaces the
// second look-back pass and the RLE kernel.  Ranges longer than kBucketCap
// (a bucket of more than kBucketCap - kBucketWindow lookups) are sorted
// bucket by bucket in chunks of kBucketCap through global memory.

constexpr int kBucketThreads = 1024;
constexpr int kBucketWaves = kBucketThreads / kWave;
constexpr int kBucketKpt = 8;
constexpr int kBucketCap = kBucketThreads * kBucketKpt;
constexpr int64_t kBucketMeanMax = 1024;  // largest mean bucket the path is used for

// One stable counting pass in LDS over elements held in registers: wave w
// holds relative positions [w*64*rr, (w+1)*64*rr), round r of lane l position
// q = w*64*rr + r*64 + l, and the elements with qlo <= q < qhi take part
// (qhi - qlo <= kBucketCap); digit(key) < 1024.  Afterwards s_k/s_v hold
// those elements in digit order (position order among equal digits) at
// 0 .. qhi - qlo - 1, and s_dstart[d] is the first position of digit d.
// s_cnt must be zero on entry and is zero again on return (after a barrier of
// the caller).
template <typename Digit>
__device__ __forceinline__ void lds_counting_pass(const uint32_t (&key)[kBucketKpt],
                                                  const uint32_t (&val)[kBucketKpt], int rr,
                                                  int qlo, int qhi, Digit digit, uint32_t* s_k,
                                                  uint32_t* s_v,
                                                  uint16_t (*s_cnt)[kBucketThreads],
                                                  uint64_t (*s_slots)[256], uint32_t* s_dstart,
                                                  uint32_t* scratch) {
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const int wseg = wave * kWave * rr;
  uint32_t rank[kBucketKpt];
#pragma unroll
  for (int r = 0; r < kBucketKpt; ++r) {
    rank[r] = 0u;
    if (r < rr) {
      const int q = wseg + r * kWave + lane;
      const bool ok = q >= qlo && q < qhi;
      const uint32_t d = ok ? digit(key[r]) : 0u;
      const uint64_t peers = match_digit<10>(s_slots[wave], d, ok);
      const uint32_t below = popc_below(peers);
      const uint32_t pre = ok ? static_cast<uint32_t>(s_cnt[wave][d]) : 0u;
      rank[r] = pre + below;
      if (ok && below == 0) s_cnt[wave][d] = static_cast<uint16_t>(pre + __popcll(peers));
    }
  }
  __syncthreads();
  // digit tid: the waves' offsets inside the digit, then the digit's start
  // (waves past the last element hold no counts)
  const int nwa = (qhi + kWave * rr - 1) / (kWave * rr);
  uint32_t c[kBucketWaves];
#pragma unroll
  for (int w = 0; w < kBucketWaves; ++w) c[w] = w < nwa ? s_cnt[w][tid] : 0u;
  uint32_t mine = 0;
#pragma unroll
  for (int w = 0; w < kBucketWaves; ++w) {
    if (w < nwa) s_cnt[w][tid] = static_cast<uint16_t>(mine);
    mine += c[w];
  }
  uint32_t total;
  s_dstart[tid] = block_excl_n<kBucketWaves>(mine, scratch, &total);
  __syncthreads();
#pragma unroll
  for (int r = 0; r < kBucketKpt; ++r) {
    const int q = wseg + r * kWave + lane;
    if (r < rr && q >= qlo && q < qhi) {
      const uint32_t d = digit(key[r]);
      const uint32_t lp = s_dstart[d] + s_cnt[wave][d] + rank[r];
      s_k[lp] = key[r];
      s_v[lp] = val[r];
    }
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kBucketWaves; ++w)
    if (w < nwa) s_cnt[w][tid] = 0;
}

// Stable partition of the elements held in registers (the layout of
// lds_counting_pass, positions [0, len)) by their bucket b = bucket(key) < nb
// <= 64, into s_k / s_v, bucket b starting at bstart(b).  Each wave counts
// its elements per bucket (lanes with equal buckets matched by ballots); lane
// b of a wave then adds the counts of the earlier waves to bstart(b), and
// every element takes that base plus its rank.  Two barriers, against five
// for a counting pass over 1024 digits.  s_pc must be zero on entry (the
// caller clears it before a barrier); the caller's elements must all have
// been read out of s_k / s_v before the call.
template <typename Bucket, typename Start>
__device__ __forceinline__ void bucket_partition(const uint32_t (&key)[kBucketKpt],
                                                 const uint32_t (&val)[kBucketKpt], int rr,
                                                 int len, int nb, Bucket bucket, Start bstart,
                                                 uint32_t* s_k, uint32_t* s_v,
                                                 uint32_t (*s_pc)[64]) {
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int wseg = wave * kWave * rr;
  const int bits = nb <= 1 ? 0 : 32 - __clz(nb - 1);
  uint32_t rank[kBucketKpt], bk[kBucketKpt];
#pragma unroll
  for (int r = 0; r < kBucketKpt; ++r) {
    rank[r] = 0u;
    bk[r] = 0u;
    if (r < rr) {
      const bool ok = wseg + r * kWave + lane < len;
      bk[r] = ok ? bucket(key[r]) : 0u;
      const uint64_t peers = match_bits(__ballot(ok), bk[r], bits);
      const uint32_t below = popc_below(peers);
      const uint32_t pre = ok ? s_pc[wave][bk[r]] : 0u;
      rank[r] = pre + below;
      if (ok && below == 0) s_pc[wave][bk[r]] = pre + __popcll(peers);
    }
  }
  __syncthreads();
  uint32_t base = 0;
  if (lane < nb) {
    base = bstart(lane);
    for (int w = 0; w < wave; ++w) base += s_pc[w][lane];
  }
#pragma unroll
  for (int r = 0; r < kBucketKpt; ++r) {
    if (r < rr) {
      const uint32_t pos = __shfl(base, static_cast<int>(bk[r]), kWave) + rank[r];
      if (wseg + r * kWave + lane < len) {
        s_k[pos] = key[r];
        s_v[pos] = val[r];
      }
    }
  }
  __syncthreads();
}

// Load positions [start, start + len) (len <= kBucketCap) into registers in
// the layout of lds_counting_pass.
__device__ __forceinline__ void load_range(const uint32_t* kin, const uint32_t* vin, int64_t start,
                                           int len, int rr, uint32_t (&key)[kBucketKpt],
                                           uint32_t (&val)[kBucketKpt]) {
  const int wseg = (threadIdx.x >> 6) * kWave * rr;
#pragma unroll
  for (int r = 0; r < kBucketKpt; ++r) {
    const int p = wseg + r * kWave + lane_id();
    const bool ok = r < rr && p < len;
    key[r] = ok ? kin[start + p] : 0u;
    val[r] = ok ? vin[start + p] : 0u;
  }
}

// Queue a run of len > q.short_max lookups starting at sorted position s:
// one medium item, or the long-run record and one item per 256-lookup chunk.
// Only a small share of runs is this long, so each is queued on its own.
__device__ __forceinline__ void queue_run(const RunQueue& q, uint32_t* counters, uint32_t s,
                                          uint32_t len, uint32_t key) {
  if (len >= static_cast<uint32_t>(q.long_threshold)) {
    const uint32_t n1 = (len + q.chunk - 1) / q.chunk;
    const uint32_t li = atomicAdd(&counters[kCntLong], 1u);
    const uint32_t b1 = atomicAdd(&counters[kCntChunks], n1);
    const uint32_t it = atomicAdd(&counters[kCntItems1], n1);
    q.longs[li] = make_uint4(s, len, b1, n1);
    q.long_keys[li] = key;
    if (n1 >= kFinPieceMin) atomicOr(&counters[kCntPieced], 1u);
    for (uint32_t c = 0; c < n1; ++c) q.items1[it + c] = make_uint2(li, c);
  } else {
    const uint32_t it = atomicAdd(&counters[kCntItems1], 1u);
    q.items1[it] = make_uint2(s, kMediumItem | len);
  }
}

// Keys sorted by the high digit inside each linearize tile (linearize_bucket)
// are read through a segment table: for the buckets [b0, b1), tile i's keys
// lie at [rows_i[b0], rows_i[b1]); concatenated in tile order they are in
// lookup order within each bucket.  s_segoff[i] is the first element of
// segment i in the concatenation, s_seglo[i] its first position in the keys.
// Contains barriers: call from the whole workgroup.
__device__ __forceinline__ void build_segments(const uint32_t* rows, int nseg, uint32_t b0,
                                               uint32_t b1, uint32_t* s_seglo,
                                               uint32_t* s_segoff, uint32_t* scratch) {
  const int tid = threadIdx.x;
  uint32_t len = 0;
  if (tid < nseg) {
    const uint32_t lo = rows[static_cast<int64_t>(tid) * kTileRowWords + b0];
    const uint32_t hi = rows[static_cast<int64_t>(tid) * kTileRowWords + b1];
    s_seglo[tid] = lo;
    len = hi - lo;
  }
  uint32_t total;
  const uint32_t off = block_excl_n<kBucketWaves>(len, scratch, &total);
  if (tid < nseg) s_segoff[tid] = off;
  __syncthreads();
}

// Position in the keys of element e of the concatenated segments (the last
// segment i with s_segoff[i] <= e; an empty segment shares its offset with the
// next one, so the one found holds element e).
__device__ __forceinline__ uint32_t seg_position(const uint32_t* s_seglo, const uint32_t* s_segoff,
                                                 int nseg, uint32_t e) {
  int lo = 0, hi = nseg;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (s_segoff[mid] <= e)
      lo = mid;
    else
      hi = mid;
  }
  return s_seglo[lo] + (e - s_segoff[lo]);
}

// Elements [e0, e0 + len) of the concatenated segments (len <= kBucketCap)
// into registers in the layout of lds_counting_pass; every load is issued
// before any is used, and positions past n read nothing.
__device__ __forceinline__ void gather_range(const uint32_t* kin, const uint32_t* vin, int64_t n,
                                             const uint32_t* s_seglo, const uint32_t* s_segoff,
                                             int nseg, uint32_t e0, int len, int rr,
                                             uint32_t (&key)[kBucketKpt],
                                             uint32_t (&val)[kBucketKpt]) {
  const int wseg = (threadIdx.x >> 6) * kWave * rr;
  uint32_t pos[kBucketKpt];
#pragma unroll
  for (int r = 0; r < kBucketKpt; ++r) {
    const int e = wseg + r * kWave + lane_id();
    pos[r] = (r < rr && e < len) ? seg_position(s_seglo, s_segoff, nseg, e0 + e) : 0xFFFFFFFFu;
  }
#pragma unroll
  for (int r = 0; r < kBucketKpt; ++r) {
    const bool ok = pos[r] < static_cast<uint64_t>(n);
    key[r] = ok ? kin[pos[r]] : 0u;
    val[r] = ok ? vin[pos[r]] : 0u;
  }
}

// SEG: the keys come sorted by the high digit inside each linearize tile
// (rows: the tiles' segment bounds, nseg tiles); each window finds its range
// from the high digit's counts and gathers it from the segments.  Otherwise
// they come from the pass on the high digit (globally bucketed) with the
// windows' range records in wtable.
template <bool SEG>
__global__ __launch_bounds__(kBucketThreads) void bucket_sort_rle(
    const uint32_t* __restrict__ kin, const uint32_t* __restrict__ vin, uint32_t* kout,
    uint32_t* vout, int64_t n, int lbits, int nbuckets, const uint32_t* __restrict__ htotals,
    const uint32_t* __restrict__ wtable, int ntiles, uint32_t* status, uint32_t* ticket,
    uint32_t* counters, uint32_t* unique_keys, uint32_t* run_start, uint32_t* run_first,
    int fstride, RunQueue q, uint32_t spin_limit, const uint32_t* __restrict__ rows, int nseg,
    int bpw, int nbk, uint32_t* estatus) {
  constexpr int NT = kBucketThreads, NW = kBucketWaves, CAP = kBucketCap;
  constexpr int SEGS = SEG ? kTileBucketMaxTiles : 1;
  __shared__ uint32_t s_k[CAP];
  __shared__ uint32_t s_v[CAP];
  __shared__ uint32_t s_seglo[SEGS];
  __shared__ uint32_t s_segoff[SEGS];
  __shared__ uint32_t s_segend[SEGS];
  __shared__ uint32_t s_colsum[SEG ? kBucketMaxPerWindow + 1 : 1];
  __shared__ uint32_t s_start;
  __shared__ uint32_t s_pc[SEG ? NW : 1][64];  // bucket_partition's per-wave counts
  __shared__ uint16_t s_cnt[NW][NT];
  __shared__ uint64_t s_slots[NW][256];
  __shared__ uint32_t s_bstart[NT + 1];  // long ranges: bucket starts in the sorted order
  __shared__ uint32_t s_dstart[NT];
  __shared__ uint32_t s_dbase[NT];       // long ranges: digit starts inside the bucket
  __shared__ uint32_t s_run[NT];         // long ranges: digit positions used so far
  __shared__ uint32_t scratch[NW];
  __shared__ uint32_t s_tile, s_base;
  __shared__ uint32_t s_qbase[3];        // queue slots: items, long runs, chunks

  const int tid = threadIdx.x, wave = tid >> 6;
  int tile = static_cast<int>(blockIdx.x);
  if (ticket) {
    if (tid == 0) s_tile = atomicAdd(ticket, 1u);
    __syncthreads();
    tile = static_cast<int>(s_tile);
  }
  // The window's range record and its first CAP sorted positions are loaded
  // together; a range starts inside the window, so it usually lies within
  // them.  Wave w loads positions w0 + [w*64*KPT, (w+1)*64*KPT).
  const int64_t w0 = static_cast<int64_t>(tile) * kBucketWindow;
  uint32_t key[kBucketKpt], val[kBucketKpt];
  int64_t start, len64;
  uint32_t hf, hl;
  if constexpr (SEG) {
    // window `tile`: the high-digit buckets [hf, h1), bpw of them (fewer at
    // the end).  Every tile's segment bounds at hf .. h1 come in one round
    // trip: the window's segment table (tile i: [row_i[hf], row_i[h1])) and
    // column sums, whose differences are the buckets' sizes, so bucket starts
    // inside the window need no scan.  The window's place in the sorted
    // order comes from a look-back over the earlier windows' sizes, which
    // are published at once.
    hf = static_cast<uint32_t>(tile) * static_cast<uint32_t>(bpw);
    const uint32_t h1 = min(hf + static_cast<uint32_t>(bpw), static_cast<uint32_t>(nbk));
    hl = h1 - 1u;
    const int nbw = static_cast<int>(h1 - hf);
#pragma unroll
    for (int w = 0; w < NW; ++w) s_cnt[w][tid] = 0;
    for (int i = tid; i < NW * 256; i += NT) (&s_slots[0][0])[i] = 0u;
    if (tid <= nbw) s_colsum[tid] = 0u;
    __syncthreads();
    // thread (k, i) reads tile i's bound k; each wave adds its values per
    // bound (waves span at most two bounds when nseg >= 64) before one LDS
    // atomic per bound
    for (int base = 0; base < (nbw + 1) * nseg; base += NT) {
      const int idx = base + tid;
      const bool ok = idx < (nbw + 1) * nseg;
      const int k = ok ? idx / nseg : 0, i = idx - k * nseg;
      const uint32_t v = ok ? rows[static_cast<int64_t>(i) * kTileRowWords + hf + k] : 0u;
      if (ok && k == 0) s_seglo[i] = v;
      if (ok && k == nbw) s_segend[i] = v;
      const uint64_t peers = match_bits(__ballot(ok), static_cast<uint32_t>(k), 7);
      uint32_t sum = v;  // sum over the lanes with this k (they are contiguous)
      const int lane = lane_id();
      const int first = __builtin_ctzll(peers ? peers : 1ull);
      const int last = 63 - __builtin_clzll(peers ? peers : 1ull);
      for (int o = 1; o < kWave; o <<= 1) {
        const uint32_t y = __shfl_down(sum, o, kWave);
        if (lane + o <= last) sum += y;
      }
      if (ok && lane == first) atomicAdd(&s_colsum[k], sum);
    }
    __syncthreads();
    const uint32_t sl = tid < nseg ? s_segend[tid] - s_seglo[tid] : 0u;
    uint32_t tot;
    const uint32_t off = block_excl_n<NW>(sl, scratch, &tot);
    if (tid < nseg) s_segoff[tid] = off;
    if (tid <= nbw) s_bstart[tid] = s_colsum[tid] - s_colsum[0];  // inside the window
    if (tid == 0) st_status(estatus + tile, (tile == 0 ? kFlagIncl : kFlagAgg) | tot);
    __syncthreads();
    start = 0;  // known after the look-back
    len64 = tot;
  } else {
    const uint4 rec = *reinterpret_cast<const uint4*>(wtable + 4 * static_cast<int64_t>(tile));
#pragma unroll
    for (int r = 0; r < kBucketKpt; ++r) {
      const int64_t p = w0 + wave * kWave * kBucketKpt + r * kWave + lane_id();
      key[r] = p < n ? kin[p] : 0u;
      val[r] = p < n ? vin[p] : 0u;
    }
#pragma unroll
    for (int w = 0; w < NW; ++w) s_cnt[w][tid] = 0;
    for (int i = tid; i < NW * 256; i += NT) (&s_slots[0][0])[i] = 0u;
    const bool empty = rec.w == 0u;
    start = empty ? 0 : static_cast<int64_t>(~rec.x);
    len64 = empty ? 0 : static_cast<int64_t>(rec.y) - start;
    hf = ~rec.z;
    hl = rec.w - 1u;
  }
  const uint32_t lmask = (1u << lbits) - 1u;
  const auto low = [lmask](uint32_t k) { return k & lmask; };

  uint32_t my_heads = 0;  // run heads among this thread's positions
  int rr = 0;             // positions per thread in the sorted range
  if (len64 <= CAP) {
    const int len = static_cast<int>(len64);
    rr = (len + NT - 1) / NT;
    if (len > 0) {
      if constexpr (SEG) {
        gather_range(kin, vin, n, s_seglo, s_segoff, nseg, 0u, len, rr, key, val);
      } else if (start + len <= w0 + CAP) {
        // the range's positions go to LDS in order, then back in the layout
        // of lds_counting_pass
#pragma unroll
        for (int r = 0; r < kBucketKpt; ++r) {
          const int64_t q = w0 + wave * kWave * kBucketKpt + r * kWave + lane_id() - start;
          if (q >= 0 && q < len) {
            s_k[q] = key[r];
            s_v[q] = val[r];
          }
        }
        __syncthreads();
        const int wseg = wave * kWave * rr;
#pragma unroll
        for (int r = 0; r < kBucketKpt; ++r) {
          const int q = wseg + r * kWave + lane_id();
          if (r < rr && q < len) {
            key[r] = s_k[q];
            val[r] = s_v[q];
          }
        }
      } else {
        load_range(kin, vin, start, len, rr, key, val);
      }
      __syncthreads();
      lds_counting_pass(key, val, rr, 0, len, low, s_k, s_v, s_cnt, s_slots, s_dstart, scratch);
      if (hl > hf) {  // several buckets: a stable pass on the bucket restores their order
        const int wseg = wave * kWave * rr;
#pragma unroll
        for (int r = 0; r < kBucketKpt; ++r) {
          const int p = wseg + r * kWave + lane_id();
          if (r < rr && p < len) {
            key[r] = s_k[p];
            val[r] = s_v[p];
          }
        }
        const uint32_t hspan = hl - hf;
        const bool few = SEG && hspan < 64u;  // the same on every thread
        if (few)
          for (int i = tid; i < (SEG ? NW : 1) * 64; i += NT) (&s_pc[0][0])[i] = 0u;
        __syncthreads();
        // a key's bucket lies in [hf, hl]; the clamp only matters for a batch
        // whose pass on the high digit gave up a wait (its output then holds
        // stale positions), and keeps the LDS counters in range
        const uint32_t hmask = static_cast<uint32_t>(nbuckets) - 1u;
        const auto bucket = [lbits, hf, hmask, hspan](uint32_t k) {
          return min(((k >> lbits) & hmask) - hf, hspan);
        };
        if (few) {
          // bucket starts inside the window are known (s_bstart)
          const auto bstart = [](int b) { return s_bstart[b]; };
          bucket_partition(key, val, rr, len, static_cast<int>(hspan) + 1, bucket, bstart, s_k,
                           s_v, s_pc);
        } else {
          lds_counting_pass(key, val, rr, 0, len, bucket, s_k, s_v, s_cnt, s_slots, s_dstart,
                            scratch);
        }
      }
      // the sorted range goes out before the look-back when its place is known
      if constexpr (!SEG) {
        for (int i = tid; i < len; i += NT) {
          kout[start + i] = s_k[i];
          vout[start + i] = s_v[i];
        }
      }
      // a range starts a bucket, so its first position is always a run head
      for (int j = 0; j < rr; ++j) {
        const int i = tid * rr + j;
        if (i < len && (i == 0 || s_k[i] != s_k[i - 1])) ++my_heads;
      }
    }
  } else {
    // long range: bucket by bucket, chunks of CAP positions in order
    if constexpr (!SEG) {
      const uint32_t my_count = tid < nbuckets ? htotals[tid] : 0u;
      uint32_t tot;
      s_bstart[tid] = block_excl_n<NW>(my_count, scratch, &tot);
      if (tid == 0) s_bstart[NT] = tot;
      __syncthreads();
    } else {
      // the buckets are written as they are sorted: the window's place first
      if (tid < kWave) {
        const uint32_t before =
            tile > 0 ? lookback_wave(estatus, tile, WaitCtl{counters + kCntError, spin_limit}) : 0u;
        if (tid == 0) {
          if (tile > 0)
            st_status(estatus + tile, kFlagIncl | ((before + static_cast<uint32_t>(len64)) & kValueMask));
          s_start = before;
        }
      }
      __syncthreads();
      start = s_start;
    }
    for (uint32_t h = hf; h <= hl; ++h) {
      const uint32_t bs = SEG ? static_cast<uint32_t>(start) + s_bstart[h - hf] : s_bstart[h];
      const uint32_t bn = SEG ? s_bstart[h - hf + 1] - s_bstart[h - hf] : s_bstart[h + 1] - s_bstart[h];
      if (bn == 0) continue;
      if constexpr (SEG) build_segments(rows, nseg, h, h + 1u, s_seglo, s_segoff, scratch);
      s_dbase[tid] = 0u;
      __syncthreads();
      for (uint32_t i = tid; i < bn; i += NT) {
        uint32_t kk;
        if constexpr (SEG) {
          const uint32_t pp = seg_position(s_seglo, s_segoff, nseg, i);
          kk = pp < static_cast<uint64_t>(n) ? kin[pp] : 0u;
        } else {
          kk = kin[bs + i];
        }
        atomicAdd(&s_dbase[kk & lmask], 1u);
      }
      __syncthreads();
      const uint32_t hc = s_dbase[tid];
      uint32_t t2;
      const uint32_t dbase = block_excl_n<NW>(hc, scratch, &t2);
      s_dbase[tid] = dbase;
      s_run[tid] = 0u;
      __syncthreads();
      for (uint32_t c0 = 0; c0 < bn; c0 += CAP) {
        const int clen = static_cast<int>(min(static_cast<uint32_t>(CAP), bn - c0));
        const int crr = (clen + NT - 1) / NT;
        if constexpr (SEG)
          gather_range(kin, vin, n, s_seglo, s_segoff, nseg, c0, clen, crr, key, val);
        else
          load_range(kin, vin, static_cast<int64_t>(bs) + c0, clen, crr, key, val);
        lds_counting_pass(key, val, crr, 0, clen, low, s_k, s_v, s_cnt, s_slots, s_dstart,
                          scratch);
        for (int i = tid; i < clen; i += NT) {
          const uint32_t k = s_k[i];
          const uint32_t d = k & lmask;
          const uint32_t gp = bs + s_dbase[d] + s_run[d] + (static_cast<uint32_t>(i) - s_dstart[d]);
          if (gp < static_cast<uint64_t>(n)) {
            kout[gp] = k;
            vout[gp] = s_v[i];
          }
        }
        __syncthreads();
        const uint32_t next = tid + 1 < NT ? s_dstart[tid + 1] : static_cast<uint32_t>(clen);
        s_run[tid] += next - s_dstart[tid];
        __syncthreads();
      }
    }
    __threadfence_block();
    __syncthreads();
    for (int64_t i = tid; i < len64; i += NT) {
      const uint32_t k = kout[start + i];
      if (i == 0 || k != kout[start + i - 1]) ++my_heads;
    }
  }

  // run ids: this window's first one from the look-back over earlier windows
  uint32_t htotal;
  const uint32_t hex = block_excl_n<NW>(my_heads, scratch, &htotal);
  // the window's run count goes out at once; the look-back comes later
  if (tid == 0) st_status(status + tile, (tile == 0 ? kFlagIncl : kFlagAgg) | htotal);
  // in-LDS ranges: head positions by run id inside the range (the count
  // buffer is free now), so every run knows where it ends; then the queue
  // slots the runs longer than q.short_max need: items, and long runs packed
  // with their chunks (long runs << 16 | chunks; a range holds fewer than 2^16)
  uint32_t* s_hpos = reinterpret_cast<uint32_t*>(&s_cnt[0][0]);
  const int len_l = len64 <= CAP ? static_cast<int>(len64) : 0;
  {
    uint32_t lr = hex;
    for (int j = 0; j < rr; ++j) {
      const int i = tid * rr + j;
      if (i < len_l && (i == 0 || s_k[i] != s_k[i - 1])) s_hpos[lr++] = static_cast<uint32_t>(i);
    }
  }
  __syncthreads();
  const auto run_len = [&](uint32_t lr, int i) {
    return (lr + 1 < htotal ? s_hpos[lr + 1] : static_cast<uint32_t>(len_l)) -
           static_cast<uint32_t>(i);
  };
  uint32_t need_items = 0, need_lc = 0;
  if (q.short_max > 0) {
    uint32_t lr = hex;
    for (int j = 0; j < rr; ++j) {
      const int i = tid * rr + j;
      if (i < len_l && (i == 0 || s_k[i] != s_k[i - 1])) {
        const uint32_t rl = run_len(lr++, i);
        if (rl > static_cast<uint32_t>(q.short_max)) {
          if (rl >= static_cast<uint32_t>(q.long_threshold)) {
            const uint32_t n1 = (rl + q.chunk - 1) / q.chunk;
            need_items += n1;
            need_lc += (1u << 16) + n1;
          } else {
            need_items += 1;
          }
        }
      }
    }
  }
  uint32_t t_items, t_lc;
  const uint32_t x_items = block_excl_n<NW>(need_items, scratch, &t_items);
  const uint32_t x_lc = block_excl_n<NW>(need_lc, scratch, &t_lc);
  if (tid < kWave) {
    uint32_t before = 0;
    if (tile > 0) before = lookback_wave(status, tile, WaitCtl{counters + kCntError, spin_limit});
    if (tid == 0) {
      if (tile > 0) st_status(status + tile, kFlagIncl | ((before + htotal) & kValueMask));
      s_base = before;
      if (tile == ntiles - 1) {
        // U <= n always, unless a look-back gave up; keep every index in range regardless
        const uint32_t U = min(before + htotal, static_cast<uint32_t>(n));
        counters[kCntUnique] = U;
        run_start[U] = static_cast<uint32_t>(n);
      }
    }
  } else if (SEG && len64 <= CAP && tid < 2 * kWave) {
    // the window's place in the sorted order, beside the run-id look-back
    // (the sizes were published at the start, so it rarely waits)
    const uint32_t before =
        tile > 0 ? lookback_wave(estatus, tile, WaitCtl{counters + kCntError, spin_limit}) : 0u;
    if (tid == kWave) {
      if (tile > 0)
        st_status(estatus + tile, kFlagIncl | ((before + static_cast<uint32_t>(len64)) & kValueMask));
      s_start = before;
    }
  } else if (tid == 2 * kWave && (t_items | t_lc) != 0u) {
    // the window's queue slots, reserved while wave 0 looks back
    s_qbase[0] = t_items ? atomicAdd(&counters[kCntItems1], t_items) : 0u;
    s_qbase[1] = (t_lc >> 16) ? atomicAdd(&counters[kCntLong], t_lc >> 16) : 0u;
    s_qbase[2] = (t_lc & 0xFFFFu) ? atomicAdd(&counters[kCntChunks], t_lc & 0xFFFFu) : 0u;
  }
  __syncthreads();
  if (len64 <= CAP) {
    if constexpr (SEG) {
      start = s_start;
      for (int i = tid; i < len_l; i += NT) {
        kout[start + i] = s_k[i];
        vout[start + i] = s_v[i];
      }
    }
    uint32_t lr = hex;
    uint32_t it = s_qbase[0] + x_items;
    uint32_t li = s_qbase[1] + (x_lc >> 16);
    uint32_t b1 = s_qbase[2] + (x_lc & 0xFFFFu);
    for (int j = 0; j < rr; ++j) {
      const int i = tid * rr + j;
      if (i < len_l && (i == 0 || s_k[i] != s_k[i - 1])) {
        const uint32_t r = s_base + lr;
        const uint32_t rl = run_len(lr, i);
        const uint32_t ps = static_cast<uint32_t>(start + i);
        if (r < static_cast<uint64_t>(n)) {
          unique_keys[r] = s_k[i];
          run_start[r] = ps;
          if (fstride == 4) {  // 16-byte aligned: the region starts 256-byte aligned
            uint4 f4;
            f4.x = s_v[i];
            f4.y = i + 1 < len_l ? s_v[i + 1] : 0u;
            f4.z = i + 2 < len_l ? s_v[i + 2] : 0u;
            f4.w = i + 3 < len_l ? s_v[i + 3] : 0u;
            reinterpret_cast<uint4*>(run_first)[r] = f4;
          } else {
            run_first[r] = s_v[i];
          }
        }
        if (q.short_max > 0 && rl > static_cast<uint32_t>(q.short_max)) {
          if (rl >= static_cast<uint32_t>(q.long_threshold)) {
            const uint32_t n1 = (rl + q.chunk - 1) / q.chunk;
            q.longs[li] = make_uint4(ps, rl, b1, n1);
            q.long_keys[li] = s_k[i];
            if (n1 >= kFinPieceMin) atomicOr(&counters[kCntPieced], 1u);
            for (uint32_t c = 0; c < n1; ++c) q.items1[it + c] = make_uint2(li, c);
            ++li;
            b1 += n1;
            it += n1;
          } else {
            q.items1[it++] = make_uint2(ps, kMediumItem | rl);
          }
        }
        ++lr;
      }
    }
  } else {
    uint32_t r0 = s_base;
    for (int64_t c0 = 0; c0 < len64; c0 += NT) {
      const int64_t i = c0 + tid;
      uint32_t k = 0;
      bool head = false;
      if (i < len64) {
        k = kout[start + i];
        head = i == 0 || k != kout[start + i - 1];
      }
      uint32_t t3;
      const uint32_t ex = block_excl_n<NW>(head ? 1u : 0u, scratch, &t3);
      if (head && r0 + ex < static_cast<uint64_t>(n)) {
        unique_keys[r0 + ex] = k;
        run_start[r0 + ex] = static_cast<uint32_t>(start + i);
        for (int f = 0; f < fstride; ++f)
          run_first[static_cast<int64_t>(r0 + ex) * fstride + f] =
              i + f < len64 ? vout[start + i + f] : 0u;
      }
      r0 += t3;
    }
    if (q.short_max > 0) {
      // run lengths from the run starts just written (the range's last run
      // ends with the range)
      __threadfence_block();
      __syncthreads();
      for (uint32_t lr = tid; lr < htotal; lr += NT) {
        const uint32_t r = s_base + lr;
        if (r + 1 >= static_cast<uint64_t>(n) + 1) break;
        const uint32_t s0 = run_start[r];
        const uint32_t e0 = lr + 1 < htotal ? run_start[r + 1] : static_cast<uint32_t>(start + len64);
        if (e0 - s0 > static_cast<uint32_t>(q.short_max))
          queue_run(q, counters, s0, e0 - s0, unique_keys[r]);
      }
    }
  }
}

}  // namespace

// Larger batches use 8192-key tiles: a tile's keys spread over every bucket of
// an 8-bit digit, and 32 keys per bucket make the scatter write whole 128-byte
// lines (16-key tiles left half lines shared with the next tile, usually on
// another XCD: the first pass over 16.8 M uniform 16-bit ids took 323 us
// against 138 us).
int sort_keys_per_thread(int64_t n) { return n <= (int64_t{1} << 20) ? 8 : kCountedKpt; }
int sort_tile_keys(int64_t n, int key_bits) {
  return radix_digit_bits(key_bits, n) > 8 ? 4096 : kBlock * sort_keys_per_thread(n);
}

hipError_t launch_init_workspace(const BackwardLaunch& a, hipStream_t stream,
                                 const KernelTimer* kt) {
  // the counters, histograms and look-back status words the later kernels chain through
  // the radix passes' status words come last and are not needed when the
  // linearize step sorts each tile by the high digit
  const int64_t words = (uses_tile_buckets(a) || counted_passes(a.num_indices))
                            ? static_cast<int64_t>(a.buf.sort_status - a.buf.counters)
                            : a.buf.zero_words;
  const int64_t nvec = (words + 3) / 4;
  int64_t zblocks = (nvec + kBlock - 1) / kBlock;
  if (zblocks > 1024) zblocks = 1024;
  launch_timed(kt, "init_workspace", init_workspace,
               dim3(static_cast<unsigned>(zblocks > 0 ? zblocks : 1)), dim3(kBlock), 0, stream,
               reinterpret_cast<uint4*>(a.buf.counters), nvec);
  return hipGetLastError();
}

hipError_t launch_linearize(const BackwardLaunch& a, hipStream_t stream, const KernelTimer* kt) {
  // a linearize step that sorts the tiles clears the workspace itself
  if (!uses_tile_buckets(a)) {
    const hipError_t e = launch_init_workspace(a, stream, kt);
    if (e != hipSuccess) return e;
  }
  return launch_linearize_kernel(a, stream, kt);
}

template <int BAGS>
hipError_t launch_linearize_bags(const BackwardLaunch& a, hipStream_t stream,
                                 const KernelTimer* kt) {
  const dim3 grid(static_cast<unsigned>(linearize_blocks(a.num_bags, BAGS)));
  const int64_t tiles = (a.num_bags + BAGS - 1) / BAGS;
  const bool deep = a.num_indices > tiles * kLinThreads;
  if (a.index64) {
    if (deep)
      launch_timed(kt, "linearize_kernel", linearize_kernel<int64_t, 2, BAGS>, grid,
                   dim3(kLinThreads), 0, stream, a);
    else
      launch_timed(kt, "linearize_kernel", linearize_kernel<int64_t, 1, BAGS>, grid,
                   dim3(kLinThreads), 0, stream, a);
  } else {
    if (deep)
      launch_timed(kt, "linearize_kernel", linearize_kernel<int32_t, 2, BAGS>, grid,
                   dim3(kLinThreads), 0, stream, a);
    else
      launch_timed(kt, "linearize_kernel", linearize_kernel<int32_t, 1, BAGS>, grid,
                   dim3(kLinThreads), 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_linearize_kernel(const BackwardLaunch& a, hipStream_t stream,
                                   const KernelTimer* kt) {
  if (a.num_bags <= 0) return hipSuccess;
  if (uses_tile_buckets(a)) {
    const dim3 grid(static_cast<unsigned>((a.num_bags + kLinBags - 1) / kLinBags));
    if (a.index64)
      launch_timed(kt, "linearize_kernel", linearize_bucket_kernel<int64_t>, grid,
                   dim3(kLinThreads), 0, stream, a);
    else
      launch_timed(kt, "linearize_kernel", linearize_bucket_kernel<int32_t>, grid,
                   dim3(kLinThreads), 0, stream, a);
    return hipGetLastError();
  }
  return a.num_bags > int64_t{kLinBags} * kLinMaxBlocks
             ? launch_linearize_bags<kLinBagsLarge>(a, stream, kt)
             : launch_linearize_bags<kLinBags>(a, stream, kt);
}

// One pass over keys/values (kin, vin) -> (kout, vout) on the digit
// (key >> shift) & (2^bits - 1).  Batches of up to 2^20 lookups: one look-back
// kernel on the digit counts `totals` (from the linearize step); `pass`
// selects the pass's status words and ticket, and with wtable the pass also
// records the window ranges of the bucket-local sort.  Larger batches: the
// counted pass (count, scan, place), whose scan writes `totals`.
hipError_t launch_pass(const BackwardLaunch& a, int pass, int shift, uint32_t* totals,
                       const uint32_t* kin, const uint32_t* vin, uint32_t* kout, uint32_t* vout,
                       uint32_t* wtable, hipStream_t stream, const KernelTimer* kt) {
  const int64_t n = a.num_indices;
  const int64_t ts = sort_tile_keys(n, a.key_bits);
  const int ntiles = static_cast<int>((n + ts - 1) / ts);
  const int bits = radix_digit_bits(a.key_bits, n);
  const int slots = radix_slots(bits);
  uint32_t* status = a.buf.sort_status + static_cast<int64_t>(pass) * ntiles * slots;
  uint32_t* ticket = ntiles <= kResidentTiles ? nullptr : a.buf.tickets + pass;
  if (counted_passes(n)) {
    // counts of this pass's tiles (every pass reuses the first pass's words),
    // then the digit totals, written by the scan
    uint32_t* cnt = a.buf.sort_status;
    const WaitCtl none{a.buf.counters + kCntError, a.spin_limit};
    launch_timed(kt, "radix_count", radix_count<kCountedKpt>, dim3(ntiles), dim3(kBlock), 0,
                 stream, kin, n, shift, bits, cnt, ntiles);
    launch_timed(kt, "radix_scan", radix_scan, dim3(slots), dim3(kBlock), 0, stream, cnt, ntiles,
                 totals);
    launch_timed(kt, "radix_pass", radix_pass<kCountedKpt, 8, true>, dim3(ntiles), dim3(kBlock),
                 0, stream, kin, vin, kout, vout, n, shift, bits, totals, cnt, nullptr, none,
                 nullptr);
    return hipGetLastError();
  }
  if (bits > 8)
    launch_timed(kt, "radix_pass", radix_pass_wide<4, 10>, dim3(ntiles), dim3(1024), 0, stream,
                 kin, vin, kout, vout, n, shift, bits, totals, status, ticket,
                 WaitCtl{a.buf.counters + kCntError, a.spin_limit}, wtable);
  else
    launch_timed(kt, "radix_pass", radix_pass<8, 8>, dim3(ntiles), dim3(kBlock), 0, stream, kin,
                 vin, kout, vout, n, shift, bits, totals, status, ticket,
                 WaitCtl{a.buf.counters + kCntError, a.spin_limit}, wtable);
  return hipGetLastError();
}

hipError_t launch_radix_sort(const BackwardLaunch& a, hipStream_t stream, int* result_buffer,
                             const KernelTimer* kt) {
  const int passes = radix_passes(a.key_bits, a.num_indices);
  const int bits = radix_digit_bits(a.key_bits, a.num_indices);
  const int slots = radix_slots(bits);
  int cur = 0;
  for (int pass = 0; pass < passes; ++pass) {
    const hipError_t e =
        launch_pass(a, pass, pass * bits, a.buf.digit_hist + pass * slots, a.buf.keys[cur],
                    a.buf.vals[cur], a.buf.keys[cur ^ 1], a.buf.vals[cur ^ 1], nullptr, stream,
                    kt);
    if (e != hipSuccess) return e;
    cur ^= 1;
  }
  *result_buffer = cur;
  return hipSuccess;
}

// Two digits, and buckets of the high digit short on average (they are sorted
// in LDS; a bucket longer than kBucketCap - kBucketWindow takes the slower
// chunked path).
bool uses_bucket_sort(const BackwardLaunch& a) {
  const int64_t n = a.num_indices;
  const int passes = radix_passes(a.key_bits, n);
  const int bits = radix_digit_bits(a.key_bits, n);
  return a.bucket_sort && n > 0 && passes == 2 && n <= kWideRadixMaxKeys &&
         (n >> (a.key_bits - bits)) <= kBucketMeanMax;
}

bool uses_tile_buckets(const BackwardLaunch& a) {
  return uses_bucket_sort(a) && a.num_bags > 0 &&
         (a.num_bags + kLinBags - 1) / kLinBags <= kTileBucketMaxTiles;
}

hipError_t launch_sort_encode(const BackwardLaunch& a, hipStream_t stream, const KernelTimer* kt) {
  const int64_t n = a.num_indices;
  if (n <= 0) return hipSuccess;
  if (!uses_bucket_sort(a)) {
    int sorted = 0;
    const hipError_t e = launch_radix_sort(a, stream, &sorted, kt);
    if (e != hipSuccess) return e;
    return launch_run_length_encode(a, a.buf.keys[sorted], a.buf.vals[sorted], stream, kt);
  }
  const int bits = radix_digit_bits(a.key_bits, n);
  uint32_t* htotals = a.buf.digit_hist + radix_slots(bits);  // counts of the high digit
  // look-back status words of the windows, then their range records
  const int windows = static_cast<int>(bucket_windows(n));
  uint32_t* wstatus = a.buf.rle_status;
  uint32_t* wtable = bucket_window_table(a.buf.rle_status, n);  // 16-byte records
  // the pass on the high digit, unless the linearize step sorted each tile
  const bool seg = uses_tile_buckets(a);
  if (!seg) {
    const hipError_t e = launch_pass(a, 0, bits, htotals, a.buf.keys[0], a.buf.vals[0],
                                     a.buf.keys[1], a.buf.vals[1], wtable, stream, kt);
    if (e != hipSuccess) return e;
  }
  const int nseg = seg ? static_cast<int>((a.num_bags + kLinBags - 1) / kLinBags) : 0;
  const int nbk = 1 << (a.key_bits - bits);        // buckets of the high digit
  const int bpw = seg ? buckets_per_window(n, nbk) : 0;
  const int nwin = seg ? (nbk + bpw - 1) / bpw : windows;
  launch_timed(kt, "bucket_sort_rle", seg ? bucket_sort_rle<true> : bucket_sort_rle<false>,
               dim3(nwin), dim3(kBucketThreads), 0, stream, a.buf.keys[1], a.buf.vals[1],
               a.buf.keys[0], a.buf.vals[0], n, bits, 1 << bits, htotals, wtable, nwin,
               wstatus, nwin <= kResidentTiles ? nullptr : a.buf.tickets + kMaxRadixPasses,
               a.buf.counters, a.buf.unique_keys, a.buf.run_start, a.buf.run_first,
               a.buf.first_stride,
               RunQueue{a.buf.items1, a.buf.longs, a.buf.long_keys, a.short_max,
                        a.long_threshold, a.chunk},
               a.spin_limit, static_cast<const uint32_t*>(a.buf.tile_rows), nseg, bpw, nbk,
               wstatus + kBucketMaxWindows);
  return hipGetLastError();
}

hipError_t launch_run_length_encode(const BackwardLaunch& a, const uint32_t* sorted_keys,
                                    const uint32_t* sorted_vals, hipStream_t stream,
                                    const KernelTimer* kt) {
  const int64_t n = a.num_indices;
  const int ntiles = static_cast<int>((n + kRleTile - 1) / kRleTile);
  if (counted_passes(n)) {
    // head counts of the tiles, then their scan (the radix passes' count words
    // are free again; the scan's total goes to the word after them)
    uint32_t* cnt = a.buf.sort_status;
    launch_timed(kt, "rle_count", rle_count, dim3(ntiles), dim3(1024), 0, stream, sorted_keys, n,
                 cnt);
    launch_timed(kt, "radix_scan", radix_scan, dim3(1), dim3(kBlock), 0, stream, cnt, ntiles,
                 cnt + ntiles);
    launch_timed(kt, "rle_kernel", rle_kernel<true>, dim3(ntiles), dim3(1024), 0, stream,
                 sorted_keys, sorted_vals, n, ntiles, cnt, nullptr, a.buf.counters,
                 a.buf.unique_keys, a.buf.run_start, a.buf.run_first, a.buf.first_stride,
                 a.spin_limit);
    return hipGetLastError();
  }
  launch_timed(kt, "rle_kernel", rle_kernel<false>, dim3(ntiles), dim3(1024), 0, stream,
               sorted_keys, sorted_vals, n, ntiles, a.buf.rle_status,
               ntiles <= kResidentTiles ? nullptr : a.buf.tickets + kMaxRadixPasses,
               a.buf.counters, a.buf.unique_keys, a.buf.run_start, a.buf.run_first,
               a.buf.first_stride, a.spin_limit);
  return hipGetLastError();
}

}  // namespace tbe
