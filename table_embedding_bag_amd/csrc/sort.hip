// sort.hip -- the grouping front of the TBE backward on gfx950: linearize the
// lookups to (table, row) ids, sort them with an LDS radix sort and
// run-length encode the sorted ids.
//
// kimbodo.com/?p=28372, "What Happened": updates are grouped by table and row
// so that each row gets one optimizer update; "Kimbodo Engineering
// Perspective": the grouping is a transpose, a sort and a run-length encoding.
//
//   linearize   key_i = roff_t + x_i (one 32-bit id space over all tables),
//               value_i = bag id k (plain sums) or lookup id i, with a side
//               record {k, p_i * s_k} when the lookup carries a coefficient.
//   radix sort  stable least-significant-digit radix sort of (key, value) on
//               ceil(log2(sum E_t)) bits, 8 bits per pass.  Each pass is
//               three kernels: per-tile digit counts, a per-digit scan over
//               tiles, and a scatter that ranks every key of a 2048-key tile in
//               LDS (wave-level match of equal digits through ballots, per-wave
//               digit counters in LDS) and writes the tile out bucket by
//               bucket so that the global stores are coalesced.
//   RLE         run heads (key differs from its predecessor), a scan of head
//               counts over 4096-key tiles, then unique ids and run starts.
//               The number of runs U stays on the device.
#include "common.hpp"

namespace tbe {
namespace {

template <typename IT>
__device__ __forceinline__ int64_t ld_index(const void* p, int64_t i) {
  return static_cast<int64_t>(static_cast<const IT*>(p)[i]);
}

// One workgroup per 256 consecutive bags.  The bags' offsets are staged in
// LDS; the workgroup then walks all of their lookups with consecutive threads
// on consecutive lookups and finds each lookup's bag by binary search in LDS.
template <typename IT>
__global__ __launch_bounds__(kBlock) void linearize_kernel(BackwardLaunch a) {
  __shared__ int64_t s_off[kBlock + 1];
  __shared__ uint32_t s_roff[kBlock];
  __shared__ float s_scale[kBlock];

  const int tid = threadIdx.x;
  if (blockIdx.x == 0 && tid < kNumCounters) a.buf.counters[tid] = 0u;

  const int64_t k0 = static_cast<int64_t>(blockIdx.x) * kBlock;
  const int nb = static_cast<int>(min(static_cast<int64_t>(kBlock), a.num_bags - k0));
  if (tid < nb) {
    const int64_t k = k0 + tid;
    const int64_t lo = ld_index<IT>(a.offsets, k);
    const int64_t hi = ld_index<IT>(a.offsets, k + 1);
    s_off[tid] = lo;
    if (tid == nb - 1) s_off[nb] = hi;
    const int t = static_cast<int>(k / a.B);
    s_roff[tid] = static_cast<uint32_t>(a.meta[t].roff);
    s_scale[tid] = a.mean ? ((hi > lo) ? 1.0f / static_cast<float>(hi - lo) : 0.0f) : 1.0f;
  }
  __syncthreads();

  const int64_t p0 = s_off[0], p1 = s_off[nb];
  for (int64_t p = p0 + tid; p < p1; p += kBlock) {
    // bag slot s with s_off[s] <= p < s_off[s + 1]
    int lo = 0, hi = nb;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_off[mid] <= p)
        lo = mid;
      else
        hi = mid;
    }
    const uint32_t key = s_roff[lo] + static_cast<uint32_t>(ld_index<IT>(a.indices, p));
    a.buf.keys[0][p] = key;
    const uint32_t bag = static_cast<uint32_t>(k0 + lo);
    if (a.use_rec) {
      a.buf.vals[0][p] = static_cast<uint32_t>(p);
      const float coef = (a.psw ? a.psw[p] : 1.0f) * s_scale[lo];
      a.buf.rec[p] = make_uint2(bag, __float_as_uint(coef));
    } else {
      a.buf.vals[0][p] = bag;
    }
  }
}

// Per-tile digit counts, stored digit-major: hist[d * ntiles + tile].
__global__ __launch_bounds__(kBlock) void radix_upsweep(const uint32_t* __restrict__ keys,
                                                        int64_t n, int shift, uint32_t* hist,
                                                        int ntiles) {
  __shared__ uint32_t h[kRadix];
  const int tid = threadIdx.x;
  h[tid] = 0u;
  __syncthreads();
  const int64_t base = static_cast<int64_t>(blockIdx.x) * kSortTile;
#pragma unroll
  for (int i = 0; i < kSortKeysPerThread; ++i) {
    const int64_t p = base + i * kBlock + tid;
    if (p < n) atomicAdd(&h[(keys[p] >> shift) & (kRadix - 1)], 1u);
  }
  __syncthreads();
  hist[static_cast<int64_t>(tid) * ntiles + blockIdx.x] = h[tid];
}

// One workgroup per digit: exclusive scan of that digit's per-tile counts
// (in place) and the digit's total.
__global__ __launch_bounds__(kBlock) void radix_scan(uint32_t* hist, int ntiles,
                                                     uint32_t* totals) {
  __shared__ uint32_t scratch[kWavesPerBlock];
  uint32_t* row = hist + static_cast<int64_t>(blockIdx.x) * ntiles;
  uint32_t carry = 0;
  for (int base = 0; base < ntiles; base += kBlock) {
    const int i = base + threadIdx.x;
    const uint32_t v = (i < ntiles) ? row[i] : 0u;
    uint32_t total;
    const uint32_t excl = block_exclusive_sum(v, scratch, &total);
    if (i < ntiles) row[i] = carry + excl;
    carry += total;
  }
  if (threadIdx.x == 0) totals[blockIdx.x] = carry;
}

// Stable scatter of one 2048-key tile.  Wave w owns tile positions
// [w*512, (w+1)*512) and ranks them in 8 rounds of 64 consecutive keys; the
// rank of a key is (keys with its digit in earlier waves) + (in earlier rounds
// of its wave) + (in lower lanes of its round), which preserves input order.
__global__ __launch_bounds__(kBlock) void radix_downsweep(
    const uint32_t* __restrict__ kin, const uint32_t* __restrict__ vin, uint32_t* __restrict__ kout,
    uint32_t* __restrict__ vout, int64_t n, int shift, const uint32_t* __restrict__ hist,
    const uint32_t* __restrict__ totals, int ntiles) {
  constexpr int KPT = kSortKeysPerThread;
  __shared__ uint32_t s_k[kSortTile];
  __shared__ uint32_t s_v[kSortTile];
  __shared__ uint32_t s_cnt[kWavesPerBlock][kRadix];
  __shared__ uint32_t s_dstart[kRadix];
  __shared__ uint32_t s_gbase[kRadix];
  __shared__ uint32_t scratch[kWavesPerBlock];

  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const int tile = blockIdx.x;
  const int64_t base = static_cast<int64_t>(tile) * kSortTile;
  const uint32_t dmask = kRadix - 1;

  for (int i = tid; i < kWavesPerBlock * kRadix; i += kBlock) (&s_cnt[0][0])[i] = 0u;
  {
    uint32_t total;
    const uint32_t dbase = block_exclusive_sum(totals[tid], scratch, &total);
    s_gbase[tid] = dbase + hist[static_cast<int64_t>(tid) * ntiles + tile];
  }
  __syncthreads();

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
    uint64_t peers = __ballot(ok);
#pragma unroll
    for (int bit = 0; bit < kRadixBits; ++bit) {
      const bool set = (d >> bit) & 1u;
      const uint64_t bal = __ballot(set);
      peers &= set ? bal : ~bal;
    }
    const uint32_t below = popc_below(peers);
    const uint32_t cnt = __popcll(peers);
    const uint32_t pre = ok ? s_cnt[wave][d] : 0u;
    rank[r] = pre + below;
    if (ok && below == 0) s_cnt[wave][d] = pre + cnt;
  }
  __syncthreads();
  {
    const uint32_t c0 = s_cnt[0][tid], c1 = s_cnt[1][tid], c2 = s_cnt[2][tid], c3 = s_cnt[3][tid];
    s_cnt[0][tid] = 0u;
    s_cnt[1][tid] = c0;
    s_cnt[2][tid] = c0 + c1;
    s_cnt[3][tid] = c0 + c1 + c2;
    uint32_t total;
    s_dstart[tid] = block_exclusive_sum(c0 + c1 + c2 + c3, scratch, &total);
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
  const int tile_n = static_cast<int>(min(static_cast<int64_t>(kSortTile), n - base));
  for (int i = tid; i < tile_n; i += kBlock) {
    const uint32_t k = s_k[i];
    const uint32_t d = (k >> shift) & dmask;
    const uint32_t gp = s_gbase[d] + (static_cast<uint32_t>(i) - s_dstart[d]);
    kout[gp] = k;
    vout[gp] = s_v[i];
  }
}

// Run heads per 4096-key tile.
__global__ __launch_bounds__(kBlock) void rle_count(const uint32_t* __restrict__ keys, int64_t n,
                                                    uint32_t* tile_heads) {
  __shared__ uint32_t scratch[kWavesPerBlock];
  const int64_t base = static_cast<int64_t>(blockIdx.x) * kRleTile;
  uint32_t c = 0;
  for (int i = 0; i < kRleTile / kBlock; ++i) {
    const int64_t p = base + i * kBlock + threadIdx.x;
    if (p < n) c += (p == 0 || keys[p] != keys[p - 1]) ? 1u : 0u;
  }
  uint32_t total;
  block_exclusive_sum(c, scratch, &total);
  if (threadIdx.x == 0) tile_heads[blockIdx.x] = total;
}

// One workgroup: exclusive scan of the per-tile head counts; U = total.
__global__ __launch_bounds__(kBlock) void rle_scan(uint32_t* tile_heads, int ntiles,
                                                   uint32_t* counters, uint32_t* run_start,
                                                   int64_t n) {
  __shared__ uint32_t scratch[kWavesPerBlock];
  uint32_t carry = 0;
  for (int base = 0; base < ntiles; base += kBlock) {
    const int i = base + threadIdx.x;
    const uint32_t v = (i < ntiles) ? tile_heads[i] : 0u;
    uint32_t total;
    const uint32_t excl = block_exclusive_sum(v, scratch, &total);
    if (i < ntiles) tile_heads[i] = carry + excl;
    carry += total;
  }
  if (threadIdx.x == 0) {
    counters[kCntUnique] = carry;
    run_start[carry] = static_cast<uint32_t>(n);
  }
}

// Unique ids and run starts.  The tile (plus the key before it) is staged in
// LDS; each thread then owns 16 consecutive positions so that run ids follow
// position order.
__global__ __launch_bounds__(kBlock) void rle_write(const uint32_t* __restrict__ keys, int64_t n,
                                                    const uint32_t* __restrict__ tile_base,
                                                    uint32_t* unique_keys, uint32_t* run_start) {
  constexpr int PER = kRleTile / kBlock;
  __shared__ uint32_t s_k[kRleTile + 1];
  __shared__ uint32_t scratch[kWavesPerBlock];
  const int tid = threadIdx.x;
  const int64_t base = static_cast<int64_t>(blockIdx.x) * kRleTile;
  for (int i = tid; i < kRleTile + 1; i += kBlock) {
    const int64_t p = base - 1 + i;
    s_k[i] = (p >= 0 && p < n) ? keys[p] : 0u;
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
  uint32_t r = tile_base[blockIdx.x] + block_exclusive_sum(c, scratch, &total);
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = tid * PER + j;
    const int64_t p = base + i;
    if (p < n && (p == 0 || s_k[i + 1] != s_k[i])) {
      unique_keys[r] = s_k[i + 1];
      run_start[r] = static_cast<uint32_t>(p);
      ++r;
    }
  }
}

}  // namespace

hipError_t launch_linearize(const BackwardLaunch& a, hipStream_t stream) {
  const int64_t blocks = (a.num_bags + kBlock - 1) / kBlock;
  if (blocks <= 0) return hipSuccess;
  if (a.index64)
    hipLaunchKernelGGL(linearize_kernel<int64_t>, dim3(static_cast<unsigned>(blocks)),
                       dim3(kBlock), 0, stream, a);
  else
    hipLaunchKernelGGL(linearize_kernel<int32_t>, dim3(static_cast<unsigned>(blocks)),
                       dim3(kBlock), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_radix_sort(const BackwardLaunch& a, hipStream_t stream, int* result_buffer,
                             StageHook hook, void* ctx) {
  const int64_t n = a.num_indices;
  const int ntiles = static_cast<int>((n + kSortTile - 1) / kSortTile);
  int cur = 0;
  for (int shift = 0; shift < a.key_bits; shift += kRadixBits) {
    hipLaunchKernelGGL(radix_upsweep, dim3(ntiles), dim3(kBlock), 0, stream, a.buf.keys[cur], n,
                       shift, a.buf.hist, ntiles);
    if (hook) hook(ctx, "radix_upsweep");
    hipLaunchKernelGGL(radix_scan, dim3(kRadix), dim3(kBlock), 0, stream, a.buf.hist, ntiles,
                       a.buf.digit_totals);
    if (hook) hook(ctx, "radix_scan");
    hipLaunchKernelGGL(radix_downsweep, dim3(ntiles), dim3(kBlock), 0, stream, a.buf.keys[cur],
                       a.buf.vals[cur], a.buf.keys[cur ^ 1], a.buf.vals[cur ^ 1], n, shift,
                       a.buf.hist, a.buf.digit_totals, ntiles);
    if (hook) hook(ctx, "radix_downsweep");
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    cur ^= 1;
  }
  *result_buffer = cur;
  return hipSuccess;
}

hipError_t launch_run_length_encode(const BackwardLaunch& a, const uint32_t* sorted_keys,
                                    hipStream_t stream, StageHook hook, void* ctx) {
  const int64_t n = a.num_indices;
  const int ntiles = static_cast<int>((n + kRleTile - 1) / kRleTile);
  hipLaunchKernelGGL(rle_count, dim3(ntiles), dim3(kBlock), 0, stream, sorted_keys, n,
                     a.buf.rle_tiles);
  if (hook) hook(ctx, "rle_count");
  hipLaunchKernelGGL(rle_scan, dim3(1), dim3(kBlock), 0, stream, a.buf.rle_tiles, ntiles,
                     a.buf.counters, a.buf.run_start, n);
  if (hook) hook(ctx, "rle_scan");
  hipLaunchKernelGGL(rle_write, dim3(ntiles), dim3(kBlock), 0, stream, sorted_keys, n,
                     a.buf.rle_tiles, a.buf.unique_keys, a.buf.run_start);
  if (hook) hook(ctx, "rle_write");
  return hipGetLastError();
}

}  // namespace tbe
