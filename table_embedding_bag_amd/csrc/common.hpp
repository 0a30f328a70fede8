// common.hpp -- device helpers and internal launch interfaces of the gfx950
// TBE library.  Everything here is internal; the public interface is tbe.h.
#pragma once

#include <algorithm>

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tbe {

constexpr int kWave = 64;        // CDNA wavefront width
constexpr int kBlock = 256;      // threads per workgroup for every kernel here
constexpr int kWavesPerBlock = kBlock / kWave;

// Storage dtype codes (same values as tbe_dtype).
constexpr int kF32 = 0, kF16 = 1, kBF16 = 2;

// Per-table metadata, computed once at handle creation and kept on the device.
struct TableMeta {
  int64_t woff;      // element offset of the table's row 0 in the flat weights
  int32_t roff;      // linear row id of the table's row 0
  int32_t rows;      // E_t
  int32_t dim;       // D_t
  int32_t doff;      // first output column of the table
  int32_t fwd_gshift;  // log2(lanes that cover one row in the forward)
  // log2(lanes that cover one fp32 gradient row in the backward's short-run
  // kernel): bits 0-7 with 16-byte chunks, bits 8-15 with one value per lane
  int32_t bwd_gshift;
};
static_assert(sizeof(TableMeta) == 32, "TableMeta layout");

// ---------------------------------------------------------------------------
// Small device helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// Number of set bits of m in lanes below this one.
__device__ __forceinline__ uint32_t popc_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u));
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ uint32_t wave_inclusive_sum(uint32_t x) {
  const int lane = lane_id();
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const uint32_t y = __shfl_up(x, d, kWave);
    if (lane >= d) x += y;
  }
  return x;
}

// Exclusive prefix sum over a 256-thread block; *total receives the sum.
// scratch: 4 words of shared memory.  Contains barriers: call from all threads.
__device__ __forceinline__ uint32_t block_exclusive_sum(uint32_t x, uint32_t* scratch,
                                                        uint32_t* total) {
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const uint32_t incl = wave_inclusive_sum(x);
  if (lane == kWave - 1) scratch[wave] = incl;
  __syncthreads();
  uint32_t base = 0, sum = 0;
#pragma unroll
  for (int w = 0; w < kWavesPerBlock; ++w) {
    const uint32_t s = scratch[w];
    base += (w < wave) ? s : 0u;
    sum += s;
  }
  __syncthreads();
  *total = sum;
  return base + incl - x;
}

// Lanes among `active` whose value v (its low `bits` bits) equals this lane's:
// one ballot per bit.  Each bit is taken as a mask of all ones or all zeros
// (its sign-extended copy), so a lane keeps the ballot's lanes whose bit equals
// its own with one xor and and per half (two selects and two ands per bit
// otherwise; the radix passes' ranking is bound by this VALU work).  Call with
// the whole wave.
__device__ __forceinline__ uint64_t match_low_bits(uint64_t active, uint32_t v, int bits) {
  uint64_t peers = active;
  for (int bit = 0; bit < bits; ++bit) {
    const uint32_t m = static_cast<uint32_t>(static_cast<int32_t>(v << (31 - bit)) >> 31);
    const uint64_t bal = __ballot(m != 0u);
    peers &= ~(bal ^ ((static_cast<uint64_t>(m) << 32) | m));
  }
  return peers;
}

// Workgroups are handed to the 8 XCDs of the chip round robin.  Renumber them
// so that each XCD works on one contiguous range of logical work items (and so
// keeps that range's data in its own L2).
__device__ __forceinline__ int xcd_contiguous_block(int bid, int nblocks) {
  const int xcd = bid & 7, pos = bid >> 3;
  const int q = nblocks >> 3, r = nblocks & 7;
  return xcd * q + (xcd < r ? xcd : r) + pos;
}

// bf16 / fp16 widening (exact) and narrowing (round to nearest even).
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }
__device__ __forceinline__ float f16_lo(uint32_t u) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(u & 0xFFFFu)));
}
__device__ __forceinline__ float f16_hi(uint32_t u) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(u >> 16)));
}
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;  // NaN stays a quiet NaN
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;                   // ties to even
}
__device__ __forceinline__ uint32_t f32_to_f16_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));  // v_cvt_f16_f32, RNE mode
}

template <int ST>
struct StorageTraits;
template <>
struct StorageTraits<kF32> { static constexpr int bytes = 4; };
template <>
struct StorageTraits<kF16> { static constexpr int bytes = 2; };
template <>
struct StorageTraits<kBF16> { static constexpr int bytes = 2; };

// Load VE consecutive stored elements starting at element e of base and widen
// them to fp32.  VE * bytes is 16, 8, 4 or 2 and the address is aligned to it.
template <int ST, int VE>
__device__ __forceinline__ void load_widen(const void* base, int64_t e, float* out) {
  if constexpr (ST == kF32) {
    const float* p = static_cast<const float*>(base) + e;
    if constexpr (VE == 4) {
      const float4 v = *reinterpret_cast<const float4*>(p);
      out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
    } else {
#pragma unroll
      for (int i = 0; i < VE; ++i) out[i] = p[i];
    }
  } else {
    const uint16_t* p = static_cast<const uint16_t*>(base) + e;
    if constexpr (VE == 8) {
      const uint4 v = *reinterpret_cast<const uint4*>(p);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        out[2 * i] = (ST == kBF16) ? bf16_lo(w[i]) : f16_lo(w[i]);
        out[2 * i + 1] = (ST == kBF16) ? bf16_hi(w[i]) : f16_hi(w[i]);
      }
    } else if constexpr (VE == 4) {
      const uint2 v = *reinterpret_cast<const uint2*>(p);
      out[0] = (ST == kBF16) ? bf16_lo(v.x) : f16_lo(v.x);
      out[1] = (ST == kBF16) ? bf16_hi(v.x) : f16_hi(v.x);
      out[2] = (ST == kBF16) ? bf16_lo(v.y) : f16_lo(v.y);
      out[3] = (ST == kBF16) ? bf16_hi(v.y) : f16_hi(v.y);
    } else {
#pragma unroll
      for (int i = 0; i < VE; ++i) {
        const uint32_t u = p[i];
        out[i] = (ST == kBF16) ? bf16_lo(u) : f16_lo(u);
      }
    }
  }
}

// Widen one 16-byte chunk of stored elements (4 fp32 or 8 fp16/bf16) to fp32,
// as load_widen does with VE * bytes = 16.
template <int ST>
__device__ __forceinline__ void widen_chunk(const uint4& v, float* out) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  if constexpr (ST == kF32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = __uint_as_float(w[i]);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = (ST == kBF16) ? bf16_lo(w[i]) : f16_lo(w[i]);
      out[2 * i + 1] = (ST == kBF16) ? bf16_hi(w[i]) : f16_hi(w[i]);
    }
  }
}

// Narrow VE fp32 values to the storage dtype and store them at element e.
template <int ST, int VE>
__device__ __forceinline__ void narrow_store(void* base, int64_t e, const float* v) {
  if constexpr (ST == kF32) {
    float* p = static_cast<float*>(base) + e;
    if constexpr (VE == 4) {
      *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    } else {
#pragma unroll
      for (int i = 0; i < VE; ++i) p[i] = v[i];
    }
  } else {
    uint16_t* p = static_cast<uint16_t*>(base) + e;
    auto cvt = [](float f) { return (ST == kBF16) ? f32_to_bf16_bits(f) : f32_to_f16_bits(f); };
    if constexpr (VE == 4) {
      *reinterpret_cast<uint2*>(p) =
          make_uint2(cvt(v[0]) | (cvt(v[1]) << 16), cvt(v[2]) | (cvt(v[3]) << 16));
    } else {
#pragma unroll
      for (int i = 0; i < VE; ++i) p[i] = static_cast<uint16_t>(cvt(v[i]));
    }
  }
}

// ---------------------------------------------------------------------------
// Launch interfaces (host side, implemented next to their kernels)
// ---------------------------------------------------------------------------

// Kernel timing for profiling: when a timer is given and hands out a pair of
// events, the launch records the kernel's own start and end in them
// (hipExtLaunchKernelGGL), so host gaps between launches are not counted.
struct KernelTimer {
  void* ctx;
  bool (*take)(void* ctx, const char* kernel_name, hipEvent_t* start, hipEvent_t* stop);
};

template <typename... KArgs, typename... Args>
inline void launch_timed(const KernelTimer* kt, const char* name, void (*kernel)(KArgs...),
                         dim3 grid, dim3 block, uint32_t shmem, hipStream_t s, Args... args) {
  hipEvent_t e0, e1;
  if (kt && kt->take(kt->ctx, name, &e0, &e1))
    hipExtLaunchKernelGGL(kernel, grid, block, shmem, s, e0, e1, 0u, static_cast<KArgs>(args)...);
  else
    hipLaunchKernelGGL(kernel, grid, block, shmem, s, static_cast<KArgs>(args)...);
}

struct ForwardLaunch {
  const void* weights;
  const void* indices;
  const void* offsets;
  const float* psw;         // may be null
  float* out;
  const TableMeta* meta;
  int32_t T, B, sum_dims;
  int32_t tiles_per_table;  // workgroups per table
  int32_t lshift;           // log2(rows in flight per bag per lane group)
  int32_t mean;
  int32_t dtype;            // storage dtype code
  int32_t index64;          // indices/offsets are int64
  int32_t vec;              // 16-byte row chunks (else one element per lane)
  int32_t uncond_loads;     // row loads issued unconditionally (batches above
                            // kFusedMaxLookups lookups)
  const int32_t* table_list;  // tables to cover (T entries), or null for tables 0..T-1
  // Bags longer than split_len lookups (0: none) pool only their first
  // split_len lookups here; the rest is queued as segments of split_len for
  // launch_forward_split (host-checked: the segments always fit).
  int32_t split_len;
  uint32_t* split_ctr;      // [2]: segments queued, long bags queued (zeroed per call)
  uint2* split_seg;         // {bag, segment index >= 1}
  uint4* split_long;        // {bag, first segment slot, segments, 0}
  float* split_part;        // [segments][split_pstride] scaled segment sums
  int32_t split_pstride;
};
// Segment sums of the bags split by the pooled lookup, then their addition to
// the output in segment order.
hipError_t launch_forward_split(const ForwardLaunch& a, int64_t num_indices, hipStream_t stream,
                                const KernelTimer* kt);
hipError_t launch_forward_gather(const ForwardLaunch& a, hipStream_t stream,
                                 const KernelTimer* kt);
// Small tables pooled from LDS (a.table_list: the tables, a.T of them), the
// same bits as launch_forward_gather with the same lshift.  Every listed table
// has rows * 2^gshift 16-byte chunk slots (rows padded to 2^gshift chunks) of
// at most kLdsFwdBytes, rows of at most 2^gshift 16-byte chunks with
// gshift in [kLdsFwdMinGshift, kLdsFwdMaxGshift], and R = 2^min(6 - gshift,
// lshift) <= lds_forward_max_r(gshift, per-sample weights); no split bags.
constexpr int kLdsFwdThreads = 1024;
constexpr int kLdsFwdBytes = 128 * 1024;
constexpr int kLdsFwdMinGshift = 2;
constexpr int kLdsFwdMaxGshift = 3;
constexpr int kLdsFwdMaxR = 4;  // partial sums per bag (more would spill registers)
inline int lds_forward_max_r(int gshift, bool psw) {
  return std::min(1 << gshift, (psw && gshift == 3) ? 2 : kLdsFwdMaxR);
}
hipError_t launch_forward_lds(const ForwardLaunch& a, int gshift, int wgs_per_table,
                              hipStream_t stream, const KernelTimer* kt);
// dL/dp_i for every lookup (a.table_list must be null: all tables).
hipError_t launch_psw_grad(const ForwardLaunch& a, const float* grad, float* gpsw,
                           hipStream_t stream, const KernelTimer* kt);

// Count-matrix forward of small 16-bit tables.  Each such table has a
// transposed, zero-padded copy W^T[d][e] (e < epad, epad a multiple of
// kHistKc) at element wt_off of a handle-owned buffer.
constexpr int kHistKc = 64;        // table rows per K chunk
constexpr int kHistMaxRows = 1024; // eligibility: E_t
constexpr int kHistMaxDim = 256;   // eligibility: D_t (and a multiple of 16)
struct HistTable {
  int32_t table;
  int32_t epad;
  int64_t wt_off;
};
struct HistLaunch {
  const void* weights;
  const void* indices;
  const void* offsets;
  float* out;
  const TableMeta* meta;
  const HistTable* list;
  uint16_t* wt;
  int32_t H;                // tables in list
  int32_t B, sum_dims;
  int32_t etiles, dtiles;   // max over the listed tables of epad/64 and ceil(D/64)
  int32_t mean;
  int32_t dtype;            // kF16 or kBF16
  int32_t index64;
};
hipError_t launch_forward_histogram(const HistLaunch& a, hipStream_t stream,
                                    const KernelTimer* kt);

// Device workspace of the backward, carved by the host.
struct BackwardBuffers {
  uint32_t* keys[2];
  uint32_t* vals[2];
  uint2* rec;               // per lookup {bag, coefficient bits} when needed, else null
  // One contiguous region zeroed at the start of every backward call:
  //   counters [kNumCounters], tickets [kNumTickets], digit_hist [passes][slots],
  //   rle_status [rle tiles], piece_tickets [chunks cap / kFinPiece + 1],
  //   run_tickets [long runs cap],
  //   sort_status [passes][sort tiles][slots] (not cleared when no radix pass runs)
  // (slots = radix_slots(digit bits))
  uint32_t* counters;
  uint32_t* tickets;        // tile tickets: one per radix pass, then the RLE's
  uint32_t* digit_hist;     // digit counts of every radix pass
  uint32_t* sort_status;    // look-back status words of the radix passes
  uint32_t* rle_status;     // look-back status words of the RLE
  uint32_t* piece_tickets;  // finished chunks of each piece of a very long run, by the piece's
                            // first partial slot / kFinPiece (long runs finished by seg_fused)
  uint32_t* run_tickets;    // finished chunks (or pieces) of each long run
  int64_t zero_words;       // size of the zeroed region, in 32-bit words
  uint32_t* unique_keys;    // [N]
  uint32_t* run_start;      // [N + 1]
  uint32_t* run_first;      // [N][first_stride]: sorted values of each run's first lookups
  int32_t first_stride;     // 4 for batches of at most 2^20 lookups (the first four), else 1
  uint32_t* table_runs;     // [T + 1]: first run id of each table (per-table lane groups)
  uint32_t* tile_rows;      // [linearize tiles][kTileRowWords] segment bounds (linearize_bucket)
  uint2* items1;            // workgroup items: {first position, medium flag | length}
                            // or {long run, chunk}
  uint4* longs;             // {first position, length, first chunk partial, chunk count}
  uint32_t* long_keys;      // row id of each long run (loaded with its list entry)
  float* partial1;          // [chunks cap, pstride]
};

// Device counters of the backward (zeroed at the start of every call), each
// on a 128-byte line of its own so that atomics on different counters do not
// queue behind each other.  kCntError is raised if a look-back wait ever
// gives up (results then invalid); kCntPieced once a long run of at least
// kFinPieceMin chunks is queued.
enum { kCntUnique = 0, kCntLong = 32, kCntItems1 = 64, kCntChunks = 96, kCntError = 128,
       kCntPieced = 160, kNumCounters = 192 };

// A long run of at least kFinPieceMin chunks has its chunk partials added in
// pieces of kFinPiece chunks (the last piece takes the remainder, so every
// piece has at least kFinPiece); each piece's sum is left as doubles in its
// first two partial slots.  Piece starts are thus at least kFinPiece slots
// apart, and first slot / kFinPiece numbers them.
constexpr uint32_t kFinPiece = 64;
constexpr uint32_t kFinPieceMin = 2 * kFinPiece;
// Batches of at most this many lookups have their long runs finished inside
// the segment kernel by the workgroup that stores a run's last chunk partial
// (a ticket per run), which saves a launch; larger ones, whose many long runs
// would each add a ticket round trip to a workgroup item, take a separate
// finishing kernel.
constexpr int64_t kFinishInItemsMaxKeys = int64_t{1} << 20;
// L2 of one XCD: the short runs are split into one range per XCD when an
// eighth of the upstream gradient fits in it.
constexpr int64_t kXcdL2Bytes = int64_t{4} << 20;

// Workgroup items of the segment kernels: {first position, kMediumItem | length}
// for a medium run, {long run, chunk} for a 256-lookup chunk of a long run.
constexpr uint32_t kMediumItem = 0x80000000u;

// Where a run-length encoder that sees whole runs queues those longer than
// short_max lookups (medium runs and the chunks of long runs), so that the
// segment kernels need not queue them.
struct RunQueue {
  uint2* items1;
  uint4* longs;            // {first position, length, first partial, chunks}
  uint32_t* long_keys;
  int32_t short_max;
  int32_t long_threshold;
  int32_t chunk;
};
constexpr int kNumTickets = 8;           // kMaxRadixPasses radix passes + the RLE

// Keys per thread of a radix tile for a batch of n lookups (8, or 16 above 2^20).
int sort_keys_per_thread(int64_t n);
// Keys per radix tile for a batch of n lookups sorted on key_bits bits.
int sort_tile_keys(int64_t n, int key_bits);

// Upper bounds of the segment work lists for a batch of n lookups.
struct SegmentBounds {
  int64_t longs, chunks, items1;
};
SegmentBounds segment_bounds(int64_t n, int64_t long_threshold, int chunk, int short_max);

// A bounded wait of one workgroup for another: past `limit` empty polls it
// raises *err and stops waiting (limit 0: it gives up at once; the host sets
// that only to test that a failed call is reported).
struct WaitCtl {
  uint32_t* err;
  uint32_t limit;
};

struct BackwardLaunch {
  const void* indices;
  const void* offsets;
  const float* psw;
  const float* grad;
  void* weights;
  float* state;
  const TableMeta* meta;
  int64_t num_indices;
  int64_t num_bags;
  int32_t T, B, sum_dims;
  int32_t key_bits;
  int32_t mean, index64, dtype, adagrad;
  int32_t use_rec;
  int32_t vec;              // G_Y rows read as 16-byte chunks
  int32_t nch;              // chunk sets per lane in the segment kernels (1, 4 or 16)
  int32_t gshift;           // log2(lanes per gradient row) in the segment kernels
  int32_t per_table;        // short runs use each table's own lane-group width
  int32_t short_max;        // runs of at most this many lookups are short (a lane group's)
  int32_t front_queued;     // the run-length encoder queued the longer runs
  int32_t finish_in_items;  // seg_fused finishes the long runs (else seg_finalize does)
  int32_t xcd_runs;         // short runs in one contiguous range per XCD
  int32_t pstride;          // floats per partial row
  int32_t long_threshold;   // runs at least this long use split accumulation
  int32_t chunk;            // lookups per level-1 partial
  int32_t bucket_sort;      // two-digit ids: high-digit pass + bucket-local sort and RLE
  uint32_t spin_limit;      // polls before a waiting workgroup gives up
  uint32_t* error_mark;     // handle's device word: set when a call gave up (sticky)
  float lr, eps;
  int32_t* out_unique;      // optional run outputs
  int32_t* out_lengths;
  int32_t* out_num;
  BackwardBuffers buf;
};

// Zeroes the workspace's counters, digit counts and look-back status words.
hipError_t launch_init_workspace(const BackwardLaunch& a, hipStream_t stream,
                                 const KernelTimer* kt);
// The linearize kernel alone (workspace zeroed before).
hipError_t launch_linearize_kernel(const BackwardLaunch& a, hipStream_t stream,
                                   const KernelTimer* kt);
// launch_init_workspace, then the linearize kernel.
hipError_t launch_linearize(const BackwardLaunch& a, hipStream_t stream, const KernelTimer* kt);
// One launch that pools the gather tables of f (as launch_forward_gather) and
// linearizes the batch of b (its workspace zeroed before); for batches of at
// most kFusedMaxLookups lookups.
constexpr int64_t kFusedMaxLookups = int64_t{1} << 20;
hipError_t launch_forward_linearize(const ForwardLaunch& f, const BackwardLaunch& b,
                                    hipStream_t stream, const KernelTimer* kt);
// Sorts buf.keys[0]/vals[0]; returns the index (0 or 1) of the buffer pair
// that holds the sorted result.
hipError_t launch_radix_sort(const BackwardLaunch& a, hipStream_t stream, int* result_buffer,
                             const KernelTimer* kt);
hipError_t launch_run_length_encode(const BackwardLaunch& a, const uint32_t* sorted_keys,
                                    const uint32_t* sorted_vals, hipStream_t stream,
                                    const KernelTimer* kt);
// Sort and run-length encoding of the linearized batch in buf.keys[0] /
// buf.vals[0]: for ids of two radix digits (and a.bucket_sort), a pass on the
// high digit and the bucket-local sort with its run-length encoding; else the
// LSD passes and the RLE kernel.  Either way the sorted pair ends in buffer
// radix_passes() % 2 and the order is the same (stable on the id).
hipError_t launch_sort_encode(const BackwardLaunch& a, hipStream_t stream, const KernelTimer* kt);
// True when the grouping of this launch's batch takes the bucket-local sort
// (whose run-length encoding also queues the longer runs).
bool uses_bucket_sort(const BackwardLaunch& a);
constexpr int kLinBags = 128;  // bags per linearize tile
// Batches of at most this many linearize tiles: the linearize step also
// sorts each tile's lookups by the high digit (linearize_bucket) and the
// bucket-local sort gathers its buckets from the tiles' segments, so no radix
// pass runs (the gather keeps one segment per tile in LDS).
constexpr int kTileBucketMaxTiles = 256;
bool uses_tile_buckets(const BackwardLaunch& a);

hipError_t launch_segment_reduce_update(const BackwardLaunch& a, const uint32_t* sorted_keys,
                                        const uint32_t* sorted_vals, hipStream_t stream,
                                        const KernelTimer* kt);

// Row loads a forward lane group issues before it accumulates (shared by the
// kernel and the host planner that sizes sub-waves from the mean bag length).
constexpr int kFwdUnroll = 4;

// Tables whose metadata the segment kernels stage in LDS; handles with more
// tables read it from global memory and use one lane-group width for all.
constexpr int kSegLdsTables = 256;

// Largest embedding dimension handled.
constexpr int kMaxDim = 1024;

// Tile sizes shared by the planner (workspace sizing) and the kernels.
constexpr int kRleTile = 8192;
// Sorted positions per window of the bucket-local sort: a window takes the
// buckets of the high digit that start inside it.
constexpr int kBucketWindow = 2048;
// The windows' look-back status words come first in the RLE status region
// (rounded up to 4 words), then their 16-byte range records.
__host__ __device__ inline int64_t bucket_windows(int64_t n) {
  return (n + kBucketWindow - 1) / kBucketWindow;
}
__host__ __device__ inline uint32_t* bucket_window_table(uint32_t* rle_status, int64_t n) {
  return rle_status + ((bucket_windows(n) + 3) & ~int64_t{3});
}
// When the linearize step sorts each tile by the high digit (at most 1024
// buckets), a window takes a fixed range of buckets instead: the largest power
// of two, at most kBucketMaxPerWindow, that holds at most 3/4 of kBucketWindow
// lookups on average.  Windows of fixed bucket ranges are less even than
// windows of positions (a hot bucket's window keeps its other buckets), so
// they are kept smaller: on the 270k-lookup batch 4 / 8 / 16 buckets per
// window (about 1.1k / 2.1k / 4.2k lookups) took 28.3 / 35.9 / 150 us, the
// last because some windows outgrow LDS.  Its look-back status words are the
// windows' run counts at rle_status and their sizes at rle_status +
// kBucketMaxWindows.
constexpr int kBucketMaxPerWindow = 64;
constexpr int kBucketMaxWindows = 1024;
inline int buckets_per_window(int64_t n, int nbk) {
  const int64_t mean = nbk > 0 ? (n + nbk - 1) / nbk : n;
  int b = 1;
  while (b < kBucketMaxPerWindow && 2 * b * (mean > 0 ? mean : 1) * 4 <= 3 * kBucketWindow) b *= 2;
  return b;
}

// LSD radix sort plan for n keys of key_bits bits: the fewest passes of
// digits of at most kMaxRadixBits bits, the bits split evenly over the
// passes.  Digits of up to 8 bits use 256-thread tiles (one digit per
// thread); 9- and 10-bit digits use 1024-thread tiles of 4096 keys, again one
// digit per thread, so that the look-back keeps 16 status words in flight per
// digit (with several digits per thread a 10-bit pass measured twice as slow
// as an 8-bit one).  Wide digits pay only while a pass is bound by latency
// (batches of up to 2^20 lookups); larger batches are bound by bandwidth and
// sort with 8-bit digits.  Every per-pass table (digit counts, look-back
// status words) has radix_slots(bits) entries.
constexpr int kMaxRadixBits = 10;
constexpr int kMaxRadixPasses = 4;  // ids of up to 31 bits: at most 4 passes
// Words per tile row of linearize_bucket: segment bounds of the 2^kMaxRadixBits
// high digits and the tile's end.
constexpr int kTileRowWords = (1 << kMaxRadixBits) + 1;
constexpr int64_t kWideRadixMaxKeys = int64_t{1} << 20;
__host__ __device__ inline int radix_passes(int key_bits, int64_t n) {
  const int w = n <= kWideRadixMaxKeys ? kMaxRadixBits : 8;
  return (key_bits + w - 1) / w;
}
__host__ __device__ inline int radix_digit_bits(int key_bits, int64_t n) {
  const int p = radix_passes(key_bits, n);
  return (key_bits + p - 1) / p;
}
__host__ __device__ inline int radix_slots(int digit_bits) {
  return digit_bits > 8 ? 1024 : 256;  // the wide pass has 1024 digit slots
}
// Batches of more than 2^20 lookups (8-bit digits) sort with counted passes:
// each pass counts every tile's digits, scans the counts over the tiles and
// then places the tiles, with no look-back between tiles.
__host__ __device__ inline bool counted_passes(int64_t n) { return n > kWideRadixMaxKeys; }

}  // namespace tbe
