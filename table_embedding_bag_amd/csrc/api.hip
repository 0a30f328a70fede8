// api.hip -- host side of the C ABI declared in include/tbe.h: configuration
// checks, table layout, per-call launch planning, workspace carving,
// optional validation and profiling.  No exception leaves this file.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "common.hpp"
#include "count_backward.hpp"
#include "tbe.h"

using namespace tbe;

// The workspace of tbe_backward_update_no_alloc, for callers that cannot
// allocate: one copy per GPU the library runs on, held until the process
// ends.  In host code this name stands for the array, not for its device
// address: kernels and copies get the address that hipGetSymbolAddress
// returns for the current device (static_scratch_address below).
static __device__ __align__(256) unsigned char scratch[TBE_STATIC_SCRATCH_BYTES];

// What a tbe_forward_group call left in a workspace, for the
// tbe_backward_update_grouped call that must follow it on the same batch.
struct GroupRecord {
  const void* workspace;
  const void* indices;
  const void* offsets;
  const float* psw;
  int32_t B, index_dtype;
  int64_t n;
  int64_t long_threshold;  // the handle's option when the grouping was made
  bool bucket_sort;
  bool queued;             // its run-length encoding queued the longer runs
  bool count_matrix;       // the call takes the count-matrix backward (no grouping made)
};

struct tbe_handle {
  int32_t T = 0;
  std::vector<int64_t> rows;
  std::vector<int32_t> dims;
  int32_t dtype = 0, pooling = 0, optimizer = 0;
  uint32_t flags = 0;
  void* weights = nullptr;
  float* state = nullptr;
  int64_t sum_rows = 0;
  int32_t sum_dims = 0;
  int32_t dmax = 0;
  int32_t key_bits = 1;
  bool fwd_vec = false;  // every row is a whole number of 16-byte chunks
  bool bwd_vec = false;  // every dim is a multiple of 4 (16-byte gradient chunks)
  int device = 0;
  std::vector<TableMeta> meta_host;
  TableMeta* meta = nullptr;     // device copy
  uint32_t* flag = nullptr;      // device word for the validation kernel
  uint32_t* error_mark = nullptr;  // device word: a backward call's wait gave up (sticky)
  uint32_t spin_limit = 1u << 20;  // TBE_OPTION_SPIN_LIMIT
  void* static_scratch = nullptr;  // device address of `scratch` on this handle's device
  // count-matrix forward: eligible tables (device list), the other tables
  // (device list for the gather kernel) and the transposed-table buffer
  std::vector<HistTable> hist_host;
  std::vector<int32_t> gather_host;
  HistTable* hist = nullptr;
  int32_t* gather_list = nullptr;
  uint16_t* wt = nullptr;
  int32_t hist_etiles = 0, hist_dtiles = 0;
  int64_t wt_elems = 0;
  // count-matrix backward (TBE_FLAG_COUNT_BACKWARD): (table, 64-column slice)
  // units (device list) and the row groups they hold
  std::vector<CountUnit> cb_host;
  CountUnit* cb_units = nullptr;
  int64_t cb_groups = 0;
  // small tables pooled from LDS (TBE_OPTION_LDS_FORWARD): those tables
  // (device list, all with rows of 2^lds_gshift chunks), the other tables
  // (device list for the gather kernel), the largest such table's rows
  std::vector<int32_t> lds_host, lds_rest_host;
  int32_t* lds_list = nullptr;
  int32_t* lds_rest = nullptr;
  int32_t lds_gshift = 0;
  int64_t lds_max_rows = 0;
  bool lds_forward = true;
  int32_t num_cus = 256;
  int64_t weight_elems = 0;  // sum of rows * dims
  int64_t long_threshold = 256;
  bool bucket_sort = true;  // TBE_OPTION_SORT
  // TBE_FLAG_SPLIT_BAGS scratch: counters, segment list, split-bag list and
  // segment sums for at most split_cap segments of split_pstride floats
  char* split = nullptr;
  int64_t split_cap = 0;
  int32_t split_pstride = 0;
  // the caller's forward scratch (tbe_set_forward_scratch): the transposed
  // tables (wt) first, then the split-bag scratch; fscratch_bytes is what the
  // handle's paths need (0: none)
  size_t fscratch_bytes = 0;
  size_t fscratch_split_off = 0;
  bool fscratch_set = false;
  // groupings made by tbe_forward_group and not yet used, by workspace
  std::vector<GroupRecord> groups;
  // profiling: pairs of events handed to timed kernel launches (start and end
  // of that kernel), kept until tbe_stage_times reads them
  bool profile = false;
  std::vector<hipEvent_t> pool;
  std::vector<std::pair<size_t, const char*>> timed;  // start event index in pool, kernel name
  size_t used = 0;
};

namespace {

// Device address of `scratch` on each device, looked up once per device (with
// that device current) by the first tbe_create on it.
constexpr int kMaxDevices = 256;
std::mutex g_scratch_mutex;
void* g_scratch_address[kMaxDevices] = {};

void* static_scratch_address(int device) {
  if (device < 0 || device >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_address[device]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) == hipSuccess) g_scratch_address[device] = p;
  }
  return g_scratch_address[device];
}

constexpr int kChunk = 256;       // lookups per level-1 partial of a long run
constexpr size_t kAlign = 256;

int ceil_log2(int64_t x) {
  int b = 0;
  while ((int64_t{1} << b) < x) ++b;
  return b;
}

int64_t next_pow2(int64_t x) { return int64_t{1} << ceil_log2(x < 1 ? 1 : x); }

int storage_bytes(int dtype) { return dtype == TBE_F32 ? 4 : 2; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

tbe_status from_hip(hipError_t e) { return e == hipSuccess ? TBE_OK : TBE_ERR_HIP; }

// --- profiling -------------------------------------------------------------

constexpr size_t kMaxMarks = size_t{1} << 16;

bool take_events(void* ctx, const char* name, hipEvent_t* start, hipEvent_t* stop) {
  auto* h = static_cast<tbe_handle*>(ctx);
  if (!h->profile || h->timed.size() >= kMaxMarks) return false;
  while (h->pool.size() < h->used + 2) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) return false;
    h->pool.push_back(e);
  }
  *start = h->pool[h->used];
  *stop = h->pool[h->used + 1];
  h->timed.emplace_back(h->used, name);
  h->used += 2;
  return true;
}

// --- validation kernel -----------------------------------------------------

template <typename IT>
__global__ __launch_bounds__(kBlock) void validate_batch(const IT* idx, const IT* off,
                                                         const TableMeta* meta, int32_t B,
                                                         int64_t nbags, int64_t n,
                                                         uint32_t* flag) {
  const int64_t k = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
  if (k > nbags) return;
  bool bad = false;
  if (k == 0 && off[0] != 0) bad = true;
  if (k == nbags) {
    if (static_cast<int64_t>(off[nbags]) != n) bad = true;
  } else {
    const int64_t lo = off[k], hi = off[k + 1];
    if (hi < lo || lo < 0 || hi > n) {
      bad = true;
    } else {
      const int64_t E = meta[k / B].rows;
      for (int64_t i = lo; i < hi; ++i) {
        const int64_t x = idx[i];
        if (x < 0 || x >= E) {
          bad = true;
          break;
        }
      }
    }
  }
  if (bad) atomicOr(flag, 1u);
}

__global__ void fill_u32(uint32_t* p, uint32_t v, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

tbe_status run_validation(tbe_handle* h, int32_t B, const void* indices, const void* offsets,
                          int32_t index_dtype, int64_t n, hipStream_t s) {
  const int64_t nbags = static_cast<int64_t>(h->T) * B;
  hipLaunchKernelGGL(fill_u32, dim3(1), dim3(64), 0, s, h->flag, 0u, int64_t{1});
  const unsigned blocks = static_cast<unsigned>((nbags + 1 + kBlock - 1) / kBlock);
  if (index_dtype == TBE_I64)
    hipLaunchKernelGGL(validate_batch<int64_t>, dim3(blocks), dim3(kBlock), 0, s,
                       static_cast<const int64_t*>(indices), static_cast<const int64_t*>(offsets),
                       h->meta, B, nbags, n, h->flag);
  else
    hipLaunchKernelGGL(validate_batch<int32_t>, dim3(blocks), dim3(kBlock), 0, s,
                       static_cast<const int32_t*>(indices), static_cast<const int32_t*>(offsets),
                       h->meta, B, nbags, n, h->flag);
  if (hipGetLastError() != hipSuccess) return TBE_ERR_HIP;
  uint32_t host_flag = 0;
  if (hipMemcpyAsync(&host_flag, h->flag, sizeof(host_flag), hipMemcpyDeviceToHost, s) !=
      hipSuccess)
    return TBE_ERR_HIP;
  if (hipStreamSynchronize(s) != hipSuccess) return TBE_ERR_HIP;
  return host_flag ? TBE_ERR_INDEX_OUT_OF_RANGE : TBE_OK;
}

tbe_status check_batch_args(const tbe_handle* h, int32_t B, const void* indices,
                            const void* offsets, int32_t index_dtype, int64_t n) {
  if (!h || B < 0 || n < 0) return TBE_ERR_INVALID_ARGUMENT;
  if (index_dtype != TBE_I32 && index_dtype != TBE_I64) return TBE_ERR_INVALID_ARGUMENT;
  if (B > 0 && !offsets) return TBE_ERR_INVALID_ARGUMENT;
  if (n > 0 && !indices) return TBE_ERR_INVALID_ARGUMENT;
  // lookup ids and the sort's chained counts are 30-bit on the device
  if (n >= (int64_t{1} << 30)) return TBE_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(h->T) * B >= 0x7FFFFFFF) return TBE_ERR_UNSUPPORTED;
  return TBE_OK;
}

// --- backward workspace layout ---------------------------------------------

struct Carve {
  size_t off = 0;
  size_t take(size_t bytes) {
    const size_t o = off;
    off += (bytes + kAlign - 1) / kAlign * kAlign;
    return o;
  }
};

// Skew balancing (TBE_FLAG_SPLIT_BAGS): bags longer than kSplitLen lookups
// are pooled in segments of kSplitLen.
constexpr int32_t kSplitLen = 128;
constexpr int64_t kSplitMaxSegments = int64_t{1} << 18;
constexpr int64_t kSplitScratchBytes = int64_t{64} << 20;

// Scratch layout: counters (256 bytes), segment list, split-bag list, sums.
size_t split_bytes(int64_t cap, int32_t pstride) {
  return 256 + static_cast<size_t>(cap) * (8 + 16 + 4 * static_cast<size_t>(pstride));
}

struct BwdPlan {
  int64_t n = 0;
  int sort_tiles = 0, rle_tiles = 0;
  int64_t long_ub = 0, chunks_ub = 0, items1_ub = 0;
  int32_t pstride = 0;
  int32_t nch = 1, gshift = 0;
  int32_t short_max = 1;  // longest short run: the lane group with 16-byte chunks if every
                          // dim allows them (the same for a forward_group and its backward)
  bool vec = false;
  int passes = 1, slots = 256;
  int64_t zero_words = 0;
  size_t o_keys[2], o_vals[2], o_rec, o_zero, o_uniq, o_start, o_first, o_longs, o_long_keys,
      o_items1, o_p1, o_truns, o_rows;
  int64_t row_words = 0;
  int32_t first_stride = 1;
  bool per_table = false;
  size_t bytes = 0;
};

// Bag slices of the count-matrix backward: about 1024 workgroups (one per
// CU four times over; every slice adds a pass over the weights' partial sums
// in the update), at least one 32-bag step per slice.
int count_slices(const tbe_handle* h, int32_t B) {
  const int64_t g = std::max<int64_t>(1, h->cb_groups);
  int64_t s = (1024 + g - 1) / g;
  s = std::min<int64_t>(s, std::max<int64_t>(1, B / 32));
  return static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(s, 64)));
}

// Whether a backward call of this handle takes the count-matrix path.
bool uses_count_backward(const tbe_handle* h, const float* psw) {
  return !h->cb_host.empty() && psw == nullptr;
}

bool plan_backward(const tbe_handle* h, int32_t B, int64_t n, bool vec, int64_t long_threshold,
                   BwdPlan* p) {
  p->n = n;
  p->vec = vec;
  const int ve = vec ? 4 : 1;
  const int64_t c = (h->dmax + ve - 1) / ve;  // chunks per gradient row
  if (c <= kWave) {
    p->nch = 1;
    p->gshift = ceil_log2(next_pow2(c));
  } else {
    p->gshift = 6;
    const int64_t sets = (c + kWave - 1) / kWave;
    if (vec) {
      if (sets > 4) return false;
      p->nch = 4;
    } else {
      if (sets > 16) return false;
      p->nch = 16;
    }
  }
  p->pstride = static_cast<int32_t>((h->dmax + 3) / 4 * 4);
  const int64_t sort_tile = sort_tile_keys(n, h->key_bits);
  p->sort_tiles = static_cast<int>((n + sort_tile - 1) / sort_tile);
  // segment bounds of a linearize step that sorts each tile by the high digit
  const int64_t lin_tiles = (static_cast<int64_t>(h->T) * B + kLinBags - 1) / kLinBags;
  p->row_words = lin_tiles <= kTileBucketMaxTiles ? lin_tiles * kTileRowWords : 0;
  // look-back status words of the RLE kernel, or those of the bucket-local
  // sort's windows followed by the windows' 4-word range records
  p->rle_tiles = std::max(5 * static_cast<int>((n + kBucketWindow - 1) / kBucketWindow) + 4,
                          2 * kBucketMaxWindows);
  p->passes = radix_passes(h->key_bits, n);
  p->slots = radix_slots(radix_digit_bits(h->key_bits, n));
  {
    const int ve_h = h->bwd_vec ? 4 : 1;
    const int64_t ch = (h->dmax + ve_h - 1) / ve_h;
    p->short_max = 1 << (ch <= kWave ? ceil_log2(next_pow2(ch)) : 6);
  }
  const SegmentBounds ub = segment_bounds(n, long_threshold, kChunk, p->short_max);
  p->long_ub = ub.longs;
  p->chunks_ub = ub.chunks;
  p->items1_ub = ub.items1;
  p->zero_words = kNumCounters + kNumTickets + int64_t{p->passes} * p->slots +
                  int64_t{p->passes} * p->sort_tiles * p->slots + p->rle_tiles +
                  p->chunks_ub / kFinPiece + 1 + p->long_ub;
  Carve cv;
  for (int i = 0; i < 2; ++i) {
    p->o_keys[i] = cv.take(4 * static_cast<size_t>(n));
    p->o_vals[i] = cv.take(4 * static_cast<size_t>(n));
  }
  p->o_rec = cv.take(8 * static_cast<size_t>(n));
  p->o_zero = cv.take(4 * static_cast<size_t>(p->zero_words));
  p->o_uniq = cv.take(4 * static_cast<size_t>(n));
  p->o_start = cv.take(4 * static_cast<size_t>(n + 1));
  p->first_stride = n <= kWideRadixMaxKeys ? 4 : 1;
  p->o_first = cv.take(4 * static_cast<size_t>(n) * p->first_stride);
  p->o_longs = cv.take(16 * static_cast<size_t>(p->long_ub));
  p->o_long_keys = cv.take(4 * static_cast<size_t>(p->long_ub));
  p->o_items1 = cv.take(8 * static_cast<size_t>(p->items1_ub));
  p->o_p1 = cv.take(4 * static_cast<size_t>(p->pstride) * p->chunks_ub);
  p->o_truns = cv.take(4 * static_cast<size_t>(h->T + 1));
  p->o_rows = cv.take(4 * static_cast<size_t>(p->row_words));
  // short runs in lane groups of each table's own width, when some table's
  // rows are narrower than the widest (metadata staged in LDS)
  if (h->T <= kSegLdsTables)
    for (int t = 0; t < h->T; ++t)
      if (((h->meta_host[t].bwd_gshift >> (vec ? 0 : 8)) & 0xFF) < p->gshift) p->per_table = true;
  p->bytes = cv.off;
  return true;
}

// The launch description of a backward call on a planned workspace.
void fill_backward(const tbe_handle* h, int32_t B, const void* indices, const void* offsets,
                   int32_t index_dtype, int64_t n, const float* psw, const float* grad_output,
                   float lr, float eps, void* workspace, const tbe_runs* runs, bool vec,
                   int64_t long_threshold, bool bucket_sort, const BwdPlan& p,
                   BackwardLaunch* out) {
  char* w = static_cast<char*>(workspace);
  BackwardLaunch& a = *out;
  a = BackwardLaunch{};
  a.indices = indices;
  a.offsets = offsets;
  a.psw = psw;
  a.grad = grad_output;
  a.weights = h->weights;
  a.state = h->state;
  a.meta = h->meta;
  a.num_indices = n;
  a.num_bags = static_cast<int64_t>(h->T) * B;
  a.T = h->T;
  a.B = B;
  a.sum_dims = h->sum_dims;
  a.key_bits = h->key_bits;
  a.mean = h->pooling == TBE_POOL_MEAN;
  a.index64 = index_dtype == TBE_I64;
  a.dtype = h->dtype;
  a.adagrad = h->optimizer == TBE_OPT_ROWWISE_ADAGRAD;
  a.use_rec = (psw != nullptr) || a.mean;
  a.vec = vec;
  a.nch = p.nch;
  a.gshift = p.gshift;
  a.short_max = p.short_max;
  a.per_table = p.per_table ? 1 : 0;
  a.pstride = p.pstride;
  a.long_threshold = static_cast<int32_t>(std::min<int64_t>(long_threshold, 0x7FFFFFFF));
  a.finish_in_items = n <= kFinishInItemsMaxKeys ? 1 : 0;
  a.xcd_runs = int64_t{4} * B * h->sum_dims <= 8 * kXcdL2Bytes ? 1 : 0;
  a.bucket_sort = bucket_sort ? 1 : 0;
  a.spin_limit = h->spin_limit;
  a.error_mark = h->error_mark;
  a.chunk = kChunk;
  a.lr = lr;
  a.eps = eps;
  if (runs) {
    a.out_unique = runs->unique_ids;
    a.out_lengths = runs->run_lengths;
    a.out_num = runs->num_unique;
  }
  BackwardBuffers& b = a.buf;
  for (int i = 0; i < 2; ++i) {
    b.keys[i] = reinterpret_cast<uint32_t*>(w + p.o_keys[i]);
    b.vals[i] = reinterpret_cast<uint32_t*>(w + p.o_vals[i]);
  }
  b.rec = reinterpret_cast<uint2*>(w + p.o_rec);
  b.counters = reinterpret_cast<uint32_t*>(w + p.o_zero);
  b.tickets = b.counters + kNumCounters;
  b.digit_hist = b.tickets + kNumTickets;
  b.rle_status = b.digit_hist + p.passes * p.slots;
  b.piece_tickets = b.rle_status + p.rle_tiles;
  b.run_tickets = b.piece_tickets + p.chunks_ub / kFinPiece + 1;
  // last, so that a call whose linearize step sorts the tiles (no radix pass)
  // clears only what comes before
  b.sort_status = b.run_tickets + p.long_ub;
  b.zero_words = p.zero_words;
  b.unique_keys = reinterpret_cast<uint32_t*>(w + p.o_uniq);
  b.run_start = reinterpret_cast<uint32_t*>(w + p.o_start);
  b.run_first = reinterpret_cast<uint32_t*>(w + p.o_first);
  b.first_stride = p.first_stride;
  b.longs = reinterpret_cast<uint4*>(w + p.o_longs);
  b.long_keys = reinterpret_cast<uint32_t*>(w + p.o_long_keys);
  b.items1 = reinterpret_cast<uint2*>(w + p.o_items1);
  b.partial1 = reinterpret_cast<float*>(w + p.o_p1);
  b.table_runs = reinterpret_cast<uint32_t*>(w + p.o_truns);
  b.tile_rows = reinterpret_cast<uint32_t*>(w + p.o_rows);
}

// The grouping (linearize, sort, run-length encoding) of a backward call.
// The sorted pair ends in buffer passes % 2.
hipError_t launch_front(const BackwardLaunch& a, hipStream_t s, const KernelTimer* kt) {
  hipError_t e = launch_linearize(a, s, kt);
  if (e != hipSuccess) return e;
  return launch_sort_encode(a, s, kt);
}

// The count-matrix backward of a call (every table small, no per-sample
// weights): the product, the update of touched rows, the runs if asked.
tbe_status count_backward_impl(tbe_handle* h, int32_t B, const void* indices, const void* offsets,
                               int32_t index_dtype, int64_t n, const float* grad_output, float lr,
                               float eps, void* workspace, size_t workspace_bytes,
                               const tbe_runs* runs, hipStream_t s, bool with_front, bool timed);

// Reads and clears the handle's error mark once the stream's work is done.
tbe_status check_error_mark(tbe_handle* h, hipStream_t s) {
  uint32_t mark = 0;
  if (hipMemcpyAsync(&mark, h->error_mark, sizeof mark, hipMemcpyDeviceToHost, s) != hipSuccess)
    return TBE_ERR_HIP;
  if (hipStreamSynchronize(s) != hipSuccess) return TBE_ERR_HIP;
  if (mark == 0u) return TBE_OK;
  hipLaunchKernelGGL(fill_u32, dim3(1), dim3(64), 0, s, h->error_mark, 0u, int64_t{1});
  if (hipGetLastError() != hipSuccess) return TBE_ERR_HIP;
  return TBE_ERR_DEVICE_WAIT;
}

constexpr size_t kMaxGroupRecords = 64;

tbe_status count_backward_impl(tbe_handle* h, int32_t B, const void* indices, const void* offsets,
                               int32_t index_dtype, int64_t n, const float* grad_output, float lr,
                               float eps, void* workspace, size_t workspace_bytes,
                               const tbe_runs* runs, hipStream_t s, bool with_front, bool timed) {
  auto rec = std::find_if(h->groups.begin(), h->groups.end(),
                          [&](const GroupRecord& g) { return g.workspace == workspace; });
  if (!with_front &&
      (rec == h->groups.end() || !rec->count_matrix || rec->indices != indices ||
       rec->offsets != offsets || rec->psw != nullptr || rec->B != B || rec->n != n ||
       rec->index_dtype != index_dtype))
    return TBE_ERR_INVALID_ARGUMENT;
  const int slices = count_slices(h, B);
  const size_t need = count_backward_bytes(h->weight_elems, h->sum_rows, slices);
  if (workspace_bytes < need) return TBE_ERR_WORKSPACE_TOO_SMALL;
  if (h->flags & TBE_FLAG_VALIDATE) {
    const tbe_status st = run_validation(h, B, indices, offsets, index_dtype, n, s);
    if (st != TBE_OK) return st;
  }
  if (rec != h->groups.end()) h->groups.erase(rec);
  KernelTimer timer{h, take_events};
  const KernelTimer* kt = (h->profile && timed) ? &timer : nullptr;
  CountLaunch c{};
  c.indices = indices;
  c.offsets = offsets;
  c.grad = grad_output;
  c.weights = h->weights;
  c.state = h->state;
  c.meta = h->meta;
  c.units = h->cb_units;
  c.nunits = static_cast<int32_t>(h->cb_host.size());
  c.T = h->T;
  c.B = B;
  c.sum_dims = h->sum_dims;
  c.slices = slices;
  c.mean = h->pooling == TBE_POOL_MEAN;
  c.index64 = index_dtype == TBE_I64;
  c.dtype = h->dtype;
  c.adagrad = h->optimizer == TBE_OPT_ROWWISE_ADAGRAD;
  c.lr = lr;
  c.eps = eps;
  c.sum_rows = h->sum_rows;
  char* w = static_cast<char*>(workspace);
  auto up = [](size_t x) { return (x + kAlign - 1) / kAlign * kAlign; };
  c.partial = reinterpret_cast<float*>(w);
  c.counts = reinterpret_cast<uint32_t*>(w + up(4 * static_cast<size_t>(h->weight_elems) * slices));
  c.scan = c.counts + up(4 * static_cast<size_t>(h->sum_rows) * slices) / 4;
  if (runs) {
    c.out_unique = runs->unique_ids;
    c.out_lengths = runs->run_lengths;
    c.out_num = runs->num_unique;
  }
  return from_hip(launch_count_backward(c, s, kt));
}

std::vector<GroupRecord>::iterator find_group(tbe_handle* h, const void* workspace) {
  return std::find_if(h->groups.begin(), h->groups.end(),
                      [&](const GroupRecord& g) { return g.workspace == workspace; });
}

tbe_status backward_impl(tbe_handle* h, int32_t B, const void* indices, const void* offsets,
                         int32_t index_dtype, int64_t n, const float* psw,
                         const float* grad_output, float lr, float eps, void* workspace,
                         size_t workspace_bytes, const tbe_runs* runs, hipStream_t s,
                         bool with_front, bool timed = true) {
  tbe_status st = check_batch_args(h, B, indices, offsets, index_dtype, n);
  if (st != TBE_OK) return st;
  if (B > 0 && (!grad_output || !aligned(grad_output, 4))) return TBE_ERR_INVALID_ARGUMENT;
  if (runs && (!runs->num_unique || (n > 0 && (!runs->unique_ids || !runs->run_lengths))))
    return TBE_ERR_INVALID_ARGUMENT;
  if (!std::isfinite(lr) || !std::isfinite(eps)) return TBE_ERR_INVALID_ARGUMENT;
  try {
    if (B == 0 || n == 0) {
      if (runs) {
        hipLaunchKernelGGL(fill_u32, dim3(1), dim3(64), 0, s,
                           reinterpret_cast<uint32_t*>(runs->num_unique), 0u, int64_t{1});
        return from_hip(hipGetLastError());
      }
      return TBE_OK;
    }
    const bool vec = h->bwd_vec && aligned(grad_output, 16);
    if (!workspace || !aligned(workspace, kAlign)) return TBE_ERR_INVALID_ARGUMENT;
    if (uses_count_backward(h, psw))
      return count_backward_impl(h, B, indices, offsets, index_dtype, n, grad_output, lr, eps,
                                 workspace, workspace_bytes, runs, s, with_front, timed);
    // the grouped variant takes the grouping that tbe_forward_group made of this
    // very batch in this workspace, with the options in force at that time
    int64_t threshold = h->long_threshold;
    bool bucket_sort = h->bucket_sort, queued = false;
    auto rec = find_group(h, workspace);
    if (!with_front) {
      if (rec == h->groups.end() || rec->indices != indices || rec->offsets != offsets ||
          rec->psw != psw || rec->B != B || rec->n != n || rec->index_dtype != index_dtype)
        return TBE_ERR_INVALID_ARGUMENT;
      threshold = rec->long_threshold;
      bucket_sort = rec->bucket_sort;
      queued = rec->queued;
    }
    BwdPlan p;
    if (!plan_backward(h, B, n, vec, threshold, &p)) return TBE_ERR_UNSUPPORTED;
    if (workspace_bytes < p.bytes) return TBE_ERR_WORKSPACE_TOO_SMALL;
    if (h->flags & TBE_FLAG_VALIDATE) {
      st = run_validation(h, B, indices, offsets, index_dtype, n, s);
      if (st != TBE_OK) return st;
    }
    // from here on the workspace is this call's: a grouping left in it is used
    // (grouped) or overwritten (plain)
    if (rec != h->groups.end()) h->groups.erase(rec);
    KernelTimer timer{h, take_events};
    const KernelTimer* kt = (h->profile && timed) ? &timer : nullptr;
    BackwardLaunch a;
    fill_backward(h, B, indices, offsets, index_dtype, n, psw, grad_output, lr, eps, workspace,
                  runs, vec, threshold, bucket_sort, p, &a);
    a.front_queued = (with_front ? uses_bucket_sort(a) : queued) ? 1 : 0;
    if (with_front) {
      const hipError_t e = launch_front(a, s, kt);
      if (e != hipSuccess) return TBE_ERR_HIP;
    }
    st = from_hip(launch_segment_reduce_update(a, a.buf.keys[p.passes % 2],
                                               a.buf.vals[p.passes % 2], s, kt));
    if (st == TBE_OK && (h->flags & TBE_FLAG_VALIDATE)) st = check_error_mark(h, s);
    return st;
  } catch (...) {
    return TBE_ERR_OUT_OF_MEMORY;
  }
}

}  // namespace

extern "C" {

const char* tbe_status_string(tbe_status status) {
  switch (status) {
    case TBE_OK: return "ok";
    case TBE_ERR_INVALID_ARGUMENT: return "invalid argument";
    case TBE_ERR_UNSUPPORTED: return "unsupported configuration";
    case TBE_ERR_INDEX_OUT_OF_RANGE: return "row id or offsets out of range";
    case TBE_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case TBE_ERR_HIP: return "HIP runtime error";
    case TBE_ERR_OUT_OF_MEMORY: return "out of device memory";
    case TBE_ERR_DEVICE_WAIT: return "a device-side wait gave up; that backward update was skipped";
  }
  return "unknown status";
}

int32_t tbe_abi_version(void) { return TBE_ABI_VERSION; }

tbe_status tbe_create(const tbe_config* cfg, void* weights, float* optim_state, tbe_handle** out) {
  if (!out) return TBE_ERR_INVALID_ARGUMENT;
  *out = nullptr;
  if (!cfg || !weights || cfg->num_tables <= 0 || !cfg->rows || !cfg->dims)
    return TBE_ERR_INVALID_ARGUMENT;
  if (cfg->weight_dtype < TBE_F32 || cfg->weight_dtype > TBE_BF16) return TBE_ERR_INVALID_ARGUMENT;
  if (cfg->pooling != TBE_POOL_SUM && cfg->pooling != TBE_POOL_MEAN)
    return TBE_ERR_INVALID_ARGUMENT;
  if (cfg->optimizer != TBE_OPT_SGD && cfg->optimizer != TBE_OPT_ROWWISE_ADAGRAD)
    return TBE_ERR_INVALID_ARGUMENT;
  if (cfg->optimizer == TBE_OPT_ROWWISE_ADAGRAD && !optim_state) return TBE_ERR_INVALID_ARGUMENT;
  if (cfg->flags & ~63u) return TBE_ERR_INVALID_ARGUMENT;
  if ((cfg->flags & TBE_FLAG_NO_HISTOGRAM) &&
      (cfg->flags & (TBE_FLAG_FORCE_HISTOGRAM | TBE_FLAG_HISTOGRAM)))
    return TBE_ERR_INVALID_ARGUMENT;
  const int sb = storage_bytes(cfg->weight_dtype);
  if (!aligned(weights, 16)) return TBE_ERR_INVALID_ARGUMENT;
  int64_t sum_rows = 0, sum_dims = 0;
  for (int t = 0; t < cfg->num_tables; ++t) {
    if (cfg->rows[t] < 1 || cfg->dims[t] < 1 || cfg->dims[t] > kMaxDim)
      return TBE_ERR_INVALID_ARGUMENT;
    sum_rows += cfg->rows[t];
    sum_dims += cfg->dims[t];
    if (sum_rows > 0x7FFFFFFF || sum_dims > 0x7FFFFFFF) return TBE_ERR_UNSUPPORTED;
  }

  tbe_handle* h = nullptr;
  try {
    h = new tbe_handle();
    h->T = cfg->num_tables;
    h->rows.assign(cfg->rows, cfg->rows + h->T);
    h->dims.assign(cfg->dims, cfg->dims + h->T);
    h->dtype = cfg->weight_dtype;
    h->pooling = cfg->pooling;
    h->optimizer = cfg->optimizer;
    h->flags = cfg->flags;
    h->weights = weights;
    h->state = cfg->optimizer == TBE_OPT_ROWWISE_ADAGRAD ? optim_state : nullptr;
    h->sum_rows = sum_rows;
    h->sum_dims = static_cast<int32_t>(sum_dims);
    h->key_bits = std::max(1, ceil_log2(sum_rows));
    h->fwd_vec = true;
    h->bwd_vec = true;
    for (int t = 0; t < h->T; ++t) {
      h->dmax = std::max(h->dmax, h->dims[t]);
      if ((h->dims[t] * sb) % 16 != 0) h->fwd_vec = false;
      if (h->dims[t] % 4 != 0) h->bwd_vec = false;
    }
    const int fwd_ve = h->fwd_vec ? 16 / sb : 1;
    h->meta_host.resize(h->T);
    int64_t woff = 0, roff = 0, doff = 0;
    for (int t = 0; t < h->T; ++t) {
      TableMeta& m = h->meta_host[t];
      std::memset(&m, 0, sizeof m);
      m.woff = woff;
      m.roff = static_cast<int32_t>(roff);
      m.rows = static_cast<int32_t>(h->rows[t]);
      m.dim = h->dims[t];
      m.doff = static_cast<int32_t>(doff);
      const int64_t chunks = (h->dims[t] + fwd_ve - 1) / fwd_ve;
      m.fwd_gshift = ceil_log2(next_pow2(std::min<int64_t>(chunks, kWave)));
      const int64_t gchunks4 = (h->dims[t] + 3) / 4, gchunks1 = h->dims[t];
      m.bwd_gshift = ceil_log2(next_pow2(std::min<int64_t>(gchunks4, kWave))) |
                     (ceil_log2(next_pow2(std::min<int64_t>(gchunks1, kWave))) << 8);
      woff += h->rows[t] * h->dims[t];
      roff += h->rows[t];
      doff += h->dims[t];
    }
    // count-matrix forward eligibility (16-bit storage, small tables, dims in
    // 16-column MFMA tiles, 16-byte aligned rows)
    int64_t wt_off = 0;
    const bool use_hist =
        h->dtype != TBE_F32 && (h->flags & (TBE_FLAG_HISTOGRAM | TBE_FLAG_FORCE_HISTOGRAM));
    for (int t = 0; t < h->T; ++t) {
      const TableMeta& m = h->meta_host[t];
      const bool ok = use_hist && m.rows <= kHistMaxRows && m.dim <= kHistMaxDim &&
                      m.dim % 16 == 0 && m.woff % 8 == 0;
      if (!ok) {
        if (h->flags & TBE_FLAG_FORCE_HISTOGRAM) {
          delete h;
          return TBE_ERR_UNSUPPORTED;
        }
        h->gather_host.push_back(t);
        continue;
      }
      HistTable ht{};
      ht.table = t;
      ht.epad = (m.rows + kHistKc - 1) / kHistKc * kHistKc;
      ht.wt_off = wt_off;
      wt_off += static_cast<int64_t>(ht.epad) * m.dim;
      h->hist_host.push_back(ht);
      h->hist_etiles = std::max(h->hist_etiles, ht.epad / 64);
      h->hist_dtiles = std::max(h->hist_dtiles, (m.dim + 63) / 64);
    }
    h->wt_elems = wt_off;
    h->weight_elems = woff;
    // LDS-pooled small tables (not with the count-matrix forward): those of
    // the most common row width among the qualifying ones
    if (!use_hist && h->fwd_vec && h->dtype != TBE_F32) {
      auto fits = [&](int t) {
        const TableMeta& m = h->meta_host[t];
        return m.fwd_gshift >= kLdsFwdMinGshift && m.fwd_gshift <= kLdsFwdMaxGshift &&
               (h->rows[t] << m.fwd_gshift) * 16 <= kLdsFwdBytes;
      };
      int count[kLdsFwdMaxGshift + 1] = {};
      for (int t = 0; t < h->T; ++t)
        if (fits(t)) ++count[h->meta_host[t].fwd_gshift];
      int best = kLdsFwdMaxGshift;
      for (int g = kLdsFwdMaxGshift; g >= kLdsFwdMinGshift; --g)
        if (count[g] > count[best]) best = g;
      if (count[best] > 0) {
        h->lds_gshift = best;
        for (int t = 0; t < h->T; ++t) {
          if (fits(t) && h->meta_host[t].fwd_gshift == best) {
            h->lds_host.push_back(t);
            h->lds_max_rows = std::max(h->lds_max_rows, h->rows[t]);
          } else {
            h->lds_rest_host.push_back(t);
          }
        }
      }
    }
    // count-matrix backward: every table at most kCbMaxRows rows, dims in
    // 16-column MFMA tiles up to kCbMaxDim
    if (h->flags & TBE_FLAG_COUNT_BACKWARD) {
      for (int t = 0; t < h->T; ++t) {
        const TableMeta& m = h->meta_host[t];
        if (m.rows > kCbMaxRows || m.dim % 16 != 0 || m.dim > kCbMaxDim) {
          delete h;
          return TBE_ERR_UNSUPPORTED;
        }
        for (int c0 = 0; c0 < m.dim; c0 += kCbCols) {
          h->cb_host.push_back(CountUnit{t, c0});
          h->cb_groups += (m.rows + kCbGroupRows - 1) / kCbGroupRows;
        }
      }
    }
  } catch (...) {
    delete h;
    return TBE_ERR_OUT_OF_MEMORY;
  }

  if (hipGetDevice(&h->device) != hipSuccess) {
    delete h;
    return TBE_ERR_HIP;
  }
  // null if the lookup fails: only tbe_backward_update_no_alloc needs it, and
  // it then returns TBE_ERR_HIP
  h->static_scratch = static_scratch_address(h->device);
  // one device block: table metadata | validation flag | count-matrix table
  // list | gather table list
  auto up = [](size_t x) { return (x + kAlign - 1) / kAlign * kAlign; };
  const size_t meta_bytes = sizeof(TableMeta) * static_cast<size_t>(h->T);
  const size_t flag_off = up(meta_bytes);
  const size_t hist_off = flag_off + kAlign;
  const size_t hist_bytes = sizeof(HistTable) * h->hist_host.size();
  const size_t gather_off = hist_off + up(hist_bytes);
  const size_t gather_bytes = sizeof(int32_t) * h->gather_host.size();
  const size_t cb_off = gather_off + up(gather_bytes);
  const size_t cb_bytes = sizeof(CountUnit) * h->cb_host.size();
  const size_t lds_off = cb_off + up(cb_bytes);
  const size_t lds_bytes = sizeof(int32_t) * h->lds_host.size();
  const size_t rest_off = lds_off + up(lds_bytes);
  const size_t rest_bytes = sizeof(int32_t) * h->lds_rest_host.size();
  const size_t block_bytes = rest_off + up(rest_bytes);
  void* block = nullptr;
  if (hipMalloc(&block, block_bytes) != hipSuccess) {
    delete h;
    return TBE_ERR_OUT_OF_MEMORY;
  }
  char* base = static_cast<char*>(block);
  h->meta = static_cast<TableMeta*>(block);
  h->flag = reinterpret_cast<uint32_t*>(base + flag_off);
  h->error_mark = reinterpret_cast<uint32_t*>(base + flag_off + 128);
  h->hist = hist_bytes ? reinterpret_cast<HistTable*>(base + hist_off) : nullptr;
  h->gather_list = gather_bytes ? reinterpret_cast<int32_t*>(base + gather_off) : nullptr;
  h->cb_units = cb_bytes ? reinterpret_cast<CountUnit*>(base + cb_off) : nullptr;
  h->lds_list = lds_bytes ? reinterpret_cast<int32_t*>(base + lds_off) : nullptr;
  h->lds_rest = rest_bytes ? reinterpret_cast<int32_t*>(base + rest_off) : nullptr;
  bool ok = hipMemset(block, 0, block_bytes) == hipSuccess;
  if (ok)
    ok = hipMemcpy(h->meta, h->meta_host.data(), meta_bytes, hipMemcpyHostToDevice) == hipSuccess;
  if (ok && hist_bytes)
    ok = hipMemcpy(h->hist, h->hist_host.data(), hist_bytes, hipMemcpyHostToDevice) == hipSuccess;
  if (ok && gather_bytes)
    ok = hipMemcpy(h->gather_list, h->gather_host.data(), gather_bytes, hipMemcpyHostToDevice) ==
         hipSuccess;
  if (ok && cb_bytes)
    ok = hipMemcpy(h->cb_units, h->cb_host.data(), cb_bytes, hipMemcpyHostToDevice) == hipSuccess;
  if (ok && lds_bytes)
    ok = hipMemcpy(h->lds_list, h->lds_host.data(), lds_bytes, hipMemcpyHostToDevice) == hipSuccess;
  if (ok && rest_bytes)
    ok = hipMemcpy(h->lds_rest, h->lds_rest_host.data(), rest_bytes, hipMemcpyHostToDevice) ==
         hipSuccess;
  if (ok) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, h->device) ==
            hipSuccess &&
        cus > 0)
      h->num_cus = cus;
  }
  if (!ok) {
    (void)hipFree(block);
    delete h;
    return TBE_ERR_HIP;
  }
  // the forward's opt-in paths take their scratch from the caller
  // (tbe_set_forward_scratch): the transposed tables, then the split-bag sums
  if (h->flags & TBE_FLAG_SPLIT_BAGS) {
    h->split_pstride = (h->dmax + 3) / 4 * 4;
    h->split_cap = std::min<int64_t>(kSplitMaxSegments,
                                     kSplitScratchBytes / (4 * int64_t{h->split_pstride})) /
                   16 * 16;  // keeps the 16-byte split-bag records aligned
  }
  h->fscratch_split_off = up(sizeof(uint16_t) * static_cast<size_t>(h->wt_elems));
  h->fscratch_bytes =
      h->fscratch_split_off +
      ((h->flags & TBE_FLAG_SPLIT_BAGS) ? up(split_bytes(h->split_cap, h->split_pstride)) : 0);
  *out = h;
  return TBE_OK;
}

void tbe_destroy(tbe_handle* h) {
  if (!h) return;
  for (auto& e : h->pool) (void)hipEventDestroy(e);
  if (h->meta) (void)hipFree(h->meta);
  delete h;
}

tbe_status tbe_forward_scratch_size(const tbe_handle* h, size_t* bytes) {
  if (!h || !bytes) return TBE_ERR_INVALID_ARGUMENT;
  *bytes = h->fscratch_bytes;
  return TBE_OK;
}

tbe_status tbe_set_forward_scratch(tbe_handle* h, void* scratch, size_t bytes) {
  if (!h) return TBE_ERR_INVALID_ARGUMENT;
  if (!scratch) {  // detach
    if (bytes != 0) return TBE_ERR_INVALID_ARGUMENT;
    h->wt = nullptr;
    h->split = nullptr;
    h->fscratch_set = false;
    return TBE_OK;
  }
  if (!aligned(scratch, kAlign)) return TBE_ERR_INVALID_ARGUMENT;
  if (bytes < h->fscratch_bytes) return TBE_ERR_WORKSPACE_TOO_SMALL;
  char* base = static_cast<char*>(scratch);
  h->wt = h->wt_elems > 0 ? reinterpret_cast<uint16_t*>(base) : nullptr;
  h->split = (h->flags & TBE_FLAG_SPLIT_BAGS) ? base + h->fscratch_split_off : nullptr;
  h->fscratch_set = true;
  return TBE_OK;
}

tbe_status tbe_set_option(tbe_handle* h, int32_t option, int64_t value) {
  if (!h) return TBE_ERR_INVALID_ARGUMENT;
  switch (option) {
    case TBE_OPTION_LONG_RUN_THRESHOLD:
      if (value < 1) return TBE_ERR_INVALID_ARGUMENT;
      h->long_threshold = value;
      return TBE_OK;
    case TBE_OPTION_PROFILE:
      h->profile = value != 0;
      return TBE_OK;
    case TBE_OPTION_SORT:
      if (value != 0 && value != 1) return TBE_ERR_INVALID_ARGUMENT;
      h->bucket_sort = value == 0;
      return TBE_OK;
    case TBE_OPTION_SPIN_LIMIT:
      if (value < 0 || value > 0x7FFFFFFF) return TBE_ERR_INVALID_ARGUMENT;
      h->spin_limit = static_cast<uint32_t>(value);
      return TBE_OK;
    case TBE_OPTION_LDS_FORWARD:
      if (value != 0 && value != 1) return TBE_ERR_INVALID_ARGUMENT;
      h->lds_forward = value == 1;
      return TBE_OK;
  }
  return TBE_ERR_INVALID_ARGUMENT;
}

tbe_status tbe_check_device_status(tbe_handle* h, void* stream) {
  if (!h) return TBE_ERR_INVALID_ARGUMENT;
  return check_error_mark(h, static_cast<hipStream_t>(stream));
}

tbe_status tbe_stage_times(tbe_handle* h, float* ms, const char** names, int32_t capacity,
                           int32_t* count) {
  if (!h || !count || (capacity > 0 && !ms)) return TBE_ERR_INVALID_ARGUMENT;
  *count = 0;
  if (h->timed.empty()) return TBE_OK;
  if (hipEventSynchronize(h->pool[h->timed.back().first + 1]) != hipSuccess) return TBE_ERR_HIP;
  int n = 0;
  for (size_t i = 0; i < h->timed.size() && n < capacity; ++i) {
    float t = 0.0f;
    const size_t e = h->timed[i].first;
    if (hipEventElapsedTime(&t, h->pool[e], h->pool[e + 1]) != hipSuccess) return TBE_ERR_HIP;
    ms[n] = t;
    if (names) names[n] = h->timed[i].second;
    ++n;
  }
  h->timed.clear();
  h->used = 0;
  *count = n;
  return TBE_OK;
}

}  // extern "C"

namespace {

// The pooled lookup; with fuse set, the gather kernel also linearizes that
// backward batch (its workspace already zeroed).
tbe_status forward_impl(tbe_handle* h, int32_t B, const void* indices, const void* offsets,
                        int32_t index_dtype, int64_t n, const float* psw, float* output,
                        hipStream_t s, bool validate, const BackwardLaunch* fuse = nullptr) {
  tbe_status st = check_batch_args(h, B, indices, offsets, index_dtype, n);
  if (st != TBE_OK) return st;
  if (B == 0) return TBE_OK;
  if (!output || !aligned(output, 16)) return TBE_ERR_INVALID_ARGUMENT;
  if (psw && !aligned(psw, 4)) return TBE_ERR_INVALID_ARGUMENT;
  // per-sample weights rule out the count-matrix forward
  if (psw && (h->flags & TBE_FLAG_FORCE_HISTOGRAM)) return TBE_ERR_UNSUPPORTED;
  // the opt-in paths' scratch comes from the caller
  if (h->fscratch_bytes > 0 && !h->fscratch_set) return TBE_ERR_WORKSPACE_TOO_SMALL;
  try {
    // Sub-wave size: enough lane groups per bag that one round of row loads
    // covers a mean-length bag.
    const double mean_len = static_cast<double>(n) / (static_cast<double>(h->T) * B);
    int lshift = 0;
    while (lshift < 6 && (int64_t{kFwdUnroll} << lshift) < mean_len) ++lshift;
    int64_t tiles = 1;
    for (int t = 0; t < h->T; ++t) {
      const int sw = std::min(6, h->meta_host[t].fwd_gshift + lshift);
      const int64_t bags_per_block = int64_t{kWavesPerBlock} << (6 - sw);
      tiles = std::max<int64_t>(tiles, (B + bags_per_block - 1) / bags_per_block);
    }
    if (tiles * h->T > 0x7FFFFFFF) return TBE_ERR_UNSUPPORTED;
    if (validate && (h->flags & TBE_FLAG_VALIDATE)) {
      st = run_validation(h, B, indices, offsets, index_dtype, n, s);
      if (st != TBE_OK) return st;
    }
    KernelTimer timer{h, take_events};
    const KernelTimer* kt = h->profile ? &timer : nullptr;
    // Count-matrix forward for the eligible tables unless lookups carry
    // per-sample weights; the gather kernel covers every other table.
    const bool hist = !psw && !h->hist_host.empty();
    if (hist) {
      HistLaunch ha{};
      ha.weights = h->weights;
      ha.indices = indices;
      ha.offsets = offsets;
      ha.out = output;
      ha.meta = h->meta;
      ha.list = h->hist;
      ha.wt = h->wt;
      ha.H = static_cast<int32_t>(h->hist_host.size());
      ha.B = B;
      ha.sum_dims = h->sum_dims;
      ha.etiles = h->hist_etiles;
      ha.dtiles = h->hist_dtiles;
      ha.mean = h->pooling == TBE_POOL_MEAN;
      ha.dtype = h->dtype;
      ha.index64 = index_dtype == TBE_I64;
      const hipError_t e = launch_forward_histogram(ha, s, kt);
      if (e != hipSuccess) return from_hip(e);
      if (h->gather_host.empty() && !fuse) return TBE_OK;
    }
    ForwardLaunch a{};
    a.table_list = hist ? h->gather_list : nullptr;
    a.weights = h->weights;
    a.indices = indices;
    a.offsets = offsets;
    a.psw = psw;
    a.out = output;
    a.meta = h->meta;
    a.T = hist ? static_cast<int32_t>(h->gather_host.size()) : h->T;
    a.B = B;
    a.sum_dims = h->sum_dims;
    a.tiles_per_table = static_cast<int32_t>(tiles);
    a.lshift = lshift;
    a.mean = h->pooling == TBE_POOL_MEAN;
    a.dtype = h->dtype;
    a.index64 = index_dtype == TBE_I64;
    a.vec = h->fwd_vec;
    a.uncond_loads = n > kFusedMaxLookups ? 1 : 0;
    // bags split only when every possible segment fits the scratch (at most
    // n / kSplitLen segments after the first ones)
    const bool split = h->split && n > kSplitLen && n / kSplitLen + 1 <= h->split_cap;
    // small tables from LDS when each workgroup's staging is small next to
    // its lookups and the bag's partial sums fit the LDS kernel
    if (!hist && !fuse && !split && h->lds_forward && !h->lds_host.empty() &&
        n / h->T >= 16 * h->lds_max_rows &&
        (1 << std::min(6 - h->lds_gshift, lshift)) <= lds_forward_max_r(h->lds_gshift, psw)) {
      ForwardLaunch l = a;
      l.table_list = h->lds_list;
      l.T = static_cast<int32_t>(h->lds_host.size());
      const int64_t nblk = (static_cast<int64_t>(B) + kWave - 1) / kWave;
      const int64_t wgs =
          std::max<int64_t>(1, std::min<int64_t>(nblk, (h->num_cus + l.T - 1) / l.T));
      hipError_t e = launch_forward_lds(l, h->lds_gshift, static_cast<int>(wgs), s, kt);
      if (e == hipSuccess && !h->lds_rest_host.empty()) {
        a.table_list = h->lds_rest;
        a.T = static_cast<int32_t>(h->lds_rest_host.size());
        e = launch_forward_gather(a, s, kt);
      }
      return from_hip(e);
    }
    if (split) {
      a.split_len = kSplitLen;
      a.split_ctr = reinterpret_cast<uint32_t*>(h->split);
      a.split_seg = reinterpret_cast<uint2*>(h->split + 256);
      a.split_long = reinterpret_cast<uint4*>(h->split + 256 + 8 * h->split_cap);
      a.split_part = reinterpret_cast<float*>(h->split + 256 + 24 * h->split_cap);
      a.split_pstride = h->split_pstride;
      hipLaunchKernelGGL(fill_u32, dim3(1), dim3(64), 0, s, a.split_ctr, 0u, int64_t{2});
    }
    hipError_t e =
        fuse ? launch_forward_linearize(a, *fuse, s, kt) : launch_forward_gather(a, s, kt);
    if (e == hipSuccess && split) e = launch_forward_split(a, n, s, kt);
    return from_hip(e);
  } catch (...) {
    return TBE_ERR_OUT_OF_MEMORY;
  }
}

}  // namespace

extern "C" {

tbe_status tbe_forward(tbe_handle* h, int32_t B, const void* indices, const void* offsets,
                       int32_t index_dtype, int64_t n, const float* psw, float* output,
                       void* stream) {
  return forward_impl(h, B, indices, offsets, index_dtype, n, psw, output,
                      static_cast<hipStream_t>(stream), true);
}

tbe_status tbe_psw_grad(tbe_handle* h, int32_t B, const void* indices, const void* offsets,
                        int32_t index_dtype, int64_t n, const float* grad_output, float* grad_psw,
                        void* stream) {
  tbe_status st = check_batch_args(h, B, indices, offsets, index_dtype, n);
  if (st != TBE_OK) return st;
  if (B == 0 || n == 0) return TBE_OK;
  if (!grad_output || !grad_psw || !aligned(grad_output, 4) || !aligned(grad_psw, 4))
    return TBE_ERR_INVALID_ARGUMENT;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  try {
    const double mean_len = static_cast<double>(n) / (static_cast<double>(h->T) * B);
    int lshift = 0;
    while (lshift < 6 && (int64_t{kFwdUnroll} << lshift) < mean_len) ++lshift;
    int64_t tiles = 1;
    for (int t = 0; t < h->T; ++t) {
      const int sw = std::min(6, h->meta_host[t].fwd_gshift + lshift);
      const int64_t bags_per_block = int64_t{kWavesPerBlock} << (6 - sw);
      tiles = std::max<int64_t>(tiles, (B + bags_per_block - 1) / bags_per_block);
    }
    if (tiles * h->T > 0x7FFFFFFF) return TBE_ERR_UNSUPPORTED;
    if (h->flags & TBE_FLAG_VALIDATE) {
      st = run_validation(h, B, indices, offsets, index_dtype, n, s);
      if (st != TBE_OK) return st;
    }
    KernelTimer timer{h, take_events};
    ForwardLaunch a{};
    a.weights = h->weights;
    a.indices = indices;
    a.offsets = offsets;
    a.meta = h->meta;
    a.T = h->T;
    a.B = B;
    a.sum_dims = h->sum_dims;
    a.tiles_per_table = static_cast<int32_t>(tiles);
    a.lshift = lshift;
    a.mean = h->pooling == TBE_POOL_MEAN;
    a.dtype = h->dtype;
    a.index64 = index_dtype == TBE_I64;
    // 16-byte row chunks of the weights need 16-byte aligned gradient rows too
    a.vec = h->fwd_vec && aligned(grad_output, 16);
    return from_hip(launch_psw_grad(a, grad_output, grad_psw, s, h->profile ? &timer : nullptr));
  } catch (...) {
    return TBE_ERR_OUT_OF_MEMORY;
  }
}

tbe_status tbe_backward_workspace_size(const tbe_handle* h, int32_t B, int64_t n, size_t* bytes) {
  if (!h || !bytes || B < 0 || n < 0) return TBE_ERR_INVALID_ARGUMENT;
  BwdPlan p;
  if (!plan_backward(h, B, n, h->bwd_vec, h->long_threshold, &p)) return TBE_ERR_UNSUPPORTED;
  *bytes = p.bytes;
  // with the count-matrix backward, room for it too (calls with per-sample
  // weights take the sort path)
  if (!h->cb_host.empty())
    *bytes = std::max(*bytes, count_backward_bytes(h->weight_elems, h->sum_rows,
                                                   count_slices(h, B)));
  return TBE_OK;
}

tbe_status tbe_backward_update(tbe_handle* h, int32_t B, const void* indices, const void* offsets,
                               int32_t index_dtype, int64_t n, const float* psw,
                               const float* grad_output, float lr, float eps, void* workspace,
                               size_t workspace_bytes, const tbe_runs* runs, void* stream) {
  return backward_impl(h, B, indices, offsets, index_dtype, n, psw, grad_output, lr, eps,
                       workspace, workspace_bytes, runs, static_cast<hipStream_t>(stream), true);
}

tbe_status tbe_backward_update_no_alloc(tbe_handle* h, int32_t B, const void* indices,
                                        const void* offsets, int32_t index_dtype, int64_t n,
                                        const float* psw, const float* grad_output, float lr,
                                        float eps, const tbe_runs* runs, void* stream) {
  if (!h) return TBE_ERR_INVALID_ARGUMENT;
  if (!h->static_scratch) return TBE_ERR_HIP;
  // the same kernels as tbe_backward_update on the device's static scratch (a
  // batch that needs more gets TBE_ERR_WORKSPACE_TOO_SMALL); no kernel timing,
  // whose events would be created on demand
  return backward_impl(h, B, indices, offsets, index_dtype, n, psw, grad_output, lr, eps,
                       h->static_scratch, TBE_STATIC_SCRATCH_BYTES, runs,
                       static_cast<hipStream_t>(stream), true, false);
}

tbe_status tbe_backward_update_grouped(tbe_handle* h, int32_t B, const void* indices,
                                       const void* offsets, int32_t index_dtype, int64_t n,
                                       const float* psw, const float* grad_output, float lr,
                                       float eps, void* workspace, size_t workspace_bytes,
                                       const tbe_runs* runs, void* stream) {
  return backward_impl(h, B, indices, offsets, index_dtype, n, psw, grad_output, lr, eps,
                       workspace, workspace_bytes, runs, static_cast<hipStream_t>(stream), false);
}

tbe_status tbe_forward_group(tbe_handle* h, int32_t B, const void* indices, const void* offsets,
                             int32_t index_dtype, int64_t n, const float* psw, float* output,
                             void* workspace, size_t workspace_bytes, void* stream) {
  tbe_status st = check_batch_args(h, B, indices, offsets, index_dtype, n);
  if (st != TBE_OK) return st;
  if (B == 0) return TBE_OK;
  if (!output || !aligned(output, 16)) return TBE_ERR_INVALID_ARGUMENT;
  if (psw && !aligned(psw, 4)) return TBE_ERR_INVALID_ARGUMENT;
  if (psw && (h->flags & TBE_FLAG_FORCE_HISTOGRAM)) return TBE_ERR_UNSUPPORTED;
  if (n == 0) return tbe_forward(h, B, indices, offsets, index_dtype, n, psw, output, stream);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (uses_count_backward(h, psw)) {
    // the count-matrix backward needs no grouping: the pooled lookup alone,
    // and a record that its backward may use this workspace
    if (!workspace || !aligned(workspace, kAlign)) return TBE_ERR_INVALID_ARGUMENT;
    size_t need = 0;
    st = tbe_backward_workspace_size(h, B, n, &need);
    if (st != TBE_OK) return st;
    if (workspace_bytes < need) return TBE_ERR_WORKSPACE_TOO_SMALL;
    st = forward_impl(h, B, indices, offsets, index_dtype, n, psw, output, s, true);
    if (st != TBE_OK) return st;
    try {
      auto old = find_group(h, workspace);
      if (old != h->groups.end()) h->groups.erase(old);
      if (h->groups.size() >= kMaxGroupRecords) h->groups.erase(h->groups.begin());
      h->groups.push_back(GroupRecord{workspace, indices, offsets, psw, B, index_dtype, n,
                                      h->long_threshold, h->bucket_sort, false, true});
    } catch (...) {
      return TBE_ERR_OUT_OF_MEMORY;
    }
    return TBE_OK;
  }
  try {
    BwdPlan p;
    if (!plan_backward(h, B, n, h->bwd_vec, h->long_threshold, &p)) return TBE_ERR_UNSUPPORTED;
    if (!workspace || !aligned(workspace, kAlign)) return TBE_ERR_INVALID_ARGUMENT;
    if (workspace_bytes < p.bytes) return TBE_ERR_WORKSPACE_TOO_SMALL;
    BackwardLaunch a{};
    fill_backward(h, B, indices, offsets, index_dtype, n, psw, nullptr, 0.0f, 0.0f, workspace,
                  nullptr, h->bwd_vec, h->long_threshold, h->bucket_sort, p, &a);
    // ids are checked (when asked) before anything is enqueued
    if (h->flags & TBE_FLAG_VALIDATE) {
      st = run_validation(h, B, indices, offsets, index_dtype, n, s);
      if (st != TBE_OK) return st;
    }
    KernelTimer timer{h, take_events};
    const KernelTimer* kt = h->profile ? &timer : nullptr;
    // workspace clear; the pooled lookup with the linearize step in the same
    // launch (the two one after the other for large batches); then the sort
    // and the run-length encoding
    // a grouping this workspace held before is overwritten from here on
    auto old = find_group(h, workspace);
    if (old != h->groups.end()) h->groups.erase(old);
    // (a linearize step that sorts the tiles clears the workspace itself)
    if (!uses_tile_buckets(a) && launch_init_workspace(a, s, kt) != hipSuccess)
      return TBE_ERR_HIP;
    const bool fused = n <= kFusedMaxLookups;
    st = forward_impl(h, B, indices, offsets, index_dtype, n, psw, output, s, false,
                      fused ? &a : nullptr);
    if (st != TBE_OK) return st;
    if (!fused && launch_linearize_kernel(a, s, kt) != hipSuccess) return TBE_ERR_HIP;
    if (launch_sort_encode(a, s, kt) != hipSuccess) return TBE_ERR_HIP;
    if (h->groups.size() >= kMaxGroupRecords) h->groups.erase(h->groups.begin());
    h->groups.push_back(GroupRecord{workspace, indices, offsets, psw, B, index_dtype, n,
                                    h->long_threshold, h->bucket_sort, uses_bucket_sort(a),
                                    false});
    return TBE_OK;
  } catch (...) {
    return TBE_ERR_OUT_OF_MEMORY;
  }
}

}  // extern "C"
