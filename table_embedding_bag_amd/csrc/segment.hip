// segment.hip -- segment reduce of the upstream gradients per run of equal
// (table, row) ids, fused with the row-wise optimizer update, for gfx950.
//
// kimbodo.com/?p=28372, "What Happened": every touched row receives one
// optimizer update; short runs are summed by a streaming path and runs of at
// least 256 lookups by split accumulation.  "FBTriton Rewrites Table Batched
// Embedding", "Responsibilities of the forward and backward passes": the
// gradients of a row hit several times are added up.
//
//   Gamma_r = sum_{i in run r} c_i * G[b(i), doff_t : doff_t + D_t]
//   c_i = p_i * s_k (per-sample weight times the mean scale, 1 for plain sums)
//   SGD:              W_r <- W_r - lr * Gamma_r
//   row-wise Adagrad: m_r <- m_r + mean_d Gamma_r[d]^2
//                     W_r <- W_r - lr * Gamma_r / (sqrt(m_r) + eps)
// The pages name no optimizer; these two are the plainest readings.
//
// The cost of a run is the latency of its dependent loads (sorted position ->
// bag -> gradient row), so the work is shaped to keep many gradient rows in
// flight per run.  Runs longer than a lane group takes (short_max lookups) are
// queued as workgroup items before the reduce: by the bucket-local run-length
// encoder, which sees whole runs, or else by queue_runs (one lane per run).
//   seg_fused     every workgroup first takes its share of the queued items,
//                 then its share of the short runs, so bandwidth-bound and
//                 latency-bound work overlap across the chip:
//     items       one workgroup per item: a medium run (shorter than the
//                 long-run threshold, streamed in one pass and updated at once)
//                 or a 256-lookup chunk of a long run (split accumulation: an
//                 fp32 partial sum per chunk).  The workgroup stages 256 lookups
//                 in LDS and its 256/Gs lane groups keep 4 rows each in flight;
//                 the groups' sums are added in LDS in a fixed order.  In a
//                 batch of at most 2^20 lookups the workgroup that stores a
//                 run's last partial (a ticket per run) adds the run's
//                 partials in chunk order and updates the row.
//     short runs  one lane group (Gs lanes = one gradient row of 16-byte
//                 chunks; per table when tables differ in width) per run: every
//                 lane prefetches one lookup, the group gathers the run's
//                 gradient rows with 2 or 4 in flight (matched to the run's
//                 length), sums them in fp32 and updates the row.  Most runs
//                 are this short.  When an eighth of the upstream gradient
//                 fits one XCD's L2, each XCD takes one contiguous range of
//                 runs (so of tables) and keeps their gradient rows there.
//   seg_finalize  larger batches: the long runs' partials added in the same
//                 order and the rows updated, in a launch of their own.
// Summation order never depends on scheduling (no float atomics), so results
// are reproducible bit for bit.  Sums inside workgroup items are kept in fp64:
// a run may add the same gradient row many times over (a hot row hit
// repeatedly inside one bag), and fp32 rounding errors of such correlated sums
// grow linearly; products c_i * g are exact in fp64.  No workgroup waits for
// another: a ticket only decides which one finishes a run.  The partials go
// through agent-scope atomic stores and loads, which other XCDs see without
// the writeback of the whole L2 that a device-scope release fence costs.
#include "common.hpp"

namespace tbe {
namespace {


// Gradient rows kept in flight per lane group: 8 for short runs (4 inside a
// workgroup item) for rows of one 16-byte chunk per lane, fewer when a lane
// holds several chunks, so that registers stay below 128 per lane.
template <int VE, int NCH>
constexpr int group_unroll() {
  return (32 / (VE * NCH)) < 1 ? 1 : ((32 / (VE * NCH)) > 8 ? 8 : 32 / (VE * NCH));
}
// Short runs keep at most 4 rows in flight: the registers saved buy more
// resident waves, which hides more latency than a deeper unroll.
template <int VE, int NCH>
constexpr int short_unroll() {
  return group_unroll<VE, NCH>() > 4 ? 4 : group_unroll<VE, NCH>();
}
template <int VE, int NCH>
constexpr int wg_unroll() {
  return group_unroll<VE, NCH>() > 1 ? group_unroll<VE, NCH>() / 2 : 1;
}

// The slice of a summed gradient row held by one lane: NCH chunk sets of VE
// values (chunk c*Gs + gl of the row).
template <int VE, int NCH>
struct Acc {
  double v[NCH][VE];
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int c = 0; c < NCH; ++c)
#pragma unroll
      for (int e = 0; e < VE; ++e) v[c][e] = 0.0;
  }
};

struct GroupCtx {
  int gl;      // lane within group
  int Gs;      // lanes per group
};

// Bag and coefficient of the lookup stored at a sorted position.
template <bool REC>
__device__ __forceinline__ void lookup_of(const BackwardLaunch& a, uint32_t val, uint32_t* bag,
                                          float* coef) {
  if constexpr (REC) {
    const uint2 r = a.buf.rec[val];
    *bag = r.x;
    *coef = __uint_as_float(r.y);
  } else {
    *bag = val;
    *coef = 1.0f;
  }
}

// This lane's chunks of gradient row b of table m (zeros where absent),
// loads under a predicate: for the short-run gather, whose unroll already
// matches the run's length.
template <int VE, int NCH>
__device__ __forceinline__ void load_grad(const BackwardLaunch& a, const TableMeta& m, int64_t b,
                                          int gl, int Gs, bool valid, float (&v)[NCH][VE]) {
  const float* grow = a.grad + b * a.sum_dims + m.doff;
  const int C = m.dim / VE;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int chunk = c * Gs + gl;
    if (valid && chunk < C) {
      if constexpr (VE == 4) {
        const float4 x = *reinterpret_cast<const float4*>(grow + chunk * 4);
        v[c][0] = x.x; v[c][1] = x.y; v[c][2] = x.z; v[c][3] = x.w;
      } else {
#pragma unroll
        for (int q = 0; q < VE; ++q) v[c][q] = grow[chunk * VE + q];
      }
    } else {
#pragma unroll
      for (int q = 0; q < VE; ++q) v[c][q] = 0.0f;
    }
  }
}

// The same, branch-free: absent chunks load from the start of G and are
// zeroed after, so the loads of several rows stay in flight together (a load
// under a branch whose other side writes the same registers is waited for at
// once).  For the workgroup items, whose unrolled batches are mostly full.
template <int VE, int NCH>
__device__ __forceinline__ void load_grad_all(const BackwardLaunch& a, const TableMeta& m,
                                              int64_t b, int gl, int Gs, bool valid,
                                              float (&v)[NCH][VE]) {
  const int64_t row = b * a.sum_dims + m.doff;
  const int C = m.dim / VE;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int chunk = c * Gs + gl;
    const bool ok = valid && chunk < C;
    const float* src = a.grad + (ok ? row + chunk * VE : 0);
    if constexpr (VE == 4) {
      const float4 x = *reinterpret_cast<const float4*>(src);
      v[c][0] = ok ? x.x : 0.0f;
      v[c][1] = ok ? x.y : 0.0f;
      v[c][2] = ok ? x.z : 0.0f;
      v[c][3] = ok ? x.w : 0.0f;
    } else {
#pragma unroll
      for (int q = 0; q < VE; ++q) {
        const float x = src[q];
        v[c][q] = ok ? x : 0.0f;
      }
    }
  }
}

template <int VE, int NCH>
__device__ __forceinline__ void accumulate(Acc<VE, NCH>& acc, float coef, const float (&v)[NCH][VE]) {
#pragma unroll
  for (int c = 0; c < NCH; ++c)
#pragma unroll
    for (int q = 0; q < VE; ++q)
      acc.v[c][q] = fma(static_cast<double>(coef), static_cast<double>(v[c][q]), acc.v[c][q]);
}

// Table of a run, from the bag of its first lookup.
template <bool REC>
__device__ __forceinline__ int table_of_run(const BackwardLaunch& a, const uint32_t* sorted_vals,
                                            int64_t first) {
  uint32_t bag;
  float coef;
  lookup_of<REC>(a, sorted_vals[first], &bag, &coef);
  return static_cast<int>(bag / static_cast<uint32_t>(a.B));
}

// Row-wise optimizer step size for a row whose summed gradient has squared
// norm ss and whose state was m_old; updates the state (one lane writes it).
// Every thread must have read m_old before a barrier that the writer passes
// before its store, else a late reader sees the new state.
__device__ __forceinline__ float step_size(const BackwardLaunch& a, uint32_t key, float m_old,
                                           double ss, int D, bool writer) {
  if (!a.adagrad) return a.lr;
  const float mnew = static_cast<float>(static_cast<double>(m_old) + ss / D);
  if (writer) a.state[key] = mnew;
  return a.lr / (sqrtf(mnew) + a.eps);
}

struct GroupIds {
  int gid, ngroups;
  GroupCtx g;
};

__device__ __forceinline__ GroupIds group_ids(const BackwardLaunch& a, uint32_t bid,
                                              uint32_t nblk) {
  GroupIds r;
  const int Gs = 1 << a.gshift;
  const int per_wave = kWave >> a.gshift;
  const int lane = lane_id();
  const int wave_global = bid * kWavesPerBlock + (threadIdx.x >> 6);
  r.gid = wave_global * per_wave + (lane >> a.gshift);
  r.ngroups = nblk * kWavesPerBlock * per_wave;
  r.g.gl = lane & (Gs - 1);
  r.g.Gs = Gs;
  return r;
}

// Table metadata staged in LDS (handles with at most kLdsTables tables), so
// that a run's table follows from its row id without a dependent global load.
constexpr int kLdsTables = kSegLdsTables;

__device__ __forceinline__ void stage_meta(const BackwardLaunch& a, TableMeta* s_meta) {
  if (a.T <= kLdsTables)
    for (int i = threadIdx.x; i < a.T; i += kBlock) s_meta[i] = a.meta[i];
  __syncthreads();
}

// Table of linear row id `key`: the last t with roff_t <= key.
__device__ __forceinline__ int table_of_key(const BackwardLaunch& a, const TableMeta* s_meta,
                                            uint32_t key) {
  int lo = 0, hi = a.T;
  if (a.T <= kLdsTables) {
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (static_cast<uint32_t>(s_meta[mid].roff) <= key) lo = mid; else hi = mid;
    }
  } else {
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (static_cast<uint32_t>(a.meta[mid].roff) <= key) lo = mid; else hi = mid;
    }
  }
  return lo;
}

__device__ __forceinline__ TableMeta meta_of(const BackwardLaunch& a, const TableMeta* s_meta,
                                             int t) {
  return a.T <= kLdsTables ? s_meta[t] : a.meta[t];
}

// Short runs (at most Gs lookups): one lane group per run, grid-stride over
// runs.  Most runs have one to three lookups and the kernel is bound by the
// latency of its dependent loads (run bounds -> lookup -> gradient rows), so
// it is kept lean (about 70 registers, 7 resident waves per SIMD): every lane loads one
// lookup, the row to update and its state are loaded before the gradient rows
// arrive, the gather keeps 2 or 4 rows in flight (matched to the run's
// length) and sums are kept in fp32 (at most Gs terms: error below
// Gs * 2^-24 of the sum of magnitudes; longer runs are summed in fp64 by the
// kernels below).  Loading the next run while working on the current one
// costs more registers, hence resident waves, than it saves.
template <int U, int VE, int NCH, bool REC>
__device__ __forceinline__ void gather_short(const BackwardLaunch& a, const TableMeta& m,
                                             int64_t tb, int leader, int gl, int Gs, int len,
                                             uint32_t my_bag, float my_coef,
                                             float (&acc)[NCH][VE]) {
  for (int j = 0; j < len; j += U) {
    float v[U][NCH][VE];
    float cf[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int jj = j + u;
      const int src = leader + min(jj, Gs - 1);
      const uint32_t bag = __shfl(my_bag, src, kWave);
      cf[u] = jj < len ? __shfl(my_coef, src, kWave) : 0.0f;
      load_grad<VE, NCH>(a, m, static_cast<int64_t>(bag) - tb, gl, Gs, jj < len, v[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int c = 0; c < NCH; ++c)
#pragma unroll
        for (int q = 0; q < VE; ++q) acc[c][q] = fmaf(cf[u], v[u][c][q], acc[c][q]);
  }
}

// One run per lane group of Gs lanes (Gs = 2^k <= 64, groups aligned within
// the wave), called by every lane of the wave together.  Runs longer than Gq
// lookups were queued as workgroup items (by the run-length encoder or
// queue_runs) and are skipped; shorter ones are gathered here in batches of Gs
// lookups (one batch when Gs >= Gq).  t is the run's table, or -1 to find it
// from the row id.
template <int ST, int VE, int NCH, bool REC, bool PT>
__device__ __forceinline__ void short_run(const BackwardLaunch& a, const uint32_t* sorted_vals,
                                          const TableMeta* s_meta, uint32_t r, bool valid,
                                          int t_known, int Gs, int gl, int leader, int Gq) {
  int64_t s = 0, e = 0;
  uint32_t key = 0, first = 0;
  const int fs = a.buf.first_stride;
  if (valid) {
    s = a.buf.run_start[r];
    e = a.buf.run_start[r + 1];
    key = a.buf.unique_keys[r];
    if (gl < fs) first = a.buf.run_first[static_cast<int64_t>(r) * fs + gl];
  }
  const int len = valid ? static_cast<int>(e - s) : 0;
  if (valid && a.out_unique && gl == 0) {
    a.out_unique[r] = static_cast<int32_t>(key);
    a.out_lengths[r] = len;
  }
  if (!valid || len > Gq) return;
  uint32_t my_bag = 0;
  float my_coef = 0.0f;
  // the run's first lookups (one, or four for batches of at most 2^20) came
  // with its bounds, so a run of that many reads no sorted value
  if (gl < len) lookup_of<REC>(a, gl < fs ? first : sorted_vals[s + gl], &my_bag, &my_coef);
  const int t = t_known >= 0 ? t_known : table_of_key(a, s_meta, key);
  const TableMeta m = meta_of(a, s_meta, t);
  const int64_t tb = static_cast<int64_t>(t) * a.B;
  const int64_t row0 = m.woff + static_cast<int64_t>(key - static_cast<uint32_t>(m.roff)) * m.dim;
  const int C = m.dim / VE;
  float w[NCH][VE];
#pragma unroll
  for (int c = 0; c < NCH; ++c)
    if (c * Gs + gl < C) load_widen<ST, VE>(a.weights, row0 + (c * Gs + gl) * VE, w[c]);
  const float m_old = a.adagrad ? a.state[key] : 0.0f;
  float acc[NCH][VE];
#pragma unroll
  for (int c = 0; c < NCH; ++c)
#pragma unroll
    for (int q = 0; q < VE; ++q) acc[c][q] = 0.0f;
  for (int b0 = 0;;) {
    const int blen = PT ? min(Gs, len - b0) : len;
    if (blen <= 2)
      gather_short<2, VE, NCH, REC>(a, m, tb, leader, gl, Gs, blen, my_bag, my_coef, acc);
    else if (blen <= 4)
      gather_short<4, VE, NCH, REC>(a, m, tb, leader, gl, Gs, blen, my_bag, my_coef, acc);
    else
      gather_short<short_unroll<VE, NCH>(), VE, NCH, REC>(a, m, tb, leader, gl, Gs, blen,
                                                           my_bag, my_coef, acc);
    if constexpr (!PT) break;  // Gs = Gq: one batch
    b0 += Gs;
    if (b0 >= len) break;
    my_bag = 0;
    my_coef = 0.0f;
    if (gl < len - b0) lookup_of<REC>(a, sorted_vals[s + b0 + gl], &my_bag, &my_coef);
  }
  float step = a.lr;
  if (a.adagrad) {
    float ss = 0.0f;
#pragma unroll
    for (int c = 0; c < NCH; ++c)
#pragma unroll
      for (int q = 0; q < VE; ++q) ss = fmaf(acc[c][q], acc[c][q], ss);
    for (int o = Gs >> 1; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, kWave);
    const float mnew = m_old + ss / static_cast<float>(m.dim);
    if (gl == 0) a.state[key] = mnew;
    step = a.lr / (sqrtf(mnew) + a.eps);
  }
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    if (c * Gs + gl < C) {
#pragma unroll
      for (int q = 0; q < VE; ++q) w[c][q] = fmaf(-step, acc[c][q], w[c][q]);
      narrow_store<ST, VE>(a.weights, row0 + (c * Gs + gl) * VE, w[c]);
    }
  }
}

// log2 of the lane-group width of table m's gradient rows.
template <int VE>
__device__ __forceinline__ int table_gshift(const TableMeta& m) {
  return (m.bwd_gshift >> (VE == 4 ? 0 : 8)) & 0xFF;
}

// Short runs.  Uniform mode: one lane group of Gs = 2^gshift lanes per run
// (the widest table's row), grid-stride over runs.  Per-table mode (tables of
// different widths, metadata in LDS): a wave takes a task of 64 / Gs_t
// consecutive runs of one table t in lane groups of that table's own width,
// so narrow tables fill the wave; tasks are numbered table after table from
// the tables' first run ids (table_run_starts).  Either way the loop runs the
// same number of times on every lane of a wave (groups past the last run
// idle), so the queueing in short_run can use wave-wide scans.
template <int ST, int VE, int NCH, bool REC, bool PT>
__device__ __forceinline__ void short_runs(const BackwardLaunch& a, const uint32_t* sorted_vals,
                                           uint32_t bid, uint32_t nblk) {
  __shared__ TableMeta s_meta[kLdsTables];
  const bool failed = a.buf.counters[kCntError] != 0u;  // a look-back wait gave up earlier
  const uint32_t U = a.buf.counters[kCntUnique];
  if (bid == 0 && threadIdx.x == 0) {
    if (a.out_num) *a.out_num = failed ? -1 : static_cast<int32_t>(U);
    if (failed && a.error_mark) atomicOr(a.error_mark, 1u);  // read by tbe_check_device_status
  }
  if (failed) return;
  stage_meta(a, s_meta);
  const int Gq = a.short_max;
  const int lane = lane_id();
  if constexpr (!PT) {
    // With xcd_runs the runs are split into G = min(8, workgroups) contiguous
    // ranges, range g taken by workgroups b = g mod G.  Workgroups go to the 8
    // XCDs round robin and sorted runs are table-major, so each XCD gathers
    // the gradient rows of its own stretch of tables, which then stay in its
    // L2 (the host sets xcd_runs when an eighth of the upstream gradient fits
    // one).  Otherwise one range.
    const uint32_t G = a.xcd_runs ? (nblk < 8u ? nblk : 8u) : 1u;
    const uint32_t g = bid % G;
    const uint32_t r_lo = static_cast<uint32_t>(static_cast<uint64_t>(U) * g / G);
    const uint32_t r_hi = static_cast<uint32_t>(static_cast<uint64_t>(U) * (g + 1u) / G);
    const GroupIds id = group_ids(a, bid / G, (nblk - g + G - 1u) / G);
    const int Gs = 1 << a.gshift;  // >= Gq
    const int leader = lane & ~(Gs - 1);
    const uint32_t wave_first = r_lo + id.gid - static_cast<uint32_t>(lane >> a.gshift);
    const uint32_t ng = id.ngroups;
    uint32_t r = r_lo + id.gid;
    for (uint32_t rb = wave_first; rb < r_hi; rb += ng, r += ng)
      short_run<ST, VE, NCH, REC, false>(a, sorted_vals, s_meta, r, r < r_hi, -1, Gs, id.g.gl,
                                         leader, Gq);
    return;
  }
  __shared__ uint32_t s_task[kLdsTables + 1];    // tasks before table t
  __shared__ uint32_t s_ustart[kLdsTables + 1];  // first run of table t
  __shared__ uint32_t s_scr[kWavesPerBlock];
  const int tid = threadIdx.x;
  uint32_t my_tasks = 0;
  if (tid < a.T) {
    const uint32_t u0 = a.buf.table_runs[tid], u1 = a.buf.table_runs[tid + 1];
    s_ustart[tid] = u0;
    if (tid == a.T - 1) s_ustart[a.T] = u1;
    const int gsh = table_gshift<VE>(s_meta[tid]);
    my_tasks = (u1 - u0 + (kWave >> gsh) - 1) >> (6 - gsh);
  }
  uint32_t ntasks;
  const uint32_t before = block_exclusive_sum(my_tasks, s_scr, &ntasks);
  if (tid < a.T) s_task[tid] = before;
  if (tid == 0) s_task[a.T] = ntasks;
  __syncthreads();
  const uint32_t nwaves = nblk * kWavesPerBlock;
  for (uint32_t k = bid * kWavesPerBlock + (tid >> 6); k < ntasks; k += nwaves) {
    int lo = 0, hi = a.T;  // the table of task k: s_task[lo] <= k < s_task[lo + 1]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_task[mid] <= k) lo = mid; else hi = mid;
    }
    const int gsh = table_gshift<VE>(s_meta[lo]);
    const int Gs = 1 << gsh;
    const uint32_t r = s_ustart[lo] + ((k - s_task[lo]) << (6 - gsh)) + (lane >> gsh);
    short_run<ST, VE, NCH, REC, true>(a, sorted_vals, s_meta, r, r < s_ustart[lo + 1], lo, Gs,
                                      lane & (Gs - 1), lane & ~(Gs - 1), Gq);
  }
}


// First run id of every table: the lower bound of the table's first row id in
// the sorted unique ids, by a 256-way search (three rounds cover 2^24 runs).
// One workgroup per table; workgroup T writes U.
__global__ __launch_bounds__(kBlock) void table_run_starts(BackwardLaunch a) {
  const int t = blockIdx.x;
  const uint32_t U = a.buf.counters[kCntUnique];
  if (t == a.T) {
    if (threadIdx.x == 0) a.buf.table_runs[t] = U;
    return;
  }
  const uint32_t target = static_cast<uint32_t>(a.meta[t].roff);
  uint32_t lo = 0, hi = U;  // the answer lies in [lo, hi]
  while (lo < hi) {
    const uint32_t span = hi - lo;
    const uint32_t step = (span + kBlock - 1) / kBlock;
    const uint32_t p = lo + threadIdx.x * step;
    const bool below = p < hi && a.buf.unique_keys[p] < target;
    const uint32_t c = static_cast<uint32_t>(__syncthreads_count(below));
    if (step == 1 || c == 0) {
      lo += c * step;  // step 1: exact; c = 0: unique_keys[lo] >= target
      break;
    }
    // unique_keys[lo + (c-1)*step] < target <= unique_keys[lo + c*step] (or hi)
    const uint32_t nlo = lo + (c - 1) * step + 1;
    hi = min(hi, lo + c * step);
    lo = nlo;
  }
  if (threadIdx.x == 0) a.buf.table_runs[t] = min(lo, U);
}

// Sum of a double over the 256 threads of a block (every thread gets it).
__device__ __forceinline__ double block_sum(double x, double* scratch) {
#pragma unroll
  for (int o = kWave >> 1; o >= 1; o >>= 1) x += __shfl_xor(x, o, kWave);
  __syncthreads();
  if (lane_id() == 0) scratch[threadIdx.x >> 6] = x;
  __syncthreads();
  double s = 0.0;
#pragma unroll
  for (int w = 0; w < kWavesPerBlock; ++w) s += scratch[w];
  return s;
}

// Data one workgroup hands to another inside a kernel is stored and loaded
// with relaxed agent-scope atomics: those go to the device's point of
// coherence rather than stopping in the XCD's own L2, so a workgroup on any
// XCD sees them without the L2 writeback a release fence would cost.  The
// writer waits until its stores are performed (wait_stores) before it takes a
// ticket; the workgroup whose ticket completes the set then reads the data.
template <typename T>
__device__ __forceinline__ void st_agent(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ T ld_agent(const T* p) {
  return __hip_atomic_load(const_cast<T*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// s_waitcnt vmcnt(0): every load and store this wave issued is performed.
__device__ __forceinline__ void wait_stores() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Takes one of `total` tickets at *ticket for the whole workgroup, once every
// thread's earlier stores are performed, and tells every thread whether it
// was the last one.  Call from the whole workgroup.
__device__ __forceinline__ bool last_ticket(uint32_t* ticket, uint32_t total, uint32_t* s_flag) {
  wait_stores();
  __syncthreads();
  if (threadIdx.x == 0)
    *s_flag = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                      total - 1u
                  ? 1u
                  : 0u;
  __syncthreads();
  return *s_flag != 0u;
}

// Finish of a long run of fewer than kFinPieceMin chunks by a workgroup: lane
// group g adds the chunk partials g, g + ngroups, ... in chunk order (fp64),
// the groups' sums are added in group order, and the row is updated.  The row
// and its state are loaded while the partials are in flight (KU per group).
// AGENT: the partials were stored in this kernel (agent-scope loads), else in
// an earlier one.
template <int ST, int VE, int NCH, bool AGENT, int KU>
__device__ __forceinline__ void finish_run(const BackwardLaunch& a, const uint4& L,
                                           const TableMeta& m, uint32_t key, double* s_red,
                                           double* s_scratch) {
  constexpr int NV = VE * NCH;
  constexpr int kElemsPerThread = kMaxDim / kBlock;
  constexpr int kU = KU;
  const int tid = threadIdx.x;
  const int Gs = 1 << a.gshift;
  const int ngroups = kBlock >> a.gshift;
  const int g = tid >> a.gshift, gl = tid & (Gs - 1);
  const int row_elems = Gs * NV;
  const int D = m.dim, C = D / VE;
  const int64_t row0 = m.woff + static_cast<int64_t>(key - static_cast<uint32_t>(m.roff)) * D;
  float w[kElemsPerThread];
#pragma unroll
  for (int k = 0; k < kElemsPerThread; ++k) {
    const int d = tid + k * kBlock;
    w[k] = 0.0f;
    if (d < D) load_widen<ST, 1>(a.weights, row0 + d, &w[k]);
  }
  const float m_old = a.adagrad ? a.state[key] : 0.0f;
  Acc<VE, NCH> acc;
  acc.zero();
  for (uint32_t c0 = g; c0 < L.w; c0 += static_cast<uint32_t>(ngroups * kU)) {
    float v[kU][NCH][VE];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const uint32_t c = c0 + static_cast<uint32_t>(u * ngroups);
      const float* row = a.buf.partial1 + static_cast<int64_t>(L.z + c) * a.pstride;
#pragma unroll
      for (int q = 0; q < NCH; ++q) {
        const int chunk = q * Gs + gl;
        const bool ok = c < L.w && chunk < C;
        if constexpr (AGENT) {
#pragma unroll
          for (int e = 0; e < VE; ++e) v[u][q][e] = ok ? ld_agent(row + chunk * VE + e) : 0.0f;
        } else if (ok) {
          if constexpr (VE == 4) {
            const float4 x = *reinterpret_cast<const float4*>(row + chunk * 4);
            v[u][q][0] = x.x; v[u][q][1] = x.y; v[u][q][2] = x.z; v[u][q][3] = x.w;
          } else {
#pragma unroll
            for (int e = 0; e < VE; ++e) v[u][q][e] = row[chunk * VE + e];
          }
        } else {
#pragma unroll
          for (int e = 0; e < VE; ++e) v[u][q][e] = 0.0f;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kU; ++u)
#pragma unroll
      for (int q = 0; q < NCH; ++q)
#pragma unroll
        for (int e = 0; e < VE; ++e) acc.v[q][e] += static_cast<double>(v[u][q][e]);
  }
#pragma unroll
  for (int q = 0; q < NCH; ++q)
#pragma unroll
    for (int e = 0; e < VE; ++e) s_red[g * row_elems + (q * Gs + gl) * VE + e] = acc.v[q][e];
  __syncthreads();
  double gam[kElemsPerThread];
  double ss = 0.0;
#pragma unroll
  for (int k = 0; k < kElemsPerThread; ++k) {
    const int d = tid + k * kBlock;
    double x = 0.0;
    if (d < D)
      for (int gg = 0; gg < ngroups; ++gg) x += s_red[gg * row_elems + d];
    gam[k] = x;
    ss = fma(x, x, ss);
  }
  float step = a.lr;
  if (a.adagrad) {
    ss = block_sum(ss, s_scratch);
    step = step_size(a, key, m_old, ss, D, tid == 0);
  }
#pragma unroll
  for (int k = 0; k < kElemsPerThread; ++k) {
    const int d = tid + k * kBlock;
    if (d < D) {
      float x = fmaf(-step, static_cast<float>(gam[k]), w[k]);
      narrow_store<ST, 1>(a.weights, row0 + d, &x);
    }
  }
}

// Piece j of a long run of at least kFinPieceMin chunks (cnt chunk partials
// from slot L.z + j * kFinPiece): with H thread sets (all threads when
// D < kBlock), set h adds chunks h, h + H, ... in order (fp64), the sets'
// sums are added in set order and left, as doubles, over the piece's first
// two slots.  So a row hit hundreds of thousands of times is not finished by
// one workgroup reading every partial.
__device__ __forceinline__ void sum_piece(const BackwardLaunch& a, const uint4& L, uint32_t j,
                                          uint32_t cnt, int D, double* s_sum) {
  constexpr int kBatch = 8;  // partial loads in flight per thread
  const int tid = threadIdx.x;
  const int64_t ps = a.pstride;
  float* first = a.buf.partial1 + static_cast<int64_t>(L.z + j * kFinPiece) * ps;
  const int H = D < kBlock ? kBlock / D : 1;
  for (int e = tid; e < H * D; e += kBlock) {
    const int h = e / D, d = e - h * D;
    double x = 0.0;
    uint32_t q = static_cast<uint32_t>(h);
    for (; q + (kBatch - 1) * H < cnt; q += kBatch * H) {
      float v[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) v[u] = ld_agent(first + static_cast<int64_t>(q + u * H) * ps + d);
#pragma unroll
      for (int u = 0; u < kBatch; ++u) x += static_cast<double>(v[u]);
    }
    for (; q < cnt; q += H) x += static_cast<double>(ld_agent(first + static_cast<int64_t>(q) * ps + d));
    s_sum[e] = x;
  }
  __syncthreads();  // every read of the first two slots is done
  for (int d = tid; d < D; d += kBlock) {
    double x = 0.0;
    for (int h = 0; h < H; ++h) x += s_sum[h * D + d];
    st_agent(reinterpret_cast<double*>(first) + d, x);
  }
}

// Finish of a long run from its np piece sums, added in piece order.
template <int ST>
__device__ __forceinline__ void finish_run_pieces(const BackwardLaunch& a, const uint4& L,
                                                  const TableMeta& m, uint32_t key,
                                                  double* s_sum, double* s_scratch) {
  constexpr int kBatch = 8;
  const int tid = threadIdx.x;
  const int D = m.dim;
  const uint32_t np = L.w / kFinPiece;
  // read by every thread before block_sum's barriers (thread 0 writes the new
  // state after them)
  const float m_old = a.adagrad ? a.state[key] : 0.0f;
  const int64_t row0 = m.woff + static_cast<int64_t>(key - static_cast<uint32_t>(m.roff)) * D;
  const int64_t dstep = static_cast<int64_t>(kFinPiece) * a.pstride / 2;  // doubles per piece
  const double* p0 = reinterpret_cast<const double*>(a.buf.partial1 +
                                                     static_cast<int64_t>(L.z) * a.pstride);
  double ss = 0.0;
  for (int d = tid; d < D; d += kBlock) {
    double x = 0.0;
    uint32_t p = 0;
    for (; p + kBatch <= np; p += kBatch) {
      double v[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) v[u] = ld_agent(p0 + (p + u) * dstep + d);
#pragma unroll
      for (int u = 0; u < kBatch; ++u) x += v[u];
    }
    for (; p < np; ++p) x += ld_agent(p0 + p * dstep + d);
    s_sum[d] = x;
    ss = fma(x, x, ss);
  }
  float step = a.lr;
  if (a.adagrad) {
    ss = block_sum(ss, s_scratch);
    step = step_size(a, key, m_old, ss, D, tid == 0);
  }
  for (int d = tid; d < D; d += kBlock) {
    float w;
    load_widen<ST, 1>(a.weights, row0 + d, &w);
    w = fmaf(-step, static_cast<float>(s_sum[d]), w);
    narrow_store<ST, 1>(a.weights, row0 + d, &w);
  }
}

// After chunk c of long run li has stored its partial: the workgroup that
// completes the run (a ticket per run) finishes it; a run of at least
// kFinPieceMin chunks first has each piece summed by the workgroup that
// completes the piece (a ticket per piece), and the one that completes the
// last piece finishes the run.  The sums follow chunk and piece order
// whichever workgroup does them, so results do not depend on scheduling.
template <int ST, int VE, int NCH>
__device__ __forceinline__ void finish_after_chunk(const BackwardLaunch& a, uint32_t li,
                                                   uint32_t c, const uint4& L, const TableMeta& m,
                                                   uint32_t key, double* s_red,
                                                   double* s_scratch, uint32_t* s_flag) {
  uint32_t* run_ticket = a.buf.run_tickets + li;
  if (L.w < kFinPieceMin) {
    // two partials in flight per group (one for wide rows) cover most runs in
    // one round and leave the item loop's registers as they were
    if (last_ticket(run_ticket, L.w, s_flag))
      finish_run<ST, VE, NCH, true, VE * NCH <= 4 ? 2 : 1>(a, L, m, key, s_red, s_scratch);
    return;
  }
  const uint32_t np = L.w / kFinPiece;
  const uint32_t j = min(c / kFinPiece, np - 1u);
  const uint32_t cnt = j == np - 1u ? L.w - j * kFinPiece : kFinPiece;
  if (!last_ticket(a.buf.piece_tickets + (L.z + j * kFinPiece) / kFinPiece, cnt, s_flag)) return;
  sum_piece(a, L, j, cnt, m.dim, s_red);
  if (last_ticket(run_ticket, np, s_flag))
    finish_run_pieces<ST>(a, L, m, key, s_red, s_scratch);
}

template <int ST, int VE, int NCH, bool REC>
__device__ __forceinline__ void wg_items(const BackwardLaunch& a, const uint32_t* __restrict__ keys,
                                         const uint32_t* __restrict__ sorted_vals, uint32_t bid,
                                         uint32_t nblk) {
  if (a.buf.counters[kCntError] != 0u) return;  // a look-back wait gave up earlier
  constexpr int NV = VE * NCH;                 // values per lane
  constexpr int kElemsPerThread = kMaxDim / kBlock;
  __shared__ uint32_t s_bag[kBlock];
  __shared__ float s_coef[kBlock];
  __shared__ double s_red[kBlock * NV];        // [group][row element]
  __shared__ double s_scratch[kWavesPerBlock];
  __shared__ uint32_t s_flag;

  const int tid = threadIdx.x;
  const uint32_t n = a.buf.counters[kCntItems1];

  for (uint32_t item = bid; item < n; item += nblk) {
    const uint2 it = a.buf.items1[item];
    const bool medium = (it.y & kMediumItem) != 0;
    uint32_t slot = 0;
    int64_t s, e;
    uint4 L = make_uint4(0u, 0u, 0u, 0u);
    if (medium) {  // {first position, medium flag | length}
      s = it.x;
      e = s + (it.y & ~kMediumItem);
    } else {       // {long run, chunk}
      L = a.buf.longs[it.x];
      s = static_cast<int64_t>(L.x) + static_cast<int64_t>(it.y) * a.chunk;
      e = min(static_cast<int64_t>(L.x) + L.y, s + a.chunk);
      slot = L.z + it.y;
    }
    const int t = table_of_run<REC>(a, sorted_vals, s);
    const TableMeta m = a.meta[t];
    const int64_t tb = static_cast<int64_t>(t) * a.B;
    // lane groups of the table's own width when tables differ in width, so
    // narrow rows keep more lookups in flight
    const int gsh = a.per_table ? table_gshift<VE>(m) : a.gshift;
    const int Gs = 1 << gsh;
    const int ngroups = kBlock >> gsh;
    const int g = tid >> gsh, gl = tid & (Gs - 1);
    const int row_elems = Gs * NV;             // elements per group row in s_red (>= D)
    Acc<VE, NCH> acc;
    acc.zero();
    for (int64_t base = s; base < e; base += kBlock) {
      const int nb = static_cast<int>(min(static_cast<int64_t>(kBlock), e - base));
      __syncthreads();  // staging buffers are free again
      if (tid < nb) lookup_of<REC>(a, sorted_vals[base + tid], &s_bag[tid], &s_coef[tid]);
      __syncthreads();
      constexpr int kU = wg_unroll<VE, NCH>();
      for (int j = g; j < nb; j += ngroups * kU) {
        float v[kU][NCH][VE];
        float cf[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          const int jj = j + u * ngroups;
          const bool ok = jj < nb;
          const uint32_t bag = ok ? s_bag[jj] : static_cast<uint32_t>(tb);
          cf[u] = ok ? s_coef[jj] : 0.0f;
          load_grad_all<VE, NCH>(a, m, static_cast<int64_t>(bag) - tb, gl, Gs, ok, v[u]);
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) accumulate<VE, NCH>(acc, cf[u], v[u]);
      }
    }
    // add the groups' sums in group order
#pragma unroll
    for (int c = 0; c < NCH; ++c)
#pragma unroll
      for (int q = 0; q < VE; ++q) s_red[g * row_elems + (c * Gs + gl) * VE + q] = acc.v[c][q];
    __syncthreads();
    const int D = m.dim;
    double gam[kElemsPerThread];
    double ss = 0.0;
#pragma unroll
    for (int k = 0; k < kElemsPerThread; ++k) {
      const int d = tid + k * kBlock;
      double x = 0.0;
      if (d < D)
        for (int gg = 0; gg < ngroups; ++gg) x += s_red[gg * row_elems + d];
      gam[k] = x;
      ss = fma(x, x, ss);
    }
    if (medium) {
      const uint32_t key = keys[s];
      // read by every thread before block_sum's barriers, so no thread sees
      // the state thread 0 writes after them
      const float m_old = a.adagrad ? a.state[key] : 0.0f;
      if (a.adagrad) ss = block_sum(ss, s_scratch);
      const float step = step_size(a, key, m_old, ss, D, tid == 0);
      const int64_t row0 = m.woff + static_cast<int64_t>(key - static_cast<uint32_t>(m.roff)) * D;
#pragma unroll
      for (int k = 0; k < kElemsPerThread; ++k) {
        const int d = tid + k * kBlock;
        if (d < D) {
          float w;
          load_widen<ST, 1>(a.weights, row0 + d, &w);
          w = fmaf(-step, static_cast<float>(gam[k]), w);
          narrow_store<ST, 1>(a.weights, row0 + d, &w);
        }
      }
    } else {
      float* dst = a.buf.partial1 + static_cast<int64_t>(slot) * a.pstride;
      if (a.finish_in_items) {
#pragma unroll
        for (int k = 0; k < kElemsPerThread; ++k) {
          const int d = tid + k * kBlock;
          if (d < D) st_agent(dst + d, static_cast<float>(gam[k]));
        }
        finish_after_chunk<ST, VE, NCH>(a, it.x, it.y, L, m, keys[s], s_red, s_scratch, &s_flag);
      } else {
#pragma unroll
        for (int k = 0; k < kElemsPerThread; ++k) {
          const int d = tid + k * kBlock;
          if (d < D) dst[d] = static_cast<float>(gam[k]);
        }
      }
    }
  }
}

// Queue the runs longer than a.short_max lookups when the run-length encoder
// did not (it cannot see whole runs in the LSD path).  A workgroup takes 1024
// runs at a time (4 per thread, strided so loads coalesce) and reserves the
// slots they need with one atomic per counter: queue slots are few, but
// reserving them per wave put tens of thousands of same-address atomics in a
// row (60 us on 1 M runs; 16 runs per thread left too few workgroups).  Items carry the run's first position and length, so the workgroup
// code needs no run-list lookup.
constexpr int kQueueRunsPerThread = 4;
// Long runs with more chunks than this have their chunk items written by the
// whole workgroup (a run of 271k lookups has over a thousand).
constexpr uint32_t kQueueOwnChunks = 16;

__global__ __launch_bounds__(kBlock) void queue_runs(BackwardLaunch a) {
  __shared__ uint32_t s_scr[kWavesPerBlock];
  __shared__ uint32_t s_base[3];
  __shared__ uint4 s_big[kBlock];  // {long run, first item, chunks}
  __shared__ uint32_t s_nbig;
  if (threadIdx.x == 0) s_nbig = 0u;
  if (a.buf.counters[kCntError] != 0u) return;  // a look-back wait gave up earlier
  const uint32_t U = a.buf.counters[kCntUnique];
  constexpr uint32_t kRuns = kBlock * kQueueRunsPerThread;
  for (uint32_t r0 = blockIdx.x * kRuns; r0 < U; r0 += gridDim.x * kRuns) {
    uint32_t st[kQueueRunsPerThread], ln[kQueueRunsPerThread];
    uint32_t n_items = 0, n_long = 0, n_chunks = 0, n_big = 0;
#pragma unroll
    for (int j = 0; j < kQueueRunsPerThread; ++j) {
      const uint32_t r = r0 + j * kBlock + threadIdx.x;
      st[j] = 0u;
      ln[j] = 0u;
      if (r < U) {
        st[j] = a.buf.run_start[r];
        ln[j] = a.buf.run_start[r + 1] - st[j];
      }
    }
#pragma unroll
    for (int j = 0; j < kQueueRunsPerThread; ++j) {
      if (ln[j] > static_cast<uint32_t>(a.short_max)) {
        if (ln[j] >= static_cast<uint32_t>(a.long_threshold)) {
          const uint32_t n1 = (ln[j] + a.chunk - 1) / a.chunk;
          ++n_long;
          n_chunks += n1;
          n_items += n1;
          n_big += n1 > kQueueOwnChunks ? 1u : 0u;
        } else {
          ++n_items;
        }
      }
    }
    uint32_t t_items, t_long, t_chunks;
    uint32_t x_items = block_exclusive_sum(n_items, s_scr, &t_items);
    uint32_t x_long = block_exclusive_sum(n_long, s_scr, &t_long);
    uint32_t x_chunks = block_exclusive_sum(n_chunks, s_scr, &t_chunks);
    if (t_items == 0u) continue;  // the same on every thread
    if (threadIdx.x == 0) {
      s_base[0] = atomicAdd(&a.buf.counters[kCntItems1], t_items);
      s_base[1] = t_long ? atomicAdd(&a.buf.counters[kCntLong], t_long) : 0u;
      s_base[2] = t_chunks ? atomicAdd(&a.buf.counters[kCntChunks], t_chunks) : 0u;
    }
    __syncthreads();
    x_items += s_base[0];
    x_long += s_base[1];
    x_chunks += s_base[2];
    __syncthreads();  // s_base is reused by the next round
    const bool any_big = __syncthreads_or(n_big != 0u);
#pragma unroll
    for (int j = 0; j < kQueueRunsPerThread; ++j) {
      if (ln[j] > static_cast<uint32_t>(a.short_max)) {
        if (ln[j] >= static_cast<uint32_t>(a.long_threshold)) {
          const uint32_t r = r0 + j * kBlock + threadIdx.x;
          const uint32_t n1 = (ln[j] + a.chunk - 1) / a.chunk;
          a.buf.longs[x_long] = make_uint4(st[j], ln[j], x_chunks, n1);
          a.buf.long_keys[x_long] = a.buf.unique_keys[r];
          if (n1 >= kFinPieceMin) atomicOr(&a.buf.counters[kCntPieced], 1u);
          if (n1 <= kQueueOwnChunks)
            for (uint32_t c = 0; c < n1; ++c) a.buf.items1[x_items + c] = make_uint2(x_long, c);
          else
            s_big[atomicAdd(&s_nbig, 1u)] = make_uint4(x_long, x_items, n1, 0u);
          ++x_long;
          x_chunks += n1;
          x_items += n1;
        } else {
          a.buf.items1[x_items++] = make_uint2(st[j], kMediumItem | ln[j]);
        }
      }
      if (any_big) {  // the same on every thread; at most one entry per thread per round
        __syncthreads();
        const uint32_t m = s_nbig;
        for (uint32_t e = 0; e < m; ++e) {
          const uint4 b = s_big[e];
          for (uint32_t c = threadIdx.x; c < b.z; c += kBlock)
            a.buf.items1[b.y + c] = make_uint2(b.x, c);
        }
        __syncthreads();
        if (threadIdx.x == 0) s_nbig = 0u;
        __syncthreads();
      }
    }
  }
}

// The segment reduce of short runs and of the queued workgroup items in one
// launch: every workgroup first takes its share of the items (medium runs and
// 256-lookup chunks of long runs: bandwidth-bound row gathers), then its share
// of the short runs (bound by the latency of their dependent loads), so the
// two overlap across the chip.
template <int ST, int VE, int NCH, bool REC, bool PT>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(7))) void seg_fused(
    BackwardLaunch a, const uint32_t* keys, const uint32_t* sorted_vals) {
  wg_items<ST, VE, NCH, REC>(a, keys, sorted_vals, blockIdx.x, gridDim.x);
  short_runs<ST, VE, NCH, REC, PT>(a, sorted_vals, blockIdx.x, gridDim.x);
}

// Long runs of at most this many chunks (one round of partial loads in
// flight) are finished by one lane group each; longer ones by a whole
// workgroup, whose groups load their partials side by side (with up to 16
// chunks per group, the finish of a 270k-lookup Zipf(1.05) batch took 8.4 us
// against 4.8).
constexpr uint32_t kFinGroupChunks = 4;

// A long run finished by one lane group: each lane adds its columns of the
// run's chunk partials in chunk order (fp64), the group reduces the squared
// norm with shuffles, and the row is updated.  Called by the whole group.
template <int ST, int VE, int NCH>
__device__ __forceinline__ void finish_long_in_group(const BackwardLaunch& a,
                                                     const TableMeta* s_meta, const uint4& L,
                                                     uint32_t key, int Gs, int gl) {
  constexpr int kU = VE * NCH >= 16 ? 1 : 4;  // partial rows in flight
  const TableMeta m = meta_of(a, s_meta, table_of_key(a, s_meta, key));
  const int D = m.dim, C = D / VE;
  const int64_t row0 = m.woff + static_cast<int64_t>(key - static_cast<uint32_t>(m.roff)) * D;
  float w[NCH][VE];
#pragma unroll
  for (int q = 0; q < NCH; ++q)
    if (q * Gs + gl < C) load_widen<ST, VE>(a.weights, row0 + (q * Gs + gl) * VE, w[q]);
  const float m_old = a.adagrad ? a.state[key] : 0.0f;
  double acc[NCH][VE];
#pragma unroll
  for (int q = 0; q < NCH; ++q)
#pragma unroll
    for (int e = 0; e < VE; ++e) acc[q][e] = 0.0;
  for (uint32_t c0 = 0; c0 < L.w; c0 += kU) {
    float v[kU][NCH][VE];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const uint32_t c = c0 + u;
      const float* row = a.buf.partial1 + static_cast<int64_t>(L.z + c) * a.pstride;
#pragma unroll
      for (int q = 0; q < NCH; ++q) {
        const int chunk = q * Gs + gl;
        if (c < L.w && chunk < C) {
          if constexpr (VE == 4) {
            const float4 x = *reinterpret_cast<const float4*>(row + chunk * 4);
            v[u][q][0] = x.x; v[u][q][1] = x.y; v[u][q][2] = x.z; v[u][q][3] = x.w;
          } else {
#pragma unroll
            for (int e = 0; e < VE; ++e) v[u][q][e] = row[chunk * VE + e];
          }
        } else {
#pragma unroll
          for (int e = 0; e < VE; ++e) v[u][q][e] = 0.0f;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kU; ++u)
#pragma unroll
      for (int q = 0; q < NCH; ++q)
#pragma unroll
        for (int e = 0; e < VE; ++e) acc[q][e] += static_cast<double>(v[u][q][e]);
  }
  float step = a.lr;
  if (a.adagrad) {
    double ss = 0.0;
#pragma unroll
    for (int q = 0; q < NCH; ++q)
#pragma unroll
      for (int e = 0; e < VE; ++e) ss = fma(acc[q][e], acc[q][e], ss);
    for (int o = Gs >> 1; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, kWave);
    const float mnew = static_cast<float>(static_cast<double>(m_old) + ss / D);
    if (gl == 0) a.state[key] = mnew;
    step = a.lr / (sqrtf(mnew) + a.eps);
  }
#pragma unroll
  for (int q = 0; q < NCH; ++q) {
    if (q * Gs + gl < C) {
#pragma unroll
      for (int e = 0; e < VE; ++e) w[q][e] = fmaf(-step, static_cast<float>(acc[q][e]), w[q][e]);
      narrow_store<ST, VE>(a.weights, row0 + (q * Gs + gl) * VE, w[q]);
    }
  }
}

// The long runs of a batch whose workgroup items only stored their chunk
// partials (batches of more than kFinishInItemsMaxKeys lookups, with many
// long runs: there a separate launch costs less than the ticket round trip
// per chunk): runs of at most kFinGroupChunks chunks by one lane group each,
// longer ones by a workgroup each (finish_run), and runs of at least
// kFinPieceMin chunks piece by piece (sum_piece), the workgroup that sums a
// run's last piece finishing the run.  Either way a run's partials are added
// in the order seg_fused's own finish uses (only the squared norm of a run of
// at most kFinGroupChunks chunks is reduced in another order).
template <int ST, int VE, int NCH, bool REC>
__global__ __launch_bounds__(kBlock) void seg_finalize(BackwardLaunch a) {
  if (a.buf.counters[kCntError] != 0u) return;  // a look-back wait gave up earlier
  constexpr int NV = VE * NCH;
  __shared__ TableMeta s_meta[kLdsTables];
  __shared__ double s_red[kBlock * NV];        // [group][row element]
  __shared__ double s_scratch[kWavesPerBlock];
  stage_meta(a, s_meta);
  const int tid = threadIdx.x;
  const uint32_t n = a.buf.counters[kCntLong];
  if (a.buf.counters[kCntPieced] != 0u) {
    // the pieces of runs of at least kFinPieceMin chunks: the workgroups scan
    // the item list for the first chunk of each piece, kFinPiece adjacent items
    // each, so one workgroup meets at most one piece of a run (pieces are
    // kFinPiece items apart).  Interleaving the items over the workgroups was
    // slower (34 -> 42 us on 4.2 M lookups): the pieces then sit in
    // high-numbered workgroups, which start last.
    __shared__ uint32_t s_np, s_last;
    __shared__ uint2 s_piece[kFinPiece];
    const uint32_t nitems = a.buf.counters[kCntItems1];
    for (uint32_t base = blockIdx.x * kFinPiece; base < nitems; base += gridDim.x * kFinPiece) {
      if (tid == 0) s_np = 0u;
      __syncthreads();
      const uint32_t item = base + static_cast<uint32_t>(tid);
      if (tid < static_cast<int>(kFinPiece) && item < nitems) {
        const uint2 it = a.buf.items1[item];
        if (!(it.y & kMediumItem) && it.y % kFinPiece == 0u) {
          const uint32_t w = a.buf.longs[it.x].w;
          if (w >= kFinPieceMin && it.y / kFinPiece < w / kFinPiece)
            s_piece[atomicAdd(&s_np, 1u)] = make_uint2(it.x, it.y / kFinPiece);
        }
      }
      __syncthreads();
      const uint32_t np = s_np;
      for (uint32_t q = 0; q < np; ++q) {
        // piece j of run li, then the run by the workgroup that sums its last piece
        const uint32_t li = s_piece[q].x, j = s_piece[q].y;
        const uint4 L = a.buf.longs[li];
        const uint32_t key = a.buf.long_keys[li];
        const TableMeta m = meta_of(a, s_meta, table_of_key(a, s_meta, key));
        const uint32_t npc = L.w / kFinPiece;
        const uint32_t cnt = j == npc - 1u ? L.w - j * kFinPiece : kFinPiece;
        sum_piece(a, L, j, cnt, m.dim, s_red);
        if (last_ticket(a.buf.run_tickets + li, npc, &s_last))
          finish_run_pieces<ST>(a, L, m, key, s_red, s_scratch);
        __syncthreads();  // s_red, s_scratch and s_last are reused
      }
    }
  }
  {
    // runs of few chunks: one lane group each (the loop runs the same number
    // of times on every lane of a wave).  Groups are numbered from the last
    // workgroup down, so that the workgroups finishing the longer runs below
    // (from the first up) do not also take these first.
    const GroupIds id = group_ids(a, gridDim.x - 1 - blockIdx.x, gridDim.x);
    const uint32_t wave_first = id.gid - static_cast<uint32_t>(lane_id() >> a.gshift);
    uint32_t r = id.gid;
    for (uint32_t rb = wave_first; rb < n; rb += id.ngroups, r += id.ngroups) {
      if (r < n) {
        const uint4 L = a.buf.longs[r];
        const uint32_t key = a.buf.long_keys[r];
        if (L.w <= kFinGroupChunks)  // the same on every lane of the group
          finish_long_in_group<ST, VE, NCH>(a, s_meta, L, key, id.g.Gs, id.g.gl);
      }
    }
  }
  // The runs this workgroup finishes as a whole (more than kFinGroupChunks and
  // fewer than kFinPieceMin chunks) among its share li = blockIdx.x + k *
  // gridDim.x: every thread tests one of them, so the share costs one round
  // trip instead of one per run; the runs are then finished one by one (each
  // on its own: the order does not change any result).
  __shared__ uint32_t s_whole[kBlock];
  __shared__ uint32_t s_nwhole;
  const uint32_t span = gridDim.x * static_cast<uint32_t>(kBlock);
  for (uint32_t l0 = blockIdx.x; l0 < n; l0 += span) {
    if (tid == 0) s_nwhole = 0u;
    __syncthreads();
    const uint32_t lt = l0 + static_cast<uint32_t>(tid) * gridDim.x;
    if (lt < n) {
      const uint32_t w = a.buf.longs[lt].w;
      if (w > kFinGroupChunks && w < kFinPieceMin) s_whole[atomicAdd(&s_nwhole, 1u)] = lt;
    }
    __syncthreads();
    const uint32_t nwhole = s_nwhole;
    for (uint32_t q = 0; q < nwhole; ++q) {
      const uint32_t li = s_whole[q];
      const uint4 L = a.buf.longs[li];  // {first position, length, first partial, chunks}
      const uint32_t key = a.buf.long_keys[li];
      const TableMeta m = meta_of(a, s_meta, table_of_key(a, s_meta, key));
      finish_run<ST, VE, NCH, false, group_unroll<VE, NCH>()>(a, L, m, key, s_red, s_scratch);
      __syncthreads();  // s_red is reused by the next run
    }
    __syncthreads();  // s_whole and s_nwhole are reused
  }
}

// Grid bounds of seg_fused.  Large batches take more workgroups than fit at
// once, so that the dispatcher keeps refilling the chip as workgroups with few
// items finish (5.2 M lookups: 570 -> 485 us against 4096; 32768 was slower
// again); batches of at most 2^20 lookups are faster with 4096 (0.7 us at
// 270k lookups).
constexpr int64_t kMaxSegBlocks = 16384;
constexpr int64_t kMaxSegBlocksSmall = 4096;
// Grid bound of seg_finalize (a larger grid slowed the finish of many short
// long runs: 16.8 M lookups in 39k long runs, 35 -> 48 us at 32768).
constexpr int64_t kMaxFinBlocks = 4096;

int64_t blocks_for(int64_t items, int gshift, int64_t cap) {
  const int64_t per_block = static_cast<int64_t>(kWavesPerBlock) * (kWave >> gshift);
  int64_t b = (items + per_block - 1) / per_block;
  if (b < 1) b = 1;
  return b < cap ? b : cap;
}

template <int ST, int VE, int NCH, bool REC>
hipError_t run_segments(const BackwardLaunch& a, const uint32_t* keys, const uint32_t* sorted_vals,
                        hipStream_t s, const KernelTimer* kt) {
  const int64_t n = a.num_indices;
  const SegmentBounds ub = segment_bounds(n, a.long_threshold, a.chunk, a.short_max);
  if (!a.front_queued) {
    const int64_t per = int64_t{kBlock} * kQueueRunsPerThread;
    const int64_t qb = (n + per - 1) / per;  // U <= n runs
    launch_timed(kt, "queue_runs", queue_runs, dim3(static_cast<unsigned>(qb < 1024 ? qb : 1024)),
                 dim3(kBlock), 0, s, a);
  }
  if (a.per_table)
    launch_timed(kt, "table_run_starts", table_run_starts, dim3(a.T + 1), dim3(kBlock), 0, s, a);
  const int64_t cap = n > (int64_t{1} << 20) ? kMaxSegBlocks : kMaxSegBlocksSmall;
  int64_t blocks = blocks_for(n, a.gshift, cap);
  if (ub.items1 > blocks) blocks = ub.items1 < cap ? ub.items1 : cap;
  if (a.per_table)
    launch_timed(kt, "seg_fused", seg_fused<ST, VE, NCH, REC, true>, dim3(blocks), dim3(kBlock),
                 0, s, a, keys, sorted_vals);
  else
    launch_timed(kt, "seg_fused", seg_fused<ST, VE, NCH, REC, false>, dim3(blocks), dim3(kBlock),
                 0, s, a, keys, sorted_vals);
  if (!a.finish_in_items) {
    const int64_t fin = ub.longs < kMaxFinBlocks ? ub.longs : kMaxFinBlocks;
    launch_timed(kt, "seg_finalize", seg_finalize<ST, VE, NCH, REC>, dim3(fin), dim3(kBlock), 0,
                 s, a);
  }
  return hipGetLastError();
}

template <int ST, int VE, int NCH>
hipError_t dispatch_rec(const BackwardLaunch& a, const uint32_t* k, const uint32_t* v,
                        hipStream_t s, const KernelTimer* kt) {
  return a.use_rec ? run_segments<ST, VE, NCH, true>(a, k, v, s, kt)
                   : run_segments<ST, VE, NCH, false>(a, k, v, s, kt);
}

template <int ST>
hipError_t dispatch_shape(const BackwardLaunch& a, const uint32_t* k, const uint32_t* v,
                          hipStream_t s, const KernelTimer* kt) {
  if (a.vec) {
    if (a.nch == 1) return dispatch_rec<ST, 4, 1>(a, k, v, s, kt);
    if (a.nch == 4) return dispatch_rec<ST, 4, 4>(a, k, v, s, kt);
  } else {
    if (a.nch == 1) return dispatch_rec<ST, 1, 1>(a, k, v, s, kt);
    if (a.nch == 16) return dispatch_rec<ST, 1, 16>(a, k, v, s, kt);
  }
  return hipErrorInvalidValue;
}

}  // namespace

SegmentBounds segment_bounds(int64_t n, int64_t long_threshold, int chunk, int short_max) {
  SegmentBounds b;
  const int64_t thr = long_threshold > 0 ? long_threshold : 1;
  const int64_t group_max = short_max;  // longest run a lane group takes
  b.longs = n / thr + 1;
  b.chunks = n / chunk + b.longs;
  // queued items: runs longer than group_max that are not long, plus long-run chunks
  b.items1 = n / (group_max + 1) + b.chunks + 1;
  return b;
}

hipError_t launch_segment_reduce_update(const BackwardLaunch& a, const uint32_t* sorted_keys,
                                        const uint32_t* sorted_vals, hipStream_t stream,
                                        const KernelTimer* kt) {
  switch (a.dtype) {
    case kF32: return dispatch_shape<kF32>(a, sorted_keys, sorted_vals, stream, kt);
    case kF16: return dispatch_shape<kF16>(a, sorted_keys, sorted_vals, stream, kt);
    case kBF16: return dispatch_shape<kBF16>(a, sorted_keys, sorted_vals, stream, kt);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tbe
