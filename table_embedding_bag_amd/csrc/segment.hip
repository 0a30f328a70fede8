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
// flight per run:
//   seg_short     one lane group (Gs lanes = one gradient row of 16-byte
//                 chunks) per run of at most Gs lookups: every lane prefetches
//                 one lookup, the group then keeps 8 gradient rows in flight
//                 and updates the row.  Most runs are this short.  Longer runs
//                 are queued (atomic counters give each a contiguous range of
//                 work items).
//   seg_wg        one workgroup per queued item: a medium run (shorter than the
//                 long-run threshold, streamed in one pass and updated at once)
//                 or a 256-lookup chunk of a long run (split accumulation: an
//                 fp32 partial sum per chunk).  The workgroup stages 256 lookups
//                 in LDS and its 256/Gs lane groups keep 4 rows each in flight;
//                 the groups' sums are added in LDS in a fixed order.
//   seg_reduce2   long runs with more than 32 chunks: sums of 32 consecutive
//                 chunk partials.
//   seg_finalize  per long run: its partials summed in chunk order, then the
//                 update.
// Summation order never depends on scheduling (no float atomics), so results
// are reproducible bit for bit.  Sums are kept in fp64: a run may add the same
// gradient row many times over (a hot row hit repeatedly inside one bag), and
// fp32 rounding errors of such correlated sums grow linearly; products c_i * g
// are exact in fp64.  Every stage is its own kernel: no workgroup waits for
// another.
#include "common.hpp"

namespace tbe {
namespace {

constexpr uint32_t kMediumItem = 0x80000000u;

// Gradient rows kept in flight per lane group: 8 in seg_short (4 inside a
// workgroup item) for rows of one 16-byte chunk per lane, fewer when a lane
// holds several chunks, so that registers stay below 128 per lane.
template <int VE, int NCH>
constexpr int group_unroll() {
  return (32 / (VE * NCH)) < 1 ? 1 : ((32 / (VE * NCH)) > 8 ? 8 : 32 / (VE * NCH));
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

// This lane's chunks of gradient row b of table m (zeros where absent).
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
// norm ss; updates the state (one lane writes it).
__device__ __forceinline__ float step_size(const BackwardLaunch& a, uint32_t key, double ss, int D,
                                           bool writer) {
  if (!a.adagrad) return a.lr;
  const float mnew = static_cast<float>(static_cast<double>(a.state[key]) + ss / D);
  if (writer) a.state[key] = mnew;
  return a.lr / (sqrtf(mnew) + a.eps);
}

// Group-wide update of row `key` (this lane's chunks).
template <int ST, int VE, int NCH>
__device__ __forceinline__ void group_update(const BackwardLaunch& a, const TableMeta& m,
                                             uint32_t key, const GroupCtx& g,
                                             const Acc<VE, NCH>& acc) {
  const int D = m.dim;
  const int C = D / VE;
  double ss = 0.0;
  if (a.adagrad) {
#pragma unroll
    for (int c = 0; c < NCH; ++c)
#pragma unroll
      for (int q = 0; q < VE; ++q) ss = fma(acc.v[c][q], acc.v[c][q], ss);
    for (int o = g.Gs >> 1; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, kWave);
  }
  const float step = step_size(a, key, ss, D, g.gl == 0);
  const int64_t row0 = m.woff + static_cast<int64_t>(key - static_cast<uint32_t>(m.roff)) * D;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int chunk = c * g.Gs + g.gl;
    if (chunk < C) {
      float w[VE];
      load_widen<ST, VE>(a.weights, row0 + chunk * VE, w);
#pragma unroll
      for (int q = 0; q < VE; ++q) w[q] = fmaf(-step, static_cast<float>(acc.v[c][q]), w[q]);
      narrow_store<ST, VE>(a.weights, row0 + chunk * VE, w);
    }
  }
}

struct GroupIds {
  int gid, ngroups;
  GroupCtx g;
};

__device__ __forceinline__ GroupIds group_ids(const BackwardLaunch& a) {
  GroupIds r;
  const int Gs = 1 << a.gshift;
  const int per_wave = kWave >> a.gshift;
  const int lane = lane_id();
  const int wave_global = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  r.gid = wave_global * per_wave + (lane >> a.gshift);
  r.ngroups = gridDim.x * kWavesPerBlock * per_wave;
  r.g.gl = lane & (Gs - 1);
  r.g.Gs = Gs;
  return r;
}

// Table metadata staged in LDS (handles with at most kLdsTables tables), so
// that a run's table follows from its row id without a dependent global load.
constexpr int kLdsTables = 256;

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
// runs.  Most runs have one to three lookups, so the per-run instruction
// count is what matters here: the next run's bounds are loaded while the
// current one is processed, every lane prefetches one lookup, the row to
// update and its state are loaded before the gradient rows arrive, the gather
// is unrolled to the run's length (2, 4 or 8 rows in flight) and sums are
// kept in fp32 (at most Gs terms: error below Gs * 2^-24 of the sum of
// magnitudes; longer runs are summed in fp64 by the kernels below).
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

template <int ST, int VE, int NCH, bool REC>
__global__ __launch_bounds__(kBlock) void seg_short(BackwardLaunch a, const uint32_t* sorted_vals) {
  __shared__ TableMeta s_meta[kLdsTables];
  const GroupIds id = group_ids(a);
  const int Gs = id.g.Gs, gl = id.g.gl;
  const int leader = lane_id() & ~(Gs - 1);
  const bool failed = a.buf.counters[kCntError] != 0u;  // a look-back wait gave up earlier
  const uint32_t U = a.buf.counters[kCntUnique];
  if (a.out_num && id.gid == 0 && gl == 0) *a.out_num = failed ? -1 : static_cast<int32_t>(U);
  if (failed) return;
  stage_meta(a, s_meta);
  uint32_t r = id.gid;
  int64_t ns = 0, ne = 0;
  uint32_t nkey = 0;
  if (r < U) {
    ns = a.buf.run_start[r];
    ne = a.buf.run_start[r + 1];
    nkey = a.buf.unique_keys[r];
  }
  for (; r < U; r += id.ngroups) {
    const int64_t s = ns, e = ne;
    const uint32_t key = nkey;
    const uint32_t rn = r + id.ngroups;
    if (rn < U) {
      ns = a.buf.run_start[rn];
      ne = a.buf.run_start[rn + 1];
      nkey = a.buf.unique_keys[rn];
    }
    const int len = static_cast<int>(e - s);
    if (a.out_unique && gl == 0) {
      a.out_unique[r] = static_cast<int32_t>(key);
      a.out_lengths[r] = len;
    }
    if (len > Gs) {
      // queue: a medium run as one workgroup item, a long run as its chunks
      if (len >= a.long_threshold) {
        const uint32_t n1 = static_cast<uint32_t>((len + a.chunk - 1) / a.chunk);
        const uint32_t n2 = n1 > static_cast<uint32_t>(a.super_chunk)
                                ? (n1 + a.super_chunk - 1) / a.super_chunk
                                : 0u;
        uint32_t li = 0, b1 = 0, b2 = 0, it = 0;
        if (gl == 0) {
          li = atomicAdd(&a.buf.counters[kCntLong], 1u);
          b1 = atomicAdd(&a.buf.counters[kCntChunks], n1);
          it = atomicAdd(&a.buf.counters[kCntItems1], n1);
          if (n2) b2 = atomicAdd(&a.buf.counters[kCntItems2], n2);
          a.buf.longs[li] = make_uint4(r, b1, n1, b2);
        }
        li = __shfl(li, leader, kWave);
        b2 = __shfl(b2, leader, kWave);
        it = __shfl(it, leader, kWave);
        for (uint32_t c = gl; c < n1; c += Gs) a.buf.items1[it + c] = make_uint2(li, c);
        for (uint32_t c = gl; c < n2; c += Gs) a.buf.items2[b2 + c] = make_uint2(li, c);
      } else if (gl == 0) {
        const uint32_t it = atomicAdd(&a.buf.counters[kCntItems1], 1u);
        a.buf.items1[it] = make_uint2(r, kMediumItem);
      }
      continue;
    }
    uint32_t my_bag = 0;
    float my_coef = 0.0f;
    if (gl < len) lookup_of<REC>(a, sorted_vals[s + gl], &my_bag, &my_coef);
    const int t = table_of_key(a, s_meta, key);
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
    if (len <= 2)
      gather_short<2, VE, NCH, REC>(a, m, tb, leader, gl, Gs, len, my_bag, my_coef, acc);
    else if (len <= 4)
      gather_short<4, VE, NCH, REC>(a, m, tb, leader, gl, Gs, len, my_bag, my_coef, acc);
    else
      gather_short<group_unroll<VE, NCH>(), VE, NCH, REC>(a, m, tb, leader, gl, Gs, len, my_bag,
                                                           my_coef, acc);
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

template <int ST, int VE, int NCH, bool REC>
__global__ __launch_bounds__(kBlock) void seg_wg(BackwardLaunch a, const uint32_t* sorted_vals) {
  if (a.buf.counters[kCntError] != 0u) return;  // a look-back wait gave up earlier
  constexpr int NV = VE * NCH;                 // values per lane
  constexpr int kElemsPerThread = kMaxDim / kBlock;
  __shared__ uint32_t s_bag[kBlock];
  __shared__ float s_coef[kBlock];
  __shared__ double s_red[kBlock * NV];        // [group][row element]
  __shared__ double s_scratch[kWavesPerBlock];

  const int tid = threadIdx.x;
  const int Gs = 1 << a.gshift;
  const int ngroups = kBlock >> a.gshift;
  const int g = tid >> a.gshift, gl = tid & (Gs - 1);
  const int row_elems = Gs * NV;               // elements per group row in s_red (>= D)
  const uint32_t n = a.buf.counters[kCntItems1];

  for (uint32_t item = blockIdx.x; item < n; item += gridDim.x) {
    const uint2 it = a.buf.items1[item];
    const bool medium = (it.y & kMediumItem) != 0;
    uint32_t r, slot = 0;
    int64_t s, e;
    if (medium) {
      r = it.x;
      s = a.buf.run_start[r];
      e = a.buf.run_start[r + 1];
    } else {
      const uint4 L = a.buf.longs[it.x];
      r = L.x;
      const int64_t rs = a.buf.run_start[r], re = a.buf.run_start[r + 1];
      s = rs + static_cast<int64_t>(it.y) * a.chunk;
      e = min(re, s + a.chunk);
      slot = L.y + it.y;
    }
    const int t = table_of_run<REC>(a, sorted_vals, s);
    const TableMeta m = a.meta[t];
    const int64_t tb = static_cast<int64_t>(t) * a.B;
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
          load_grad<VE, NCH>(a, m, static_cast<int64_t>(bag) - tb, gl, Gs, ok, v[u]);
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
      const uint32_t key = a.buf.unique_keys[r];
      if (a.adagrad) ss = block_sum(ss, s_scratch);
      const float step = step_size(a, key, ss, D, tid == 0);
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
#pragma unroll
      for (int k = 0; k < kElemsPerThread; ++k) {
        const int d = tid + k * kBlock;
        if (d < D) dst[d] = static_cast<float>(gam[k]);
      }
    }
  }
}

// acc += rows [first, first + count) of a partial buffer, in order.
template <int VE, int NCH>
__device__ __forceinline__ void sum_partials(const float* part, int pstride, uint32_t first,
                                             uint32_t count, const GroupCtx& g, int C,
                                             Acc<VE, NCH>& acc) {
  constexpr int kU = group_unroll<VE, NCH>();
  for (uint32_t j = 0; j < count; j += kU) {
    float v[kU][NCH][VE];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const float* row = part + static_cast<int64_t>(first + j + u) * pstride;
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const int chunk = c * g.Gs + g.gl;
        if (j + u < count && chunk < C) {
          if constexpr (VE == 4) {
            const float4 x = *reinterpret_cast<const float4*>(row + chunk * 4);
            v[u][c][0] = x.x; v[u][c][1] = x.y; v[u][c][2] = x.z; v[u][c][3] = x.w;
          } else {
#pragma unroll
            for (int q = 0; q < VE; ++q) v[u][c][q] = row[chunk * VE + q];
          }
        } else {
#pragma unroll
          for (int q = 0; q < VE; ++q) v[u][c][q] = 0.0f;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kU; ++u)
#pragma unroll
      for (int c = 0; c < NCH; ++c)
#pragma unroll
        for (int q = 0; q < VE; ++q) acc.v[c][q] += static_cast<double>(v[u][c][q]);
  }
}

template <int VE, int NCH>
__device__ __forceinline__ void store_partial(float* dst, const GroupCtx& g, int C,
                                              const Acc<VE, NCH>& acc) {
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int chunk = c * g.Gs + g.gl;
    if (chunk < C) {
      if constexpr (VE == 4)
        *reinterpret_cast<float4*>(dst + chunk * 4) =
            make_float4(static_cast<float>(acc.v[c][0]), static_cast<float>(acc.v[c][1]),
                        static_cast<float>(acc.v[c][2]), static_cast<float>(acc.v[c][3]));
      else
#pragma unroll
        for (int q = 0; q < VE; ++q) dst[chunk * VE + q] = static_cast<float>(acc.v[c][q]);
    }
  }
}

template <int VE, int NCH, bool REC>
__global__ __launch_bounds__(kBlock) void seg_reduce2(BackwardLaunch a, const uint32_t* sorted_vals) {
  if (a.buf.counters[kCntError] != 0u) return;  // a look-back wait gave up earlier
  const GroupIds id = group_ids(a);
  const uint32_t n = a.buf.counters[kCntItems2];
  for (uint32_t j = id.gid; j < n; j += id.ngroups) {
    const uint2 it = a.buf.items2[j];
    const uint4 L = a.buf.longs[it.x];
    const uint32_t c0 = it.y * a.super_chunk;
    const uint32_t cnt = min(static_cast<uint32_t>(a.super_chunk), L.z - c0);
    const int t = table_of_run<REC>(a, sorted_vals, a.buf.run_start[L.x]);
    const int C = a.meta[t].dim / VE;
    Acc<VE, NCH> acc;
    acc.zero();
    sum_partials<VE, NCH>(a.buf.partial1, a.pstride, L.y + c0, cnt, id.g, C, acc);
    store_partial<VE, NCH>(a.buf.partial2 + static_cast<int64_t>(j) * a.pstride, id.g, C, acc);
  }
}

template <int ST, int VE, int NCH, bool REC>
__global__ __launch_bounds__(kBlock) void seg_finalize(BackwardLaunch a, const uint32_t* sorted_vals) {
  if (a.buf.counters[kCntError] != 0u) return;  // a look-back wait gave up earlier
  const GroupIds id = group_ids(a);
  const uint32_t n = a.buf.counters[kCntLong];
  for (uint32_t li = id.gid; li < n; li += id.ngroups) {
    const uint4 L = a.buf.longs[li];
    const int t = table_of_run<REC>(a, sorted_vals, a.buf.run_start[L.x]);
    const TableMeta m = a.meta[t];
    const int C = m.dim / VE;
    Acc<VE, NCH> acc;
    acc.zero();
    if (L.z > static_cast<uint32_t>(a.super_chunk)) {
      const uint32_t n2 = (L.z + a.super_chunk - 1) / a.super_chunk;
      sum_partials<VE, NCH>(a.buf.partial2, a.pstride, L.w, n2, id.g, C, acc);
    } else {
      sum_partials<VE, NCH>(a.buf.partial1, a.pstride, L.y, L.z, id.g, C, acc);
    }
    group_update<ST, VE, NCH>(a, m, a.buf.unique_keys[L.x], id.g, acc);
  }
}

// Upper bound of concurrently useful workgroups for the grid-stride kernels.
constexpr int64_t kMaxSegBlocks = 4096;

int64_t blocks_for(int64_t items, int gshift) {
  const int64_t per_block = static_cast<int64_t>(kWavesPerBlock) * (kWave >> gshift);
  int64_t b = (items + per_block - 1) / per_block;
  if (b < 1) b = 1;
  return b < kMaxSegBlocks ? b : kMaxSegBlocks;
}

template <int ST, int VE, int NCH, bool REC>
hipError_t run_segments(const BackwardLaunch& a, const uint32_t* sorted_vals, hipStream_t s,
                        StageHook hook, void* ctx) {
  const int64_t n = a.num_indices;
  const SegmentBounds ub = segment_bounds(n, a.long_threshold, a.chunk, a.super_chunk, a.gshift);
  hipLaunchKernelGGL((seg_short<ST, VE, NCH, REC>), dim3(blocks_for(n, a.gshift)), dim3(kBlock),
                     0, s, a, sorted_vals);
  if (hook) hook(ctx, "seg_short");
  const int64_t wg = ub.items1 < kMaxSegBlocks ? (ub.items1 > 0 ? ub.items1 : 1) : kMaxSegBlocks;
  hipLaunchKernelGGL((seg_wg<ST, VE, NCH, REC>), dim3(wg), dim3(kBlock), 0, s, a, sorted_vals);
  if (hook) hook(ctx, "seg_wg");
  hipLaunchKernelGGL((seg_reduce2<VE, NCH, REC>), dim3(blocks_for(ub.items2, a.gshift)),
                     dim3(kBlock), 0, s, a, sorted_vals);
  if (hook) hook(ctx, "seg_reduce2");
  hipLaunchKernelGGL((seg_finalize<ST, VE, NCH, REC>), dim3(blocks_for(ub.longs, a.gshift)),
                     dim3(kBlock), 0, s, a, sorted_vals);
  if (hook) hook(ctx, "seg_finalize");
  return hipGetLastError();
}

template <int ST, int VE, int NCH>
hipError_t dispatch_rec(const BackwardLaunch& a, const uint32_t* v, hipStream_t s, StageHook h,
                        void* c) {
  return a.use_rec ? run_segments<ST, VE, NCH, true>(a, v, s, h, c)
                   : run_segments<ST, VE, NCH, false>(a, v, s, h, c);
}

template <int ST>
hipError_t dispatch_shape(const BackwardLaunch& a, const uint32_t* v, hipStream_t s, StageHook h,
                          void* c) {
  if (a.vec) {
    if (a.nch == 1) return dispatch_rec<ST, 4, 1>(a, v, s, h, c);
    if (a.nch == 4) return dispatch_rec<ST, 4, 4>(a, v, s, h, c);
  } else {
    if (a.nch == 1) return dispatch_rec<ST, 1, 1>(a, v, s, h, c);
    if (a.nch == 16) return dispatch_rec<ST, 1, 16>(a, v, s, h, c);
  }
  return hipErrorInvalidValue;
}

}  // namespace

SegmentBounds segment_bounds(int64_t n, int64_t long_threshold, int chunk, int super_chunk,
                             int gshift) {
  SegmentBounds b;
  const int64_t thr = long_threshold > 0 ? long_threshold : 1;
  const int64_t group_max = int64_t{1} << gshift;  // longest run a lane group takes alone
  b.longs = n / thr + 1;
  b.chunks = n / chunk + b.longs;
  // queued items: runs longer than group_max that are not long, plus long-run chunks
  b.items1 = n / (group_max + 1) + b.chunks + 1;
  b.items2 = b.chunks / super_chunk + b.longs;
  return b;
}

hipError_t launch_segment_reduce_update(const BackwardLaunch& a, const uint32_t* sorted_vals,
                                        hipStream_t stream, StageHook hook, void* ctx) {
  switch (a.dtype) {
    case kF32: return dispatch_shape<kF32>(a, sorted_vals, stream, hook, ctx);
    case kF16: return dispatch_shape<kF16>(a, sorted_vals, stream, hook, ctx);
    case kBF16: return dispatch_shape<kBF16>(a, sorted_vals, stream, hook, ctx);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tbe
