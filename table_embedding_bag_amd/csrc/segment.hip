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
// Work layout.  A lane group of Gs lanes holds one gradient row (16-byte fp32
// chunks; rows wider than 256 use chunk sets per lane), so a wave runs 64/Gs
// runs side by side.
//   seg_short     grid-stride over runs: a run shorter than the threshold is
//                 summed in one pass (U gradient rows in flight per lane group)
//                 and its row updated at once; a long run is cut into chunks
//                 of `chunk` lookups and queued (atomic counters give each
//                 long run a contiguous range of work items).
//   seg_partial   one fp32 partial sum per chunk of a long run.
//   seg_reduce2   for long runs with more than `super_chunk` chunks: partial
//                 sums of super_chunk consecutive chunk partials.
//   seg_finalize  per long run: sums its partials in chunk order, then the
//                 update.  Summation order is fixed, so results do not depend
//                 on scheduling (no float atomics anywhere).
// Each stage is its own kernel, so no workgroup ever waits for another.
#include "common.hpp"

namespace tbe {
namespace {

constexpr int kSegUnroll = 4;  // gradient rows in flight per lane group

// The slice of a summed gradient row held by one lane: NCH chunk sets of VE
// values.  Sums are kept in fp64: a run may add the same gradient row many
// times over (a hot row hit repeatedly inside one bag), and fp32 rounding
// errors of such correlated sums grow linearly.  The products c_i * g are
// exact in fp64, so each add rounds once at 2^-53; the kernels stay bound by
// memory traffic, not by the fp64 adds.
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

// Sum c_i * G rows over sorted positions [s, e) of a run of table t.
template <int VE, int NCH, bool REC>
__device__ __forceinline__ void gather_sum(const BackwardLaunch& a, const uint32_t* sorted_vals,
                                           int t, const TableMeta& m, const GroupCtx& g,
                                           int64_t s, int64_t e, Acc<VE, NCH>& acc) {
  const int C = m.dim / VE;  // chunks per row
  const float* gcol = a.grad + m.doff;
  for (int64_t j = s; j < e; j += kSegUnroll) {
    uint32_t bag[kSegUnroll];
    float coef[kSegUnroll];
#pragma unroll
    for (int u = 0; u < kSegUnroll; ++u) {
      bag[u] = 0u;
      coef[u] = 0.0f;
      if (j + u < e) lookup_of<REC>(a, sorted_vals[j + u], &bag[u], &coef[u]);
    }
    float v[kSegUnroll][NCH][VE];
#pragma unroll
    for (int u = 0; u < kSegUnroll; ++u) {
      const int64_t b = static_cast<int64_t>(bag[u]) - static_cast<int64_t>(t) * a.B;
      const float* grow = gcol + b * a.sum_dims;
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const int chunk = c * g.Gs + g.gl;
        if (j + u < e && chunk < C) {
          if constexpr (VE == 4) {
            const float4 x = *reinterpret_cast<const float4*>(grow + chunk * 4);
            v[u][c][0] = x.x; v[u][c][1] = x.y; v[u][c][2] = x.z; v[u][c][3] = x.w;
          } else {
#pragma unroll
            for (int q = 0; q < VE; ++q) v[u][c][q] = grow[chunk * VE + q];
          }
        } else {
#pragma unroll
          for (int q = 0; q < VE; ++q) v[u][c][q] = 0.0f;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kSegUnroll; ++u)
#pragma unroll
      for (int c = 0; c < NCH; ++c)
#pragma unroll
        for (int q = 0; q < VE; ++q)
          acc.v[c][q] = fma(static_cast<double>(coef[u]), static_cast<double>(v[u][c][q]), acc.v[c][q]);
  }
}

// Apply the optimizer to row `key` of table t with summed gradient acc.
template <int ST, int VE, int NCH>
__device__ __forceinline__ void apply_update(const BackwardLaunch& a, const TableMeta& m,
                                             uint32_t key, const GroupCtx& g,
                                             const Acc<VE, NCH>& acc) {
  const int D = m.dim;
  const int C = D / VE;
  float step = a.lr;
  if (a.adagrad) {
    double ss = 0.0;
#pragma unroll
    for (int c = 0; c < NCH; ++c)
#pragma unroll
      for (int q = 0; q < VE; ++q) ss = fma(acc.v[c][q], acc.v[c][q], ss);
    for (int o = g.Gs >> 1; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, kWave);
    const float mnew = static_cast<float>(static_cast<double>(a.state[key]) + ss / D);
    if (g.gl == 0) a.state[key] = mnew;
    step = a.lr / (sqrtf(mnew) + a.eps);
  }
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

// Table of a run, from the bag of its first lookup.
template <bool REC>
__device__ __forceinline__ int table_of_run(const BackwardLaunch& a, const uint32_t* sorted_vals,
                                            int64_t first) {
  uint32_t bag;
  float coef;
  lookup_of<REC>(a, sorted_vals[first], &bag, &coef);
  return static_cast<int>(bag / static_cast<uint32_t>(a.B));
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

template <int ST, int VE, int NCH, bool REC>
__global__ __launch_bounds__(kBlock) void seg_short(BackwardLaunch a, const uint32_t* sorted_vals) {
  const GroupIds id = group_ids(a);
  const uint32_t U = a.buf.counters[kCntUnique];
  if (a.out_num && id.gid == 0 && id.g.gl == 0) *a.out_num = static_cast<int32_t>(U);
  for (uint32_t r = id.gid; r < U; r += id.ngroups) {
    const int64_t s = a.buf.run_start[r], e = a.buf.run_start[r + 1];
    const int64_t len = e - s;
    const uint32_t key = a.buf.unique_keys[r];
    if (a.out_unique && id.g.gl == 0) {
      a.out_unique[r] = static_cast<int32_t>(key);
      a.out_lengths[r] = static_cast<int32_t>(len);
    }
    if (len >= a.long_threshold) {
      // queue the long run: level-1 chunks, and level-2 groups of chunks
      const uint32_t n1 = static_cast<uint32_t>((len + a.chunk - 1) / a.chunk);
      const uint32_t n2 = n1 > static_cast<uint32_t>(a.super_chunk)
                              ? (n1 + a.super_chunk - 1) / a.super_chunk
                              : 0u;
      uint32_t li = 0, b1 = 0, b2 = 0;
      if (id.g.gl == 0) {
        li = atomicAdd(&a.buf.counters[kCntLong], 1u);
        b1 = atomicAdd(&a.buf.counters[kCntItems1], n1);
        if (n2) b2 = atomicAdd(&a.buf.counters[kCntItems2], n2);
        a.buf.longs[li] = make_uint4(r, b1, n1, b2);
      }
      const int leader = lane_id() & ~(id.g.Gs - 1);
      li = __shfl(li, leader, kWave);
      b1 = __shfl(b1, leader, kWave);
      b2 = __shfl(b2, leader, kWave);
      for (uint32_t c = id.g.gl; c < n1; c += id.g.Gs) a.buf.items1[b1 + c] = make_uint2(li, c);
      for (uint32_t c = id.g.gl; c < n2; c += id.g.Gs) a.buf.items2[b2 + c] = make_uint2(li, c);
      continue;
    }
    const int t = table_of_run<REC>(a, sorted_vals, s);
    const TableMeta m = a.meta[t];
    Acc<VE, NCH> acc;
    acc.zero();
    gather_sum<VE, NCH, REC>(a, sorted_vals, t, m, id.g, s, e, acc);
    apply_update<ST, VE, NCH>(a, m, key, id.g, acc);
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

// acc += sum of rows [first, first + count) of a partial buffer, in order.
template <int VE, int NCH>
__device__ __forceinline__ void sum_partials(const float* part, int pstride, uint32_t first,
                                             uint32_t count, const GroupCtx& g, int C,
                                             Acc<VE, NCH>& acc) {
  for (uint32_t j = 0; j < count; j += kSegUnroll) {
    float v[kSegUnroll][NCH][VE];
#pragma unroll
    for (int u = 0; u < kSegUnroll; ++u) {
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
    for (int u = 0; u < kSegUnroll; ++u)
#pragma unroll
      for (int c = 0; c < NCH; ++c)
#pragma unroll
        for (int q = 0; q < VE; ++q) acc.v[c][q] += static_cast<double>(v[u][c][q]);
  }
}

template <int VE, int NCH, bool REC>
__global__ __launch_bounds__(kBlock) void seg_partial(BackwardLaunch a, const uint32_t* sorted_vals) {
  const GroupIds id = group_ids(a);
  const uint32_t n = a.buf.counters[kCntItems1];
  for (uint32_t j = id.gid; j < n; j += id.ngroups) {
    const uint2 it = a.buf.items1[j];
    const uint4 L = a.buf.longs[it.x];
    const int64_t rs = a.buf.run_start[L.x], re = a.buf.run_start[L.x + 1];
    const int64_t s = rs + static_cast<int64_t>(it.y) * a.chunk;
    const int64_t e = min(re, s + a.chunk);
    const int t = table_of_run<REC>(a, sorted_vals, rs);
    const TableMeta m = a.meta[t];
    Acc<VE, NCH> acc;
    acc.zero();
    gather_sum<VE, NCH, REC>(a, sorted_vals, t, m, id.g, s, e, acc);
    store_partial<VE, NCH>(a.buf.partial1 + static_cast<int64_t>(j) * a.pstride, id.g, m.dim / VE,
                           acc);
  }
}

template <int VE, int NCH, bool REC>
__global__ __launch_bounds__(kBlock) void seg_reduce2(BackwardLaunch a, const uint32_t* sorted_vals) {
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
    apply_update<ST, VE, NCH>(a, m, a.buf.unique_keys[L.x], id.g, acc);
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
  const int64_t runs_ub = n;
  const int64_t long_ub = n / (a.long_threshold > 0 ? a.long_threshold : 1) + 1;
  const int64_t items1_ub = n / a.chunk + long_ub;
  const int64_t items2_ub = items1_ub / a.super_chunk + long_ub;
  hipLaunchKernelGGL((seg_short<ST, VE, NCH, REC>), dim3(blocks_for(runs_ub, a.gshift)),
                     dim3(kBlock), 0, s, a, sorted_vals);
  if (hook) hook(ctx, "segment_short");
  hipLaunchKernelGGL((seg_partial<VE, NCH, REC>), dim3(blocks_for(items1_ub, a.gshift)),
                     dim3(kBlock), 0, s, a, sorted_vals);
  hipLaunchKernelGGL((seg_reduce2<VE, NCH, REC>), dim3(blocks_for(items2_ub, a.gshift)),
                     dim3(kBlock), 0, s, a, sorted_vals);
  hipLaunchKernelGGL((seg_finalize<ST, VE, NCH, REC>), dim3(blocks_for(long_ub, a.gshift)),
                     dim3(kBlock), 0, s, a, sorted_vals);
  if (hook) hook(ctx, "segment_long");
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
