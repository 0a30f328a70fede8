// forward.hip -- pooled multi-table lookup (the TBE forward) for gfx950.
//
// What it computes (kimbodo.com/?p=28372, "What Happened"; "FBTriton Rewrites
// Table Batched Embedding", "Responsibilities of the forward and backward
// passes"): for every bag k = t*B + b,
//     Y[b, doff_t + d] = s_k * sum_{i in bag k} p_i * W_t[x_i, d]
// with s_k = 1 (sum) or 1/L_k (mean; empty bags give 0), p_i the optional
// per-sample weight, and fp32 accumulation whatever the storage dtype.  All
// tables are covered by a single launch.
//
// Mapping onto CDNA4:
//  * A lane group of Gs = 2^gshift lanes covers one table row: each lane loads
//    one 16-byte chunk (4 fp32 or 8 fp16/bf16 elements), so a row read is one
//    coalesced access.  Rows wider than 64 chunks are walked in chunk sets.
//  * A bag is handled by a sub-wave of SW = Gs * 2^lshift lanes (at most the
//    whole wave): its R = SW / Gs lane groups read R different rows of the bag
//    per instruction and U instructions are issued before the first result
//    is consumed, so a bag keeps R*U row reads in flight.  lshift is picked per
//    call from the mean bag length so that one such round usually covers a
//    bag.  Small rows and short bags therefore pack several bags per wave;
//    wide rows or long bags get a whole wave per bag.
//  * The bag's row ids are loaded once, one per lane of the sub-wave
//    (coalesced), and broadcast to the lane groups with ds_bpermute.
//  * At the end the R partial sums are folded with cross-lane adds and the
//    first lane group writes the fp32 output with 16-byte stores.
//  * Workgroups are renumbered so that every XCD works on a contiguous range
//    of tables, which keeps each table's hot rows in one XCD's L2.
#include <algorithm>

#include "common.hpp"
#include "linearize.hpp"

namespace tbe {
namespace {

constexpr int kUnroll = kFwdUnroll;

template <typename IT>
__device__ __forceinline__ int64_t ld_index(const void* p, int64_t i) {
  return static_cast<int64_t>(static_cast<const IT*>(p)[i]);
}

// One tile (kWavesPerBlock waves' worth of bags of one table) of the pooled
// lookup.  ST: storage dtype code; IT: index type; VEC: 16-byte chunks (else
// one element per lane); PSW: per-sample weights present.  logical numbers
// the tiles table after table; wave is the wave's index inside the tile.
// UNC: each batch of rows is loaded unconditionally (absent lookups and lanes
// past the row read the table's first chunk and add nothing), so that all of
// the batch's loads are in flight together; otherwise only present lookups
// load, under a branch the compiler resolves one load at a time.  The first
// pays on large batches, whose rows come from HBM (5.2 M lookups over 32
// tables of up to 1e7 rows: 249 -> 180 us); on small ones, whose rows are
// mostly in L2 and whose ragged bags leave many lanes idle, the extra loads
// cost more than they hide (270 k lookups: +0.4 us).
template <int ST, typename IT, bool VEC, bool PSW, bool UNC = false>
__device__ __forceinline__ void fwd_tile(const ForwardLaunch& a, int logical, int wave) {
  constexpr int SB = StorageTraits<ST>::bytes;
  constexpr int VE = VEC ? 16 / SB : 1;  // elements per lane chunk

  if (logical >= a.T * a.tiles_per_table) return;
  const int listed = logical / a.tiles_per_table;
  const int tile = logical - listed * a.tiles_per_table;
  const int t = a.table_list ? a.table_list[listed] : listed;
  const TableMeta m = a.meta[t];

  const int lane = lane_id();
  const int gshift = m.fwd_gshift;
  const int swshift = min(6, gshift + a.lshift);
  const int SW = 1 << swshift;                  // lanes per bag
  const int Gs = 1 << gshift;                   // lanes per row
  const int R = SW >> gshift;                   // rows per instruction per bag
  const int sl = lane & (SW - 1);               // lane within the bag's sub-wave
  const int g = sl >> gshift;                   // lane group within the sub-wave
  const int gl = sl & (Gs - 1);                 // lane within the lane group
  const int sub_base = lane & ~(SW - 1);

  const int b = ((tile * kWavesPerBlock + wave) << (6 - swshift)) + (lane >> swshift);
  const bool bag_ok = b < a.B;
  const int64_t k = static_cast<int64_t>(t) * a.B + b;
  int64_t start = 0, end = 0;
  if (bag_ok) {
    start = ld_index<IT>(a.offsets, k);
    end = ld_index<IT>(a.offsets, k + 1);
  }
  const int D = m.dim;
  const int C = VEC ? D / VE : D;               // chunks per row
  const void* wbase = static_cast<const char*>(a.weights) + m.woff * SB;
  float scale = 1.0f;
  if (a.mean) scale = (end > start) ? 1.0f / static_cast<float>(end - start) : 0.0f;
  float* orow = a.out + static_cast<int64_t>(b) * a.sum_dims + m.doff;
  if (a.split_len > 0 && end - start > a.split_len) {  // the same on the bag's sub-wave
    // a long bag: this sub-wave pools its first split_len lookups and its
    // first lane queues the other segments (slots always fit: host-checked)
    if (sl == 0) {
      const int64_t L = end - start;
      const uint32_t nseg = static_cast<uint32_t>((L - 1) / a.split_len);  // segments after the first
      const uint32_t base = atomicAdd(&a.split_ctr[0], nseg);
      const uint32_t li = atomicAdd(&a.split_ctr[1], 1u);
      a.split_long[li] = make_uint4(static_cast<uint32_t>(k), base, nseg, 0u);
      for (uint32_t j = 0; j < nseg; ++j)
        a.split_seg[base + j] = make_uint2(static_cast<uint32_t>(k), j + 1);
    }
    end = start + a.split_len;
  }

  for (int cb = 0; cb < C; cb += Gs) {
    const int chunk = cb + gl;
    const bool lane_ok = chunk < C;
    float acc[VE];
#pragma unroll
    for (int e = 0; e < VE; ++e) acc[e] = 0.0f;

    for (int64_t j0 = start; j0 < end; j0 += SW) {
      const int n = static_cast<int>(min(static_cast<int64_t>(SW), end - j0));
      int my_row = 0;
      float my_p = 1.0f;
      if (sl < n) {
        my_row = static_cast<int>(ld_index<IT>(a.indices, j0 + sl));
        if constexpr (PSW) my_p = a.psw[j0 + sl];
      }
      for (int r = 0; r < n; r += R * kUnroll) {
        float v[kUnroll][VE];
        float p[kUnroll];
        bool ok[kUnroll];
        if constexpr (UNC) {
          int row[kUnroll];
#pragma unroll
          for (int u = 0; u < kUnroll; ++u) {
            const int jj = r + u * R + g;
            const int src = sub_base + min(jj, SW - 1);
            row[u] = __shfl(my_row, src, kWave);
            p[u] = PSW ? __shfl(my_p, src, kWave) : 1.0f;
            ok[u] = jj < n && lane_ok;
          }
#pragma unroll
          for (int u = 0; u < kUnroll; ++u)
            load_widen<ST, VE>(wbase, ok[u] ? static_cast<int64_t>(row[u]) * D + chunk * VE : 0,
                               v[u]);
        } else {
#pragma unroll
          for (int u = 0; u < kUnroll; ++u) {
            const int jj = r + u * R + g;
            const int src = sub_base + min(jj, SW - 1);
            const int row = __shfl(my_row, src, kWave);
            p[u] = PSW ? __shfl(my_p, src, kWave) : 1.0f;
            ok[u] = true;
            if (jj < n && lane_ok) {
              load_widen<ST, VE>(wbase, static_cast<int64_t>(row) * D + chunk * VE, v[u]);
            } else {
#pragma unroll
              for (int e = 0; e < VE; ++e) v[u][e] = 0.0f;
            }
          }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
#pragma unroll
          for (int e = 0; e < VE; ++e) {
            const float x = ok[u] ? v[u][e] : 0.0f;
            if constexpr (PSW)
              acc[e] = fmaf(p[u], x, acc[e]);
            else
              acc[e] += x;
          }
        }
      }
    }
    // fold the R lane groups of the bag
    for (int o = SW >> 1; o >= Gs; o >>= 1) {
#pragma unroll
      for (int e = 0; e < VE; ++e) acc[e] += __shfl_xor(acc[e], o, kWave);
    }
    if (bag_ok && g == 0 && lane_ok) {
      float* dst = orow + chunk * VE;
      if constexpr (VE % 4 == 0) {
#pragma unroll
        for (int e = 0; e < VE; e += 4)
          *reinterpret_cast<float4*>(dst + e) =
              make_float4(acc[e] * scale, acc[e + 1] * scale, acc[e + 2] * scale, acc[e + 3] * scale);
      } else {
#pragma unroll
        for (int e = 0; e < VE; ++e) dst[e] = acc[e] * scale;
      }
    }
  }
}

template <int ST, typename IT, bool VEC, bool PSW, bool UNC>
__global__ __launch_bounds__(kBlock) void fwd_gather_pool(ForwardLaunch a) {
  fwd_tile<ST, IT, VEC, PSW, UNC>(a, xcd_contiguous_block(blockIdx.x, gridDim.x),
                                  threadIdx.x >> 6);
}

// Pooled lookup of small tables from LDS.  A workgroup stages one table in
// LDS once (row r at chunk slots r*GS .. r*GS + C - 1, then a row of zeros)
// and its waves pool blocks of 64 consecutive bags of that table: a block's
// offsets are one load per lane, then every bag's first GS ids are loaded (one
// per lane), and the rows are read from LDS.  A wave's blocks are pipelined:
// the next block's ids and the offsets of the block after it are loaded before
// a block is pooled.  Within a block, steps of NB = 64 / GS bags give each bag
// one lane group of GS lanes (lane gl holds chunk gl of a row).  A round reads
// the rows of GS lookups at once, those past the bag's end from the zero row;
// adding those zeros changes no sum, as in the gather kernel.  A bag keeps the
// gather kernel's R partial sums (rows j = g mod R, in lookup order) and folds
// them in the same tree, so both kernels give the same bits.  Requires
// R <= min(GS, kLdsFwdMaxR) and rows of at most GS chunks; no split bags.
template <int ST, typename IT, bool PSW, int GSH, int R>
__global__ __launch_bounds__(kLdsFwdThreads) void fwd_lds_pool(ForwardLaunch a,
                                                               int wgs_per_table) {
  constexpr int SB = StorageTraits<ST>::bytes;
  constexpr int VE = 16 / SB;
  constexpr int GS = 1 << GSH;
  constexpr int NB = kWave / GS;
  constexpr int NW = kLdsFwdThreads / kWave;
  constexpr int kStage = 8;  // staging loads in flight per thread
  // lookups whose rows are read at once (half a round with weights and rows of
  // 8 chunks, which would otherwise spill registers)
  constexpr int PART = (PSW && GSH == 3) ? GS / 2 : GS;
  static_assert(PART % R == 0, "partial sums stay aligned to the reads");
  static_assert(R <= GS && R <= kLdsFwdMaxR, "a bag's partial sums fit a round of GS lookups");
  __shared__ uint4 s_tab[kLdsFwdBytes / 16 + (1 << kLdsFwdMaxGshift)];

  const int wg = xcd_contiguous_block(blockIdx.x, gridDim.x);
  const int listed = wg / wgs_per_table, part = wg - listed * wgs_per_table;
  const int t = a.table_list ? a.table_list[listed] : listed;
  const TableMeta m = a.meta[t];
  const int C = m.dim / VE;  // chunks per row (at most GS, host-checked)
  const int zrow = m.rows;   // the row of zeros
  {
    const uint4* src =
        reinterpret_cast<const uint4*>(static_cast<const char*>(a.weights) + m.woff * SB);
    const int nslot = (m.rows + 1) << GSH;
    for (int i0 = 0; i0 < nslot; i0 += kLdsFwdThreads * kStage) {
      uint4 v[kStage];
#pragma unroll
      for (int q = 0; q < kStage; ++q) {
        const int i = i0 + q * kLdsFwdThreads + static_cast<int>(threadIdx.x);
        const int r = i >> GSH, c = i & (GS - 1);
        v[q] = make_uint4(0u, 0u, 0u, 0u);
        if (r < m.rows && c < C) v[q] = src[r * C + c];
      }
#pragma unroll
      for (int q = 0; q < kStage; ++q) {
        const int i = i0 + q * kLdsFwdThreads + static_cast<int>(threadIdx.x);
        if (i < nslot) s_tab[i] = v[q];
      }
    }
  }
  __syncthreads();

  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int g = lane >> GSH, gl = lane & (GS - 1);
  const int nblk = (a.B + kWave - 1) / kWave;
  const int64_t k0 = static_cast<int64_t>(t) * a.B;
  const int bstride = wgs_per_table * NW;
  // software pipeline over the wave's blocks: while one block is pooled, the
  // next block's first ids and the offsets of the block after it are in flight
  // Loads and stores below take no branch that depends on the lane: absent
  // bags past B repeat bag B - 1 and lanes past a row's chunks repeat chunk 0,
  // storing the same values to the same places, and ids past a bag's end read
  // an id of the batch and take the zero row instead.  (With lane-dependent
  // branches the compiler made every block wait for all of its stores.)
  const int cg = gl < C ? gl : 0;
  auto load_offsets = [&](int blk, int64_t& lo, int64_t& hi) {
    const int b = min(min(blk, nblk - 1) * kWave + lane, a.B - 1);
    lo = ld_index<IT>(a.offsets, k0 + b);
    hi = ld_index<IT>(a.offsets, k0 + b + 1);
  };
  // ids r0 + gl of the bag [st, st + len) (the zero row past its end)
  auto load_id = [&](int64_t st, int len, int r0, int& x, float& pw) {
    const bool in = r0 + gl < len;
    const int64_t p = in ? st + r0 + gl : (len > 0 ? st : 0);  // (n > 0 here)
    const int v = static_cast<int>(ld_index<IT>(a.indices, p));
    x = in ? v : zrow;
    pw = 1.0f;
    if constexpr (PSW) {
      const float q = a.psw[p];
      pw = in ? q : 1.0f;
    }
  };
  auto load_ids = [&](int64_t lo, int64_t hi, int (&x)[GS], float (&pw)[GS]) {
#pragma unroll
    for (int s = 0; s < GS; ++s) {
      const int64_t st = __shfl(lo, s * NB + g, kWave);
      const int len = static_cast<int>(__shfl(hi, s * NB + g, kWave) - st);
      load_id(st, len, 0, x[s], pw[s]);
    }
  };
  int blk = part * NW + wave;
  int64_t lo, hi, lo_n, hi_n;
  int x[GS], x_n[GS];
  float pw[GS], pw_n[GS];
  load_offsets(blk, lo, hi);
  load_ids(lo, hi, x, pw);
  load_offsets(blk + bstride, lo_n, hi_n);
  for (; blk < nblk; blk += bstride) {
    const int b0 = blk * kWave;
    load_ids(lo_n, hi_n, x_n, pw_n);
    int64_t lo_nn, hi_nn;
    load_offsets(blk + 2 * bstride, lo_nn, hi_nn);
#pragma unroll
    for (int s = 0; s < GS; ++s) {
      const int b = min(b0 + s * NB + g, a.B - 1);
      // (the bag's start and length again: cheaper than keeping them in registers)
      const int64_t st = __shfl(lo, s * NB + g, kWave);
      const int len = static_cast<int>(__shfl(hi, s * NB + g, kWave) - st);
      float acc[R][VE];
#pragma unroll
      for (int u = 0; u < R; ++u)
#pragma unroll
        for (int e = 0; e < VE; ++e) acc[u][e] = 0.0f;
      // one round: the rows of ids r0 .. r0 + GS - 1 of every bag of the step,
      // read PART lookups at a time (all GS unless the weights' registers are
      // needed too)
      auto round = [&](int xr, float pr) {
#pragma unroll
        for (int h0 = 0; h0 < GS; h0 += PART) {
          uint4 w[PART];
          float p[PART];
#pragma unroll
          for (int j = 0; j < PART; ++j) {
            const int row = __shfl(xr, (g << GSH) + h0 + j, kWave);
            p[j] = PSW ? __shfl(pr, (g << GSH) + h0 + j, kWave) : 1.0f;
            w[j] = s_tab[(row << GSH) + cg];
          }
#pragma unroll
          for (int j0 = 0; j0 < PART; j0 += R) {
#pragma unroll
            for (int u = 0; u < R; ++u) {
              float v[VE];
              widen_chunk<ST>(w[j0 + u], v);
#pragma unroll
              for (int e = 0; e < VE; ++e) {
                if constexpr (PSW)
                  acc[u][e] = fmaf(p[j0 + u], v[e], acc[u][e]);
                else
                  acc[u][e] += v[e];
              }
            }
          }
        }
      };
      round(x[s], pw[s]);
      // ids past the first GS of the longer bags: loaded when needed (kept
      // out of the first round, whose ids were loaded a block ahead)
      if (__any(GS < len)) {
        for (int r0 = GS;; r0 += GS) {
          int xr;
          float pr;
          load_id(st, len, r0, xr, pr);
          round(xr, pr);
          if (!__any(r0 + GS < len)) break;
        }
      }
      // fold the R partial sums as the gather kernel's lane groups do
#pragma unroll
      for (int h = R >> 1; h >= 1; h >>= 1)
#pragma unroll
        for (int u = 0; u < h; ++u)
#pragma unroll
          for (int e = 0; e < VE; ++e) acc[u][e] += acc[u + h][e];
      float scale = 1.0f;
      if (a.mean) scale = len > 0 ? 1.0f / static_cast<float>(len) : 0.0f;
      float* dst = a.out + static_cast<int64_t>(b) * a.sum_dims + m.doff + cg * VE;
#pragma unroll
      for (int e = 0; e < VE; e += 4)
        *reinterpret_cast<float4*>(dst + e) = make_float4(acc[0][e] * scale, acc[0][e + 1] * scale,
                                                          acc[0][e + 2] * scale, acc[0][e + 3] * scale);
    }
    lo = lo_n;
    hi = hi_n;
    lo_n = lo_nn;
    hi_n = hi_nn;
#pragma unroll
    for (int s = 0; s < GS; ++s) x[s] = x_n[s], pw[s] = pw_n[s];
  }
}

// Segments of split bags (skew balancing: kimbodo.com/?p=28372, "Kimbodo
// Engineering Perspective", names load imbalance across lookups as a risk):
// one wave per queued segment pools its up to split_len lookups with lane
// groups as the pooled lookup does and writes the scaled sum.
template <int ST, typename IT, bool VEC, bool PSW>
__global__ __launch_bounds__(kBlock) void fwd_split_segments(ForwardLaunch a) {
  constexpr int SB = StorageTraits<ST>::bytes;
  constexpr int VE = VEC ? 16 / SB : 1;
  const uint32_t nseg = a.split_ctr[0];
  const int lane = lane_id();
  for (uint32_t si = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6); si < nseg;
       si += gridDim.x * kWavesPerBlock) {
    const uint2 sd = a.split_seg[si];
    const int64_t k = sd.x;
    const int t = static_cast<int>(k / a.B);
    const TableMeta m = a.meta[t];
    const int gshift = m.fwd_gshift;
    const int Gs = 1 << gshift, R = kWave >> gshift;
    const int g = lane >> gshift, gl = lane & (Gs - 1);
    const int64_t b0 = ld_index<IT>(a.offsets, k), b1 = ld_index<IT>(a.offsets, k + 1);
    const int64_t start = b0 + static_cast<int64_t>(sd.y) * a.split_len;
    const int64_t end = min(b1, start + a.split_len);
    const float scale = a.mean ? 1.0f / static_cast<float>(b1 - b0) : 1.0f;
    const int D = m.dim;
    const int C = VEC ? D / VE : D;
    const void* wbase = static_cast<const char*>(a.weights) + m.woff * SB;
    float* dst_row = a.split_part + static_cast<int64_t>(si) * a.split_pstride;
    for (int cb = 0; cb < C; cb += Gs) {
      const int chunk = cb + gl;
      const bool lane_ok = chunk < C;
      float acc[VE];
#pragma unroll
      for (int e = 0; e < VE; ++e) acc[e] = 0.0f;
      for (int64_t j0 = start; j0 < end; j0 += kWave) {
        const int n = static_cast<int>(min(static_cast<int64_t>(kWave), end - j0));
        int my_row = 0;
        float my_p = 1.0f;
        if (lane < n) {
          my_row = static_cast<int>(ld_index<IT>(a.indices, j0 + lane));
          if constexpr (PSW) my_p = a.psw[j0 + lane];
        }
        for (int r = 0; r < n; r += R * kUnroll) {
          float v[kUnroll][VE];
          float p[kUnroll];
#pragma unroll
          for (int u = 0; u < kUnroll; ++u) {
            const int jj = r + u * R + g;
            const int src = min(jj, kWave - 1);
            const int row = __shfl(my_row, src, kWave);
            p[u] = PSW ? __shfl(my_p, src, kWave) : 1.0f;
            if (jj < n && lane_ok) {
              load_widen<ST, VE>(wbase, static_cast<int64_t>(row) * D + chunk * VE, v[u]);
            } else {
#pragma unroll
              for (int e = 0; e < VE; ++e) v[u][e] = 0.0f;
            }
          }
#pragma unroll
          for (int u = 0; u < kUnroll; ++u)
#pragma unroll
            for (int e = 0; e < VE; ++e) acc[e] = PSW ? fmaf(p[u], v[u][e], acc[e]) : acc[e] + v[u][e];
        }
      }
      for (int o = kWave >> 1; o >= Gs; o >>= 1) {
#pragma unroll
        for (int e = 0; e < VE; ++e) acc[e] += __shfl_xor(acc[e], o, kWave);
      }
      if (g == 0 && lane_ok) {
#pragma unroll
        for (int e = 0; e < VE; ++e) dst_row[chunk * VE + e] = acc[e] * scale;
      }
    }
  }
}

// Adds each split bag's segment sums to its output row.  One workgroup per
// split bag: wave w adds the w-th quarter of the bag's segments in segment
// order, and the quarters are then added to the row in wave order (the result
// does not depend on scheduling).
constexpr int kCombineBatch = 16;
__global__ __launch_bounds__(kBlock) void fwd_split_combine(ForwardLaunch a) {
  __shared__ float s_q[kWavesPerBlock][kMaxDim];
  const uint32_t nlong = a.split_ctr[1];
  const uint32_t wave = threadIdx.x >> 6;
  const int64_t ps = a.split_pstride;
  for (uint32_t li = blockIdx.x; li < nlong; li += gridDim.x) {
    const uint4 L = a.split_long[li];  // {bag, first segment slot, segments, 0}
    const int64_t k = L.x;
    const int t = static_cast<int>(k / a.B);
    const int64_t b = k - static_cast<int64_t>(t) * a.B;
    const TableMeta m = a.meta[t];
    float* orow = a.out + b * a.sum_dims + m.doff;
    const uint32_t per = (L.z + kWavesPerBlock - 1) / kWavesPerBlock;
    const uint32_t j0 = min(L.z, wave * per);
    const uint32_t nj = min(L.z, j0 + per) - j0;
    for (int d = lane_id(); d < m.dim; d += kWave) {
      const float* p = a.split_part + static_cast<int64_t>(L.y + j0) * ps + d;
      float y = 0.0f;
      uint32_t j = 0;
      // kCombineBatch loads in flight, then added in segment order
      for (; j + kCombineBatch <= nj; j += kCombineBatch) {
        float v[kCombineBatch];
#pragma unroll
        for (int u = 0; u < kCombineBatch; ++u) v[u] = p[static_cast<int64_t>(j + u) * ps];
#pragma unroll
        for (int u = 0; u < kCombineBatch; ++u) y += v[u];
      }
      for (; j < nj; ++j) y += p[static_cast<int64_t>(j) * ps];
      s_q[wave][d] = y;
    }
    __syncthreads();
    for (int d = static_cast<int>(threadIdx.x); d < m.dim; d += kBlock) {
      float y = orow[d];
#pragma unroll
      for (int w = 0; w < kWavesPerBlock; ++w) y += s_q[w][d];
      orow[d] = y;
    }
    __syncthreads();  // s_q is reused by the next split bag
  }
}

// The pooled lookup and the linearize step of the backward's grouping in one
// launch (kimbodo.com/?p=28372, "Kimbodo Engineering Perspective": the
// grouping can be done during the forward).  Workgroups of kFusedThreads
// threads: the first lin_blocks linearize (kFusedK lookups in flight per
// thread, at most kFusedLinCap workgroups, each striding over tiles of bags);
// every later workgroup takes kFusedThreads / kBlock consecutive tiles of the
// pooled lookup.  The two kinds share no data, so the linearize workgroups,
// which wait on memory most of the time, run beside the bandwidth-bound
// forward instead of after it.  Used for batches of at most
// kFusedMaxLookups lookups: on larger ones the linearize workgroups fill the
// chip before the forward's start and the two kernels one after the other
// are faster (measured: 512 threads, two lookups in flight per thread, best of
// 256-1024 threads and 1-8 lookups on the workload of 270k lookups).  lin_blocks is a multiple of 8, so the forward
// workgroups keep the XCD-contiguous numbering of the stand-alone kernel.
constexpr int kFusedThreads = 512;
constexpr int kFusedK = 2;
constexpr int64_t kFusedLinCap = 1024;

template <int ST, typename IT, bool VEC, bool PSW, bool BUCKET>
__global__ __launch_bounds__(kFusedThreads) void fwd_linearize(ForwardLaunch f, BackwardLaunch b,
                                                               int lin_blocks) {
  const int bid = static_cast<int>(blockIdx.x);
  if (bid < lin_blocks) {
    if constexpr (BUCKET) {
      if (bid < (b.num_bags + kLinBags - 1) / kLinBags)
        linearize_bucket<IT, kFusedThreads>(b, bid);
    } else {
      linearize_tiles<IT, kFusedThreads, kFusedK>(b, bid, lin_blocks);
    }
    return;
  }
  constexpr int kPer = kFusedThreads / kBlock;
  const int logical =
      xcd_contiguous_block(bid - lin_blocks, static_cast<int>(gridDim.x) - lin_blocks);
  fwd_tile<ST, IT, VEC, PSW>(f, logical * kPer + static_cast<int>(threadIdx.x) / kBlock,
                             (static_cast<int>(threadIdx.x) % kBlock) >> 6);
}

// Sums v[0..3] of each lookup over the Gs lanes of a lane group (Gs >= 4, a
// power of two): two exchange steps leave every lane with one of the four
// partial sums (lookup 2*[gl & Gs/2] + [gl & Gs/4]), a butterfly over the
// remaining lanes completes it.  6 shuffles for Gs = 32 instead of 20.
__device__ __forceinline__ float group_sum4(const float (&v)[4], int gl, int Gs, int* which) {
  const int o1 = Gs >> 1, o2 = Gs >> 2;
  const bool hi1 = gl & o1, hi2 = gl & o2;
  float w0, w1;
  {
    const float s0 = hi1 ? v[0] : v[2], s1 = hi1 ? v[1] : v[3];
    const float r0 = __shfl_xor(s0, o1, kWave), r1 = __shfl_xor(s1, o1, kWave);
    w0 = (hi1 ? v[2] : v[0]) + r0;
    w1 = (hi1 ? v[3] : v[1]) + r1;
  }
  const float send = hi2 ? w0 : w1;
  float x = (hi2 ? w1 : w0) + __shfl_xor(send, o2, kWave);
  for (int o = o2 >> 1; o >= 1; o >>= 1) x += __shfl_xor(x, o, kWave);
  *which = (hi1 ? 2 : 0) + (hi2 ? 1 : 0);
  return x;
}

// Gradient with respect to the per-sample weights: the forward is linear in
// p_i, so dL/dp_i = s_k * <G[b, doff_t : doff_t + D_t], W_t[x_i]>.  Same lane
// layout as the forward: a lane group covers a row in 16-byte chunks, a
// sub-wave serves a bag, and each lane group computes the dot products of
// kUnroll lookups at a time (the bag's gradient chunk is loaded once per
// chunk set and shared by them), folded across the group's lanes.
template <int ST, typename IT, bool VEC>
__global__ __launch_bounds__(kBlock) void psw_grad(ForwardLaunch a, const float* __restrict__ grad,
                                                   float* __restrict__ gpsw) {
  static_assert(kUnroll == 4, "group_sum4 reduces four lookups");
  constexpr int SB = StorageTraits<ST>::bytes;
  constexpr int VE = VEC ? 16 / SB : 1;
  const int logical = xcd_contiguous_block(blockIdx.x, gridDim.x);
  const int t = logical / a.tiles_per_table;
  const int tile = logical - t * a.tiles_per_table;
  const TableMeta m = a.meta[t];
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int gshift = m.fwd_gshift;
  const int swshift = min(6, gshift + a.lshift);
  const int SW = 1 << swshift;
  const int Gs = 1 << gshift;
  const int R = SW >> gshift;
  const int sl = lane & (SW - 1);
  const int g = sl >> gshift;
  const int gl = sl & (Gs - 1);
  const int sub_base = lane & ~(SW - 1);
  const int b = ((tile * kWavesPerBlock + wave) << (6 - swshift)) + (lane >> swshift);
  const bool bag_ok = b < a.B;
  const int64_t k = static_cast<int64_t>(t) * a.B + b;
  int64_t start = 0, end = 0;
  if (bag_ok) {
    start = ld_index<IT>(a.offsets, k);
    end = ld_index<IT>(a.offsets, k + 1);
  }
  const int D = m.dim;
  const int C = VEC ? D / VE : D;
  const void* wbase = static_cast<const char*>(a.weights) + m.woff * SB;
  const float scale = (a.mean && end > start) ? 1.0f / static_cast<float>(end - start) : 1.0f;
  const float* grow = grad + static_cast<int64_t>(b) * a.sum_dims + m.doff;
  for (int64_t j0 = start; j0 < end; j0 += SW) {
    const int n = static_cast<int>(min(static_cast<int64_t>(SW), end - j0));
    int my_row = 0;
    if (sl < n) my_row = static_cast<int>(ld_index<IT>(a.indices, j0 + sl));
    for (int r = 0; r < n; r += R * kUnroll) {
      float dot[kUnroll];
      int rows[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        dot[u] = 0.0f;
        rows[u] = __shfl(my_row, sub_base + min(r + u * R + g, SW - 1), kWave);
      }
      for (int cb = 0; cb < C; cb += Gs) {
        const int chunk = cb + gl;
        const bool lane_ok = chunk < C;
        float gv[VE];
        if (lane_ok) {
          if constexpr (VEC) {  // 16-byte aligned rows of the gradient (checked on the host)
#pragma unroll
            for (int e = 0; e < VE; e += 4) {
              const float4 x = *reinterpret_cast<const float4*>(grow + chunk * VE + e);
              gv[e] = x.x, gv[e + 1] = x.y, gv[e + 2] = x.z, gv[e + 3] = x.w;
            }
          } else {
#pragma unroll
            for (int e = 0; e < VE; ++e) gv[e] = grow[chunk * VE + e];
          }
        } else {
#pragma unroll
          for (int e = 0; e < VE; ++e) gv[e] = 0.0f;
        }
        float w[kUnroll][VE];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
          if (r + u * R + g < n && lane_ok) {
            load_widen<ST, VE>(wbase, static_cast<int64_t>(rows[u]) * D + chunk * VE, w[u]);
          } else {
#pragma unroll
            for (int e = 0; e < VE; ++e) w[u][e] = 0.0f;
          }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
#pragma unroll
          for (int e = 0; e < VE; ++e) dot[u] = fmaf(w[u][e], gv[e], dot[u]);
      }
      if (Gs >= 4) {
        int u;
        const float x = group_sum4(dot, gl, Gs, &u);
        const int jj = r + u * R + g;
        if ((gl & ((Gs >> 2) - 1)) == 0 && jj < n) gpsw[j0 + jj] = x * scale;
      } else {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
          for (int o = Gs >> 1; o >= 1; o >>= 1) dot[u] += __shfl_xor(dot[u], o, kWave);
          const int jj = r + u * R + g;
          if (gl == 0 && jj < n) gpsw[j0 + jj] = dot[u] * scale;
        }
      }
    }
  }
}

template <int ST, typename IT, bool UNC>
void dispatch_vec_psw_unc(const ForwardLaunch& a, hipStream_t s, dim3 grid,
                          const KernelTimer* kt) {
  if (a.vec) {
    if (a.psw)
      launch_timed(kt, "fwd_gather_pool", fwd_gather_pool<ST, IT, true, true, UNC>, grid, dim3(kBlock), 0, s, a);
    else
      launch_timed(kt, "fwd_gather_pool", fwd_gather_pool<ST, IT, true, false, UNC>, grid, dim3(kBlock), 0, s, a);
  } else {
    if (a.psw)
      launch_timed(kt, "fwd_gather_pool", fwd_gather_pool<ST, IT, false, true, UNC>, grid, dim3(kBlock), 0, s, a);
    else
      launch_timed(kt, "fwd_gather_pool", fwd_gather_pool<ST, IT, false, false, UNC>, grid, dim3(kBlock), 0, s, a);
  }
}

template <int ST, typename IT>
hipError_t dispatch_vec_psw(const ForwardLaunch& a, hipStream_t s, dim3 grid,
                            const KernelTimer* kt) {
  if (a.uncond_loads)
    dispatch_vec_psw_unc<ST, IT, true>(a, s, grid, kt);
  else
    dispatch_vec_psw_unc<ST, IT, false>(a, s, grid, kt);
  return hipGetLastError();
}

template <int ST>
hipError_t dispatch_index(const ForwardLaunch& a, hipStream_t s, dim3 grid,
                          const KernelTimer* kt) {
  return a.index64 ? dispatch_vec_psw<ST, int64_t>(a, s, grid, kt)
                   : dispatch_vec_psw<ST, int32_t>(a, s, grid, kt);
}

template <int ST, typename IT, bool SC>
void launch_fused_sc(const ForwardLaunch& f, const BackwardLaunch& b, int lin, hipStream_t s,
                     dim3 grid, const KernelTimer* kt) {
  const dim3 block(kFusedThreads);
  if (f.vec) {
    if (f.psw)
      launch_timed(kt, "fwd_linearize", fwd_linearize<ST, IT, true, true, SC>, grid, block, 0, s, f, b, lin);
    else
      launch_timed(kt, "fwd_linearize", fwd_linearize<ST, IT, true, false, SC>, grid, block, 0, s, f, b, lin);
  } else {
    if (f.psw)
      launch_timed(kt, "fwd_linearize", fwd_linearize<ST, IT, false, true, SC>, grid, block, 0, s, f, b, lin);
    else
      launch_timed(kt, "fwd_linearize", fwd_linearize<ST, IT, false, false, SC>, grid, block, 0, s, f, b, lin);
  }
}

template <int ST, typename IT>
hipError_t launch_fused(const ForwardLaunch& f, const BackwardLaunch& b, int lin, hipStream_t s,
                        dim3 grid, const KernelTimer* kt) {
  if (uses_tile_buckets(b))
    launch_fused_sc<ST, IT, true>(f, b, lin, s, grid, kt);
  else
    launch_fused_sc<ST, IT, false>(f, b, lin, s, grid, kt);
  return hipGetLastError();
}

template <int ST>
hipError_t launch_fused_index(const ForwardLaunch& f, const BackwardLaunch& b, int lin,
                              hipStream_t s, dim3 grid, const KernelTimer* kt) {
  return f.index64 ? launch_fused<ST, int64_t>(f, b, lin, s, grid, kt)
                   : launch_fused<ST, int32_t>(f, b, lin, s, grid, kt);
}

template <int ST, typename IT>
void launch_psw(const ForwardLaunch& a, const float* grad, float* gpsw, hipStream_t s, dim3 grid,
                const KernelTimer* kt) {
  if (a.vec)
    launch_timed(kt, "psw_grad", psw_grad<ST, IT, true>, grid, dim3(kBlock), 0, s, a, grad, gpsw);
  else
    launch_timed(kt, "psw_grad", psw_grad<ST, IT, false>, grid, dim3(kBlock), 0, s, a, grad, gpsw);
}

template <int ST>
void launch_psw_index(const ForwardLaunch& a, const float* grad, float* gpsw, hipStream_t s,
                      dim3 grid, const KernelTimer* kt) {
  if (a.index64)
    launch_psw<ST, int64_t>(a, grad, gpsw, s, grid, kt);
  else
    launch_psw<ST, int32_t>(a, grad, gpsw, s, grid, kt);
}

}  // namespace

hipError_t launch_forward_gather(const ForwardLaunch& a, hipStream_t stream,
                                 const KernelTimer* kt) {
  const int64_t blocks = static_cast<int64_t>(a.T) * a.tiles_per_table;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  const dim3 grid(static_cast<unsigned>(blocks));
  switch (a.dtype) {
    case kF32: return dispatch_index<kF32>(a, stream, grid, kt);
    case kF16: return dispatch_index<kF16>(a, stream, grid, kt);
    case kBF16: return dispatch_index<kBF16>(a, stream, grid, kt);
    default: return hipErrorInvalidValue;
  }
}

template <int ST, typename IT>
void launch_split_segments(const ForwardLaunch& a, hipStream_t s, dim3 grid,
                           const KernelTimer* kt) {
  if (a.vec) {
    if (a.psw)
      launch_timed(kt, "fwd_split_segments", fwd_split_segments<ST, IT, true, true>, grid,
                   dim3(kBlock), 0, s, a);
    else
      launch_timed(kt, "fwd_split_segments", fwd_split_segments<ST, IT, true, false>, grid,
                   dim3(kBlock), 0, s, a);
  } else {
    if (a.psw)
      launch_timed(kt, "fwd_split_segments", fwd_split_segments<ST, IT, false, true>, grid,
                   dim3(kBlock), 0, s, a);
    else
      launch_timed(kt, "fwd_split_segments", fwd_split_segments<ST, IT, false, false>, grid,
                   dim3(kBlock), 0, s, a);
  }
}

template <int ST, typename IT, bool PSW, int GSH>
hipError_t launch_lds_r(const ForwardLaunch& a, int R, dim3 grid, int wgs, hipStream_t s,
                        const KernelTimer* kt) {
  const dim3 block(kLdsFwdThreads);
  switch (R) {
    case 1: launch_timed(kt, "fwd_lds_pool", fwd_lds_pool<ST, IT, PSW, GSH, 1>, grid, block, 0, s, a, wgs); break;
    case 2: launch_timed(kt, "fwd_lds_pool", fwd_lds_pool<ST, IT, PSW, GSH, 2>, grid, block, 0, s, a, wgs); break;
    case 4:
      if constexpr (!(PSW && GSH == 3)) {  // (that one would spill registers)
        launch_timed(kt, "fwd_lds_pool", fwd_lds_pool<ST, IT, PSW, GSH, 4>, grid, block, 0, s, a, wgs);
        break;
      }
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;  // (8 partial sums would spill registers)
  }
  return hipGetLastError();
}

template <int ST, typename IT, bool PSW>
hipError_t launch_lds_g(const ForwardLaunch& a, int gshift, int R, dim3 grid, int wgs,
                        hipStream_t s, const KernelTimer* kt) {
  static_assert(kLdsFwdMinGshift == 2 && kLdsFwdMaxGshift == 3, "instantiated gshifts");
  if (gshift == 2) return launch_lds_r<ST, IT, PSW, 2>(a, R, grid, wgs, s, kt);
  if (gshift == 3) return launch_lds_r<ST, IT, PSW, 3>(a, R, grid, wgs, s, kt);
  return hipErrorInvalidValue;
}

template <int ST>
hipError_t launch_lds_st(const ForwardLaunch& a, int gshift, int R, dim3 grid, int wgs,
                         hipStream_t s, const KernelTimer* kt) {
  if (a.index64)
    return a.psw ? launch_lds_g<ST, int64_t, true>(a, gshift, R, grid, wgs, s, kt)
                 : launch_lds_g<ST, int64_t, false>(a, gshift, R, grid, wgs, s, kt);
  return a.psw ? launch_lds_g<ST, int32_t, true>(a, gshift, R, grid, wgs, s, kt)
               : launch_lds_g<ST, int32_t, false>(a, gshift, R, grid, wgs, s, kt);
}

template <int ST>
void launch_split_index(const ForwardLaunch& a, hipStream_t s, dim3 grid, const KernelTimer* kt) {
  if (a.index64)
    launch_split_segments<ST, int64_t>(a, s, grid, kt);
  else
    launch_split_segments<ST, int32_t>(a, s, grid, kt);
}

hipError_t launch_forward_lds(const ForwardLaunch& a, int gshift, int wgs_per_table,
                              hipStream_t stream, const KernelTimer* kt) {
  const int64_t blocks = static_cast<int64_t>(a.T) * wgs_per_table;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7FFFFFFF || a.split_len > 0) return hipErrorInvalidConfiguration;
  const int R = 1 << std::min(6 - gshift, static_cast<int>(a.lshift));
  const dim3 grid(static_cast<unsigned>(blocks));
  switch (a.dtype) {
    case kF16: return launch_lds_st<kF16>(a, gshift, R, grid, wgs_per_table, stream, kt);
    case kBF16: return launch_lds_st<kBF16>(a, gshift, R, grid, wgs_per_table, stream, kt);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_forward_split(const ForwardLaunch& a, int64_t num_indices, hipStream_t stream,
                                const KernelTimer* kt) {
  // at most num_indices / split_len segments after the first ones, and as
  // many split bags
  const int64_t segs = num_indices / a.split_len + 1;
  int64_t blocks = (segs + kWavesPerBlock - 1) / kWavesPerBlock;
  if (blocks > 4096) blocks = 4096;
  const dim3 grid(static_cast<unsigned>(blocks));
  switch (a.dtype) {
    case kF32: launch_split_index<kF32>(a, stream, grid, kt); break;
    case kF16: launch_split_index<kF16>(a, stream, grid, kt); break;
    case kBF16: launch_split_index<kBF16>(a, stream, grid, kt); break;
    default: return hipErrorInvalidValue;
  }
  // one workgroup per split bag
  const dim3 cgrid(static_cast<unsigned>(segs < 4096 ? segs : 4096));
  launch_timed(kt, "fwd_split_combine", fwd_split_combine, cgrid, dim3(kBlock), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_forward_linearize(const ForwardLaunch& f, const BackwardLaunch& b,
                                    hipStream_t stream, const KernelTimer* kt) {
  if (f.index64 != b.index64) return hipErrorInvalidValue;
  const int64_t tiles = static_cast<int64_t>(f.T) * f.tiles_per_table;
  constexpr int kPer = kFusedThreads / kBlock;
  // linearize workgroups first, rounded up to a multiple of the 8 XCDs
  const int64_t lin = (std::min(linearize_blocks(b.num_bags), kFusedLinCap) + 7) / 8 * 8;
  const int64_t blocks = lin + (tiles + kPer - 1) / kPer;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  const dim3 grid(static_cast<unsigned>(blocks));
  switch (f.dtype) {
    case kF32: return launch_fused_index<kF32>(f, b, static_cast<int>(lin), stream, grid, kt);
    case kF16: return launch_fused_index<kF16>(f, b, static_cast<int>(lin), stream, grid, kt);
    case kBF16: return launch_fused_index<kBF16>(f, b, static_cast<int>(lin), stream, grid, kt);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tbe

namespace tbe {

hipError_t launch_psw_grad(const ForwardLaunch& a, const float* grad, float* gpsw,
                           hipStream_t stream, const KernelTimer* kt) {
  const int64_t blocks = static_cast<int64_t>(a.T) * a.tiles_per_table;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  const dim3 grid(static_cast<unsigned>(blocks));
  switch (a.dtype) {
    case kF32: launch_psw_index<kF32>(a, grad, gpsw, stream, grid, kt); break;
    case kF16: launch_psw_index<kF16>(a, grad, gpsw, stream, grid, kt); break;
    case kBF16: launch_psw_index<kBF16>(a, grad, gpsw, stream, grid, kt); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace tbe
