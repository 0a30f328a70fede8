// count_backward.hip -- count-matrix backward of small tables on gfx950.
//
// kimbodo.com/?p=28372, "What Happened": small tables that qualify go through
// a histogram and the matrix cores in the forward (Y_t = C_t W_t, C_t the
// bag-by-row count matrix).  The same matrix gives the backward's summed row
// gradients of such a table in one dense product,
//     Gamma_t = C_t^T G_t,   C_t[b, r] = #{i in bag (t, b) : x_i = r},
// with G_t the table's columns of the upstream gradient (each bag's row
// scaled by 1/L_k for mean pooling).  Every touched row then gets its one
// optimizer update ("each row receives one optimizer update", same section),
// without the grouping's sort: for tables of at most 1024 rows the counts
// stand in for the transpose, sort and run-length encoding.  This is an
// extension by symmetry; the pages show the count-matrix path for the forward
// only.
//
// Precision: G is fp32 and the matrix cores take bf16, so every G value is
// split exactly into three bf16 parts, g = hi + mid + lo (hi = bf16(g),
// mid = bf16(g - hi), lo = g - hi - mid, each exact), and the product is
// accumulated as C^T hi + C^T mid + C^T lo.  Counts up to 256 are exact in
// bf16 (a bag longer than 256 lookups is counted in passes of 256 positions),
// so every product count * part is exact in fp32 and the sums are fp32 in a
// fixed order: the accuracy of an fp32 segment sum, reproducible bit for bit.
//
// Mapping onto CDNA4:
//  * cb_product: a workgroup of 16 waves owns all rows of one table (up to
//    1024; 64 per wave: four 16-row tiles) x 64 columns (four 16-column
//    tiles) and one slice of its bags, and walks the slice in steps of 32
//    bags (the K of v_mfma_f32_16x16x32_bf16).  Per step: the 32 bags'
//    gradient columns are split and staged in LDS transposed
//    ([part][column][bag], so a lane's B operand -- eight consecutive bags of
//    one column -- is one 16-byte read; each thread splits two values), the
//    step's lookups are counted into each wave's [64 rows][32 bags] count
//    tile, each wave with rows reads its A operands, clears its tile and
//    issues 3 x 16 MFMAs.  The next step's gradient values and ids (and the
//    offsets of the one after) are loaded into registers before the current
//    step's barrier and products, so global latency overlaps them (two
//    barriers per step).  C never exists in HBM.  The slice's partial Gamma
//    (fp32) and the rows' lookup counts are written to the workspace.  One
//    workgroup per table (rather than one per 256 rows) splits and counts
//    each step once for the whole table, and over 1024 threads: that per-step
//    work, not the matrix cores, sets the time.
//  * cb_update: one 16-lane group per table row; rows with no lookup are
//    skipped (their weights and state stay bit-identical); the slices'
//    partials are added in slice order in fp64, then the SGD or row-wise
//    Adagrad step is applied.
//  * cb_runs (only when the caller asks for the runs): the touched rows in
//    ascending order with their lookup counts, and U.
#include "count_backward.hpp"

namespace tbe {
namespace {

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

constexpr int kK = 32;               // bags per MFMA step
constexpr int kWaves = 16;
constexpr int kThreads = kWaves * kWave;
constexpr int kRowsPerWave = 64;
constexpr int kTS = kK + 8;          // LDS row stride (16-bit elements) of the tiles
constexpr int kParts = 3;            // g = hi + mid + lo
constexpr int kCountCap = 256;       // every count 0..256 is exact in bf16
constexpr int kGB = kK * kCbCols / kThreads;  // bags of one column a thread stages per step
enum { kFast = 0, kAtomic = 1, kPasses = 2 };  // counting modes of a step
// DPP lane selects (gfx9 encoding): quad permutations lane ^ 1, ^ 2, ^ 3 within
// each group of 4 lanes, and the half-row mirror lane ^ 7 within each group of 8
constexpr int kDppQuadXor1 = 0xB1;   // quad_perm [1, 0, 3, 2]
constexpr int kDppQuadXor2 = 0x4E;   // quad_perm [2, 3, 0, 1]
constexpr int kDppQuadXor3 = 0x1B;   // quad_perm [3, 2, 1, 0]
constexpr int kDppHalfMirror = 0x141;
static_assert(kWaves * kRowsPerWave == kCbGroupRows && kCbGroupRows == kCbMaxRows,
              "one workgroup holds every row of a table");

template <typename IT>
__device__ __forceinline__ int64_t ld_index(const void* p, int64_t i) {
  return static_cast<int64_t>(static_cast<const IT*>(p)[i]);
}

__device__ __forceinline__ f32x4 mma(const uint4& a, const uint4& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Two values rounded to a packed bf16 pair (first in the low half):
// v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t cvt_pair(float x, float y) {
  return __builtin_bit_cast(uint32_t, bf16x2{static_cast<__bf16>(x), static_cast<__bf16>(y)});
}

// Two values split into packed bf16 parts with g = hi + mid + lo exactly: hi
// rounds g; g - hi is exact in fp32 and fits 17 significant bits; mid rounds
// that, and the rest (at most 8 significant bits) is exactly a bf16.
__device__ __forceinline__ void split_pair(float g0, float g1, uint32_t& hi, uint32_t& mid,
                                           uint32_t& lo) {
  hi = cvt_pair(g0, g1);
  const float r0 = g0 - __uint_as_float(hi << 16);
  const float r1 = g1 - __uint_as_float(hi & 0xFFFF0000u);
  mid = cvt_pair(r0, r1);
  lo = cvt_pair(r0 - __uint_as_float(mid << 16), r1 - __uint_as_float(mid & 0xFFFF0000u));
}

// +1 to the bf16 count at element el of a tile (packed 16-bit LDS atomic).
__device__ __forceinline__ void count_add(uint16_t* tile, int el) {
  const bf16x2 one = (el & 1) ? bf16x2{static_cast<__bf16>(0.0f), static_cast<__bf16>(1.0f)}
                              : bf16x2{static_cast<__bf16>(1.0f), static_cast<__bf16>(0.0f)};
  __builtin_amdgcn_ds_atomic_fadd_v2bf16(
      (__attribute__((address_space(3))) bf16x2*)(reinterpret_cast<uint32_t*>(tile) + (el >> 1)),
      one);
}

template <typename IT, bool MEAN>
__global__ __launch_bounds__(kThreads) void cb_product(CountLaunch a) {
  __shared__ __align__(16) uint16_t s_cnt[kWaves][kRowsPerWave * kTS];  // count tiles
  __shared__ __align__(16) uint16_t s_g[kParts][kCbCols * kTS];         // G parts, transposed
  __shared__ int64_t s_off[2][kK + 1];       // bag bounds of two steps
  __shared__ int s_mode[2];                  // counting mode of the step (kFast, kAtomic, kPasses)
  __shared__ uint32_t s_rowcnt[kCbGroupRows];

  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  // logical block -> (unit, bag slice), slice fastest; the workgroup holds
  // every row of the table.  Logical blocks are contiguous per XCD, so one
  // XCD takes the units of a band of adjacent tables, whose gradient columns
  // are neighbours in every row of G (3.5% faster than plain numbering on 64
  // tables of up to 1024 rows).
  const int logical = xcd_contiguous_block(blockIdx.x, gridDim.x);
  const int u = logical / a.slices;
  const int slice = logical - u * a.slices;
  const CountUnit unit = a.units[u];
  const TableMeta m = a.meta[unit.table];
  const int col0 = unit.col0;
  const int NT = min(kCbCols, m.dim - col0) >> 4;  // 16-column tiles (dims are multiples of 16)
  const int wrow0 = wave * kRowsPerWave;
  const bool active = wrow0 < m.rows;
  // bag slice, whole 32-bag steps except the last
  const int per_slice = ((a.B + a.slices - 1) / a.slices + kK - 1) / kK * kK;
  const int b_begin = min(a.B, slice * per_slice);
  const int b_end = min(a.B, b_begin + per_slice);
  const int nsteps = (b_end - b_begin + kK - 1) / kK;
  const int64_t kbase = static_cast<int64_t>(unit.table) * a.B;
  const float* gbase = a.grad + m.doff + col0;

  for (int i = tid; i < kWaves * kRowsPerWave * kTS / 8; i += kThreads)
    reinterpret_cast<uint4*>(&s_cnt[0][0])[i] = make_uint4(0u, 0u, 0u, 0u);
  s_rowcnt[tid] = 0u;
  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  // thread roles: G staging takes one column of kGB consecutive bags; the ids
  // are taken bag by bag, 8 adjacent lanes per bag (bag tid / 8, in-bag
  // positions tid % 8 + 8k), so only the first 256 threads hold ids
  const int gcol = tid & 63, gbag = (tid >> 6) * kGB;
  const int ibag = tid >> 3, ij = tid & 7;
  const bool want_counts = a.out_num != nullptr;  // exact counts per row only for the runs
  auto step_bags = [&](int step) { return min(kK, b_end - (b_begin + step * kK)); };
  // The prefetch loads below are issued unconditionally, from clamped (always
  // valid) addresses, and zeroed or marked when out of range: their number
  // is then fixed, so a wait for the oldest leaves the younger ones in flight.
  auto load_offsets = [&](int step) -> int64_t {
    const int st = min(step, nsteps - 1);
    const int nb = step_bags(st);
    const int b = tid <= kK ? min(tid, nb) : 0;
    return ld_index<IT>(a.offsets, kbase + b_begin + st * kK + b);
  };
  auto store_offsets = [&](int buf, int step, int64_t v) {
    if (tid <= kK) s_off[buf][tid] = v;
    if (wave == 0) {  // threads 0..32 are lanes of wave 0
      const int64_t next = __shfl_down(v, 1, kWave);
      const int64_t len = lane < step_bags(step) ? next - v : 0;
      const bool over8 = __ballot(len > 8) != 0u, over_cap = __ballot(len > kCountCap) != 0u;
      if (lane == 0) s_mode[buf] = over_cap ? kPasses : (over8 ? kAtomic : kFast);
    }
  };
  auto load_g = [&](int step, float (&g)[kGB]) {
    const int st = min(step, nsteps - 1);
    const int nb = step_bags(st), c0 = b_begin + st * kK;
    const bool col_ok = gcol < NT * 16 && step < nsteps;
#pragma unroll
    for (int j = 0; j < kGB; ++j) {
      const int b = gbag + j;
      const bool ok = col_ok && b < nb;
      const float v = gbase[static_cast<int64_t>(c0 + min(b, nb - 1)) * a.sum_dims +
                            (col_ok ? gcol : 0)];
      g[j] = ok ? v : 0.0f;
    }
  };
  auto load_ids = [&](int buf, int step, int64_t (&x)[2]) {
    const bool in_step = step < nsteps && ibag < step_bags(min(step, nsteps - 1));
    const int cb = min(ibag, kK - 1);  // threads past the step's bags hold no ids
    const int64_t s0 = s_off[buf][cb], s1 = s_off[buf][cb + 1];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int64_t p = s0 + ij + 8 * r;
      const bool ok = in_step && p < s1;
      const int64_t v = ld_index<IT>(a.indices, ok ? p : 0);  // position 0 exists (n > 0)
      x[r] = ok ? v : -1;
    }
  };
  auto add = [&](int64_t x, int bag) {
    const int64_t r = x;
    if (r >= 0 && r < kCbGroupRows) {
      count_add(s_cnt[r >> 6], static_cast<int>(r & 63) * kTS + bag);
      if (want_counts) atomicAdd(&s_rowcnt[r], 1u); else s_rowcnt[r] = 1u;
    }
  };
  // one wave's products of a counted step; the wave's tile is cleared again.
  // All four column tiles are multiplied whatever the dim (columns past it
  // hold zeros and are not written), so the products need no branch; a
  // part's four B operands are read before its sixteen MFMAs.
  auto multiply = [&]() {
    if (!active) return;
    uint4 af[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
      af[mt] = *reinterpret_cast<const uint4*>(s_cnt[wave] + (mt * 16 + (lane & 15)) * kTS +
                                               (lane >> 4) * 8);
    uint4 bf[2][4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
      bf[0][nt] = *reinterpret_cast<const uint4*>(s_g[0] + (nt * 16 + (lane & 15)) * kTS +
                                                  (lane >> 4) * 8);
    uint4* t4 = reinterpret_cast<uint4*>(s_cnt[wave]);  // a wave's LDS operations complete in order
#pragma unroll
    for (int i = 0; i < kRowsPerWave * kTS / 8 / kWave; ++i)
      t4[i * kWave + lane] = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int part = 0; part < kParts; ++part) {
      if (part + 1 < kParts) {
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
          bf[(part + 1) & 1][nt] = *reinterpret_cast<const uint4*>(
              s_g[part + 1] + (nt * 16 + (lane & 15)) * kTS + (lane >> 4) * 8);
      }
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) acc[mt][nt] = mma(af[mt], bf[part & 1][nt], acc[mt][nt]);
    }
  };

  if (nsteps > 0) {
    // prologue: offsets of steps 0 and 1 stored, of step 2 in a register; G
    // values and ids of step 0 in registers
    store_offsets(0, 0, load_offsets(0));
    int64_t off_a = load_offsets(1);   // offsets of step c + 2 at iteration c
    __syncthreads();
    float g_cur[kGB];
    int64_t x_cur[2];
    load_g(0, g_cur);
    load_ids(0, 0, x_cur);
    store_offsets(1, 1, off_a);
    off_a = load_offsets(2);

    for (int c = 0; c < nsteps; ++c) {
      const int buf = c & 1, nb = step_bags(c);
      // the previous step's products are done (tiles cleared, s_g free) and the
      // offsets of step c + 1 are visible
      __syncthreads();
      {
        if constexpr (MEAN) {
#pragma unroll
          for (int j = 0; j < kGB; ++j) {
            const int b = gbag + j;
            const int64_t len = b < nb ? s_off[buf][b + 1] - s_off[buf][b] : 0;
            g_cur[j] = len > 0 ? g_cur[j] * (1.0f / static_cast<float>(len)) : 0.0f;
          }
        }
        static_assert(kGB == 2, "one packed pair per part and thread");
        uint32_t hi, mid, lo;
        split_pair(g_cur[0], g_cur[1], hi, mid, lo);
        *reinterpret_cast<uint32_t*>(s_g[0] + gcol * kTS + gbag) = hi;
        *reinterpret_cast<uint32_t*>(s_g[1] + gcol * kTS + gbag) = mid;
        *reinterpret_cast<uint32_t*>(s_g[2] + gcol * kTS + gbag) = lo;
      }
      // count a pass of the step.  kFast (no bag over 8 lookups): the 8 lanes
      // of a bag compare their ids by shuffles and the first lane holding an
      // id stores its count with a plain LDS write (each (row, bag) cell has
      // one writer).  kAtomic (no bag over kCountCap): every lookup adds 1
      // with an LDS atomic.  kPasses: the same over in-bag positions
      // [q * kCountCap, (q + 1) * kCountCap), so no count exceeds what bf16
      // holds exactly.
      const int mode = s_mode[buf];
      const bool long_step = mode == kPasses;
      auto count_pass = [&](int q) -> bool {
        bool added = false;
        if (mode == kFast) {  // the same on every lane of the wave
          const int x = static_cast<int>(x_cur[0]);  // a row (< kCbMaxRows), or -1
          // the ids of the 7 other lanes of the bag's 8-lane group, lane ij ^ o at
          // y[o - 1], by DPP moves (no LDS round trips): the quad permutations give
          // o = 1, 2, 3; the half-row mirror gives o = 7, and the quad permutations
          // of the mirrored ids give o = 6, 5, 4
          const int m7 = __builtin_amdgcn_mov_dpp(x, kDppHalfMirror, 0xF, 0xF, false);
          const int y[7] = {__builtin_amdgcn_mov_dpp(x, kDppQuadXor1, 0xF, 0xF, false),
                            __builtin_amdgcn_mov_dpp(x, kDppQuadXor2, 0xF, 0xF, false),
                            __builtin_amdgcn_mov_dpp(x, kDppQuadXor3, 0xF, 0xF, false),
                            __builtin_amdgcn_mov_dpp(m7, kDppQuadXor3, 0xF, 0xF, false),
                            __builtin_amdgcn_mov_dpp(m7, kDppQuadXor2, 0xF, 0xF, false),
                            __builtin_amdgcn_mov_dpp(m7, kDppQuadXor1, 0xF, 0xF, false),
                            m7};
          int same = 0;
          bool first = true;
#pragma unroll
          for (int o = 1; o < 8; ++o) {
            same += y[o - 1] == x ? 1 : 0;
            first &= !(y[o - 1] == x && (ij ^ o) < ij);
          }
          const int r = x;
          if (x >= 0 && first && r >= 0 && r < kCbGroupRows) {
            s_cnt[r >> 6][(r & 63) * kTS + ibag] =
                static_cast<uint16_t>(__float_as_uint(static_cast<float>(same + 1)) >> 16);
            if (want_counts) atomicAdd(&s_rowcnt[r], static_cast<uint32_t>(same + 1));
            else s_rowcnt[r] = 1u;
          }
          return true;
        }
        if (ibag >= nb) return false;
        const int64_t s0 = s_off[buf][ibag], s1 = s_off[buf][ibag + 1];
        if (!long_step) {
#pragma unroll
          for (int r = 0; r < 2; ++r)
            if (x_cur[r] >= 0) add(x_cur[r], ibag);
          for (int64_t p = s0 + ij + 16; p < s1; p += 8) add(ld_index<IT>(a.indices, p), ibag);
          return true;
        }
        const int64_t lo = s0 + static_cast<int64_t>(q) * kCountCap;
        const int64_t hi = min(s1, lo + kCountCap);
        for (int64_t p = lo + ij; p < hi; p += 8) {
          add(ld_index<IT>(a.indices, p), ibag);
          added = true;
        }
        return added;
      };
      bool added = count_pass(0);
      // prefetch: G values and ids of step c + 1, offsets of step c + 3
      float g_nxt[kGB];
      int64_t x_nxt[2];
      load_g(c + 1, g_nxt);
      load_ids(buf ^ 1, c + 1, x_nxt);
      const int64_t off_b = load_offsets(c + 3);
      for (int q = 0;; ++q) {
        if (long_step) {
          if (!__syncthreads_or(added)) break;
        } else {
          __syncthreads();
        }
        multiply();
        if (!long_step) break;
        __syncthreads();  // every tile cleared before the next pass counts
        added = count_pass(q + 1);
      }
      // the offsets of step c are read no more: the buffer takes step c + 2's
      // (loaded one iteration ago)
      if (c + 2 < nsteps) store_offsets(buf, c + 2, off_a);
      off_a = off_b;
#pragma unroll
      for (int j = 0; j < kGB; ++j) g_cur[j] = g_nxt[j];
      x_cur[0] = x_nxt[0];
      x_cur[1] = x_nxt[1];
    }
  }

  // the slice's partial sums: lane holds rows 4*(lane/16) + i of each 16-row
  // tile, column lane % 16 of each 16-column tile
  float* pt = a.partial + static_cast<int64_t>(a.slices) * m.woff +
              static_cast<int64_t>(slice) * m.rows * m.dim + col0 + (lane & 15);
  if (active) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = wrow0 + mt * 16 + (lane >> 4) * 4 + i;
        if (row < m.rows) {
#pragma unroll
          for (int nt = 0; nt < 4; ++nt)
            if (nt < NT) pt[static_cast<int64_t>(row) * m.dim + nt * 16] = acc[mt][nt][i];
        }
      }
  }
  __syncthreads();  // s_rowcnt
  if (col0 == 0 && tid < m.rows)
    a.counts[static_cast<int64_t>(a.slices) * m.roff + static_cast<int64_t>(slice) * m.rows +
             tid] = s_rowcnt[tid];
}

// Table of linear row id r: the last t with roff_t <= r.
__device__ __forceinline__ int table_of_row(const CountLaunch& a, int64_t r) {
  int lo = 0, hi = a.T;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a.meta[mid].roff <= r) lo = mid; else hi = mid;
  }
  return lo;
}

__device__ __forceinline__ uint32_t row_count(const CountLaunch& a, const TableMeta& m,
                                              int64_t rr) {
  uint32_t c = 0;
  const uint32_t* cp = a.counts + static_cast<int64_t>(a.slices) * m.roff + rr;
  int s = 0;
  for (; s + 8 <= a.slices; s += 8) {  // eight loads in flight
    uint32_t v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = cp[static_cast<int64_t>(s + k) * m.rows];
#pragma unroll
    for (int k = 0; k < 8; ++k) c += v[k];
  }
  for (; s < a.slices; ++s) c += cp[static_cast<int64_t>(s) * m.rows];
  return c;
}

// One 16-lane group per row (4 columns per lane per 64-column step).
template <int ST>
__global__ __launch_bounds__(kBlock) void cb_update(CountLaunch a) {
  constexpr int kG = 16;
  constexpr int kSteps = kCbMaxDim / (kG * 4);
  const int gl = threadIdx.x & (kG - 1);
  const int64_t group = (static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x) / kG;
  const int64_t ngroups = static_cast<int64_t>(gridDim.x) * kBlock / kG;
  for (int64_t r = group; r < a.sum_rows; r += ngroups) {
    const int t = table_of_row(a, r);
    const TableMeta m = a.meta[t];
    const int64_t rr = r - m.roff;
    if (row_count(a, m, rr) == 0u) continue;  // untouched: weights and state unchanged
    const float m_old = a.adagrad ? a.state[r] : 0.0f;
    const float* p = a.partial + static_cast<int64_t>(a.slices) * m.woff + rr * m.dim;
    const int64_t sstride = static_cast<int64_t>(m.rows) * m.dim;
    const int64_t row_e = m.woff + rr * m.dim;
    float gam[kSteps][4], w[kSteps][4];
    double ss = 0.0;
#pragma unroll
    for (int j = 0; j < kSteps; ++j) {
      const int d = j * kG * 4 + gl * 4;
      if (d < m.dim) {
        load_widen<ST, 4>(a.weights, row_e + d, w[j]);
        // slice order; eight slices' loads in flight at a time
        double x[4] = {0.0, 0.0, 0.0, 0.0};
        int s = 0;
        for (; s + 8 <= a.slices; s += 8) {
          float4 v[8];
#pragma unroll
          for (int k = 0; k < 8; ++k)
            v[k] = *reinterpret_cast<const float4*>(p + (s + k) * sstride + d);
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            x[0] += v[k].x; x[1] += v[k].y; x[2] += v[k].z; x[3] += v[k].w;
          }
        }
        for (; s < a.slices; ++s) {
          const float4 v = *reinterpret_cast<const float4*>(p + s * sstride + d);
          x[0] += v.x; x[1] += v.y; x[2] += v.z; x[3] += v.w;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          gam[j][q] = static_cast<float>(x[q]);
          ss = fma(x[q], x[q], ss);
        }
      }
    }
    float step = a.lr;
    if (a.adagrad) {
#pragma unroll
      for (int o = kG / 2; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, kWave);
      const float mnew = static_cast<float>(static_cast<double>(m_old) + ss / m.dim);
      if (gl == 0) a.state[r] = mnew;
      step = a.lr / (sqrtf(mnew) + a.eps);
    }
#pragma unroll
    for (int j = 0; j < kSteps; ++j) {
      const int d = j * kG * 4 + gl * 4;
      if (d < m.dim) {
#pragma unroll
        for (int q = 0; q < 4; ++q) w[j][q] = fmaf(-step, gam[j][q], w[j][q]);
        narrow_store<ST, 4>(a.weights, row_e + d, w[j]);
      }
    }
  }
}

// The runs: touched rows ascending with their counts, and U.  One workgroup
// walks all rows in blocks of 1024 (a block scan per block).
__global__ __launch_bounds__(1024) void cb_runs(CountLaunch a) {
  __shared__ uint32_t s_scr[16];
  __shared__ uint32_t s_base;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  if (tid == 0) s_base = 0u;
  __syncthreads();
  for (int64_t r0 = 0; r0 < a.sum_rows; r0 += 1024) {
    const int64_t r = r0 + tid;
    uint32_t c = 0;
    if (r < a.sum_rows) {
      const TableMeta m = a.meta[table_of_row(a, r)];
      c = row_count(a, m, r - m.roff);
    }
    const uint32_t flag = c > 0u ? 1u : 0u;
    const uint32_t incl = wave_inclusive_sum(flag);
    if (lane == kWave - 1) s_scr[wave] = incl;
    __syncthreads();
    uint32_t before = s_base, total = 0;
    for (int w = 0; w < 16; ++w) {
      before += w < wave ? s_scr[w] : 0u;
      total += s_scr[w];
    }
    if (flag) {
      const uint32_t pos = before + incl - 1u;
      a.out_unique[pos] = static_cast<int32_t>(r);
      a.out_lengths[pos] = static_cast<int32_t>(c);
    }
    __syncthreads();
    if (tid == 0) s_base += total;
    __syncthreads();
  }
  if (tid == 0) *a.out_num = static_cast<int32_t>(s_base);
}

template <typename IT>
void launch_product(const CountLaunch& a, dim3 grid, hipStream_t s, const KernelTimer* kt) {
  if (a.mean)
    launch_timed(kt, "cb_product", cb_product<IT, true>, grid, dim3(kThreads), 0, s, a);
  else
    launch_timed(kt, "cb_product", cb_product<IT, false>, grid, dim3(kThreads), 0, s, a);
}

}  // namespace

hipError_t launch_count_backward(const CountLaunch& a, hipStream_t stream, const KernelTimer* kt) {
  if (a.B <= 0 || a.nunits <= 0) return hipSuccess;
  const int64_t blocks = static_cast<int64_t>(a.nunits) * a.slices;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  if (a.index64)
    launch_product<int64_t>(a, dim3(static_cast<unsigned>(blocks)), stream, kt);
  else
    launch_product<int32_t>(a, dim3(static_cast<unsigned>(blocks)), stream, kt);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  int64_t ub = (a.sum_rows * 16 + kBlock - 1) / kBlock;
  const unsigned ublocks = static_cast<unsigned>(ub < 1 ? 1 : (ub > 4096 ? 4096 : ub));
  switch (a.dtype) {
    case kF32: launch_timed(kt, "cb_update", cb_update<kF32>, dim3(ublocks), dim3(kBlock), 0, stream, a); break;
    case kF16: launch_timed(kt, "cb_update", cb_update<kF16>, dim3(ublocks), dim3(kBlock), 0, stream, a); break;
    case kBF16: launch_timed(kt, "cb_update", cb_update<kBF16>, dim3(ublocks), dim3(kBlock), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  e = hipGetLastError();
  if (e != hipSuccess || !a.out_num) return e;
  launch_timed(kt, "cb_runs", cb_runs, dim3(1), dim3(1024), 0, stream, a);
  return hipGetLastError();
}

}  // namespace tbe
