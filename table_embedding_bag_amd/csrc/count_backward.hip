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
//  * cb_product: a workgroup of 4 waves owns 256 rows (64 per wave: four
//    16-row tiles) x 64 columns (four 16-column tiles) of one table and one
//    slice of its bags, and walks the slice in steps of 32 bags (the K of
//    v_mfma_f32_16x16x32_bf16).  Per step: the 32 bags' gradient columns are
//    staged in LDS transposed ([part][column][bag], so a lane's B operand --
//    eight consecutive bags of one column -- is one 16-byte read), the
//    step's lookups are counted into each wave's [64 rows][32 bags] count
//    tile with packed bf16 LDS atomic adds, each wave reads its A operands,
//    clears its tile and issues 3 x 16 MFMAs.  C never exists in HBM.  The
//    slice's partial Gamma (fp32) and the rows' lookup counts are written to
//    the workspace.  Workgroups are numbered so that the row groups of one
//    bag slice, which stage the same gradient columns, are neighbours on one
//    XCD (the second and later reads come from its L2).
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
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr int kRowsPerWave = 64;
constexpr int kTS = kK + 8;          // LDS row stride (16-bit elements) of the tiles
constexpr int kParts = 3;            // g = hi + mid + lo
constexpr int kCountCap = 256;       // every count 0..256 is exact in bf16
static_assert(kWaves * kRowsPerWave == kCbGroupRows, "row group");

template <typename IT>
__device__ __forceinline__ int64_t ld_index(const void* p, int64_t i) {
  return static_cast<int64_t>(static_cast<const IT*>(p)[i]);
}

__device__ __forceinline__ f32x4 mma(const uint4& a, const uint4& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ float bf16_value(uint32_t bits) { return __uint_as_float(bits << 16); }

// g = hi + mid + lo exactly, each part a bf16 (bit patterns in the low 16 bits).
__device__ __forceinline__ void split3(float g, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
  hi = f32_to_bf16_bits(g);
  const float r1 = g - bf16_value(hi);    // exact: g and hi share an exponent range
  mid = f32_to_bf16_bits(r1);
  lo = f32_to_bf16_bits(r1 - bf16_value(mid));  // exact: at most 8 significant bits remain
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
  __shared__ int64_t s_off[kK + 1];          // the step's bag bounds
  __shared__ uint32_t s_rowcnt[kCbGroupRows];
  __shared__ int s_maxlen;

  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  // logical block -> (unit, bag slice, row group), row group fastest
  const int logical = xcd_contiguous_block(blockIdx.x, gridDim.x);
  const int per_unit = a.slices * kCbGroupsPerTable;
  const int u = logical / per_unit;
  const int rem = logical - u * per_unit;
  const int slice = rem / kCbGroupsPerTable;
  const int rg = rem - slice * kCbGroupsPerTable;
  const CountUnit unit = a.units[u];
  const TableMeta m = a.meta[unit.table];
  const int row0 = rg * kCbGroupRows;
  if (row0 >= m.rows) return;                // the whole workgroup: no rows here
  const int col0 = unit.col0;
  const int NT = min(kCbCols, m.dim - col0) >> 4;  // 16-column tiles (dims are multiples of 16)
  const int wrow0 = row0 + wave * kRowsPerWave;
  const bool active = wrow0 < m.rows;
  // bag slice, whole 32-bag steps except the last
  const int per_slice = ((a.B + a.slices - 1) / a.slices + kK - 1) / kK * kK;
  const int b_begin = min(a.B, slice * per_slice);
  const int b_end = min(a.B, b_begin + per_slice);
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

  const int gcol = tid & 63, gbag = (tid >> 6) * 8;  // G staging: one column, 8 bags
  for (int c0 = b_begin; c0 < b_end; c0 += kK) {
    const int nb = min(kK, b_end - c0);
    __syncthreads();  // the previous step's readers of s_g, s_off and the tiles are done
    // this step's gradient columns (loads in flight across the barrier below)
    float g[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int b = gbag + j;
      g[j] = (b < nb && gcol < NT * 16) ? gbase[static_cast<int64_t>(c0 + b) * a.sum_dims + gcol]
                                        : 0.0f;
    }
    if (tid <= kK) s_off[tid] = ld_index<IT>(a.offsets, kbase + c0 + min(tid, nb));
    if (tid == 0) s_maxlen = 0;
    __syncthreads();
    if (tid < nb) atomicMax(&s_maxlen, static_cast<int>(s_off[tid + 1] - s_off[tid]));
    {
      uint32_t hi[8], mid[8], lo[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float v = g[j];
        if constexpr (MEAN) {
          const int b = gbag + j;
          const int64_t len = b < nb ? s_off[b + 1] - s_off[b] : 0;
          v = len > 0 ? v * (1.0f / static_cast<float>(len)) : 0.0f;
        }
        split3(v, hi[j], mid[j], lo[j]);
      }
      uint4* dst0 = reinterpret_cast<uint4*>(s_g[0] + gcol * kTS + gbag);
      uint4* dst1 = reinterpret_cast<uint4*>(s_g[1] + gcol * kTS + gbag);
      uint4* dst2 = reinterpret_cast<uint4*>(s_g[2] + gcol * kTS + gbag);
      *dst0 = make_uint4(hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16), hi[4] | (hi[5] << 16),
                         hi[6] | (hi[7] << 16));
      *dst1 = make_uint4(mid[0] | (mid[1] << 16), mid[2] | (mid[3] << 16),
                         mid[4] | (mid[5] << 16), mid[6] | (mid[7] << 16));
      *dst2 = make_uint4(lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16), lo[4] | (lo[5] << 16),
                         lo[6] | (lo[7] << 16));
    }
    __syncthreads();  // s_maxlen
    const int64_t p0 = s_off[0], p1 = s_off[nb];
    const int passes = max(1, (s_maxlen + kCountCap - 1) / kCountCap);
    for (int pass = 0; pass < passes; ++pass) {
      if (pass > 0) __syncthreads();  // the previous pass's tiles were read and cleared
      // this pass's lookups of the step (positions [pass*256, pass*256 + 256) of each bag)
      for (int64_t p = p0 + tid; p < p1; p += kThreads) {
        const int64_t x = ld_index<IT>(a.indices, p);
        int lo = 0, hi = nb;  // the bag: s_off[lo] <= p < s_off[hi]
        while (hi - lo > 1) {
          const int mid = (lo + hi) >> 1;
          if (s_off[mid] <= p) lo = mid; else hi = mid;
        }
        if ((p - s_off[lo]) / kCountCap != pass) continue;
        const int64_t r = x - row0;
        if (r >= 0 && r < kCbGroupRows) {
          count_add(s_cnt[r >> 6], static_cast<int>(r & 63) * kTS + lo);
          atomicAdd(&s_rowcnt[r], 1u);
        }
      }
      __syncthreads();
      if (active) {
        uint4 af[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
          af[mt] = *reinterpret_cast<const uint4*>(s_cnt[wave] + (mt * 16 + (lane & 15)) * kTS +
                                                   (lane >> 4) * 8);
        // clear the tile for the next step (a wave's LDS operations complete in order)
        uint4* t4 = reinterpret_cast<uint4*>(s_cnt[wave]);
#pragma unroll
        for (int i = 0; i < kRowsPerWave * kTS / 8 / kWave; ++i)
          t4[i * kWave + lane] = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
        for (int part = 0; part < kParts; ++part) {
#pragma unroll
          for (int nt = 0; nt < 4; ++nt) {
            if (nt < NT) {
              const uint4 bf = *reinterpret_cast<const uint4*>(
                  s_g[part] + (nt * 16 + (lane & 15)) * kTS + (lane >> 4) * 8);
#pragma unroll
              for (int mt = 0; mt < 4; ++mt) acc[mt][nt] = mma(af[mt], bf, acc[mt][nt]);
            }
          }
        }
      }
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
  if (col0 == 0 && row0 + tid < m.rows)
    a.counts[static_cast<int64_t>(a.slices) * m.roff + static_cast<int64_t>(slice) * m.rows +
             row0 + tid] = s_rowcnt[tid];
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
  for (int s = 0; s < a.slices; ++s) c += cp[static_cast<int64_t>(s) * m.rows];
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
        double x[4] = {0.0, 0.0, 0.0, 0.0};
        for (int s = 0; s < a.slices; ++s) {
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
  const int64_t blocks = static_cast<int64_t>(a.nunits) * a.slices * kCbGroupsPerTable;
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
