// histogram.hip -- count-matrix forward of small 16-bit tables on gfx950.
//
// kimbodo.com/?p=28372, "What Happened": next to the generic gather path
// (which also takes per-sample weights), small tables that qualify are pooled
// through a histogram and the matrix cores.  For such a table t the pooled
// output of all bags is one dense product
//     Y_t = diag(s) * C_t * W_t,   C_t[b, r] = #{i in bag (t, b) : x_i = r},
// with s_k = 1 (sum) or 1/L_k (mean).  It equals the gather result exactly up
// to fp32 rounding order: counts are small integers and the stored rows are
// fp16/bf16, so every product C*W is exact in fp32.
//
// Eligible: fp16 or bf16 storage, E_t <= 1024, D_t <= 256 with D_t a multiple
// of 16, no per-sample weights.  A bag longer than 256 lookups (bf16; 2048 for
// fp16) could hold a count the 16-bit operand does not represent exactly; such
// bags are left out of C and pooled by a plain gather loop in the same
// workgroup.  Because C is dense, a NaN or infinity anywhere in W_t reaches
// every bag of table t (0 * inf); the gather path does not have this property.
//
// Mapping onto CDNA4:
//  * hist_transpose writes W_t^T[d][e] (zero for e >= E_t, up to a multiple of
//    64 rows) to a handle-owned buffer, so that the MFMA's B operand -- eight
//    consecutive K (= table row) values per lane -- is one 16-byte read.
//  * fwd_histogram: a workgroup owns 256 bags x 64 output columns of one table
//    (a wave owns 64 bags x 64 columns: 16 accumulators of
//    v_mfma_f32_16x16x32_{bf16,f16}).  C never exists in HBM: the K range is
//    walked in chunks of 64 table rows, and for each chunk the count tile
//    [256 bags][64 rows] is built in LDS with packed 16-bit LDS atomic adds
//    (+1 per lookup; the lookups of the workgroup are bucketed by chunk once),
//    multiplied, then cleared again with -1 adds for the same lookups.
//  * Chunks that no lookup of the workgroup touches are skipped (their
//    product is zero).
//  * Workgroups are renumbered so that every XCD works on a contiguous range
//    of tables (each table's W^T stays in one XCD's L2).
#include "common.hpp"

namespace tbe {
namespace {

constexpr int kHB = 256;              // bags per workgroup (64 per wave)
constexpr int kDB = 64;               // output columns per workgroup
constexpr int kCS = kHistKc + 8;      // LDS row stride in 16-bit elements (bank spread)
constexpr int kRegIds = 8;            // row ids of a bag held in registers (bags of at most 8)
constexpr int kEntCap = 512;          // listed lookups per wave and batch
constexpr int kListSteps = kEntCap / kWave;
constexpr float kNoBag = -1.0f, kLongBag = -2.0f;
constexpr int kMaxChunks = kHistMaxRows / kHistKc;

typedef __attribute__((ext_vector_type(4))) float f32x4;

template <int ST>
struct Mma;

template <>
struct Mma<kBF16> {
  typedef __attribute__((ext_vector_type(8))) __bf16 v8;
  typedef __attribute__((ext_vector_type(2))) __bf16 v2;
  static constexpr int kCountCap = 256;  // largest integer n with all of 0..n exact
  static __device__ __forceinline__ f32x4 mma(const uint4& a, const uint4& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8, a),
                                                   __builtin_bit_cast(v8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ void lds_add(uint32_t* word, bool high, float v) {
    const v2 x = high ? v2{static_cast<__bf16>(0.0f), static_cast<__bf16>(v)}
                      : v2{static_cast<__bf16>(v), static_cast<__bf16>(0.0f)};
    __builtin_amdgcn_ds_atomic_fadd_v2bf16(
        (__attribute__((address_space(3))) v2*)(word), x);
  }
};

template <>
struct Mma<kF16> {
  typedef __attribute__((ext_vector_type(8))) _Float16 v8;
  typedef __attribute__((ext_vector_type(2))) _Float16 v2;
  static constexpr int kCountCap = 2048;
  static __device__ __forceinline__ f32x4 mma(const uint4& a, const uint4& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8, a),
                                                  __builtin_bit_cast(v8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ void lds_add(uint32_t* word, bool high, float v) {
    const v2 x = high ? v2{static_cast<_Float16>(0.0f), static_cast<_Float16>(v)}
                      : v2{static_cast<_Float16>(v), static_cast<_Float16>(0.0f)};
    __builtin_amdgcn_ds_atomic_fadd_v2f16(
        (__attribute__((address_space(3))) v2*)(word), x);
  }
};

// Exclusive prefix sum over the 64 lanes of a wave; *total gets the sum.
__device__ __forceinline__ uint32_t wave_excl(uint32_t v, uint32_t* total) {
  const int lane = lane_id();
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const uint32_t y = __shfl_up(x, o, kWave);
    if (lane >= o) x += y;
  }
  *total = __shfl(x, kWave - 1, kWave);
  return x - v;
}

template <typename IT>
__device__ __forceinline__ int64_t ld_index(const void* p, int64_t i) {
  return static_cast<int64_t>(static_cast<const IT*>(p)[i]);
}

// One workgroup per (listed table, 64-row e tile, 64-column d tile): a
// 64 x 64 block of W_t goes through LDS and leaves as rows of W_t^T.
__global__ __launch_bounds__(kBlock) void hist_transpose(HistLaunch a) {
  __shared__ uint16_t s[64][66];
  const int per_table = a.etiles * a.dtiles;
  const int h = blockIdx.x / per_table;
  const int rem = blockIdx.x - h * per_table;
  const int et = rem / a.dtiles, dt = rem - et * a.dtiles;
  const HistTable ht = a.list[h];
  const TableMeta m = a.meta[ht.table];
  const int e0 = et * 64, d0 = dt * 64;
  if (e0 >= ht.epad || d0 >= m.dim) return;
  const uint16_t* w = static_cast<const uint16_t*>(a.weights) + m.woff;
  const int tid = threadIdx.x;
  for (int idx = tid; idx < 64 * 8; idx += kBlock) {
    const int r = idx >> 3, c8 = (idx & 7) * 8;
    const int e = e0 + r, d = d0 + c8;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (e < m.rows && d < m.dim)
      v = *reinterpret_cast<const uint4*>(w + static_cast<int64_t>(e) * m.dim + d);
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      s[r][c8 + 2 * j] = static_cast<uint16_t>(u[j] & 0xFFFFu);
      s[r][c8 + 2 * j + 1] = static_cast<uint16_t>(u[j] >> 16);
    }
  }
  __syncthreads();
  uint16_t* wt = a.wt + ht.wt_off;
  for (int idx = tid; idx < 64 * 8; idx += kBlock) {
    const int dr = idx >> 3, c8 = (idx & 7) * 8;
    const int d = d0 + dr;
    if (d >= m.dim) continue;
    uint32_t u[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      u[j] = static_cast<uint32_t>(s[c8 + 2 * j][dr]) |
             (static_cast<uint32_t>(s[c8 + 2 * j + 1][dr]) << 16);
    *reinterpret_cast<uint4*>(wt + static_cast<int64_t>(d) * ht.epad + e0 + c8) =
        make_uint4(u[0], u[1], u[2], u[3]);
  }
}

// Adds v (+1 or -1) to the count rows of a wave's bags for the lookups that
// fall in one chunk: entries {bag slot in wave << 6 | row in chunk}, listed
// by chunk.
template <typename M>
__device__ __forceinline__ void add_listed(uint32_t* cw, const uint16_t* ent, int n, int row0,
                                           float v) {
  for (int e = lane_id(); e < n; e += kWave) {
    const uint32_t q = ent[e];
    const int el = (row0 + static_cast<int>(q >> 6)) * kCS + static_cast<int>(q & 63u);
    M::lds_add(cw + (el >> 1), el & 1, v);
  }
}

// Lanes among `active` whose value c (of `bits` bits) equals this lane's: one
// ballot per bit.  Call with the whole wave.
__device__ __forceinline__ uint64_t match_value(uint64_t active, uint32_t c, int bits) {
  return match_low_bits(active, c, bits);
}

template <int ST, typename IT>
__global__ __launch_bounds__(kBlock) void fwd_histogram(HistLaunch a) {
  using M = Mma<ST>;
  __shared__ __align__(16) uint16_t s_c[kHB * kCS];  // count rows [bag][row in chunk]
  __shared__ float s_scale[kHB];  // output scale per bag; kNoBag: no bag, kLongBag: gathered
  __shared__ uint16_t s_ent[kWavesPerBlock][kEntCap];  // per wave and batch, by chunk
  __shared__ uint32_t s_boff[kWavesPerBlock][kWave + 1];  // the wave's bag starts, from its first lookup
  __shared__ uint32_t s_cnt[kWavesPerBlock][kMaxChunks];
  __shared__ uint32_t s_fill[kWavesPerBlock][kMaxChunks];
  __shared__ uint32_t s_start[kWavesPerBlock][kMaxChunks + 1];

  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const int logical = xcd_contiguous_block(blockIdx.x, gridDim.x);
  const int tiles = (a.B + kHB - 1) / kHB;
  const int per_table = tiles * a.dtiles;
  const int h = logical / per_table;
  const int rem = logical - h * per_table;
  const int dt = rem / tiles, tile = rem - dt * tiles;
  const HistTable ht = a.list[h];
  const TableMeta m = a.meta[ht.table];
  const int d0 = dt * kDB;
  if (d0 >= m.dim) return;  // whole workgroup
  const int NT = min(kDB, m.dim - d0) >> 4;  // 16-column MFMA tiles
  const int b0 = tile * kHB;
  const int nb = min(kHB, a.B - b0);
  const int nchunks = ht.epad / kHistKc;
  uint32_t* cw = reinterpret_cast<uint32_t*>(s_c);

  // thread tid owns bag slot tid: its lookups, first kRegIds ids in registers
  // (ids outside [0, epad) match no chunk)
  int64_t p0 = 0;
  int len = 0;
  if (tid < nb) {
    const int64_t k = static_cast<int64_t>(ht.table) * a.B + b0 + tid;
    p0 = ld_index<IT>(a.offsets, k);
    len = static_cast<int>(ld_index<IT>(a.offsets, k + 1) - p0);
  }
  const bool fallback = len > M::kCountCap;  // pooled by the gather loop below
  const int my_len = fallback ? 0 : len;
  s_scale[tid] = tid >= nb ? kNoBag
                 : fallback ? kLongBag
                            : (a.mean ? (len > 0 ? 1.0f / static_cast<float>(len) : 0.0f) : 1.0f);
  // this thread's count row (rows of a wave's bags are used by that wave only)
  {
    uint4* c4 = reinterpret_cast<uint4*>(s_c + tid * kCS);
#pragma unroll
    for (int i = 0; i < kCS / 8; ++i) c4[i] = make_uint4(0u, 0u, 0u, 0u);
  }
  // The wave's bags are consecutive, so its lookups are the positions
  // [P0, P1).  Waves whose bags all have at most kRegIds lookups keep their
  // ids in registers (one load round); the others list all their lookups with
  // the whole wave on consecutive positions, kEntCap at a time.
  const int64_t P0 = __shfl(p0, 0, kWave);
  int64_t P1 = tid < nb ? p0 + len : 0;
#pragma unroll
  for (int o = kWave >> 1; o >= 1; o >>= 1) {
    const int64_t y = __shfl_xor(P1, o, kWave);
    P1 = y > P1 ? y : P1;
  }
  if (P1 < P0) P1 = P0;  // a wave without bags
  s_boff[wave][lane] = static_cast<uint32_t>((tid < nb ? p0 : P1) - P0);
  if (lane == 0) s_boff[wave][kWave] = static_cast<uint32_t>(P1 - P0);
  const bool rest = __any(my_len > kRegIds);  // some bag of the wave is longer than kRegIds
  int32_t x[kRegIds];
#pragma unroll
  for (int j = 0; j < kRegIds; ++j) {
    int64_t v = -1;
    if (!rest && j < my_len) v = ld_index<IT>(a.indices, p0 + j);
    x[j] = (v >= 0 && v < ht.epad) ? static_cast<int32_t>(v) : -kHistKc - 1;
  }
  const int cbits = nchunks <= 1 ? 0 : 32 - __clz(nchunks - 1);
  // the bag of a listed position: bags of 16 or more lookups on average are
  // followed lane by lane (positions only grow), shorter ones binary searched
  const bool follow = P1 - P0 >= int64_t{16} * kWave;
  int cur = 0;
  const auto bag_of = [&](uint32_t rel) {
    if (follow) {
      while (cur < kWave - 1 && s_boff[wave][cur + 1] <= rel) ++cur;
      return cur;
    }
    int lo = 0, hi = kWave;  // the last slot starting at or before rel
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_boff[wave][mid] <= rel)
        lo = mid;
      else
        hi = mid;
    }
    return lo;
  };
  const int nbatch = rest ? static_cast<int>((P1 - P0 + kEntCap - 1) / kEntCap) : 1;

  // B operands (W^T) straight from L2 into registers:
  // lane holds column n0 + (lane & 15), rows k0 + ks*32 + (lane >> 4)*8 .. +8
  const uint16_t* wcol =
      a.wt + ht.wt_off + static_cast<int64_t>(d0 + (lane & 15)) * ht.epad + (lane >> 4) * 8;
  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  // Lookups are listed by chunk (entries {bag slot << 6 | row in chunk}):
  // counts, offsets, then entries.  LDS operations of one wave complete in
  // order, so the wave's lists need no barrier.
  const auto offsets_by_chunk = [&]() {
    const uint32_t cnt = lane < kMaxChunks ? s_cnt[wave][lane] : 0u;
    uint32_t tot;
    const uint32_t st = wave_excl(cnt, &tot);
    if (lane < kMaxChunks) s_start[wave][lane] = st;
    if (lane == 0) s_start[wave][kMaxChunks] = tot;
  };
  if (!rest) {  // the registered ids, once
    if (lane < kMaxChunks) s_cnt[wave][lane] = 0u, s_fill[wave][lane] = 0u;
#pragma unroll
    for (int j = 0; j < kRegIds; ++j)
      if (j < my_len && x[j] >= 0) atomicAdd(&s_cnt[wave][x[j] / kHistKc], 1u);
    offsets_by_chunk();
#pragma unroll
    for (int j = 0; j < kRegIds; ++j)
      if (j < my_len && x[j] >= 0) {
        const int c = x[j] / kHistKc;
        s_ent[wave][s_start[wave][c] + atomicAdd(&s_fill[wave][c], 1u)] =
            static_cast<uint16_t>((lane << 6) | (x[j] & (kHistKc - 1)));
      }
  }
  __syncthreads();  // s_scale
  for (int bt = 0; bt < nbatch; ++bt) {
    const int64_t q0 = P0 + static_cast<int64_t>(bt) * kEntCap;
    const int64_t q1 = q0 + kEntCap < P1 ? q0 + kEntCap : P1;
    // a table of one row chunk: the batch's lookups go straight into the
    // count tile, which is multiplied once and then cleared (no lists)
    const bool direct = rest && nchunks == 1;
    if (direct) {
#pragma unroll
      for (int u = 0; u < kListSteps; ++u) {
        const int64_t p = q0 + u * kWave + lane;
        int lo = 0;
        int64_t v = -1;
        if (q0 + u * kWave < q1 && p < q1) {
          lo = bag_of(static_cast<uint32_t>(p - P0));
          v = ld_index<IT>(a.indices, p);
        }
        if (v >= 0 && v < ht.epad && s_scale[wave * kWave + lo] >= 0.0f) {
          const int el = (wave * kWave + lo) * kCS + static_cast<int>(v);
          M::lds_add(cw + (el >> 1), el & 1, 1.0f);
        }
      }
    }
    if (rest && !direct) {
      // the batch's positions, listed by the whole wave: the kListSteps steps
      // of 64 positions issue their id loads together, and each lookup's entry
      // stays in a register from the count to the fill
      if (lane < kMaxChunks) s_cnt[wave][lane] = 0u, s_fill[wave][lane] = 0u;
      int64_t v[kListSteps];
      int slot[kListSteps];
#pragma unroll
      for (int u = 0; u < kListSteps; ++u) {
        const int64_t p = q0 + u * kWave + lane;
        v[u] = -1;
        slot[u] = 0;
        if (q0 + u * kWave < q1 && p < q1) {
          slot[u] = bag_of(static_cast<uint32_t>(p - P0));
          v[u] = ld_index<IT>(a.indices, p);
        }
      }
      uint32_t ent[kListSteps];  // chunk << 16 | entry, or ~0 for no lookup
#pragma unroll
      for (int u = 0; u < kListSteps; ++u) {
        if (q0 + u * kWave >= q1) break;
        const bool valid = v[u] >= 0 && v[u] < ht.epad && s_scale[wave * kWave + slot[u]] >= 0.0f;
        const uint32_t c = valid ? static_cast<uint32_t>(v[u] / kHistKc) : 0u;
        ent[u] = valid ? (c << 16) | static_cast<uint32_t>((slot[u] << 6) |
                                                           static_cast<int>(v[u] & (kHistKc - 1)))
                       : ~0u;
        const uint64_t peers = match_value(__ballot(valid), c, cbits);
        if (valid && popc_below(peers) == 0) s_cnt[wave][c] += __popcll(peers);
      }
      offsets_by_chunk();
#pragma unroll
      for (int u = 0; u < kListSteps; ++u) {
        if (q0 + u * kWave >= q1) break;
        const bool valid = ent[u] != ~0u;
        const uint32_t c = valid ? ent[u] >> 16 : 0u;
        const uint64_t peers = match_value(__ballot(valid), c, cbits);
        const uint32_t below = popc_below(peers);
        const uint32_t pre = valid ? s_fill[wave][c] : 0u;
        if (valid) s_ent[wave][s_start[wave][c] + pre + below] = static_cast<uint16_t>(ent[u] & 0xFFFFu);
        if (valid && below == 0) s_fill[wave][c] = pre + __popcll(peers);
      }
    }

    for (int c = 0; c < nchunks; ++c) {
      const int k0 = c * kHistKc;
      uint4 bf[2][4];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
          bf[ks][nt] = nt < NT ? *reinterpret_cast<const uint4*>(
                                     wcol + static_cast<int64_t>(nt * 16) * ht.epad + k0 + ks * 32)
                               : make_uint4(0u, 0u, 0u, 0u);
      // the wave's count rows for chunk c
      const int es = direct ? 0 : static_cast<int>(s_start[wave][c]);
      const int en = direct ? 0 : static_cast<int>(s_start[wave][c + 1]) - es;
      if (!direct) {
        if (en == 0) continue;  // no lookup of this wave's bags in this chunk
        add_listed<M>(cw, s_ent[wave] + es, en, wave * 64, 1.0f);
      }
#pragma unroll
      for (int ks = 0; ks < kHistKc / 32; ++ks) {
        const int col = ks * 32 + (lane >> 4) * 8;
        uint4 af[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
          af[mt] = *reinterpret_cast<const uint4*>(s_c + (wave * 64 + mt * 16 + (lane & 15)) * kCS + col);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
          if (nt < NT) {
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) acc[mt][nt] = M::mma(af[mt], bf[ks][nt], acc[mt][nt]);
          }
      }
      if (direct) {  // this lane's count row back to zero
        uint4* c4 = reinterpret_cast<uint4*>(s_c + tid * kCS);
#pragma unroll
        for (int i = 0; i < kCS / 8; ++i) c4[i] = make_uint4(0u, 0u, 0u, 0u);
      } else {
        add_listed<M>(cw, s_ent[wave] + es, en, wave * 64, -1.0f);
      }
    }
  }

  // results: lane holds rows 4*(lane/16) + r of each 16 x 16 tile, column lane % 16
  float* const out0 = a.out + static_cast<int64_t>(b0) * a.sum_dims + m.doff + d0;
  float* const obase = out0 + (lane & 15);
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int slot = wave * 64 + mt * 16 + (lane >> 4) * 4 + r;
      const float sc = s_scale[slot];
      if (sc >= 0.0f) {
        float* o = obase + static_cast<int64_t>(slot) * a.sum_dims;
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
          if (nt < NT) o[nt * 16] = acc[mt][nt][r] * sc;
      }
    }
  }

  // bags too long for exact 16-bit counts: plain gather, one wave per bag
  const uint16_t* w = static_cast<const uint16_t*>(a.weights) + m.woff;
  const int DN = NT * 16;
  for (int slot = wave; slot < nb; slot += kWavesPerBlock) {
    if (s_scale[slot] != kLongBag) continue;
    const int64_t kk = static_cast<int64_t>(ht.table) * a.B + b0 + slot;
    const int64_t s0 = ld_index<IT>(a.offsets, kk), s1 = ld_index<IT>(a.offsets, kk + 1);
    if (lane < DN) {
      float sum = 0.0f;
      for (int64_t p = s0; p < s1; ++p) {
        const int64_t xr = ld_index<IT>(a.indices, p);
        const uint32_t u = w[xr * m.dim + d0 + lane];
        sum += ST == kBF16 ? bf16_lo(u) : f16_lo(u);
      }
      const float sc = a.mean ? 1.0f / static_cast<float>(s1 - s0) : 1.0f;
      out0[static_cast<int64_t>(slot) * a.sum_dims + lane] = sum * sc;
    }
  }
}

template <int ST>
hipError_t dispatch(const HistLaunch& a, hipStream_t s, dim3 grid, const KernelTimer* kt) {
  if (a.index64)
    launch_timed(kt, "fwd_histogram", fwd_histogram<ST, int64_t>, grid, dim3(kBlock), 0, s, a);
  else
    launch_timed(kt, "fwd_histogram", fwd_histogram<ST, int32_t>, grid, dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_forward_histogram(const HistLaunch& a, hipStream_t stream,
                                    const KernelTimer* kt) {
  if (a.H <= 0 || a.B <= 0) return hipSuccess;
  const int64_t tgrid = static_cast<int64_t>(a.H) * a.etiles * a.dtiles;
  const int64_t tiles = (a.B + kHB - 1) / kHB;
  const int64_t fgrid = static_cast<int64_t>(a.H) * tiles * a.dtiles;
  if (tgrid > 0x7FFFFFFF || fgrid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  launch_timed(kt, "hist_transpose", hist_transpose, dim3(static_cast<unsigned>(tgrid)),
               dim3(kBlock), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid(static_cast<unsigned>(fgrid));
  e = a.dtype == kBF16 ? dispatch<kBF16>(a, stream, grid, kt)
                       : (a.dtype == kF16 ? dispatch<kF16>(a, stream, grid, kt) : hipErrorInvalidValue);
  return e;
}

}  // namespace tbe
