// count_backward.hpp -- launch interface of the count-matrix backward for
// small tables (count_backward.hip).  Internal; the public interface is tbe.h.
#pragma once

#include "common.hpp"

namespace tbe {

// Eligibility of a table (every table of the handle must qualify): at most
// kCbMaxRows rows and a dim that is a multiple of 16 up to kCbMaxDim.  Calls
// with per-sample weights use the sort path instead.
constexpr int kCbMaxRows = 1024;
constexpr int kCbMaxDim = 256;
constexpr int kCbGroupRows = 1024;  // table rows per workgroup (16 waves x 64 rows)
constexpr int kCbCols = 64;         // columns per workgroup (4 MFMA column tiles)

// One (table, 64-column slice) of the product.  Its bag slices make the
// workgroups (one row group of kCbGroupRows rows holds the whole table).
struct CountUnit {
  int32_t table;
  int32_t col0;
};

struct CountLaunch {
  const void* indices;
  const void* offsets;
  const float* grad;
  void* weights;
  float* state;
  const TableMeta* meta;
  const CountUnit* units;
  int32_t nunits;
  int32_t T, B, sum_dims;
  int32_t slices;           // bag slices per unit (partial sums added in slice order)
  int32_t mean, index64, dtype, adagrad;
  float lr, eps;
  int64_t sum_rows;
  // workspace: partial sums of table t at slices * woff_t (slice-major, then
  // rows of D_t floats), row counts of table t at slices * roff_t
  float* partial;
  uint32_t* counts;
  uint32_t* scan;           // [2 + ceil(sum_rows / 1024)] block totals of the runs output
  int32_t* out_unique;      // optional run outputs
  int32_t* out_lengths;
  int32_t* out_num;
};

// Workspace bytes of the count-matrix backward for `slices` bag slices.
inline size_t count_backward_bytes(int64_t weights_elems, int64_t sum_rows, int slices) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  return up(4 * static_cast<size_t>(weights_elems) * slices) +
         up(4 * static_cast<size_t>(sum_rows) * slices) +
         up(4 * (2 + static_cast<size_t>((sum_rows + 1023) / 1024)));
}

// The product (partial sums per bag slice), then the update of every row a
// lookup touched (partials added in slice order), then -- when asked for --
// the runs (touched rows ascending, their lookup counts, U).
hipError_t launch_count_backward(const CountLaunch& a, hipStream_t stream, const KernelTimer* kt);

}  // namespace tbe
