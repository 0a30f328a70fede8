/*
 * tbe_oracle.h -- plain CPU reference for the table-batched-embedding (TBE)
 * forward pooling and the one-update-per-row backward.
 *
 * TEST INFRASTRUCTURE ONLY.  This library exists so that tests, the smoke check
 * and the benchmark's CPU-baseline leg can check the GPU library against an
 * independent, obviously correct implementation.  No product code may link,
 * load or call it.  It shares no code, header or constant table with the GPU
 * library.
 *
 * Arithmetic is fp64 throughout (inputs are widened exactly from their storage
 * type); results that must be stored in a narrower type are rounded once,
 * round-to-nearest-even.
 *
 * Conventions (all host pointers, caller-owned):
 *   T tables; table t has rows[t] rows of dims[t] elements, stored row-major
 *   one after another in one flat buffer (table t starts at element
 *   sum_{t'<t} rows[t']*dims[t']).  Storage dtype: 0 = fp32, 1 = fp16, 2 = bf16.
 *   Bags are table-major: bag k = t*B + b.  offsets has T*B+1 entries
 *   (CSR with a trailing total); indices are table-local row ids.
 *   Output Y is [B, sum_t dims[t]] with table t in columns
 *   [sum_{t'<t} dims[t'], +dims[t]).
 *
 * Every function returns 0 on success and a negative value on invalid input
 * (null pointer, bad sizes, an index outside [0, rows[t]), offsets that are
 * not a CSR array over num_indices entries).
 */
#ifndef TBE_ORACLE_H
#define TBE_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORACLE_F32 = 0, ORACLE_F16 = 1, ORACLE_BF16 = 2 };
enum { ORACLE_POOL_SUM = 0, ORACLE_POOL_MEAN = 1 };
enum { ORACLE_OPT_SGD = 0, ORACLE_OPT_ROWWISE_ADAGRAD = 1 };

/* Storage conversions, written from the IEEE-754 binary16 and bfloat16
 * definitions.  widen: exact.  narrow: round-to-nearest-even, overflow to
 * infinity, NaN to a quiet NaN of the same sign. */
double   tbe_oracle_widen(int32_t dtype, uint32_t bits);
uint32_t tbe_oracle_narrow(int32_t dtype, double x);
/* Array versions: n elements. */
void tbe_oracle_widen_array(int32_t dtype, const void* src, double* dst, int64_t n);
void tbe_oracle_narrow_array(int32_t dtype, const double* src, void* dst, int64_t n);

/* Pooled forward for every bag.  out: [B, sum dims] fp64. */
int tbe_oracle_forward(int32_t T, const int64_t* rows, const int32_t* dims, int32_t dtype,
                       int32_t pooling, const void* weights, int64_t B,
                       const int64_t* indices, const int64_t* offsets, int64_t num_indices,
                       const float* per_sample_weights, double* out);

/* Pooled forward for a chosen list of bags (ids k = t*B + b).  out is packed:
 * the j-th requested bag's dims[t] values follow the previous bag's. */
int tbe_oracle_forward_bags(int32_t T, const int64_t* rows, const int32_t* dims, int32_t dtype,
                            int32_t pooling, const void* weights, int64_t B,
                            const int64_t* indices, const int64_t* offsets, int64_t num_indices,
                            const float* per_sample_weights, int64_t num_bags,
                            const int64_t* bag_ids, double* out);

/* Grouping of the lookups by destination row: the ascending distinct linear
 * row ids (row_offset[t] + index) and how many lookups hit each.
 * unique_ids, counts: capacity num_indices.  *num_unique receives U. */
int tbe_oracle_runs(int32_t T, const int64_t* rows, int64_t B,
                    const int64_t* indices, const int64_t* offsets, int64_t num_indices,
                    int64_t* unique_ids, int64_t* counts, int64_t* num_unique);

/* Summed gradient of every table row, dense, in the weights' flat layout:
 * grad[woff_t + r*dims[t] + d] = sum over lookups i of row r of table t of
 * p_i * s_k * grad_output[b, doff_t + d].  grad: fp64 [sum rows*dims]. */
int tbe_oracle_dense_grad(int32_t T, const int64_t* rows, const int32_t* dims, int32_t pooling,
                          int64_t B, const int64_t* indices, const int64_t* offsets,
                          int64_t num_indices, const float* per_sample_weights,
                          const float* grad_output, double* grad);

/* dL/dp_i for every lookup: s_k * sum_d grad_output[b, doff_t + d] *
 * W_t[x_i, d] (the forward is linear in the per-sample weights).
 * grad_psw: fp64 [num_indices]. */
int tbe_oracle_psw_grad(int32_t T, const int64_t* rows, const int32_t* dims, int32_t dtype,
                        int32_t pooling, const void* weights, int64_t B, const int64_t* indices,
                        const int64_t* offsets, int64_t num_indices, const float* grad_output,
                        double* grad_psw);

/* Backward with the fused optimizer: exactly one update per touched row.
 * weights (storage dtype) and state (fp32, one per table row, indexed by the
 * linear row id; may be NULL for SGD) are updated in place.
 * If num_selected > 0, only the listed linear row ids (ascending) that are
 * touched get updated; all other rows are left as they are (used to check a
 * sample of rows of a large problem). */
int tbe_oracle_backward_update(int32_t T, const int64_t* rows, const int32_t* dims,
                               int32_t dtype, int32_t pooling, int32_t optimizer,
                               void* weights, float* state, int64_t B,
                               const int64_t* indices, const int64_t* offsets,
                               int64_t num_indices, const float* per_sample_weights,
                               const float* grad_output, double lr, double eps,
                               int64_t num_selected, const int64_t* selected_rows);

/* OpenMP thread count used by the calls above (<= 0: leave the default). */
void tbe_oracle_set_threads(int32_t n);
int32_t tbe_oracle_get_threads(void);

#ifdef __cplusplus
}
#endif
#endif
