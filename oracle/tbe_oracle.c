/*
 * tbe_oracle.c -- plain CPU reference for table-batched embedding (TBE).
 *
 * TEST INFRASTRUCTURE ONLY (see tbe_oracle.h).  Slow on purpose: every result
 * is computed straight from its definition, in fp64, with no blocking, no
 * fusion and no reordering beyond what the definition states.  OpenMP only
 * splits independent bags / independent rows across threads.
 *
 * What is computed, and where it is described:
 *
 *  Forward (pooled lookup).  "FBTriton Rewrites Table Batched Embedding"
 *  (kongchang.com), sections "What are embedding tables and sparse features?"
 *  and "Responsibilities of the forward and backward passes": each bag of
 *  sparse ids selects rows of its table and the rows are aggregated into one
 *  dense vector per sample and table.  kimbodo.com/?p=28372, "What Happened":
 *  all tables are handled together, per-sample weights are optional and the
 *  accumulation is done at a higher precision than the storage.
 *  "Optimizing Recommendation Systems with FBTriton Table Batched Embeddings"
 *  (explore.n1n.ai), "Implementation Guide: Integrating TBE": the batch is a
 *  flat index list plus an offsets list whose last entry is the index count;
 *  "Pro Tips for TBE Scaling": tables may be stored in fp16 / bf16.
 *
 *      Y[b, doff_t + d] = s_k * sum_{i in bag k} p_i * W_t[x_i, d],  k = t*B + b
 *      s_k = 1 (sum) or 1/L_k (mean, L_k = bag length; an empty bag gives 0).
 *
 *  Backward with the optimizer.  kongchang.com page, "Responsibilities ...":
 *  upstream gradients are scattered back to the rows that were looked up and
 *  added up where a row was hit more than once.  kimbodo.com/?p=28372, "What
 *  Happened": updates are grouped by (table, row) so that each touched row
 *  gets a single optimizer update; "Kimbodo Engineering Perspective": the
 *  grouping is a transpose, a sort and a run-length encoding.
 *
 *      g_i      = p_i * s_k * G[b, doff_t : doff_t + D_t]
 *      l_i      = roff_t + x_i                       (linear row id)
 *      Gamma_r  = sum_{i : l_i = r} g_i              (summed in ascending i)
 *      one update per distinct r:
 *        SGD:                 W_r <- W_r - lr * Gamma_r
 *        row-wise Adagrad:    m_r <- m_r + mean_d Gamma_r[d]^2
 *                             W_r <- W_r - lr * Gamma_r / (sqrt(m_r) + eps)
 *  The pages name no optimizer; SGD and the row-wise Adagrad above (state
 *  updated before it is used, eps outside the square root, mean over the row)
 *  are the plainest readings and are documented as readings.  On rows of one
 *  column the row-wise Adagrad is plain Adagrad, and the tests pin it there
 *  against torch.optim.Adagrad (update order, place of eps).
 *
 *  Storage conversions follow the IEEE-754 binary16 definition and the
 *  bfloat16 definition (the upper half of an IEEE binary32).
 */
#include "tbe_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Accumulator of the sums and of the update.  The default, double, is the
 * parity reference the tests compare against.  The same source compiled with
 * -DORACLE_ACC=float is the timing build (fp32 sums, as a plain CPU
 * implementation would run); it is timed as a CPU baseline and never used as
 * a reference. */
#ifndef ORACLE_ACC
#define ORACLE_ACC double
#endif
typedef ORACLE_ACC acc_t;

/* ------------------------------------------------------------------------ */
/* Storage conversions                                                       */
/* ------------------------------------------------------------------------ */

/* A binary floating-point format with an implicit leading bit: p fraction
 * bits, ebits exponent bits, normal exponents in [emin, emax], bias = emax. */
typedef struct { int p; int ebits; int emin; int emax; } fmt_t;

static const fmt_t FMT_F16 = {10, 5, -14, 15};
static const fmt_t FMT_BF16 = {7, 8, -126, 127};

static double decode_small(const fmt_t* f, uint32_t bits) {
  const uint32_t sign = (bits >> (f->p + f->ebits)) & 1u;
  const uint32_t efield = (bits >> f->p) & ((1u << f->ebits) - 1u);
  const uint32_t frac = bits & ((1u << f->p) - 1u);
  double v;
  if (efield == 0) {
    v = ldexp((double)frac, f->emin - f->p); /* zero or subnormal */
  } else if (efield == (1u << f->ebits) - 1u) {
    v = frac ? NAN : INFINITY;
  } else {
    v = ldexp((double)((1u << f->p) + frac), (int)efield - f->emax - f->p);
  }
  return sign ? -v : v;
}

/* Round x to the nearest value of format f (ties to even) and encode it. */
static uint32_t encode_small(const fmt_t* f, double x) {
  const uint32_t signbit = 1u << (f->p + f->ebits);
  const uint32_t expmask = (1u << f->ebits) - 1u;
  const uint32_t sign = signbit(x) ? signbit : 0u;
  if (isnan(x)) return sign | (expmask << f->p) | (1u << (f->p - 1)); /* quiet NaN */
  const double a = fabs(x);
  if (isinf(a)) return sign | (expmask << f->p);
  if (a == 0.0) return sign;
  /* Spacing of representable values around a: 2^(e - p) for normal numbers,
   * 2^(emin - p) in the subnormal range. */
  int e = ilogb(a);
  if (e < f->emin) e = f->emin;
  const double q = ldexp(1.0, e - f->p);
  const double n = nearbyint(a / q); /* a / q is exact; default mode is ties-to-even */
  const double v = n * q;
  if (v >= ldexp(1.0, f->emax + 1)) return sign | (expmask << f->p); /* overflow */
  if (v == 0.0) return sign;
  const int ev = ilogb(v);
  if (ev < f->emin) {
    return sign | (uint32_t)(v / ldexp(1.0, f->emin - f->p)); /* subnormal */
  }
  const uint32_t frac = (uint32_t)(v / ldexp(1.0, ev - f->p)) - (1u << f->p);
  return sign | ((uint32_t)(ev + f->emax) << f->p) | frac;
}

double tbe_oracle_widen(int32_t dtype, uint32_t bits) {
  if (dtype == ORACLE_F32) {
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
  }
  if (dtype == ORACLE_F16) return decode_small(&FMT_F16, bits & 0xFFFFu);
  return decode_small(&FMT_BF16, bits & 0xFFFFu);
}

uint32_t tbe_oracle_narrow(int32_t dtype, double x) {
  if (dtype == ORACLE_F32) {
    const float f = (float)x; /* C conversion: round to nearest even */
    uint32_t bits;
    memcpy(&bits, &f, sizeof bits);
    return bits;
  }
  if (dtype == ORACLE_F16) return encode_small(&FMT_F16, x);
  return encode_small(&FMT_BF16, x);
}

static uint32_t load_bits(int32_t dtype, const void* base, int64_t e) {
  if (dtype == ORACLE_F32) return ((const uint32_t*)base)[e];
  return ((const uint16_t*)base)[e];
}

static void store_bits(int32_t dtype, void* base, int64_t e, uint32_t bits) {
  if (dtype == ORACLE_F32)
    ((uint32_t*)base)[e] = bits;
  else
    ((uint16_t*)base)[e] = (uint16_t)bits;
}

void tbe_oracle_widen_array(int32_t dtype, const void* src, double* dst, int64_t n) {
  for (int64_t i = 0; i < n; ++i) dst[i] = tbe_oracle_widen(dtype, load_bits(dtype, src, i));
}

void tbe_oracle_narrow_array(int32_t dtype, const double* src, void* dst, int64_t n) {
  for (int64_t i = 0; i < n; ++i) store_bits(dtype, dst, i, tbe_oracle_narrow(dtype, src[i]));
}

/* ------------------------------------------------------------------------ */
/* Table layout and input checks                                             */
/* ------------------------------------------------------------------------ */

typedef struct {
  int32_t T;
  const int64_t* rows;
  const int32_t* dims;
  int64_t* woff; /* element offset of table t in the flat weights */
  int64_t* roff; /* linear row id of row 0 of table t */
  int64_t* doff; /* first output column of table t */
  int64_t sum_dims;
} layout_t;

static int layout_init(layout_t* L, int32_t T, const int64_t* rows, const int32_t* dims) {
  L->woff = L->roff = L->doff = NULL;
  if (T <= 0 || !rows || !dims) return -1;
  L->T = T;
  L->rows = rows;
  L->dims = dims;
  L->woff = (int64_t*)malloc(sizeof(int64_t) * (size_t)(T + 1));
  L->roff = (int64_t*)malloc(sizeof(int64_t) * (size_t)(T + 1));
  L->doff = (int64_t*)malloc(sizeof(int64_t) * (size_t)(T + 1));
  if (!L->woff || !L->roff || !L->doff) return -2;
  L->woff[0] = L->roff[0] = L->doff[0] = 0;
  for (int32_t t = 0; t < T; ++t) {
    if (rows[t] <= 0 || dims[t] <= 0) return -1;
    L->woff[t + 1] = L->woff[t] + rows[t] * (int64_t)dims[t];
    L->roff[t + 1] = L->roff[t] + rows[t];
    L->doff[t + 1] = L->doff[t] + dims[t];
  }
  L->sum_dims = L->doff[T];
  return 0;
}

static void layout_free(layout_t* L) {
  free(L->woff);
  free(L->roff);
  free(L->doff);
}

/* offsets must be CSR over num_indices entries and every index must be a
 * valid row of its bag's table. */
static int check_batch(const layout_t* L, int64_t B, const int64_t* indices,
                       const int64_t* offsets, int64_t num_indices) {
  if (B < 0 || num_indices < 0 || !offsets) return -1;
  if (num_indices > 0 && !indices) return -1;
  const int64_t nbags = (int64_t)L->T * B;
  if (offsets[0] != 0 || offsets[nbags] != num_indices) return -3;
  for (int64_t k = 0; k < nbags; ++k) {
    if (offsets[k + 1] < offsets[k]) return -3;
    const int64_t t = k / B;
    for (int64_t i = offsets[k]; i < offsets[k + 1]; ++i)
      if (indices[i] < 0 || indices[i] >= L->rows[t]) return -4;
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Forward                                                                   */
/* ------------------------------------------------------------------------ */

/* Pool one bag into out[0 .. dims[t]): every column summed over the bag's
 * lookups in index order, then divided by the bag length for mean pooling. */
static void pool_bag(const layout_t* L, int32_t dtype, int32_t pooling, const void* weights,
                     int64_t B, const int64_t* indices, const int64_t* offsets,
                     const float* psw, int64_t k, double* out) {
  const int64_t t = k / B;
  const int64_t D = L->dims[t];
  const int64_t begin = offsets[k], end = offsets[k + 1];
  for (int64_t d = 0; d < D; ++d) {
    acc_t acc = 0;
    for (int64_t i = begin; i < end; ++i) {
      const acc_t p = psw ? (acc_t)psw[i] : (acc_t)1;
      const int64_t e = L->woff[t] + indices[i] * D + d;
      acc += p * (acc_t)tbe_oracle_widen(dtype, load_bits(dtype, weights, e));
    }
    if (pooling == ORACLE_POOL_MEAN && end > begin) acc /= (acc_t)(end - begin);
    out[d] = (double)acc;
  }
}

int tbe_oracle_forward(int32_t T, const int64_t* rows, const int32_t* dims, int32_t dtype,
                       int32_t pooling, const void* weights, int64_t B,
                       const int64_t* indices, const int64_t* offsets, int64_t num_indices,
                       const float* psw, double* out) {
  layout_t L;
  int rc = layout_init(&L, T, rows, dims);
  if (rc == 0 && (!weights || !out)) rc = -1;
  if (rc == 0) rc = check_batch(&L, B, indices, offsets, num_indices);
  if (rc == 0) {
    const int64_t nbags = (int64_t)T * B;
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t k = 0; k < nbags; ++k) {
      const int64_t t = k / B, b = k % B;
      pool_bag(&L, dtype, pooling, weights, B, indices, offsets, psw, k,
               out + b * L.sum_dims + L.doff[t]);
    }
  }
  layout_free(&L);
  return rc;
}

int tbe_oracle_forward_bags(int32_t T, const int64_t* rows, const int32_t* dims, int32_t dtype,
                            int32_t pooling, const void* weights, int64_t B,
                            const int64_t* indices, const int64_t* offsets, int64_t num_indices,
                            const float* psw, int64_t num_bags, const int64_t* bag_ids,
                            double* out) {
  layout_t L;
  int rc = layout_init(&L, T, rows, dims);
  if (rc == 0 && (!weights || !out || num_bags < 0 || (num_bags > 0 && !bag_ids))) rc = -1;
  if (rc == 0) rc = check_batch(&L, B, indices, offsets, num_indices);
  if (rc == 0) {
    for (int64_t j = 0; j < num_bags; ++j)
      if (bag_ids[j] < 0 || bag_ids[j] >= (int64_t)T * B) rc = -1;
  }
  if (rc == 0) {
    int64_t* pos = (int64_t*)malloc(sizeof(int64_t) * (size_t)(num_bags + 1));
    if (!pos) {
      rc = -2;
    } else {
      pos[0] = 0;
      for (int64_t j = 0; j < num_bags; ++j) pos[j + 1] = pos[j] + dims[bag_ids[j] / B];
#pragma omp parallel for schedule(dynamic, 16)
      for (int64_t j = 0; j < num_bags; ++j)
        pool_bag(&L, dtype, pooling, weights, B, indices, offsets, psw, bag_ids[j], out + pos[j]);
      free(pos);
    }
  }
  layout_free(&L);
  return rc;
}

/* ------------------------------------------------------------------------ */
/* Backward: linearize, sort, group                                          */
/* ------------------------------------------------------------------------ */

typedef struct {
  int64_t key;    /* linear row id */
  int64_t lookup; /* position i in the index list */
  int64_t bag;    /* bag id k */
} entry_t;

static int entry_cmp(const void* a, const void* b) {
  const entry_t* x = (const entry_t*)a;
  const entry_t* y = (const entry_t*)b;
  if (x->key != y->key) return x->key < y->key ? -1 : 1;
  if (x->lookup != y->lookup) return x->lookup < y->lookup ? -1 : 1;
  return 0;
}

/* Linearize every lookup to (row id, lookup, bag) and sort by (row id, lookup). */
static entry_t* sorted_entries(const layout_t* L, int64_t B, const int64_t* indices,
                               const int64_t* offsets, int64_t num_indices) {
  entry_t* e = (entry_t*)malloc(sizeof(entry_t) * (size_t)(num_indices > 0 ? num_indices : 1));
  if (!e) return NULL;
  const int64_t nbags = (int64_t)L->T * B;
  for (int64_t k = 0; k < nbags; ++k) {
    const int64_t t = k / B;
    for (int64_t i = offsets[k]; i < offsets[k + 1]; ++i) {
      e[i].key = L->roff[t] + indices[i];
      e[i].lookup = i;
      e[i].bag = k;
    }
  }
  qsort(e, (size_t)num_indices, sizeof(entry_t), entry_cmp);
  return e;
}

int tbe_oracle_runs(int32_t T, const int64_t* rows, int64_t B, const int64_t* indices,
                    const int64_t* offsets, int64_t num_indices, int64_t* unique_ids,
                    int64_t* counts, int64_t* num_unique) {
  /* dims are not needed for the grouping; use 1 so the layout check passes */
  int32_t* ones = (int32_t*)malloc(sizeof(int32_t) * (size_t)(T > 0 ? T : 1));
  if (!ones) return -2;
  for (int32_t t = 0; t < T; ++t) ones[t] = 1;
  layout_t L;
  int rc = layout_init(&L, T, rows, ones);
  if (rc == 0 && (!num_unique || (num_indices > 0 && (!unique_ids || !counts)))) rc = -1;
  if (rc == 0) rc = check_batch(&L, B, indices, offsets, num_indices);
  if (rc == 0) {
    entry_t* e = sorted_entries(&L, B, indices, offsets, num_indices);
    if (!e) {
      rc = -2;
    } else {
      int64_t u = 0;
      for (int64_t j = 0; j < num_indices; ++j) {
        if (j == 0 || e[j].key != e[j - 1].key) {
          unique_ids[u] = e[j].key;
          counts[u] = 0;
          ++u;
        }
        ++counts[u - 1];
      }
      *num_unique = u;
      free(e);
    }
  }
  layout_free(&L);
  free(ones);
  return rc;
}

/* Table of a linear row id. */
static int32_t table_of_key(const layout_t* L, int64_t key) {
  int32_t t = 0;
  while (t + 1 < L->T && L->roff[t + 1] <= key) ++t;
  return t;
}

/* Gamma of the run e[begin..end) (all with the same key): every column summed
 * over the run's lookups in lookup order. */
static void run_gradient(const layout_t* L, int32_t pooling, int64_t B, const int64_t* offsets,
                         const float* psw, const float* grad_output, const entry_t* e,
                         int64_t begin, int64_t end, int32_t t, double* gamma) {
  const int64_t D = L->dims[t];
  for (int64_t d = 0; d < D; ++d) {
    acc_t acc = 0;
    for (int64_t j = begin; j < end; ++j) {
      const int64_t k = e[j].bag, b = k % B;
      acc_t coef = psw ? (acc_t)psw[e[j].lookup] : (acc_t)1;
      if (pooling == ORACLE_POOL_MEAN) coef /= (acc_t)(offsets[k + 1] - offsets[k]);
      acc += coef * (acc_t)grad_output[b * L->sum_dims + L->doff[t] + d];
    }
    gamma[d] = (double)acc;
  }
}

/* Start of every run of equal keys in the sorted entries; returns the count. */
static int64_t run_starts(const entry_t* e, int64_t n, int64_t* starts) {
  int64_t u = 0;
  for (int64_t j = 0; j < n; ++j)
    if (j == 0 || e[j].key != e[j - 1].key) starts[u++] = j;
  starts[u] = n;
  return u;
}

int tbe_oracle_dense_grad(int32_t T, const int64_t* rows, const int32_t* dims, int32_t pooling,
                          int64_t B, const int64_t* indices, const int64_t* offsets,
                          int64_t num_indices, const float* psw, const float* grad_output,
                          double* grad) {
  layout_t L;
  int rc = layout_init(&L, T, rows, dims);
  if (rc == 0 && (!grad || (B > 0 && !grad_output))) rc = -1;
  if (rc == 0) rc = check_batch(&L, B, indices, offsets, num_indices);
  if (rc == 0) {
    for (int64_t j = 0; j < L.woff[T]; ++j) grad[j] = 0.0;
    entry_t* e = sorted_entries(&L, B, indices, offsets, num_indices);
    int64_t* starts = (int64_t*)malloc(sizeof(int64_t) * (size_t)(num_indices + 1));
    if (!e || !starts) {
      rc = -2;
    } else {
      const int64_t U = run_starts(e, num_indices, starts);
#pragma omp parallel for schedule(dynamic, 16)
      for (int64_t r = 0; r < U; ++r) {
        const int64_t key = e[starts[r]].key;
        const int32_t t = table_of_key(&L, key);
        double* out = grad + L.woff[t] + (key - L.roff[t]) * (int64_t)dims[t];
        run_gradient(&L, pooling, B, offsets, psw, grad_output, e, starts[r], starts[r + 1], t,
                     out);
      }
    }
    free(e);
    free(starts);
  }
  layout_free(&L);
  return rc;
}

/* Gradient of the loss with respect to every per-sample weight (the pages
 * take per-sample weights in the forward: kimbodo.com/?p=28372, "What
 * Happened").  The forward is linear in p_i,
 * Y[b, doff_t + d] = s_k * sum_i p_i * W_t[x_i, d], so
 * dL/dp_i = s_k * sum_d G[b, doff_t + d] * W_t[x_i, d].
 * grad_psw: fp64 [num_indices]. */
int tbe_oracle_psw_grad(int32_t T, const int64_t* rows, const int32_t* dims, int32_t dtype,
                        int32_t pooling, const void* weights, int64_t B, const int64_t* indices,
                        const int64_t* offsets, int64_t num_indices, const float* grad_output,
                        double* grad_psw) {
  layout_t L;
  int rc = layout_init(&L, T, rows, dims);
  if (rc == 0 && (!weights || (num_indices > 0 && (!grad_psw || !grad_output)))) rc = -1;
  if (rc == 0) rc = check_batch(&L, B, indices, offsets, num_indices);
  if (rc == 0) {
    const int64_t nbags = (int64_t)T * B;
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t k = 0; k < nbags; ++k) {
      const int64_t t = k / B, b = k % B;
      const int64_t D = dims[t];
      const int64_t begin = offsets[k], end = offsets[k + 1];
      const double s = (pooling == ORACLE_POOL_MEAN && end > begin) ? 1.0 / (double)(end - begin)
                                                                     : 1.0;
      const float* g = grad_output + b * L.sum_dims + L.doff[t];
      for (int64_t i = begin; i < end; ++i) {
        const int64_t row = L.woff[t] + indices[i] * D;
        double dot = 0.0;
        for (int64_t d = 0; d < D; ++d)
          dot += (double)g[d] * tbe_oracle_widen(dtype, load_bits(dtype, weights, row + d));
        grad_psw[i] = s * dot;
      }
    }
  }
  layout_free(&L);
  return rc;
}

static int is_selected(int64_t key, int64_t n, const int64_t* sel) {
  int64_t lo = 0, hi = n;
  while (lo < hi) {
    const int64_t mid = lo + (hi - lo) / 2;
    if (sel[mid] < key)
      lo = mid + 1;
    else
      hi = mid;
  }
  return lo < n && sel[lo] == key;
}

int tbe_oracle_backward_update(int32_t T, const int64_t* rows, const int32_t* dims,
                               int32_t dtype, int32_t pooling, int32_t optimizer, void* weights,
                               float* state, int64_t B, const int64_t* indices,
                               const int64_t* offsets, int64_t num_indices, const float* psw,
                               const float* grad_output, double lr, double eps,
                               int64_t num_selected, const int64_t* selected_rows) {
  layout_t L;
  int rc = layout_init(&L, T, rows, dims);
  if (rc == 0 && (!weights || (B > 0 && !grad_output))) rc = -1;
  if (rc == 0 && optimizer == ORACLE_OPT_ROWWISE_ADAGRAD && !state) rc = -1;
  if (rc == 0 && optimizer != ORACLE_OPT_SGD && optimizer != ORACLE_OPT_ROWWISE_ADAGRAD) rc = -1;
  if (rc == 0 && num_selected > 0 && !selected_rows) rc = -1;
  if (rc == 0) rc = check_batch(&L, B, indices, offsets, num_indices);
  if (rc == 0) {
    int32_t dmax = 0;
    for (int32_t t = 0; t < T; ++t)
      if (dims[t] > dmax) dmax = dims[t];
    entry_t* e = sorted_entries(&L, B, indices, offsets, num_indices);
    int64_t* starts = (int64_t*)malloc(sizeof(int64_t) * (size_t)(num_indices + 1));
    if (!e || !starts) {
      rc = -2;
    } else {
      const int64_t U = run_starts(e, num_indices, starts);
#pragma omp parallel
      {
        double* gamma = (double*)malloc(sizeof(double) * (size_t)dmax);
#pragma omp for schedule(dynamic, 16)
        for (int64_t r = 0; r < U; ++r) {
          const int64_t key = e[starts[r]].key;
          if (num_selected > 0 && !is_selected(key, num_selected, selected_rows)) continue;
          const int32_t t = table_of_key(&L, key);
          const int64_t D = dims[t];
          run_gradient(&L, pooling, B, offsets, psw, grad_output, e, starts[r], starts[r + 1], t,
                       gamma);
          const int64_t row = L.woff[t] + (key - L.roff[t]) * D;
          acc_t step = (acc_t)lr; /* SGD: W <- W - lr * Gamma */
          if (optimizer == ORACLE_OPT_ROWWISE_ADAGRAD) {
            acc_t sq = 0;
            for (int64_t d = 0; d < D; ++d) sq += (acc_t)gamma[d] * (acc_t)gamma[d];
            const acc_t m = (acc_t)state[key] + sq / (acc_t)D;
            state[key] = (float)m;
            step = (acc_t)lr / ((acc_t)sqrt((double)m) + (acc_t)eps);
          }
          for (int64_t d = 0; d < D; ++d) {
            const acc_t w = (acc_t)tbe_oracle_widen(dtype, load_bits(dtype, weights, row + d));
            const acc_t w_new = w - step * (acc_t)gamma[d];
            store_bits(dtype, weights, row + d, tbe_oracle_narrow(dtype, (double)w_new));
          }
        }
        free(gamma);
      }
    }
    free(e);
    free(starts);
  }
  layout_free(&L);
  return rc;
}

void tbe_oracle_set_threads(int32_t n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

int32_t tbe_oracle_get_threads(void) {
#ifdef _OPENMP
  return (int32_t)omp_get_max_threads();
#else
  return 1;
#endif
}
