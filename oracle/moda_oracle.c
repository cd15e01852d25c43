/*
 * MoDA forward oracle: plain, slow, fp64 CPU reference.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: it is used by tests/, by the smoke check and by the bench's
 * cpu_baseline leg, and by nothing else.  It shares no code, header or table
 * with the HIP library.
 *
 * What it computes (Mixture-of-Depths Attention, forward):
 *   hyper.ai summary of arXiv 2603.15619, section "Mixture-of-Depths Attention
 *   (MoDA)": every token attends at the same time to the sequence-level keys
 *   and values of the current layer and to its own depth keys and values from
 *   the preceding layers, and all of these attention scores are normalised
 *   together (one softmax).
 *   Same page, section "Depth stream mechanism": the depth set of a token at
 *   layer l is {K_i, V_i}, i = 0..l-1, taken at the same token position.
 *   shijienb.com article, "second half" section: one unified softmax, every
 *   head sees the current layer's sequence KV and the depth KV of all earlier
 *   layers.
 *   chatpaper.ai abstract (English): sequence KV pairs of the current layer
 *   and depth KV pairs of the preceding layers.
 *
 * The pages fix no scale and print no formula that survived extraction; the
 * scale is 1/sqrt(d) for both kinds of logit, the causal set is keys 0..t
 * (diagonal included), and query head h reads KV head floor(h / G) with
 * G = Hq / Hkv (grouped-query attention: G query heads share one KV head).
 *
 * The method (the same page, section "Hardware-efficient implementation")
 * folds sequence and depth logits into one online-softmax state before a
 * single normalisation.  That is an exact reformulation of the plain
 * definition, so this oracle is the plain definition written out, step by
 * step, for one query row at a time:
 *   1. a_j = s * <q_t, K_j>                for j = 0..t      (sequence logits)
 *   2. c_i = s * <q_t, Kd_{t,i}>           for i = 0..L-1    (depth logits)
 *   3. x   = [a_0 .. a_t, c_0 .. c_{L-1}]  (explicit list, length t+1+L)
 *   4. m = max x ; w_n = exp(x_n - m) ; Z = sum w ; p_n = w_n / Z
 *   5. o_t = sum_j p_j V_j + sum_i p_{t+1+i} Vd_{t,i}
 *   6. lse = m + ln Z
 * All arithmetic is in double.  Inputs are read exactly (fp32, bf16 or fp64
 * element values all convert to double without rounding).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_F32 0
#define ORACLE_BF16 1
#define ORACLE_F64 2

/* One input element as an exact double. bf16 is the upper half of an IEEE
 * binary32 word, so widening it is a 16-bit shift. */
static double elem(const void *base, int64_t idx, int dtype) {
  if (dtype == ORACLE_F32) return (double)((const float *)base)[idx];
  if (dtype == ORACLE_F64) return ((const double *)base)[idx];
  uint32_t bits = (uint32_t)((const uint16_t *)base)[idx] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

static double dot(const void *a, int64_t ia, const void *b, int64_t ib,
                  int64_t d, int dtype) {
  double acc = 0.0;
  for (int64_t k = 0; k < d; ++k) acc += elem(a, ia + k, dtype) * elem(b, ib + k, dtype);
  return acc;
}

/*
 * One query row.  Element offsets (not bytes) locate the operands:
 *   q    + q_off            : d values of the query row
 *   k, v + kv_off           : the KV head's sequence rows, row j at + j*d
 *   kd, vd + dep_off        : the token's L depth rows, row i at + i*d
 * x (scratch) holds t+1+L doubles.  If p_out is not NULL the normalised
 * weights p_0..p_{t+L} are written there (same order as x).
 */
static void moda_row(int64_t t, int64_t L, int64_t d, int dtype,
                     const void *q, int64_t q_off,
                     const void *k, const void *v, int64_t kv_off,
                     const void *kd, const void *vd, int64_t dep_off,
                     double *out, double *lse, double *x, double *p_out) {
  const double s = 1.0 / sqrt((double)d);
  const int64_t n = t + 1 + L;

  /* steps 1-3: the explicit score list */
  for (int64_t j = 0; j <= t; ++j)
    x[j] = s * dot(q, q_off, k, kv_off + j * d, d, dtype);
  for (int64_t i = 0; i < L; ++i)
    x[t + 1 + i] = s * dot(q, q_off, kd, dep_off + i * d, d, dtype);

  /* step 4: one softmax over the whole list */
  double m = x[0];
  for (int64_t nn = 1; nn < n; ++nn) m = x[nn] > m ? x[nn] : m;
  double Z = 0.0;
  for (int64_t nn = 0; nn < n; ++nn) {
    x[nn] = exp(x[nn] - m);
    Z += x[nn];
  }
  for (int64_t nn = 0; nn < n; ++nn) x[nn] /= Z;
  if (p_out) memcpy(p_out, x, (size_t)n * sizeof(double));

  /* step 5: weighted sum of the matching values */
  for (int64_t c = 0; c < d; ++c) {
    double acc = 0.0;
    for (int64_t j = 0; j <= t; ++j) acc += x[j] * elem(v, kv_off + j * d + c, dtype);
    for (int64_t i = 0; i < L; ++i) acc += x[t + 1 + i] * elem(vd, dep_off + i * d + c, dtype);
    out[c] = acc;
  }
  /* step 6 */
  if (lse) *lse = m + log(Z);
}

static int bad_shape(int64_t B, int64_t Hq, int64_t Hkv, int64_t T, int64_t L,
                     int64_t d, int dtype) {
  if (B < 1 || Hq < 1 || Hkv < 1 || T < 1 || L < 0 || d < 1) return 1;
  if (Hq % Hkv != 0) return 1;
  if (dtype != ORACLE_F32 && dtype != ORACLE_BF16 && dtype != ORACLE_F64) return 1;
  return 0;
}

/*
 * Full forward over every (b, h, t).
 *   q  [B,Hq,T,d]   k, v [B,Hkv,T,d]   kd, vd [B,Hkv,T,L,d]  (may be NULL if L == 0)
 *   out [B,Hq,T,d] double;  lse [B,Hq,T] double (may be NULL)
 * Returns 0 on success, nonzero on a bad shape or an allocation failure.
 */
int oracle_moda_fwd(int64_t B, int64_t Hq, int64_t Hkv, int64_t T, int64_t L,
                    int64_t d, int dtype, const void *q, const void *k,
                    const void *v, const void *kd, const void *vd, double *out,
                    double *lse) {
  if (bad_shape(B, Hq, Hkv, T, L, d, dtype)) return 1;
  const int64_t G = Hq / Hkv;
  const int64_t rows = B * Hq * T;
  int fail = 0;
#pragma omp parallel
  {
    double *x = (double *)malloc((size_t)(T + L) * sizeof(double));
    if (!x) {
#pragma omp atomic write
      fail = 1;
    } else {
#pragma omp for schedule(dynamic, 16)
      for (int64_t r = 0; r < rows; ++r) {
        const int64_t t = r % T, h = (r / T) % Hq, b = r / (T * Hq);
        const int64_t g = h / G;
        moda_row(t, L, d, dtype, q, r * d, k, v, (b * Hkv + g) * T * d, kd, vd,
                 ((b * Hkv + g) * T + t) * L * d, out + r * d,
                 lse ? lse + r : NULL, x, NULL);
      }
      free(x);
    }
  }
  return fail ? 2 : 0;
}

/*
 * Selected rows only (for shapes whose full forward would take too long).
 *   rows    [R,3] int64: (b, h, t) of each row
 *   q_rows  [R,d]       : the query row of each selected row
 *   k, v    [B,Hkv,T,d] : full sequence keys and values
 *   kd_rows, vd_rows [R,L,d]: the depth rows of each selected row's token
 *   out [R,d] double, lse [R] double (may be NULL)
 */
int oracle_moda_rows(int64_t R, const int64_t *rows, int64_t B, int64_t Hq,
                     int64_t Hkv, int64_t T, int64_t L, int64_t d, int dtype,
                     const void *q_rows, const void *k, const void *v,
                     const void *kd_rows, const void *vd_rows, double *out,
                     double *lse) {
  if (bad_shape(B, Hq, Hkv, T, L, d, dtype) || R < 0) return 1;
  for (int64_t r = 0; r < R; ++r) {
    const int64_t b = rows[3 * r], h = rows[3 * r + 1], t = rows[3 * r + 2];
    if (b < 0 || b >= B || h < 0 || h >= Hq || t < 0 || t >= T) return 1;
  }
  const int64_t G = Hq / Hkv;
  int fail = 0;
#pragma omp parallel
  {
    double *x = (double *)malloc((size_t)(T + L) * sizeof(double));
    if (!x) {
#pragma omp atomic write
      fail = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t r = 0; r < R; ++r) {
        const int64_t b = rows[3 * r], h = rows[3 * r + 1], t = rows[3 * r + 2];
        const int64_t g = h / G;
        moda_row(t, L, d, dtype, q_rows, r * d, k, v, (b * Hkv + g) * T * d,
                 kd_rows, vd_rows, r * L * d, out + r * d, lse ? lse + r : NULL,
                 x, NULL);
      }
      free(x);
    }
  }
  return fail ? 2 : 0;
}

/*
 * The explicit normalised weights of one row (b, h, t) of a full problem:
 * p_out receives t+1+L doubles, sequence keys 0..t first, then depth 0..L-1.
 */
int oracle_moda_row_weights(int64_t B, int64_t Hq, int64_t Hkv, int64_t T,
                            int64_t L, int64_t d, int dtype, int64_t b,
                            int64_t h, int64_t t, const void *q, const void *k,
                            const void *v, const void *kd, const void *vd,
                            double *out_row, double *p_out) {
  if (bad_shape(B, Hq, Hkv, T, L, d, dtype)) return 1;
  if (b < 0 || b >= B || h < 0 || h >= Hq || t < 0 || t >= T) return 1;
  const int64_t g = h / (Hq / Hkv);
  double *x = (double *)malloc((size_t)(T + L) * sizeof(double));
  if (!x) return 2;
  moda_row(t, L, d, dtype, q, ((b * Hq + h) * T + t) * d, k, v,
           (b * Hkv + g) * T * d, kd, vd, ((b * Hkv + g) * T + t) * L * d,
           out_row, NULL, x, p_out);
  free(x);
  return 0;
}

/* Threads the OpenMP runtime will use for the parallel loops above. */
int oracle_num_threads(void) {
  int n = 1;
#pragma omp parallel
  {
#pragma omp single
    {
#ifdef _OPENMP
      extern int omp_get_num_threads(void);
      n = omp_get_num_threads();
#endif
    }
  }
  return n;
}

/*
 * Depth attention alone: the read step of the depth stream (hyper.ai summary
 * of arXiv 2603.15619, section "Depth stream mechanism": the input of layer l
 * comes from attention over the keys and values {K_i, V_i}, i = 0..l-1, that
 * the preceding layers left at the same token position).  The query row of
 * token t attends over its own token's L depth entries and nothing else,
 * under one softmax scaled by 1/sqrt(d):
 *   1. c_i = sd * <q_t, Kd_{t,i}>          for i = 0..L-1
 *   2. mx = max c ; w_i = exp(c_i - mx) ; Zd = sum w ; p_i = w_i / Zd
 *   3. o_t = sum_i p_i Vd_{t,i} ;  lse = mx + ln Zd
 *   q [B,Hq,T,d]  kd, vd [B,Hkv,T,L,d] (L >= 1)
 *   out [B,Hq,T,d] double;  lse [B,Hq,T] double (may be NULL)
 * Returns 0 on success, nonzero on a bad shape or an allocation failure.
 */
int oracle_depth_fwd(int64_t B, int64_t Hq, int64_t Hkv, int64_t T, int64_t L,
                     int64_t d, int dtype, const void *q, const void *kd,
                     const void *vd, double *out, double *lse) {
  if (bad_shape(B, Hq, Hkv, T, L, d, dtype) || L < 1) return 1;
  const int64_t grp = Hq / Hkv;
  const int64_t nrows = B * Hq * T;
  const double sd = 1.0 / sqrt((double)d);
  int failed = 0;
#pragma omp parallel
  {
    double *c = (double *)malloc((size_t)L * sizeof(double));
    if (!c) {
#pragma omp atomic write
      failed = 1;
    } else {
#pragma omp for schedule(dynamic, 16)
      for (int64_t r = 0; r < nrows; ++r) {
        const int64_t t = r % T, h = (r / T) % Hq, b = r / (T * Hq);
        const int64_t own = ((b * Hkv + h / grp) * T + t) * L * d;  /* token t's entries */
        for (int64_t i = 0; i < L; ++i) c[i] = sd * dot(q, r * d, kd, own + i * d, d, dtype);
        double mx = c[0];
        for (int64_t i = 1; i < L; ++i) mx = c[i] > mx ? c[i] : mx;
        double Zd = 0.0;
        for (int64_t i = 0; i < L; ++i) {
          c[i] = exp(c[i] - mx);
          Zd += c[i];
        }
        for (int64_t col = 0; col < d; ++col) {
          double acc = 0.0;
          for (int64_t i = 0; i < L; ++i) acc += (c[i] / Zd) * elem(vd, own + i * d + col, dtype);
          out[r * d + col] = acc;
        }
        if (lse) lse[r] = mx + log(Zd);
      }
      free(c);
    }
  }
  return failed ? 2 : 0;
}

/*
 * MoDA backward: gradients of a scalar loss through the forward above, given
 * the loss's gradient dO with respect to the output.  Calculus on the plain
 * definition (the forward's steps 1-6), one query row at a time:
 *   7. recompute the explicit list x, the weights p and o_t as in steps 1-5
 *   8. D = <dO_t, o_t>
 *   9. dp_n = <dO_t, value_n>   for every entry n of the list
 *  10. ds_n = p_n * (dp_n - D)  (gradient through the softmax)
 *  11. dq_t      = s * sum_n ds_n key_n
 *      dK_j     += s * ds_j q_t ;  dV_j     += p_j dO_t          (j = 0..t)
 *      dKd_{t,i}+= s * ds_{t+1+i} q_t ; dVd_{t,i} += p_{t+1+i} dO_t
 * The sums over query rows run over every row that reads the entry: the G
 * query heads of the KV group and, for sequence keys, every token t >= j.
 *   dout [B,Hq,T,d] in the input element type
 *   dq [B,Hq,T,d]; dk, dv [B,Hkv,T,d]; dkd, dvd [B,Hkv,T,L,d] (NULL if L == 0),
 *   all double, fully written.
 * Returns 0 on success, nonzero on a bad shape or an allocation failure.
 */
int oracle_moda_bwd(int64_t B, int64_t Hq, int64_t Hkv, int64_t T, int64_t L,
                    int64_t d, int dtype, const void *q, const void *k,
                    const void *v, const void *kd, const void *vd,
                    const void *dout, double *dq, double *dk, double *dv,
                    double *dkd, double *dvd) {
  if (bad_shape(B, Hq, Hkv, T, L, d, dtype)) return 1;
  const int64_t G = Hq / Hkv;
  const double s = 1.0 / sqrt((double)d);
  memset(dk, 0, (size_t)(B * Hkv * T * d) * sizeof(double));
  memset(dv, 0, (size_t)(B * Hkv * T * d) * sizeof(double));
  if (L > 0) {
    memset(dkd, 0, (size_t)(B * Hkv * T * L * d) * sizeof(double));
    memset(dvd, 0, (size_t)(B * Hkv * T * L * d) * sizeof(double));
  }
  int fail = 0;
  /* one (b, kv head) per iteration: it owns its dK, dV, dKd, dVd */
#pragma omp parallel
  {
    double *x = (double *)malloc((size_t)(T + L) * sizeof(double));
    double *o = (double *)malloc((size_t)d * sizeof(double));
    if (!x || !o) {
#pragma omp atomic write
      fail = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t bg = 0; bg < B * Hkv; ++bg) {
        const int64_t kv_off = bg * T * d;
        for (int64_t h = (bg % Hkv) * G; h < (bg % Hkv + 1) * G; ++h) {
          for (int64_t t = 0; t < T; ++t) {
            const int64_t r = ((bg / Hkv) * Hq + h) * T + t; /* query row */
            const int64_t dep_off = (bg * T + t) * L * d;
            const int64_t n = t + 1 + L;
            /* step 7: weights p (in x) and o_t, as in the forward */
            moda_row(t, L, d, dtype, q, r * d, k, v, kv_off, kd, vd, dep_off, o, NULL, x, NULL);
            /* step 8 */
            double D = 0.0;
            for (int64_t c = 0; c < d; ++c) D += elem(dout, r * d + c, dtype) * o[c];
            for (int64_t c = 0; c < d; ++c) dq[r * d + c] = 0.0;
            for (int64_t nn = 0; nn < n; ++nn) {
              const int is_seq = nn <= t;
              const void *key = is_seq ? k : kd, *val = is_seq ? v : vd;
              const int64_t off = is_seq ? kv_off + nn * d : dep_off + (nn - t - 1) * d;
              /* steps 9 and 10 */
              const double dp = dot(dout, r * d, val, off, d, dtype);
              const double ds = x[nn] * (dp - D);
              /* step 11 */
              double *dkey = is_seq ? dk + off : dkd + off;
              double *dval = is_seq ? dv + off : dvd + off;
              for (int64_t c = 0; c < d; ++c) {
                dq[r * d + c] += s * ds * elem(key, off + c, dtype);
                dkey[c] += s * ds * elem(q, r * d + c, dtype);
                dval[c] += x[nn] * elem(dout, r * d + c, dtype);
              }
            }
          }
        }
      }
    }
    free(x);
    free(o);
  }
  return fail ? 2 : 0;
}

/*
 * The backward's per-row steps 7-10 and the dq_t of step 11 for selected rows
 * only (the same calculus as oracle_moda_bwd, restricted to rows, for checks
 * of large problems one row at a time).  The sums of step 11 over the rows
 * that read a key are left to the caller, which gets each row's weights and
 * ds over the entries it reads:
 *   rows [R,3] (b, h, t); q_rows, dout_rows [R,d] in the input element type;
 *   k, v [B,Hkv,T,d] full; kd_rows, vd_rows [R,L,d] (the row's token's depth
 *   rows; NULL if L == 0)
 *   dq_rows [R,d] double;
 *   p, ds [R, T+L] double: entry n of row r at r*(T+L) + n, sequence keys
 *   0..t first, then depth 0..L-1 at t+1+i; the rest of the row is zero.
 */
int oracle_moda_bwd_rows(int64_t R, const int64_t *rows, int64_t B, int64_t Hq,
                         int64_t Hkv, int64_t T, int64_t L, int64_t d, int dtype,
                         const void *q_rows, const void *dout_rows, const void *k,
                         const void *v, const void *kd_rows, const void *vd_rows,
                         double *dq_rows, double *p, double *ds) {
  if (bad_shape(B, Hq, Hkv, T, L, d, dtype) || R < 0) return 1;
  for (int64_t r = 0; r < R; ++r) {
    const int64_t b = rows[3 * r], h = rows[3 * r + 1], t = rows[3 * r + 2];
    if (b < 0 || b >= B || h < 0 || h >= Hq || t < 0 || t >= T) return 1;
  }
  const int64_t G = Hq / Hkv;
  const int64_t W = T + L;
  const double s = 1.0 / sqrt((double)d);
  int fail = 0;
#pragma omp parallel
  {
    double *x = (double *)malloc((size_t)W * sizeof(double));
    double *o = (double *)malloc((size_t)d * sizeof(double));
    if (!x || !o) {
#pragma omp atomic write
      fail = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t r = 0; r < R; ++r) {
        const int64_t b = rows[3 * r], h = rows[3 * r + 1], t = rows[3 * r + 2];
        const int64_t kv_off = (b * Hkv + h / G) * T * d;
        const int64_t dep_off = r * L * d;
        const int64_t n = t + 1 + L;
        double *pr = p + r * W, *dsr = ds + r * W, *dqr = dq_rows + r * d;
        /* step 7 */
        moda_row(t, L, d, dtype, q_rows, r * d, k, v, kv_off, kd_rows, vd_rows, dep_off, o,
                 NULL, x, NULL);
        /* step 8 */
        double D = 0.0;
        for (int64_t c = 0; c < d; ++c) D += elem(dout_rows, r * d + c, dtype) * o[c];
        for (int64_t c = 0; c < d; ++c) dqr[c] = 0.0;
        for (int64_t nn = 0; nn < W; ++nn) pr[nn] = dsr[nn] = 0.0;
        for (int64_t nn = 0; nn < n; ++nn) {
          const int is_seq = nn <= t;
          const void *key = is_seq ? k : kd_rows, *val = is_seq ? v : vd_rows;
          const int64_t off = is_seq ? kv_off + nn * d : dep_off + (nn - t - 1) * d;
          /* steps 9 and 10 */
          const double dp = dot(dout_rows, r * d, val, off, d, dtype);
          const double dsn = x[nn] * (dp - D);
          pr[nn] = x[nn];
          dsr[nn] = dsn;
          /* step 11, dq_t */
          for (int64_t c = 0; c < d; ++c) dqr[c] += s * dsn * elem(key, off + c, dtype);
        }
      }
    }
    free(x);
    free(o);
  }
  return fail ? 2 : 0;
}
