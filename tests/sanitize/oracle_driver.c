/*
 * Runs every entry point of the fp64 oracle (oracle/moda_oracle.c) on small
 * shapes in all three input encodings, built with AddressSanitizer and
 * UndefinedBehaviorSanitizer, to catch out-of-bounds reads and writes and
 * undefined behaviour in the oracle itself.  Beside the sanitizers it checks
 * cheap consistency facts that hold whatever the arithmetic is:
 *   - the rows entry point reproduces the full forward's rows;
 *   - one row's explicit weights sum to 1 and rebuild its output;
 *   - the row-restricted backward's dQ equals the full backward's;
 *   - every output is finite; bad shapes are refused.
 * Exit status 0 when all hold.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_moda_fwd(int64_t B, int64_t Hq, int64_t Hkv, int64_t T, int64_t L, int64_t d,
                    int dtype, const void *q, const void *k, const void *v, const void *kd,
                    const void *vd, double *out, double *lse);
int oracle_moda_rows(int64_t R, const int64_t *rows, int64_t B, int64_t Hq, int64_t Hkv,
                     int64_t T, int64_t L, int64_t d, int dtype, const void *q_rows,
                     const void *k, const void *v, const void *kd_rows, const void *vd_rows,
                     double *out, double *lse);
int oracle_moda_row_weights(int64_t B, int64_t Hq, int64_t Hkv, int64_t T, int64_t L,
                            int64_t d, int dtype, int64_t b, int64_t h, int64_t t,
                            const void *q, const void *k, const void *v, const void *kd,
                            const void *vd, double *out_row, double *p_out);
int oracle_depth_fwd(int64_t B, int64_t Hq, int64_t Hkv, int64_t T, int64_t L, int64_t d,
                     int dtype, const void *q, const void *kd, const void *vd, double *out,
                     double *lse);
int oracle_moda_bwd(int64_t B, int64_t Hq, int64_t Hkv, int64_t T, int64_t L, int64_t d,
                    int dtype, const void *q, const void *k, const void *v, const void *kd,
                    const void *vd, const void *dout, double *dq, double *dk, double *dv,
                    double *dkd, double *dvd);
int oracle_moda_bwd_rows(int64_t R, const int64_t *rows, int64_t B, int64_t Hq, int64_t Hkv,
                         int64_t T, int64_t L, int64_t d, int dtype, const void *q_rows,
                         const void *dout_rows, const void *k, const void *v,
                         const void *kd_rows, const void *vd_rows, double *dq_rows, double *p,
                         double *ds);

static int g_fail = 0;
#define EXPECT(c, msg)                                   \
  do {                                                   \
    if (!(c)) {                                          \
      fprintf(stderr, "FAIL: %s (line %d)\n", msg, __LINE__); \
      ++g_fail;                                          \
    }                                                    \
  } while (0)

static uint64_t g_rng = 88172645463325252ull;
static double uniform(void) { /* xorshift64, in [-1, 1) */
  g_rng ^= g_rng << 13;
  g_rng ^= g_rng >> 7;
  g_rng ^= g_rng << 17;
  return (double)(g_rng >> 11) / 4503599627370496.0 - 1.0;
}

/* n elements of the given encoding (0 f32, 1 bf16 bits, 2 f64), exact sizes */
static void *fill(int64_t n, int dtype) {
  const size_t es = dtype == 0 ? 4 : dtype == 1 ? 2 : 8;
  void *p = malloc((size_t)(n > 0 ? n : 1) * es);
  for (int64_t i = 0; i < n; ++i) {
    const double x = 2.0 * uniform();
    if (dtype == 0) ((float *)p)[i] = (float)x;
    else if (dtype == 2) ((double *)p)[i] = x;
    else {
      float f = (float)x;
      uint32_t u;
      memcpy(&u, &f, 4);
      ((uint16_t *)p)[i] = (uint16_t)(u >> 16);
    }
  }
  return p;
}

static size_t esz(int dtype) { return dtype == 0 ? 4 : dtype == 1 ? 2 : 8; }

static int finite_all(const double *x, int64_t n) {
  for (int64_t i = 0; i < n; ++i)
    if (!isfinite(x[i])) return 0;
  return 1;
}

static void run_case(int64_t B, int64_t Hq, int64_t Hkv, int64_t T, int64_t L, int64_t d,
                     int dt) {
  const int64_t G = Hq / Hkv;
  const int64_t nq = B * Hq * T * d, nk = B * Hkv * T * d, nd = B * Hkv * T * L * d;
  void *q = fill(nq, dt), *k = fill(nk, dt), *v = fill(nk, dt);
  void *kd = fill(nd, dt), *vd = fill(nd, dt), *dout = fill(nq, dt);
  double *o = malloc((size_t)nq * 8), *lse = malloc((size_t)(B * Hq * T) * 8);
  EXPECT(oracle_moda_fwd(B, Hq, Hkv, T, L, d, dt, q, k, v, L ? kd : NULL, L ? vd : NULL, o,
                         lse) == 0, "forward");
  EXPECT(finite_all(o, nq) && finite_all(lse, B * Hq * T), "forward finite");

  /* every row through the rows entry point */
  const int64_t R = B * Hq * T;
  int64_t *rows = malloc((size_t)R * 3 * 8);
  void *qr = malloc((size_t)(R * d) * esz(dt));
  void *kdr = malloc((size_t)(R * L * d + 1) * esz(dt)), *vdr = malloc((size_t)(R * L * d + 1) * esz(dt));
  void *dor = malloc((size_t)(R * d) * esz(dt));
  int64_t r = 0;
  for (int64_t b = 0; b < B; ++b)
    for (int64_t h = 0; h < Hq; ++h)
      for (int64_t t = 0; t < T; ++t, ++r) {
        rows[3 * r] = b, rows[3 * r + 1] = h, rows[3 * r + 2] = t;
        memcpy((char *)qr + r * d * esz(dt), (char *)q + ((b * Hq + h) * T + t) * d * esz(dt),
               (size_t)d * esz(dt));
        memcpy((char *)dor + r * d * esz(dt),
               (char *)dout + ((b * Hq + h) * T + t) * d * esz(dt), (size_t)d * esz(dt));
        if (L) {
          const int64_t src = ((b * Hkv + h / G) * T + t) * L * d;
          memcpy((char *)kdr + r * L * d * esz(dt), (char *)kd + src * esz(dt),
                 (size_t)(L * d) * esz(dt));
          memcpy((char *)vdr + r * L * d * esz(dt), (char *)vd + src * esz(dt),
                 (size_t)(L * d) * esz(dt));
        }
      }
  double *o2 = malloc((size_t)nq * 8), *lse2 = malloc((size_t)R * 8);
  EXPECT(oracle_moda_rows(R, rows, B, Hq, Hkv, T, L, d, dt, qr, k, v, L ? kdr : NULL,
                          L ? vdr : NULL, o2, lse2) == 0, "rows");
  double e = 0;
  for (int64_t i = 0; i < nq; ++i) e = fmax(e, fabs(o[i] - o2[i]));
  for (int64_t i = 0; i < R; ++i) e = fmax(e, fabs(lse[i] - lse2[i]));
  EXPECT(e <= 1e-12, "rows reproduce the full forward");

  /* explicit weights of the last row of the last head */
  double *orow = malloc((size_t)d * 8), *p = malloc((size_t)(T + L) * 8);
  EXPECT(oracle_moda_row_weights(B, Hq, Hkv, T, L, d, dt, B - 1, Hq - 1, T - 1, q, k, v,
                                 L ? kd : NULL, L ? vd : NULL, orow, p) == 0, "row weights");
  double sum = 0;
  for (int64_t n = 0; n < T + L; ++n) sum += p[n];
  EXPECT(fabs(sum - 1.0) <= 1e-12, "weights sum to 1");
  e = 0;
  for (int64_t c = 0; c < d; ++c) e = fmax(e, fabs(orow[c] - o[((B * Hq - 1) * T + T - 1) * d + c]));
  EXPECT(e <= 1e-12, "weights' row equals the forward's");

  if (L) {
    double *od = malloc((size_t)nq * 8), *ld = malloc((size_t)(B * Hq * T) * 8);
    EXPECT(oracle_depth_fwd(B, Hq, Hkv, T, L, d, dt, q, kd, vd, od, ld) == 0, "depth alone");
    EXPECT(finite_all(od, nq) && finite_all(ld, B * Hq * T), "depth alone finite");
    free(od);
    free(ld);
  }

  /* backward, full and row-restricted */
  double *dq = malloc((size_t)nq * 8), *dk = malloc((size_t)nk * 8), *dv = malloc((size_t)nk * 8);
  double *dkd = malloc((size_t)(nd + 1) * 8), *dvd = malloc((size_t)(nd + 1) * 8);
  EXPECT(oracle_moda_bwd(B, Hq, Hkv, T, L, d, dt, q, k, v, L ? kd : NULL, L ? vd : NULL, dout,
                         dq, dk, dv, L ? dkd : NULL, L ? dvd : NULL) == 0, "backward");
  EXPECT(finite_all(dq, nq) && finite_all(dk, nk) && finite_all(dv, nk) &&
             finite_all(dkd, nd) && finite_all(dvd, nd), "backward finite");
  double *dq2 = malloc((size_t)nq * 8), *pw = malloc((size_t)(R * (T + L)) * 8);
  double *ds = malloc((size_t)(R * (T + L)) * 8);
  EXPECT(oracle_moda_bwd_rows(R, rows, B, Hq, Hkv, T, L, d, dt, qr, dor, k, v, L ? kdr : NULL,
                              L ? vdr : NULL, dq2, pw, ds) == 0, "backward rows");
  e = 0;
  for (int64_t i = 0; i < nq; ++i) e = fmax(e, fabs(dq[i] - dq2[i]));
  EXPECT(e <= 1e-10, "row-restricted dQ equals the full backward's");

  /* refused shapes */
  EXPECT(oracle_moda_fwd(B, Hq, Hq + 1, T, L, d, dt, q, k, v, kd, vd, o, lse) != 0,
         "Hq not a multiple of Hkv refused");
  EXPECT(oracle_moda_fwd(B, Hq, Hkv, T, L, d, 7, q, k, v, kd, vd, o, lse) != 0,
         "unknown dtype refused");
  const int64_t badrow[3] = {0, 0, T};
  EXPECT(oracle_moda_rows(1, badrow, B, Hq, Hkv, T, L, d, dt, qr, k, v, kdr, vdr, o2, lse2) != 0,
         "row past T refused");

  free(q), free(k), free(v), free(kd), free(vd), free(dout), free(o), free(lse), free(rows);
  free(qr), free(kdr), free(vdr), free(dor), free(o2), free(lse2), free(orow), free(p);
  free(dq), free(dk), free(dv), free(dkd), free(dvd), free(dq2), free(pw), free(ds);
}

int main(void) {
  for (int dt = 0; dt < 3; ++dt) {
    run_case(1, 2, 1, 9, 4, 8, dt);   /* G = 2 */
    run_case(2, 6, 2, 5, 0, 4, dt);   /* L = 0, G = 3 */
    run_case(1, 4, 4, 1, 7, 3, dt);   /* T = 1, MHA, odd d */
    run_case(1, 8, 1, 13, 1, 16, dt); /* G = 8, one depth entry */
  }
  if (g_fail) {
    fprintf(stderr, "%d expectation(s) failed\n", g_fail);
    return 1;
  }
  printf("oracle driver: all expectations hold\n");
  return 0;
}
