/* Runs every function of the oracle (oracle/oracle.c) on small seeded inputs,
 * built with AddressSanitizer and UndefinedBehaviorSanitizer: odd sizes, empty
 * sizes, optional inputs absent and present, several threads, the chunked
 * form.  Buffers are allocated at their exact sizes.  Besides the sanitizers'
 * own checks it asserts that every output is finite, that the thread count
 * does not change a result (bitwise) and that the chunked form agrees with the
 * sequential one.  Prints "oracle driver ok" and exits 0 on success. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_scan_fwd_from(const double*, const double*, const double*, const double*, const double*, const double*,
                         const double*, const double*, int, int, const double*, double*, double*, int64_t, int64_t,
                         int64_t, int64_t, int64_t, int);
int oracle_state_update(double*, const double*, const double*, const double*, const double*, const double*,
                        const double*, const double*, const double*, int, int, double*, int64_t, int64_t, int64_t);
void oracle_affine_compose(const double*, const double*, const double*, const double*, double*, double*, int64_t);
void oracle_step_size(const double*, const double*, int, double*, int64_t, int64_t);
int oracle_conv1d_fwd(const double*, const double*, const double*, int, const double*, double*, double*, int64_t,
                      int64_t, int64_t, int64_t);
int oracle_conv1d_update(double*, const double*, const double*, const double*, int, double*, int64_t, int64_t,
                         int64_t);
int oracle_scan_bwd(const double*, const double*, const double*, const double*, const double*, const double*,
                    const double*, const double*, int, const double*, const double*, const double*, double*, double*,
                    double*, double*, double*, double*, double*, double*, double*, int64_t, int64_t, int64_t, int64_t);
int oracle_ssd_fwd(const double*, const double*, const double*, const double*, const double*, const double*,
                   const double*, const double*, int, const double*, double*, double*, int64_t, int64_t, int64_t,
                   int64_t, int64_t, int64_t, int);
int oracle_ssd_state_update(double*, const double*, const double*, const double*, const double*, const double*,
                            const double*, const double*, const double*, int, double*, int64_t, int64_t, int64_t,
                            int64_t, int64_t);

static int failures = 0;
static uint64_t rng = 0x9e3779b97f4a7c15ull;

static double uni(void) { /* xorshift64*, uniform in [-1, 1) */
  rng ^= rng >> 12;
  rng ^= rng << 25;
  rng ^= rng >> 27;
  return (double)((rng * 0x2545f4914f6cdd1dull) >> 11) / 4503599627370496.0 - 1.0;
}

static double* arr(int64_t n, double lo, double hi) {
  double* p = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
  for (int64_t i = 0; i < n; ++i) p[i] = lo + (hi - lo) * 0.5 * (uni() + 1.0);
  return p;
}

static void check(const char* what, int cond) {
  if (!cond) {
    fprintf(stderr, "failed: %s\n", what);
    ++failures;
  }
}

static int finite(const double* p, int64_t n) {
  for (int64_t i = 0; i < n; ++i)
    if (!isfinite(p[i])) return 0;
  return 1;
}

static double maxdiff(const double* a, const double* b, int64_t n) {
  double m = 0;
  for (int64_t i = 0; i < n; ++i) m = fmax(m, fabs(a[i] - b[i]));
  return m;
}

static void scan_cases(int64_t b, int64_t L, int64_t d, int64_t N) {
  const int64_t n = b * L * d, r = b * L * N, st = b * d * N;
  double *x = arr(n, -1, 1), *dl = arr(n, -4, 1), *z = arr(n, -2, 2), *B = arr(r, -1, 1), *C = arr(r, -1, 1);
  double *A = arr(d * N, -3, -0.1), *D = arr(d, 0.5, 1.5), *bias = arr(d, -1, 0), *h0 = arr(st, -1, 1);
  double *y1 = arr(n, 0, 0), *y2 = arr(n, 0, 0), *y3 = arr(n, 0, 0);
  double *l1 = arr(st, 0, 0), *l2 = arr(st, 0, 0), *l3 = arr(st, 0, 0);
  for (int zoh = 0; zoh < 2; ++zoh) {
    check("scan 1 thread", oracle_scan_fwd_from(x, dl, A, B, C, D, z, bias, 1, zoh, h0, y1, l1, b, L, d, N, 0, 1) == 0);
    check("scan 3 threads", oracle_scan_fwd_from(x, dl, A, B, C, D, z, bias, 1, zoh, h0, y2, l2, b, L, d, N, 0, 3) == 0);
    check("scan chunked", oracle_scan_fwd_from(x, dl, A, B, C, D, z, bias, 1, zoh, h0, y3, l3, b, L, d, N, 5, 2) == 0);
    check("scan finite", finite(y1, n) && finite(l1, st));
    check("threads bitwise", memcmp(y1, y2, sizeof(double) * (size_t)n) == 0 &&
                                 memcmp(l1, l2, sizeof(double) * (size_t)st) == 0);
    check("chunked agrees", maxdiff(y1, y3, n) < 1e-10 && maxdiff(l1, l3, st) < 1e-10);
  }
  check("scan no options",
        oracle_scan_fwd_from(x, dl, A, B, C, NULL, NULL, NULL, 0, 0, NULL, y1, NULL, b, L, d, N, 0, 2) == 0);
  /* decode: L steps from h0 equal the scan from h0 */
  double* state = arr(st, 0, 0);
  memcpy(state, h0, sizeof(double) * (size_t)st);
  double *xs = arr(b * d, 0, 0), *ds = arr(b * d, 0, 0), *zs = arr(b * d, 0, 0), *ys = arr(b * d, 0, 0);
  double *Bs = arr(b * N, 0, 0), *Cs = arr(b * N, 0, 0);
  oracle_scan_fwd_from(x, dl, A, B, C, D, z, bias, 1, 0, h0, y1, l1, b, L, d, N, 0, 1);
  double dec_err = 0;
  for (int64_t t = 0; t < L; ++t) {
    for (int64_t i = 0; i < b; ++i) {
      memcpy(xs + i * d, x + (i * L + t) * d, sizeof(double) * (size_t)d);
      memcpy(ds + i * d, dl + (i * L + t) * d, sizeof(double) * (size_t)d);
      memcpy(zs + i * d, z + (i * L + t) * d, sizeof(double) * (size_t)d);
      memcpy(Bs + i * N, B + (i * L + t) * N, sizeof(double) * (size_t)N);
      memcpy(Cs + i * N, C + (i * L + t) * N, sizeof(double) * (size_t)N);
    }
    check("decode", oracle_state_update(state, xs, ds, A, Bs, Cs, D, zs, bias, 1, 0, ys, b, d, N) == 0);
    for (int64_t i = 0; i < b; ++i)
      for (int64_t c = 0; c < d; ++c) dec_err = fmax(dec_err, fabs(ys[i * d + c] - y1[(i * L + t) * d + c]));
  }
  check("decode equals the scan", dec_err == 0.0 && (L == 0 || maxdiff(state, l1, st) == 0.0));
  /* backward */
  double *dout = arr(n, -1, 1), *dlast = arr(st, -1, 1), *dx = arr(n, 0, 0), *ddl = arr(n, 0, 0), *dz = arr(n, 0, 0);
  double *dA = arr(d * N, 0, 0), *dB = arr(r, 0, 0), *dC = arr(r, 0, 0), *dD = arr(d, 0, 0), *db = arr(d, 0, 0);
  double* dh0 = arr(st, 0, 0);
  check("bwd", oracle_scan_bwd(x, dl, A, B, C, D, z, bias, 1, h0, dout, dlast, dx, ddl, dA, dB, dC, dD, dz, db, dh0,
                               b, L, d, N) == 0);
  check("bwd finite", finite(dx, n) && finite(ddl, n) && finite(dA, d * N) && finite(dB, r) && finite(dh0, st));
  check("bwd no options", oracle_scan_bwd(x, dl, A, B, C, NULL, NULL, NULL, 0, NULL, dout, NULL, dx, ddl, dA, dB, dC,
                                          NULL, NULL, NULL, NULL, b, L, d, N) == 0);
  double* ss = arr(n, 0, 0);
  oracle_step_size(dl, bias, 1, ss, b * L, d);
  check("step size positive", L == 0 || b == 0 || d == 0 || ss[0] > 0);
  double *a2 = arr(n, 0, 1), *b2 = arr(n, -1, 1), *oa = arr(n, 0, 0), *ob = arr(n, 0, 0);
  oracle_affine_compose(a2, b2, x, dl, oa, ob, n);
  check("compose finite", finite(oa, n) && finite(ob, n));
  double* ptrs[] = {x, dl, z, B, C, A, D, bias, h0, y1, y2, y3, l1, l2, l3, state, xs, ds, zs, ys, Bs, Cs, dout,
                    dlast, dx, ddl, dz, dA, dB, dC, dD, db, dh0, ss, a2, b2, oa, ob};
  for (size_t i = 0; i < sizeof(ptrs) / sizeof(ptrs[0]); ++i) free(ptrs[i]);
}

static void conv_cases(int64_t b, int64_t L, int64_t d, int64_t K) {
  const int64_t n = b * L * d, st = b * d * K;
  double *x = arr(n, -1, 1), *w = arr(d * K, -1, 1), *bias = arr(d, -1, 1), *si = arr(st, -1, 1);
  double *y = arr(n, 0, 0), *so = arr(st, 0, 0), *y1 = arr(b * d, 0, 0), *x1 = arr(b * d, -1, 1);
  check("conv", oracle_conv1d_fwd(x, w, bias, 1, si, y, so, b, L, d, K) == 0);
  check("conv no cache", oracle_conv1d_fwd(x, w, NULL, 0, NULL, y, NULL, b, L, d, K) == 0);
  check("conv update", oracle_conv1d_update(so, x1, w, bias, 1, y1, b, d, K) == 0);
  check("conv finite", finite(y, n) && finite(so, st) && finite(y1, b * d));
  double* ptrs[] = {x, w, bias, si, y, so, y1, x1};
  for (size_t i = 0; i < sizeof(ptrs) / sizeof(ptrs[0]); ++i) free(ptrs[i]);
}

static void ssd_cases(int64_t b, int64_t L, int64_t H, int64_t P, int64_t G, int64_t N) {
  const int64_t tok = b * L, ch = H * P, st = b * ch * N;
  double *x = arr(tok * ch, -1, 1), *dt = arr(tok * H, -4, 1), *z = arr(tok * ch, -2, 2);
  double *B = arr(tok * G * N, -1, 1), *C = arr(tok * G * N, -1, 1), *A = arr(H, -3, -0.1);
  double *D = arr(ch, 0.5, 1.5), *bias = arr(H, -1, 0), *h0 = arr(st, -1, 1);
  double *y = arr(tok * ch, 0, 0), *y2 = arr(tok * ch, 0, 0), *last = arr(st, 0, 0), *last2 = arr(st, 0, 0);
  check("ssd", oracle_ssd_fwd(x, dt, A, B, C, D, z, bias, 1, h0, y, last, b, L, H, P, G, N, 1) == 0);
  check("ssd 4 threads", oracle_ssd_fwd(x, dt, A, B, C, D, z, bias, 1, h0, y2, last2, b, L, H, P, G, N, 4) == 0);
  check("ssd threads bitwise", memcmp(y, y2, sizeof(double) * (size_t)(tok * ch)) == 0);
  check("ssd finite", finite(y, tok * ch) && finite(last, st));
  check("ssd no options", oracle_ssd_fwd(x, dt, A, B, C, NULL, NULL, NULL, 0, NULL, y, NULL, b, L, H, P, G, N, 2) == 0);
  double *x1 = arr(b * ch, -1, 1), *dt1 = arr(b * H, -4, 1), *B1 = arr(b * G * N, -1, 1), *C1 = arr(b * G * N, -1, 1);
  double* y1 = arr(b * ch, 0, 0);
  check("ssd decode", oracle_ssd_state_update(last, x1, dt1, A, B1, C1, D, NULL, bias, 1, y1, b, H, P, G, N) == 0);
  check("ssd decode finite", finite(y1, b * ch) && finite(last, st));
  double* ptrs[] = {x, dt, z, B, C, A, D, bias, h0, y, y2, last, last2, x1, dt1, B1, C1, y1};
  for (size_t i = 0; i < sizeof(ptrs) / sizeof(ptrs[0]); ++i) free(ptrs[i]);
}

int main(void) {
  scan_cases(2, 23, 5, 16);
  scan_cases(1, 1, 1, 16);
  scan_cases(3, 17, 2, 3);
  scan_cases(0, 4, 3, 16);
  scan_cases(2, 0, 3, 16);
  scan_cases(2, 4, 0, 16);
  conv_cases(2, 9, 5, 4);
  conv_cases(1, 2, 3, 3);
  conv_cases(0, 2, 3, 2);
  ssd_cases(2, 19, 4, 3, 2, 5);
  ssd_cases(1, 1, 1, 1, 1, 1);
  ssd_cases(1, 0, 2, 2, 1, 4);
  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("oracle driver ok\n");
  return 0;
}
