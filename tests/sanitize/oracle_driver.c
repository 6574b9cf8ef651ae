/*
 * oracle_driver.c -- runs every entry point of the fp64 oracle
 * (oracle/pararnn_oracle.c) on small seeded problems, for a build with
 * AddressSanitizer and UndefinedBehaviorSanitizer: both cells, with and
 * without an initial state, one and several threads (more threads than
 * channels included), every optional output present and absent, and the
 * argument checks. It also checks two facts that need no reference values:
 * every output is finite, and after K >= L Newton iterations the iterate is
 * the sequential trajectory (finite termination). Exit status 0 when all
 * hold; the sanitizers abort on the first memory or undefined-behaviour error.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_seq(int cell, int B, int L, int D, const float* u, const float* a, const double* s0, double* out,
               int nthreads);
int oracle_newton(int cell, int B, int L, int D, int K, const float* u, const float* a, const double* s0,
                  double* out, double* max_update, double* iterates, int nthreads);
int oracle_adjoint(int cell, int B, int L, int D, const float* u, const float* a, const double* s0,
                   const double* S, const float* dh, double* du, double* ds0, double* da, int nthreads);
int oracle_cell(int cell, int n, const double* s, const double* u, const double* a, double* f, double* J,
                double* dfdu, double* dfda);
int oracle_scan(int ns, int B, int L, int D, const double* A, const double* b, const double* s0, double* s,
                int nthreads);
int oracle_scan_dense(int B, int L, int n, const double* A, const double* b, const double* s0, double* s,
                      int nthreads);

static uint64_t rng = 88172645463325252ull;
static double uniform(void) { /* xorshift64 in [-1, 1) */
  rng ^= rng << 13;
  rng ^= rng >> 7;
  rng ^= rng << 17;
  return (double)(rng >> 11) * (2.0 / 9007199254740992.0) - 1.0;
}

static int failures = 0;
#define CHECK(cond, ...)                       \
  do {                                         \
    if (!(cond)) {                             \
      fprintf(stderr, "FAIL: " __VA_ARGS__);   \
      fprintf(stderr, "\n");                   \
      ++failures;                              \
    }                                          \
  } while (0)

static int all_finite(const double* x, size_t n) {
  for (size_t i = 0; i < n; ++i)
    if (!isfinite(x[i])) return 0;
  return 1;
}

static double* dalloc(size_t n) { return (double*)malloc((n ? n : 1) * sizeof(double)); }
static float* falloc(size_t n) { return (float*)malloc((n ? n : 1) * sizeof(float)); }

static void run_cell_problem(int cell, int B, int L, int D, int with_s0, int threads) {
  const int G = cell ? 4 : 3, NS = cell ? 2 : 1;
  const size_t nu = (size_t)B * L * G * D, ns = (size_t)NS * B * L * D, n0 = (size_t)NS * B * D;
  float* u = falloc(nu);
  float* a = falloc((size_t)G * D);
  float* dh = falloc((size_t)B * L * D);
  double* s0 = with_s0 ? dalloc(n0) : NULL;
  for (size_t i = 0; i < nu; ++i) u[i] = (float)(2.0 * uniform());
  for (int i = 0; i < G * D; ++i) a[i] = (float)uniform();
  for (size_t i = 0; i < (size_t)B * L * D; ++i) dh[i] = (float)uniform();
  for (size_t i = 0; s0 && i < n0; ++i) s0[i] = uniform();

  double* seq = dalloc(ns);
  CHECK(oracle_seq(cell, B, L, D, u, a, s0, seq, threads) == 0, "oracle_seq");
  CHECK(all_finite(seq, ns), "oracle_seq finite");

  const int K = L + 1; /* K >= L: finite termination */
  double* out = dalloc(ns);
  double* upd = dalloc((size_t)K * B);
  double* its = dalloc((size_t)K * ns);
  CHECK(oracle_newton(cell, B, L, D, K, u, a, s0, out, upd, its, threads) == 0, "oracle_newton");
  CHECK(all_finite(out, ns) && all_finite(upd, (size_t)K * B) && all_finite(its, (size_t)K * ns),
        "oracle_newton finite");
  for (size_t i = 0; i < ns; ++i)
    CHECK(fabs(out[i] - seq[i]) <= 1e-12 * (1.0 + fabs(seq[i])), "finite termination (cell %d, %zu)", cell, i);
  for (size_t i = 0; i < ns; ++i)
    CHECK(its[(size_t)(K - 1) * ns + i] == out[i], "last stored iterate is the output");
  /* optional outputs absent */
  CHECK(oracle_newton(cell, B, L, D, 2, u, a, s0, out, NULL, NULL, threads) == 0, "oracle_newton, no extras");

  double* du = dalloc((size_t)B * L * G * D);
  double* ds0 = dalloc(n0);
  double* da = dalloc((size_t)G * D);
  CHECK(oracle_adjoint(cell, B, L, D, u, a, s0, seq, dh, du, ds0, da, threads) == 0, "oracle_adjoint");
  CHECK(all_finite(du, (size_t)B * L * G * D) && all_finite(ds0, n0) && all_finite(da, (size_t)G * D),
        "oracle_adjoint finite");
  CHECK(oracle_adjoint(cell, B, L, D, u, a, s0, seq, dh, du, NULL, NULL, threads) == 0, "oracle_adjoint, du only");

  /* argument checks */
  CHECK(oracle_seq(cell, 0, L, D, u, a, s0, seq, threads) != 0, "B = 0 rejected");
  CHECK(oracle_seq(7, B, L, D, u, a, s0, seq, threads) != 0, "bad cell rejected");
  CHECK(oracle_newton(cell, B, L, D, 0, u, a, s0, out, upd, NULL, threads) != 0, "K = 0 rejected");
  CHECK(oracle_adjoint(cell, B, L, D, u, a, s0, NULL, dh, du, NULL, NULL, threads) != 0, "NULL S rejected");

  free(u); free(a); free(dh); free(s0); free(seq); free(out); free(upd); free(its); free(du); free(ds0); free(da);
}

static void run_cell_eval(int cell, int n) {
  const int G = cell ? 4 : 3, NS = cell ? 2 : 1;
  double* s = dalloc((size_t)NS * n);
  double* u = dalloc((size_t)G * n);
  double* a = dalloc((size_t)G * n);
  for (int i = 0; i < NS * n; ++i) s[i] = uniform();
  for (int i = 0; i < G * n; ++i) { u[i] = 2.0 * uniform(); a[i] = uniform(); }
  double* f = dalloc((size_t)NS * n);
  double* J = dalloc((size_t)NS * NS * n);
  double* fu = dalloc((size_t)NS * G * n);
  double* fa = dalloc((size_t)NS * G * n);
  CHECK(oracle_cell(cell, n, s, u, a, f, J, fu, fa) == 0, "oracle_cell");
  CHECK(all_finite(f, (size_t)NS * n) && all_finite(J, (size_t)NS * NS * n), "oracle_cell finite");
  CHECK(oracle_cell(cell, n, s, u, a, f, NULL, NULL, NULL) == 0, "oracle_cell, f only");
  CHECK(oracle_cell(cell, -1, s, u, a, f, J, fu, fa) != 0, "n < 0 rejected");
  free(s); free(u); free(a); free(f); free(J); free(fu); free(fa);
}

static void run_scans(int B, int L, int D, int threads) {
  for (int nsx = 1; nsx <= 2; ++nsx) {
    const size_t n = (size_t)B * L * D;
    double* A = dalloc((size_t)nsx * nsx * n);
    double* b = dalloc((size_t)nsx * n);
    double* s0 = dalloc((size_t)nsx * B * D);
    double* s = dalloc((size_t)nsx * n);
    for (size_t i = 0; i < (size_t)nsx * nsx * n; ++i) A[i] = 0.45 * uniform();
    for (size_t i = 0; i < (size_t)nsx * n; ++i) b[i] = uniform();
    for (size_t i = 0; i < (size_t)nsx * B * D; ++i) s0[i] = uniform();
    CHECK(oracle_scan(nsx, B, L, D, A, b, s0, s, threads) == 0, "oracle_scan");
    CHECK(oracle_scan(nsx, B, L, D, A, b, NULL, s, threads) == 0, "oracle_scan, no s0");
    CHECK(all_finite(s, (size_t)nsx * n), "oracle_scan finite");
    CHECK(oracle_scan(3, B, L, D, A, b, s0, s, threads) != 0, "ns = 3 rejected");
    free(A); free(b); free(s0); free(s);
  }
  for (int nn = 1; nn <= 5; nn += 2) {
    const size_t steps = (size_t)B * L;
    double* A = dalloc(steps * nn * nn);
    double* b = dalloc(steps * nn);
    double* s0 = dalloc((size_t)B * nn);
    double* s = dalloc(steps * nn);
    for (size_t i = 0; i < steps * nn * nn; ++i) A[i] = 0.3 * uniform();
    for (size_t i = 0; i < steps * nn; ++i) b[i] = uniform();
    for (int i = 0; i < B * nn; ++i) s0[i] = uniform();
    CHECK(oracle_scan_dense(B, L, nn, A, b, s0, s, threads) == 0, "oracle_scan_dense");
    CHECK(oracle_scan_dense(B, L, nn, A, b, NULL, s, threads) == 0, "oracle_scan_dense, no s0");
    CHECK(all_finite(s, steps * nn), "oracle_scan_dense finite");
    CHECK(oracle_scan_dense(B, L, 0, A, b, s0, s, threads) != 0, "n = 0 rejected");
    free(A); free(b); free(s0); free(s);
  }
}

int main(void) {
  const int shapes[][3] = {{1, 1, 1}, {2, 5, 3}, {3, 9, 7}, {1, 12, 2}};
  for (int cell = 0; cell < 2; ++cell)
    for (size_t k = 0; k < sizeof(shapes) / sizeof(shapes[0]); ++k)
      for (int with_s0 = 0; with_s0 < 2; ++with_s0)
        for (int threads = 1; threads <= 9; threads += 4)
          run_cell_problem(cell, shapes[k][0], shapes[k][1], shapes[k][2], with_s0, threads);
  for (int cell = 0; cell < 2; ++cell) run_cell_eval(cell, 6);
  run_scans(2, 11, 5, 1);
  run_scans(3, 4, 2, 8);
  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("oracle driver: all checks passed\n");
  return 0;
}
