/*
 * coalesce_oracle.c -- plain fp64 CPU oracle for the fused GEMM epilogue and
 * the softplus MLP chain.  TEST INFRASTRUCTURE ONLY: the tests, the smoke
 * check and the benchmark's CPU-baseline leg may call it; the product path
 * never does.  It shares no code, header or table with the HIP library.
 *
 * What it computes (sources are the pages' titles and sections):
 *
 *  - "Coalesce" README, section "Fusion study" and the status table
 *    ("Fused GEMM + bias + GELU -- the anchor"): Y = GELU(A.B + bias), the
 *    epilogue applied to every GEMM output element.  The bias is a length-N
 *    vector broadcast over the rows (the Linear-layer reading; the page says
 *    only "bias").
 *  - same README, "Notes for future sessions": GELU is the exact erf form,
 *    GELU(z) = z * Phi(z) = 0.5 z (1 + erf(z / sqrt 2)), not the tanh
 *    approximation.
 *  - "MLP Megakernel" README, section "Architecture": the 3- and 5-layer
 *    chains out = softplus(...softplus(x W1) W2 ...) W_L, no biases, the last
 *    layer linear.
 *  - same README, "Ablation Study / Key findings": softplus(x) = log(1 + e^x)
 *    (the page's guarded form switches to x above 20; the oracle instead
 *    evaluates the exact function in fp64, see oracle_softplus).
 *
 * Everything is computed in double precision from inputs that the caller has
 * already widened exactly to double (bf16/fp16/fp32 -> fp64 is exact).  The
 * GEMM is the naive triple loop; each output element's k-sum runs k = 0..K-1
 * in order, so the result does not depend on the thread count.  Rows are
 * split over OpenMP threads.
 *
 * Build: gcc -O2 -fno-fast-math -ffp-contract=off -fopenmp -shared -fPIC
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_ACT_NONE = 0, ORACLE_ACT_GELU_ERF = 1, ORACLE_ACT_SOFTPLUS = 2, ORACLE_ACT_RELU = 3 };

/* GELU, erf form ("Coalesce" README, notes: use erf, not tanh). */
double oracle_gelu(double z) { return 0.5 * z * (1.0 + erf(z / sqrt(2.0))); }

/* softplus(z) = ln(1 + e^z).  Written as max(z,0) + ln(1 + e^-|z|), which is
 * the same function rearranged exactly (ln(1+e^z) = z + ln(1+e^-z)); it keeps
 * full fp64 accuracy for large |z| where 1 + e^z would overflow or round to 1.
 * The page's thresholded form (x above 20 -> x) differs from this by at most
 * ln(1 + e^-20) ~ 2.1e-9. */
double oracle_softplus(double z) {
  double a = fabs(z);
  return (z > 0.0 ? z : 0.0) + log1p(exp(-a));
}

static double apply_act(double z, int act) {
  if (act == ORACLE_ACT_GELU_ERF) return oracle_gelu(z);
  if (act == ORACLE_ACT_SOFTPLUS) return oracle_softplus(z);
  if (act == ORACLE_ACT_RELU) return z > 0.0 ? z : 0.0; /* the matmul-relu of the "Coalesce" README */
  return z;
}

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/*
 * Y[r][j] = act( sum_k A[rows[r]][k] * B[k][j] + bias[j] ),  r = 0..nrows-1.
 * A is M x K, B is K x N, Y is nrows x N, all row-major and dense.  bias may
 * be NULL (no bias term).  rows == NULL means rows[r] = r (all M rows, and
 * nrows must equal M).  nthreads <= 0 uses the OpenMP default.
 * Returns 0, or -1 on a bad argument.
 */
int oracle_gemm_bias_act(const double* A, const double* B, const double* bias, double* Y,
                         const int64_t* rows, int64_t nrows, int64_t M, int64_t N, int64_t K,
                         int act, int nthreads) {
  if (nrows < 0 || M < 0 || N < 0 || K < 0) return -1;
  if ((nrows > 0 && N > 0) && (!Y || (K > 0 && (!A || !B)))) return -1;
  if (nthreads <= 0) nthreads = oracle_max_threads();
  int bad = 0;
#pragma omp parallel num_threads(nthreads) reduction(| : bad)
  {
    double* acc = (double*)malloc((size_t)(N > 0 ? N : 1) * sizeof(double));
    if (!acc) bad = 1;
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r) {
      if (!acc) continue;
      int64_t i = rows ? rows[r] : r;
      if (i < 0 || i >= M) { bad = 1; continue; }
      for (int64_t j = 0; j < N; ++j) acc[j] = 0.0;
      /* i-k-j order: for every (i, j) the products are added for k = 0, 1, ... */
      for (int64_t k = 0; k < K; ++k) {
        double a = A[i * K + k];
        const double* brow = B + k * N;
        for (int64_t j = 0; j < N; ++j) acc[j] += a * brow[j];
      }
      double* yrow = Y + r * N;
      for (int64_t j = 0; j < N; ++j) {
        double z = acc[j] + (bias ? bias[j] : 0.0);
        yrow[j] = apply_act(z, act);
      }
    }
    free(acc);
  }
  return bad ? -1 : 0;
}

/*
 * Single elements: out[s] = act( sum_k A[rows[s]][k] * B[k][cols[s]] + bias[cols[s]] ).
 * Same definition as above, evaluated one output at a time (used to check
 * sampled outputs of the full-size problems).
 */
int oracle_gemm_bias_act_at(const double* A, const double* B, const double* bias,
                            const int64_t* rows, const int64_t* cols, int64_t nsamples,
                            double* out, int64_t M, int64_t N, int64_t K, int act, int nthreads) {
  if (nsamples < 0 || M < 0 || N < 0 || K < 0) return -1;
  if (nsamples > 0 && (!rows || !cols || !out || (K > 0 && (!A || !B)))) return -1;
  if (nthreads <= 0) nthreads = oracle_max_threads();
  int bad = 0;
#pragma omp parallel for num_threads(nthreads) schedule(static) reduction(| : bad)
  for (int64_t s = 0; s < nsamples; ++s) {
    int64_t i = rows[s], j = cols[s];
    if (i < 0 || i >= M || j < 0 || j >= N) { bad = 1; continue; }
    double acc = 0.0;
    for (int64_t k = 0; k < K; ++k) acc += A[i * K + k] * B[k * N + j];
    out[s] = apply_act(acc + (bias ? bias[j] : 0.0), act);
  }
  return bad ? -1 : 0;
}

/*
 * MLP chain ("MLP Megakernel" README, Architecture):
 *   h_0 = x;  z_l = h_{l-1} W_l;  h_l = softplus(z_l) for l < L;  out = z_L.
 * x is M x dims[0]; W[l] (l = 0..L-1) is dims[l] x dims[l+1] row-major (the
 * x @ W orientation of the page); out is nrows x dims[L].  rows selects which
 * rows of x to evaluate (NULL = all M, nrows == M).  hidden_act is the
 * activation between layers (softplus on the page; NONE and GELU are also
 * accepted so the chain can be checked piecewise).
 */
int oracle_mlp_forward(const double* x, const double* const* W, const int64_t* dims, int L,
                       double* out, const int64_t* rows, int64_t nrows, int64_t M,
                       int hidden_act, int nthreads) {
  if (L < 1 || nrows < 0 || M < 0 || !dims || !W) return -1;
  int64_t maxw = 0;
  for (int l = 0; l <= L; ++l) {
    if (dims[l] < 0) return -1;
    if (dims[l] > maxw) maxw = dims[l];
  }
  for (int l = 0; l < L; ++l)
    if (dims[l] > 0 && dims[l + 1] > 0 && !W[l]) return -1;
  if (nrows > 0 && (!x || !out)) return -1;
  if (nthreads <= 0) nthreads = oracle_max_threads();
  int bad = 0;
#pragma omp parallel num_threads(nthreads) reduction(| : bad)
  {
    double* h = (double*)malloc((size_t)(maxw > 0 ? maxw : 1) * sizeof(double));
    double* z = (double*)malloc((size_t)(maxw > 0 ? maxw : 1) * sizeof(double));
    if (!h || !z) bad = 1;
#pragma omp for schedule(dynamic, 64)
    for (int64_t r = 0; r < nrows; ++r) {
      if (!h || !z) continue;
      int64_t i = rows ? rows[r] : r;
      if (i < 0 || i >= M) { bad = 1; continue; }
      for (int64_t k = 0; k < dims[0]; ++k) h[k] = x[i * dims[0] + k];
      for (int l = 0; l < L; ++l) {
        int64_t din = dims[l], dout = dims[l + 1];
        const double* w = W[l];
        for (int64_t j = 0; j < dout; ++j) {
          double acc = 0.0;
          for (int64_t k = 0; k < din; ++k) acc += h[k] * w[k * dout + j];
          z[j] = acc;
        }
        int last = (l == L - 1);
        for (int64_t j = 0; j < dout; ++j) h[j] = last ? z[j] : apply_act(z[j], hidden_act);
      }
      memcpy(out + r * dims[L], h, (size_t)dims[L] * sizeof(double));
    }
    free(h);
    free(z);
  }
  return bad ? -1 : 0;
}
