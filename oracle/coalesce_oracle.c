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
 *  - same README, "Key ideas" (fused weight normalisation W = g v / ||v||):
 *    the norm is taken per output unit -- over each column of the x @ W
 *    matrix, torch's weight_norm on a Linear weight -- with one gain g per
 *    output unit; oracle_weight_norm and its backward.
 *  - same README, "Key ideas" (training: the forward keeps the hidden
 *    activations, the backward multiplies by the derivative of softplus) and
 *    the quick start's out.sum().backward(): the gradients of the chain with
 *    respect to every W_l and to x, given dL/d(out), by the chain rule.
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

/* Derivative of the hidden activation at z.  softplus: d/dz ln(1 + e^z) =
 * e^z / (1 + e^z), the logistic sigmoid, evaluated without overflow on either
 * side.  relu: 1 for z > 0, else 0 (0 at the kink z = 0 itself).  none: 1. */
double oracle_act_deriv(double z, int act) {
  if (act == ORACLE_ACT_SOFTPLUS) {
    if (z >= 0.0) return 1.0 / (1.0 + exp(-z));
    double e = exp(z);
    return e / (1.0 + e);
  }
  if (act == ORACLE_ACT_RELU) return z > 0.0 ? 1.0 : 0.0;
  return 1.0;
}

static int check_chain(const double* const* W, const int64_t* dims, int L, int64_t* maxw) {
  if (L < 1 || !dims || !W) return -1;
  int64_t m = 0;
  for (int l = 0; l <= L; ++l) {
    if (dims[l] < 0) return -1;
    if (dims[l] > m) m = dims[l];
  }
  for (int l = 0; l < L; ++l)
    if (dims[l] > 0 && dims[l + 1] > 0 && !W[l]) return -1;
  *maxw = m;
  return 0;
}

/* z = h W for one row: z[j] = sum_k h[k] W[k][j], k in order. */
static void row_times_w(const double* h, const double* w, int64_t din, int64_t dout, double* z) {
  for (int64_t j = 0; j < dout; ++j) {
    double acc = 0.0;
    for (int64_t k = 0; k < din; ++k) acc += h[k] * w[k * dout + j];
    z[j] = acc;
  }
}

/* g = d W^T for one row: g[k] = sum_j d[j] W[k][j], j in order. */
static void row_times_wt(const double* d, const double* w, int64_t din, int64_t dout, double* g) {
  for (int64_t k = 0; k < din; ++k) {
    double acc = 0.0;
    for (int64_t j = 0; j < dout; ++j) acc += d[j] * w[k * dout + j];
    g[k] = acc;
  }
}

/*
 * Training forward: the chain of oracle_mlp_forward over all M rows, and
 * acts[l - 1] (l = 1..L-1, each M x dims[l], dense) receives the hidden
 * activation h_l = act(z_l) that the backward consumes.  acts may be NULL
 * when L == 1.
 */
int oracle_mlp_forward_train(const double* x, const double* const* W, const int64_t* dims, int L, double* out,
                             double* const* acts, int64_t M, int hidden_act, int nthreads) {
  int64_t maxw = 0;
  if (M < 0 || check_chain(W, dims, L, &maxw)) return -1;
  if (M > 0 && (!x || !out || (L > 1 && !acts))) return -1;
  for (int l = 1; l < L; ++l)
    if (M > 0 && dims[l] > 0 && !acts[l - 1]) return -1;
  if (nthreads <= 0) nthreads = oracle_max_threads();
  int bad = 0;
#pragma omp parallel num_threads(nthreads) reduction(| : bad)
  {
    double* h = (double*)malloc((size_t)(maxw > 0 ? maxw : 1) * sizeof(double));
    double* z = (double*)malloc((size_t)(maxw > 0 ? maxw : 1) * sizeof(double));
    if (!h || !z) bad = 1;
#pragma omp for schedule(dynamic, 64)
    for (int64_t r = 0; r < M; ++r) {
      if (!h || !z) continue;
      memcpy(h, x + r * dims[0], (size_t)dims[0] * sizeof(double));
      for (int l = 0; l < L; ++l) {
        row_times_w(h, W[l], dims[l], dims[l + 1], z);
        if (l == L - 1) {
          memcpy(out + r * dims[L], z, (size_t)dims[L] * sizeof(double));
        } else {
          for (int64_t j = 0; j < dims[l + 1]; ++j) h[j] = apply_act(z[j], hidden_act);
          memcpy(acts[l] + r * dims[l + 1], h, (size_t)dims[l + 1] * sizeof(double));
        }
      }
    }
    free(h);
    free(z);
  }
  return bad ? -1 : 0;
}

/*
 * Backward of the chain by the chain rule, all in fp64.  With W[l] mapping
 * width dims[l] to dims[l + 1] (layer l + 1 of the page), h_0 = x,
 * z_{l+1} = h_l W[l], h_l = act(z_l) (0 < l < L), out = z_L and the upstream
 * gradient dz_L = dout (M x dims[L]):
 *   dW[l]  = h_l^T dz_{l+1}                       (dims[l] x dims[l+1])
 *   dh_l   = dz_{l+1} W[l]^T
 *   dz_l   = dh_l * act'(z_l)   elementwise, 0 < l < L
 *   dx     = dh_0                                  (M x dims[0]; skipped when dx is NULL)
 * The forward is recomputed here from x and W (the oracle takes no stored
 * activations).  Every dW element sums its row terms for r = 0, 1, ..., M-1
 * in that order, so the result does not depend on the thread count; rows
 * are processed in blocks to bound the memory.  Returns 0, or -1 on a bad
 * argument.
 */
int oracle_mlp_backward(const double* x, const double* const* W, const int64_t* dims, int L, const double* dout,
                        double* const* dW, double* dx, int64_t M, int hidden_act, int nthreads) {
  int64_t maxw = 0;
  if (M < 0 || check_chain(W, dims, L, &maxw) || !dW) return -1;
  for (int l = 0; l < L; ++l)
    if (dims[l] > 0 && dims[l + 1] > 0 && !dW[l]) return -1;
  if (M > 0 && (!x || !dout)) return -1;
  if (nthreads <= 0) nthreads = oracle_max_threads();
  for (int l = 0; l < L; ++l) memset(dW[l], 0, (size_t)(dims[l] * dims[l + 1]) * sizeof(double));
  if (M == 0) return 0;
  /* per-row record: h_0..h_{L-1}, then dz_1..dz_L, then z_1..z_{L-1} */
  int64_t hoff[17], doff[17], zoff[17], S = 0;
  if (L > 16) return -1;
  for (int l = 0; l < L; ++l) { hoff[l] = S; S += dims[l]; }
  for (int l = 1; l <= L; ++l) { doff[l] = S; S += dims[l]; }
  for (int l = 1; l < L; ++l) { zoff[l] = S; S += dims[l]; }
  const int64_t BR = 2048;
  double* buf = (double*)malloc((size_t)(BR * (S > 0 ? S : 1)) * sizeof(double));
  if (!buf) return -1;
  int bad = 0;
  for (int64_t r0 = 0; r0 < M; r0 += BR) {
    const int64_t nb = M - r0 < BR ? M - r0 : BR;
#pragma omp parallel num_threads(nthreads) reduction(| : bad)
    {
      double* g = (double*)malloc((size_t)(maxw > 0 ? maxw : 1) * sizeof(double));
      if (!g) bad = 1;
#pragma omp for schedule(dynamic, 16)
      for (int64_t b = 0; b < nb; ++b) {
        if (!g) continue;
        const int64_t r = r0 + b;
        double* rec = buf + b * S;
        memcpy(rec + hoff[0], x + r * dims[0], (size_t)dims[0] * sizeof(double));
        for (int l = 0; l < L - 1; ++l) {
          double* z = rec + zoff[l + 1];
          row_times_w(rec + hoff[l], W[l], dims[l], dims[l + 1], z);
          for (int64_t j = 0; j < dims[l + 1]; ++j) rec[hoff[l + 1] + j] = apply_act(z[j], hidden_act);
        }
        memcpy(rec + doff[L], dout + r * dims[L], (size_t)dims[L] * sizeof(double));
        for (int l = L - 1; l >= 0; --l) {
          row_times_wt(rec + doff[l + 1], W[l], dims[l], dims[l + 1], g);
          if (l > 0) {
            for (int64_t k = 0; k < dims[l]; ++k)
              rec[doff[l] + k] = g[k] * oracle_act_deriv(rec[zoff[l] + k], hidden_act);
          } else if (dx) {
            memcpy(dx + r * dims[0], g, (size_t)dims[0] * sizeof(double));
          }
        }
      }
      free(g);
    }
    /* dW[l][k][n] += h_l[r][k] dz_{l+1}[r][n] for the block's rows in order */
    for (int l = 0; l < L; ++l) {
      const int64_t din = dims[l], dn = dims[l + 1];
      double* dw = dW[l];
#pragma omp parallel for num_threads(nthreads) schedule(static)
      for (int64_t k = 0; k < din; ++k)
        for (int64_t b = 0; b < nb; ++b) {
          const double a = buf[b * S + hoff[l] + k];
          const double* d = buf + b * S + doff[l + 1];
          for (int64_t n = 0; n < dn; ++n) dw[k * dn + n] += a * d[n];
        }
    }
  }
  free(buf);
  return bad ? -1 : 0;
}

/*
 * Weight normalisation ("MLP Megakernel" README, "Key ideas"):
 *   W[k][n] = g[n] v[k][n] / ||v[:, n]||,   ||v[:, n]|| = sqrt(sum_k v[k][n]^2)
 * for a din x dout matrix v (row-major, the x @ W orientation) and a gain per
 * output unit n.  A zero column gives 0 * g / 0 = NaN (no guard, as in the
 * plain formula).  Returns 0, or -1 on a bad argument.
 */
int oracle_weight_norm(const double* v, const double* g, double* W, int64_t din, int64_t dout) {
  if (din < 0 || dout < 0) return -1;
  if (din > 0 && dout > 0 && (!v || !g || !W)) return -1;
  for (int64_t n = 0; n < dout; ++n) {
    double ss = 0.0;
    for (int64_t k = 0; k < din; ++k) ss += v[k * dout + n] * v[k * dout + n];
    const double nrm = sqrt(ss);
    for (int64_t k = 0; k < din; ++k) W[k * dout + n] = g[n] * v[k * dout + n] / nrm;
  }
  return 0;
}

/*
 * Backward of oracle_weight_norm given dW = dLoss/dW, by the chain rule:
 *   dg[n]    = sum_k dW[k][n] v[k][n] / ||v_n||
 *   dv[k][n] = g[n] / ||v_n|| * (dW[k][n] - v[k][n] (sum_j v[j][n] dW[j][n]) / ||v_n||^2)
 */
int oracle_weight_norm_backward(const double* v, const double* g, const double* dW, double* dv, double* dg,
                                int64_t din, int64_t dout) {
  if (din < 0 || dout < 0) return -1;
  if (din > 0 && dout > 0 && (!v || !g || !dW || !dv || !dg)) return -1;
  for (int64_t n = 0; n < dout; ++n) {
    double ss = 0.0, dot = 0.0;
    for (int64_t k = 0; k < din; ++k) {
      ss += v[k * dout + n] * v[k * dout + n];
      dot += v[k * dout + n] * dW[k * dout + n];
    }
    const double nrm = sqrt(ss);
    dg[n] = dot / nrm;
    for (int64_t k = 0; k < din; ++k)
      dv[k * dout + n] = g[n] / nrm * (dW[k * dout + n] - v[k * dout + n] * dot / ss);
  }
  return 0;
}
