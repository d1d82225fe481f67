/*
 * CPU oracle for the fused RMSNorm+MatMul path -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg may
 * load this library.  It shares no code, header or constant with the HIP
 * library: it is the plain, slow, unfused program in double precision.
 *
 * What it computes.  The Mirage paper review ("Mirage: A Multi-Level
 * Superoptimizer for Tensor Programs", section "核心概念 / μGraph示例")
 * takes RMSNorm followed by MatMul as its worked example: existing systems
 * run the two as separate kernels, Mirage fuses them so the normalised
 * tensor is never materialised.  The same page's abstract expression
 * (section "核心公式 / 抽象表达式") is E(O) = sum(k, div(mul(I1, I2), I3)):
 * a k-sum of a product divided by a per-row quantity that does not depend
 * on k.  The oracle is the unfused program those sections describe:
 *
 *   1. per row m:  S[m] = (sum_k X[m,k]^2) / K,  r[m] = sqrt(S[m] + eps)
 *   2. per (m,k):  Nrm[m,k] = (X[m,k] / r[m]) * g[k]     -- materialised
 *   3. per (m,n):  Y[m,n] = sum_k Nrm[m,k] * W[k,n]        -- i-k-j loops
 *
 * RMSNorm itself is not written out on the pages; the reading used is the
 * conventional one: root-mean-square over the contraction dimension K
 * (divide by K), eps added inside the square root, gain g applied per k.
 * The matmul is the plain broadcast-multiply-then-sum-over-k definition
 * (the Luminal talk page describes matmul the same way).
 *
 * Gated MLP (paper review, section "五、实验结果", the GatedMLP benchmark row;
 * the page does not define it, the reading is SwiGLU):
 *   Z1 = Nrm * W1,  Z3 = Nrm * W3,  Y = Z1 / (1 + exp(-Z1)) * Z3.
 *
 * LoRA (paper review, section "五、实验结果", the LoRA row; the page names the
 * benchmark only, the reading is the usual low-rank adapter): the frozen
 * product plus a rank-R update applied as two thin products,
 *   T = Act * A^T   (A: R x K, row r is the r-th down-projection vector),
 *   Y = Act * W + T * B   (B: R x N),
 * with Act = Nrm (rmm_oracle_rmsnorm_lora_f64) or X itself
 * (rmm_oracle_lora_matmul_f64, the adapter alone).
 *
 * QKNorm + attention (paper review, section "五、实验结果", the QKNorm + Attention
 * row; the page names the benchmark only).  Reading: RMSNorm over the head
 * dimension D with per-dimension gains, applied to the query and to every
 * key, then scaled dot-product attention over the cached keys (one query per
 * batch-head, no mask):
 *   qn = q / rms(q) * gq,   kn_s = k_s / rms(k_s) * gk,
 *   p_s = softmax_s(qn . kn_s / sqrt(D)),   o = sum_s p_s v_s.
 * (rmm_oracle_qknorm_attention_f64; the normalised vectors are materialised.)
 * The attention step alone, on given (already normalised) vectors, is
 * rmm_oracle_attention_f64: the second kernel of the unfused program.
 * Many queries per head (prefill): every query row of a head attends, with
 * the same normalisations, to its key/value head's keys; G query heads may
 * share one key/value head (query head h G + g reads key head h), and with
 * the causal mask query position i of Sq sees keys 0 .. i + Skv - Sq (the
 * queries are the last Sq positions of the Skv cached ones)
 * (rmm_oracle_qknorm_attention_prefill_f64).
 *
 * The steps are also exported one by one (rmm_oracle_rmsnorm_f64: steps 1-2,
 * rmm_oracle_matmul_f64: step 3, rmm_oracle_gated_matmul_f64: the two
 * products and the gate), because the unfused program is itself measured:
 * it is the comparison point of the same section.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off (no fast-math).  OpenMP splits
 * rows across threads only for timing; each output element is computed by
 * one thread in the same order as the serial program.
 *
 * Parity pins live in tests/test_oracle_pins.py (closed forms, invariants,
 * special cases that reduce to a library matmul, brute force on tiny
 * shapes).  No function here is "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

/* Step 1: r[m] = sqrt(mean_k X[m,k]^2 + eps). */
static void row_rms(const double* X, int64_t M, int64_t K, double eps, double* r) {
#pragma omp parallel for schedule(static)
  for (int64_t m = 0; m < M; ++m) {
    double ss = 0.0;
    for (int64_t k = 0; k < K; ++k) ss += X[m * K + k] * X[m * K + k];
    r[m] = sqrt(ss / (double)K + eps);
  }
}

/* Step 2: the normalised, gained activations (the tensor fusion avoids). */
static void normalise(const double* X, const double* g, const double* r, int64_t M,
                      int64_t K, double* Nrm) {
#pragma omp parallel for schedule(static)
  for (int64_t m = 0; m < M; ++m)
    for (int64_t k = 0; k < K; ++k) Nrm[m * K + k] = (X[m * K + k] / r[m]) * g[k];
}

/* Step 3: Y = A * B, A: M x K, B: K x N (B[k*N + n]), i-k-j order. */
static void matmul(const double* A, const double* B, int64_t M, int64_t N, int64_t K,
                   double* Y) {
#pragma omp parallel for schedule(static)
  for (int64_t m = 0; m < M; ++m) {
    double* y = Y + m * N;
    for (int64_t n = 0; n < N; ++n) y[n] = 0.0;
    for (int64_t k = 0; k < K; ++k) {
      const double a = A[m * K + k];
      const double* b = B + k * N;
      for (int64_t n = 0; n < N; ++n) y[n] += a * b[n];
    }
  }
}

/* Returns 0 on success, 1 on bad shape, 2 on allocation failure. */
int rmm_oracle_rmsnorm_matmul_f64(const double* X, const double* g, const double* W,
                                  double eps, int64_t M, int64_t N, int64_t K, double* Y) {
  if (M < 0 || N < 0 || K <= 0) return 1;
  double* r = (double*)malloc(sizeof(double) * (size_t)(M > 0 ? M : 1));
  double* Nrm = (double*)malloc(sizeof(double) * (size_t)(M > 0 ? M * K : 1));
  if (!r || !Nrm) {
    free(r);
    free(Nrm);
    return 2;
  }
  row_rms(X, M, K, eps, r);
  normalise(X, g, r, M, K, Nrm);
  matmul(Nrm, W, M, N, K, Y);
  free(r);
  free(Nrm);
  return 0;
}

/* Gated products on activations A: Y = silu(A W1) * (A W3). */
static int gated_products(const double* A, const double* W1, const double* W3, int64_t M,
                          int64_t N, int64_t K, double* Y) {
  double* Z3 = (double*)malloc(sizeof(double) * (size_t)(M * N > 0 ? M * N : 1));
  if (!Z3) return 2;
  matmul(A, W1, M, N, K, Y); /* Y holds Z1 until the gate below */
  matmul(A, W3, M, N, K, Z3);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < M * N; ++i) {
    const double z1 = Y[i];
    Y[i] = z1 / (1.0 + exp(-z1)) * Z3[i];
  }
  free(Z3);
  return 0;
}

int rmm_oracle_rmsnorm_gated_mlp_f64(const double* X, const double* g, const double* W1,
                                     const double* W3, double eps, int64_t M, int64_t N,
                                     int64_t K, double* Y) {
  if (M < 0 || N < 0 || K <= 0) return 1;
  double* r = (double*)malloc(sizeof(double) * (size_t)(M > 0 ? M : 1));
  double* Nrm = (double*)malloc(sizeof(double) * (size_t)(M > 0 ? M * K : 1));
  if (!r || !Nrm) {
    free(r);
    free(Nrm);
    return 2;
  }
  row_rms(X, M, K, eps, r);
  normalise(X, g, r, M, K, Nrm);
  const int rc = gated_products(Nrm, W1, W3, M, N, K, Y);
  free(r);
  free(Nrm);
  return rc;
}

/* Steps 1-2 alone: the normalised, gained rows, M x K. */
int rmm_oracle_rmsnorm_f64(const double* X, const double* g, double eps, int64_t M, int64_t K,
                           double* Nrm) {
  if (M < 0 || K <= 0) return 1;
  double* r = (double*)malloc(sizeof(double) * (size_t)(M > 0 ? M : 1));
  if (!r) return 2;
  row_rms(X, M, K, eps, r);
  normalise(X, g, r, M, K, Nrm);
  free(r);
  return 0;
}

/* Step 3 alone: Y = A * B. */
int rmm_oracle_matmul_f64(const double* A, const double* B, int64_t M, int64_t N, int64_t K,
                          double* Y) {
  if (M < 0 || N < 0 || K <= 0) return 1;
  matmul(A, B, M, N, K, Y);
  return 0;
}

/* Gated products on given activations: Y = silu(A W1) * (A W3). */
int rmm_oracle_gated_matmul_f64(const double* A, const double* W1, const double* W3, int64_t M,
                                int64_t N, int64_t K, double* Y) {
  if (M < 0 || N < 0 || K <= 0) return 1;
  return gated_products(A, W1, W3, M, N, K, Y);
}

/* LoRA on activations Act: Y = Act W + (Act A^T) B.  A: R x K, B: R x N. */
static int lora_products(const double* Act, const double* W, const double* A, const double* B,
                         int64_t M, int64_t N, int64_t K, int64_t R, double* Y) {
  double* T = (double*)malloc(sizeof(double) * (size_t)(M * R > 0 ? M * R : 1));
  if (!T) return 2;
  matmul(Act, W, M, N, K, Y);
#pragma omp parallel for schedule(static)
  for (int64_t m = 0; m < M; ++m) {
    for (int64_t r = 0; r < R; ++r) {
      double t = 0.0;
      for (int64_t k = 0; k < K; ++k) t += Act[m * K + k] * A[r * K + k];
      T[m * R + r] = t;
    }
    for (int64_t r = 0; r < R; ++r) {
      const double t = T[m * R + r];
      for (int64_t n = 0; n < N; ++n) Y[m * N + n] += t * B[r * N + n];
    }
  }
  free(T);
  return 0;
}

/* Y = Nrm W + (Nrm A^T) B with Nrm the normalised, gained rows. */
int rmm_oracle_rmsnorm_lora_f64(const double* X, const double* g, const double* W,
                                const double* A, const double* B, double eps, int64_t M,
                                int64_t N, int64_t K, int64_t R, double* Y) {
  if (M < 0 || N < 0 || K <= 0 || R <= 0) return 1;
  double* r = (double*)malloc(sizeof(double) * (size_t)(M > 0 ? M : 1));
  double* Nrm = (double*)malloc(sizeof(double) * (size_t)(M > 0 ? M * K : 1));
  if (!r || !Nrm) {
    free(r);
    free(Nrm);
    return 2;
  }
  row_rms(X, M, K, eps, r);
  normalise(X, g, r, M, K, Nrm);
  const int rc = lora_products(Nrm, W, A, B, M, N, K, R, Y);
  free(r);
  free(Nrm);
  return rc;
}

/* The adapter on raw activations: Y = X W + (X A^T) B. */
int rmm_oracle_lora_matmul_f64(const double* X, const double* W, const double* A,
                               const double* B, int64_t M, int64_t N, int64_t K, int64_t R,
                               double* Y) {
  if (M < 0 || N < 0 || K <= 0 || R <= 0) return 1;
  return lora_products(X, W, A, B, M, N, K, R, Y);
}

/* QKNorm + attention for one query per batch-head.  Q: BH x D, K and V:
 * BH x S x D (row s of head h at (h*S + s)*D), O: BH x D. */
/* The attention step for one batch-head: p_s = softmax_s(q . k_s / sqrt(D))
 * (the largest score subtracted before exp), o = sum_s p_s v_s.  sc: S
 * doubles of scratch. */
static void attend(const double* q, const double* Kh, const double* Vh, int64_t S, int64_t D,
                   double* sc, double* o) {
  for (int64_t s = 0; s < S; ++s) {
    const double* k = Kh + s * D;
    double dot = 0.0;
    for (int64_t d = 0; d < D; ++d) dot += q[d] * k[d];
    sc[s] = dot / sqrt((double)D);
  }
  double mx = sc[0];
  for (int64_t s = 1; s < S; ++s) mx = sc[s] > mx ? sc[s] : mx;
  double den = 0.0;
  for (int64_t s = 0; s < S; ++s) {
    sc[s] = exp(sc[s] - mx);
    den += sc[s];
  }
  for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
  for (int64_t s = 0; s < S; ++s) {
    const double p = sc[s] / den;
    const double* v = Vh + s * D;
    for (int64_t d = 0; d < D; ++d) o[d] += p * v[d];
  }
}

/* Scaled dot-product attention on the given vectors (no normalisation):
 * Q [BH, D], K and V [BH, S, D] -> O [BH, D]. */
int rmm_oracle_attention_f64(const double* Q, const double* K, const double* V, int64_t BH,
                             int64_t S, int64_t D, double* O) {
  if (BH < 0 || S <= 0 || D <= 0) return 1;
  int rc = 0;
#pragma omp parallel for schedule(static)
  for (int64_t h = 0; h < BH; ++h) {
    double* sc = (double*)malloc(sizeof(double) * (size_t)S);
    if (!sc) {
#pragma omp atomic write
      rc = 2;
      continue;
    }
    attend(Q + h * D, K + h * S * D, V + h * S * D, S, D, sc, O + h * D);
    free(sc);
  }
  return rc;
}

/* QKNorm + attention: the query and every key normalised (steps 1-2 on rows
 * of length D), then the attention step. */
int rmm_oracle_qknorm_attention_f64(const double* Q, const double* K, const double* V,
                                    const double* gq, const double* gk, double eps, int64_t BH,
                                    int64_t S, int64_t D, double* O) {
  if (BH < 0 || S <= 0 || D <= 0) return 1;
  int rc = 0;
#pragma omp parallel for schedule(static)
  for (int64_t h = 0; h < BH; ++h) {
    double* qn = (double*)malloc(sizeof(double) * (size_t)D);
    double* kn = (double*)malloc(sizeof(double) * (size_t)(S * D));
    double* sc = (double*)malloc(sizeof(double) * (size_t)S);
    if (!qn || !kn || !sc) {
      free(qn);
      free(kn);
      free(sc);
#pragma omp atomic write
      rc = 2;
      continue;
    }
    double rq;
    row_rms(Q + h * D, 1, D, eps, &rq);
    normalise(Q + h * D, gq, &rq, 1, D, qn);
    for (int64_t s = 0; s < S; ++s) {
      const double* k = K + (h * S + s) * D;
      double rk;
      row_rms(k, 1, D, eps, &rk);
      normalise(k, gk, &rk, 1, D, kn + s * D);
    }
    attend(qn, kn, V + h * S * D, S, D, sc, O + h * D);
    free(qn);
    free(kn);
    free(sc);
  }
  return rc;
}

/* QKNorm + attention for many queries per head.  Q and O: (BH G) x Sq x D,
 * K and V: BH x Skv x D; query head qh reads key/value head qh / G; causal:
 * query i attends to keys 0 .. i + Skv - Sq (needs Skv >= Sq), else to all. */
int rmm_oracle_qknorm_attention_prefill_f64(const double* Q, const double* K, const double* V,
                                            const double* gq, const double* gk, double eps,
                                            int64_t BH, int64_t G, int64_t Sq, int64_t Skv,
                                            int64_t D, int causal, double* O) {
  if (BH < 0 || G < 1 || Sq <= 0 || Skv <= 0 || D <= 0 || (causal && Skv < Sq)) return 1;
  int rc = 0;
#pragma omp parallel for schedule(static)
  for (int64_t qh = 0; qh < BH * G; ++qh) {
    const int64_t h = qh / G;
    double* qn = (double*)malloc(sizeof(double) * (size_t)D);
    double* kn = (double*)malloc(sizeof(double) * (size_t)(Skv * D));
    double* sc = (double*)malloc(sizeof(double) * (size_t)Skv);
    if (!qn || !kn || !sc) {
      free(qn);
      free(kn);
      free(sc);
#pragma omp atomic write
      rc = 2;
      continue;
    }
    for (int64_t s = 0; s < Skv; ++s) {
      const double* key = K + (h * Skv + s) * D;
      double rkey;
      row_rms(key, 1, D, eps, &rkey);
      normalise(key, gk, &rkey, 1, D, kn + s * D);
    }
    for (int64_t i = 0; i < Sq; ++i) {
      const double* q = Q + (qh * Sq + i) * D;
      double rq;
      row_rms(q, 1, D, eps, &rq);
      normalise(q, gq, &rq, 1, D, qn);
      const int64_t nk = causal ? i + Skv - Sq + 1 : Skv;
      attend(qn, kn, V + h * Skv * D, nk, D, sc, O + (qh * Sq + i) * D);
    }
    free(qn);
    free(kn);
    free(sc);
  }
  return rc;
}
