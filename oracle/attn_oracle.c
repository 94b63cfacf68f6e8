/*
 * attn_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, fp64 CPU evaluation of the attention forward with three
 * score-to-weight maps.  It exists to check the GPU library and to time a CPU
 * baseline; nothing in the product path may call it.  It shares no code,
 * header, constant or helper with the HIP library.
 *
 * Sources (the pages this follows):
 *   [P1] "Softmax-Free Attention in JAX/Flax NNX", section "One module, two
 *        compatibility functions": the softmax branch and the Yat branch
 *        (dots, the pairwise distance from the same dots, softplus of the raw
 *        per-head scalars, kappa, the 0.0 causal mask, mass, w = kappa /
 *        (mass + 1e-9)).
 *   [P2] "The Kernel Between the Roles", section "What the exponential was
 *        hired to do": weights kappa / sum(kappa), peak (|q|^2 + b)^2 / eps.
 *   [P3] "NNX Scaled Dot-Product Attention", sections "Shapes and the three
 *        steps", "Mask before softmax" and the displayed equation
 *        A = softmax(QK^T / sqrt(d_k) + M), O = AV.
 *   [P2'] "The Kernel Between the Roles", section "The run": the numerator
 *        power (q.k)^(2m) as the dial that sharpens the kernel's peak, and the
 *        b = 0 ablation.  Options of the Yat branch here:
 *        kappa = (dots + b)^(2m) / (max(d2, 0) + eps), b = 0 when bias-free.
 *   [P5] "s^tau" forum post, section with the core formula:
 *        a_i = phi(s_i)^tau / sum_j phi(s_j)^tau, phi(s) = softplus(s) + eps,
 *        tau = softplus(log_tau) + 1.
 *
 * Readings where the pages leave a step open (each listed in the design
 * notes of the repository):
 *   - GQA: query head h reads key/value head h / (Hq / Hkv).
 *   - causal: key j is allowed for query i iff j <= i (requires Tq == Tk).
 *   - masked keys contribute exactly 0 to numerator and denominator in all
 *     three branches (for s^tau this is a reading: the page feeds -inf
 *     through softplus instead).
 *   - s^tau: s = q.k / sqrt(d_k), phi floor eps = 1e-6.
 *   - mass: Yat sum(kappa); softmax sum(exp(s - max s)); s^tau sum(phi^tau).
 *   - max_score: Yat max kappa; softmax and s^tau max s, over allowed keys.
 *
 * Layout: q [B,Hq,Tq,dk], k [B,Hkv,Tk,dk], v [B,Hkv,Tk,dv], all contiguous
 * fp64.  Outputs for the n_rows requested rows: out [n_rows, dv],
 * mass [n_rows], max_score [n_rows].  A row id is (b*Hq + h)*Tq + i; rows ==
 * NULL means every row in order.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_SOFTMAX = 0, ORACLE_YAT = 1, ORACLE_STAU = 2 };

/* softplus(x) = log(1 + e^x), written so that neither branch overflows;
 * softplus(-inf) = 0 (the bias-free ablation), softplus(0) = ln 2. [P1] */
static double softplus(double x) { return fmax(x, 0.0) + log1p(exp(-fabs(x))); }

static double dot(const double* a, const double* b, int64_t n) {
  double s = 0.0;
  for (int64_t d = 0; d < n; ++d) s += a[d] * b[d];
  return s;
}

/* One query row.  score[] is scratch of length Tk. */
static void one_row(int variant, int causal, int64_t Hq, int64_t Hkv, int64_t Tq,
                    int64_t Tk, int64_t dk, int64_t dv, const double* q,
                    const double* k, const double* v, const double* b_raw,
                    const double* eps_raw, const double* log_tau, int yat_power,
                    int yat_bias_free, int64_t row, double* score, double* out,
                    double* mass, double* max_score) {
  const int64_t i = row % Tq;
  const int64_t bh = row / Tq;
  const int64_t h = bh % Hq;
  const int64_t b = bh / Hq;
  const int64_t hk = h / (Hq / Hkv);
  const double* qi = q + row * dk;
  const double* kb = k + (b * Hkv + hk) * Tk * dk;
  const double* vb = v + (b * Hkv + hk) * Tk * dv;
  const int64_t n_allowed = causal ? i + 1 : Tk; /* keys 0..n_allowed-1 */

  double m = -INFINITY, total = 0.0;
  if (variant == ORACLE_YAT) {
    /* [P1]: dots, d2 = |q|^2 + |k|^2 - 2 dots, b = softplus(b_raw),
     * eps = softplus(eps_raw), kappa = (dots + b)^2 / (max(d2, 0) + eps),
     * kappa = 0 where masked, mass = sum kappa, w = kappa / (mass + 1e-9). */
    const double bias = yat_bias_free ? 0.0 : softplus(b_raw[h]);
    const double eps = softplus(eps_raw[h]);
    const double nq = dot(qi, qi, dk);
    for (int64_t j = 0; j < Tk; ++j) {
      if (j >= n_allowed) { score[j] = 0.0; continue; }
      const double* kj = kb + j * dk;
      const double s = dot(qi, kj, dk);
      const double d2 = nq + dot(kj, kj, dk) - 2.0 * s;
      /* [P2']: numerator (s + b)^(2m), m = yat_power (m = 1: [P1]) */
      double num = 1.0;
      for (int e = 0; e < yat_power; ++e) num *= (s + bias) * (s + bias);
      const double kappa = num / (fmax(d2, 0.0) + eps);
      score[j] = kappa;
      total += kappa;
      if (kappa > m) m = kappa;
    }
    for (int64_t j = 0; j < Tk; ++j) score[j] = score[j] / (total + 1e-9);
  } else if (variant == ORACLE_SOFTMAX) {
    /* [P3]: scores = q.k / sqrt(d_k); blocked scores become -inf, whose
     * exponential is 0; softmax along the key axis with the row maximum
     * subtracted first. */
    const double scale = 1.0 / sqrt((double)dk);
    for (int64_t j = 0; j < n_allowed; ++j) {
      score[j] = dot(qi, kb + j * dk, dk) * scale;
      if (score[j] > m) m = score[j];
    }
    for (int64_t j = 0; j < Tk; ++j) {
      score[j] = j < n_allowed ? exp(score[j] - m) : 0.0;
      total += score[j];
    }
    for (int64_t j = 0; j < Tk; ++j) score[j] /= total;
  } else {
    /* [P5]: a_j = phi(s_j)^tau / sum phi^tau, phi = softplus(s) + 1e-6,
     * tau = softplus(log_tau) + 1; masked keys weigh exactly 0. */
    const double scale = 1.0 / sqrt((double)dk);
    const double tau = softplus(log_tau[h]) + 1.0;
    for (int64_t j = 0; j < Tk; ++j) {
      if (j >= n_allowed) { score[j] = 0.0; continue; }
      const double s = dot(qi, kb + j * dk, dk) * scale;
      if (s > m) m = s;
      score[j] = pow(softplus(s) + 1e-6, tau);
      total += score[j];
    }
    for (int64_t j = 0; j < Tk; ++j) score[j] /= total;
  }
  /* O = A V: each output row is the weighted average of the value rows. */
  for (int64_t d = 0; d < dv; ++d) {
    double acc = 0.0;
    for (int64_t j = 0; j < Tk; ++j) acc += score[j] * vb[j * dv + d];
    out[d] = acc;
  }
  *mass = total;
  *max_score = m;
}

/* Returns 0 on success, -1 on a bad argument, -2 when scratch can't be had. */
static int attn_rows(int variant, int causal, int64_t B, int64_t Hq, int64_t Hkv, int64_t Tq,
                     int64_t Tk, int64_t dk, int64_t dv, const double* q, const double* k,
                     const double* v, const double* b_raw, const double* eps_raw,
                     const double* log_tau, int yat_power, int yat_bias_free,
                     const int64_t* rows, int64_t n_rows, double* out, double* mass,
                     double* max_score) {
  if (B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || Tq < 0 || Tk <= 0 || dk <= 0 ||
      dv <= 0 || (causal && Tq != Tk) || variant < 0 || variant > 2 || yat_power < 1)
    return -1;
  if (variant == ORACLE_YAT && ((!b_raw && !yat_bias_free) || !eps_raw)) return -1;
  if (variant == ORACLE_STAU && !log_tau) return -1;
  const int64_t total_rows = B * Hq * Tq;
  if (!rows) n_rows = total_rows;
  for (int64_t r = 0; rows && r < n_rows; ++r)
    if (rows[r] < 0 || rows[r] >= total_rows) return -1;
  int failed = 0;
#pragma omp parallel
  {
    double* score = (double*)malloc(sizeof(double) * (size_t)Tk);
#pragma omp for schedule(dynamic, 16)
    for (int64_t r = 0; r < n_rows; ++r) {
      if (!score) {
#pragma omp atomic write
        failed = 1;
        continue;
      }
      const int64_t row = rows ? rows[r] : r;
      one_row(variant, causal, Hq, Hkv, Tq, Tk, dk, dv, q, k, v, b_raw, eps_raw, log_tau,
              yat_power, yat_bias_free, row, score, out + r * dv, mass + r, max_score + r);
    }
    free(score);
  }
  return failed ? -2 : 0;
}

int oracle_attn_fwd(int variant, int causal, int64_t B, int64_t Hq, int64_t Hkv,
                    int64_t Tq, int64_t Tk, int64_t dk, int64_t dv, const double* q,
                    const double* k, const double* v, const double* b_raw,
                    const double* eps_raw, const double* log_tau, const int64_t* rows,
                    int64_t n_rows, double* out, double* mass, double* max_score) {
  return attn_rows(variant, causal, B, Hq, Hkv, Tq, Tk, dk, dv, q, k, v, b_raw, eps_raw,
                   log_tau, 1, 0, rows, n_rows, out, mass, max_score);
}

/* The Yat branch with the kernel-family options of [P2']: numerator power
 * m = yat_power >= 1, and b = 0 exactly when yat_bias_free (b_raw unused). */
int oracle_attn_fwd_yat(int causal, int64_t B, int64_t Hq, int64_t Hkv, int64_t Tq,
                        int64_t Tk, int64_t dk, int64_t dv, const double* q, const double* k,
                        const double* v, const double* b_raw, const double* eps_raw,
                        int yat_power, int yat_bias_free, const int64_t* rows,
                        int64_t n_rows, double* out, double* mass, double* max_score) {
  return attn_rows(ORACLE_YAT, causal, B, Hq, Hkv, Tq, Tk, dk, dv, q, k, v, b_raw, eps_raw,
                   NULL, yat_power, yat_bias_free, rows, n_rows, out, mass, max_score);
}

/* Threads the parallel loop above runs on (1 without OpenMP). */
int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
