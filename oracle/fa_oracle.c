/*
 * fa_oracle.c -- CPU oracle for the fused attention forward.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously-correct
 * reference the GPU kernels are checked against.  Only the test suite, the
 * smoke entry point and the benchmark's CPU-baseline leg may load it.  It
 * shares no code, header or table with the HIP library.
 *
 * What it computes -- the plain definition of attention, with the score row
 * materialised in full and the softmax taken in the "safe" form:
 *
 *   "[CS336] Assignment 2: Systems", section "FlashAttention V2 / High level":
 *       S = Q K^T * scale,  P_ij = softmax_j(S)_ij,  O = P V,
 *       L_i = log sum_j exp(S_ij)      (the per-row logsumexp output)
 *   "Understanding Triton Tutorials Part 2", section "Fused Attention 2":
 *       the reference implementation builds the causal mask with a lower
 *       triangle (query i may see key j iff j <= i) and subtracts the row
 *       maximum before exponentiating (safe softmax).
 *
 * Readings taken where the pages are silent (all in double precision):
 *   - causal alignment for seq_q != seq_k is top-left: key j is visible to
 *     query i iff j <= i (the pages' kernels compare absolute indices);
 *   - keys j >= seq_k do not exist: they take no part in max, sum or output;
 *   - the scale multiplies the exact dot product (no rounding of Q first);
 *   - the logsumexp is the natural log, returned in double;
 *   - P is not rounded to a 16-bit type before the product with V.
 *
 * Layout: q [batch, heads, seq_q, head_dim], k and v [batch, heads, seq_k,
 * head_dim], all contiguous double.  Outputs: o [batch, heads, seq_q,
 * head_dim] and lse [batch, heads, seq_q] when rows == NULL; otherwise rows
 * lists n_rows flat query indices ((b*heads + h)*seq_q + i) and o is
 * [n_rows, head_dim], lse [n_rows].  lse may be NULL.
 *
 * Returns 0 on success, -1 on invalid arguments (nothing written).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int fa_oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* One query row: materialise its scores, then max, exp, sum, normalise, P.V. */
static void attend_one_row(const double* q_row, const double* k_head, const double* v_head,
                           int64_t i, int64_t seq_k, int64_t head_dim, double sm_scale,
                           int causal, double* score, double* o_row, double* lse_out) {
  /* the keys this query may see: all j < seq_k, and j <= i when causal */
  int64_t n_visible = seq_k;
  if (causal && i + 1 < n_visible) n_visible = i + 1;

  for (int64_t j = 0; j < n_visible; ++j) {
    const double* k_row = k_head + j * head_dim;
    double dot = 0.0;
    for (int64_t t = 0; t < head_dim; ++t) dot += q_row[t] * k_row[t];
    score[j] = sm_scale * dot;
  }

  double m = score[0];
  for (int64_t j = 1; j < n_visible; ++j)
    if (score[j] > m) m = score[j];

  double l = 0.0;
  for (int64_t j = 0; j < n_visible; ++j) {
    score[j] = exp(score[j] - m); /* unnormalised probability */
    l += score[j];
  }

  for (int64_t t = 0; t < head_dim; ++t) o_row[t] = 0.0;
  for (int64_t j = 0; j < n_visible; ++j) {
    const double p = score[j] / l;
    const double* v_row = v_head + j * head_dim;
    for (int64_t t = 0; t < head_dim; ++t) o_row[t] += p * v_row[t];
  }
  if (lse_out) *lse_out = m + log(l);
}

int fa_oracle_fwd(const double* q, const double* k, const double* v, double* o, double* lse,
                  int64_t batch, int64_t heads, int64_t seq_q, int64_t seq_k, int64_t head_dim,
                  const int64_t* rows, int64_t n_rows, double sm_scale, int causal) {
  if (!q || !k || !v || !o) return -1;
  if (batch < 0 || heads < 0 || seq_q < 0 || seq_k < 1 || head_dim < 1) return -1;
  const int64_t total_rows = batch * heads * seq_q;
  const int64_t n = rows ? n_rows : total_rows;
  if (n < 0) return -1;
  if (rows)
    for (int64_t r = 0; r < n; ++r)
      if (rows[r] < 0 || rows[r] >= total_rows) return -1;

  int failed = 0;
#pragma omp parallel
  {
    double* score = (double*)malloc((size_t)seq_k * sizeof(double));
#pragma omp for schedule(dynamic, 16)
    for (int64_t r = 0; r < n; ++r) {
      if (!score) {
#pragma omp atomic write
        failed = 1;
        continue;
      }
      const int64_t flat = rows ? rows[r] : r;
      const int64_t bh = flat / seq_q;
      const int64_t i = flat % seq_q;
      attend_one_row(q + flat * head_dim, k + bh * seq_k * head_dim, v + bh * seq_k * head_dim,
                     i, seq_k, head_dim, sm_scale, causal, score, o + r * head_dim,
                     lse ? lse + r : NULL);
    }
    free(score);
  }
  return failed ? -2 : 0;
}
