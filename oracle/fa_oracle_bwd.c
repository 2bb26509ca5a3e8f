/*
 * fa_oracle_bwd.c -- CPU oracle for the gradients of the fused attention.
 *
 * TEST INFRASTRUCTURE ONLY.  The slow, obviously-correct reference the GPU
 * backward kernels are checked against.  Only the test suite and the
 * benchmark's CPU-baseline leg may load it.  It shares no code, header or
 * table with the HIP library (nor with fa_oracle.c: it recomputes the
 * forward quantities it needs from their definition).
 *
 * What it computes, in double precision, per (batch, head):
 *
 *   "[CS336] Assignment 2: Systems", section "FlashAttention V2" (the
 *   standard backward and its recomputation form):
 *       S = scale * Q K^T,  P_ij = exp(S_ij - L_i),  L_i = log sum_j exp(S_ij)
 *       D_i  = sum_t dO_it O_it            (O = P V; equals rowsum(P o dP))
 *       dV   = P^T dO,        dP = dO V^T
 *       dS_ij = P_ij (dP_ij - D_i)
 *       dQ   = scale * dS K,  dK = scale * dS^T Q
 *   with the page's 1/sqrt(d) generalised to the explicit scale argument.
 *   L and O are recomputed here from Q, K, V with the row of scores
 *   materialised (safe softmax); nothing is taken from the GPU.
 *
 * Readings (as for the forward): top-left causal alignment (key j visible to
 * query i iff j <= i), keys j >= seq_k do not exist, natural log, and no
 * rounding of P or dS to a 16-bit type.
 *
 * Layout: q, dout [batch, heads, seq_q, head_dim]; k, v [batch, heads, seq_k,
 * head_dim]; all contiguous double.  Every entry point returns 0 on success,
 * -1 on invalid arguments (nothing written), -2 if a work buffer could not be
 * allocated.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static int64_t visible_keys(int64_t i, int64_t seq_k, int causal) {
  int64_t n = seq_k;
  if (causal && i + 1 < n) n = i + 1;
  return n;
}

/* Row i of one head: L_i (logsumexp of the scaled scores), O_i and
 * D_i = dO_i . O_i.  score must hold seq_k doubles. */
static void row_forward(const double* q_row, const double* k_head, const double* v_head,
                        const double* do_row, int64_t i, int64_t seq_k, int64_t head_dim,
                        double sm_scale, int causal, double* score, double* o_row, double* L_out,
                        double* D_out) {
  const int64_t n = visible_keys(i, seq_k, causal);
  for (int64_t j = 0; j < n; ++j) {
    double dot = 0.0;
    for (int64_t t = 0; t < head_dim; ++t) dot += q_row[t] * k_head[j * head_dim + t];
    score[j] = sm_scale * dot;
  }
  double m = score[0];
  for (int64_t j = 1; j < n; ++j)
    if (score[j] > m) m = score[j];
  double l = 0.0;
  for (int64_t j = 0; j < n; ++j) l += exp(score[j] - m);
  const double L = m + log(l);
  for (int64_t t = 0; t < head_dim; ++t) o_row[t] = 0.0;
  for (int64_t j = 0; j < n; ++j) {
    const double p = exp(score[j] - L);
    for (int64_t t = 0; t < head_dim; ++t) o_row[t] += p * v_head[j * head_dim + t];
  }
  double D = 0.0;
  for (int64_t t = 0; t < head_dim; ++t) D += do_row[t] * o_row[t];
  *L_out = L;
  *D_out = D;
}

/* Contribution of the pair (query i, key j) given L_i and D_i:
 * returns P_ij and writes dS_ij. */
static double pair_grad(const double* q_row, const double* k_row, const double* v_row,
                        const double* do_row, double L, double D, int64_t head_dim,
                        double sm_scale, double* ds_out) {
  double s = 0.0, dp = 0.0;
  for (int64_t t = 0; t < head_dim; ++t) {
    s += q_row[t] * k_row[t];
    dp += do_row[t] * v_row[t];
  }
  const double p = exp(sm_scale * s - L);
  *ds_out = p * (dp - D);
  return p;
}

static int check_shape(int64_t batch, int64_t heads, int64_t seq_q, int64_t seq_k,
                       int64_t head_dim) {
  return batch >= 0 && heads >= 0 && seq_q >= 0 && seq_k >= 1 && head_dim >= 1;
}

/* Full gradients: dq [B,H,Sq,D], dk and dv [B,H,Sk,D]; delta [B,H,Sq] (the
 * D_i above) when not NULL.  Parallel over (batch, head). */
int fa_oracle_bwd(const double* q, const double* k, const double* v, const double* dout,
                  double* dq, double* dk, double* dv, double* delta, int64_t batch,
                  int64_t heads, int64_t seq_q, int64_t seq_k, int64_t head_dim,
                  double sm_scale, int causal) {
  if (!q || !k || !v || !dout || !dq || !dk || !dv) return -1;
  if (!check_shape(batch, heads, seq_q, seq_k, head_dim)) return -1;
  const int64_t n_bh = batch * heads;
  int failed = 0;
#pragma omp parallel
  {
    double* score = (double*)malloc((size_t)seq_k * sizeof(double));
    double* o_row = (double*)malloc((size_t)head_dim * sizeof(double));
#pragma omp for schedule(dynamic, 1)
    for (int64_t bh = 0; bh < n_bh; ++bh) {
      if (!score || !o_row) {
#pragma omp atomic write
        failed = 1;
        continue;
      }
      const double* qh = q + bh * seq_q * head_dim;
      const double* doh = dout + bh * seq_q * head_dim;
      const double* kh = k + bh * seq_k * head_dim;
      const double* vh = v + bh * seq_k * head_dim;
      double* dqh = dq + bh * seq_q * head_dim;
      double* dkh = dk + bh * seq_k * head_dim;
      double* dvh = dv + bh * seq_k * head_dim;
      memset(dqh, 0, (size_t)(seq_q * head_dim) * sizeof(double));
      memset(dkh, 0, (size_t)(seq_k * head_dim) * sizeof(double));
      memset(dvh, 0, (size_t)(seq_k * head_dim) * sizeof(double));
      for (int64_t i = 0; i < seq_q; ++i) {
        const double* q_row = qh + i * head_dim;
        const double* do_row = doh + i * head_dim;
        double L, D;
        row_forward(q_row, kh, vh, do_row, i, seq_k, head_dim, sm_scale, causal, score, o_row,
                    &L, &D);
        if (delta) delta[bh * seq_q + i] = D;
        const int64_t n = visible_keys(i, seq_k, causal);
        for (int64_t j = 0; j < n; ++j) {
          const double* k_row = kh + j * head_dim;
          double ds;
          const double p =
              pair_grad(q_row, k_row, vh + j * head_dim, do_row, L, D, head_dim, sm_scale, &ds);
          for (int64_t t = 0; t < head_dim; ++t) {
            dqh[i * head_dim + t] += sm_scale * ds * k_row[t];
            dkh[j * head_dim + t] += sm_scale * ds * q_row[t];
            dvh[j * head_dim + t] += p * do_row[t];
          }
        }
      }
    }
    free(score);
    free(o_row);
  }
  return failed ? -2 : 0;
}

/* dQ of selected flat query rows ((b*H + h)*Sq + i): dq [n_rows, D]. */
int fa_oracle_bwd_dq_rows(const double* q, const double* k, const double* v, const double* dout,
                          const int64_t* rows, int64_t n_rows, double* dq, int64_t batch,
                          int64_t heads, int64_t seq_q, int64_t seq_k, int64_t head_dim,
                          double sm_scale, int causal) {
  if (!q || !k || !v || !dout || !rows || !dq || n_rows < 0) return -1;
  if (!check_shape(batch, heads, seq_q, seq_k, head_dim)) return -1;
  const int64_t total = batch * heads * seq_q;
  for (int64_t r = 0; r < n_rows; ++r)
    if (rows[r] < 0 || rows[r] >= total) return -1;
  int failed = 0;
#pragma omp parallel
  {
    double* score = (double*)malloc((size_t)seq_k * sizeof(double));
    double* o_row = (double*)malloc((size_t)head_dim * sizeof(double));
#pragma omp for schedule(dynamic, 4)
    for (int64_t r = 0; r < n_rows; ++r) {
      if (!score || !o_row) {
#pragma omp atomic write
        failed = 1;
        continue;
      }
      const int64_t bh = rows[r] / seq_q, i = rows[r] % seq_q;
      const double* q_row = q + rows[r] * head_dim;
      const double* do_row = dout + rows[r] * head_dim;
      const double* kh = k + bh * seq_k * head_dim;
      const double* vh = v + bh * seq_k * head_dim;
      double L, D;
      row_forward(q_row, kh, vh, do_row, i, seq_k, head_dim, sm_scale, causal, score, o_row, &L,
                  &D);
      double* out = dq + r * head_dim;
      for (int64_t t = 0; t < head_dim; ++t) out[t] = 0.0;
      const int64_t n = visible_keys(i, seq_k, causal);
      for (int64_t j = 0; j < n; ++j) {
        double ds;
        pair_grad(q_row, kh + j * head_dim, vh + j * head_dim, do_row, L, D, head_dim, sm_scale,
                  &ds);
        for (int64_t t = 0; t < head_dim; ++t) out[t] += sm_scale * ds * kh[j * head_dim + t];
      }
    }
    free(score);
    free(o_row);
  }
  return failed ? -2 : 0;
}

/* dK and dV of selected flat key rows ((b*H + h)*Sk + j): dk, dv [n_keys, D].
 * L and D of the query rows that see a selected key (every row of its head,
 * or rows i >= the head's smallest selected key when causal) are computed
 * first. */
int fa_oracle_bwd_dkv_rows(const double* q, const double* k, const double* v, const double* dout,
                           const int64_t* keys, int64_t n_keys, double* dk, double* dv,
                           int64_t batch, int64_t heads, int64_t seq_q, int64_t seq_k,
                           int64_t head_dim, double sm_scale, int causal) {
  if (!q || !k || !v || !dout || !keys || !dk || !dv || n_keys < 0) return -1;
  if (!check_shape(batch, heads, seq_q, seq_k, head_dim)) return -1;
  const int64_t n_bh = batch * heads;
  for (int64_t r = 0; r < n_keys; ++r)
    if (keys[r] < 0 || keys[r] >= n_bh * seq_k) return -1;
  /* first query row needed per head (seq_q: none) */
  int64_t* need = (int64_t*)malloc((size_t)(n_bh > 0 ? n_bh : 1) * sizeof(int64_t));
  double* Lall = (double*)malloc((size_t)(n_bh * seq_q + 1) * sizeof(double));
  double* Dall = (double*)malloc((size_t)(n_bh * seq_q + 1) * sizeof(double));
  if (!need || !Lall || !Dall) {
    free(need);
    free(Lall);
    free(Dall);
    return -2;
  }
  for (int64_t bh = 0; bh < n_bh; ++bh) need[bh] = seq_q;
  for (int64_t r = 0; r < n_keys; ++r) {
    const int64_t bh = keys[r] / seq_k, first = causal ? keys[r] % seq_k : 0;
    if (first < need[bh]) need[bh] = first;
  }
  int failed = 0;
#pragma omp parallel
  {
    double* score = (double*)malloc((size_t)seq_k * sizeof(double));
    double* o_row = (double*)malloc((size_t)head_dim * sizeof(double));
#pragma omp for schedule(dynamic, 16)
    for (int64_t flat = 0; flat < n_bh * seq_q; ++flat) {
      const int64_t bh = flat / seq_q, i = flat % seq_q;
      if (i < need[bh]) continue;
      if (!score || !o_row) {
#pragma omp atomic write
        failed = 1;
        continue;
      }
      row_forward(q + flat * head_dim, k + bh * seq_k * head_dim, v + bh * seq_k * head_dim,
                  dout + flat * head_dim, i, seq_k, head_dim, sm_scale, causal, score, o_row,
                  &Lall[flat], &Dall[flat]);
    }
#pragma omp for schedule(dynamic, 4)
    for (int64_t r = 0; r < n_keys; ++r) {
      const int64_t bh = keys[r] / seq_k, j = keys[r] % seq_k;
      const double* k_row = k + keys[r] * head_dim;
      const double* v_row = v + keys[r] * head_dim;
      double* dk_out = dk + r * head_dim;
      double* dv_out = dv + r * head_dim;
      for (int64_t t = 0; t < head_dim; ++t) dk_out[t] = dv_out[t] = 0.0;
      /* queries that see key j: all i, or i >= j when causal */
      for (int64_t i = causal ? j : 0; i < seq_q; ++i) {
        const int64_t flat = bh * seq_q + i;
        const double* q_row = q + flat * head_dim;
        const double* do_row = dout + flat * head_dim;
        double ds;
        const double p = pair_grad(q_row, k_row, v_row, do_row, Lall[flat], Dall[flat],
                                   head_dim, sm_scale, &ds);
        for (int64_t t = 0; t < head_dim; ++t) {
          dk_out[t] += sm_scale * ds * q_row[t];
          dv_out[t] += p * do_row[t];
        }
      }
    }
    free(score);
    free(o_row);
  }
  free(need);
  free(Lall);
  free(Dall);
  return failed ? -2 : 0;
}
