/*
 * fp64 C oracle of the Gated DeltaNet token mixer: the token-serial
 * recurrence, update form 1, for every (sequence, V head).
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path may link, load or
 * call this file: only tests/, __graft_entry__.smoke() and the cpu_baseline
 * leg of bench.py use it. It shares no code with the HIP library and
 * includes none of its headers.
 *
 * Method source: page "Qwen3.8-Flash-Next 技术总结：Qwen4 架构的'探路者'",
 * section 2.1 "Gated DeltaNet", first form of the state-update equation:
 *
 *     S_t = a_t S_{t-1} + b_t k_t (v_t - a_t S_{t-1}^T k_t)^T
 *
 * with the readings of the NumPy oracle (gdn_oracle.py): readout
 * o_t = S_t^T q_t with the post-update state and no scale (R1); V head h
 * reads QK head h / (h_v / h_qk) (R2); a_t = exp(log_alpha) and b_t per
 * (token, V head) (R3); packed sequences, each from its own initial state
 * or zeros (R4). S is dk x dv, stored row-major (dv fastest).
 *
 * This is the same computation as gdn_oracle.recurrent_form1, written in
 * plain C so that full-size workloads (tens of thousands of tokens, 48
 * heads) finish in seconds: every (sequence, V head) pair is independent
 * and runs on its own thread. Per token it makes three plain passes over
 * the state, in the order of the equation: the prediction p = S^T k, the
 * update S <- a S + k u^T with u = b (v - a p), and the readout o = S^T q.
 * Inputs are float32 (bfloat16 and float32 values convert exactly) and are
 * widened to double on use; outputs are double.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* One (sequence, V head): tokens [t0, t1), QK head g. */
static void run_pair(int64_t t0, int64_t t1, int64_t h, int64_t g, int64_t h_qk, int64_t h_v,
                     int64_t dk, int64_t dv, const float* q, const float* k, const float* v,
                     const float* log_alpha, const float* beta, const double* s0, double* o,
                     double* s_out, double* work) {
  double* S = s_out;                 /* the state lives in the output slot */
  double* kd = work;                 /* k_t [dk] */
  double* qd = kd + dk;              /* q_t [dk] */
  double* p = qd + dk;               /* S^T k_t [dv] */
  double* u = p + dv;                /* b (v - a p) [dv] */
  if (s0)
    memcpy(S, s0, (size_t)(dk * dv) * sizeof(double));
  else
    memset(S, 0, (size_t)(dk * dv) * sizeof(double));
  for (int64_t t = t0; t < t1; ++t) {
    const double a = exp((double)log_alpha[t * h_v + h]);
    const double b = (double)beta[t * h_v + h];
    const float* kt = k + (t * h_qk + g) * dk;
    const float* qt = q + (t * h_qk + g) * dk;
    const float* vt = v + (t * h_v + h) * dv;
    for (int64_t i = 0; i < dk; ++i) {
      kd[i] = (double)kt[i];
      qd[i] = (double)qt[i];
    }
    /* p = S_{t-1}^T k_t */
    for (int64_t j = 0; j < dv; ++j) p[j] = 0.0;
    for (int64_t i = 0; i < dk; ++i)
      for (int64_t j = 0; j < dv; ++j) p[j] += S[i * dv + j] * kd[i];
    /* u = b (v - a p) */
    for (int64_t j = 0; j < dv; ++j) u[j] = b * ((double)vt[j] - a * p[j]);
    /* S_t = a S_{t-1} + k u^T */
    for (int64_t i = 0; i < dk; ++i)
      for (int64_t j = 0; j < dv; ++j) S[i * dv + j] = a * S[i * dv + j] + kd[i] * u[j];
    /* o_t = S_t^T q_t */
    double* ot = o + (t * h_v + h) * dv;
    for (int64_t j = 0; j < dv; ++j) ot[j] = 0.0;
    for (int64_t i = 0; i < dk; ++i)
      for (int64_t j = 0; j < dv; ++j) ot[j] += S[i * dv + j] * qd[i];
  }
}

/*
 * q, k [T, h_qk, dk]; v [T, h_v, dv]; log_alpha, beta [T, h_v] (float32).
 * cu_seqlens [num_seqs + 1] (int64, first 0, non-decreasing, last T), or
 * NULL for one sequence of T tokens. init_state [num_seqs, h_v, dk, dv]
 * (double) or NULL for zeros. o [T, h_v, dv] and final_state
 * [num_seqs, h_v, dk, dv] (double) are written. threads <= 0 means the
 * runtime's default. Returns 0, or -1 for bad sizes or sequence bounds.
 */
int gdn_ref_form1(int64_t total_tokens, int64_t num_seqs, const int64_t* cu_seqlens, int64_t h_qk,
                  int64_t h_v, int64_t dk, int64_t dv, const float* q, const float* k, const float* v,
                  const float* log_alpha, const float* beta, const double* init_state, double* o,
                  double* final_state, int threads) {
  if (total_tokens < 0 || num_seqs < 1 || h_qk < 1 || h_v < 1 || h_v % h_qk || dk < 1 || dv < 1) return -1;
  if (!cu_seqlens && num_seqs != 1) return -1;
  if (cu_seqlens) {
    if (cu_seqlens[0] != 0 || cu_seqlens[num_seqs] != total_tokens) return -1;
    for (int64_t n = 0; n < num_seqs; ++n)
      if (cu_seqlens[n + 1] < cu_seqlens[n]) return -1;
  }
  const int64_t group = h_v / h_qk;
  const int64_t units = num_seqs * h_v;
  int bad = 0;
#ifdef _OPENMP
  if (threads > 0) omp_set_num_threads(threads);
#else
  (void)threads;
#endif
#pragma omp parallel reduction(| : bad)
  {
    double* work = (double*)malloc((size_t)(2 * dk + 2 * dv) * sizeof(double));
    if (!work) bad = 1;
#pragma omp for schedule(dynamic, 1)
    for (int64_t x = 0; x < units; ++x) {
      if (!work) continue;
      const int64_t n = x / h_v, h = x % h_v;
      const int64_t t0 = cu_seqlens ? cu_seqlens[n] : 0;
      const int64_t t1 = cu_seqlens ? cu_seqlens[n + 1] : total_tokens;
      run_pair(t0, t1, h, h / group, h_qk, h_v, dk, dv, q, k, v, log_alpha, beta,
               init_state ? init_state + x * dk * dv : NULL, o, final_state + x * dk * dv, work);
    }
    free(work);
  }
  return bad ? -1 : 0;
}

/* Threads the runtime would use by default (1 without OpenMP). */
int gdn_ref_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
