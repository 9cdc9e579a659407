/*
 * KDA oracle: the channel-wise gated delta rule evaluated token by token in
 * float64 on the CPU.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the correctness reference for the
 * HIP library; only the test suite, the smoke check and the CPU-baseline leg
 * of the benchmark may build, load or call it.  It shares no code, header or
 * constant with the HIP path.
 *
 * Definition followed (Kimi Linear report as summarised on the pages):
 *   "Kimi Linear" notes (docsaid.org), section "KDA: Splitting the Decay
 *   Across Channels", and the greeksharifa.github.io summary, section 3
 *   "Kimi Delta Attention":
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *     o_t = S_t^T q_t,            alpha_t = exp(g_t) (per key channel)
 *
 * The state is decayed first, then the delta-rule correction and write are
 * applied, and the output is read from the updated state.  Written out per
 * token this is:
 *
 *     S[i][:] *= exp(g_t[i])               (forget, one factor per key row)
 *     u       = beta_t * (v_t - S^T k_t)   (delta-rule pseudo-value)
 *     S      += k_t u^T                    (= (I - b k k^T) S + b k v^T)
 *     o_t     = S^T q_t
 *
 * Layouts: token-major q,k,g [T_total, H, dk], v [T_total, H, dv],
 * beta [T_total, H], o [T_total, H, dv]; states [N, H, dk, dv] with dv
 * contiguous.  Sequence n covers tokens [cu[n], cu[n+1]).
 *
 * Parallelism: OpenMP over (sequence, head, block of 16 value columns).
 * Every value column of S evolves independently of the others, and each
 * column's sums run over the key index in the same order for any split, so
 * the split changes no arithmetic.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define COLS_PER_TASK 16

int kda_oracle_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Returns 0 on success, -1 on bad arguments. */
int kda_oracle_prefill(const double* q, const double* k, const double* v,
                       const double* g, const double* beta,
                       const double* initial_state, double* final_state,
                       double* o, const int64_t* cu_seqlens, int N, int H,
                       int dk, int dv, int nthreads) {
  if (!q || !k || !v || !g || !beta || !o || !cu_seqlens) return -1;
  if (N < 0 || H <= 0 || dk <= 0 || dv <= 0) return -1;
  for (int n = 0; n < N; ++n)
    if (cu_seqlens[n + 1] < cu_seqlens[n] || cu_seqlens[n] < 0) return -1;

  const int col_tasks = (dv + COLS_PER_TASK - 1) / COLS_PER_TASK;
  const int64_t ntasks = (int64_t)N * H * col_tasks;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif

#pragma omp parallel
  {
    double* S = (double*)malloc(sizeof(double) * (size_t)dk * COLS_PER_TASK);
    double* alpha = (double*)malloc(sizeof(double) * (size_t)dk);
#pragma omp for schedule(dynamic, 1)
    for (int64_t task = 0; task < ntasks; ++task) {
      const int n = (int)(task / ((int64_t)H * col_tasks));
      const int h = (int)((task / col_tasks) % H);
      const int c0 = (int)(task % col_tasks) * COLS_PER_TASK;
      const int nc = (dv - c0) < COLS_PER_TASK ? (dv - c0) : COLS_PER_TASK;
      const size_t sbase = ((size_t)n * H + h) * (size_t)dk * dv;

      /* S <- initial state (or zeros). */
      for (int i = 0; i < dk; ++i)
        for (int j = 0; j < nc; ++j)
          S[i * COLS_PER_TASK + j] =
              initial_state ? initial_state[sbase + (size_t)i * dv + c0 + j] : 0.0;

      for (int64_t t = cu_seqlens[n]; t < cu_seqlens[n + 1]; ++t) {
        const double* qt = q + ((size_t)t * H + h) * dk;
        const double* kt = k + ((size_t)t * H + h) * dk;
        const double* gt = g + ((size_t)t * H + h) * dk;
        const double* vt = v + ((size_t)t * H + h) * dv;
        const double bt = beta[(size_t)t * H + h];
        double* ot = o + ((size_t)t * H + h) * dv;

        /* Forget: Diag(alpha_t) S, alpha_t = exp(g_t). */
        for (int i = 0; i < dk; ++i) alpha[i] = exp(gt[i]);
        for (int i = 0; i < dk; ++i)
          for (int j = 0; j < nc; ++j) S[i * COLS_PER_TASK + j] *= alpha[i];

        for (int j = 0; j < nc; ++j) {
          /* Prediction S^T k_t for this value column. */
          double pred = 0.0;
          for (int i = 0; i < dk; ++i) pred += S[i * COLS_PER_TASK + j] * kt[i];
          /* Pseudo-value and rank-1 write. */
          const double u = bt * (vt[c0 + j] - pred);
          for (int i = 0; i < dk; ++i) S[i * COLS_PER_TASK + j] += kt[i] * u;
          /* Output from the updated state. */
          double out = 0.0;
          for (int i = 0; i < dk; ++i) out += S[i * COLS_PER_TASK + j] * qt[i];
          ot[c0 + j] = out;
        }
      }

      if (final_state)
        for (int i = 0; i < dk; ++i)
          for (int j = 0; j < nc; ++j)
            final_state[sbase + (size_t)i * dv + c0 + j] = S[i * COLS_PER_TASK + j];
    }
    free(S);
    free(alpha);
  }
  return 0;
}
