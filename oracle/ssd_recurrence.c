/*
 * TEST INFRASTRUCTURE ONLY -- the fp64 CPU oracle of the Mamba-2 SSD forward.
 *
 * Only tests/, the smoke check and the benchmark's CPU-baseline leg may load
 * this library.  The GPU library shares no code, header, table or helper with
 * it; this file includes nothing but the C standard library (and OpenMP).
 *
 * What it computes: the selective state space recurrence with a scalar-identity
 * transition, evaluated token by token (the "recurrent mode"), in fp64.
 *   - Recurrence h_t = A_t h_{t-1} + B_t x_t, y_t = C_t h_t:
 *     page "State Space Duality and Mamba-2: Unifying Transformers and
 *     Semiseparable Matrices", section "Mathematical Foundations" (first
 *     equation) and "The Dual Perspectives of Semiseparable Multiplication",
 *     item 1 (recurrent mode).
 *   - Scalar-identity transition A_t = a_t I: same page, section "The
 *     Scalar-Identity Structural Constraint".
 *   - Discretisation a_t = exp(dt_t * A_h): page "Mamba-2 Architecture: State
 *     Space Duality Explained", Step 1 (the chunked code builds its decay as the
 *     exponential of dt times A).  The pages give no discretisation of B and no
 *     skip term; the reading taken is the Euler input weight dt_t on B_t x_t and
 *     a skip D_h x_t, i.e. h_t = exp(dt_t A) h_{t-1} + dt_t x_t B_t^T and
 *     y_t = C_t h_t + D x_t.
 *   - Heads share B and C within a group (grouped-query analogue): same page,
 *     "2. The Chunked SSD Algorithm", item 4.  Head h uses group
 *     g = floor(h * G / H) (consecutive heads share).
 *
 * Per (sequence s, head h), with state H in R^{P x N} (row p, column n):
 *   H_{-1} = h0[s, h] (zeros if h0 is NULL)
 *   for t in the sequence, in order:
 *     a_t     = exp(dt[t,h] * A[h])
 *     H[p,n]  = a_t * H[p,n] + dt[t,h] * x[t,h,p] * B[t,g,n]
 *     y[t,h,p] = sum_n C[t,g,n] * H[p,n] + D[h] * x[t,h,p]
 *   final[s,h] = H after the last token (= h0 for an empty sequence)
 *
 * All arithmetic is fp64; the float32 inputs are upcast exactly.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Evaluate the recurrence for a list of (sequence, head) pairs.
 *
 * seq_off[nseq+1]: token offsets of the sequences (non-decreasing, from 0).
 * x [T,H,P], dt [T,H], A [H], B/C [T,G,N], D [H] or NULL, h0 [nseq,H,P,N] or NULL.
 * pairs [npairs][2] = (s, h); NULL means every pair, in order s-major.
 * y_out: compact, pair k's block is len(s_k) x P doubles, blocks in pair order.
 * h_out: [npairs][P][N] doubles, or NULL.
 * nthreads <= 0: OpenMP default.
 * Returns 0, or -1 for invalid arguments (nothing is written then).
 */
int ssd_oracle_recurrence(int64_t nseq, const int64_t *seq_off, int64_t H, int64_t P,
                          int64_t N, int64_t G, const float *x, const float *dt,
                          const float *A, const float *B, const float *C, const float *D,
                          const float *h0, int64_t npairs, const int64_t *pairs,
                          double *y_out, double *h_out, int nthreads) {
  if (nseq < 0 || H <= 0 || P <= 0 || N <= 0 || G <= 0 || H % G != 0) return -1;
  if (!seq_off || !x || !dt || !A || !B || !C || !y_out) return -1;
  if (seq_off[0] != 0) return -1;
  for (int64_t s = 0; s < nseq; ++s)
    if (seq_off[s + 1] < seq_off[s]) return -1;
  int64_t np = pairs ? npairs : nseq * H;
  if (np < 0) return -1;
  for (int64_t k = 0; pairs && k < np; ++k)
    if (pairs[2 * k] < 0 || pairs[2 * k] >= nseq || pairs[2 * k + 1] < 0 || pairs[2 * k + 1] >= H)
      return -1;

  int64_t *yoff = (int64_t *)malloc((size_t)(np + 1) * sizeof(int64_t));
  if (!yoff) return -1;
  yoff[0] = 0;
  for (int64_t k = 0; k < np; ++k) {
    int64_t s = pairs ? pairs[2 * k] : k / H;
    yoff[k + 1] = yoff[k] + (seq_off[s + 1] - seq_off[s]) * P;
  }

#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel
#endif
  {
    double *st = (double *)malloc((size_t)(P * N) * sizeof(double));
    double *bn = (double *)malloc((size_t)N * sizeof(double));
    double *cn = (double *)malloc((size_t)N * sizeof(double));
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
    for (int64_t k = 0; k < np; ++k) {
      const int64_t s = pairs ? pairs[2 * k] : k / H;
      const int64_t h = pairs ? pairs[2 * k + 1] : k % H;
      const int64_t g = h * G / H;
      const double Ah = (double)A[h];
      const double Dh = D ? (double)D[h] : 0.0;
      if (h0) {
        const float *src = h0 + (size_t)((s * H + h) * P * N);
        for (int64_t i = 0; i < P * N; ++i) st[i] = (double)src[i];
      } else {
        memset(st, 0, (size_t)(P * N) * sizeof(double));
      }
      double *yk = y_out + yoff[k];
      for (int64_t t = seq_off[s]; t < seq_off[s + 1]; ++t) {
        const double dtt = (double)dt[(size_t)(t * H + h)];
        const double a = exp(dtt * Ah);
        const float *bt = B + (size_t)((t * G + g) * N);
        const float *ct = C + (size_t)((t * G + g) * N);
        const float *xt = x + (size_t)((t * H + h) * P);
        for (int64_t n = 0; n < N; ++n) {
          bn[n] = (double)bt[n];
          cn[n] = (double)ct[n];
        }
        double *yt = yk + (t - seq_off[s]) * P;
        for (int64_t p = 0; p < P; ++p) {
          const double xp = (double)xt[p];
          const double u = dtt * xp;
          double *row = st + p * N;
          double acc = 0.0;
          for (int64_t n = 0; n < N; ++n) {
            const double v = a * row[n] + u * bn[n];
            row[n] = v;
            acc += cn[n] * v;
          }
          yt[p] = acc + Dh * xp;
        }
      }
      if (h_out) memcpy(h_out + (size_t)(k * P * N), st, (size_t)(P * N) * sizeof(double));
    }
    free(st);
    free(bn);
    free(cn);
  }
  free(yoff);
  return 0;
}

/* Number of OpenMP threads a parallel region would use (1 without OpenMP). */
int ssd_oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
