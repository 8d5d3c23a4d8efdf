/*
 * TEST INFRASTRUCTURE ONLY -- the fp64 CPU oracle of the SSD forward's
 * gradients (the backward pass).
 *
 * Only tests/ may load this library.  Like ssd_recurrence.c it includes
 * nothing but the C standard library (and OpenMP) and shares nothing with
 * the GPU library.
 *
 * The pages do not give the backward pass (training throughput is claimed,
 * its form is not stated).  It is derived here by the chain rule from the
 * recurrence the forward oracle evaluates (page "State Space Duality and
 * Mamba-2: Unifying Transformers and Semiseparable Matrices", section
 * "Mathematical Foundations", with the scalar-identity transition of "The
 * Scalar-Identity Structural Constraint" and the decay exp(dt A) of page
 * "Mamba-2 Architecture: State Space Duality Explained", Step 1):
 *
 *   a_t = exp(dt_t A),  h_t = a_t h_{t-1} + dt_t x_t B_t^T,  y_t = h_t C_t + D x_t
 *
 * For the scalar loss  L = sum_t <dy_t, y_t> + <dfinal, h_last>,  with
 * g_t = dL/dh_t (a P x N matrix), walking the tokens in reverse:
 *
 *   g_t        = dy_t C_t^T + a_{t+1} g_{t+1}        (g_last starts from dfinal)
 *   dL/dC_t[n] = sum_p dy_t[p] h_t[p,n]
 *   dL/dx_t[p] = D dy_t[p] + dt_t sum_n g_t[p,n] B_t[n]
 *   dL/dB_t[n] = dt_t sum_p g_t[p,n] x_t[p]
 *   dL/ddt_t   = sum_{p,n} g_t[p,n] x_t[p] B_t[n] + A a_t <g_t, h_{t-1}>
 *   dL/dA      = sum_t dt_t a_t <g_t, h_{t-1}>
 *   dL/dD      = sum_t <dy_t, x_t>
 *   dL/dh0     = a_first g_first
 *
 * B and C gradients are returned per head; heads of a group share B and C, so
 * the caller sums them over the group.  The states h_{t-1} are recomputed
 * from checkpoints taken every 64 tokens of a forward sweep.  All arithmetic
 * is fp64; the float32 inputs are upcast exactly.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define KB 64 /* tokens between checkpoints */

/* Gradients for a list of (sequence, head) pairs (NULL: every pair).
 *
 * Inputs as ssd_oracle_recurrence, plus dy [T,H,P] and dfinal [nseq,H,P,N]
 * (NULL: zero).  Outputs (doubles, caller-zeroed, full size; only the pairs'
 * entries are written):
 *   dx [T,H,P], ddt [T,H], dBh [T,H,N], dCh [T,H,N]  (per head),
 *   dA_pair [npairs], dD_pair [npairs], dh0_pair [npairs][P][N].
 * Returns 0, or -1 for invalid arguments.
 */
int ssd_oracle_recurrence_bwd(int64_t nseq, const int64_t *seq_off, int64_t H, int64_t P,
                              int64_t N, int64_t G, const float *x, const float *dt,
                              const float *A, const float *B, const float *C, const float *D,
                              const float *h0, const float *dy, const float *dfinal,
                              int64_t npairs, const int64_t *pairs, double *dx, double *ddt,
                              double *dBh, double *dCh, double *dA_pair, double *dD_pair,
                              double *dh0_pair, int nthreads) {
  if (nseq < 0 || H <= 0 || P <= 0 || N <= 0 || G <= 0 || H % G != 0) return -1;
  if (!seq_off || !x || !dt || !A || !B || !C || !dy) return -1;
  if (!dx || !ddt || !dBh || !dCh || !dA_pair || !dD_pair || !dh0_pair) return -1;
  if (seq_off[0] != 0) return -1;
  for (int64_t s = 0; s < nseq; ++s)
    if (seq_off[s + 1] < seq_off[s]) return -1;
  const int64_t np = pairs ? npairs : nseq * H;
  if (np < 0) return -1;
  for (int64_t k = 0; pairs && k < np; ++k)
    if (pairs[2 * k] < 0 || pairs[2 * k] >= nseq || pairs[2 * k + 1] < 0 || pairs[2 * k + 1] >= H)
      return -1;
  int64_t maxlen = 0;
  for (int64_t s = 0; s < nseq; ++s)
    if (seq_off[s + 1] - seq_off[s] > maxlen) maxlen = seq_off[s + 1] - seq_off[s];
  const int64_t nbmax = (maxlen + KB - 1) / KB + 1;
  const int64_t PN = P * N;

#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel
#endif
  {
    double *ckpt = (double *)malloc((size_t)(nbmax * PN) * sizeof(double));
    double *hs = (double *)malloc((size_t)((KB + 1) * PN) * sizeof(double));
    double *g = (double *)malloc((size_t)PN * sizeof(double));
    double *bn = (double *)malloc((size_t)N * sizeof(double));
    double *cn = (double *)malloc((size_t)N * sizeof(double));
    double *gb = (double *)malloc((size_t)P * sizeof(double));
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
    for (int64_t k = 0; k < np; ++k) {
      const int64_t s = pairs ? pairs[2 * k] : k / H;
      const int64_t h = pairs ? pairs[2 * k + 1] : k % H;
      const int64_t gr = h * G / H;
      const double Ah = (double)A[h];
      const double Dh = D ? (double)D[h] : 0.0;
      const int64_t t0 = seq_off[s], len = seq_off[s + 1] - t0;
      const int64_t nb = (len + KB - 1) / KB;

      /* forward sweep: the state before each block of KB tokens */
      double *st = hs; /* scratch for the sweep */
      if (h0) {
        const float *src = h0 + (size_t)((s * H + h) * PN);
        for (int64_t i = 0; i < PN; ++i) st[i] = (double)src[i];
      } else {
        memset(st, 0, (size_t)PN * sizeof(double));
      }
      for (int64_t i = 0; i < len; ++i) {
        if (i % KB == 0) memcpy(ckpt + (i / KB) * PN, st, (size_t)PN * sizeof(double));
        const int64_t t = t0 + i;
        const double d = (double)dt[(size_t)(t * H + h)];
        const double a = exp(d * Ah);
        const float *bt = B + (size_t)((t * G + gr) * N);
        const float *xt = x + (size_t)((t * H + h) * P);
        for (int64_t p = 0; p < P; ++p) {
          const double u = d * (double)xt[p];
          for (int64_t n = 0; n < N; ++n) st[p * N + n] = a * st[p * N + n] + u * (double)bt[n];
        }
      }

      /* reverse sweep */
      if (dfinal) {
        const float *src = dfinal + (size_t)((s * H + h) * PN);
        for (int64_t i = 0; i < PN; ++i) g[i] = (double)src[i];
      } else {
        memset(g, 0, (size_t)PN * sizeof(double));
      }
      double dA_acc = 0.0, dD_acc = 0.0;
      for (int64_t b = nb - 1; b >= 0; --b) {
        const int64_t i0 = b * KB;
        const int64_t blen = (len - i0 < KB) ? len - i0 : KB;
        /* states before (hs[0]) and after each token of the block */
        memcpy(hs, ckpt + b * PN, (size_t)PN * sizeof(double));
        for (int64_t i = 0; i < blen; ++i) {
          const int64_t t = t0 + i0 + i;
          const double d = (double)dt[(size_t)(t * H + h)];
          const double a = exp(d * Ah);
          const float *bt = B + (size_t)((t * G + gr) * N);
          const float *xt = x + (size_t)((t * H + h) * P);
          const double *prev = hs + i * PN;
          double *next = hs + (i + 1) * PN;
          for (int64_t p = 0; p < P; ++p) {
            const double u = d * (double)xt[p];
            for (int64_t n = 0; n < N; ++n) next[p * N + n] = a * prev[p * N + n] + u * (double)bt[n];
          }
        }
        for (int64_t i = blen - 1; i >= 0; --i) {
          const int64_t t = t0 + i0 + i;
          const double d = (double)dt[(size_t)(t * H + h)];
          const double a = exp(d * Ah);
          const float *bt = B + (size_t)((t * G + gr) * N);
          const float *ct = C + (size_t)((t * G + gr) * N);
          const float *xt = x + (size_t)((t * H + h) * P);
          const float *dyt = dy + (size_t)((t * H + h) * P);
          const double *hprev = hs + i * PN;
          const double *hcur = hs + (i + 1) * PN;
          for (int64_t n = 0; n < N; ++n) {
            bn[n] = (double)bt[n];
            cn[n] = (double)ct[n];
          }
          /* g_t = dy_t C_t^T + (a_{t+1} g_{t+1}, already in g) */
          for (int64_t p = 0; p < P; ++p) {
            const double dyp = (double)dyt[p];
            for (int64_t n = 0; n < N; ++n) g[p * N + n] += dyp * cn[n];
          }
          /* dC_t (this head's share) */
          double *dc = dCh + (size_t)((t * H + h) * N);
          for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t p = 0; p < P; ++p) acc += (double)dyt[p] * hcur[p * N + n];
            dc[n] = acc;
          }
          /* g B_t per row, dx_t, and the x-B term of ddt_t */
          double gxb = 0.0, dd = 0.0;
          double *dxt = dx + (size_t)((t * H + h) * P);
          for (int64_t p = 0; p < P; ++p) {
            double acc = 0.0;
            for (int64_t n = 0; n < N; ++n) acc += g[p * N + n] * bn[n];
            gb[p] = acc;
            dxt[p] = Dh * (double)dyt[p] + d * acc;
            gxb += (double)xt[p] * acc;
            dd += (double)dyt[p] * (double)xt[p];
          }
          /* dB_t (this head's share) */
          double *db = dBh + (size_t)((t * H + h) * N);
          for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t p = 0; p < P; ++p) acc += g[p * N + n] * (double)xt[p];
            db[n] = d * acc;
          }
          /* <g_t, h_{t-1}> */
          double gh = 0.0;
          for (int64_t i2 = 0; i2 < PN; ++i2) gh += g[i2] * hprev[i2];
          ddt[(size_t)(t * H + h)] = gxb + Ah * a * gh;
          dA_acc += d * a * gh;
          dD_acc += dd;
          /* g_{t-1} <- a_t g_t */
          for (int64_t i2 = 0; i2 < PN; ++i2) g[i2] *= a;
        }
      }
      dA_pair[k] = dA_acc;
      dD_pair[k] = dD_acc;
      memcpy(dh0_pair + k * PN, g, (size_t)PN * sizeof(double));
    }
    free(ckpt);
    free(hs);
    free(g);
    free(bn);
    free(cn);
    free(gb);
  }
  return 0;
}
