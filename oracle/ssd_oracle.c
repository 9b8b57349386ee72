/*
 * CPU oracle for the Mamba-2 SSD scan: the token-by-token recurrence in fp64.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The GPU library never
 * links, includes or calls it, and it shares no code with the GPU library.
 *
 * What it computes ("Compiler-First State Space Duality and Portable O(1)
 * Autoregressive Caching", Background, Eq. 1 and Eq. 2, and the O(1) cache
 * section): a diagonal-per-head discrete SSM whose input matrix B, output
 * matrix C and step size Delta depend on the token (Mamba-2 selectivity, same
 * section), run one token at a time:
 *
 *   z_t   = dt[b,t,h] + dt_bias[h]
 *   d_t   = clip(softplus(z_t), dt_min, dt_max)   (softplus optional)
 *   abar  = exp(d_t * A[h])                         (A[h] < 0, scalar per head)
 *   h_t[p,n] = abar * h_{t-1}[p,n] + d_t * x[b,t,h,p] * B[b,t,g,n]
 *   y[b,t,h,p] = sum_n C[b,t,g,n] * h_t[p,n] + D[h] * x[b,t,h,p]
 *
 * with g = h / (H/G) the B/C group of head h and h_{-1} = h0 (or zeros).
 * The page states zero-order-hold discretisation but its equation was lost;
 * the reading taken here is Abar = exp(Delta*A) and Bbar = Delta*B, the form
 * whose unrolled kernel is the decay-only lower-triangular matrix of the dual
 * form (Eq. 3 and the "diagonal state matrix" property).
 *
 * Every input is a float32 array (bfloat16 inputs are upcast exactly before
 * the call); every operation is carried out in double.  Layouts are dense,
 * row-major: x,y [Bt,T,H,P]; dt [Bt,T,H]; A, D, dt_bias [H];
 * B, C [Bt,T,G,N]; h0, final [Bt,H,P,N].
 *
 * Independent (b,h) pairs run in parallel with OpenMP; each pair runs serially
 * in token order, so the result does not depend on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double softplus_exact(double z) {
  /* log(1 + e^z) written so that neither branch overflows */
  return (z > 0.0 ? z : 0.0) + log1p(exp(-fabs(z)));
}

int ssd_oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Returns 0 on success, 1 on a bad argument, 2 when scratch allocation fails. */
int ssd_oracle_scan(int64_t Bt, int64_t T, int64_t H, int64_t P, int64_t N, int64_t G,
                    const float* x, const float* dt, const float* dt_bias,
                    const float* A, const float* Bm, const float* Cm, const float* D,
                    const double* h0, int dt_softplus, double dt_min, double dt_max,
                    double* y, double* final_state, int nthreads) {
  if (Bt < 0 || T < 0 || H <= 0 || P <= 0 || N <= 0 || G <= 0 || H % G != 0) return 1;
  if (!A || (T > 0 && (!x || !dt || !Bm || !Cm || !y))) return 1;
  const int64_t heads_per_group = H / G;
  const int64_t npairs = Bt * H;
  int failed = 0;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel
#endif
  {
    double* S = (double*)malloc(sizeof(double) * (size_t)(P * N));
    if (!S) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
      failed = 1;
    }
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
    for (int64_t pair = 0; pair < npairs; ++pair) {
      if (!S) continue;
      const int64_t b = pair / H, h = pair % H, g = h / heads_per_group;
      if (h0)
        memcpy(S, h0 + (size_t)((b * H + h) * P * N), sizeof(double) * (size_t)(P * N));
      else
        memset(S, 0, sizeof(double) * (size_t)(P * N));
      const double Ah = (double)A[h];
      const double Dh = D ? (double)D[h] : 0.0;
      const double bias = dt_bias ? (double)dt_bias[h] : 0.0;
      for (int64_t t = 0; t < T; ++t) {
        double z = (double)dt[(b * T + t) * H + h] + bias;
        double d = dt_softplus ? softplus_exact(z) : z;
        if (d < dt_min) d = dt_min;
        if (d > dt_max) d = dt_max;
        const double abar = exp(d * Ah);
        const float* xt = x + (size_t)(((b * T + t) * H + h) * P);
        const float* Bt_ = Bm + (size_t)(((b * T + t) * G + g) * N);
        const float* Ct_ = Cm + (size_t)(((b * T + t) * G + g) * N);
        double* yt = y + (size_t)(((b * T + t) * H + h) * P);
        for (int64_t p = 0; p < P; ++p) {
          const double dx = d * (double)xt[p];
          double* Sp = S + p * N;
          double acc = 0.0;
          for (int64_t n = 0; n < N; ++n) {
            Sp[n] = abar * Sp[n] + dx * (double)Bt_[n];
            acc += (double)Ct_[n] * Sp[n];
          }
          yt[p] = acc + Dh * (double)xt[p];
        }
      }
      if (final_state)
        memcpy(final_state + (size_t)((b * H + h) * P * N), S, sizeof(double) * (size_t)(P * N));
    }
    free(S);
  }
  return failed ? 2 : 0;
}

/*
 * Depthwise causal convolution over time, the step that precedes the SSD scan
 * in a Mamba-2 block ("Compiler-First State Space Duality and Portable O(1)
 * Autoregressive Caching", O(1) cache: decoding updates a depthwise convolution
 * over a sliding window of the k-1 previous inputs, held in a cache of shape
 * (B, D_conv, k-1); Setup: kernel size k = 4).  Per batch row b and channel c,
 * with the window w[c][0..k-1] applied oldest input first:
 *
 *   xp[j] = state_in[b][c][j]          for j < k-1     (zeros if no state)
 *   xp[j] = x[b][j-(k-1)][c]           for k-1 <= j < k-1+T
 *   z[t]  = bias[c] + sum_{i<k} w[c][i] * xp[t+i]
 *   y[b][t][c] = silu ? z / (1 + exp(-z)) : z
 *   state_out[b][c][i] = xp[T+i]       for i < k-1     (the last k-1 inputs)
 *
 * Layouts: x, y [Bt,T,D]; w [D,k]; bias [D]; states [Bt,D,k-1].  Inputs are
 * float32 values (bfloat16 upcast exactly), states and outputs double, every
 * operation in double.  (b, c) pairs run in parallel; each is serial in t.
 * Returns 0 on success, 1 on a bad argument, 2 when scratch allocation fails.
 */
int ssd_oracle_conv1d(int64_t Bt, int64_t T, int64_t D, int64_t K, const float* x,
                      const float* w, const float* bias, const double* state_in, int silu,
                      double* y, double* state_out, int nthreads) {
  if (Bt < 0 || T < 0 || D <= 0 || K <= 0 || !w) return 1;
  if (T > 0 && (!x || !y)) return 1;
  const int64_t npairs = Bt * D;
  int failed = 0;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel
#endif
  {
    double* xp = (double*)malloc(sizeof(double) * (size_t)(K - 1 + T + 1));
    if (!xp) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
      failed = 1;
    }
#ifdef _OPENMP
#pragma omp for schedule(static)
#endif
    for (int64_t pair = 0; pair < npairs; ++pair) {
      if (!xp) continue;
      const int64_t b = pair / D, c = pair % D;
      for (int64_t j = 0; j < K - 1; ++j)
        xp[j] = state_in ? state_in[(b * D + c) * (K - 1) + j] : 0.0;
      for (int64_t t = 0; t < T; ++t) xp[K - 1 + t] = (double)x[(b * T + t) * D + c];
      for (int64_t t = 0; t < T; ++t) {
        double z = bias ? (double)bias[c] : 0.0;
        for (int64_t i = 0; i < K; ++i) z += (double)w[c * K + i] * xp[t + i];
        y[(b * T + t) * D + c] = silu ? z / (1.0 + exp(-z)) : z;
      }
      if (state_out)
        for (int64_t i = 0; i < K - 1; ++i) state_out[(b * D + c) * (K - 1) + i] = xp[T + i];
    }
    free(xp);
  }
  return failed ? 2 : 0;
}

/*
 * Gradients of the scan (the backward pass of a training step; Results and
 * Setup of "Compiler-First State Space Duality and Portable O(1)
 * Autoregressive Caching" time the forward only, the training step is the
 * pages' stated next use).  For the loss L = sum(dy * y) + sum(dfinal * final)
 * the adjoint of the recurrence above runs backwards in time with
 * G_t = dL/dh_t:
 *
 *   G_{T-1} = dfinal;   for t = T-1 .. 0:
 *     G      += dy_t (x) C_t                         (G = dL/dh_t)
 *     dC_t[n] += sum_p dy_t[p] h_t[p,n]              (summed over a group's heads)
 *     dx_t[p]  = d_t sum_n G[p,n] B_t[n] + D dy_t[p]
 *     dB_t[n] += d_t sum_p G[p,n] x_t[p]             (summed over a group's heads)
 *     dd_t     = sum_{p,n} G[p,n] x_t[p] B_t[n] + A abar_t sum_{p,n} G[p,n] h_{t-1}[p,n]
 *     dA      += d_t abar_t sum_{p,n} G[p,n] h_{t-1}[p,n]
 *     dD      += sum_p dy_t[p] x_t[p]
 *     G       *= abar_t                              (G = dL/dh_{t-1})
 *   dh0 = G;  ddt_t = dd_t * softplus'(z_t) where lo <= softplus(z_t) <= hi, else 0
 *   (dlda, if not NULL, receives dL/d(d_t A) = abar_t sum G h_{t-1} per token)
 *   (softplus'(z) = 1 / (1 + exp(-z)); without softplus, 1); ddt_bias = sum_t ddt_t.
 *
 * The states h_t are recomputed segment by segment (SEG tokens) from
 * checkpoints taken on a forward pass, all in double.  Per-head partial dB and
 * dC are summed over the heads of a group after the parallel loop.
 * Returns 0 on success, 1 on a bad argument, 2 when scratch allocation fails.
 */
int ssd_oracle_scan_backward(int64_t Bt, int64_t T, int64_t H, int64_t P, int64_t N, int64_t G,
                             const float* x, const float* dt, const float* dt_bias,
                             const float* A, const float* Bm, const float* Cm, const float* D,
                             const double* h0, int dt_softplus, double dt_min, double dt_max,
                             const double* dy, const double* dfinal,
                             double* dx, double* ddt, double* dA, double* dB, double* dC,
                             double* dD, double* ddt_bias, double* dh0, double* dlda,
                             int nthreads) {
  enum { SEG = 64 };
  if (Bt < 0 || T < 0 || H <= 0 || P <= 0 || N <= 0 || G <= 0 || H % G != 0) return 1;
  if (!A || !dA || !dD || !ddt_bias || !dh0) return 1;
  if (T > 0 && (!x || !dt || !Bm || !Cm || !dy || !dx || !ddt || !dB || !dC)) return 1;
  const int64_t hpg = H / G, npairs = Bt * H, PN = P * N;
  const int64_t nseg = (T + SEG - 1) / SEG;
  /* per-head partials of dB and dC: [Bt,T,H,N] */
  double* dBh = (double*)calloc((size_t)(Bt * T * H * N) + 1, sizeof(double));
  double* dCh = (double*)calloc((size_t)(Bt * T * H * N) + 1, sizeof(double));
  double* dAh = (double*)calloc((size_t)(Bt * H) + 1, sizeof(double));
  double* dDh = (double*)calloc((size_t)(Bt * H) + 1, sizeof(double));
  double* dbh = (double*)calloc((size_t)(Bt * H) + 1, sizeof(double));
  if (!dBh || !dCh || !dAh || !dDh || !dbh) {
    free(dBh); free(dCh); free(dAh); free(dDh); free(dbh);
    return 2;
  }
  int failed = 0;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel
#endif
  {
    double* ck = (double*)malloc(sizeof(double) * (size_t)((nseg + 1) * PN));
    double* hs = (double*)malloc(sizeof(double) * (size_t)((SEG + 1) * PN));
    double* Gm = (double*)malloc(sizeof(double) * (size_t)PN);
    double* dv = (double*)malloc(sizeof(double) * (size_t)(T + 1));
    double* zv = (double*)malloc(sizeof(double) * (size_t)(T + 1));
    if (!ck || !hs || !Gm || !dv || !zv) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
      failed = 1;
    }
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
    for (int64_t pair = 0; pair < npairs; ++pair) {
      if (!ck || !hs || !Gm || !dv || !zv) continue;
      const int64_t b = pair / H, h = pair % H, g = h / hpg;
      const double Ah = (double)A[h];
      const double Dh = D ? (double)D[h] : 0.0;
      const double bias = dt_bias ? (double)dt_bias[h] : 0.0;
      for (int64_t t = 0; t < T; ++t) {
        const double z = (double)dt[(b * T + t) * H + h] + bias;
        double d = dt_softplus ? softplus_exact(z) : z;
        zv[t] = z;
        if (d < dt_min) d = dt_min;
        if (d > dt_max) d = dt_max;
        dv[t] = d;
      }
      /* forward: checkpoint the state entering every segment */
      double* hcur = ck;
      if (h0)
        memcpy(hcur, h0 + (size_t)((b * H + h) * PN), sizeof(double) * (size_t)PN);
      else
        memset(hcur, 0, sizeof(double) * (size_t)PN);
      for (int64_t s = 0; s < nseg; ++s) {
        double* hn = ck + (s + 1) * PN;
        memcpy(hn, ck + s * PN, sizeof(double) * (size_t)PN);
        for (int64_t t = s * SEG; t < T && t < (s + 1) * SEG; ++t) {
          const double abar = exp(dv[t] * Ah);
          const float* xt = x + (size_t)(((b * T + t) * H + h) * P);
          const float* Bt_ = Bm + (size_t)(((b * T + t) * G + g) * N);
          for (int64_t p = 0; p < P; ++p)
            for (int64_t n = 0; n < N; ++n)
              hn[p * N + n] = abar * hn[p * N + n] + dv[t] * (double)xt[p] * (double)Bt_[n];
        }
      }
      /* reverse */
      if (dfinal)
        memcpy(Gm, dfinal + (size_t)((b * H + h) * PN), sizeof(double) * (size_t)PN);
      else
        memset(Gm, 0, sizeof(double) * (size_t)PN);
      double dA_acc = 0.0, dD_acc = 0.0, db_acc = 0.0;
      for (int64_t s = nseg - 1; s >= 0; --s) {
        const int64_t t0 = s * SEG, t1 = (T < (s + 1) * SEG ? T : (s + 1) * SEG);
        /* hs[k] = state after token t0 + k - 1 (hs[0] = entering state) */
        memcpy(hs, ck + s * PN, sizeof(double) * (size_t)PN);
        for (int64_t t = t0; t < t1; ++t) {
          const double abar = exp(dv[t] * Ah);
          const float* xt = x + (size_t)(((b * T + t) * H + h) * P);
          const float* Bt_ = Bm + (size_t)(((b * T + t) * G + g) * N);
          const double* hp = hs + (t - t0) * PN;
          double* hn = hs + (t - t0 + 1) * PN;
          for (int64_t p = 0; p < P; ++p)
            for (int64_t n = 0; n < N; ++n)
              hn[p * N + n] = abar * hp[p * N + n] + dv[t] * (double)xt[p] * (double)Bt_[n];
        }
        for (int64_t t = t1 - 1; t >= t0; --t) {
          const double abar = exp(dv[t] * Ah);
          const double d = dv[t];
          const float* xt = x + (size_t)(((b * T + t) * H + h) * P);
          const float* Bt_ = Bm + (size_t)(((b * T + t) * G + g) * N);
          const float* Ct_ = Cm + (size_t)(((b * T + t) * G + g) * N);
          const double* dyt = dy + (size_t)(((b * T + t) * H + h) * P);
          const double* hprev = hs + (t - t0) * PN;
          const double* hcur2 = hs + (t - t0 + 1) * PN;
          double* dxt = dx + (size_t)(((b * T + t) * H + h) * P);
          double* dBt = dBh + (size_t)(((b * T + t) * H + h) * N);
          double* dCt = dCh + (size_t)(((b * T + t) * H + h) * N);
          for (int64_t p = 0; p < P; ++p)
            for (int64_t n = 0; n < N; ++n) Gm[p * N + n] += dyt[p] * (double)Ct_[n];
          for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t p = 0; p < P; ++p) acc += dyt[p] * hcur2[p * N + n];
            dCt[n] = acc;
          }
          double din = 0.0, dec = 0.0;
          for (int64_t p = 0; p < P; ++p) {
            double gb = 0.0;
            for (int64_t n = 0; n < N; ++n) {
              gb += Gm[p * N + n] * (double)Bt_[n];
              dec += Gm[p * N + n] * hprev[p * N + n];
            }
            dxt[p] = d * gb + Dh * dyt[p];
            din += gb * (double)xt[p];
            dD_acc += dyt[p] * (double)xt[p];
          }
          for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t p = 0; p < P; ++p) acc += Gm[p * N + n] * (double)xt[p];
            dBt[n] = d * acc;
          }
          const double dd = din + Ah * abar * dec;
          dA_acc += d * abar * dec;
          if (dlda) dlda[(b * T + t) * H + h] = abar * dec;
          double pre = dt_softplus ? softplus_exact(zv[t]) : zv[t];
          double gate = (pre >= dt_min && pre <= dt_max) ? 1.0 : 0.0;
          if (dt_softplus) gate *= 1.0 / (1.0 + exp(-zv[t]));
          const double g_dt = dd * gate;
          ddt[(b * T + t) * H + h] = g_dt;
          db_acc += g_dt;
          for (int64_t k = 0; k < PN; ++k) Gm[k] *= abar;
        }
      }
      memcpy(dh0 + (size_t)((b * H + h) * PN), Gm, sizeof(double) * (size_t)PN);
      dAh[pair] = dA_acc;
      dDh[pair] = dD_acc;
      dbh[pair] = db_acc;
    }
    free(ck); free(hs); free(Gm); free(dv); free(zv);
  }
  if (!failed) {
    for (int64_t h = 0; h < H; ++h) {
      double a = 0.0, dd = 0.0, bb = 0.0;
      for (int64_t b = 0; b < Bt; ++b) {
        a += dAh[b * H + h];
        dd += dDh[b * H + h];
        bb += dbh[b * H + h];
      }
      dA[h] = a;
      dD[h] = dd;
      ddt_bias[h] = bb;
    }
    for (int64_t b = 0; b < Bt; ++b)
      for (int64_t t = 0; t < T; ++t)
        for (int64_t g = 0; g < G; ++g)
          for (int64_t n = 0; n < N; ++n) {
            double sb = 0.0, sc = 0.0;
            for (int64_t h = g * hpg; h < (g + 1) * hpg; ++h) {
              sb += dBh[((b * T + t) * H + h) * N + n];
              sc += dCh[((b * T + t) * H + h) * N + n];
            }
            dB[((b * T + t) * G + g) * N + n] = sb;
            dC[((b * T + t) * G + g) * N + n] = sc;
          }
  }
  free(dBh); free(dCh); free(dAh); free(dDh); free(dbh);
  return failed ? 2 : 0;
}
