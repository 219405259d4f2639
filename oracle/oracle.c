/*
 * oracle.c -- plain fp64 CPU reference for the Mamba-1 selective scan (S6)
 * forward and the single-token state update.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark load this library.  The GPU path shares no
 * code, header, table or helper with it.
 *
 * What it computes, step by step, with the passage each step follows:
 *
 *   Pages cited:
 *     [P1] "Mamba 模型" (gaos6e.github.io, AI-Agent-Engineer notes):
 *          the full-step flowchart (nodes H to M) and its step notes.
 *     [P3] "Mamba 与状态空间模型" (world.lapla.si, plate F56):
 *          sections 03, 06 and 07.
 *     [P4] "Mamba 状态空间模型架构深度解析：从 S4 到 Mamba-3" (pnsm.cn):
 *          "状态空间模型（SSM）基础" (ZOH) and "Mamba-1：选择性状态空间"
 *          (diagonal A, one independent SSM per channel).
 *     [P5] "Mamba模型：高效序列建模的新突破" (mhpn.cn), section 3.1:
 *          the zero-order-hold formulas for A-bar and B-bar.
 *
 *   For every channel (b, d) independently ([P4] diagonal A):
 *     h(-1) = h0[b,d,:]  (zero for a fresh scan)
 *     for l = 0 .. L-1:
 *       delta  = softplus(delta_raw[b,d,l] + bias[d])          [P1] node H
 *       for n = 0 .. N-1:
 *         Abar = exp(delta * A[d,n])                            [P1] node I, [P5] 3.1
 *         Bbar = (Abar - 1) / A[d,n] * B[b,n,l]   (ZOH)         [P5] 3.1, [P4]
 *                (limit delta * B[b,n,l] when A[d,n] == 0)
 *              or delta * B[b,n,l]                (simplified)  [P3] "模型省略了什么"
 *         h[n] = Abar * h[n] + Bbar * u[b,d,l]                  [P1] node J
 *       y = sum_n C[b,n,l] * h[n] + Dskip[d] * u[b,d,l]         [P1] node K
 *       y = y * z * sigmoid(z)          (skipped when z is NULL) [P1] nodes L, M
 *     final_state[b,d,:] = h
 *
 *   Readings where the pages leave a point open (each is listed in the design
 *   notes): the bias is added before softplus; the readout uses the updated
 *   state h_t; the D-term is inside the gate; B_t and C_t are shared by all D
 *   channels of a batch row; softplus is the exact function with no
 *   threshold, evaluated as max(x,0) + log1p(exp(-|x|)).
 *
 * Layout: all arrays are dense row-major float64.
 *   u, delta_raw, z : (B, D, L)      Bt, Ct : (B, N, L)
 *   A : (D, N)      Dskip, bias : (D)      h0, final_state : (B, D, N)
 *   y : (B, D, L)
 *
 * Threads split the channel list only; each channel's time loop is sequential.
 */
#include <math.h>
#include <pthread.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>

enum { ORACLE_ZOH = 0, ORACLE_DELTA_B = 1 };

/* softplus(x) = log(1 + e^x), written so that neither branch overflows. */
double oracle_softplus(double x) { return fmax(x, 0.0) + log1p(exp(-fabs(x))); }

/* z * sigmoid(z), written as z / (1 + e^-z): e^-z may overflow to +inf for very
 * negative z, and the quotient then goes to -0, which is the right limit. */
static double silu(double z) { return z / (1.0 + exp(-z)); }

/* Input coefficient multiplying B * u for one (delta, a) pair. */
static double bbar_coef(double delta, double a, int mode) {
  if (mode == ORACLE_DELTA_B) return delta;
  if (a == 0.0) return delta;           /* lim_{a->0} (e^{delta a} - 1)/a */
  return expm1(delta * a) / a;          /* (Abar - 1)/a, with no cancellation */
}

typedef struct {
  int64_t B, D, N, L;
  const double *u, *delta_raw, *z, *Bt, *Ct, *A, *Dskip, *bias, *h0;
  int mode;
  double *y, *final_state;
  int64_t ch_begin, ch_end; /* range of flattened channel ids b*D + d */
} job_t;

static void scan_one_channel(const job_t* j, int64_t ch, double* h) {
  const int64_t b = ch / j->D, d = ch % j->D;
  const int64_t N = j->N, L = j->L;
  const double* u = j->u + ch * L;
  const double* dr = j->delta_raw + ch * L;
  const double* z = j->z ? j->z + ch * L : NULL;
  const double* Bb = j->Bt + b * N * L;
  const double* Cb = j->Ct + b * N * L;
  const double* Ad = j->A + d * N;
  const double Dd = j->Dskip ? j->Dskip[d] : 0.0;
  const double bias = j->bias ? j->bias[d] : 0.0;
  double* y = j->y + ch * L;

  for (int64_t n = 0; n < N; ++n) h[n] = j->h0 ? j->h0[ch * N + n] : 0.0;

  for (int64_t l = 0; l < L; ++l) {
    const double delta = oracle_softplus(dr[l] + bias);
    const double x = u[l];
    double acc = 0.0;
    for (int64_t n = 0; n < N; ++n) {
      const double a = Ad[n];
      const double abar = exp(delta * a);
      const double bbar = bbar_coef(delta, a, j->mode) * Bb[n * L + l];
      h[n] = abar * h[n] + bbar * x;
      acc += Cb[n * L + l] * h[n];
    }
    double out = acc + Dd * x;
    if (z) out *= silu(z[l]);
    y[l] = out;
  }
  if (j->final_state)
    for (int64_t n = 0; n < N; ++n) j->final_state[ch * N + n] = h[n];
}

static void* run_job(void* arg) {
  const job_t* j = (const job_t*)arg;
  double* h = (double*)malloc(sizeof(double) * (size_t)(j->N > 0 ? j->N : 1));
  if (!h) return (void*)1;
  for (int64_t ch = j->ch_begin; ch < j->ch_end; ++ch) scan_one_channel(j, ch, h);
  free(h);
  return NULL;
}

/* Returns 0 on success, -1 on bad arguments, -2 on allocation/thread failure. */
int oracle_scan(int64_t B, int64_t D, int64_t N, int64_t L,
                const double* u, const double* delta_raw, const double* z,
                const double* Bt, const double* Ct, const double* A,
                const double* Dskip, const double* bias, const double* h0,
                int mode, double* y, double* final_state, int nthreads) {
  if (B < 0 || D < 0 || N < 0 || L < 0) return -1;
  if (!u || !delta_raw || !Bt || !Ct || !A || !y) return -1;
  if (mode != ORACLE_ZOH && mode != ORACLE_DELTA_B) return -1;
  const int64_t nch = B * D;
  if (nch == 0) return 0;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > nch) nthreads = (int)nch;

  job_t* jobs = (job_t*)calloc((size_t)nthreads, sizeof(job_t));
  pthread_t* tids = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
  if (!jobs || !tids) { free(jobs); free(tids); return -2; }
  int rc = 0, started = 0;
  for (int t = 0; t < nthreads; ++t) {
    job_t* j = &jobs[t];
    j->B = B; j->D = D; j->N = N; j->L = L;
    j->u = u; j->delta_raw = delta_raw; j->z = z; j->Bt = Bt; j->Ct = Ct;
    j->A = A; j->Dskip = Dskip; j->bias = bias; j->h0 = h0; j->mode = mode;
    j->y = y; j->final_state = final_state;
    j->ch_begin = nch * t / nthreads;
    j->ch_end = nch * (t + 1) / nthreads;
  }
  if (nthreads == 1) {
    if (run_job(&jobs[0])) rc = -2;
  } else {
    for (int t = 0; t < nthreads; ++t) {
      if (pthread_create(&tids[t], NULL, run_job, &jobs[t]) != 0) { rc = -2; break; }
      ++started;
    }
    for (int t = 0; t < started; ++t) {
      void* ret = NULL;
      pthread_join(tids[t], &ret);
      if (ret) rc = -2;
    }
  }
  free(jobs);
  free(tids);
  return rc;
}

/* One decoding step: the scan above with L = 1, starting from `state`
 * ([P1] "为什么 Mamba 推理更省": state <- update(state, x_t)).  `state` is
 * updated in place; inputs are (B, D) / (B, N). */
int oracle_state_update(int64_t B, int64_t D, int64_t N, double* state,
                        const double* u, const double* delta_raw, const double* z,
                        const double* Bt, const double* Ct, const double* A,
                        const double* Dskip, const double* bias, int mode,
                        double* y, int nthreads) {
  if (!state) return -1;
  return oracle_scan(B, D, N, 1, u, delta_raw, z, Bt, Ct, A, Dskip, bias,
                     state, mode, y, state, nthreads);
}

/* ---------------------------------------------------------------------------
 * Causal depthwise convolution along the sequence, then SiLU -- the step that
 * produces the scan input u from the in_proj branch.
 *
 *   [P1] "Mamba 模型", flowchart node E (Causal Depthwise Conv1D):
 *          Uc_t = sum_i W_conv_i * U_(t-i)  -- one filter per channel, only the
 *          current and earlier positions;
 *        node F (SiLU):  Xc_t = Uc_t * sigmoid(Uc_t).
 *   [P3] "Mamba 与状态空间模型", section 03: besides its 16 state numbers each
 *        channel keeps a short convolution's 4 most recent inputs -- the conv
 *        state carried from token to token when decoding.
 *
 * Readings (listed in the design notes): tap i = 0 multiplies the current
 * input; positions before the sequence read `state0` (the K inputs before
 * t = 0, oldest first) or zero when state0 is NULL; an optional per-channel
 * bias is added before the activation (NULL: none, as in the node formula);
 * activation 1 = SiLU (the flowchart), 0 = none (used by the pins).
 *
 * Layout: x, y (B, D, L); w (D, K) with w[d*K + i] the tap of x[t - i];
 * bias (D); state0, final_state (B, D, K) with [k] the input at time
 * L - K + k (final_state) or k - K (state0).
 */
int oracle_conv1d(int64_t B, int64_t D, int64_t L, int64_t K, const double* x, const double* w,
                  const double* bias, const double* state0, int activation, double* y,
                  double* final_state) {
  if (B < 0 || D < 0 || L < 0 || K < 1 || !w) return -2;
  if ((B * D * L > 0) && (!x || !y)) return -1;
  for (int64_t ch = 0; ch < B * D; ++ch) {
    const int64_t d = ch % D;
    const double* xr = x ? x + ch * L : NULL;
    const double* s0 = state0 ? state0 + ch * K : NULL;
    const double* wd = w + d * K;
    /* input at time s (s may be negative: before the sequence) */
#define ORACLE_CONV_IN(s) ((s) >= 0 ? xr[(s)] : (s0 ? s0[K + (s)] : 0.0))
    for (int64_t t = 0; t < L; ++t) {
      double acc = bias ? bias[d] : 0.0;
      for (int64_t i = 0; i < K; ++i) {
        const int64_t s = t - i;
        if (s < -K) break;
        acc += wd[i] * ORACLE_CONV_IN(s);
      }
      y[ch * L + t] = activation ? silu(acc) : acc;
    }
    if (final_state) {
      for (int64_t k = 0; k < K; ++k) {
        const int64_t s = L - K + k;
        final_state[ch * K + k] = (s >= -K) ? ORACLE_CONV_IN(s) : 0.0;
      }
    }
#undef ORACLE_CONV_IN
  }
  return 0;
}

/* One decoding step of the convolution: the computation above with L = 1,
 * starting from `state` (the K most recent inputs, oldest first), which is
 * replaced in place by the K most recent inputs including x ([P3] section 03).
 * x, y: (B, D). */
int oracle_conv1d_update(int64_t B, int64_t D, int64_t K, double* state, const double* x,
                         const double* w, const double* bias, int activation, double* y) {
  if (!state || K < 1) return -1;
  double* next = (double*)malloc(sizeof(double) * (size_t)(B * D * K > 0 ? B * D * K : 1));
  if (!next) return -3;
  const int rc = oracle_conv1d(B, D, 1, K, x, w, bias, state, activation, y, next);
  if (rc == 0)
    for (int64_t i = 0; i < B * D * K; ++i) state[i] = next[i];
  free(next);
  return rc;
}

/* ---------------------------------------------------------------------------
 * Backward pass of the scan: gradients of all inputs for a given dy.
 *
 *   [P2] "Mamba论文研读笔记" 3.2.3 C (recomputation) and [P3] section 07: the
 *   backward pass works from the same inputs and recomputes the states h_t
 *   instead of reading stored ones.  Here, per channel, the forward recurrence
 *   is rerun in fp64 (keeping its L x N states in a private buffer) and then
 *   walked in reverse, applying the chain rule to each forward step:
 *
 *     yc_t = sum_n C_tn h_tn + D u_t;   y_t = yc_t * silu(z_t)   (or yc_t)
 *     h_tn = Abar_tn h_(t-1)n + coef_tn B_tn u_t,
 *     Abar = exp(delta a), coef = (Abar - 1)/a (ZOH) or delta,
 *     delta_t = softplus(delta_raw_t + bias).
 *
 *   Adjoint of the state: g_tn = dyc_t C_tn + Abar_(t+1)n g_(t+1)n.
 *   d coef / d delta = Abar (ZOH), 1 (delta*B);
 *   d coef / d a     = delta^2 phi(delta a), phi(x) = (x e^x - e^x + 1) / x^2
 *                      (ZOH; series near 0, where it tends to 1/2), 0 (delta*B);
 *   d softplus / dx  = sigmoid(x);  d silu / dz = s (1 + z (1 - s)), s = sigmoid(z).
 *
 * Outputs: du, ddelta_raw, dz (B, D, L) per channel; dBt, dCt (B, N, L)
 * summed over the D channels of a batch row; dA (D, N), dDskip (D) and
 * ddelta_bias (D) summed over batch rows and time.  dz is written only when
 * z is given.  Threads split the channels; each keeps private sums that are
 * added in thread order at the end, so results do not depend on timing.
 * ------------------------------------------------------------------------- */
static double sigmoid(double x) {
  if (x >= 0.0) return 1.0 / (1.0 + exp(-x));
  const double e = exp(x);
  return e / (1.0 + e);
}

/* (x e^x - e^x + 1) / x^2 */
static double phi_coef(double x) {
  if (fabs(x) < 0.5) {
    /* sum_{k>=0} (k+1) x^k / (k+2)! */
    double term = 0.5, sum = 0.0;       /* k = 0: 1 / 2! */
    for (int k = 0; k < 40; ++k) {
      sum += term;
      term *= x * (double)(k + 2) / ((double)(k + 1) * (double)(k + 3));
    }
    return sum;
  }
  return (x * exp(x) - expm1(x)) / (x * x);
}

typedef struct {
  int64_t B, D, N, L;
  const double *u, *delta_raw, *z, *Bt, *Ct, *A, *Dskip, *bias, *dy;
  int mode;
  double *du, *ddr, *dz;
  double *dBt, *dCt, *dA, *dD, *dbias;   /* this thread's private sums */
  int64_t ch_begin, ch_end;
} bjob_t;

static void bwd_one_channel(const bjob_t* j, int64_t ch, double* H, double* dl) {
  const int64_t b = ch / j->D, d = ch % j->D;
  const int64_t N = j->N, L = j->L;
  const double* u = j->u + ch * L;
  const double* dr = j->delta_raw + ch * L;
  const double* z = j->z ? j->z + ch * L : NULL;
  const double* Bb = j->Bt + b * N * L;
  const double* Cb = j->Ct + b * N * L;
  const double* Ad = j->A + d * N;
  const double Dd = j->Dskip ? j->Dskip[d] : 0.0;
  const double bias = j->bias ? j->bias[d] : 0.0;
  const double* dy = j->dy + ch * L;

  /* forward, keeping H[(l+1)*N + n] = h_ln and H[n] = h_(-1)n = 0 */
  for (int64_t n = 0; n < N; ++n) H[n] = 0.0;
  for (int64_t l = 0; l < L; ++l) {
    dl[l] = oracle_softplus(dr[l] + bias);
    for (int64_t n = 0; n < N; ++n) {
      const double a = Ad[n];
      H[(l + 1) * N + n] = exp(dl[l] * a) * H[l * N + n] + bbar_coef(dl[l], a, j->mode) * Bb[n * L + l] * u[l];
    }
  }
  /* reverse */
  double g[16], anext[16];
  for (int64_t n = 0; n < N; ++n) { g[n] = 0.0; anext[n] = 0.0; }
  for (int64_t l = L - 1; l >= 0; --l) {
    const double x = u[l], delta = dl[l];
    double dyc = dy[l];
    if (z) {
      double yc = Dd * x;
      for (int64_t n = 0; n < N; ++n) yc += Cb[n * L + l] * H[(l + 1) * N + n];
      const double s = sigmoid(z[l]);
      j->dz[ch * L + l] = dy[l] * yc * s * (1.0 + z[l] * (1.0 - s));
      dyc = dy[l] * silu(z[l]);
    }
    double dux = dyc * Dd, ddelta = 0.0;
    j->dD[d] += dyc * x;
    for (int64_t n = 0; n < N; ++n) {
      const double a = Ad[n];
      const double abar = exp(delta * a);
      const double coef = bbar_coef(delta, a, j->mode);
      const double gn = dyc * Cb[n * L + l] + anext[n] * g[n];
      const double dabar = gn * H[l * N + n];              /* d / d Abar_ln */
      const double dcoef = gn * Bb[n * L + l] * x;         /* d / d coef_ln */
      j->dCt[b * N * L + n * L + l] += dyc * H[(l + 1) * N + n];
      j->dBt[b * N * L + n * L + l] += gn * coef * x;
      dux += gn * coef * Bb[n * L + l];
      if (j->mode == ORACLE_DELTA_B) {
        ddelta += dabar * a * abar + dcoef;
        j->dA[d * N + n] += dabar * delta * abar;
      } else {
        ddelta += dabar * a * abar + dcoef * abar;
        j->dA[d * N + n] += dabar * delta * abar + dcoef * delta * delta * phi_coef(delta * a);
      }
      g[n] = gn;
      anext[n] = abar;
    }
    j->du[ch * L + l] = dux;
    const double dr_l = ddelta * sigmoid(dr[l] + bias);
    j->ddr[ch * L + l] = dr_l;
    j->dbias[d] += dr_l;
  }
}

static void* run_bjob(void* arg) {
  const bjob_t* j = (const bjob_t*)arg;
  const int64_t N = j->N, L = j->L;
  double* H = (double*)malloc(sizeof(double) * (size_t)((L + 1) * N + 1));
  double* dl = (double*)malloc(sizeof(double) * (size_t)(L + 1));
  if (!H || !dl) { free(H); free(dl); return (void*)1; }
  for (int64_t ch = j->ch_begin; ch < j->ch_end; ++ch) bwd_one_channel(j, ch, H, dl);
  free(H);
  free(dl);
  return NULL;
}

/* Returns 0 on success, -1 on bad arguments, -2 on allocation/thread failure. */
int oracle_scan_bwd(int64_t B, int64_t D, int64_t N, int64_t L,
                    const double* u, const double* delta_raw, const double* z,
                    const double* Bt, const double* Ct, const double* A,
                    const double* Dskip, const double* bias, int mode, const double* dy,
                    double* du, double* ddelta_raw, double* dz, double* dBt, double* dCt,
                    double* dA, double* dDskip, double* dbias, int nthreads) {
  if (B < 0 || D < 0 || N < 1 || N > 16 || L < 0) return -1;
  if (!u || !delta_raw || !Bt || !Ct || !A || !dy || !du || !ddelta_raw || !dBt || !dCt || !dA ||
      !dDskip || !dbias || (z && !dz))
    return -1;
  const int64_t C = B * D;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > C) nthreads = C > 0 ? (int)C : 1;
  const size_t nbc = (size_t)(B * N * L), nda = (size_t)(D * N), nd = (size_t)D;
  const size_t per = 2 * nbc + nda + 2 * nd;
  double* priv = (double*)calloc((size_t)nthreads * per + 1, sizeof(double));
  bjob_t* jobs = (bjob_t*)calloc((size_t)nthreads, sizeof(bjob_t));
  pthread_t* tids = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
  if (!priv || !jobs || !tids) { free(priv); free(jobs); free(tids); return -2; }
  int rc = 0;
  for (int t = 0; t < nthreads; ++t) {
    bjob_t* j = &jobs[t];
    j->B = B; j->D = D; j->N = N; j->L = L;
    j->u = u; j->delta_raw = delta_raw; j->z = z; j->Bt = Bt; j->Ct = Ct; j->A = A;
    j->Dskip = Dskip; j->bias = bias; j->dy = dy; j->mode = mode;
    j->du = du; j->ddr = ddelta_raw; j->dz = dz;
    double* p = priv + (size_t)t * per;
    j->dBt = p; j->dCt = p + nbc; j->dA = p + 2 * nbc; j->dD = p + 2 * nbc + nda; j->dbias = p + 2 * nbc + nda + nd;
    j->ch_begin = C * t / nthreads;
    j->ch_end = C * (t + 1) / nthreads;
  }
  int started = 0;
  for (int t = 0; t < nthreads; ++t) {
    if (pthread_create(&tids[t], NULL, run_bjob, &jobs[t]) != 0) { rc = -2; break; }
    ++started;
  }
  for (int t = 0; t < started; ++t) {
    void* ret = NULL;
    pthread_join(tids[t], &ret);
    if (ret) rc = -2;
  }
  if (rc == 0) {
    for (size_t i = 0; i < nbc; ++i) { dBt[i] = 0.0; dCt[i] = 0.0; }
    for (size_t i = 0; i < nda; ++i) dA[i] = 0.0;
    for (size_t i = 0; i < nd; ++i) { dDskip[i] = 0.0; dbias[i] = 0.0; }
    for (int t = 0; t < nthreads; ++t) {   /* fixed order: deterministic for a given thread count */
      const bjob_t* j = &jobs[t];
      for (size_t i = 0; i < nbc; ++i) { dBt[i] += j->dBt[i]; dCt[i] += j->dCt[i]; }
      for (size_t i = 0; i < nda; ++i) dA[i] += j->dA[i];
      for (size_t i = 0; i < nd; ++i) { dDskip[i] += j->dD[i]; dbias[i] += j->dbias[i]; }
    }
  }
  free(priv);
  free(jobs);
  free(tids);
  return rc;
}
