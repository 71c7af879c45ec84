/*
 * jscan_oracle.c -- plain, slow, sequential fp64 CPU oracle for the selective
 * state-space scan (prefill) and its one-token decode update.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the HIP library it checks.
 *
 * What it computes (all arithmetic in double, std C `exp`):
 *
 *   Recurrence of a state-space model with a fixed-size state h, per token:
 *   new state = decay * old state + input term, output = C . state
 *   ("AI Engineering from Scratch" Jamba lesson, section "一页讲完 SSM": the
 *   SSM h_t = A h_{t-1} + B x_t, y_t = C h_t; "selective" means A, B, C
 *   depend on the token, section "关键术语", entry "选择性 SSM").
 *   A is real and diagonal per (channel d, state n) as in Mamba-1
 *   (same lesson, section "Mamba-3", complex-state paragraph; exercise 2 says
 *   Jamba uses Mamba-1).  Discretisation: the decay is exp(delta * A[d][n])
 *   and the input term is delta * B[n] * x ("Euler" on the input, same lesson,
 *   Mamba-3 paragraph on exponential-trapezoidal discretisation).  The output
 *   adds the D skip and is multiplied by SiLU(z) = z / (1 + exp(-z)); the
 *   pages are silent on where the gate sits and the reading taken is that it
 *   multiplies the whole output, skip included.
 *
 *   For each batch b and channel d:
 *     h[n] = h0[b][d][n]            (0 when h0 is NULL)
 *     for t in 0..L-1:
 *       dt = delta[b][t][d]; xv = x[b][t][d]; acc = 0
 *       for n in 0..N-1:
 *         h[n] = exp(dt * A[d][n]) * h[n] + dt * B[b][t][n] * xv
 *         acc += C[b][t][n] * h[n]
 *       zv = z[b][t][d]
 *       y[b][t][d] = (acc + Dv[d] * xv) * zv / (1 + exp(-zv))
 *     hT[b][d][n] = h[n]            (when hT is not NULL)
 *
 * Layouts (dense, row-major):
 *   x, delta, z, y : [batch][L][d_inner]
 *   B, C           : [batch][L][d_state]
 *   A              : [d_inner][d_state];   Dv : [d_inner]
 *   h0, hT, state  : [batch][d_inner][d_state]
 *
 * The prefill loop is parallelised over independent (b, d) channels with
 * OpenMP; each channel's arithmetic is the sequential loop above, in that
 * order, so the result does not depend on the thread count.
 *
 * oracle_step is written on its own (not by calling oracle_prefill) so that
 * "the final state of a prefill equals T chained steps" is a real check of
 * two pieces of code.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

void oracle_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* Prefill: the scan over L tokens for every (b, d) channel. */
void oracle_prefill(int64_t batch, int64_t L, int64_t d_inner, int64_t d_state,
                    const double* x, const double* delta, const double* A,
                    const double* B, const double* C, const double* Dv,
                    const double* z, const double* h0, double* y, double* hT) {
  int64_t channels = batch * d_inner;
#pragma omp parallel for schedule(dynamic, 4)
  for (int64_t bd = 0; bd < channels; ++bd) {
    int64_t b = bd / d_inner;
    int64_t d = bd % d_inner;
    double h[256];
    for (int64_t n = 0; n < d_state; ++n)
      h[n] = h0 ? h0[(b * d_inner + d) * d_state + n] : 0.0;
    for (int64_t t = 0; t < L; ++t) {
      int64_t i = (b * L + t) * d_inner + d;     /* element (b, t, d) */
      const double* Bt = B + (b * L + t) * d_state;
      const double* Ct = C + (b * L + t) * d_state;
      double dt = delta[i];
      double xv = x[i];
      double acc = 0.0;
      for (int64_t n = 0; n < d_state; ++n) {
        h[n] = exp(dt * A[d * d_state + n]) * h[n] + dt * Bt[n] * xv;
        acc += Ct[n] * h[n];
      }
      double zv = z[i];
      y[i] = (acc + Dv[d] * xv) * zv / (1.0 + exp(-zv));
    }
    if (hT)
      for (int64_t n = 0; n < d_state; ++n)
        hT[(b * d_inner + d) * d_state + n] = h[n];
  }
}

/*
 * Decode step: one token for each of n_seq independent sequences, the state
 * updated in place.  x, delta, z, y : [n_seq][d_inner];  B, C : [n_seq][d_state];
 * state : [n_seq][d_inner][d_state].
 */
void oracle_step(int64_t n_seq, int64_t d_inner, int64_t d_state, double* state,
                 const double* x, const double* delta, const double* A,
                 const double* B, const double* C, const double* Dv,
                 const double* z, double* y) {
  for (int64_t s = 0; s < n_seq; ++s) {
    for (int64_t d = 0; d < d_inner; ++d) {
      double* h = state + (s * d_inner + d) * d_state;
      double dt = delta[s * d_inner + d];
      double xv = x[s * d_inner + d];
      double acc = 0.0;
      for (int64_t n = 0; n < d_state; ++n) {
        double decay = exp(dt * A[d * d_state + n]);
        double input = dt * B[s * d_state + n] * xv;
        h[n] = decay * h[n] + input;
        acc += C[s * d_state + n] * h[n];
      }
      double zv = z[s * d_inner + d];
      double silu = zv / (1.0 + exp(-zv));
      y[s * d_inner + d] = (acc + Dv[d] * xv) * silu;
    }
  }
}

/*
 * Input prologue of a Mamba layer, applied before the scan (test
 * infrastructure, same caveats as above).
 *
 * Causal depthwise convolution of x along the sequence, then SiLU: the outer
 * convolution on x_t that Mamba-1/2 apply before the recurrence (contrasted
 * with Mamba-3's in-recurrence form in the "Mamba-3" section of the
 * "AI Engineering from Scratch" Jamba lesson).  The pages give no kernel
 * width; width is a parameter (the library supports 1..4).  For each b, d:
 *
 *   hist(t) = x[b][t][d]                               for t >= 0
 *           = conv_state[b][width-1+t][d]              for -(width-1) <= t < 0
 *             (0 when conv_state is NULL)
 *   xc[b][t][d] = SiLU(bias[d] + sum_{k=0}^{width-1} w[d][k] * hist(t - (width-1) + k))
 *
 * and the state left for the next call is the last width-1 values of hist:
 *   conv_state_out[b][j][d] = hist(L - (width-1) + j),  j = 0 .. width-2.
 *
 * Time-step prologue: delta_out = softplus(delta + dt_bias[d]) =
 * log(1 + exp(delta + dt_bias[d])) (computed as log1p(exp(.))) when
 * softplus != 0 (dt_bias NULL: 0), else delta unchanged.
 *
 * Layouts: x, delta, xc, delta_out [batch][L][d_inner]; w [d_inner][width];
 * bias, dt_bias [d_inner]; conv_state [batch][width-1][d_inner].
 */
void oracle_prologue(int64_t batch, int64_t L, int64_t d_inner, int64_t width,
                     const double* x, const double* w, const double* bias,
                     const double* conv_state, double* xc, double* conv_state_out,
                     const double* delta, const double* dt_bias, int softplus,
                     double* delta_out) {
  for (int64_t b = 0; b < batch; ++b) {
    for (int64_t d = 0; d < d_inner; ++d) {
      for (int64_t t = 0; t < L; ++t) {
        int64_t i = (b * L + t) * d_inner + d;
        if (w) {
          double acc = bias ? bias[d] : 0.0;
          for (int64_t k = 0; k < width; ++k) {
            int64_t s = t - (width - 1) + k;      /* source token */
            double v;
            if (s >= 0) v = x[(b * L + s) * d_inner + d];
            else v = conv_state ? conv_state[(b * (width - 1) + (width - 1 + s)) * d_inner + d] : 0.0;
            acc += w[d * width + k] * v;
          }
          xc[i] = acc / (1.0 + exp(-acc));
        } else {
          xc[i] = x[i];
        }
        if (softplus) {
          double v = delta[i] + (dt_bias ? dt_bias[d] : 0.0);
          delta_out[i] = log1p(exp(v));
        } else {
          delta_out[i] = delta[i];
        }
      }
      if (conv_state_out) {
        for (int64_t j = 0; j < width - 1; ++j) {
          int64_t s = L - (width - 1) + j;
          double v;
          if (s >= 0) v = x[(b * L + s) * d_inner + d];
          else v = conv_state ? conv_state[(b * (width - 1) + (width - 1 + s)) * d_inner + d] : 0.0;
          conv_state_out[(b * (width - 1) + j) * d_inner + d] = v;
        }
      }
    }
  }
}

/*
 * Backward (gradient) of the prefill, for training (test infrastructure, same
 * caveats as above).  The pages name training with sequence and tensor
 * parallelism ("Jamba: A Hybrid Transformer-Mamba Language Model — 深度解读
 * 报告", section 3.3 on the training infrastructure) but give no backward;
 * this is the reverse-mode derivative of the recurrence defined at the top of
 * this file, taken by hand (adjoint method), for a scalar loss whose
 * gradients with respect to the outputs are dy [batch][L][d_inner] and dhT
 * [batch][d_inner][d_state] (dhT NULL: zero).
 *
 * Per (b, d), with the forward states h_t (h_{-1} = h0), decays
 * a_tn = exp(dt_t A_n), pre-gate output p_t = sum_n C_tn h_tn + D xv_t and
 * gate g_t = SiLU(z_t):
 *   lambda_t = dL/dh_t  (total, through all later tokens):
 *     lambda_{L-1} = dp_{L-1} C_{L-1} + dhT,
 *     lambda_t     = dp_t C_t + a_{t+1} * lambda_{t+1}   (per n)
 *   where dp_t = dy_t g_t.  Then
 *     dz_t     = dy_t p_t SiLU'(z_t),  SiLU'(z) = s (1 + z (1 - s)), s = 1/(1+exp(-z))
 *     dx_t     = D dp_t + dt_t sum_n lambda_tn B_tn
 *     ddelta_t = sum_n lambda_tn (A_n a_tn h_{t-1,n} + B_tn xv_t)
 *     dA_n    += sum_t lambda_tn dt_t a_tn h_{t-1,n}        (over b and t)
 *     dD      += sum_t dp_t xv_t                             (over b and t)
 *     dB_tn   += lambda_tn dt_t xv_t                         (over d)
 *     dC_tn   += dp_t h_tn                                   (over d)
 *     dh0_n    = a_0n lambda_0n
 * Every output is overwritten (dA, dD, dB, dC are sums built from zero).
 * dh0 may be NULL.  Layouts as for oracle_prefill; dA [d_inner][d_state],
 * dD [d_inner], dB, dC [batch][L][d_state].
 *
 * Channels run in parallel; each thread sums its channels' dB, dC, dA and dD
 * contributions privately and the partial sums are added in thread order.
 */
#include <stdlib.h>
#include <string.h>

int oracle_backward(int64_t batch, int64_t L, int64_t d_inner, int64_t d_state,
                    const double* x, const double* delta, const double* A,
                    const double* B, const double* C, const double* Dv,
                    const double* z, const double* h0, const double* dy,
                    const double* dhT, double* dx, double* ddelta, double* dz,
                    double* dA, double* dB, double* dC, double* dD, double* dh0) {
  const int64_t N = d_state;
  const int64_t rows = batch * L * N;
  int nthreads = oracle_num_threads();
  double* accBC = (double*)calloc((size_t)nthreads * (size_t)rows * 2, sizeof(double));
  double* accAD = (double*)calloc((size_t)nthreads * (size_t)d_inner * (size_t)(N + 1), sizeof(double));
  if (!accBC || !accAD) { free(accBC); free(accAD); return 1; }
  int failed = 0;
#pragma omp parallel num_threads(nthreads)
  {
#ifdef _OPENMP
    const int tid = omp_get_thread_num();
#else
    const int tid = 0;
#endif
    double* myB = accBC + (size_t)tid * (size_t)rows * 2;
    double* myC = myB + rows;
    double* myAD = accAD + (size_t)tid * (size_t)d_inner * (size_t)(N + 1);
    double* hs = (double*)malloc((size_t)(L + 1) * (size_t)N * sizeof(double));
    if (!hs) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic, 4)
    for (int64_t bd = 0; bd < batch * d_inner; ++bd) {
      if (!hs) continue;
      const int64_t b = bd / d_inner, d = bd % d_inner;
      /* forward, keeping every state: hs[(t+1)*N + n] = h_t[n] */
      for (int64_t n = 0; n < N; ++n) hs[n] = h0 ? h0[(b * d_inner + d) * N + n] : 0.0;
      for (int64_t t = 0; t < L; ++t) {
        const int64_t i = (b * L + t) * d_inner + d;
        const double* Bt = B + (b * L + t) * N;
        for (int64_t n = 0; n < N; ++n)
          hs[(t + 1) * N + n] = exp(delta[i] * A[d * N + n]) * hs[t * N + n] + delta[i] * Bt[n] * x[i];
      }
      /* reverse sweep; mu[n] is the adjoint arriving at h_t from later tokens */
      double mu[256];
      for (int64_t n = 0; n < N; ++n) mu[n] = dhT ? dhT[(b * d_inner + d) * N + n] : 0.0;
      for (int64_t t = L - 1; t >= 0; --t) {
        const int64_t i = (b * L + t) * d_inner + d;
        const double* Bt = B + (b * L + t) * N;
        const double* Ct = C + (b * L + t) * N;
        const double* ht = hs + (t + 1) * N;
        const double* hp = hs + t * N;
        const double dt = delta[i], xv = x[i], zv = z[i];
        const double s = 1.0 / (1.0 + exp(-zv));
        double p = Dv[d] * xv;
        for (int64_t n = 0; n < N; ++n) p += Ct[n] * ht[n];
        dz[i] = dy[i] * p * s * (1.0 + zv * (1.0 - s));
        const double dp = dy[i] * zv * s;
        double sx = 0.0, sd = 0.0;
        for (int64_t n = 0; n < N; ++n) {
          const double lam = dp * Ct[n] + mu[n];
          const double a = exp(dt * A[d * N + n]);
          myC[(b * L + t) * N + n] += dp * ht[n];
          myB[(b * L + t) * N + n] += lam * dt * xv;
          sx += lam * Bt[n];
          sd += lam * (A[d * N + n] * a * hp[n] + Bt[n] * xv);
          myAD[d * (N + 1) + n] += lam * dt * a * hp[n];
          mu[n] = a * lam;
        }
        myAD[d * (N + 1) + N] += dp * xv;
        dx[i] = Dv[d] * dp + dt * sx;
        ddelta[i] = sd;
      }
      if (dh0)
        for (int64_t n = 0; n < N; ++n) dh0[(b * d_inner + d) * N + n] = mu[n];
    }
    free(hs);
  }
  if (!failed) {
    for (int64_t r = 0; r < rows; ++r) {
      double sb = 0.0, sc = 0.0;
      for (int k = 0; k < nthreads; ++k) {
        sb += accBC[(size_t)k * (size_t)rows * 2 + (size_t)r];
        sc += accBC[(size_t)k * (size_t)rows * 2 + (size_t)rows + (size_t)r];
      }
      dB[r] = sb;
      dC[r] = sc;
    }
    for (int64_t d = 0; d < d_inner; ++d) {
      for (int64_t n = 0; n <= N; ++n) {
        double s = 0.0;
        for (int k = 0; k < nthreads; ++k) s += accAD[((size_t)k * (size_t)d_inner + (size_t)d) * (size_t)(N + 1) + (size_t)n];
        if (n < N) dA[d * N + n] = s;
        else dD[d] = s;
      }
    }
  }
  free(accBC);
  free(accAD);
  return failed;
}

/*
 * Exponential-trapezoidal variant of the prefill (Mamba-3's discretisation;
 * test infrastructure, same caveats as above).  The "AI Engineering from
 * Scratch" Jamba lesson (section "Mamba-3", and its glossary entry for the
 * exponential-trapezoidal discretisation) describes it only in words: a more
 * expressive recurrence that contains the Euler rule of the earlier models as
 * a special case and applies a convolution-like operation to the state input
 * inside the recurrence.  The reading taken: the input integral of
 * h' = A h + B x over one step is approximated by a weighted two-point rule
 * with the exponential kernel applied to the earlier point,
 *
 *   h_t = a_t h_{t-1} + dt_t ((1 - lam_t) a_t B_{t-1} x_{t-1} + lam_t B_t x_t),
 *   a_t = exp(dt_t A),
 *
 * so lam_t = 1 is the Euler form of oracle_prefill and lam_t = 1/2 is the
 * trapezoidal rule.  lam [batch][L][d_inner] (NULL: 1/2 everywhere).  The
 * token before the first comes from x_prev [batch][d_inner] and B_prev
 * [batch][d_state] (NULL: zero), and the last token's x and B row are
 * written to x_last, B_last (NULL: not written).  Output as in
 * oracle_prefill: y_t = (C_t . h_t + D x_t) SiLU(z_t).
 */
void oracle_prefill_trap(int64_t batch, int64_t L, int64_t d_inner, int64_t d_state,
                         const double* x, const double* delta, const double* A,
                         const double* B, const double* C, const double* Dv,
                         const double* z, const double* h0, const double* lam,
                         const double* x_prev, const double* B_prev,
                         double* y, double* hT, double* x_last, double* B_last) {
  int64_t channels = batch * d_inner;
#pragma omp parallel for schedule(dynamic, 4)
  for (int64_t bd = 0; bd < channels; ++bd) {
    int64_t b = bd / d_inner;
    int64_t d = bd % d_inner;
    double h[256];
    for (int64_t n = 0; n < d_state; ++n)
      h[n] = h0 ? h0[(b * d_inner + d) * d_state + n] : 0.0;
    double xp = x_prev ? x_prev[b * d_inner + d] : 0.0;
    for (int64_t t = 0; t < L; ++t) {
      int64_t i = (b * L + t) * d_inner + d;
      const double* Bt = B + (b * L + t) * d_state;
      const double* Ct = C + (b * L + t) * d_state;
      double dt = delta[i], xv = x[i], lt = lam ? lam[i] : 0.5;
      double acc = 0.0;
      for (int64_t n = 0; n < d_state; ++n) {
        double Bp = t > 0 ? B[(b * L + t - 1) * d_state + n] : (B_prev ? B_prev[b * d_state + n] : 0.0);
        double a = exp(dt * A[d * d_state + n]);
        h[n] = a * h[n] + dt * ((1.0 - lt) * a * Bp * xp + lt * Bt[n] * xv);
        acc += Ct[n] * h[n];
      }
      double zv = z[i];
      y[i] = (acc + Dv[d] * xv) * zv / (1.0 + exp(-zv));
      xp = xv;
    }
    if (hT)
      for (int64_t n = 0; n < d_state; ++n) hT[(b * d_inner + d) * d_state + n] = h[n];
    if (x_last) x_last[b * d_inner + d] = L > 0 ? xp : (x_prev ? x_prev[b * d_inner + d] : 0.0);
    if (B_last && d == 0)
      for (int64_t n = 0; n < d_state; ++n)
        B_last[b * d_state + n] = L > 0 ? B[(b * L + L - 1) * d_state + n] : (B_prev ? B_prev[b * d_state + n] : 0.0);
  }
}

/*
 * RMSNorm of the scan's inputs (test infrastructure, same caveats as above).
 * Jamba inserts RMSNorm at internal activations of its Mamba layers to stop
 * loss spikes at scale ("Jamba: A Hybrid Transformer-Mamba Language Model —
 * 深度解读报告", sections 3.1 and 4.9) without saying which; the reading taken
 * is the time step and the B and C rows before the scan:
 *
 *   RMSNorm(v)_i = v_i / sqrt(mean_j v_j^2 + eps) * w_i
 *
 * over the d_inner channels of each token's delta (weights w_dt [d_inner]) and
 * over the d_state entries of each token's B and C rows (w_B, w_C [d_state]).
 * A NULL weight leaves that tensor unchanged.  Layouts as for oracle_prefill;
 * outputs have the inputs' shapes.
 *
 * The normalisation is read as part of the layer's input prologue: its
 * results feed the recurrence directly, in full precision (nothing on the
 * page says they are stored and rounded in between), so this is the plain
 * fp64 definition.
 */
void oracle_rmsnorm_inputs(int64_t batch, int64_t L, int64_t d_inner, int64_t d_state,
                           const double* delta, const double* B, const double* C,
                           const double* w_dt, const double* w_B, const double* w_C, double eps,
                           double* delta_out, double* B_out, double* C_out) {
  for (int64_t bt = 0; bt < batch * L; ++bt) {
    const double* dv = delta + bt * d_inner;
    double* dout = delta_out + bt * d_inner;
    if (w_dt) {
      double ss = 0.0;
      for (int64_t d = 0; d < d_inner; ++d) ss += dv[d] * dv[d];
      double inv = 1.0 / sqrt(ss / (double)d_inner + eps);
      for (int64_t d = 0; d < d_inner; ++d) dout[d] = dv[d] * inv * w_dt[d];
    } else {
      for (int64_t d = 0; d < d_inner; ++d) dout[d] = dv[d];
    }
    const double* rows[2] = {B + bt * d_state, C + bt * d_state};
    double* outs[2] = {B_out + bt * d_state, C_out + bt * d_state};
    const double* ws[2] = {w_B, w_C};
    for (int k = 0; k < 2; ++k) {
      if (ws[k]) {
        double ss = 0.0;
        for (int64_t n = 0; n < d_state; ++n) ss += rows[k][n] * rows[k][n];
        double inv = 1.0 / sqrt(ss / (double)d_state + eps);
        for (int64_t n = 0; n < d_state; ++n) outs[k][n] = rows[k][n] * inv * ws[k][n];
      } else {
        for (int64_t n = 0; n < d_state; ++n) outs[k][n] = rows[k][n];
      }
    }
  }
}
