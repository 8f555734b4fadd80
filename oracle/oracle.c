/*
 * oracle.c -- plain, sequential fp64 CPU reference of the selective-SSM scan.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the library calls this code; only the
 * test suite, the smoke check and the CPU-baseline leg of the benchmark load it.
 * It shares no source with the GPU library.
 *
 * What it computes (every input is upcast exactly to double by the caller):
 *
 *   for every batch row b and channel d, independently:
 *     h[0..N) = 0                                   (zero initial state)
 *     for t = 0 .. L-1:
 *       u   = delta[b,t,d] + bias[d]                (bias optional, 0 if absent)
 *       dt  = softplus(u) if softplus_on else u     (softplus(u) = log(1 + e^u))
 *       for n: h[n] = exp(dt * A[d,n]) * h[n] + (c[n] * B[b,t,n]) * x[b,t,d]
 *                c[n] = dt, or (exp(dt * A[d,n]) - 1) / A[d,n] in zoh mode
 *       y   = sum_n C[b,t,n] * h[n]
 *       y  += D[d] * x[b,t,d]                       (optional skip)
 *       y  *= z * sigmoid(z), z = z[b,t,d]          (optional SiLU gate)
 *       out[b,t,d] = y
 *     last_state[b,d,:] = h                         (optional)
 *
 * Sources (the pages this follows):
 *  - "Mamba и State Space Models" (nareshka.ru), section "Ключевая инновация:
 *    input-dependent parameters": the selective recurrence
 *    h_t = exp(Delta_t A) h_{t-1} + Delta_t B_t x_t, y_t = C_t h_t; section
 *    "Selective Scan (core algorithm)": softplus on the step, dA = exp(dt*A),
 *    dB = dt*B, h starts at zero, y is read after the update at step t;
 *    section "Реализация MambaBlock": the output is gated by SiLU of the
 *    residual branch.
 *  - "State Space Models: Mamba и альтернатива Transformer" (johe.ru), the
 *    MambaBlock "_scan" code: the D skip y_t = C_t h_t + D x_t, added before
 *    the gate that the block applies afterwards.
 *  - "Модуль 8. Альтернативы Transformer" (vladkulikov.com), section 6:
 *    softplus(u) = log(1 + e^u) keeps the step positive.
 *  - Same page, section 7: an affine step h -> a h + b is the pair (a, b) and
 *    two steps compose as (a2, b2) o (a1, b1) = (a2 a1, a2 b1 + b2), the later
 *    step written first; the chunked mode below joins chunks with it.
 *  - Same page, sections 7 and 14: the decode step is the same recurrence for
 *    one token, continuing from the stored ssm_state [batch, d_inner, d_state].
 *  - "Mamba и State Space Models", section "Mamba-2: State Space Duality", and
 *    "Модуль 8", sections 7 and 14: the Mamba-2 form (scalar A per head, state
 *    [batch, nheads, headdim, d_state]); see the SSD section at the end.
 *  - Same page, sections 4 and 5: the exact zero-order-hold discretisation
 *    holds the input constant over the step, so the input coefficient is the
 *    integral of e^{sA} over s in [0, dt]: (e^{dt A} - 1) / A per diagonal
 *    coordinate, with the limit dt at A = 0.  Mamba's own parametrisation
 *    uses dt in its place (zoh off).
 *
 * Threads split independent (b, d) rows only; the order of the arithmetic
 * within a row is exactly the loop above.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_ABI 4

int oracle_abi_version(void) { return ORACLE_ABI; }

/* softplus(u) = log(1 + e^u), written as max(u, 0) + log1p(exp(-|u|)) so that
 * neither branch overflows; the two forms are equal for every real u. */
static double softplus(double u) { return fmax(u, 0.0) + log1p(exp(-fabs(u))); }

/* SiLU(z) = z * sigmoid(z) = z / (1 + e^{-z}). */
static double silu(double z) { return z / (1.0 + exp(-z)); }

/* The step size dt for one (b, t, d). */
static double step_size(double delta, const double* bias, int64_t d, int softplus_on) {
  double u = delta + (bias ? bias[d] : 0.0);
  return softplus_on ? softplus(u) : u;
}

/* The coefficient of B_t[n] x_t in the update of a coordinate with diagonal
 * entry a: dt, or with zoh the integral of e^{sa} over [0, dt], which is
 * (e^{dt a} - 1) / a for a != 0 and dt at a = 0. */
static double input_coef(double dt, double a, int zoh) {
  if (!zoh) return dt;
  if (a == 0.0) return dt;
  return expm1(dt * a) / a;
}

/* One recurrence step of one channel: updates h[0..N) in place and returns y. */
static double scan_step(double* h, double x, double dt, int zoh, const double* A_d, const double* B_t,
                        const double* C_t, const double* D, int64_t d, const double* zp, int64_t N) {
  for (int64_t n = 0; n < N; ++n) h[n] = exp(dt * A_d[n]) * h[n] + (input_coef(dt, A_d[n], zoh) * B_t[n]) * x;
  double y = 0.0;
  for (int64_t n = 0; n < N; ++n) y += C_t[n] * h[n];
  if (D) y += D[d] * x;
  if (zp) y *= silu(*zp);
  return y;
}

typedef struct {
  const double *x, *delta, *A, *B, *C, *D, *z, *bias;
  int softplus_on, zoh;
  double *out, *last_state;
  const double* h0; /* [batch, Dn, N] initial state, or NULL for zero */
  int64_t batch, L, Dn, N, chunk;
  int64_t row_begin, row_end; /* rows are r = b * Dn + d */
} job_t;

static void scan_rows(const job_t* j) {
  double* h = (double*)calloc((size_t)j->N, sizeof(double));
  for (int64_t r = j->row_begin; r < j->row_end; ++r) {
    int64_t b = r / j->Dn, d = r % j->Dn;
    for (int64_t n = 0; n < j->N; ++n) h[n] = j->h0 ? j->h0[(b * j->Dn + d) * j->N + n] : 0.0;
    for (int64_t t = 0; t < j->L; ++t) {
      int64_t e = (b * j->L + t) * j->Dn + d;          /* [batch, L, d_inner] */
      const double* Bt = j->B + (b * j->L + t) * j->N; /* [batch, L, d_state] */
      const double* Ct = j->C + (b * j->L + t) * j->N;
      double dt = step_size(j->delta[e], j->bias, d, j->softplus_on);
      double y = scan_step(h, j->x[e], dt, j->zoh, j->A + d * j->N, Bt, Ct, j->D, d, j->z ? j->z + e : NULL, j->N);
      j->out[e] = y;
    }
    if (j->last_state)
      for (int64_t n = 0; n < j->N; ++n) j->last_state[(b * j->Dn + d) * j->N + n] = h[n];
  }
  free(h);
}

/* Chunked form: each chunk of `chunk` steps is first reduced to its affine
 * pair per state coordinate, (P, e) with P = product of the chunk's exp(dt*A)
 * and e = the chunk's end state started from zero.  The pairs are composed in
 * time order, (a2,b2) o (a1,b1) = (a2*a1, a2*b1 + b2), which gives each chunk's
 * incoming state; each chunk is then re-run from that state to produce y. */
static void scan_rows_chunked(const job_t* j) {
  const int64_t N = j->N, L = j->L, Tc = j->chunk;
  const int64_t nch = (L + Tc - 1) / Tc;
  double* P = (double*)malloc((size_t)(nch * N) * sizeof(double));
  double* E = (double*)malloc((size_t)(nch * N) * sizeof(double));
  double* h = (double*)malloc((size_t)N * sizeof(double));
  double* acc_a = (double*)malloc((size_t)N * sizeof(double));
  double* acc_b = (double*)malloc((size_t)N * sizeof(double));
  for (int64_t r = j->row_begin; r < j->row_end; ++r) {
    int64_t b = r / j->Dn, d = r % j->Dn;
    const double* A_d = j->A + d * N;
    /* pass 1: per-chunk affine pairs */
    for (int64_t k = 0; k < nch; ++k) {
      double* Pk = P + k * N;
      double* Ek = E + k * N;
      for (int64_t n = 0; n < N; ++n) { Pk[n] = 1.0; Ek[n] = 0.0; }
      int64_t t1 = (k + 1) * Tc < L ? (k + 1) * Tc : L;
      for (int64_t t = k * Tc; t < t1; ++t) {
        int64_t e = (b * L + t) * j->Dn + d;
        const double* Bt = j->B + (b * L + t) * N;
        double dt = step_size(j->delta[e], j->bias, d, j->softplus_on);
        for (int64_t n = 0; n < N; ++n) {
          double a = exp(dt * A_d[n]);
          Pk[n] = a * Pk[n];
          Ek[n] = a * Ek[n] + (input_coef(dt, A_d[n], j->zoh) * Bt[n]) * j->x[e];
        }
      }
    }
    /* pass 2: compose the pairs in time order; chunk k starts from acc applied to
     * h = 0, where acc starts as the constant map to the initial state */
    for (int64_t n = 0; n < N; ++n) { acc_a[n] = 0.0; acc_b[n] = j->h0 ? j->h0[(b * j->Dn + d) * N + n] : 0.0; }
    for (int64_t k = 0; k < nch; ++k) {
      for (int64_t n = 0; n < N; ++n) h[n] = acc_b[n]; /* acc(0) = acc_a*0 + acc_b */
      int64_t t1 = (k + 1) * Tc < L ? (k + 1) * Tc : L;
      for (int64_t t = k * Tc; t < t1; ++t) {
        int64_t e = (b * L + t) * j->Dn + d;
        const double* Bt = j->B + (b * L + t) * N;
        const double* Ct = j->C + (b * L + t) * N;
        double dt = step_size(j->delta[e], j->bias, d, j->softplus_on);
        j->out[e] = scan_step(h, j->x[e], dt, j->zoh, A_d, Bt, Ct, j->D, d, j->z ? j->z + e : NULL, N);
      }
      for (int64_t n = 0; n < N; ++n) { /* acc = (P_k, E_k) o acc */
        double a2 = P[k * N + n], b2 = E[k * N + n];
        acc_b[n] = a2 * acc_b[n] + b2;
        acc_a[n] = a2 * acc_a[n];
      }
    }
    if (j->last_state)
      for (int64_t n = 0; n < N; ++n) j->last_state[(b * j->Dn + d) * N + n] = acc_b[n];
  }
  free(P); free(E); free(h); free(acc_a); free(acc_b);
}

static void* run_job(void* p) {
  const job_t* j = (const job_t*)p;
  if (j->chunk > 0) scan_rows_chunked(j);
  else scan_rows(j);
  return NULL;
}

static int run_threads(job_t base, int nthreads) {
  int64_t rows = base.batch * base.Dn;
  if (rows <= 0) return 0;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > rows) nthreads = (int)rows;
  if (nthreads == 1) { base.row_begin = 0; base.row_end = rows; run_job(&base); return 0; }
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
  job_t* jobs = (job_t*)malloc(sizeof(job_t) * (size_t)nthreads);
  int started = 0;
  for (int i = 0; i < nthreads; ++i) {
    jobs[i] = base;
    jobs[i].row_begin = rows * i / nthreads;
    jobs[i].row_end = rows * (i + 1) / nthreads;
  }
  for (int i = 0; i < nthreads; ++i) {
    if (pthread_create(&th[i], NULL, run_job, &jobs[i]) != 0) break;
    ++started;
  }
  for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
  /* rows a failed thread creation left undone are run here */
  for (int i = started; i < nthreads; ++i) run_job(&jobs[i]);
  free(th); free(jobs);
  return 0;
}

/* Full forward scan from the initial state h0 [batch, Dn, N] (NULL: zero);
 * zoh selects the exact zero-order-hold input coefficient.
 * Shapes: x, delta, z, out [batch, L, Dn]; B, C [batch, L, N]; A [Dn, N]; D, bias
 * [Dn]; last_state [batch, Dn, N].  D, z, bias, last_state may be NULL.  chunk > 0
 * selects the chunked form with chunks of that many steps.  Returns 0, or -1 on
 * bad arguments.  Continuing a sequence from a stored state is the recurrence
 * itself (the decode cache of "Модуль 8", sections 7 and 14, vladkulikov.com). */
int oracle_scan_fwd_from(const double* x, const double* delta, const double* A, const double* B,
                         const double* C, const double* D, const double* z, const double* bias,
                         int softplus_on, int zoh, const double* h0, double* out, double* last_state,
                         int64_t batch, int64_t L, int64_t Dn, int64_t N, int64_t chunk, int nthreads) {
  if (!x || !delta || !A || !B || !C || !out) return -1;
  if (batch < 0 || L < 0 || Dn < 0 || N <= 0 || chunk < 0) return -1;
  if (L == 0) {
    if (last_state) {
      if (h0) memcpy(last_state, h0, sizeof(double) * (size_t)(batch * Dn * N));
      else memset(last_state, 0, sizeof(double) * (size_t)(batch * Dn * N));
    }
    return 0;
  }
  job_t j = {x, delta, A, B, C, D, z, bias, softplus_on, zoh, out, last_state, h0, batch, L, Dn, N, chunk, 0, 0};
  return run_threads(j, nthreads);
}

/* The scan from a zero state. */
int oracle_scan_fwd(const double* x, const double* delta, const double* A, const double* B,
                    const double* C, const double* D, const double* z, const double* bias,
                    int softplus_on, double* out, double* last_state, int64_t batch, int64_t L,
                    int64_t Dn, int64_t N, int64_t chunk, int nthreads) {
  return oracle_scan_fwd_from(x, delta, A, B, C, D, z, bias, softplus_on, 0, NULL, out, last_state,
                              batch, L, Dn, N, chunk, nthreads);
}

/* One decode step: state [batch, Dn, N] is read and overwritten; x, delta, z, out
 * [batch, Dn]; B, C [batch, N].  Same arithmetic as one step of the scan. */
int oracle_state_update(double* state, const double* x, const double* delta, const double* A,
                        const double* B, const double* C, const double* D, const double* z,
                        const double* bias, int softplus_on, int zoh, double* out, int64_t batch,
                        int64_t Dn, int64_t N) {
  if (!state || !x || !delta || !A || !B || !C || !out) return -1;
  if (batch < 0 || Dn < 0 || N <= 0) return -1;
  for (int64_t b = 0; b < batch; ++b)
    for (int64_t d = 0; d < Dn; ++d) {
      int64_t e = b * Dn + d;
      double dt = step_size(delta[e], bias, d, softplus_on);
      out[e] = scan_step(state + e * N, x[e], dt, zoh, A + d * N, B + b * N, C + b * N, D, d,
                         z ? z + e : NULL, N);
    }
  return 0;
}

/* The affine-pair operator on arrays: (a, b) = (a2, b2) o (a1, b1), later step first. */
void oracle_affine_compose(const double* a2, const double* b2, const double* a1, const double* b1,
                           double* a, double* b, int64_t n) {
  for (int64_t i = 0; i < n; ++i) {
    double na = a2[i] * a1[i];
    double nb = a2[i] * b1[i] + b2[i];
    a[i] = na;
    b[i] = nb;
  }
}

/* The step size on its own (softplus branch pinned against a library routine). */
void oracle_step_size(const double* delta, const double* bias, int softplus_on, double* out,
                      int64_t rows, int64_t Dn) {
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t d = 0; d < Dn; ++d) out[r * Dn + d] = step_size(delta[r * Dn + d], bias, d, softplus_on);
}

/* ------------------------------------------------------------------ conv1d
 *
 * The block's short causal depthwise convolution ("Mamba и State Space
 * Models", nareshka.ru, section "Реализация MambaBlock": a Conv1d with one
 * filter of width K per channel, padding K - 1, output cut to the first L
 * steps; "State Space Models: Mamba и альтернатива Transformer", johe.ru,
 * MambaBlock: the same convolution followed by SiLU):
 *
 *   out[b,t,d] = act(bias[d] + sum_{k<K} w[d,k] * x[b, t-K+1+k, d])
 *
 * act is SiLU or the identity.  Inputs before t = 0 come from the cache
 * conv_state_in [batch, Dn, K], which holds the K most recent earlier inputs,
 * oldest first (entry k is the input at time k - K), or are zero when it is
 * NULL ("Модуль 8", vladkulikov.com, sections 6 and 14: the decode cache keeps
 * the last d_conv inputs of the convolution branch, [batch, d_inner, d_conv]).
 * conv_state_out receives the K most recent inputs after the call.
 */
static double conv_input(const double* x, const double* state_in, int64_t b, int64_t t, int64_t d,
                         int64_t L, int64_t Dn, int64_t K) {
  if (t >= 0) return x[(b * L + t) * Dn + d];
  return state_in ? state_in[(b * Dn + d) * K + (t + K)] : 0.0;
}

int oracle_conv1d_fwd(const double* x, const double* w, const double* bias, int silu_on,
                      const double* state_in, double* out, double* state_out, int64_t batch,
                      int64_t L, int64_t Dn, int64_t K) {
  if (!x || !w || !out || batch < 0 || L < 0 || Dn < 0 || K <= 0) return -1;
  for (int64_t b = 0; b < batch; ++b)
    for (int64_t t = 0; t < L; ++t)
      for (int64_t d = 0; d < Dn; ++d) {
        double acc = bias ? bias[d] : 0.0;
        for (int64_t k = 0; k < K; ++k)
          acc += w[d * K + k] * conv_input(x, state_in, b, t - K + 1 + k, d, L, Dn, K);
        out[(b * L + t) * Dn + d] = silu_on ? silu(acc) : acc;
      }
  if (state_out)
    for (int64_t b = 0; b < batch; ++b)
      for (int64_t d = 0; d < Dn; ++d)
        for (int64_t k = 0; k < K; ++k)
          state_out[(b * Dn + d) * K + k] = conv_input(x, state_in, b, L - K + k, d, L, Dn, K);
  return 0;
}

/* One decode step of the convolution: the cache drops its oldest input and
 * appends x; the output is the filter applied to the updated cache. */
int oracle_conv1d_update(double* state, const double* x, const double* w, const double* bias,
                         int silu_on, double* out, int64_t batch, int64_t Dn, int64_t K) {
  if (!state || !x || !w || !out || batch < 0 || Dn < 0 || K <= 0) return -1;
  for (int64_t b = 0; b < batch; ++b)
    for (int64_t d = 0; d < Dn; ++d) {
      double* st = state + (b * Dn + d) * K;
      for (int64_t k = 0; k + 1 < K; ++k) st[k] = st[k + 1];
      st[K - 1] = x[b * Dn + d];
      double acc = bias ? bias[d] : 0.0;
      for (int64_t k = 0; k < K; ++k) acc += w[d * K + k] * st[k];
      out[b * Dn + d] = silu_on ? silu(acc) : acc;
    }
  return 0;
}

/* ---------------------------------------------------------------- backward
 *
 * Gradients of the scan by reverse-mode differentiation of the recurrence
 * above (the pages give the forward recurrence only; the gradients follow
 * from it by the chain rule).  With u = delta + bias, dt = softplus(u) (or u),
 * a_t = exp(dt_t A), h_t = a_t h_{t-1} + dt_t B_t x_t, y_t = C_t . h_t + D x_t,
 * out_t = y_t SiLU(z_t), and g_t = dL/dout_t:
 *   dy_t  = g_t SiLU(z_t);          dz_t = g_t y_t SiLU'(z_t)
 *   dh_t  = dy_t C_t + a_{t+1} dh_{t+1}   (dh after the last step: dlast)
 *   dx_t  = dy_t D + dt_t (B_t . dh_t)
 *   ddt_t = sum_n dh_t[n] (A_n a_t[n] h_{t-1}[n] + B_t[n] x_t)
 *   ddelta_t = ddt_t softplus'(u_t) (= sigmoid(u_t)), or ddt_t
 *   dB_t[n] += dh_t[n] dt_t x_t,  dC_t[n] += dy_t h_t[n]   (summed over d)
 *   dA[d,n] += dh_t[n] a_t[n] h_{t-1}[n] dt_t;  dD[d] += dy_t x_t;
 *   dbias[d] += ddelta_t;  dh0 = a_0 dh_0        (summed over b and t)
 * Every output is overwritten.  The reduced gradients (dB, dC over channels;
 * dA, dD, dbias over batch rows) are summed row by row in a fixed order on
 * one thread, so the result does not depend on the thread count.
 */
static double sigmoid(double u) { return 1.0 / (1.0 + exp(-u)); }

int oracle_scan_bwd(const double* x, const double* delta, const double* A, const double* B,
                    const double* C, const double* D, const double* z, const double* bias,
                    int softplus_on, const double* h0, const double* dout, const double* dlast,
                    double* dx, double* ddelta, double* dA, double* dB, double* dC, double* dD,
                    double* dz, double* dbias, double* dh0, int64_t batch, int64_t L, int64_t Dn,
                    int64_t N) {
  if (!x || !delta || !A || !B || !C || !dout || !dx || !ddelta || !dA || !dB || !dC) return -1;
  if (batch < 0 || L < 0 || Dn < 0 || N <= 0) return -1;
  memset(dA, 0, sizeof(double) * (size_t)(Dn * N));
  memset(dB, 0, sizeof(double) * (size_t)(batch * L * N));
  memset(dC, 0, sizeof(double) * (size_t)(batch * L * N));
  if (dD) memset(dD, 0, sizeof(double) * (size_t)Dn);
  if (dbias) memset(dbias, 0, sizeof(double) * (size_t)Dn);
  double* hs = (double*)malloc(sizeof(double) * (size_t)((L + 1) * N)); /* h_{t-1} for t = 0..L */
  double* dh = (double*)malloc(sizeof(double) * (size_t)N);
  for (int64_t b = 0; b < batch; ++b)
    for (int64_t d = 0; d < Dn; ++d) {
      const double* A_d = A + d * N;
      /* forward: hs[t] = state before step t, hs[L] = final state */
      for (int64_t n = 0; n < N; ++n) hs[n] = h0 ? h0[(b * Dn + d) * N + n] : 0.0;
      for (int64_t t = 0; t < L; ++t) {
        int64_t e = (b * L + t) * Dn + d;
        const double* Bt = B + (b * L + t) * N;
        double dt = step_size(delta[e], bias, d, softplus_on);
        for (int64_t n = 0; n < N; ++n)
          hs[(t + 1) * N + n] = exp(dt * A_d[n]) * hs[t * N + n] + (dt * Bt[n]) * x[e];
      }
      /* reverse */
      for (int64_t n = 0; n < N; ++n) dh[n] = dlast ? dlast[(b * Dn + d) * N + n] : 0.0;
      for (int64_t t = L - 1; t >= 0; --t) {
        int64_t e = (b * L + t) * Dn + d;
        const double* Bt = B + (b * L + t) * N;
        const double* Ct = C + (b * L + t) * N;
        double u = delta[e] + (bias ? bias[d] : 0.0);
        double dt = softplus_on ? softplus(u) : u;
        double dy = dout[e];
        if (z) {
          double y = 0.0;
          for (int64_t n = 0; n < N; ++n) y += Ct[n] * hs[(t + 1) * N + n];
          if (D) y += D[d] * x[e];
          double zz = z[e], s = sigmoid(zz);
          dz[e] = dout[e] * y * (s * (1.0 + zz * (1.0 - s)));
          dy = dout[e] * silu(zz);
        }
        double sB = 0.0, ddt = 0.0;
        for (int64_t n = 0; n < N; ++n) {
          double a = exp(dt * A_d[n]);
          dh[n] += dy * Ct[n];                                  /* dh_t */
          double hprev = hs[t * N + n];
          dC[(b * L + t) * N + n] += dy * hs[(t + 1) * N + n];
          dB[(b * L + t) * N + n] += dh[n] * dt * x[e];
          sB += dh[n] * Bt[n];
          ddt += dh[n] * (A_d[n] * a * hprev + Bt[n] * x[e]);
          dA[d * N + n] += dh[n] * a * hprev * dt;
          dh[n] *= a;                                           /* a_t dh_t, carried to step t-1 */
        }
        dx[e] = (D ? dy * D[d] : 0.0) + dt * sB;
        double dd = softplus_on ? ddt * sigmoid(u) : ddt;
        ddelta[e] = dd;
        if (dD) dD[d] += dy * x[e];
        if (dbias) dbias[d] += dd;
      }
      if (dh0)
        for (int64_t n = 0; n < N; ++n) dh0[(b * Dn + d) * N + n] = dh[n];
    }
  free(hs);
  free(dh);
  return 0;
}

/* ------------------------------------------------------------- Mamba-2 SSD
 *
 * The Mamba-2 form of the same recurrence ("Mamba и State Space Models",
 * nareshka.ru, section "Mamba-2: State Space Duality": A is one scalar per
 * head, A = -exp(A_log); "Модуль 8", vladkulikov.com, section 7: with the
 * transition a_t I the state is h_t = a_t h_{t-1} + B_t x_t and y_t = C_t^T h_t;
 * section 14: the state is [batch, nheads, headdim, d_state], and the input
 * term is written dt B x).  Channels are heads x headdim; every channel p of
 * head h shares the head's step dt[b,t,h], its scalar A[h], and the B/C rows
 * of the head's group (heads split into ngroups contiguous blocks):
 *
 *   for every batch row b, head h, channel p < headdim, from h0 (or zero):
 *     g   = h / (nheads / ngroups)
 *     dt  = softplus(dt_in[b,t,h] + dt_bias[h])   (or dt_in + dt_bias)
 *     for n: s[n] = exp(dt * A[h]) * s[n] + (dt * B[b,t,g,n]) * x[b,t,h,p]
 *     y   = sum_n C[b,t,g,n] * s[n]  (+ D[h*headdim+p] * x)  (* SiLU(z[b,t,h,p]))
 *
 * Layouts: x, z, out [batch, L, nheads, headdim]; dt [batch, L, nheads];
 * B, C [batch, L, ngroups, N]; A, dt_bias [nheads]; D [nheads * headdim];
 * h0, last_state [batch, nheads, headdim, N].
 */
typedef struct {
  const double *x, *dt, *A, *B, *C, *D, *z, *bias, *h0;
  int softplus_on;
  double *out, *last_state;
  int64_t batch, L, H, P, G, N;
  int64_t row_begin, row_end; /* rows are r = (b * H + h) * P + p */
} ssd_job_t;

static void* ssd_rows(void* arg) {
  const ssd_job_t* j = (const ssd_job_t*)arg;
  double* s = (double*)calloc((size_t)j->N, sizeof(double));
  for (int64_t r = j->row_begin; r < j->row_end; ++r) {
    const int64_t p = r % j->P, h = (r / j->P) % j->H, b = r / (j->P * j->H);
    const int64_t g = h / (j->H / j->G);
    const int64_t ch = h * j->P + p; /* channel index within a step */
    for (int64_t n = 0; n < j->N; ++n) s[n] = j->h0 ? j->h0[r * j->N + n] : 0.0;
    for (int64_t t = 0; t < j->L; ++t) {
      const int64_t e = (b * j->L + t) * j->H * j->P + ch;
      const double* Bt = j->B + ((b * j->L + t) * j->G + g) * j->N;
      const double* Ct = j->C + ((b * j->L + t) * j->G + g) * j->N;
      const double dt = step_size(j->dt[(b * j->L + t) * j->H + h], j->bias, h, j->softplus_on);
      const double a = exp(dt * j->A[h]);
      const double x = j->x[e];
      double y = 0.0;
      for (int64_t n = 0; n < j->N; ++n) {
        s[n] = a * s[n] + (dt * Bt[n]) * x;
        y += Ct[n] * s[n];
      }
      if (j->D) y += j->D[ch] * x;
      if (j->z) y *= silu(j->z[e]);
      j->out[e] = y;
    }
    if (j->last_state)
      for (int64_t n = 0; n < j->N; ++n) j->last_state[r * j->N + n] = s[n];
  }
  free(s);
  return NULL;
}

int oracle_ssd_fwd(const double* x, const double* dt, const double* A, const double* B, const double* C,
                   const double* D, const double* z, const double* dt_bias, int softplus_on, const double* h0,
                   double* out, double* last_state, int64_t batch, int64_t L, int64_t H, int64_t P, int64_t G,
                   int64_t N, int nthreads) {
  if (!x || !dt || !A || !B || !C || !out) return -1;
  if (batch < 0 || L < 0 || H <= 0 || P <= 0 || G <= 0 || N <= 0 || H % G != 0) return -1;
  const int64_t rows = batch * H * P;
  if (L == 0) {
    if (last_state) {
      if (h0) memcpy(last_state, h0, sizeof(double) * (size_t)(rows * N));
      else memset(last_state, 0, sizeof(double) * (size_t)(rows * N));
    }
    return 0;
  }
  if (rows == 0) return 0;
  ssd_job_t base = {x, dt, A, B, C, D, z, dt_bias, h0, softplus_on, out, last_state, batch, L, H, P, G, N, 0, rows};
  if (nthreads < 1) nthreads = 1;
  if (nthreads > rows) nthreads = (int)rows;
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
  ssd_job_t* jobs = (ssd_job_t*)malloc(sizeof(ssd_job_t) * (size_t)nthreads);
  int started = 0;
  for (int i = 0; i < nthreads; ++i) {
    jobs[i] = base;
    jobs[i].row_begin = rows * i / nthreads;
    jobs[i].row_end = rows * (i + 1) / nthreads;
  }
  for (int i = 0; i < nthreads; ++i) {
    if (pthread_create(&th[i], NULL, ssd_rows, &jobs[i]) != 0) break;
    ++started;
  }
  for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
  for (int i = started; i < nthreads; ++i) ssd_rows(&jobs[i]);
  free(th);
  free(jobs);
  return 0;
}

/* One decode step of the Mamba-2 form: state [batch, H, P, N] is read and
 * overwritten; x, z, out [batch, H, P]; dt [batch, H]; B, C [batch, G, N]. */
int oracle_ssd_state_update(double* state, const double* x, const double* dt, const double* A,
                            const double* B, const double* C, const double* D, const double* z,
                            const double* dt_bias, int softplus_on, double* out, int64_t batch, int64_t H,
                            int64_t P, int64_t G, int64_t N) {
  if (!state || !x || !dt || !A || !B || !C || !out) return -1;
  if (batch < 0 || H <= 0 || P <= 0 || G <= 0 || N <= 0 || H % G != 0) return -1;
  for (int64_t b = 0; b < batch; ++b)
    for (int64_t h = 0; h < H; ++h) {
      const int64_t g = h / (H / G);
      const double d = step_size(dt[b * H + h], dt_bias, h, softplus_on);
      const double a = exp(d * A[h]);
      const double* Bt = B + (b * G + g) * N;
      const double* Ct = C + (b * G + g) * N;
      for (int64_t p = 0; p < P; ++p) {
        const int64_t e = (b * H + h) * P + p;
        double* s = state + e * N;
        double y = 0.0;
        for (int64_t n = 0; n < N; ++n) {
          s[n] = a * s[n] + (d * Bt[n]) * x[e];
          y += Ct[n] * s[n];
        }
        if (D) y += D[h * P + p] * x[e];
        if (z) y *= silu(z[e]);
        out[e] = y;
      }
    }
  return 0;
}
