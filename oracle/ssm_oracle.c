/*
 * ssm_oracle.c -- fp64 CPU oracle for the selective scan and its decode step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link or
 * call this file; only the test-suite, the smoke check and the CPU-baseline leg
 * of the benchmark use it.  It shares no source with the HIP library.
 *
 * It is the plain definition, run sequentially in double precision:
 *
 *   "Mamba and selective state spaces" (zerotofrontier.app/ssm/mamba),
 *   section "The selective state-space model", the S6 definition box:
 *     Delta_t = softplus(raw_t + b_Delta), H_0 = 0,
 *     h_{t,cn} = abar_{t,cn} h_{t-1,cn} + bbar_{t,cn} x_t^(c),
 *     y_t^(c) = sum_n C_{t,n} h_{t,cn} + D_c x_t^(c).
 *   Same page, "The discretization the code actually uses":
 *     abar = exp(Delta*lambda) for both rules;
 *     zero-order hold:    bbar = (exp(Delta*lambda) - 1)/lambda * B
 *     exponential-Euler:  bbar = Delta * B
 *   "Mamba, annotated" (that-mathevs.github.io), "Discretization (equation 4)":
 *     the scalar ZOH form (e^{Delta A} - 1)/A * B.
 *   "The Mamba block" section of the first page: the output is gated by SiLU(z),
 *     SiLU(v) = v * sigma(v), applied to the S6 output (which includes D x).
 *   "Decoding with a constant-size cache": one step updates the state entrywise,
 *     reads it and gates it.
 *
 * Readings where the pages leave a step open:
 *   - the bias is added once, inside the softplus; softplus may be switched off,
 *     in which case Delta = raw + bias as given;
 *   - A = 0 under ZOH takes the limit bbar = Delta * B;
 *   - the gate multiplies (C.h + D x);
 *   - the state is read after it is written for the same token.
 *
 * Sequences that do not start from zero or do not fill the batch (the
 * extended scan, oracle_scan_fwd_ex):
 *   - h0 is the state before the first token (the prefill of "Decoding with a
 *     constant-size cache" keeps only the final state; a later chunk of the
 *     same prompt starts from it);
 *   - seq_lens[b] real tokens, then padding: padded tokens produce y = 0 and
 *     leave the state alone, so last_state is the state after the last real
 *     token ("Where Mamba implementations go wrong": padding is not masked out
 *     of the state by itself; here it is kept out explicitly);
 *   - reset[b, t] != 0 marks a document start: the state is zeroed before
 *     token t is written ("What each parameter does": at a document break the
 *     state should forget everything; a very large Delta does it inside the
 *     layer, the flag does it outright).
 *
 * Layouts (row-major, dense):
 *   u, delta, z, y : (batch, L, dim)      B, C : (batch, L, N)
 *   A : (dim, N)     D, delta_bias : (dim)
 *   state / h0 / last_state : (batch, dim, N)
 *   seq_lens : (batch)                    reset : (batch, L)
 * Optional pointers (D, z, delta_bias, h0, seq_lens, reset, last_state) may be NULL.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>

#define ORACLE_DT_ZOH 0
#define ORACLE_DT_EULER 1

/* softplus(v) = log(1 + e^v), written so that neither branch overflows
 * (finite for v = +-1000, as the warm-up exercise on the first page asks). */
double oracle_softplus(double v) {
  if (v > 0.0) return v + log1p(exp(-v));
  return log1p(exp(v));
}

/* logistic sigmoid, stable for both signs */
double oracle_sigmoid(double v) {
  if (v >= 0.0) return 1.0 / (1.0 + exp(-v));
  double e = exp(v);
  return e / (1.0 + e);
}

/* The step size from the raw projection: bias inside, softplus once. */
static double step_size(double raw, double bias, int softplus) {
  double v = raw + bias;
  return softplus ? oracle_softplus(v) : v;
}

/* Discretize one (channel, state) pair: abar = exp(delta*a).
 * ZOH:   bbar = (exp(delta*a) - 1) / a * b   (expm1 keeps small delta*a exact;
 *        a = 0 takes the limit delta*b).
 * EULER: bbar = delta * b. */
void oracle_discretize(double delta, double a, double b, int dt_mode,
                       double* abar, double* bbar) {
  double kappa = delta * a;
  *abar = exp(kappa);
  if (dt_mode == ORACLE_DT_ZOH) {
    *bbar = (a != 0.0) ? expm1(kappa) / a * b : delta * b;
  } else {
    *bbar = delta * b;
  }
}

/* The associative combine of two affine steps h -> a h + b, applying `first`
 * and then `then`: (a1, b1) . (a2, b2) = (a1 a2, a2 b1 + b2).
 * ("Selection breaks the convolution" on the first page; "The scan, in one
 * equation" on the second.)  The sequential scan below does not need it; it
 * is here so that the tests can check it and use it to compose segments. */
void oracle_combine(double a1, double b1, double a2, double b2,
                    double* a_out, double* b_out) {
  *a_out = a1 * a2;
  *b_out = a2 * b1 + b2;
}

typedef struct {
  const double *u, *delta, *A, *B, *C, *D, *z, *bias, *h0;
  const int64_t* seq_lens;
  const uint8_t* reset;
  double *y, *last_state;
  int64_t batch, L, dim, N;
  int softplus, dt_mode;
  int64_t row_begin, row_end; /* rows are (b, c) pairs, b-major */
} scan_job;

/* One (batch, channel) row of the scan, over all t. */
static void scan_row(const scan_job* j, int64_t b, int64_t c) {
  const int64_t L = j->L, dim = j->dim, N = j->N;
  double h[64];
  double* hp = h;
  double* heap = NULL;
  if (N > 64) {
    heap = (double*)malloc(sizeof(double) * (size_t)N);
    hp = heap;
  }
  for (int64_t n = 0; n < N; ++n)
    hp[n] = j->h0 ? j->h0[(b * dim + c) * N + n] : 0.0;
  const double bias = j->bias ? j->bias[c] : 0.0;
  const double dskip = j->D ? j->D[c] : 0.0;
  int64_t len = j->seq_lens ? j->seq_lens[b] : L; /* real tokens of this sequence */
  if (len < 0) len = 0;
  if (len > L) len = L;
  for (int64_t t = 0; t < L; ++t) {
    const int64_t xi = (b * L + t) * dim + c;
    if (t >= len) { /* padding: no output, state kept */
      j->y[xi] = 0.0;
      continue;
    }
    if (j->reset && j->reset[b * L + t]) /* a document starts at t */
      for (int64_t n = 0; n < N; ++n) hp[n] = 0.0;
    const double x = j->u[xi];
    const double dt = step_size(j->delta[xi], bias, j->softplus);
    const double* Bt = j->B + (b * L + t) * N;
    const double* Ct = j->C + (b * L + t) * N;
    double acc = 0.0;
    for (int64_t n = 0; n < N; ++n) {
      double abar, bbar;
      oracle_discretize(dt, j->A[c * N + n], Bt[n], j->dt_mode, &abar, &bbar);
      hp[n] = abar * hp[n] + bbar * x; /* write the token first ... */
      acc += Ct[n] * hp[n];            /* ... then read the state */
    }
    double out = acc + dskip * x;
    if (j->z) {
      const double zz = j->z[xi];
      out *= zz * oracle_sigmoid(zz);
    }
    j->y[xi] = out;
  }
  if (j->last_state)
    for (int64_t n = 0; n < N; ++n) j->last_state[(b * dim + c) * N + n] = hp[n];
  free(heap);
}

static void* scan_worker(void* arg) {
  const scan_job* j = (const scan_job*)arg;
  for (int64_t r = j->row_begin; r < j->row_end; ++r) scan_row(j, r / j->dim, r % j->dim);
  return NULL;
}

/* The full scan.  Rows (b, c) are independent and are split over `nthreads`
 * host threads; each row is computed exactly as written above. */
void oracle_scan_fwd_ex(const double* u, const double* delta, const double* A,
                        const double* B, const double* C, const double* D,
                        const double* z, const double* delta_bias, const double* h0,
                        const int64_t* seq_lens, const uint8_t* reset,
                        int softplus, int dt_mode, double* y, double* last_state,
                        int64_t batch, int64_t L, int64_t dim, int64_t N, int nthreads) {
  const int64_t rows = batch * dim;
  if (rows <= 0) return;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > rows) nthreads = (int)rows;
  scan_job* jobs = (scan_job*)calloc((size_t)nthreads, sizeof(scan_job));
  pthread_t* tids = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
  for (int i = 0; i < nthreads; ++i) {
    scan_job* j = &jobs[i];
    j->u = u; j->delta = delta; j->A = A; j->B = B; j->C = C; j->D = D; j->z = z;
    j->bias = delta_bias; j->h0 = h0; j->y = y; j->last_state = last_state;
    j->seq_lens = seq_lens; j->reset = reset;
    j->batch = batch; j->L = L; j->dim = dim; j->N = N;
    j->softplus = softplus; j->dt_mode = dt_mode;
    j->row_begin = rows * i / nthreads;
    j->row_end = rows * (i + 1) / nthreads;
  }
  for (int i = 1; i < nthreads; ++i) pthread_create(&tids[i], NULL, scan_worker, &jobs[i]);
  scan_worker(&jobs[0]);
  for (int i = 1; i < nthreads; ++i) pthread_join(tids[i], NULL);
  free(jobs);
  free(tids);
}

/* Every sequence full length, no document breaks. */
void oracle_scan_fwd(const double* u, const double* delta, const double* A,
                     const double* B, const double* C, const double* D,
                     const double* z, const double* delta_bias, const double* h0,
                     int softplus, int dt_mode, double* y, double* last_state,
                     int64_t batch, int64_t L, int64_t dim, int64_t N, int nthreads) {
  oracle_scan_fwd_ex(u, delta, A, B, C, D, z, delta_bias, h0, NULL, NULL, softplus, dt_mode, y,
                     last_state, batch, L, dim, N, nthreads);
}

/* One decode step: the same body as the scan for a single token, with the
 * state read from and written back to `state` (batch, dim, N).
 * u, delta, z, y : (batch, dim); B, C : (batch, N). */
typedef struct {
  double* state;
  const double *u, *delta, *A, *B, *C, *D, *z, *bias;
  double* y;
  int64_t dim, N;
  int softplus, dt_mode;
  int64_t row_begin, row_end; /* rows are (b, c) pairs, b-major */
} step_job;

static void* step_worker(void* arg) {
  const step_job* j = (const step_job*)arg;
  const int64_t dim = j->dim, N = j->N;
  for (int64_t r = j->row_begin; r < j->row_end; ++r) {
    const int64_t b = r / dim, c = r % dim;
    const int64_t xi = b * dim + c;
    const double x = j->u[xi];
    const double dt = step_size(j->delta[xi], j->bias ? j->bias[c] : 0.0, j->softplus);
    double* h = j->state + xi * N;
    double acc = 0.0;
    for (int64_t n = 0; n < N; ++n) {
      double abar, bbar;
      oracle_discretize(dt, j->A[c * N + n], j->B[b * N + n], j->dt_mode, &abar, &bbar);
      h[n] = abar * h[n] + bbar * x;
      acc += j->C[b * N + n] * h[n];
    }
    double out = acc + (j->D ? j->D[c] : 0.0) * x;
    if (j->z) out *= j->z[xi] * oracle_sigmoid(j->z[xi]);
    j->y[xi] = out;
  }
  return NULL;
}

/* The step over all rows, split over `nthreads` host threads (rows are
 * independent; each is computed exactly as written above). */
void oracle_step_mt(double* state, const double* u, const double* delta, const double* A,
                    const double* B, const double* C, const double* D, const double* z,
                    const double* delta_bias, int softplus, int dt_mode, double* y,
                    int64_t batch, int64_t dim, int64_t N, int nthreads) {
  const int64_t rows = batch * dim;
  if (rows <= 0) return;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > rows) nthreads = (int)rows;
  step_job* jobs = (step_job*)calloc((size_t)nthreads, sizeof(step_job));
  pthread_t* tids = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
  for (int i = 0; i < nthreads; ++i) {
    step_job* j = &jobs[i];
    j->state = state; j->u = u; j->delta = delta; j->A = A; j->B = B; j->C = C; j->D = D;
    j->z = z; j->bias = delta_bias; j->y = y; j->dim = dim; j->N = N;
    j->softplus = softplus; j->dt_mode = dt_mode;
    j->row_begin = rows * i / nthreads;
    j->row_end = rows * (i + 1) / nthreads;
  }
  for (int i = 1; i < nthreads; ++i) pthread_create(&tids[i], NULL, step_worker, &jobs[i]);
  step_worker(&jobs[0]);
  for (int i = 1; i < nthreads; ++i) pthread_join(tids[i], NULL);
  free(jobs);
  free(tids);
}

void oracle_step(double* state, const double* u, const double* delta, const double* A,
                 const double* B, const double* C, const double* D, const double* z,
                 const double* delta_bias, int softplus, int dt_mode, double* y,
                 int64_t batch, int64_t dim, int64_t N) {
  oracle_step_mt(state, u, delta, A, B, C, D, z, delta_bias, softplus, dt_mode, y, batch, dim, N,
                 1);
}

/* ------------------------------------------------------------------------
 * The short causal depthwise convolution in front of the scan, "The Mamba
 * block" on the first page:
 *   x_t = SiLU( sum_{i=0}^{k-1} w_i (.) xt_{t-i} + b_conv ),  xt_s = 0 before
 *   the sequence,
 * each channel with its own k weights ("It is depthwise").  w is stored
 * (dim, k) with w[c*k + i] multiplying the input i steps back.
 *
 * Decoding ("Decoding with a constant-size cache"; "One decoding step with
 * conv and state caches") keeps the last k - 1 INPUTS of the convolution,
 * oldest first, per sequence: window (batch, k - 1, dim).  "Where Mamba
 * implementations go wrong" stresses that the window holds inputs, not
 * outputs, and shifts every step.
 *
 * The prefill form takes the same optional extras as the scan: state_in (the
 * window carried in from an earlier chunk, zeros when NULL), seq_lens
 * (padding after each length: output 0; state_out holds the last k - 1 real
 * inputs) and reset (a document starting at t sees zeros before t).
 * state_out receives the window after the last real token.
 * ------------------------------------------------------------------------ */

static double act(double v, int silu) { return silu ? v * oracle_sigmoid(v) : v; }

void oracle_conv1d_fwd(const double* x, const double* w, const double* bias,
                       const double* state_in, const int64_t* seq_lens, const uint8_t* reset,
                       int silu, double* out, double* state_out, int64_t batch, int64_t L,
                       int64_t dim, int64_t k) {
  for (int64_t b = 0; b < batch; ++b) {
    int64_t len = seq_lens ? seq_lens[b] : L;
    if (len < 0) len = 0;
    if (len > L) len = L;
    for (int64_t c = 0; c < dim; ++c) {
      /* the input at position s (s may be negative: the carried-in window),
       * for a document that starts at `start` (inputs before it are zero) */
#define XT(s, start)                                                                   \
  (((s) < (start)) ? 0.0                                                               \
   : ((s) >= 0)    ? x[(b * L + (s)) * dim + c]                                        \
   : (state_in && (s) >= -(k - 1)) ? state_in[(b * (k - 1) + (k - 1 + (s))) * dim + c] \
                                   : 0.0)
      int64_t start = -(k - 1); /* no document break yet: the window counts */
      for (int64_t t = 0; t < L; ++t) {
        const int64_t oi = (b * L + t) * dim + c;
        if (t >= len) {
          out[oi] = 0.0;
          continue;
        }
        if (reset && reset[b * L + t]) start = t;
        double pre = bias ? bias[c] : 0.0;
        for (int64_t i = 0; i < k; ++i) pre += w[c * k + i] * XT(t - i, start);
        out[oi] = act(pre, silu);
      }
      if (state_out)
        for (int64_t j = 0; j < k - 1; ++j) {
          const int64_t s = len - (k - 1) + j; /* oldest first */
          state_out[(b * (k - 1) + j) * dim + c] = XT(s, start);
        }
#undef XT
    }
  }
}

/* Backward pass of oracle_conv1d_fwd, by the chain rule through the forward
 * exactly as written above (the pages define the forward only): with
 * dpre_t = dout_t act'(pre_t), act'(p) = sigma(p) (1 + p (1 - sigma(p))) for
 * SiLU and 1 without, every real token t adds
 *   dbias += dpre_t,   dw_i += dpre_t XT(t - i),
 * and w_i dpre_t to the gradient of the input it read at t - i (an x, a
 * carried-in window entry, or nothing where the forward read a zero); the
 * gradient of state_out (dstate_out, nullable) goes to the inputs the window
 * holds.  Outputs past a length are constants, so nothing flows from them.
 * dx, dw (dim, k), dbias and dstate_in are overwritten; dbias and dstate_in
 * may be NULL. */
static double act_prime(double v, int silu) {
  if (!silu) return 1.0;
  const double s = oracle_sigmoid(v);
  return s * (1.0 + v * (1.0 - s));
}

void oracle_conv1d_bwd(const double* x, const double* w, const double* bias,
                       const double* state_in, const int64_t* seq_lens, const uint8_t* reset,
                       int silu, const double* dout, const double* dstate_out, double* dx,
                       double* dw, double* dbias, double* dstate_in, int64_t batch, int64_t L,
                       int64_t dim, int64_t k) {
  for (int64_t i = 0; i < batch * L * dim; ++i) dx[i] = 0.0;
  for (int64_t i = 0; i < dim * k; ++i) dw[i] = 0.0;
  if (dbias)
    for (int64_t c = 0; c < dim; ++c) dbias[c] = 0.0;
  if (dstate_in)
    for (int64_t i = 0; i < batch * (k - 1) * dim; ++i) dstate_in[i] = 0.0;
  for (int64_t b = 0; b < batch; ++b) {
    int64_t len = seq_lens ? seq_lens[b] : L;
    if (len < 0) len = 0;
    if (len > L) len = L;
    for (int64_t c = 0; c < dim; ++c) {
#define XT(s, start)                                                                   \
  (((s) < (start)) ? 0.0                                                               \
   : ((s) >= 0)    ? x[(b * L + (s)) * dim + c]                                        \
   : (state_in && (s) >= -(k - 1)) ? state_in[(b * (k - 1) + (k - 1 + (s))) * dim + c] \
                                   : 0.0)
      /* add v to the gradient of the input the forward read at s */
#define ROUTE(s, start, v)                                                      \
  do {                                                                          \
    if ((s) >= (start)) {                                                       \
      if ((s) >= 0)                                                             \
        dx[(b * L + (s)) * dim + c] += (v);                                     \
      else if (state_in && dstate_in && (s) >= -(k - 1))                        \
        dstate_in[(b * (k - 1) + (k - 1 + (s))) * dim + c] += (v);              \
    }                                                                           \
  } while (0)
      int64_t start = -(k - 1);
      for (int64_t t = 0; t < len; ++t) {
        if (reset && reset[b * L + t]) start = t;
        double pre = bias ? bias[c] : 0.0;
        for (int64_t i = 0; i < k; ++i) pre += w[c * k + i] * XT(t - i, start);
        const double dpre = dout[(b * L + t) * dim + c] * act_prime(pre, silu);
        if (dbias) dbias[c] += dpre;
        for (int64_t i = 0; i < k; ++i) {
          dw[c * k + i] += dpre * XT(t - i, start);
          ROUTE(t - i, start, w[c * k + i] * dpre);
        }
      }
      if (dstate_out)
        for (int64_t j = 0; j < k - 1; ++j) {
          const int64_t s = len - (k - 1) + j; /* oldest first, as state_out */
          ROUTE(s, start, dstate_out[(b * (k - 1) + j) * dim + c]);
        }
#undef ROUTE
#undef XT
    }
  }
}

/* One decoding step: append x to the window, convolve, shift. */
void oracle_conv1d_step(double* window, const double* x, const double* w, const double* bias,
                        int silu, double* out, int64_t batch, int64_t dim, int64_t k) {
  for (int64_t b = 0; b < batch; ++b) {
    for (int64_t c = 0; c < dim; ++c) {
      double* win = window + b * (k - 1) * dim + c; /* win[j * dim], j = 0 oldest */
      const double xt = x[b * dim + c];
      double pre = (bias ? bias[c] : 0.0) + w[c * k] * xt;
      for (int64_t i = 1; i < k; ++i) pre += w[c * k + i] * win[(k - 1 - i) * dim];
      out[b * dim + c] = act(pre, silu);
      for (int64_t j = 0; j + 1 < k - 1; ++j) win[j * dim] = win[(j + 1) * dim];
      if (k > 1) win[(k - 2) * dim] = xt;
    }
  }
}

/* ------------------------------------------------------------------------
 * Backward pass of the scan.
 *
 * The pages fix what it must compute, not how: gradients of the forward
 * above, with the states recomputed from the inputs rather than stored ("Why
 * the scan must be fused": the backward pass reloads x, Delta, B, C and
 * recomputes the states; "the backward pass of a linear recurrence is itself
 * a linear recurrence run in reverse").  This oracle keeps every state (it is
 * only run on small cases) and runs that reverse recurrence in the plainest
 * form, derived here by the chain rule:
 *
 *   forward:  h_t = abar_t h_{t-1} + bbar_t u_t,   s_t = C_t . h_t + D u_t,
 *             y_t = s_t * silu(z_t) (or s_t),      abar = exp(Delta A),
 *             bbar = Delta B phi(Delta A) (ZOH, phi(k) = (e^k - 1)/k) or Delta B
 *   given dy (and the gradient dlast of last_state = h_{L-1}):
 *     ds_t = dy_t silu(z_t),   dz_t = dy_t s_t silu'(z_t)
 *     g_t  = ds_t C_t + abar_{t+1} g_{t+1},  g_{L-1} = ds_{L-1} C_{L-1} + dlast
 *            (g_t = dLoss/dh_t through every later use of h_t)
 *     dabar = g_t h_{t-1},  dbbar = g_t u_t
 *     dC_tn = sum_c ds_t h_tn,   du_t = sum_n g_tn bbar_tn + ds_t D
 *     dD    = sum_t ds_t u_t
 *     through kappa = Delta A (abar and phi depend on A and Delta only via
 *     kappa, and bbar carries one more factor Delta B):
 *       dDelta_t = sum_n [dabar A abar + dbbar B (phi + kappa phi')]
 *                = sum_n [dabar A abar + dbbar abar B]        (ZOH)
 *                = sum_n [dabar A abar + dbbar B]             (Euler)
 *       dA_n     = sum_t [dabar Delta abar + dbbar B Delta^2 phi'(kappa)]  (ZOH)
 *                = sum_t  dabar Delta abar                                 (Euler)
 *       dB_tn    = sum_c dbbar Delta phi (ZOH) or dbbar Delta (Euler)
 *     draw_t = dDelta_t sigma(v_t) with softplus (the derivative of softplus),
 *              dDelta_t without;  dbias = sum_t draw_t
 *     dh0 = abar_0 g_0.
 *   lengths and document starts (the forward of oracle_scan_fwd_ex): tokens
 *   at or past len are padding -- no output, the state passes unchanged -- so
 *   their gradients are zero and g passes through them unchanged; a document
 *   starting at t computes h_t = bbar_t u_t (h_{t-1} taken as zero), so
 *   dabar_t = 0 there and nothing of g reaches t - 1 (nor h0 before it).
 * phi' is taken from its series below |kappa| = 0.1 and from
 * (kappa e^kappa - expm1(kappa)) / kappa^2 above it.
 * ------------------------------------------------------------------------ */

static double phi_prime(double k) {
  if (fabs(k) < 0.1) {
    /* sum_{j>=1} j k^{j-1} / (j+1)! */
    double term_f = 1.0, s = 0.0, kp = 1.0;
    for (int j = 1; j <= 12; ++j) {
      term_f *= (double)(j + 1); /* (j+1)! */
      s += (double)j * kp / term_f;
      kp *= k;
    }
    return s;
  }
  return (k * exp(k) - expm1(k)) / (k * k);
}

void oracle_scan_bwd(const double* u, const double* delta, const double* A, const double* B,
                     const double* C, const double* D, const double* z,
                     const double* delta_bias, const double* h0, const int64_t* seq_lens,
                     const uint8_t* reset, int softplus, int dt_mode,
                     const double* dy, const double* dlast, double* du, double* ddelta,
                     double* dA, double* dB, double* dC, double* dD, double* dz,
                     double* ddelta_bias, double* dh0, int64_t batch, int64_t L, int64_t dim,
                     int64_t N) {
  /* outputs accumulated over channels or over (batch, time) start at zero */
  for (int64_t i = 0; i < dim * N; ++i) dA[i] = 0.0;
  for (int64_t i = 0; i < batch * L * N; ++i) dB[i] = dC[i] = 0.0;
  for (int64_t c = 0; c < dim; ++c) {
    if (dD) dD[c] = 0.0;
    if (ddelta_bias) ddelta_bias[c] = 0.0;
  }
  double* hs = (double*)malloc(sizeof(double) * (size_t)((L + 1) * N)); /* h_{-1} .. h_{L-1} */
  double* g = (double*)malloc(sizeof(double) * (size_t)N);
  for (int64_t b = 0; b < batch; ++b) {
    for (int64_t c = 0; c < dim; ++c) {
      const double bias = delta_bias ? delta_bias[c] : 0.0;
      const double dskip = D ? D[c] : 0.0;
      int64_t len = seq_lens ? seq_lens[b] : L; /* real tokens of this sequence */
      if (len < 0) len = 0;
      if (len > L) len = L;
      /* forward, keeping every state: hs[(t + 1) * N + n] = h_t */
      for (int64_t n = 0; n < N; ++n) hs[n] = h0 ? h0[(b * dim + c) * N + n] : 0.0;
      for (int64_t t = 0; t < L; ++t) {
        const int64_t xi = (b * L + t) * dim + c;
        if (t >= len) { /* padding: the state passes unchanged */
          for (int64_t n = 0; n < N; ++n) hs[(t + 1) * N + n] = hs[t * N + n];
          continue;
        }
        const int doc_start = reset && reset[b * L + t];
        const double dt = step_size(delta[xi], bias, softplus);
        for (int64_t n = 0; n < N; ++n) {
          double abar, bbar;
          oracle_discretize(dt, A[c * N + n], B[(b * L + t) * N + n], dt_mode, &abar, &bbar);
          const double prev = doc_start ? 0.0 : hs[t * N + n];
          hs[(t + 1) * N + n] = abar * prev + bbar * u[xi];
        }
      }
      /* reverse */
      for (int64_t n = 0; n < N; ++n) g[n] = dlast ? dlast[(b * dim + c) * N + n] : 0.0;
      for (int64_t t = L - 1; t >= 0; --t) {
        const int64_t xi = (b * L + t) * dim + c;
        if (t >= len) { /* padding: zero gradients, g passes through */
          du[xi] = 0.0;
          ddelta[xi] = 0.0;
          if (z && dz) dz[xi] = 0.0;
          continue;
        }
        const int doc_start = reset && reset[b * L + t];
        const double x = u[xi];
        const double v = delta[xi] + bias;
        const double dt = softplus ? oracle_softplus(v) : v;
        const double* Bt = B + (b * L + t) * N;
        const double* Ct = C + (b * L + t) * N;
        const double* ht = hs + (t + 1) * N;
        const double* hp = hs + t * N; /* read as zero at a document start */
        double s = dskip * x;
        for (int64_t n = 0; n < N; ++n) s += Ct[n] * ht[n];
        double ds = dy[xi];
        if (z) {
          const double zz = z[xi], sg = oracle_sigmoid(zz);
          ds = dy[xi] * zz * sg;
          if (dz) dz[xi] = dy[xi] * s * sg * (1.0 + zz * (1.0 - sg));
        }
        double ddt = 0.0, dx = ds * dskip;
        for (int64_t n = 0; n < N; ++n) {
          const double a = A[c * N + n], kap = dt * a;
          double abar, bbar;
          oracle_discretize(dt, a, Bt[n], dt_mode, &abar, &bbar);
          g[n] += ds * Ct[n];
          dC[(b * L + t) * N + n] += ds * ht[n];
          const double dabar = doc_start ? 0.0 : g[n] * hp[n];
          const double dbbar = g[n] * x;
          dx += g[n] * bbar;
          if (dt_mode == ORACLE_DT_ZOH) {
            const double phi = (a != 0.0) ? expm1(kap) / kap : 1.0;
            ddt += dabar * a * abar + dbbar * abar * Bt[n];
            dA[c * N + n] += dabar * dt * abar + dbbar * Bt[n] * dt * dt * phi_prime(kap);
            dB[(b * L + t) * N + n] += dbbar * dt * phi;
          } else {
            ddt += dabar * a * abar + dbbar * Bt[n];
            dA[c * N + n] += dabar * dt * abar;
            dB[(b * L + t) * N + n] += dbbar * dt;
          }
          g[n] = doc_start ? 0.0 : g[n] * abar; /* carry to t - 1 */
        }
        du[xi] = dx;
        if (dD) dD[c] += ds * x;
        const double dv = softplus ? ddt * oracle_sigmoid(v) : ddt;
        ddelta[xi] = dv;
        if (ddelta_bias) ddelta_bias[c] += dv;
      }
      if (dh0)
        for (int64_t n = 0; n < N; ++n) dh0[(b * dim + c) * N + n] = g[n];
    }
  }
  free(hs);
  free(g);
}

/* ------------------------------------------------------------------------
 * Mamba-2 / SSD: one scalar decay per head.  "Mamba and selective state
 * spaces", the section on what Mamba cannot do yet: Mamba-2 gives each head, a
 * group of P channels, a single scalar decay, so most of the work becomes
 * matrix products and N can grow to 64..256.  "State-space models & Mamba"
 * (llm-tutorial.darvinyi.com, ch. 12), "The Mamba CUDA kernel": with A a scalar
 * per channel group the recurrence is h_t = alpha_t h_{t-1} + Bbar_t x_t and the
 * whole layer is a structured (1-semiseparable) masked matmul.
 *
 * The plain recurrence, per batch entry b, head hd, head channel p, state n:
 *   Delta_t = softplus(dt_raw[b,t,hd] + dt_bias[hd])   (or without softplus)
 *   alpha_t = exp(Delta_t A[hd])
 *   w_t     = Delta_t (exponential-Euler) or Delta_t phi(Delta_t A[hd]) (ZOH)
 *   h_t[p,n] = alpha_t h_{t-1}[p,n] + w_t B[b,t,n] x[b,t,hd,p]
 *   y[b,t,hd,p] = (sum_n C[b,t,n] h_t[p,n] + D[hd] x) * silu(z)?
 * B and C are shared by all heads (one group).  Layouts:
 *   x, z, y : (batch, L, nheads * P)   dt_raw : (batch, L, nheads)
 *   A, D, dt_bias : (nheads)           B, C : (batch, L, N)
 *   h0 / last_state : (batch, nheads * P, N)
 * ------------------------------------------------------------------------ */
void oracle_ssd_fwd(const double* x, const double* dt_raw, const double* A, const double* B,
                    const double* C, const double* D, const double* z, const double* dt_bias,
                    const double* h0, int softplus, int dt_mode, double* y, double* last_state,
                    int64_t batch, int64_t L, int64_t nheads, int64_t P, int64_t N) {
  const int64_t dim = nheads * P;
  double* h = (double*)malloc(sizeof(double) * (size_t)N);
  for (int64_t b = 0; b < batch; ++b) {
    for (int64_t hd = 0; hd < nheads; ++hd) {
      const double a = A[hd];
      for (int64_t p = 0; p < P; ++p) {
        const int64_t c = hd * P + p;
        for (int64_t n = 0; n < N; ++n) h[n] = h0 ? h0[(b * dim + c) * N + n] : 0.0;
        for (int64_t t = 0; t < L; ++t) {
          const double dt = step_size(dt_raw[(b * L + t) * nheads + hd],
                                      dt_bias ? dt_bias[hd] : 0.0, softplus);
          const double kap = dt * a;
          const double alpha = exp(kap);
          const double w = (dt_mode == ORACLE_DT_ZOH)
                               ? ((a != 0.0) ? expm1(kap) / a : dt)  /* Delta phi(Delta A) */
                               : dt;
          const int64_t xi = (b * L + t) * dim + c;
          const double xv = x[xi];
          double acc = 0.0;
          for (int64_t n = 0; n < N; ++n) {
            h[n] = alpha * h[n] + w * B[(b * L + t) * N + n] * xv;
            acc += C[(b * L + t) * N + n] * h[n];
          }
          double out = acc + (D ? D[hd] : 0.0) * xv;
          if (z) out *= z[xi] * oracle_sigmoid(z[xi]);
          y[xi] = out;
        }
        if (last_state)
          for (int64_t n = 0; n < N; ++n) last_state[(b * dim + c) * N + n] = h[n];
      }
    }
  }
  free(h);
}
