/* Runs every entry point of the fp64 oracle (oracle/ssm_oracle.c) on small
 * inputs with optional arguments present and absent, sequence lengths and
 * document resets, so that an AddressSanitizer / UndefinedBehaviorSanitizer
 * build of the oracle reports any out-of-bounds access, leak or undefined
 * arithmetic.  Compiled and run by tests/test_sanitizers.py; exits 0 when the
 * sanitizers stay silent (they abort the process otherwise). */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

double oracle_softplus(double v);
double oracle_sigmoid(double v);
void oracle_discretize(double delta, double a, double b, int dt_mode, double* abar, double* bbar);
void oracle_combine(double a1, double b1, double a2, double b2, double* a_out, double* b_out);
void oracle_scan_fwd_ex(const double* u, const double* delta, const double* A, const double* B,
                        const double* C, const double* D, const double* z,
                        const double* delta_bias, const double* h0, const int64_t* seq_lens,
                        const uint8_t* reset, int softplus, int dt_mode, double* y,
                        double* last_state, int64_t batch, int64_t L, int64_t dim, int64_t N,
                        int nthreads);
void oracle_scan_fwd(const double* u, const double* delta, const double* A, const double* B,
                     const double* C, const double* D, const double* z, const double* delta_bias,
                     const double* h0, int softplus, int dt_mode, double* y, double* last_state,
                     int64_t batch, int64_t L, int64_t dim, int64_t N, int nthreads);
void oracle_step_mt(double* state, const double* u, const double* delta, const double* A,
                    const double* B, const double* C, const double* D, const double* z,
                    const double* delta_bias, int softplus, int dt_mode, double* y,
                    int64_t batch, int64_t dim, int64_t N, int nthreads);
void oracle_step(double* state, const double* u, const double* delta, const double* A,
                 const double* B, const double* C, const double* D, const double* z,
                 const double* delta_bias, int softplus, int dt_mode, double* y, int64_t batch,
                 int64_t dim, int64_t N);
void oracle_conv1d_fwd(const double* x, const double* w, const double* bias,
                       const double* state_in, const int64_t* seq_lens, const uint8_t* reset,
                       int silu, double* out, double* state_out, int64_t batch, int64_t L,
                       int64_t dim, int64_t k);
void oracle_conv1d_step(double* window, const double* x, const double* w, const double* bias,
                        int silu, double* out, int64_t batch, int64_t dim, int64_t k);
void oracle_conv1d_bwd(const double* x, const double* w, const double* bias,
                       const double* state_in, const int64_t* seq_lens, const uint8_t* reset,
                       int silu, const double* dout, const double* dstate_out, double* dx,
                       double* dw, double* dbias, double* dstate_in, int64_t batch, int64_t L,
                       int64_t dim, int64_t k);
void oracle_scan_bwd(const double* u, const double* delta, const double* A, const double* B,
                     const double* C, const double* D, const double* z,
                     const double* delta_bias, const double* h0, const int64_t* seq_lens,
                     const uint8_t* reset, int softplus, int dt_mode,
                     const double* dy, const double* dlast, double* du, double* ddelta,
                     double* dA, double* dB, double* dC, double* dD, double* dz,
                     double* ddelta_bias, double* dh0, int64_t batch, int64_t L, int64_t dim,
                     int64_t N);
void oracle_ssd_fwd(const double* x, const double* dt_raw, const double* A, const double* B,
                    const double* C, const double* D, const double* z, const double* dt_bias,
                    const double* h0, int softplus, int dt_mode, double* y, double* last_state,
                    int64_t batch, int64_t L, int64_t nheads, int64_t P, int64_t N);

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static double uni(void) { /* xorshift64*, in (-1, 1) */
  rng ^= rng >> 12; rng ^= rng << 25; rng ^= rng >> 27;
  return (double)((rng * 0x2545F4914F6CDD1Dull) >> 11) / 4503599627370496.0 - 1.0;
}
/* exactly n doubles on the heap, so that any read or write past them is caught */
static double* arr(int64_t n) {
  double* p = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
  for (int64_t i = 0; i < n; ++i) p[i] = uni();
  return p;
}

int main(void) {
  double a, b;
  for (double v = -800.0; v <= 800.0; v += 37.5) {
    (void)oracle_softplus(v);
    (void)oracle_sigmoid(v);
  }
  oracle_discretize(0.5, -1.0, 1.0, 0, &a, &b);
  oracle_discretize(0.5, 0.0, 1.0, 0, &a, &b);
  oracle_discretize(0.0, -1.0, 1.0, 1, &a, &b);
  oracle_combine(0.5, 1.0, 0.25, 2.0, &a, &b);

  const int64_t batch = 3, L = 37, dim = 5, N = 7;
  for (int mode = 0; mode < 2; ++mode) {
    for (int opt = 0; opt < 2; ++opt) {
      double *u = arr(batch * L * dim), *dl = arr(batch * L * dim), *A = arr(dim * N);
      double *B = arr(batch * L * N), *C = arr(batch * L * N), *D = arr(dim), *z = arr(batch * L * dim);
      double *bias = arr(dim), *h0 = arr(batch * dim * N), *y = arr(batch * L * dim);
      double* last = arr(batch * dim * N);
      int64_t lens[3] = {0, 20, 37};
      uint8_t* reset = (uint8_t*)calloc((size_t)(batch * L), 1);
      reset[5] = reset[L + 19] = reset[2 * L] = 1;
      const int o = opt;
      oracle_scan_fwd(u, dl, A, B, C, o ? D : NULL, o ? z : NULL, o ? bias : NULL, o ? h0 : NULL,
                      1, mode, y, last, batch, L, dim, N, 4);
      oracle_scan_fwd_ex(u, dl, A, B, C, o ? D : NULL, o ? z : NULL, o ? bias : NULL,
                         o ? h0 : NULL, lens, reset, 1, mode, y, o ? last : NULL, batch, L, dim,
                         N, 2);
      oracle_scan_fwd(u, dl, A, B, C, D, z, bias, NULL, 0, mode, y, last, batch, 0, dim, N, 3);

      double* st = arr(batch * dim * N);
      oracle_step(st, u, dl, A, B, C, o ? D : NULL, o ? z : NULL, o ? bias : NULL, 1, mode, y,
                  batch, dim, N);
      oracle_step_mt(st, u, dl, A, B, C, o ? D : NULL, o ? z : NULL, o ? bias : NULL, 1, mode, y,
                     batch, dim, N, 4);

      double *dy = arr(batch * L * dim), *dlast = arr(batch * dim * N);
      double *du = arr(batch * L * dim), *ddl = arr(batch * L * dim), *dA = arr(dim * N);
      double *dB = arr(batch * L * N), *dC = arr(batch * L * N), *dD = arr(dim);
      double *dz = arr(batch * L * dim), *dbias = arr(dim), *dh0 = arr(batch * dim * N);
      oracle_scan_bwd(u, dl, A, B, C, o ? D : NULL, o ? z : NULL, o ? bias : NULL, o ? h0 : NULL,
                      o ? lens : NULL, o ? reset : NULL, 1, mode, dy, o ? dlast : NULL, du, ddl,
                      dA, dB, dC, o ? dD : NULL, o ? dz : NULL, o ? dbias : NULL,
                      o ? dh0 : NULL, batch, L, dim, N);

      const int64_t k = 4;
      double *w = arr(dim * k), *win = arr(batch * (k - 1) * dim), *wout = arr(batch * (k - 1) * dim);
      oracle_conv1d_fwd(u, w, o ? bias : NULL, o ? win : NULL, o ? lens : NULL, o ? reset : NULL,
                        o, y, o ? wout : NULL, batch, L, dim, k);
      oracle_conv1d_step(win, u, w, o ? bias : NULL, o, y, batch, dim, k);
      double *dw = arr(dim * k), *dwin = arr(batch * (k - 1) * dim);
      oracle_conv1d_bwd(u, w, o ? bias : NULL, o ? win : NULL, o ? lens : NULL, o ? reset : NULL,
                        o, dy, o ? wout : NULL, du, dw, o ? dbias : NULL, o ? dwin : NULL, batch,
                        L, dim, k);

      const int64_t nh = 2, P = 3, Ns = 4, dims = nh * P;
      double *x = arr(batch * L * dims), *dtr = arr(batch * L * nh), *Ah = arr(nh);
      double *Bs = arr(batch * L * Ns), *Cs = arr(batch * L * Ns), *Dh = arr(nh);
      double *zs = arr(batch * L * dims), *dtb = arr(nh), *h0s = arr(batch * dims * Ns);
      double *ys = arr(batch * L * dims), *ls = arr(batch * dims * Ns);
      oracle_ssd_fwd(x, dtr, Ah, Bs, Cs, o ? Dh : NULL, o ? zs : NULL, o ? dtb : NULL,
                     o ? h0s : NULL, 1, mode, ys, o ? ls : NULL, batch, L, nh, P, Ns);

      double* all[] = {u, dl, A, B, C, D, z, bias, h0, y, last, st, dy, dlast, du, ddl, dA, dB,
                       dC, dD, dz, dbias, dh0, w, win, wout, x, dtr, Ah, Bs, Cs, Dh, zs, dtb,
                       h0s, ys, ls, dw, dwin};
      for (size_t i = 0; i < sizeof(all) / sizeof(all[0]); ++i) free(all[i]);
      free(reset);
    }
  }
  printf("oracle driver: done\n");
  return 0;
}
