/* Drives every entry of the fp64 oracle (oracle/oracle.c) on small random inputs, edge cases
 * included (empty and ragged sequences, row subsets, start states, rejected arguments), so
 * that a build with AddressSanitizer and UndefinedBehaviorSanitizer checks its memory
 * accesses and arithmetic.  Exit status 0 when every call returned what it should; the
 * sanitizers abort on their own findings.  Test infrastructure (tests/test_sanitizers.py). */
#include <stdio.h>
#include <stdlib.h>

int oracle_prefill(int variant, int B, int H, long T, int dk, int dv, const double *q, const double *k,
                   const double *v, const double *alpha, const double *beta, const double *S0,
                   const double *z0, double eps, const int *rows, int nrows, double *o, double *S_T,
                   double *z_T, int nthreads);
int oracle_decode_step(int variant, int N, int dk, int dv, const double *S_in, const double *z_in,
                       const double *q, const double *k, const double *v, const double *alpha,
                       const double *beta, double eps, double *S_out, double *z_out, double *o, int nthreads);
int oracle_literal(int variant, long T, int dk, int dv, const double *q, const double *k, const double *v,
                   const double *alpha, const double *beta, const double *S0, double *o, double *S_T);
void oracle_based_phi(const double *x, int dp, double *f);
void oracle_based_phi_compact(const double *x, int dp, double *f);
int oracle_write_scores(int B, int H, long T, int dk, long C, const double *k, double *d_head, double *d_mean);
int oracle_write_windows(int B, long T, long C, long W, long tail, const double *d_mean, long *best_start,
                         double *best_sum);
int oracle_note_addresses(int B, int H, long T, int dk, int N, int drho, const double *d_head,
                          const double *q, const long *spans, const int *coords, long *t_star, double *rho);
int oracle_address_votes(int N, int J, int nQ, int drho, const double *rho, const double *u, int R,
                         const long *positions, double *score, int *choice, int *votes, int *selected);

static unsigned long long rs = 88172645463325252ull;
static double rnd(void) { /* xorshift64, uniform in [-1, 1) */
  rs ^= rs << 13; rs ^= rs >> 7; rs ^= rs << 17;
  return (double)(rs >> 11) / (double)(1ull << 52) - 1.0;
}
static double *arr(size_t n) {
  double *a = (double *)malloc((n ? n : 1) * sizeof(double));
  for (size_t i = 0; i < n; ++i) a[i] = rnd();
  return a;
}
static int fails = 0;
#define EXPECT(cond) do { if (!(cond)) { fprintf(stderr, "failed: %s (line %d)\n", #cond, __LINE__); ++fails; } } while (0)

int main(void) {
  const int B = 2, H = 3, dk = 8, dv = 5, dp = 4, Dfull = 1 + dp + dp * dp, Dc = 1 + dp + dp * (dp + 1) / 2;
  const long Ts[] = {0, 1, 17, 70};
  for (int ti = 0; ti < 4; ++ti) {
    const long T = Ts[ti];
    for (int var = 0; var <= 4; ++var) {
      const int based = var == 1 || var == 4;
      const int kd = based ? dp : dk, D = var == 4 ? Dc : Dfull;
      const size_t bht = (size_t)B * H * T;
      double *q = arr(bht * kd), *k = arr(bht * kd), *v = arr(bht * dv);
      double *al = arr(bht), *be = arr(bht);
      for (size_t i = 0; i < bht; ++i) { al[i] = 0.5 + 0.25 * (al[i] + 1.0); be[i] = 0.5 * (be[i] + 1.0); }
      const size_t sn = based ? (size_t)B * H * D * dv : (size_t)B * H * dv * kd;
      double *S0 = arr(sn), *z0 = arr((size_t)B * H * D), *o = arr(bht * dv), *ST = arr(sn), *zT = arr((size_t)B * H * D);
      for (size_t i = 0; i < (size_t)B * H * D; ++i) z0[i] = 2.0 + z0[i];
      const int gated = var == 2 || var == 3;
      EXPECT(oracle_prefill(var, B, H, T, kd, dv, q, k, v, gated ? al : NULL, gated ? be : NULL,
                            S0, based ? z0 : NULL, 1e-6, NULL, 0, o, ST, based ? zT : NULL, 2) == 0);
      const int rows[] = {4, 0, 2};
      EXPECT(oracle_prefill(var, B, H, T, kd, dv, q, k, v, gated ? al : NULL, gated ? be : NULL,
                            NULL, NULL, 1e-6, rows, 3, o, ST, based ? zT : NULL, 1) == 0);
      if (!based && T > 0) {
        double *oL = arr((size_t)T * dv), *SL = arr((size_t)dv * kd);
        EXPECT(oracle_literal(var, T, kd, dv, q, k, v, gated ? al : NULL, gated ? be : NULL, S0, oL, SL) == 0);
        free(oL); free(SL);
      }
      const int N = B * H;  /* one decode step per slice, from the start states (token 0's inputs) */
      if (T > 0)
        EXPECT(oracle_decode_step(var, N, kd, dv, S0, based ? z0 : NULL, q, k, v, gated ? al : NULL,
                                  gated ? be : NULL, 1e-6, ST, based ? zT : NULL, o, 1) == 0);
      free(q); free(k); free(v); free(al); free(be); free(S0); free(z0); free(o); free(ST); free(zT);
    }
  }
  /* rejected arguments */
  double x[64];
  EXPECT(oracle_prefill(7, 1, 1, 4, 4, 4, x, x, x, NULL, NULL, NULL, NULL, 1e-6, NULL, 0, x, NULL, NULL, 1) != 0);
  EXPECT(oracle_prefill(3, 1, 1, 4, 4, 4, x, x, x, NULL, NULL, NULL, NULL, 1e-6, NULL, 0, x, NULL, NULL, 1) != 0);
  const int bad_rows[] = {9};
  EXPECT(oracle_prefill(0, 1, 1, 4, 4, 4, x, x, x, NULL, NULL, NULL, NULL, 1e-6, bad_rows, 1, x, NULL, NULL, 1) != 0);
  { /* feature maps */
    double xin[4] = {0.3, -1.0, 2.0, 0.5}, f[32], fc[32];
    oracle_based_phi(xin, dp, f);
    oracle_based_phi_compact(xin, dp, fc);
  }
  { /* NoteBank steps: ragged write chunks, windows with a tail, addresses, votes */
    const int nb = 1, nh = 3, kd2 = 8, N = 5, drho = 4, J = nh, nQ = 6, R = 3;
    const long T = 150, Cw = 40, W = 12, tail = 8;
    double *kk = arr((size_t)nb * nh * T * kd2), *dh = arr((size_t)nb * nh * T), *dm = arr((size_t)nb * T);
    EXPECT(oracle_write_scores(nb, nh, T, kd2, Cw, kk, dh, dm) == 0);
    long starts[8];
    double sums[8];
    EXPECT(oracle_write_windows(nb, T, Cw, W, tail, dm, starts, sums) == 0);
    long spans[2 * 5] = {0, 20, 20, 25, 45, 45, 90, 30, 120, 30};  /* (start, length) */
    int coords[3 * 4] = {0, 1, 2, 3, 4, 5, 6, 7, 1, 3, 5, 7};
    long tstar[5 * 3];
    double *rho = arr((size_t)N * nh * drho);
    EXPECT(oracle_note_addresses(nb, nh, T, kd2, N, drho, dh, kk, spans, coords, tstar, rho) == 0);
    double *u = arr((size_t)nQ * J * drho), *score = arr((size_t)J * N);
    long pos[5] = {0, 20, 45, 90, 120};
    int choice[3], votes[5], sel[3];
    EXPECT(oracle_address_votes(N, J, nQ, drho, rho, u, R, pos, score, choice, votes, sel) == 0);
    EXPECT(oracle_address_votes(N, J, nQ, drho, rho, u, R, pos, NULL, choice, votes, sel) == 0);
    free(kk); free(dh); free(dm); free(rho); free(u); free(score);
  }
  if (fails) fprintf(stderr, "%d expectation(s) failed\n", fails);
  else printf("oracle driver: all calls as expected\n");
  return fails ? 1 : 0;
}
