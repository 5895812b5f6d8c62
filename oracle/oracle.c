/*
 * oracle.c -- plain, slow, fp64 CPU reference for the generalized linear-attention
 * recurrence.  TEST INFRASTRUCTURE ONLY: it is called from tests/, from the smoke
 * check and from the CPU-baseline leg of the benchmark, never from the library.
 * It shares no code, header or constant with the HIP path.
 *
 * What it computes (one layer, one head, token by token):
 *
 *   S_t = S_{t-1} A_t + beta_t v_t k_t^T ,   o_t = S_t q_t
 *
 *   [NoteBank] "History Replays Itself: Unleashing Long-Context Capability in Linear
 *   Attention", Sec. 2 (Preliminary), Eq. (1).  q_t, k_t in R^{d_k}, v_t in R^{d_v},
 *   S_t in R^{d_v x d_k}; A_t multiplies on the right.  Variants:
 *     ADDITIVE     A_t = I, beta_t = 1                    (same passage)
 *     GATED        A_t = alpha_t I                        (scalar-gated state)
 *     GATED_DELTA  A_t = alpha_t (I - beta_t k_t k_t^T)   (gated delta rule)
 *   The page names the gated and delta-rule families without printing them; the two
 *   forms above are the plainest members of those families and are the ones this
 *   library implements.  The write term beta_t v_t k_t^T is not scaled by alpha_t.
 *
 *   BASED          [BASED] "Simple linear attention language models balance the
 *   recall-throughput tradeoff" (reading notes, Sec. 2.2, paper Eqs. (1)-(3), and
 *   Sec. 2.3, paper Eq. (4)):
 *     phi(x) = [1, x, vec(x x^T)/sqrt(2)]   (D = 1 + d' + d'^2, order-2 index 1+d'+i*d'+j)
 *     s_t = s_{t-1} + phi(k_t) v_t^T  (D x d_v),   z_t = z_{t-1} + phi(k_t),  s_0 = z_0 = 0
 *     o_t = s_t^T phi(q_t) / (z_t^T phi(q_t) + eps)
 *   The notes say an implementation adds a small eps to the (positive) denominator;
 *   eps is an argument here.  No input scaling is applied (the caller pre-scales).
 *
 *   BASED_COMPACT  the same recurrence with the compact map of the same notes' feature-
 *   width table (Sec. 2.3): every cross term once,
 *     phi_c(x) = [1, x, (x_a^2/sqrt(2) if a == b else x_a x_b) for a <= b]
 *   (D = 1 + d' + d'(d'+1)/2; the pairs in row-major upper-triangle order, a outer:
 *   index 1 + d' + a d' - a(a-1)/2 + (b - a)).  phi_c(q).phi_c(k) equals
 *   phi(q).phi(k), so the outputs are those of BASED; only the state layout differs.
 *
 * Because A_t acts on the right of S, every row i of S (a d_k-vector) evolves on its
 * own:  s_i <- s_i A_t + beta_t v_t[i] k_t^T,  o_t[i] = s_i . q_t.  For the gated delta
 * rule  s_i A_t = alpha_t (s_i - beta_t (s_i . k_t) k_t^T).  The routines below walk
 * rows independently, which also lets a caller ask for a subset of rows (sampled
 * parity at very long T).  oracle_literal() instead builds the d_k x d_k matrix A_t
 * and multiplies it out, to pin the rank-1 form on tiny inputs.
 *
 * Layouts (row-major, last index fastest), identical to the library's:
 *   q, k  [B][H][T][d_k]     v, o  [B][H][T][d_v]     alpha, beta  [B][H][T]
 *   S     [B][H][d_v][d_k]   (ADDITIVE / GATED / GATED_DELTA)
 *   s     [B][H][D][d_v],  z [B][H][D]                (BASED / BASED_COMPACT, d_k = d')
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_ADDITIVE = 0, OR_BASED = 1, OR_GATED = 2, OR_GATED_DELTA = 3, OR_BASED_COMPACT = 4 };

int oracle_version(void) { return 1; }

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

static void set_threads(int nthreads) {
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
}

/* ---------------------------------------------------------------------------------
 * One row of S through T tokens (ADDITIVE, GATED, GATED_DELTA).
 *   s      : d_k doubles, in = row of S0, out = row of S_T
 *   o      : receives o_t[row] at o[t * o_stride]
 * beta == NULL means beta_t = 1 (allowed for GATED; ADDITIVE ignores alpha, beta).
 * ------------------------------------------------------------------------------- */
static void row_recurrence(int variant, long T, int dk, int dv, int row, const double *q,
                           const double *k, const double *v, const double *alpha,
                           const double *beta, double *s, double *o, long o_stride) {
  for (long t = 0; t < T; ++t) {
    const double *kt = k + (size_t)t * dk;
    const double *qt = q + (size_t)t * dk;
    const double vt = v[(size_t)t * dv + row];
    if (variant == OR_ADDITIVE) {
      /* s <- s I + 1 * v_t[row] k_t */
      for (int j = 0; j < dk; ++j) s[j] += vt * kt[j];
    } else if (variant == OR_GATED) {
      /* s <- s (alpha_t I) + beta_t v_t[row] k_t */
      const double a = alpha[t];
      const double b = beta ? beta[t] : 1.0;
      for (int j = 0; j < dk; ++j) s[j] = a * s[j] + b * vt * kt[j];
    } else { /* OR_GATED_DELTA */
      /* s <- s alpha_t (I - beta_t k_t k_t^T) + beta_t v_t[row] k_t
       *    = alpha_t (s - beta_t (s . k_t) k_t) + beta_t v_t[row] k_t           */
      const double a = alpha[t];
      const double b = beta[t];
      double r = 0.0;
      for (int j = 0; j < dk; ++j) r += s[j] * kt[j];
      for (int j = 0; j < dk; ++j) s[j] = a * (s[j] - b * r * kt[j]) + b * vt * kt[j];
    }
    /* o_t[row] = s_t . q_t  (the read happens after the write: o_t = S_t q_t) */
    double acc = 0.0;
    for (int j = 0; j < dk; ++j) acc += s[j] * qt[j];
    o[(size_t)t * o_stride] = acc;
  }
}

/* BASED feature map phi(x) = [1, x, vec(x x^T)/sqrt(2)], D = 1 + d' + d'^2. */
static void based_phi(const double *x, int dp, double *f) {
  const double inv_sqrt2 = 1.0 / sqrt(2.0);
  f[0] = 1.0;
  for (int i = 0; i < dp; ++i) f[1 + i] = x[i];
  for (int i = 0; i < dp; ++i)
    for (int j = 0; j < dp; ++j) f[1 + dp + i * dp + j] = x[i] * x[j] * inv_sqrt2;
}

void oracle_based_phi(const double *x, int dp, double *f) { based_phi(x, dp, f); }

/* Compact BASED feature map: [1, x, then for a <= b: x_a^2/sqrt(2) (a == b) or x_a x_b],
 * D = 1 + d' + d'(d'+1)/2. */
static void based_phi_compact(const double *x, int dp, double *f) {
  const double inv_sqrt2 = 1.0 / sqrt(2.0);
  int n = 0;
  f[n++] = 1.0;
  for (int i = 0; i < dp; ++i) f[n++] = x[i];
  for (int a = 0; a < dp; ++a)
    for (int b = a; b < dp; ++b) f[n++] = (a == b) ? x[a] * x[a] * inv_sqrt2 : x[a] * x[b];
}
void oracle_based_phi_compact(const double *x, int dp, double *f) { based_phi_compact(x, dp, f); }

static int based_dim(int dp, int compact) { return compact ? 1 + dp + dp * (dp + 1) / 2 : 1 + dp + dp * dp; }

/* One (b,h) slice of BASED through T tokens for a subset of value columns.
 *   s : [D][ncols] (in = s0 restricted to cols, out = s_T), z : [D] (in/out)
 *   o : [T][ncols]                                                              */
static void based_slice(int compact, long T, int dp, int dv, const int *cols, int ncols,
                        const double *q, const double *k, const double *v, double eps, double *s,
                        double *z, double *o) {
  const int D = based_dim(dp, compact);
  void (*phi)(const double *, int, double *) = compact ? based_phi_compact : based_phi;
  double *fk = (double *)malloc(sizeof(double) * D);
  double *fq = (double *)malloc(sizeof(double) * D);
  for (long t = 0; t < T; ++t) {
    phi(k + (size_t)t * dp, dp, fk);
    phi(q + (size_t)t * dp, dp, fq);
    /* s_t = s_{t-1} + phi(k_t) v_t^T,  z_t = z_{t-1} + phi(k_t) */
    for (int f = 0; f < D; ++f) {
      for (int c = 0; c < ncols; ++c) s[(size_t)f * ncols + c] += fk[f] * v[(size_t)t * dv + cols[c]];
      z[f] += fk[f];
    }
    /* o_t = s_t^T phi(q_t) / (z_t^T phi(q_t) + eps) */
    double den = 0.0;
    for (int f = 0; f < D; ++f) den += z[f] * fq[f];
    for (int c = 0; c < ncols; ++c) {
      double num = 0.0;
      for (int f = 0; f < D; ++f) num += s[(size_t)f * ncols + c] * fq[f];
      o[(size_t)t * ncols + c] = num / (den + eps);
    }
  }
  free(fk);
  free(fq);
}

/* ---------------------------------------------------------------------------------
 * oracle_prefill: the recurrence over T tokens for every (b, h).
 *
 *   rows / nrows : subset of value rows (GDN family) or value columns (BASED) to
 *                  compute; rows == NULL means all d_v of them.  Outputs are then
 *                  o [B][H][T][nrows], S_T [B][H][nrows][d_k] (GDN family) or
 *                  s_T [B][H][D][nrows], z_T [B][H][D] (BASED).
 *   S0 / z0      : NULL = zero start state (BASED: s_0 = 0, z_0 = 0).  S0 always has
 *                  the full layout [B][H][d_v][d_k] (or [B][H][D][d_v]).
 *   S_T / z_T    : may be NULL.
 * Returns 0, or -1 on invalid arguments.
 * ------------------------------------------------------------------------------- */
int oracle_prefill(int variant, int B, int H, long T, int dk, int dv, const double *q,
                   const double *k, const double *v, const double *alpha, const double *beta,
                   const double *S0, const double *z0, double eps, const int *rows, int nrows,
                   double *o, double *S_T, double *z_T, int nthreads) {
  if (B <= 0 || H <= 0 || T < 0 || dk <= 0 || dv <= 0 || !q || !k || !v || !o) return -1;
  if ((variant == OR_GATED || variant == OR_GATED_DELTA) && !alpha) return -1;
  if (variant == OR_GATED_DELTA && !beta) return -1;
  if (variant < 0 || variant > 4) return -1;
  const int nr = rows ? nrows : dv;
  for (int i = 0; i < nr; ++i)
    if (rows && (rows[i] < 0 || rows[i] >= dv)) return -1;
  set_threads(nthreads);

  if (variant == OR_BASED || variant == OR_BASED_COMPACT) {
    const int compact = variant == OR_BASED_COMPACT;
    const int dp = dk, D = based_dim(dp, compact);
    int *cols = (int *)malloc(sizeof(int) * nr);
    for (int c = 0; c < nr; ++c) cols[c] = rows ? rows[c] : c;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int b = 0; b < B; ++b)
      for (int h = 0; h < H; ++h) {
        const size_t bh = (size_t)b * H + h;
        double *s = (double *)calloc((size_t)D * nr, sizeof(double));
        double *z = (double *)calloc((size_t)D, sizeof(double));
        if (S0)
          for (int f = 0; f < D; ++f)
            for (int c = 0; c < nr; ++c) s[(size_t)f * nr + c] = S0[(bh * D + f) * dv + cols[c]];
        if (z0)
          for (int f = 0; f < D; ++f) z[f] = z0[bh * D + f];
        based_slice(compact, T, dp, dv, cols, nr, q + bh * T * dp, k + bh * T * dp, v + bh * T * dv,
                    eps, s, z, o + bh * T * nr);
        if (S_T) memcpy(S_T + bh * D * nr, s, sizeof(double) * D * nr);
        if (z_T) memcpy(z_T + bh * D, z, sizeof(double) * D);
        free(s);
        free(z);
      }
    free(cols);
    return 0;
  }

#pragma omp parallel for collapse(3) schedule(dynamic, 1)
  for (int b = 0; b < B; ++b)
    for (int h = 0; h < H; ++h)
      for (int ri = 0; ri < nr; ++ri) {
        const size_t bh = (size_t)b * H + h;
        const int row = rows ? rows[ri] : ri;
        double *s = (double *)malloc(sizeof(double) * dk);
        if (S0)
          memcpy(s, S0 + (bh * dv + row) * dk, sizeof(double) * dk);
        else
          memset(s, 0, sizeof(double) * dk);
        row_recurrence(variant, T, dk, dv, row, q + bh * T * dk, k + bh * T * dk,
                       v + bh * T * dv, alpha ? alpha + bh * T : NULL, beta ? beta + bh * T : NULL,
                       s, o + bh * T * nr + ri, nr);
        if (S_T) memcpy(S_T + (bh * nr + ri) * dk, s, sizeof(double) * dk);
        free(s);
      }
  return 0;
}

/* oracle_decode_step: one token of the recurrence for N independent (sequence, head)
 * states.  Layouts drop the T axis: q, k [N][d_k], v, o [N][d_v], alpha, beta [N],
 * S [N][d_v][d_k] (BASED: s [N][D][d_v], z [N][D]).  S_in == NULL means zero state. */
int oracle_decode_step(int variant, int N, int dk, int dv, const double *S_in, const double *z_in,
                       const double *q, const double *k, const double *v, const double *alpha,
                       const double *beta, double eps, double *S_out, double *z_out, double *o,
                       int nthreads) {
  /* One decode step is the recurrence with T = 1 on N slices (B = N, H = 1). */
  return oracle_prefill(variant, N, 1, 1, dk, dv, q, k, v, alpha, beta, S_in, z_in, eps, NULL, 0, o,
                        S_out, z_out, nthreads);
}

/* ---------------------------------------------------------------------------------
 * oracle_literal: the same recurrence with A_t built as an explicit d_k x d_k matrix
 * and S_t = S_{t-1} A_t + beta_t v_t k_t^T multiplied out in full (O(d_v d_k^2) per
 * token).  Only for tiny inputs: it pins the row-wise rank-1 form used above.
 * Variants: ADDITIVE, GATED, GATED_DELTA.  One (b,h) slice: q,k [T][dk], v,o [T][dv].
 * ------------------------------------------------------------------------------- */
int oracle_literal(int variant, long T, int dk, int dv, const double *q, const double *k,
                   const double *v, const double *alpha, const double *beta, const double *S0,
                   double *o, double *S_T) {
  if (variant == OR_BASED || variant < 0 || variant > 3) return -1;  /* not the BASED maps */
  double *S = (double *)calloc((size_t)dv * dk, sizeof(double));
  double *Sn = (double *)malloc(sizeof(double) * dv * dk);
  double *A = (double *)malloc(sizeof(double) * dk * dk);
  if (S0) memcpy(S, S0, sizeof(double) * dv * dk);
  for (long t = 0; t < T; ++t) {
    const double *kt = k + (size_t)t * dk;
    const double a = (variant == OR_ADDITIVE) ? 1.0 : alpha[t];
    const double b = (variant == OR_ADDITIVE) ? 1.0 : (beta ? beta[t] : 1.0);
    for (int i = 0; i < dk; ++i)
      for (int j = 0; j < dk; ++j) {
        double eye = (i == j) ? 1.0 : 0.0;
        A[i * dk + j] = (variant == OR_GATED_DELTA) ? a * (eye - b * kt[i] * kt[j]) : a * eye;
      }
    for (int r = 0; r < dv; ++r)
      for (int j = 0; j < dk; ++j) {
        double acc = 0.0;
        for (int i = 0; i < dk; ++i) acc += S[r * dk + i] * A[i * dk + j];
        Sn[r * dk + j] = acc + b * v[(size_t)t * dv + r] * kt[j];
      }
    memcpy(S, Sn, sizeof(double) * dv * dk);
    for (int r = 0; r < dv; ++r) {
      double acc = 0.0;
      for (int j = 0; j < dk; ++j) acc += S[r * dk + j] * q[(size_t)t * dk + j];
      o[(size_t)t * dv + r] = acc;
    }
  }
  if (S_T) memcpy(S_T, S, sizeof(double) * dv * dk);
  free(S);
  free(Sn);
  free(A);
  return 0;
}

/* =================================================================================
 * NoteBank write and address steps on the recurrence's keys and queries
 * ([NoteBank] "History Replays Itself: Unleashing Long-Context Capability in Linear
 * Attention", Sec. 3 Eqs. (3)-(5), App. B.2 Eq. (8), App. B.3 Eq. (9)).  One layer's
 * heads are the channels (l, h).  Argmax ties go to the earliest index (the pages fix
 * the tie rule only for the vote ranking, where earlier-inserted notes win).
 * ================================================================================= */

/* Key distinctiveness per write chunk of C tokens (the last, possibly partial, chunk over
 * its own tokens): khat_t = k_t/|k_t|, mu = mean of khat over the chunk, mubar = mu/|mu|,
 * d_t = 1 - <khat_t, mubar> per head; d_mean_t = mean of d_t over the H heads.
 * A zero vector normalises to zero.  k [B][H][T][dk]; d_head [B][H][T]; d_mean [B][T]. */
int oracle_write_scores(int B, int H, long T, int dk, long C, const double *k, double *d_head,
                        double *d_mean) {
  if (B <= 0 || H <= 0 || T < 0 || dk <= 0 || C <= 0 || !k || !d_head) return -1;
  double *mu = (double *)malloc(sizeof(double) * dk);
  for (int b = 0; b < B; ++b)
    for (int h = 0; h < H; ++h) {
      const double *kb = k + ((size_t)b * H + h) * T * dk;
      double *db = d_head + ((size_t)b * H + h) * T;
      for (long c0 = 0; c0 < T; c0 += C) {
        const long c1 = c0 + C < T ? c0 + C : T;
        for (int j = 0; j < dk; ++j) mu[j] = 0.0;
        for (long t = c0; t < c1; ++t) {
          double n = 0.0;
          for (int j = 0; j < dk; ++j) n += kb[t * dk + j] * kb[t * dk + j];
          n = sqrt(n);
          if (n > 0.0)
            for (int j = 0; j < dk; ++j) mu[j] += kb[t * dk + j] / n;
        }
        double mn = 0.0;
        for (int j = 0; j < dk; ++j) {
          mu[j] /= (double)(c1 - c0);
          mn += mu[j] * mu[j];
        }
        mn = sqrt(mn);
        for (long t = c0; t < c1; ++t) {
          double n = 0.0, dot = 0.0;
          for (int j = 0; j < dk; ++j) n += kb[t * dk + j] * kb[t * dk + j];
          n = sqrt(n);
          if (n > 0.0 && mn > 0.0)
            for (int j = 0; j < dk; ++j) dot += (kb[t * dk + j] / n) * (mu[j] / mn);
          db[t] = 1.0 - dot;
        }
      }
    }
  free(mu);
  if (d_mean)
    for (int b = 0; b < B; ++b)
      for (long t = 0; t < T; ++t) {
        double s = 0.0;
        for (int h = 0; h < H; ++h) s += d_head[((size_t)b * H + h) * T + t];
        d_mean[(size_t)b * T + t] = s / H;
      }
  return 0;
}

/* Best scoring window per complete write chunk (App. B.2): the candidate region of chunk
 * c is [max(0, cC - tail), (c+1)C), the chunk plus the previous chunk's last `tail`
 * tokens with their own scores; every window of W consecutive tokens inside it (the
 * whole region if it is shorter) is scored by the sum of d_mean; the highest wins.
 * A final incomplete chunk produces no note.  best_start / best_sum [B][T / C]. */
int oracle_write_windows(int B, long T, long C, long W, long tail, const double *d_mean,
                         long *best_start, double *best_sum) {
  if (B <= 0 || T < 0 || C <= 0 || W <= 0 || tail < 0 || !d_mean || !best_start) return -1;
  const long nc = T / C;
  for (int b = 0; b < B; ++b)
    for (long c = 0; c < nc; ++c) {
      const double *d = d_mean + (size_t)b * T;
      const long lo = c * C - tail > 0 ? c * C - tail : 0, hi = (c + 1) * C;
      const long w = hi - lo < W ? hi - lo : W;
      long bs = lo;
      double bv = -INFINITY;
      for (long s = lo; s + w <= hi; ++s) {
        double v = 0.0;
        for (long t = s; t < s + w; ++t) v += d[t];
        if (v > bv) {
          bv = v;
          bs = s;
        }
      }
      best_start[(size_t)b * nc + c] = bs;
      if (best_sum) best_sum[(size_t)b * nc + c] = bv;
    }
  return 0;
}

/* Note addresses (Eqs. (4), (9)): for note i with span [start, start + len) and head h,
 * t* = argmax over the span of d_head, and rho = the query at t* restricted to the head's
 * d_rho fixed coordinates.  spans [B][N][2]; coords [H][d_rho]; q [B][H][T][dk];
 * t_star [B][N][H]; rho [B][N][H][d_rho]. */
int oracle_note_addresses(int B, int H, long T, int dk, int N, int drho, const double *d_head,
                          const double *q, const long *spans, const int *coords, long *t_star,
                          double *rho) {
  if (B <= 0 || H <= 0 || T <= 0 || dk <= 0 || N < 0 || drho <= 0) return -1;
  for (int b = 0; b < B; ++b)
    for (int i = 0; i < N; ++i) {
      const long s0 = spans[((size_t)b * N + i) * 2], len = spans[((size_t)b * N + i) * 2 + 1];
      if (s0 < 0 || len < 1 || s0 + len > T) return -1;
      for (int h = 0; h < H; ++h) {
        const double *d = d_head + ((size_t)b * H + h) * T;
        long ts = s0;
        for (long t = s0 + 1; t < s0 + len; ++t)
          if (d[t] > d[ts]) ts = t;
        t_star[((size_t)b * N + i) * H + h] = ts;
        for (int r = 0; r < drho; ++r) {
          const int cidx = coords[h * drho + r];
          if (cidx < 0 || cidx >= dk) return -1;
          rho[(((size_t)b * N + i) * H + h) * drho + r] = q[(((size_t)b * H + h) * T + ts) * dk + cidx];
        }
      }
    }
  return 0;
}

/* Addressing and voting (Eq. (5)): s[j][i] = max over question positions tau of the
 * cosine of u_tau and rho_i in channel j (a zero vector has cosine 0); each channel votes
 * for its argmax note; V_i = number of channels voting for i.  Up to R notes with the
 * most votes (and at least one) are retrieved, earlier-inserted (lower index) first on
 * equal votes, then put in document order (by position, index on equal positions).
 * rho [N][J][drho]; u [nQ][J][drho]; score [J][N]; choice [J]; votes [N]; selected [R]
 * (-1 padded). */
int oracle_address_votes(int N, int J, int nQ, int drho, const double *rho, const double *u,
                         int R, const long *positions, double *score, int *choice, int *votes,
                         int *selected) {
  if (N <= 0 || J <= 0 || nQ <= 0 || drho <= 0 || R <= 0) return -1;
  for (int i = 0; i < N; ++i) votes[i] = 0;
  for (int j = 0; j < J; ++j) {
    int best = 0;
    double bestv = -INFINITY;
    for (int i = 0; i < N; ++i) {
      const double *r = rho + ((size_t)i * J + j) * drho;
      double rn = 0.0;
      for (int e = 0; e < drho; ++e) rn += r[e] * r[e];
      rn = sqrt(rn);
      double m = -INFINITY;
      for (int tau = 0; tau < nQ; ++tau) {
        const double *x = u + ((size_t)tau * J + j) * drho;
        double un = 0.0, dot = 0.0;
        for (int e = 0; e < drho; ++e) {
          un += x[e] * x[e];
          dot += x[e] * r[e];
        }
        un = sqrt(un);
        const double c = (un > 0.0 && rn > 0.0) ? dot / (un * rn) : 0.0;
        if (c > m) m = c;
      }
      if (score) score[(size_t)j * N + i] = m;
      if (m > bestv) {
        bestv = m;
        best = i;
      }
    }
    choice[j] = best;
    votes[best] += 1;
  }
  /* ranking: votes descending, index ascending */
  int nsel = 0;
  for (int r = 0; r < R; ++r) {
    int pick = -1;
    for (int i = 0; i < N; ++i) {
      if (votes[i] == 0) continue;
      int taken = 0;
      for (int s = 0; s < nsel; ++s)
        if (selected[s] == i) taken = 1;
      if (taken) continue;
      if (pick < 0 || votes[i] > votes[pick]) pick = i;
    }
    if (pick < 0) break;
    selected[nsel++] = pick;
  }
  /* document order */
  for (int a = 1; a < nsel; ++a)
    for (int c = a; c > 0; --c) {
      const int x = selected[c - 1], y = selected[c];
      if (positions[y] < positions[x] || (positions[y] == positions[x] && y < x)) {
        selected[c - 1] = y;
        selected[c] = x;
      }
    }
  for (int r = nsel; r < R; ++r) selected[r] = -1;
  return 0;
}
