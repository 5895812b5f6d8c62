// recurrent.hip -- token-recurrent prefill in fp32 arithmetic.
//
// This is the path for fp32 inputs, whose 1e-4 accuracy target rules out bf16 matrix
// operands.  It walks Eq. (1) of "History Replays Itself" (Sec. 2) token by token, one
// state row per group of lanes: because A_t multiplies S from the right, every row s_r
// of S evolves on its own, so rows are spread over waves and workgroups with no
// communication.  Per token and row, with r = s_r.k_t, p = s_r.q_t (old row):
//   GATED_DELTA  coef = beta_t (v_t[r] - alpha_t r),  GATED coef = beta_t v_t[r],
//   ADDITIVE     coef = v_t[r] (alpha = 1);
//   s_r <- alpha_t s_r + coef k_t,   o_t[r] = alpha_t p + coef (k_t.q_t)
// One reduction round (three partial sums over the 8 lanes that hold a row) serves the
// whole token.  Tokens are staged through LDS in tiles; outputs are gathered in LDS and
// written back a tile at a time.
//
// BASED: columns c of s are independent given the shared normaliser, so one
// workgroup per (b, h) keeps all of s in registers (value column per lane, features
// spread over the four waves) and reduces numerator and denominator partials per tile.
#include "la_device.h"
#include "la_launch.h"

namespace la {

template <int DK, int VAR, typename T>
__global__ __launch_bounds__(64) void recurrent_rows_kernel(int64_t T_len, int dv, int has_beta,
                                                            const T *__restrict__ q,
                                                            const T *__restrict__ k,
                                                            const T *__restrict__ v,
                                                            const T *__restrict__ alpha,
                                                            const T *__restrict__ beta,
                                                            const float *__restrict__ S0,
                                                            T *__restrict__ o, float *S_T) {
  constexpr int CPL = DK / 8;  // columns per lane
  constexpr int NG = CPL / 4;  // float4 groups per lane
  constexpr int TT = DK <= 128 ? 32 : 16;
  __shared__ float4 ks[TT][DK / 4];
  __shared__ float4 qs[TT][DK / 4];
  __shared__ float vs[TT][8];
  __shared__ float as_[TT], bs_[TT];
  __shared__ float os_[TT][8];
  const int lane = threadIdx.x;
  const int rw = lane >> 3, cgp = lane & 7;
  const int row0 = blockIdx.x * 8;
  const int row = row0 + rw;
  const int H = gridDim.y;
  const size_t bh = (size_t)blockIdx.z * H + blockIdx.y;
  const bool live = row < dv;

  float s[CPL];
#pragma unroll
  for (int g = 0; g < NG; ++g)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = 4 * (cgp + 8 * g) + j;
      s[4 * g + j] = (S0 && live) ? S0[(bh * dv + row) * DK + c] : 0.0f;
    }

  const T *qb = q + bh * (size_t)T_len * DK;
  const T *kb = k + bh * (size_t)T_len * DK;
  for (int64_t t0 = 0; t0 < T_len; t0 += TT) {
    const int nt = (int)((T_len - t0) < TT ? (T_len - t0) : TT);
    for (int i = lane; i < nt * (DK / 4); i += 64) {
      const int tt = i / (DK / 4), c4 = i % (DK / 4);
      const size_t off = (size_t)(t0 + tt) * DK + 4 * c4;
      ks[tt][c4] = make_float4(io<T>::ld(kb, off), io<T>::ld(kb, off + 1), io<T>::ld(kb, off + 2),
                               io<T>::ld(kb, off + 3));
      qs[tt][c4] = make_float4(io<T>::ld(qb, off), io<T>::ld(qb, off + 1), io<T>::ld(qb, off + 2),
                               io<T>::ld(qb, off + 3));
    }
    for (int i = lane; i < nt * 8; i += 64) {
      const int tt = i >> 3, rr = i & 7;
      vs[tt][rr] = (row0 + rr < dv) ? io<T>::ld(v, (bh * T_len + t0 + tt) * dv + row0 + rr) : 0.0f;
    }
    for (int i = lane; i < nt; i += 64) {
      as_[i] = (VAR == V_ADDITIVE) ? 1.0f : io<T>::ld(alpha, bh * T_len + t0 + i);
      bs_[i] = (VAR == V_GATED_DELTA || (VAR == V_GATED && has_beta))
                   ? io<T>::ld(beta, bh * T_len + t0 + i) : 1.0f;
    }
    __syncthreads();
    for (int tt = 0; tt < nt; ++tt) {
      float kv[CPL], qv[CPL];
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        const float4 a4 = ks[tt][cgp + 8 * g], b4 = qs[tt][cgp + 8 * g];
        kv[4 * g] = a4.x; kv[4 * g + 1] = a4.y; kv[4 * g + 2] = a4.z; kv[4 * g + 3] = a4.w;
        qv[4 * g] = b4.x; qv[4 * g + 1] = b4.y; qv[4 * g + 2] = b4.z; qv[4 * g + 3] = b4.w;
      }
      float pr = 0.f, pp = 0.f, pkq = 0.f;
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        pr += s[j] * kv[j];
        pp += s[j] * qv[j];
        pkq += kv[j] * qv[j];
      }
      pr = group_sum<8>(pr);
      pp = group_sum<8>(pp);
      pkq = group_sum<8>(pkq);
      const float a = as_[tt], b = bs_[tt], vt = vs[tt][rw];
      const float coef = (VAR == V_GATED_DELTA) ? b * (vt - a * pr) : b * vt;
#pragma unroll
      for (int j = 0; j < CPL; ++j) s[j] = a * s[j] + coef * kv[j];
      if (cgp == 0) os_[tt][rw] = a * pp + coef * pkq;
    }
    __syncthreads();
    for (int i = lane; i < nt * 8; i += 64) {
      const int tt = i >> 3, rr = i & 7;
      if (row0 + rr < dv) io<T>::st(o, (bh * T_len + t0 + tt) * dv + row0 + rr, os_[tt][rr]);
    }
    __syncthreads();
  }
  if (S_T && live) {
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
      for (int j = 0; j < 4; ++j) S_T[(bh * dv + row) * DK + 4 * (cgp + 8 * g) + j] = s[4 * g + j];
  }
}

// BASED, d' = 16, d_v = 64, D = 273 (COMPACT: D = 153, [1, x, x_a^2/sqrt 2 and x_a x_b
// for a < b in row-major upper-triangle order]).  Thread t: value column c = t % 64,
// features f = t/64 + 4 i.  z is kept per feature by every lane of the owning wave.
template <bool COMPACT, typename T>
__global__ __launch_bounds__(256) void recurrent_based_kernel(int64_t T_len, float eps,
                                                              const T *__restrict__ q,
                                                              const T *__restrict__ k,
                                                              const T *__restrict__ v,
                                                              const float *__restrict__ s0,
                                                              const float *__restrict__ z0,
                                                              T *__restrict__ o, float *s_T,
                                                              float *z_T) {
  constexpr int DP = 16, DV = 64, D = COMPACT ? 1 + DP + DP * (DP + 1) / 2 : 1 + DP + DP * DP;
  constexpr int NF = (D + 3) / 4, TT = 16;
  __shared__ float phk[TT][D + 3], phq[TT][D + 3];
  __shared__ float vs[TT][DV];
  __shared__ float part_num[4][TT][DV];
  __shared__ float part_den[4][TT];
  const int tid = threadIdx.x, c = tid & 63, fb = tid >> 6;
  const size_t bh = (size_t)blockIdx.x;
  float s[NF], z[NF];
#pragma unroll
  for (int i = 0; i < NF; ++i) {
    const int f = fb + 4 * i;
    s[i] = (s0 && f < D) ? s0[(bh * D + f) * DV + c] : 0.0f;
    z[i] = (z0 && f < D) ? z0[bh * D + f] : 0.0f;
  }
  const float rs2 = 0.70710678118654752f;
  for (int64_t t0 = 0; t0 < T_len; t0 += TT) {
    const int nt = (int)((T_len - t0) < TT ? (T_len - t0) : TT);
    for (int i = tid; i < nt * D; i += 256) {
      const int tt = i / D, f = i % D;
      const size_t base = (bh * T_len + t0 + tt) * DP;
      float fk, fq;
      if (f == 0) { fk = 1.0f; fq = 1.0f; }
      else if (f <= DP) { fk = io<T>::ld(k, base + f - 1); fq = io<T>::ld(q, base + f - 1); }
      else {
        int a, b = f - 1 - DP;  // order-2 feature: pair (a, b)
        float w = rs2;
        if (COMPACT) {
          a = 0;
          while (b >= DP - a) {
            b -= DP - a;
            ++a;
          }
          b += a;
          if (a != b) w = 1.0f;
        } else {
          a = b >> 4;
          b &= 15;
        }
        fk = io<T>::ld(k, base + a) * io<T>::ld(k, base + b) * w;
        fq = io<T>::ld(q, base + a) * io<T>::ld(q, base + b) * w;
      }
      phk[tt][f] = fk;
      phq[tt][f] = fq;
    }
    for (int i = tid; i < nt * DV; i += 256)
      vs[i / DV][i % DV] = io<T>::ld(v, (bh * T_len + t0) * DV + i);
    __syncthreads();
    for (int tt = 0; tt < nt; ++tt) {
      const float vc = vs[tt][c];
      float num = 0.f, den = 0.f;
#pragma unroll
      for (int i = 0; i < NF; ++i) {
        const int f = fb + 4 * i;
        if (f < D) {
          const float pk = phk[tt][f], pq = phq[tt][f];
          s[i] += pk * vc;
          z[i] += pk;
          num += pq * s[i];
          den += pq * z[i];
        }
      }
      part_num[fb][tt][c] = num;
      if (c == 0) part_den[fb][tt] = den;
    }
    __syncthreads();
    for (int i = tid; i < nt * DV; i += 256) {
      const int tt = i / DV, cc = i % DV;
      const float num = (part_num[0][tt][cc] + part_num[1][tt][cc]) +
                        (part_num[2][tt][cc] + part_num[3][tt][cc]);
      const float den = (part_den[0][tt] + part_den[1][tt]) + (part_den[2][tt] + part_den[3][tt]);
      io<T>::st(o, (bh * T_len + t0 + tt) * DV + cc, num / (den + eps));
    }
    __syncthreads();
  }
  if (s_T) {
#pragma unroll
    for (int i = 0; i < NF; ++i) {
      const int f = fb + 4 * i;
      if (f < D) {
        s_T[(bh * D + f) * DV + c] = s[i];
        if (c == 0) z_T[bh * D + f] = z[i];
      }
    }
  }
}

template <int DK, typename T>
static hipError_t go_rec(int variant, int B, int H, int64_t Tn, int dv, const void *q, const void *k,
                         const void *v, const void *alpha, const void *beta, const float *S0, void *o,
                         float *S_T, hipStream_t s) {
  dim3 grid((dv + 7) / 8, H, B);
  const int hb = beta != nullptr;
#define LA_REC(VAR)                                                                              \
  hipLaunchKernelGGL((recurrent_rows_kernel<DK, VAR, T>), grid, dim3(64), 0, s, Tn, dv, hb,      \
                     (const T *)q, (const T *)k, (const T *)v, (const T *)alpha, (const T *)beta, \
                     S0, (T *)o, S_T)
  if (variant == V_ADDITIVE) LA_REC(V_ADDITIVE);
  else if (variant == V_GATED) LA_REC(V_GATED);
  else LA_REC(V_GATED_DELTA);
#undef LA_REC
  return hipGetLastError();
}

template <typename T>
static hipError_t go_rec_dk(int variant, int B, int H, int64_t Tn, int dk, int dv, const void *q,
                            const void *k, const void *v, const void *alpha, const void *beta,
                            const float *S0, void *o, float *S_T, hipStream_t s) {
  if (dk == 64) return go_rec<64, T>(variant, B, H, Tn, dv, q, k, v, alpha, beta, S0, o, S_T, s);
  if (dk == 128) return go_rec<128, T>(variant, B, H, Tn, dv, q, k, v, alpha, beta, S0, o, S_T, s);
  return go_rec<256, T>(variant, B, H, Tn, dv, q, k, v, alpha, beta, S0, o, S_T, s);
}

// ---------------------------------------------------------------------------------------
// Short fp32 sequences, ADDITIVE and GATED (no delta term).  Unrolling Eq. (1) with
// g_t = sum_{i<=t} log alpha_i and gamma_t = e^{g_t}:
//   S_t = gamma_t S_0 + sum_{j<=t} beta_j e^{g_t - g_j} v_j k_j^T,
//   o_t = gamma_t S_0 q_t + sum_{j<=t} beta_j e^{g_t - g_j} (q_t . k_j) v_j,
// which is parallel over tokens (the masked attention form).  Up to QMAX_T tokens it
// replaces the token-by-token walk, whose per-token chain of reductions bounds a single
// head.  The gate prefix sums are fp64, so that g_t - g_j keeps its accuracy over thousands
// of tokens; everything else is fp32 with fixed summation orders.
constexpr int QMAX_T = 2048, QTOK = 16, QKEY = 64, QNT = 256, QDV = 128;

// g[0..n) = prefix sums of log alpha (fp64) for one (b, h), in LDS.
__device__ void gate_prefix(int n, const float *alpha, double *g, double *part) {
  const int tid = threadIdx.x, per = (n + QNT - 1) / QNT;
  const int lo = min(n, tid * per), hi = min(n, lo + per);
  double run = 0.0;
  for (int i = lo; i < hi; ++i) run += log((double)alpha[i]);
  part[tid] = run;
  __syncthreads();
  if (tid == 0) {  // exclusive scan of the 256 partial sums, in order
    double acc = 0.0;
    for (int w = 0; w < QNT; ++w) {
      const double x = part[w];
      part[w] = acc;
      acc += x;
    }
  }
  __syncthreads();
  run = part[tid];
  for (int i = lo; i < hi; ++i) {
    run += log((double)alpha[i]);
    g[i] = run;
  }
  __syncthreads();
}

// Outputs of QTOK tokens (all d_v columns) per workgroup: scores against key tiles of QKEY
// tokens in LDS, weighted and causally masked, then accumulated against the value tile.
template <int DK, int VAR>
__global__ __launch_bounds__(QNT) void quad_out_kernel(int64_t T_len, int dv, int has_beta,
                                                       const float *__restrict__ q, const float *__restrict__ k,
                                                       const float *__restrict__ v, const float *__restrict__ alpha,
                                                       const float *__restrict__ beta,
                                                       const float *__restrict__ S0, float *__restrict__ o) {
  __shared__ double g[QMAX_T];
  __shared__ double part[QNT];
  __shared__ float sq[QTOK][DK + 1], sk[QKEY][DK + 1], sv[QKEY][QDV], sp[QTOK][QKEY];
  const int tid = threadIdx.x;
  const size_t bh = blockIdx.y;
  const int T = (int)T_len;
  const int t0 = blockIdx.x * QTOK, nt = min(QTOK, T - t0), tend = t0 + nt;
  if (VAR == V_GATED) gate_prefix(tend, alpha + bh * T_len, g, part);
  for (int i = tid; i < nt * DK; i += QNT) sq[i / DK][i % DK] = q[(bh * T_len + t0 + i / DK) * DK + i % DK];
  __syncthreads();
  constexpr int NO = QTOK * QDV / QNT;  // outputs per thread (at most)
  float acc[NO];
#pragma unroll
  for (int m = 0; m < NO; ++m) {
    acc[m] = 0.0f;
    const int e = tid + QNT * m, tt = e / dv, c = e % dv;
    if (S0 && e < nt * dv) {  // gamma_t S_0 q_t
      const float *srow = S0 + (bh * dv + c) * DK;
      float x = 0.0f;
      for (int d = 0; d < DK; ++d) x += srow[d] * sq[tt][d];
      acc[m] = (VAR == V_GATED ? (float)exp(g[t0 + tt]) : 1.0f) * x;
    }
  }
  for (int j0 = 0; j0 < tend; j0 += QKEY) {
    const int nk = min(QKEY, tend - j0);
    __syncthreads();  // the previous tile is no longer read
    for (int i = tid; i < nk * DK; i += QNT) sk[i / DK][i % DK] = k[(bh * T_len + j0 + i / DK) * DK + i % DK];
    for (int i = tid; i < nk * dv; i += QNT) sv[i / dv][i % dv] = v[(bh * T_len + j0 + i / dv) * dv + i % dv];
    __syncthreads();
#pragma unroll
    for (int m = 0; m < QTOK * QKEY / QNT; ++m) {
      const int e = tid + QNT * m, tt = e / QKEY, jj = e % QKEY, t = t0 + tt, j = j0 + jj;
      float sc = 0.0f;
      if (tt < nt && jj < nk && j <= t) {
        for (int d = 0; d < DK; ++d) sc += sq[tt][d] * sk[jj][d];
        if (VAR == V_GATED)
          sc *= (has_beta ? beta[bh * T_len + j] : 1.0f) * (float)exp(g[t] - g[j]);
      }
      sp[tt][jj] = sc;
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < NO; ++m) {
      const int e = tid + QNT * m, tt = e / dv, c = e % dv;
      if (e < nt * dv)
        for (int jj = 0; jj < nk; ++jj) acc[m] += sp[tt][jj] * sv[jj][c];
    }
  }
#pragma unroll
  for (int m = 0; m < NO; ++m) {
    const int e = tid + QNT * m;
    if (e < nt * dv) o[(bh * T_len + t0 + e / dv) * dv + e % dv] = acc[m];
  }
}

// End state row c of one (b, h): S_T[c][d] = gamma_T S_0[c][d] + sum_j w_j v_j[c] k_j[d],
// w_j = beta_j e^{g_T - g_j}; the tokens are split over QNT / DK groups of threads, whose
// partial sums are added in a fixed order.
template <int DK, int VAR>
__global__ __launch_bounds__(QNT) void quad_state_kernel(int64_t T_len, int dv, int has_beta,
                                                         const float *__restrict__ k, const float *__restrict__ v,
                                                         const float *__restrict__ alpha,
                                                         const float *__restrict__ beta,
                                                         const float *__restrict__ S0, float *__restrict__ S_T) {
  __shared__ double g[QMAX_T];
  __shared__ double part[QNT];
  __shared__ float wv[QMAX_T];
  __shared__ float red[QNT];
  const int tid = threadIdx.x, c = blockIdx.x;
  const size_t bh = blockIdx.y;
  const int T = (int)T_len;
  if (VAR == V_GATED) gate_prefix(T, alpha + bh * T_len, g, part);
  for (int j = tid; j < T; j += QNT) {
    float w = 1.0f;
    if (VAR == V_GATED) w = (has_beta ? beta[bh * T_len + j] : 1.0f) * (float)exp(g[T - 1] - g[j]);
    wv[j] = w * v[(bh * T_len + j) * dv + c];
  }
  __syncthreads();
  constexpr int NG = QNT / DK;
  const int d = tid % DK, tg = tid / DK;
  float x = 0.0f;
  for (int j = tg; j < T; j += NG) x += wv[j] * k[(bh * T_len + j) * DK + d];
  red[tid] = x;
  __syncthreads();
  if (tg == 0) {
    float sum = red[d];
    for (int r = 1; r < NG; ++r) sum += red[r * DK + d];
    const size_t idx = (bh * dv + c) * DK + d;
    const float s0 = S0 ? S0[idx] : 0.0f;
    S_T[idx] = (VAR == V_GATED ? (float)exp(g[T - 1]) : 1.0f) * s0 + sum;
  }
}

// ---------------------------------------------------------------------------------------
// fp32 chunk form for short ADDITIVE / GATED prefills (fp32 inputs): Eq. (1) unrolled over
// chunks of 64 tokens (the BASED notes' Sec. 2.5 block form U_b = (M_b . Q K^T) V_b + Q S_{<b}
// with the scalar gate, derived from Eq. (1) of "History Replays Itself", Sec. 2):
//   g_t = in-chunk prefix of log alpha, G_c = g at the chunk's end, w_j = beta_j e^{G_c - g_j}
//   B_c = V^T diag(w) K                      (the chunk's contribution to the next state)
//   S_{c+1} = e^{G_c} S_c + B_c,  S_0 = S0
//   O_c = diag(e^{g}) Q S_c^T + (P . Q K^T . beta) V,  P_tj = e^{g_t - g_j} (j <= t)
// Every product runs on fp32 MFMA (v_mfma_f32_16x16x4_f32: fp32 operands, fp32 accumulate),
// so the path keeps fp32 accuracy.  Two launches: every chunk's B_c and G_c in parallel
// (fchunk_sum_kernel), then every chunk's start state as an elementwise prefix of the
// earlier B_j, held in registers in the operand layout of the Q S^T product, and the
// chunk's outputs (fchunk_out_kernel); the last chunk also writes S_T.  The first kernel
// also copies S0 into the workspace, so that S_T may be S0's own buffer.  The prefix re-reads
// up to nch - 1 sums per chunk, so the form serves short sequences (T <= FC_MAX_T).
//
// fp32 MFMA 16x16x4 layout: lane l supplies A[i][k] and B[k][j] with i = j = l % 16,
// k = l / 16; the accumulator lane l holds C[4 (l / 16) + e][l % 16], e = 0..3.
// B_c is stored so that lane (kk, j) of the wave owning value rows 16 ci .. 16 ci + 15 reads
// S[16 ci + j][4 s + kk] at ((ci (DK / 4) + s) 4 + kk) 16 + j: one coalesced 256-byte load
// per s.
constexpr int FC = 64, FC_MAX_T = 2048, FC_NT = 256, FC_MAXDV = 128;

__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Inclusive prefix sum over the 64 lanes of a wave (fixed order).
__device__ __forceinline__ float fc_wave_scan(float x, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  return x;
}

// Rows [0, n) of a [FC][ld] fp32 LDS tile from rows of `w` floats `stride` apart (rows past
// n zero); w a multiple of 4.
__device__ __forceinline__ void fc_tile(float *dst, int ld, const float *src, size_t stride, int w, int n, int tid) {
  const int w4 = w / 4;
  for (int i = tid; i < FC * w4; i += FC_NT) {
    const int r = i / w4, c4 = 4 * (i % w4);
    const float4 x = r < n ? *reinterpret_cast<const float4 *>(src + (size_t)r * stride + c4) : make_float4(0.f, 0.f, 0.f, 0.f);
    *reinterpret_cast<float4 *>(dst + r * ld + c4) = x;
  }
}

template <int DK, int VAR>
__global__ __launch_bounds__(FC_NT) void fchunk_sum_kernel(int64_t T_len, int dv, int has_beta,
                                                           const float *__restrict__ k, const float *__restrict__ v,
                                                           const float *__restrict__ alpha,
                                                           const float *__restrict__ beta, const float *S0,
                                                           float *__restrict__ bsum, float *__restrict__ gsum) {
  constexpr int LK = DK + 4, LV = FC_MAXDV + 4;
  __shared__ __attribute__((aligned(16))) float sK[FC * LK];
  __shared__ __attribute__((aligned(16))) float sV[FC * LV];
  __shared__ float sW[FC];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, i16 = lane & 15, g4 = lane >> 4;
  const int c = blockIdx.x, nch = gridDim.x;
  const size_t bh = blockIdx.y;
  const int64_t t0 = (int64_t)c * FC;
  const int n = (int)((T_len - t0) < FC ? (T_len - t0) : FC);
  fc_tile(sK, LK, k + (bh * T_len + t0) * DK, DK, DK, n, tid);
  fc_tile(sV, LV, v + (bh * T_len + t0) * dv, dv, dv, n, tid);
  if (wave == 0) {
    const size_t at = bh * T_len + t0 + lane;
    const float la = (VAR == V_GATED && lane < n) ? __logf(alpha[at]) : 0.0f;
    const float gt = fc_wave_scan(la, lane);
    const float G = __shfl(gt, 63, 64);
    const float b = lane < n ? ((VAR == V_GATED && has_beta) ? beta[at] : 1.0f) : 0.0f;
    sW[lane] = VAR == V_GATED ? b * __expf(G - gt) : b;
    if (lane == 0) gsum[bh * nch + c] = G;
  }
  __syncthreads();
  // slab 0 of (b, h): the start state in the same layout, so that the output kernel never
  // reads S0 (S_T, which its last chunk writes, may be S0's buffer)
  const int ndi = DK / 16, nci = dv / 16;
  if (c == 0) {
    float *d0 = bsum + bh * (nch + 1) * (size_t)dv * DK;
    for (int ci = wave; ci < nci; ci += 4)
      for (int s = 0; s < DK / 4; ++s)
        d0[(ci * (DK / 4) + s) * 64 + lane] = S0 ? S0[(bh * dv + 16 * ci + i16) * DK + 4 * s + g4] : 0.0f;
  }
  // tiles of B_c^T: (di, ci), k = tokens; lane (g4, i16) ends with B_c[16 ci + i16][16 di + 4 g4 + e]
  float *dst = bsum + (bh * (nch + 1) + c + 1) * (size_t)dv * DK;
  for (int tile = wave; tile < ndi * nci; tile += 4) {
    const int di = tile % ndi, ci = tile / ndi;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < FC / 4; ++s) {
      const int j = 4 * s + g4;
      acc = mfma_f32(sK[j * LK + 16 * di + i16], sW[j] * sV[j * LV + 16 * ci + i16], acc);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) dst[((ci * (DK / 4) + 4 * di + g4) * 4 + e) * 16 + i16] = acc[e];
  }
}

template <int DK, int VAR>
__global__ __launch_bounds__(FC_NT) void fchunk_out_kernel(int64_t T_len, int dv, int has_beta,
                                                           const float *__restrict__ q, const float *__restrict__ k,
                                                           const float *__restrict__ v, const float *__restrict__ alpha,
                                                           const float *__restrict__ beta,
                                                           const float *__restrict__ bsum,
                                                           const float *__restrict__ gsum, float *__restrict__ o,
                                                           float *S_T) {
  constexpr int LK = DK + 4, LV = FC_MAXDV + 4, LA = FC + 4, NS = DK / 4;
  constexpr int NCI = FC_MAXDV / 16 / 4;  // value-row tiles per wave, at most
  __shared__ __attribute__((aligned(16))) float sQ[FC * LK];
  __shared__ __attribute__((aligned(16))) float sK[FC * LK];
  __shared__ __attribute__((aligned(16))) float sV[FC * LV];
  __shared__ __attribute__((aligned(16))) float sA[FC * LA];
  __shared__ float sg[FC], sb[FC];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, i16 = lane & 15, g4 = lane >> 4;
  const int c = blockIdx.x, nch = gridDim.x;
  const size_t bh = blockIdx.y;
  const int64_t t0 = (int64_t)c * FC;
  const int n = (int)((T_len - t0) < FC ? (T_len - t0) : FC);
  const int nci = dv / 16;
  fc_tile(sQ, LK, q + (bh * T_len + t0) * DK, DK, DK, n, tid);
  fc_tile(sK, LK, k + (bh * T_len + t0) * DK, DK, DK, n, tid);
  fc_tile(sV, LV, v + (bh * T_len + t0) * dv, dv, dv, n, tid);
  if (wave == 0) {
    const size_t at = bh * T_len + t0 + lane;
    const float la = (VAR == V_GATED && lane < n) ? __logf(alpha[at]) : 0.0f;
    sg[lane] = fc_wave_scan(la, lane);
    sb[lane] = lane < n ? ((VAR == V_GATED && has_beta) ? beta[at] : 1.0f) : 0.0f;
  }

  // start state of this chunk: lane (g4, i16) of wave w keeps S[16 ci + i16][4 s + g4] for its
  // tiles ci = w + 4 m, every s; slab 0 holds S0, slab j + 1 the sum B_j of chunk j
  const float *slabs = bsum + bh * (nch + 1) * (size_t)dv * DK;
  float S[NCI][NS];
#pragma unroll
  for (int m = 0; m < NCI; ++m) {
    const int ci = wave + 4 * m;
#pragma unroll
    for (int s = 0; s < NS; ++s) S[m][s] = ci < nci ? slabs[(ci * NS + s) * 64 + lane] : 0.0f;
  }
  auto accumulate = [&](int j) {  // S <- e^{G_j} S + B_j
    const float dec = VAR == V_GATED ? __expf(gsum[bh * nch + j]) : 1.0f;
    const float *src = slabs + (size_t)(j + 1) * dv * DK;
#pragma unroll
    for (int m = 0; m < NCI; ++m) {
      const int ci = wave + 4 * m;
      if (ci < nci) {
#pragma unroll
        for (int s = 0; s < NS; ++s) S[m][s] = dec * S[m][s] + src[(ci * NS + s) * 64 + lane];
      }
    }
  };
  for (int j = 0; j < c; ++j) accumulate(j);
  __syncthreads();

  // decay-masked Q K^T into LDS (tiles above the diagonal are zero)
  for (int tile = wave; tile < 16; tile += 4) {
    const int ti = tile / 4, tj = tile % 4;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (tj <= ti) {
#pragma unroll
      for (int s = 0; s < NS; ++s)
        acc = mfma_f32(sQ[(16 * ti + i16) * LK + 4 * s + g4], sK[(16 * tj + i16) * LK + 4 * s + g4], acc);
    }
    const int jj = 16 * tj + i16;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = 16 * ti + 4 * g4 + e;
      float x = 0.0f;
      if (tj <= ti && jj <= t) x = VAR == V_GATED ? acc[e] * sb[jj] * __expf(sg[t] - sg[jj]) : acc[e];
      sA[t * LA + jj] = x;
    }
  }
  __syncthreads();

  // outputs: for each value-row tile of this wave and each token tile,
  // O = diag(e^{g}) Q S^T + A V
#pragma unroll
  for (int m = 0; m < NCI; ++m) {
    const int ci = wave + 4 * m;
    if (ci >= nci) break;
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NS; ++s) acc = mfma_f32(sQ[(16 * ti + i16) * LK + 4 * s + g4], S[m][s], acc);
      if (VAR == V_GATED) {
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] *= __expf(sg[16 * ti + 4 * g4 + e]);
      }
#pragma unroll
      for (int s = 0; s < FC / 4; ++s)
        acc = mfma_f32(sA[(16 * ti + i16) * LA + 4 * s + g4], sV[(4 * s + g4) * LV + 16 * ci + i16], acc);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * ti + 4 * g4 + e;
        if (t < n) o[(bh * T_len + t0 + t) * dv + 16 * ci + i16] = acc[e];
      }
    }
  }

  if (c == nch - 1 && S_T) {  // the end state: S_T = e^{G_c} S_c + B_c
    accumulate(c);
#pragma unroll
    for (int m = 0; m < NCI; ++m) {
      const int ci = wave + 4 * m;
      if (ci < nci) {
#pragma unroll
        for (int s = 0; s < NS; ++s) S_T[(bh * dv + 16 * ci + i16) * DK + 4 * s + g4] = S[m][s];
      }
    }
  }
}

// Whether the fp32 chunk form takes this problem: ADDITIVE or GATED, fp32, at least two
// chunks and at most FC_MAX_T tokens, d_k in {64, 128}, d_v a multiple of 16 up to 128, and
// small (B H nch^2 <= 4096: its chunk sums are re-read by every later chunk).
static bool fchunk_ok(int variant, int64_t BH, int64_t T, int dk, int dv) {
  const int64_t nch = (T + FC - 1) / FC;
  return (variant == V_ADDITIVE || variant == V_GATED) && nch >= 2 && T <= FC_MAX_T && BH * nch * nch <= 4096 &&
         (dk == 64 || dk == 128) && dv % 16 == 0 && dv >= 16 && dv <= FC_MAXDV;
}

size_t fp32_chunk_workspace_bytes(int variant, int B, int H, int64_t T, int d_k, int d_v) {
  const int64_t BH = (int64_t)B * H;
  if (!fchunk_ok(variant, BH, T, d_k, d_v)) return 0;
  const size_t nch = (size_t)((T + FC - 1) / FC);
  return ((size_t)BH * (nch + 1) * d_v * d_k * sizeof(float) + 255) / 256 * 256 + (size_t)BH * nch * sizeof(float);
}

template <int DK, int VAR>
static void go_fchunk(int B, int H, int64_t T, int dv, int has_beta, const float *q, const float *k, const float *v,
                      const float *alpha, const float *beta, const float *S0, float *o, float *S_T, void *ws,
                      hipStream_t s) {
  const unsigned bh = (unsigned)((int64_t)B * H), nch = (unsigned)((T + FC - 1) / FC);
  float *bsum = (float *)ws;  // [B H][nch + 1][d_v d_k]: the start state, then every chunk's sum
  float *gsum = (float *)((char *)ws + ((size_t)bh * (nch + 1) * dv * DK * sizeof(float) + 255) / 256 * 256);
  hipLaunchKernelGGL((fchunk_sum_kernel<DK, VAR>), dim3(nch, bh), dim3(FC_NT), 0, s, T, dv, has_beta, k, v, alpha,
                     beta, S0, bsum, gsum);
  hipLaunchKernelGGL((fchunk_out_kernel<DK, VAR>), dim3(nch, bh), dim3(FC_NT), 0, s, T, dv, has_beta, q, k, v, alpha,
                     beta, bsum, gsum, o, S_T);
}

// Whether the attention form takes this problem (fp32 inputs only): its work grows as
// B H T^2 while the token walk's time grows as T (given enough parallel rows), so only
// small problems: T <= QMAX_T and B H ceil(T / 64)^2 <= 4096 (one head of 4096 tokens' worth).
static bool quad_ok(int variant, int64_t BH, int64_t T, int dk, int dv) {
  const int64_t tiles = (T + QKEY - 1) / QKEY;
  return (variant == V_ADDITIVE || variant == V_GATED) && T >= 1 && T <= QMAX_T && BH * tiles * tiles <= 4096 &&
         (dk == 64 || dk == 128) && dv >= 1 && dv <= QDV;
}

template <int DK, int VAR>
static void go_quad(int B, int H, int64_t T, int dv, int has_beta, const float *q, const float *k, const float *v,
                    const float *alpha, const float *beta, const float *S0, float *o, float *S_T, hipStream_t s) {
  const unsigned bh = (unsigned)((int64_t)B * H);
  hipLaunchKernelGGL((quad_out_kernel<DK, VAR>), dim3((unsigned)((T + QTOK - 1) / QTOK), bh), dim3(QNT), 0, s, T,
                     dv, has_beta, q, k, v, alpha, beta, S0, o);
  if (S_T)
    hipLaunchKernelGGL((quad_state_kernel<DK, VAR>), dim3((unsigned)dv, bh), dim3(QNT), 0, s, T, dv, has_beta, k, v,
                       alpha, beta, S0, S_T);
}

hipError_t launch_recurrent_rows(int variant, int dtype, int B, int H, int64_t T, int d_k, int d_v,
                                 const void *q, const void *k, const void *v, const void *alpha,
                                 const void *beta, const float *S0, void *o, float *S_T, void *workspace,
                                 size_t ws_bytes, hipStream_t s) {
  if (dtype == T_BF16)
    return go_rec_dk<bf16_t>(variant, B, H, T, d_k, d_v, q, k, v, alpha, beta, S0, o, S_T, s);
  const size_t fws = fp32_chunk_workspace_bytes(variant, B, H, T, d_k, d_v);
  if (fws > 0 && workspace && fws <= ws_bytes) {  // short fp32 sequences: the chunk form
    const float *fq = (const float *)q, *fk = (const float *)k, *fv = (const float *)v;
    const float *fa = (const float *)alpha, *fb = (const float *)beta;
    const int hb = beta != nullptr;
    float *fo = (float *)o;
    if (variant == V_ADDITIVE) {
      if (d_k == 64) go_fchunk<64, V_ADDITIVE>(B, H, T, d_v, hb, fq, fk, fv, fa, fb, S0, fo, S_T, workspace, s);
      else go_fchunk<128, V_ADDITIVE>(B, H, T, d_v, hb, fq, fk, fv, fa, fb, S0, fo, S_T, workspace, s);
    } else {
      if (d_k == 64) go_fchunk<64, V_GATED>(B, H, T, d_v, hb, fq, fk, fv, fa, fb, S0, fo, S_T, workspace, s);
      else go_fchunk<128, V_GATED>(B, H, T, d_v, hb, fq, fk, fv, fa, fb, S0, fo, S_T, workspace, s);
    }
    return hipGetLastError();
  }
  if (quad_ok(variant, (int64_t)B * H, T, d_k, d_v)) {  // short fp32 sequences without the delta term
    const float *fq = (const float *)q, *fk = (const float *)k, *fv = (const float *)v;
    const float *fa = (const float *)alpha, *fb = (const float *)beta;
    const int hb = beta != nullptr;
    if (variant == V_ADDITIVE) {
      if (d_k == 64) go_quad<64, V_ADDITIVE>(B, H, T, d_v, hb, fq, fk, fv, fa, fb, S0, (float *)o, S_T, s);
      else go_quad<128, V_ADDITIVE>(B, H, T, d_v, hb, fq, fk, fv, fa, fb, S0, (float *)o, S_T, s);
    } else {
      if (d_k == 64) go_quad<64, V_GATED>(B, H, T, d_v, hb, fq, fk, fv, fa, fb, S0, (float *)o, S_T, s);
      else go_quad<128, V_GATED>(B, H, T, d_v, hb, fq, fk, fv, fa, fb, S0, (float *)o, S_T, s);
    }
    return hipGetLastError();
  }
  return go_rec_dk<float>(variant, B, H, T, d_k, d_v, q, k, v, alpha, beta, S0, o, S_T, s);
}

template <bool COMPACT>
static void go_rec_based(int dtype, int B, int H, int64_t T, float eps, const void *q, const void *k,
                         const void *v, const float *s0, const float *z0, void *o, float *s_T,
                         float *z_T, hipStream_t s) {
  const dim3 grid((unsigned)((int64_t)B * H));
  if (dtype == T_BF16)
    hipLaunchKernelGGL((recurrent_based_kernel<COMPACT, bf16_t>), grid, dim3(256), 0, s, T, eps,
                       (const bf16_t *)q, (const bf16_t *)k, (const bf16_t *)v, s0, z0, (bf16_t *)o,
                       s_T, z_T);
  else
    hipLaunchKernelGGL((recurrent_based_kernel<COMPACT, float>), grid, dim3(256), 0, s, T, eps,
                       (const float *)q, (const float *)k, (const float *)v, s0, z0, (float *)o, s_T,
                       z_T);
}

hipError_t launch_recurrent_based(int dtype, bool compact, int B, int H, int64_t T, float eps,
                                  const void *q, const void *k, const void *v, const float *s0,
                                  const float *z0, void *o, float *s_T, float *z_T, hipStream_t s) {
  if (compact) go_rec_based<true>(dtype, B, H, T, eps, q, k, v, s0, z0, o, s_T, z_T, s);
  else go_rec_based<false>(dtype, B, H, T, eps, q, k, v, s0, z0, o, s_T, z_T, s);
  return hipGetLastError();
}

}  // namespace la
