// decode.hip -- one recurrence step for N independent states (batched decode).
//
// This is the memory-bound half of the library: each step must read every fp32 state
// once and write it once, which is the traffic the BASED notes point out a decode
// kernel cannot avoid (Sec. 2.5, paper Appendix B.2: the decode algorithm still reads
// and writes the persistent state).  The kernels therefore stream each state exactly
// once with 16-byte coalesced accesses and do all arithmetic in registers.
//
// Rows family (ADDITIVE / GATED / GATED_DELTA), Eq. (1) of "History Replays Itself",
// Sec. 2, written per state row s_r (a d_k-vector), using r = s_r.k and p = s_r.q of the
// *old* row:
//   GATED_DELTA  s_r' = alpha s_r + beta (v_r - alpha r) k,  o_r = alpha p + beta (v_r - alpha r)(k.q)
//   GATED        s_r' = alpha s_r + beta v_r k,               o_r = alpha p + beta v_r (k.q)
//   ADDITIVE     s_r' = s_r + v_r k,                          o_r = p + v_r (k.q)
// (o_r = s_r'.q expanded, so one read of the row serves both the update and the output.)
//
// BASED ("Simple linear attention ...", reading notes Sec. 2.2-2.3): with
// phi = [1, x, x_i x_j / sqrt 2],  s' = s + phi(k) v^T, z' = z + phi(k),
// o = s'^T phi(q) / (z'^T phi(q) + eps).
#include "la_device.h"
#include "la_launch.h"

namespace la {

// One workgroup of ROWS_NT threads per state.  A row of DK floats is spread over
// LPR = DK/8 lanes, 8 columns each as two float4 at column groups lr and lr + LPR, so the
// LPR lanes of a row read one contiguous run; ROWS_NT/LPR rows per pass, UNROLL passes
// loaded before any is used.  Eight waves with few rows each keep more requests in
// flight per CU than four waves with more rows each (which run at higher register use
// and lower occupancy): about 10% more bandwidth for 128 x 128 states.
//
// STREAM: the state set is larger than the 256 MB Infinity Cache can keep between steps,
// so every step streams it from HBM: 128 rows in flight and non-temporal loads and
// stores (which do not displace other data from the caches).  Measured on 128 x 128 states:
// 5.8 TB/s against 5.2 TB/s for the cached form once the set exceeds ~384 MiB; below that
// the cached form is faster (6.2-6.4 TB/s at 256 MiB, where part of the set stays cached).
constexpr int ROWS_NT = 512;
constexpr size_t STREAM_BYTES = (size_t)320 << 20;  // state sets above this stream

template <bool NT>
__device__ __forceinline__ float4 ld_state(const float *p) {
  if (NT) {
    const f32x4 t = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p));
    return make_float4(t[0], t[1], t[2], t[3]);
  }
  return *reinterpret_cast<const float4 *>(p);
}
template <bool NT>
__device__ __forceinline__ void st_state(float *p, float a, float b, float c, float d) {
  if (NT) __builtin_nontemporal_store(f32x4{a, b, c, d}, reinterpret_cast<f32x4 *>(p));
  else *reinterpret_cast<float4 *>(p) = make_float4(a, b, c, d);
}

// Threads per state: the streaming form at d = 256 keeps a whole 256 KB state in flight with
// 1024 threads (four passes of 64 rows): 5.8 TB/s on 512 MiB of states against 5.6 with 512.
template <int DK, bool STREAM> constexpr int rows_threads() { return (STREAM && DK == 256) ? 1024 : ROWS_NT; }

template <int DK, int VAR, typename T, bool STREAM>
__global__ __launch_bounds__((rows_threads<DK, STREAM>())) void decode_rows_kernel(int dv, int has_beta,
                                                          const float *S_in,
                                                          float *S_out, const T *__restrict__ q,
                                                          const T *__restrict__ k,
                                                          const T *__restrict__ v,
                                                          const T *__restrict__ alpha,
                                                          const T *__restrict__ beta,
                                                          T *__restrict__ o) {
  constexpr int LPR = DK / 8;
  constexpr int RPP = rows_threads<DK, STREAM>() / LPR;
  // streaming: 128 rows in flight (all of a 128 x 128 state; half of a 256 x 256 one)
  constexpr int UNROLL = STREAM ? (DK == 256 ? 4 : 8) : 2;
  const int n = blockIdx.x;
  const int tid = threadIdx.x;
  const int lr = tid % LPR;
  const int rp = tid / LPR;
  const int c0 = 4 * lr, c1 = 4 * (lr + LPR);

  float kk[8], qq[8];
  const size_t bqk = (size_t)n * DK;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    kk[j] = io<T>::ld(k, bqk + c0 + j);
    kk[4 + j] = io<T>::ld(k, bqk + c1 + j);
    qq[j] = io<T>::ld(q, bqk + c0 + j);
    qq[4 + j] = io<T>::ld(q, bqk + c1 + j);
  }
  float a = 1.0f, b = 1.0f;
  if (VAR != V_ADDITIVE) a = io<T>::ld(alpha, n);
  if (VAR == V_GATED_DELTA || (VAR == V_GATED && has_beta)) b = io<T>::ld(beta, n);
  float kq = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) kq += kk[j] * qq[j];
  kq = group_sum<LPR>(kq);

  const float *Sn = S_in + (size_t)n * dv * DK;
  float *So = S_out + (size_t)n * dv * DK;
  for (int r0 = 0; r0 < dv; r0 += RPP * UNROLL) {
    float4 s0[UNROLL], s1[UNROLL];
    float vr[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int r = r0 + u * RPP + rp;
      if (r < dv) {
        s0[u] = ld_state<STREAM>(Sn + (size_t)r * DK + c0);
        s1[u] = ld_state<STREAM>(Sn + (size_t)r * DK + c1);
        vr[u] = io<T>::ld(v, (size_t)n * dv + r);
      }
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int r = r0 + u * RPP + rp;
      if (r < dv) {  // uniform over the LPR lanes of a row, so the group shuffles are safe
        float x[8] = {s0[u].x, s0[u].y, s0[u].z, s0[u].w, s1[u].x, s1[u].y, s1[u].z, s1[u].w};
        float pr = 0.0f, pp = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          pr += x[j] * kk[j];
          pp += x[j] * qq[j];
        }
        pp = group_sum<LPR>(pp);
        float coef;
        if (VAR == V_GATED_DELTA) {
          pr = group_sum<LPR>(pr);
          coef = b * (vr[u] - a * pr);
        } else {
          coef = b * vr[u];
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = a * x[j] + coef * kk[j];
        st_state<STREAM>(So + (size_t)r * DK + c0, x[0], x[1], x[2], x[3]);
        st_state<STREAM>(So + (size_t)r * DK + c1, x[4], x[5], x[6], x[7]);
        if (lr == 0) io<T>::st(o, (size_t)n * dv + r, a * pp + coef * kq);
      }
    }
  }
}

// Pair (a, b), a <= b, of compact order-2 feature idx (row-major upper triangle of n x n).
__device__ __forceinline__ void triangle_pair(int idx, int n, int &a, int &b) {
  a = 0;
  while (idx >= n - a) {
    idx -= n - a;
    ++a;
  }
  b = a + idx;
}

// BASED decode: one workgroup (NT threads) per state, d' = 16, d_v = 64, D = 273 (or the
// compact D = 153: [1, x, x_a^2/sqrt 2 and x_a x_b for a < b]).  Thread t owns value
// columns 4(t%16)..+3 for the features f = t/16 + (NT/16) i, so every wave-wide access
// to s covers four whole 256-byte feature rows.
template <int NT, bool COMPACT, typename T>
__global__ __launch_bounds__(NT) void decode_based_kernel(float eps, const float *S_in,
                                                           const float *z_in,
                                                           float *S_out, float *z_out,
                                                           const T *__restrict__ q,
                                                           const T *__restrict__ k,
                                                           const T *__restrict__ v,
                                                           T *__restrict__ o) {
  constexpr int DP = 16, DV = 64, D = COMPACT ? 1 + DP + DP * (DP + 1) / 2 : 1 + DP + DP * DP;
  constexpr int NW = NT / 64, FS = NT / 16;
  __shared__ float xk[DP], xq[DP];
  __shared__ float phk[D], phq[D];
  __shared__ float4 red_num[NW][16];
  __shared__ float red_den[NW];
  const int n = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  if (tid < DP) xk[tid] = io<T>::ld(k, (size_t)n * DP + tid);
  else if (tid < 2 * DP) xq[tid - DP] = io<T>::ld(q, (size_t)n * DP + tid - DP);
  __syncthreads();
  const float rs2 = 0.70710678118654752f;
  for (int f = tid; f < D; f += NT) {
    float fk, fq;
    if (f == 0) { fk = 1.0f; fq = 1.0f; }
    else if (f <= DP) { fk = xk[f - 1]; fq = xq[f - 1]; }
    else if (COMPACT) {
      int i, j;
      triangle_pair(f - 1 - DP, DP, i, j);
      const float w = i == j ? rs2 : 1.0f;
      fk = xk[i] * xk[j] * w;
      fq = xq[i] * xq[j] * w;
    } else {
      const int i = (f - 1 - DP) >> 4, j = (f - 1 - DP) & 15;
      fk = xk[i] * xk[j] * rs2;
      fq = xq[i] * xq[j] * rs2;
    }
    phk[f] = fk;
    phq[f] = fq;
  }
  __syncthreads();

  const int cg = tid & 15, fo = tid >> 4;
  float4 vv;
  vv.x = io<T>::ld(v, (size_t)n * DV + 4 * cg + 0);
  vv.y = io<T>::ld(v, (size_t)n * DV + 4 * cg + 1);
  vv.z = io<T>::ld(v, (size_t)n * DV + 4 * cg + 2);
  vv.w = io<T>::ld(v, (size_t)n * DV + 4 * cg + 3);
  const float *Sn = S_in + (size_t)n * D * DV;
  float *So = S_out + (size_t)n * D * DV;
  float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
  constexpr int NI = (D + FS - 1) / FS;
  float4 sv[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int f = fo + FS * i;
    if (f < D) sv[i] = *reinterpret_cast<const float4 *>(Sn + (size_t)f * DV + 4 * cg);
  }
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int f = fo + FS * i;
    if (f < D) {
      const float pk = phk[f], pq = phq[f];
      float4 s = sv[i];
      s.x += pk * vv.x; s.y += pk * vv.y; s.z += pk * vv.z; s.w += pk * vv.w;
      *reinterpret_cast<float4 *>(So + (size_t)f * DV + 4 * cg) = s;
      num.x += pq * s.x; num.y += pq * s.y; num.z += pq * s.z; num.w += pq * s.w;
    }
  }
  // features handled by lanes l, l^16, l^32, l^48 of a wave share a column group
#pragma unroll
  for (int off = 16; off < 64; off <<= 1) {
    num.x += __shfl_xor(num.x, off, 64);
    num.y += __shfl_xor(num.y, off, 64);
    num.z += __shfl_xor(num.z, off, 64);
    num.w += __shfl_xor(num.w, off, 64);
  }
  if (lane < 16) red_num[wave][lane] = num;

  float dpart = 0.0f;
  for (int f = tid; f < D; f += NT) {
    const float z = z_in[(size_t)n * D + f] + phk[f];
    z_out[(size_t)n * D + f] = z;
    dpart += phq[f] * z;
  }
  dpart = group_sum<64>(dpart);
  if (lane == 0) red_den[wave] = dpart;
  __syncthreads();
  if (tid < 16) {
    float4 acc = red_num[0][tid];
#pragma unroll
    for (int w = 1; w < NW; ++w) {
      acc.x += red_num[w][tid].x; acc.y += red_num[w][tid].y;
      acc.z += red_num[w][tid].z; acc.w += red_num[w][tid].w;
    }
    float den = red_den[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) den += red_den[w];
    den += eps;
    io<T>::st(o, (size_t)n * DV + 4 * tid + 0, acc.x / den);
    io<T>::st(o, (size_t)n * DV + 4 * tid + 1, acc.y / den);
    io<T>::st(o, (size_t)n * DV + 4 * tid + 2, acc.z / den);
    io<T>::st(o, (size_t)n * DV + 4 * tid + 3, acc.w / den);
  }
}

template <int DK, int VAR, typename T>
static hipError_t go_rows(int n, int dv, int has_beta, const float *S_in, float *S_out,
                          const void *q, const void *k, const void *v, const void *alpha,
                          const void *beta, void *o, hipStream_t s) {
  if ((size_t)n * dv * DK * sizeof(float) > STREAM_BYTES)
    hipLaunchKernelGGL((decode_rows_kernel<DK, VAR, T, true>), dim3(n), dim3(rows_threads<DK, true>()), 0, s, dv,
                       has_beta, S_in,
                       S_out, (const T *)q, (const T *)k, (const T *)v, (const T *)alpha, (const T *)beta,
                       (T *)o);
  else
    hipLaunchKernelGGL((decode_rows_kernel<DK, VAR, T, false>), dim3(n), dim3(ROWS_NT), 0, s, dv, has_beta, S_in,
                       S_out, (const T *)q, (const T *)k, (const T *)v, (const T *)alpha, (const T *)beta,
                       (T *)o);
  return hipGetLastError();
}

template <int DK, typename T>
static hipError_t go_rows_v(int variant, int n, int dv, const float *S_in, float *S_out,
                            const void *q, const void *k, const void *v, const void *alpha,
                            const void *beta, void *o, hipStream_t s) {
  const int hb = beta != nullptr;
  switch (variant) {
    case V_ADDITIVE: return go_rows<DK, V_ADDITIVE, T>(n, dv, hb, S_in, S_out, q, k, v, alpha, beta, o, s);
    case V_GATED: return go_rows<DK, V_GATED, T>(n, dv, hb, S_in, S_out, q, k, v, alpha, beta, o, s);
    default: return go_rows<DK, V_GATED_DELTA, T>(n, dv, hb, S_in, S_out, q, k, v, alpha, beta, o, s);
  }
}

template <typename T>
static hipError_t go_rows_dk(int variant, int n, int dk, int dv, const float *S_in, float *S_out,
                             const void *q, const void *k, const void *v, const void *alpha,
                             const void *beta, void *o, hipStream_t s) {
  switch (dk) {
    case 64: return go_rows_v<64, T>(variant, n, dv, S_in, S_out, q, k, v, alpha, beta, o, s);
    case 128: return go_rows_v<128, T>(variant, n, dv, S_in, S_out, q, k, v, alpha, beta, o, s);
    default: return go_rows_v<256, T>(variant, n, dv, S_in, S_out, q, k, v, alpha, beta, o, s);
  }
}

hipError_t launch_decode_rows(int variant, int dtype, int n, int d_k, int d_v, const float *S_in,
                              float *S_out, const void *q, const void *k, const void *v,
                              const void *alpha, const void *beta, void *o, hipStream_t s) {
  if (dtype == T_BF16)
    return go_rows_dk<bf16_t>(variant, n, d_k, d_v, S_in, S_out, q, k, v, alpha, beta, o, s);
  return go_rows_dk<float>(variant, n, d_k, d_v, S_in, S_out, q, k, v, alpha, beta, o, s);
}

// Four waves per state: eight (512 threads, nine features per thread) measured no faster.
constexpr int BASED_NT = 256;

template <bool COMPACT>
static void go_based(int dtype, int n, float eps, const float *S_in, const float *z_in, float *S_out,
                     float *z_out, const void *q, const void *k, const void *v, void *o, hipStream_t s) {
  if (dtype == T_BF16)
    hipLaunchKernelGGL((decode_based_kernel<BASED_NT, COMPACT, bf16_t>), dim3(n), dim3(BASED_NT), 0, s, eps, S_in,
                       z_in, S_out, z_out, (const bf16_t *)q, (const bf16_t *)k, (const bf16_t *)v, (bf16_t *)o);
  else
    hipLaunchKernelGGL((decode_based_kernel<BASED_NT, COMPACT, float>), dim3(n), dim3(BASED_NT), 0, s, eps, S_in,
                       z_in, S_out, z_out, (const float *)q, (const float *)k, (const float *)v, (float *)o);
}

hipError_t launch_decode_based(int dtype, bool compact, int n, float eps, const float *S_in,
                               const float *z_in, float *S_out, float *z_out, const void *q,
                               const void *k, const void *v, void *o, hipStream_t s) {
  if (compact) go_based<true>(dtype, n, eps, S_in, z_in, S_out, z_out, q, k, v, o, s);
  else go_based<false>(dtype, n, eps, S_in, z_in, S_out, z_out, q, k, v, o, s);
  return hipGetLastError();
}

}  // namespace la
