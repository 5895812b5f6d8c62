// notebank.hip -- the NoteBank write and address steps that sit on the recurrence's keys
// and queries ("History Replays Itself: Unleashing Long-Context Capability in Linear
// Attention", Sec. 3 Eqs. (3)-(5), App. B.2 Eq. (8), App. B.3 Eq. (9)).  One layer's heads
// are the channels (l, h).
//
//   write_scores_kernel   per write chunk of C tokens and head: khat_t = k_t / |k_t|, the
//                         normalised mean mubar of the chunk's khat, d_t = 1 - <khat_t, mubar>
//                         (Eqs. (3), (8)); a partial last chunk uses its own tokens.
//   head_mean_kernel      d_mean_t = mean of d_t over the heads (the channel average).
//   write_windows_kernel  per complete write chunk, the W-token window with the largest sum
//                         of d_mean over the chunk plus the previous chunk's last `tail`
//                         tokens (App. B.2); the earliest window wins ties.
//   note_address_kernel   per note and head, t* = argmax of d_t over the note's span (the
//                         earliest on ties) and rho = q_{t*} on the head's fixed coordinates
//                         (Eqs. (4), (9)).
//   channel_vote_kernel   per channel, s_i = max over question positions of the fp32 cosine
//                         of u_tau and rho_i, and the channel's vote = argmax_i s_i (Eq. (5)).
//   select_notes_kernel   votes per note, the (at most R) notes with the most votes (earlier
//                         notes first on equal votes) and their document order.
//
// All of it is bandwidth- or latency-light next to the recurrence: the write scores read
// each bf16 key once from HBM (a chunk of up to 512 tokens is held in registers), the rest
// touch kilobytes.  Every reduction has a fixed order, so results are bitwise reproducible.
#include "la_device.h"
#include "la_launch.h"

namespace la {
namespace nb {

constexpr int WS_THREADS = 256;

template <typename T> __device__ __forceinline__ void load8(const T *p, float (&x)[8]);
template <> __device__ __forceinline__ void load8<float>(const float *p, float (&x)[8]) {
  const float4 a = *reinterpret_cast<const float4 *>(p), b = *reinterpret_cast<const float4 *>(p + 4);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
template <> __device__ __forceinline__ void load8<bf16_t>(const bf16_t *p, float (&x)[8]) {
  const u32x4 w = gld16(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

// One workgroup per (write chunk, head, batch).  A key of DK values is spread over
// LPT = DK/8 lanes (8 values, 16 or 32 bytes each); a wave covers 64/LPT tokens per step.
template <int DK, typename T>
__global__ __launch_bounds__(WS_THREADS) void write_scores_kernel(int64_t T_len, int C,
                                                                  const T *__restrict__ k,
                                                                  float *__restrict__ d_head) {
  constexpr int LPT = DK / 8, TPW = 64 / LPT, NW = WS_THREADS / 64, TPS = NW * TPW;
  __shared__ float s_mu[NW][DK];
  __shared__ float s_mubar[DK];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sub = lane % LPT, tok = lane / LPT;
  const size_t bh = (size_t)blockIdx.z * gridDim.y + blockIdx.y;
  const int64_t c0 = (int64_t)blockIdx.x * C;
  const int n = (int)((T_len - c0) < C ? (T_len - c0) : C);
  const T *kc = k + (bh * T_len + c0) * DK;

  // pass 1: sum of the unit keys (the 1/|chunk| of the mean cancels in the normalisation);
  // UNR token steps loaded before any is used
  constexpr int UNR = 4;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int t0 = wave * TPW + tok; t0 < n; t0 += UNR * TPS) {
    float x[UNR][8];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int t = t0 + u * TPS;
      if (t < n) load8<T>(kc + (size_t)t * DK + 8 * sub, x[u]);
      else
#pragma unroll
        for (int j = 0; j < 8; ++j) x[u][j] = 0.0f;
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      float ss = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) ss += x[u][j] * x[u][j];
      ss = group_sum<LPT>(ss);
      const float inv = ss > 0.0f ? 1.0f / sqrtf(ss) : 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] += x[u][j] * inv;
    }
  }
  // lanes with the same `sub` hold the same 8 coordinates: fold the token groups
#pragma unroll
  for (int off = LPT; off < 64; off <<= 1)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] += __shfl_xor(acc[j], off, 64);
  if (tok == 0)
#pragma unroll
    for (int j = 0; j < 8; ++j) s_mu[wave][8 * sub + j] = acc[j];
  __syncthreads();
  if (tid < DK) {
    float m = s_mu[0][tid];
#pragma unroll
    for (int w = 1; w < NW; ++w) m += s_mu[w][tid];
    s_mubar[tid] = m;
  }
  __syncthreads();
  if (wave == 0) {  // |mu|, then mubar = mu / |mu| (zero stays zero)
    float ss = 0.0f;
    for (int i = lane; i < DK; i += 64) ss += s_mubar[i] * s_mubar[i];
    ss = group_sum<64>(ss);
    const float inv = ss > 0.0f ? 1.0f / sqrtf(ss) : 0.0f;
    for (int i = lane; i < DK; i += 64) s_mubar[i] *= inv;
  }
  __syncthreads();

  // pass 2: d_t = 1 - <k_t, mubar> / |k_t| (the chunk was just read: an L2 hit)
  float mb[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) mb[j] = s_mubar[8 * sub + j];
  float *dh = d_head + bh * T_len + c0;
  for (int t0 = wave * TPW + tok; t0 < n; t0 += UNR * TPS) {
    float x[UNR][8];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int t = t0 + u * TPS;
      if (t < n) load8<T>(kc + (size_t)t * DK + 8 * sub, x[u]);
      else
#pragma unroll
        for (int j = 0; j < 8; ++j) x[u][j] = 0.0f;
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      float ss = 0.0f, dot = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        ss += x[u][j] * x[u][j];
        dot += x[u][j] * mb[j];
      }
      ss = group_sum<LPT>(ss);
      dot = group_sum<LPT>(dot);
      const int t = t0 + u * TPS;
      if (sub == 0 && t < n) dh[t] = 1.0f - (ss > 0.0f ? dot / sqrtf(ss) : 0.0f);
    }
  }
}

// bf16 keys and write chunks of at most 512 tokens: one 1024-thread workgroup holds the whole
// chunk in registers (a lane keeps 16 bytes of a key per token step: 32 registers at d_k = 128,
// 64 at 256), so each key is read from HBM once and both the unit-key sum and the scores are
// formed from the registers.  (The two-pass kernel above re-reads the chunk, and with many
// chunks in flight per XCD that second read mostly misses L2.)  Same arithmetic, same
// fixed reduction order within a workgroup.
constexpr int WR_THREADS = 1024, WR_MAXC = 512;
// (d_k <= 128: two workgroups per CU, so one streams its chunk in while the other reduces)
template <int DK>
__global__ __launch_bounds__(WR_THREADS, DK <= 128 ? 8 : 4) void write_scores_reg_kernel(int64_t T_len, int C,
                                                                      const bf16_t *__restrict__ k,
                                                                      float *__restrict__ d_head) {
  constexpr int LPT = DK / 8, TPS = WR_THREADS / LPT, NS = WR_MAXC / TPS, NW = WR_THREADS / 64;
  __shared__ float s_mu[NW][DK];
  __shared__ float s_mubar[DK];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sub = lane % LPT, tok = tid / LPT;  // token of this lane within a step
  const size_t bh = (size_t)blockIdx.z * gridDim.y + blockIdx.y;
  const int64_t c0 = (int64_t)blockIdx.x * C;
  const int n = (int)((T_len - c0) < C ? (T_len - c0) : C);
  // buffer loads: tokens past the chunk's end read zeros
  const rsrc_t rk = make_rsrc(k + (bh * T_len + c0) * DK, (uint32_t)n * DK * 2);

  u32x4 raw[NS];  // every load issued before any is used
#pragma unroll
  for (int s = 0; s < NS; ++s) raw[s] = bld16(rk, 2u * (uint32_t)((s * TPS + tok) * DK + 8 * sub));
  auto unpack = [](u32x4 w, float (&x)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  };
  // sum of the unit keys (the 1/|chunk| of the mean cancels in the normalisation)
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    float x[8];
    unpack(raw[s], x);
    float ss = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) ss += x[j] * x[j];
    ss = group_sum<LPT>(ss);
    const float inv = ss > 0.0f ? 1.0f / sqrtf(ss) : 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] += x[j] * inv;
  }
#pragma unroll
  for (int off = LPT; off < 64; off <<= 1)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] += __shfl_xor(acc[j], off, 64);
  if (lane < LPT)
#pragma unroll
    for (int j = 0; j < 8; ++j) s_mu[wave][8 * sub + j] = acc[j];
  __syncthreads();
  if (tid < DK) {
    float m = s_mu[0][tid];
#pragma unroll
    for (int w = 1; w < NW; ++w) m += s_mu[w][tid];
    s_mubar[tid] = m;
  }
  __syncthreads();
  if (wave == 0) {  // |mu|, then mubar = mu / |mu| (zero stays zero)
    float ss = 0.0f;
    for (int i = lane; i < DK; i += 64) ss += s_mubar[i] * s_mubar[i];
    ss = group_sum<64>(ss);
    const float inv = ss > 0.0f ? 1.0f / sqrtf(ss) : 0.0f;
    for (int i = lane; i < DK; i += 64) s_mubar[i] *= inv;
  }
  __syncthreads();
  float mb[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) mb[j] = s_mubar[8 * sub + j];
  // keep the packed words (not both passes' unpacked floats) live across the reduction
#pragma unroll
  for (int s = 0; s < NS; ++s) asm volatile("" : "+v"(raw[s]));
  float *dh = d_head + bh * T_len + c0;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    float x[8];
    unpack(raw[s], x);
    float ss = 0.0f, dot = 0.0f;  // the norm again, from the registers
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      ss += x[j] * x[j];
      dot += x[j] * mb[j];
    }
    ss = group_sum<LPT>(ss);
    dot = group_sum<LPT>(dot);
    const int t = s * TPS + tok;
    if (sub == 0 && t < n) dh[t] = 1.0f - (ss > 0.0f ? dot / sqrtf(ss) : 0.0f);
  }
}

// d_mean[b][t] = (1/H) sum_h d_head[b][h][t], heads in order.
__global__ __launch_bounds__(256) void head_mean_kernel(int H, int64_t T_len, const float *__restrict__ d_head,
                                                        float *__restrict__ d_mean) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int b = blockIdx.y;
  if (t >= T_len) return;
  float s = 0.0f;
  for (int h = 0; h < H; ++h) s += d_head[((size_t)b * H + h) * T_len + t];
  d_mean[(size_t)b * T_len + t] = s / (float)H;
}

// Larger value wins; on equal values the smaller index.
__device__ __forceinline__ bool better(float v, long long i, float bv, long long bi) {
  return v > bv || (v == bv && i < bi);
}

// Block-wide argmax of (v, i) over 256 threads (fixed reduction order).
__device__ __forceinline__ void block_argmax(float &v, long long &i, float *sv, long long *si) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const float ov = __shfl_xor(v, off, 64);
    const long long oi = __shfl_xor(i, off, 64);
    if (better(ov, oi, v, i)) {
      v = ov;
      i = oi;
    }
  }
  if ((tid & 63) == 0) {
    sv[tid >> 6] = v;
    si[tid >> 6] = i;
  }
  __syncthreads();
  v = sv[0];
  i = si[0];
  for (int w = 1; w < (int)(blockDim.x >> 6); ++w)
    if (better(sv[w], si[w], v, i)) {
      v = sv[w];
      i = si[w];
    }
}

// One workgroup (256 threads) per (complete write chunk, batch).
__global__ __launch_bounds__(256) void write_windows_kernel(int64_t T_len, int C, int W, int tail,
                                                            const float *__restrict__ d_mean,
                                                            int64_t *__restrict__ best_start,
                                                            float *__restrict__ best_sum) {
  __shared__ float sv[4];
  __shared__ long long si[4];
  const int c = blockIdx.x, b = blockIdx.y, nc = gridDim.x;
  const int64_t hi = (int64_t)(c + 1) * C, lo = (int64_t)c * C - tail > 0 ? (int64_t)c * C - tail : 0;
  const int w = (int)((hi - lo) < W ? (hi - lo) : W);
  const float *d = d_mean + (size_t)b * T_len;
  float bv = -INFINITY;
  long long bi = lo;
  for (int64_t s = lo + threadIdx.x; s + w <= hi; s += 256) {
    float v = 0.0f;
    for (int t = 0; t < w; ++t) v += d[s + t];
    if (better(v, s, bv, bi)) {
      bv = v;
      bi = s;
    }
  }
  block_argmax(bv, bi, sv, si);
  if (threadIdx.x == 0) {
    best_start[(size_t)b * nc + c] = bi;
    if (best_sum) best_sum[(size_t)b * nc + c] = bv;
  }
}

// One wave per (note, batch) and head: blockIdx.x = note, blockIdx.y = batch, 64 x H threads.
template <typename T>
__global__ void note_address_kernel(int H, int64_t T_len, int DK, int N, int DR,
                                    const float *__restrict__ d_head, const T *__restrict__ q,
                                    const int64_t *__restrict__ spans, const int *__restrict__ coords,
                                    int64_t *__restrict__ t_star, T *__restrict__ rho) {
  const int i = blockIdx.x, b = blockIdx.y, h = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t s0 = spans[((size_t)b * N + i) * 2], len = spans[((size_t)b * N + i) * 2 + 1];
  const size_t out = ((size_t)b * N + i) * H + h;
  const bool ok = s0 >= 0 && len >= 1 && s0 + len <= T_len;  // else t* = -1 and rho = 0
  float bv = -INFINITY;
  long long bi = s0;
  if (ok) {
    const float *d = d_head + ((size_t)b * H + h) * T_len;
    for (int64_t t = s0 + lane; t < s0 + len; t += 64)
      if (better(d[t], t, bv, bi)) {
        bv = d[t];
        bi = t;
      }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const float ov = __shfl_xor(bv, off, 64);
      const long long oi = __shfl_xor(bi, off, 64);
      if (better(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
  }
  if (lane == 0) t_star[out] = ok ? bi : -1;
  for (int r = lane; r < DR; r += 64) {
    const int ci = coords[h * DR + r];
    T x = T(0);
    if (ok && ci >= 0 && ci < DK) x = q[(((size_t)b * H + h) * T_len + bi) * DK + ci];
    rho[out * DR + r] = x;
  }
}

// One workgroup (1024 threads) per channel j.  The question vectors are normalised once into
// LDS; each thread takes notes i = tid, tid + 1024, ... two at a time (every LDS read of a
// question vector serves both) and keeps their addresses in registers.
constexpr int VT = 1024;
template <int DR, typename T>
__device__ __forceinline__ float unit_address(const T *r, float (&x)[DR]) {
  float ss = 0.0f;
#pragma unroll
  for (int e = 0; e < DR; ++e) {
    x[e] = io<T>::ld(r, e);
    ss += x[e] * x[e];
  }
  return ss > 0.0f ? 1.0f / sqrtf(ss) : 0.0f;
}
template <int DR, typename T>
__global__ __launch_bounds__(VT) void channel_vote_kernel(int N, int J, int nQ, const T *__restrict__ rho,
                                                          const T *__restrict__ u, float *__restrict__ score,
                                                          int *__restrict__ choice) {
  extern __shared__ float s_u[];  // [nQ][DR], normalised
  __shared__ float sv[VT / 64];
  __shared__ long long si[VT / 64];
  const int j = blockIdx.x, tid = threadIdx.x;
  for (int tau = tid; tau < nQ; tau += VT) {
    float x[DR];
    const float inv = unit_address<DR, T>(u + ((size_t)tau * J + j) * DR, x);
#pragma unroll
    for (int e = 0; e < DR; ++e) s_u[tau * DR + e] = x[e] * inv;
  }
  __syncthreads();
  float bv = -INFINITY;
  long long bi = 0;
  for (int i0 = tid; i0 < N; i0 += 2 * VT) {
    const int i1 = i0 + VT;
    const bool has1 = i1 < N;
    float r0[DR], r1[DR];
    const float n0 = unit_address<DR, T>(rho + ((size_t)i0 * J + j) * DR, r0);
    const float n1 = has1 ? unit_address<DR, T>(rho + ((size_t)i1 * J + j) * DR, r1) : 0.0f;
#pragma unroll
    for (int e = 0; e < DR; ++e) {
      r0[e] *= n0;
      r1[e] = has1 ? r1[e] * n1 : 0.0f;
    }
    float m0 = -INFINITY, m1 = -INFINITY;
    for (int tau = 0; tau < nQ; ++tau) {
      float d0 = 0.0f, d1 = 0.0f;
#pragma unroll
      for (int e = 0; e < DR; ++e) {
        const float x = s_u[tau * DR + e];
        d0 += x * r0[e];
        d1 += x * r1[e];
      }
      m0 = fmaxf(m0, d0);
      m1 = fmaxf(m1, d1);
    }
    if (score) score[(size_t)j * N + i0] = m0;
    if (better(m0, i0, bv, bi)) {
      bv = m0;
      bi = i0;
    }
    if (has1) {
      if (score) score[(size_t)j * N + i1] = m1;
      if (better(m1, i1, bv, bi)) {
        bv = m1;
        bi = i1;
      }
    }
  }
  block_argmax(bv, bi, sv, si);
  if (tid == 0) choice[j] = (int)bi;
}

// One workgroup of 1024 threads: votes, the R best notes by (votes, earlier index), then
// document order by (position, index).
constexpr int MAX_NOTES = 16384;  // votes counted in LDS
__global__ __launch_bounds__(1024) void select_notes_kernel(int N, int J, int R, const int *__restrict__ choice,
                                                            const int64_t *__restrict__ positions,
                                                            int *__restrict__ votes, int *__restrict__ selected) {
  __shared__ int s_sel[64];
  __shared__ int s_v[16];
  __shared__ int s_i[16];
  __shared__ int s_votes[MAX_NOTES];
  const int tid = threadIdx.x;
  for (int i = tid; i < N; i += 1024) s_votes[i] = 0;
  __syncthreads();
  for (int j = tid; j < J; j += 1024) atomicAdd(&s_votes[choice[j]], 1);  // integer counts: order-free
  __syncthreads();
  for (int i = tid; i < N; i += 1024) votes[i] = s_votes[i];
  int nsel = 0;
  for (int r = 0; r < R; ++r) {
    int bv = 0, bi = -1;  // only notes with at least one vote
    for (int i = tid; i < N; i += 1024) {
      int taken = 0;
      for (int s = 0; s < nsel; ++s) taken |= s_sel[s] == i;
      const int v = s_votes[i];
      if (!taken && v > 0 && (v > bv || (v == bv && (bi < 0 || i < bi)))) {
        bv = v;
        bi = i;
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const int ov = __shfl_xor(bv, off, 64), oi = __shfl_xor(bi, off, 64);
      if (oi >= 0 && (bi < 0 || ov > bv || (ov == bv && oi < bi))) {
        bv = ov;
        bi = oi;
      }
    }
    if ((tid & 63) == 0) {
      s_v[tid >> 6] = bv;
      s_i[tid >> 6] = bi;
    }
    __syncthreads();
    if (tid == 0) {
      int v = s_v[0], ix = s_i[0];
      for (int w = 1; w < 16; ++w)
        if (s_i[w] >= 0 && (ix < 0 || s_v[w] > v || (s_v[w] == v && s_i[w] < ix))) {
          v = s_v[w];
          ix = s_i[w];
        }
      s_sel[r] = ix;
    }
    __syncthreads();
    if (s_sel[r] < 0) break;
    nsel = r + 1;
    __syncthreads();
  }
  if (tid == 0) {
    for (int a = 1; a < nsel; ++a)
      for (int c = a; c > 0; --c) {
        const int x = s_sel[c - 1], y = s_sel[c];
        if (positions[y] < positions[x] || (positions[y] == positions[x] && y < x)) {
          s_sel[c - 1] = y;
          s_sel[c] = x;
        }
      }
    for (int r = 0; r < R; ++r) selected[r] = r < nsel ? s_sel[r] : -1;
  }
}

template <int DK, typename T>
static void go_scores(int B, int H, int64_t T_len, int C, const void *k, float *d_head, hipStream_t s) {
  const dim3 grid((unsigned)((T_len + C - 1) / C), H, B);
  if (sizeof(T) == 2 && C <= WR_MAXC)
    hipLaunchKernelGGL((write_scores_reg_kernel<DK>), grid, dim3(WR_THREADS), 0, s, T_len, C, (const bf16_t *)k, d_head);
  else
    hipLaunchKernelGGL((write_scores_kernel<DK, T>), grid, dim3(WS_THREADS), 0, s, T_len, C, (const T *)k, d_head);
}

}  // namespace nb

hipError_t launch_write_scores(int dtype, int B, int H, int64_t T, int d_k, int chunk, const void *k,
                               float *d_head, float *d_mean, hipStream_t s) {
  using namespace nb;
  if (dtype == T_BF16) {
    if (d_k == 64) go_scores<64, bf16_t>(B, H, T, chunk, k, d_head, s);
    else if (d_k == 128) go_scores<128, bf16_t>(B, H, T, chunk, k, d_head, s);
    else go_scores<256, bf16_t>(B, H, T, chunk, k, d_head, s);
  } else {
    if (d_k == 64) go_scores<64, float>(B, H, T, chunk, k, d_head, s);
    else if (d_k == 128) go_scores<128, float>(B, H, T, chunk, k, d_head, s);
    else go_scores<256, float>(B, H, T, chunk, k, d_head, s);
  }
  if (d_mean)
    hipLaunchKernelGGL(head_mean_kernel, dim3((unsigned)((T + 255) / 256), B), dim3(256), 0, s, H, T, d_head, d_mean);
  return hipGetLastError();
}

hipError_t launch_write_windows(int B, int64_t T, int chunk, int window, int tail, const float *d_mean,
                                int64_t *best_start, float *best_sum, hipStream_t s) {
  const int64_t nc = T / chunk;
  if (nc > 0)
    hipLaunchKernelGGL(nb::write_windows_kernel, dim3((unsigned)nc, B), dim3(256), 0, s, T, chunk, window, tail,
                       d_mean, best_start, best_sum);
  return hipGetLastError();
}

hipError_t launch_note_addresses(int dtype, int B, int H, int64_t T, int d_k, int N, int d_rho,
                                 const float *d_head, const void *q, const int64_t *spans, const int *coords,
                                 int64_t *t_star, void *rho, hipStream_t s) {
  if (N > 0) {
    if (dtype == T_BF16)
      hipLaunchKernelGGL(nb::note_address_kernel<bf16_t>, dim3(N, B), dim3(64 * H), 0, s, H, T, d_k, N, d_rho,
                         d_head, (const bf16_t *)q, spans, coords, t_star, (bf16_t *)rho);
    else
      hipLaunchKernelGGL(nb::note_address_kernel<float>, dim3(N, B), dim3(64 * H), 0, s, H, T, d_k, N, d_rho,
                         d_head, (const float *)q, spans, coords, t_star, (float *)rho);
  }
  return hipGetLastError();
}

hipError_t launch_address_votes(int dtype, int N, int J, int nQ, int d_rho, const void *rho, const void *u,
                                int R, const int64_t *positions, float *score, int *choice, int *votes,
                                int *selected, hipStream_t s) {
  const size_t lds = (size_t)nQ * d_rho * sizeof(float);
#define LA_VOTE(DR)                                                                                  \
  do {                                                                                               \
    if (dtype == T_BF16)                                                                             \
      hipLaunchKernelGGL((nb::channel_vote_kernel<DR, bf16_t>), dim3(J), dim3(nb::VT), lds, s, N, J, nQ, \
                         (const bf16_t *)rho, (const bf16_t *)u, score, choice);                     \
    else                                                                                             \
      hipLaunchKernelGGL((nb::channel_vote_kernel<DR, float>), dim3(J), dim3(nb::VT), lds, s, N, J, nQ,  \
                         (const float *)rho, (const float *)u, score, choice);                       \
  } while (0)
  switch (d_rho) {
    case 8: LA_VOTE(8); break;
    case 16: LA_VOTE(16); break;
    default: LA_VOTE(32); break;
  }
#undef LA_VOTE
  hipLaunchKernelGGL(nb::select_notes_kernel, dim3(1), dim3(1024), 0, s, N, J, R, choice, positions, votes,
                     selected);
  return hipGetLastError();
}

}  // namespace la
