// chunk.hip -- chunkwise bf16 prefill for ADDITIVE / GATED / GATED_DELTA (d_k = d_v = 128).
//
// Method.  Eq. (1) of "History Replays Itself" (Sec. 2) is evaluated on chunks of C = 64
// tokens with the state carried across chunk boundaries, as the NoteBank paper's
// backbone does (Sec. 3.2: chunks of C tokens, state carried across boundaries); the
// block algebra below is the plainest reading of that, derived from Eq. (1) itself
// (the BASED notes' Sec. 2.5 block form U_b = (M_b . Phi_Q Phi_K^T) V_b + Phi_Q S_{<b} is
// its additive case).  Inside a chunk with entering state S (d_v x d_k), g_t = sum_{i<=t}
// log alpha_i, gamma_t = e^{g_t}, P_tj = e^{g_t - g_j} for j <= t:
//
//   gated delta  L_tj = beta_t e^{g_t-g_j} k_t.k_j (j < t),  T = (I + L)^{-1}
//                W = T diag(beta gamma) K,  U~ = T diag(beta) V,  U = U~ - W S^T
//   gated/add.   U = diag(beta) V
//   O  = diag(gamma) Q S^T + (P . Q K^T) U
//   S' = gamma_C S + U^T diag(e^{g_C - g}) K  =  S M_c + B_c
//
// T is the UT/WY transform of the chunk; it is computed in fp32 in LDS by blocked
// forward substitution (16 x 16 diagonal blocks, off-diagonal blocks on fp32 MFMA).
// Every product with a 64- or 128-wide inner dimension runs on bf16 MFMA
// (v_mfma_f32_16x16x32_bf16) with fp32 accumulation; the state stays fp32.
//
// Sequence parallelism.  One workgroup owns the whole 128 x 128 state of one (b, h),
// which fits its registers, so a workgroup streams chunks with no inter-workgroup
// traffic.  A 1M-token sequence is split into segments so that B*H*segments fills the
// chip, in three passes:
//   pass 1 (MODE_MAP)  every segment from a zero start: its end state B_seg and, for the
//                      delta rule, its d_k x d_k transition M_seg (the same chunk
//                      recurrence run on the identity), or the scalar log decay
//   pass 2 (scan)      S_{i+1} = S_i M_i + B_i sequentially over segments, row-parallel
//   pass 3 (MODE_OUT)  every segment replayed from its start state, writing o
// With one segment (enough heads to fill the chip) only pass 3 runs.
#include "la_device.h"
#include "la_launch.h"

namespace la {
namespace gdn {

constexpr int C = 64;     // tokens per chunk
constexpr int DK = 128;   // key width
constexpr int DV = 128;   // value width
constexpr int NW = 8;     // waves per workgroup
constexpr int NTHR = NW * 64;

constexpr int LDK = DK + 8;  // row-major bf16 tiles [C][DK]: K, Q, W, staging
constexpr int LDT = C + 8;   // transposed bf16 tiles [D][C]: K^T, V^T
constexpr int LDA = C + 8;   // bf16 [C][C]: decay-masked Q K^T
constexpr int LDL = C + 4;   // fp32 [C][C]: L, T

constexpr int SZ_ROW = C * LDK * 2;
constexpr int SZ_TR = DK * LDT * 2;
constexpr int SZ_L = C * LDL * 4;
constexpr int SZ_A = C * LDA * 2;
constexpr int OFF_K = 0;
constexpr int OFF_Q = OFF_K + SZ_ROW;
constexpr int OFF_KT = OFF_Q + SZ_ROW;
constexpr int OFF_VT = OFF_KT + SZ_TR;
constexpr int OFF_LW = OFF_VT + SZ_TR;  // L (fp32) then -W (bf16); O staging without delta
constexpr int OFF_T = OFF_LW + SZ_L;    // V staging then T (fp32)
constexpr int OFF_A = OFF_T + SZ_L;
constexpr int OFF_VEC = OFF_A + SZ_A;   // g, beta, gamma, decay-to-end, beta*gamma
constexpr int SMEM = OFF_VEC + 5 * C * 4;
static_assert(SZ_ROW <= SZ_L && SZ_ROW <= SZ_TR, "staging buffers fit their regions");
static_assert(DK == DV, "square state");

enum { MODE_MAP = 0, MODE_OUT = 1 };

struct Args {
  const bf16_t *q, *k, *v, *alpha, *beta;
  const float *S0;   // start state when there is a single segment (may be NULL)
  bf16_t *o;
  float *S_T;        // end state written by pass 3 when there is a single segment
  float *maps;       // [BH][nseg][maprows][DK] per-segment maps (rows: B_seg, then M_seg)
  float *gsum;       // [BH][nseg] per-segment log decay (no delta rule)
  float *starts;     // [BH][nseg][DV][DK] segment start states
  int64_t T;
  int H, nseg, seg_chunks, variant, has_beta;
};

// Reads the MFMA operand for rows `row`, 32-wide k-step starting at col0 = 32 s: the
// lane group g supplies columns col0+4g..+3 and col0+16+4g..+3, matching the column
// order of two stacked 16x16 accumulator tiles (rows 4g..4g+3 of each).
__device__ __forceinline__ bf16x8 frag_pair(const bf16_t *base, int ld, int row, int col0, int g) {
  const uint2 lo = *reinterpret_cast<const uint2 *>(base + row * ld + col0 + 4 * g);
  const uint2 hi = *reinterpret_cast<const uint2 *>(base + row * ld + col0 + 16 + 4 * g);
  u16x8 u;
  u[0] = (uint16_t)lo.x; u[1] = (uint16_t)(lo.x >> 16); u[2] = (uint16_t)lo.y; u[3] = (uint16_t)(lo.y >> 16);
  u[4] = (uint16_t)hi.x; u[5] = (uint16_t)(hi.x >> 16); u[6] = (uint16_t)hi.y; u[7] = (uint16_t)(hi.y >> 16);
  return as_bf16x8(u);
}

__device__ __forceinline__ bf16x8 pack_pair(f32x4 a, f32x4 b) {
  return pack8(a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]);
}

__device__ __forceinline__ f32x4 ld4(const float *p) { return *reinterpret_cast<const f32x4 *>(p); }

__device__ __forceinline__ void tri_index(int idx, int &ti, int &tj) {
  ti = idx >= 6 ? 3 : (idx >= 3 ? 2 : (idx >= 1 ? 1 : 0));
  tj = idx - ti * (ti + 1) / 2;
}

template <int MODE, bool DELTA>
__global__ __launch_bounds__(NTHR) void chunk_kernel(const Args a) {
  // column tiles (16 state rows each) owned by one wave
  constexpr int NCT = (MODE == MODE_MAP && DELTA) ? 2 : 1;
  constexpr int MAPROWS = DELTA ? 2 * DV : DV;
  __shared__ __attribute__((aligned(16))) unsigned char smem[SMEM];
  bf16_t *sK = reinterpret_cast<bf16_t *>(smem + OFF_K);
  bf16_t *sQ = reinterpret_cast<bf16_t *>(smem + OFF_Q);
  bf16_t *sKt = reinterpret_cast<bf16_t *>(smem + OFF_KT);
  bf16_t *sVt = reinterpret_cast<bf16_t *>(smem + OFF_VT);
  float *sL = reinterpret_cast<float *>(smem + OFF_LW);
  bf16_t *sW = reinterpret_cast<bf16_t *>(smem + OFF_LW);
  float *sT = reinterpret_cast<float *>(smem + OFF_T);
  bf16_t *sVs = reinterpret_cast<bf16_t *>(smem + OFF_T);
  bf16_t *sA = reinterpret_cast<bf16_t *>(smem + OFF_A);
  bf16_t *sO = reinterpret_cast<bf16_t *>(smem + (DELTA ? OFF_VT : OFF_LW));
  float *sG = reinterpret_cast<float *>(smem + OFF_VEC);
  float *sBeta = sG + C;
  float *sGam = sG + 2 * C;
  float *sDec = sG + 3 * C;
  float *sBG = sG + 4 * C;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l16 = lane & 15, g = lane >> 4;
  const int seg = blockIdx.x;
  const size_t bh = (size_t)blockIdx.z * a.H + blockIdx.y;
  const int64_t T = a.T;
  const int row0 = wave * 16 * NCT;  // first state row owned by this wave
  const bool m_rows = (MODE == MODE_MAP) && DELTA && wave >= NW / 2;

  // ---- state: lane holds S^T[d = 16 m + 4 g + e][row0 + 16 c + l16] in st[m][c][e]
  f32x4 st[DK / 16][NCT];
  {
    const float *src = nullptr;
    if (MODE == MODE_OUT) src = a.nseg > 1 ? a.starts + (bh * a.nseg + seg) * DV * DK : (a.S0 ? a.S0 + bh * DV * DK : nullptr);
#pragma unroll
    for (int m = 0; m < DK / 16; ++m)
#pragma unroll
      for (int c = 0; c < NCT; ++c) {
        const int r = row0 + 16 * c + l16;
        if (src) {
          st[m][c] = ld4(src + (size_t)r * DK + 16 * m + 4 * g);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)  // identity for the transition rows, zero otherwise
            st[m][c][e] = (m_rows && (r - DV) == 16 * m + 4 * g + e) ? 1.0f : 0.0f;
        }
      }
  }

  float gseg = 0.0f;  // log decay over the segment (scalar-gated map)
  int64_t prev_t0 = -1;
  int prev_n = 0;
  const int64_t first = (int64_t)seg * a.seg_chunks * C;
  for (int ci = 0; ci < a.seg_chunks; ++ci) {
    const int64_t t0 = first + (int64_t)ci * C;
    if (t0 >= T) break;
    const int n = (int)((T - t0) < C ? (T - t0) : C);
    const size_t rb = bh * (size_t)T + t0;

    // ---- phase A: write out the previous chunk's O, load this chunk, gate prefix sums
    if (MODE == MODE_OUT && prev_t0 >= 0) {
      for (int id = tid; id < prev_n * (DV / 8); id += NTHR) {
        const int r = id / (DV / 8), cv = id % (DV / 8);
        *reinterpret_cast<uint4 *>(a.o + (bh * (size_t)T + prev_t0 + r) * DV + cv * 8) =
            *reinterpret_cast<const uint4 *>(sO + r * LDK + cv * 8);
      }
    }
    for (int id = tid; id < C * (DK / 8); id += NTHR) {
      const int r = id / (DK / 8), cv = id % (DK / 8);
      uint4 kv = make_uint4(0, 0, 0, 0), qv = kv, vv = kv;
      if (r < n) {
        kv = *reinterpret_cast<const uint4 *>(a.k + (rb + r) * DK + cv * 8);
        vv = *reinterpret_cast<const uint4 *>(a.v + (rb + r) * DV + cv * 8);
        if (MODE == MODE_OUT) qv = *reinterpret_cast<const uint4 *>(a.q + (rb + r) * DK + cv * 8);
      }
      *reinterpret_cast<uint4 *>(sK + r * LDK + cv * 8) = kv;
      *reinterpret_cast<uint4 *>(sVs + r * LDK + cv * 8) = vv;
      if (MODE == MODE_OUT) *reinterpret_cast<uint4 *>(sQ + r * LDK + cv * 8) = qv;
    }
    if (wave == 0) {
      float al = 1.0f, be = 0.0f;
      if (lane < n) {
        if (a.variant != V_ADDITIVE) al = bf16_to_f32(a.alpha[rb + lane]);
        be = (a.variant == V_GATED_DELTA || (a.variant == V_GATED && a.has_beta)) ? bf16_to_f32(a.beta[rb + lane]) : 1.0f;
      }
      float x = (a.variant == V_ADDITIVE) ? 0.0f : logf(al);
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
      }
      const float gC = __shfl(x, 63, 64);
      const float gam = expf(x);
      sG[lane] = x;
      sBeta[lane] = be;
      sGam[lane] = gam;
      sDec[lane] = expf(gC - x);
      sBG[lane] = be * gam;
    }
    __syncthreads();

    // ---- phase B: transposed copies of K and V; Gram tiles K K^T (-> L) and Q K^T (-> A)
    for (int id = tid; id < DK * (C / 8); id += NTHR) {
      const int d = id / (C / 8), tg = id % (C / 8);
      u16x8 kk, vv;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        kk[e] = sK[(8 * tg + e) * LDK + d];
        vv[e] = sVs[(8 * tg + e) * LDK + d];
      }
      *reinterpret_cast<u16x8 *>(sKt + d * LDT + 8 * tg) = kk;
      *reinterpret_cast<u16x8 *>(sVt + d * LDT + 8 * tg) = vv;
    }
    {
      constexpr int NJ = (DELTA ? 10 : 0) + (MODE == MODE_OUT ? 10 : 0);
      for (int job = wave; job < NJ; job += NW) {
        const bool kk = DELTA && job < 10;
        int ti, tj;
        tri_index(kk ? job : job - (DELTA ? 10 : 0), ti, tj);
        const bf16_t *X = kk ? sK : sQ;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < DK / 32; ++s) {
          const bf16x8 fa = *reinterpret_cast<const bf16x8 *>(X + (16 * ti + l16) * LDK + 32 * s + 8 * g);
          const bf16x8 fb = *reinterpret_cast<const bf16x8 *>(sK + (16 * tj + l16) * LDK + 32 * s + 8 * g);
          acc = mfma_bf16(fa, fb, acc);
        }
        const int j = 16 * tj + l16;
        const float gj = sG[j];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = 16 * ti + 4 * g + e;
          if (kk) sL[t * LDL + j] = (t > j) ? sBeta[t] * expf(sG[t] - gj) * acc[e] : 0.0f;
          else sA[t * LDA + j] = f32_to_bf16((t >= j) ? expf(sG[t] - gj) * acc[e] : 0.0f);
        }
      }
      if (MODE == MODE_OUT) {  // the two above-diagonal tiles read by the A U products
        for (int id = tid; id < 512; id += NTHR) {
          const int tile = id >> 8, e = id & 255;
          sA[(32 * tile + (e >> 4)) * LDA + 32 * tile + 16 + (e & 15)] = 0;
        }
      }
    }
    __syncthreads();

    f32x4 Ut[4][NCT];  // U~ tiles of this wave's rows (delta rule)
    if (DELTA) {
      // ---- phase C: inverses of the four 16 x 16 diagonal blocks of (I + L)
      if (wave == 0) {
        const int bi = lane >> 4, c = lane & 15;
        float col[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float acc = 0.0f;
#pragma unroll
          for (int kq = 0; kq < r; ++kq) acc += sL[(16 * bi + r) * LDL + 16 * bi + kq] * col[kq];
          col[r] = (r == c) ? 1.0f : (r > c ? -acc : 0.0f);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) sT[(16 * bi + r) * LDL + 16 * bi + c] = col[r];
      } else {
        for (int id = tid - 64; id < 512; id += NTHR - 64) {  // blocks (0,1), (2,3) of T are zero
          const int blk = id >> 8, e = id & 255;
          sT[(32 * blk + (e >> 4)) * LDL + 32 * blk + 16 + (e & 15)] = 0.0f;
        }
      }
      __syncthreads();
      // ---- phase D: off-diagonal blocks T_ij = -T_ii sum_{k=j}^{i-1} L_ik T_kj, by
      // sub-diagonal level, on fp32 MFMA (16x16x4)
#pragma unroll
      for (int level = 1; level <= 3; ++level) {
        if (wave < 4 - level) {
          const int j = wave, i = wave + level;
          f32x4 x = {0.f, 0.f, 0.f, 0.f};
          for (int kb = j; kb < i; ++kb) {
#pragma unroll
            for (int s = 0; s < 4; ++s) {
              const float fa = sL[(16 * i + l16) * LDL + 16 * kb + 4 * s + g];
              const float fb = sT[(16 * kb + 4 * s + g) * LDL + 16 * j + l16];
              x = __builtin_amdgcn_mfma_f32_16x16x4f32(fa, fb, x, 0, 0, 0);
            }
          }
          f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < 4; ++s) {  // inner index 4 g + s: x's own rows serve as B
            const float fa = sT[(16 * i + l16) * LDL + 16 * i + 4 * g + s];
            y = __builtin_amdgcn_mfma_f32_16x16x4f32(fa, x[s], y, 0, 0, 0);
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) sT[(16 * i + 4 * g + e) * LDL + 16 * j + l16] = -y[e];
        }
        __syncthreads();
      }
      // ---- phase E: W = T diag(beta gamma) K (stored negated, bf16) and U~ = T diag(beta) V
      // (kept in registers by the wave that owns those state rows)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        f32x4 accw[NCT], accu[NCT];
#pragma unroll
        for (int c = 0; c < NCT; ++c) {
          accw[c] = {0.f, 0.f, 0.f, 0.f};
          accu[c] = {0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          if (s == 1 && mt < 2) continue;  // T is lower triangular
          const f32x4 t0 = ld4(sT + (16 * mt + l16) * LDL + 32 * s + 4 * g);
          const f32x4 t1 = ld4(sT + (16 * mt + l16) * LDL + 32 * s + 16 + 4 * g);
          if (MODE == MODE_OUT || wave >= NW / 2) {
            const f32x4 b0 = ld4(sBG + 32 * s + 4 * g), b1 = ld4(sBG + 32 * s + 16 + 4 * g);
            const bf16x8 fa = pack_pair(t0 * b0, t1 * b1);
#pragma unroll
            for (int c = 0; c < NCT; ++c) {
              const int nt = MODE == MODE_OUT ? wave : 2 * (wave - NW / 2) + c;
              accw[c] = mfma_bf16(fa, frag_pair(sKt, LDT, 16 * nt + l16, 32 * s, g), accw[c]);
            }
          }
          if (MODE == MODE_OUT || wave < NW / 2) {
            const f32x4 b0 = ld4(sBeta + 32 * s + 4 * g), b1 = ld4(sBeta + 32 * s + 16 + 4 * g);
            const bf16x8 fa = pack_pair(t0 * b0, t1 * b1);
#pragma unroll
            for (int c = 0; c < NCT; ++c) {
              const int nt = MODE == MODE_OUT ? wave : 2 * wave + c;
              accu[c] = mfma_bf16(fa, frag_pair(sVt, LDT, 16 * nt + l16, 32 * s, g), accu[c]);
            }
          }
        }
        if (MODE == MODE_OUT || wave >= NW / 2) {
#pragma unroll
          for (int c = 0; c < NCT; ++c) {
            const int nt = MODE == MODE_OUT ? wave : 2 * (wave - NW / 2) + c;
#pragma unroll
            for (int e = 0; e < 4; ++e) sW[(16 * mt + 4 * g + e) * LDK + 16 * nt + l16] = f32_to_bf16(-accw[c][e]);
          }
        }
#pragma unroll
        for (int c = 0; c < NCT; ++c) Ut[mt][c] = accu[c];
      }
      __syncthreads();
    }

    // ---- phase F: the state-dependent part, per wave on its own state rows
    bf16x8 ufr[NCT][2], dufr[NCT][2];  // U and diag(decay) U as B operands (k = tokens)
    bf16x8 sfr[NCT][DK / 32];          // S^T as B operand (k = d_k)
#pragma unroll
    for (int c = 0; c < NCT; ++c)
#pragma unroll
      for (int s = 0; s < DK / 32; ++s) sfr[c][s] = pack_pair(st[2 * s][c], st[2 * s + 1][c]);
    if (DELTA) {
#pragma unroll
      for (int c = 0; c < NCT; ++c) {
        f32x4 U[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          f32x4 acc = m_rows ? f32x4{0.f, 0.f, 0.f, 0.f} : Ut[mt][c];
#pragma unroll
          for (int s = 0; s < DK / 32; ++s) acc = mfma_bf16(frag_pair(sW, LDK, 16 * mt + l16, 32 * s, g), sfr[c][s], acc);
          U[mt] = acc;
        }
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const f32x4 d0 = ld4(sDec + 32 * s2 + 4 * g), d1 = ld4(sDec + 32 * s2 + 16 + 4 * g);
          ufr[c][s2] = pack_pair(U[2 * s2], U[2 * s2 + 1]);
          dufr[c][s2] = pack_pair(U[2 * s2] * d0, U[2 * s2 + 1] * d1);
        }
      }
    } else {
#pragma unroll
      for (int c = 0; c < NCT; ++c) {
        const int dvr = row0 + 16 * c + l16;
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const bf16x8 vf = frag_pair(sVt, LDT, dvr, 32 * s2, g);
          const f32x4 b0 = ld4(sBeta + 32 * s2 + 4 * g), b1 = ld4(sBeta + 32 * s2 + 16 + 4 * g);
          const f32x4 d0 = ld4(sDec + 32 * s2 + 4 * g), d1 = ld4(sDec + 32 * s2 + 16 + 4 * g);
          f32x4 v0, v1;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v0[e] = (float)vf[e] * b0[e];
            v1[e] = (float)vf[4 + e] * b1[e];
          }
          ufr[c][s2] = pack_pair(v0, v1);
          dufr[c][s2] = pack_pair(v0 * d0, v1 * d1);
        }
      }
    }
    if (MODE == MODE_OUT) {  // O = diag(gamma) Q S^T + A U  -> bf16 staging for coalesced stores
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < DK / 32; ++s) acc = mfma_bf16(frag_pair(sQ, LDK, 16 * mt + l16, 32 * s, g), sfr[0][s], acc);
        acc = acc * ld4(sGam + 16 * mt + 4 * g);
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          if (s2 == 1 && mt < 2) continue;  // A is causal
          acc = mfma_bf16(frag_pair(sA, LDA, 16 * mt + l16, 32 * s2, g), ufr[0][s2], acc);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) sO[(16 * mt + 4 * g + e) * LDK + row0 + l16] = f32_to_bf16(acc[e]);
      }
    }
    {  // S^T <- gamma_C S^T + K^T diag(decay) U
      const float gC = sGam[C - 1];
      gseg += sG[C - 1];
#pragma unroll
      for (int m = 0; m < DK / 16; ++m)
#pragma unroll
        for (int c = 0; c < NCT; ++c) {
          f32x4 acc = st[m][c] * gC;
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) acc = mfma_bf16(frag_pair(sKt, LDT, 16 * m + l16, 32 * s2, g), dufr[c][s2], acc);
          st[m][c] = acc;
        }
    }
    __syncthreads();
    prev_t0 = t0;
    prev_n = n;
  }

  if (MODE == MODE_OUT) {
    if (prev_t0 >= 0) {
      for (int id = tid; id < prev_n * (DV / 8); id += NTHR) {
        const int r = id / (DV / 8), cv = id % (DV / 8);
        *reinterpret_cast<uint4 *>(a.o + (bh * (size_t)T + prev_t0 + r) * DV + cv * 8) =
            *reinterpret_cast<const uint4 *>(sO + r * LDK + cv * 8);
      }
    }
    if (a.nseg == 1 && a.S_T) {
#pragma unroll
      for (int m = 0; m < DK / 16; ++m) {
        const int r = row0 + l16;
        *reinterpret_cast<f32x4 *>(a.S_T + (bh * DV + r) * DK + 16 * m + 4 * g) = st[m][0];
      }
    }
  } else {
    float *dst = a.maps + (bh * a.nseg + seg) * (size_t)MAPROWS * DK;
#pragma unroll
    for (int m = 0; m < DK / 16; ++m)
#pragma unroll
      for (int c = 0; c < NCT; ++c) {
        const int r = row0 + 16 * c + l16;
        *reinterpret_cast<f32x4 *>(dst + (size_t)r * DK + 16 * m + 4 * g) = st[m][c];
      }
    if (!DELTA && tid == 0) a.gsum[bh * a.nseg + seg] = gseg;
  }
}

// Pass 2: S_{i+1} = S_i M_i + B_i (delta rule) or e^{gsum_i} S_i + B_i, row-parallel:
// each workgroup carries 4 rows of one head's state through all segments.
template <bool DELTA>
__global__ __launch_bounds__(256) void scan_kernel(const Args a) {
  constexpr int MAPROWS = DELTA ? 2 * DV : DV;
  __shared__ float sS[4][DK];
  const int tid = threadIdx.x, rr = tid >> 6, cp = 2 * (tid & 63);
  const int row = blockIdx.x * 4 + rr;
  const size_t bh = (size_t)blockIdx.z * a.H + blockIdx.y;
  float2 cur = make_float2(0.f, 0.f);
  if (a.S0) cur = *reinterpret_cast<const float2 *>(a.S0 + (bh * DV + row) * DK + cp);
  sS[rr][cp] = cur.x;
  sS[rr][cp + 1] = cur.y;
  __syncthreads();
  for (int i = 0; i < a.nseg; ++i) {
    *reinterpret_cast<float2 *>(a.starts + ((bh * a.nseg + i) * DV + row) * DK + cp) = cur;
    const float *Mb = a.maps + (bh * a.nseg + i) * (size_t)MAPROWS * DK;
    float2 acc = *reinterpret_cast<const float2 *>(Mb + (size_t)row * DK + cp);
    if (DELTA) {
      float2 acc2 = make_float2(0.f, 0.f);
#pragma unroll 8
      for (int kq = 0; kq < DK; kq += 2) {
        const float2 m0 = *reinterpret_cast<const float2 *>(Mb + (size_t)(DV + kq) * DK + cp);
        const float2 m1 = *reinterpret_cast<const float2 *>(Mb + (size_t)(DV + kq + 1) * DK + cp);
        const float s0 = sS[rr][kq], s1 = sS[rr][kq + 1];
        acc.x += s0 * m0.x;
        acc.y += s0 * m0.y;
        acc2.x += s1 * m1.x;
        acc2.y += s1 * m1.y;
      }
      acc.x += acc2.x;
      acc.y += acc2.y;
    } else {
      const float dec = expf(a.gsum[bh * a.nseg + i]);
      acc.x += dec * cur.x;
      acc.y += dec * cur.y;
    }
    __syncthreads();
    sS[rr][cp] = acc.x;
    sS[rr][cp + 1] = acc.y;
    cur = acc;
    __syncthreads();
  }
  if (a.S_T) *reinterpret_cast<float2 *>(a.S_T + (bh * DV + row) * DK + cp) = cur;
}

struct Plan {
  int nseg, seg_chunks;
};

// Segments per (b, h): enough workgroups to give every CU about four, but only when the
// heads alone cannot fill the chip (a split costs one extra pass over the keys/values).
Plan make_plan(int B, int H, int64_t T) {
  const int64_t nch = (T + C - 1) / C;
  const int64_t bhn = (int64_t)B * H;
  int64_t nseg = 1;
  if (bhn < 128) {
    nseg = (1024 + bhn - 1) / bhn;
    if (nseg > nch) nseg = nch;
    if (nseg < 1) nseg = 1;
  }
  const int64_t sc = (nch + nseg - 1) / nseg;
  nseg = (nch + sc - 1) / sc;
  return Plan{(int)nseg, (int)sc};
}

size_t ws_layout(bool delta, int B, int H, int64_t T, size_t *off_maps, size_t *off_gsum,
                 size_t *off_starts) {
  const Plan p = make_plan(B, H, T);
  if (p.nseg <= 1) return 0;
  const size_t bhs = (size_t)B * H * p.nseg;
  const size_t maprows = delta ? 2 * DV : DV;
  size_t off = 0;
  *off_maps = off;
  off += bhs * maprows * DK * 4;
  *off_gsum = off;
  off += ((bhs * 4 + 255) / 256) * 256;
  *off_starts = off;
  off += bhs * DV * DK * 4;
  return off;
}

}  // namespace gdn

size_t chunk_workspace_bytes(int variant, int B, int H, int64_t T, int d_k, int d_v) {
  if (d_k != gdn::DK || d_v != gdn::DV) return 0;
  size_t a, b, c;
  return gdn::ws_layout(variant == V_GATED_DELTA, B, H, T, &a, &b, &c);
}

hipError_t launch_chunk_prefill(int variant, int B, int H, int64_t T, int d_k, int d_v,
                                const void *q, const void *k, const void *v, const void *alpha,
                                const void *beta, const float *S0, void *o, float *S_T,
                                void *workspace, hipStream_t s) {
  using namespace gdn;
  if (d_k != DK || d_v != DV)  // other widths: the token-recurrent kernel (fp32 arithmetic)
    return launch_recurrent_rows(variant, T_BF16, B, H, T, d_k, d_v, q, k, v, alpha, beta, S0, o, S_T, s);
  const bool delta = variant == V_GATED_DELTA;
  const Plan p = make_plan(B, H, T);
  size_t om = 0, og = 0, os = 0;
  ws_layout(delta, B, H, T, &om, &og, &os);
  Args a;
  a.q = (const bf16_t *)q;
  a.k = (const bf16_t *)k;
  a.v = (const bf16_t *)v;
  a.alpha = (const bf16_t *)alpha;
  a.beta = (const bf16_t *)beta;
  a.S0 = S0;
  a.o = (bf16_t *)o;
  a.S_T = S_T;
  a.maps = p.nseg > 1 ? (float *)((char *)workspace + om) : nullptr;
  a.gsum = p.nseg > 1 ? (float *)((char *)workspace + og) : nullptr;
  a.starts = p.nseg > 1 ? (float *)((char *)workspace + os) : nullptr;
  a.T = T;
  a.H = H;
  a.nseg = p.nseg;
  a.seg_chunks = p.seg_chunks;
  a.variant = variant;
  a.has_beta = beta != nullptr;
  const dim3 grid(p.nseg, H, B);
  if (p.nseg > 1) {
    if (delta) hipLaunchKernelGGL((chunk_kernel<MODE_MAP, true>), grid, dim3(NTHR), 0, s, a);
    else hipLaunchKernelGGL((chunk_kernel<MODE_MAP, false>), grid, dim3(NTHR), 0, s, a);
    if (delta) hipLaunchKernelGGL((scan_kernel<true>), dim3(DV / 4, H, B), dim3(256), 0, s, a);
    else hipLaunchKernelGGL((scan_kernel<false>), dim3(DV / 4, H, B), dim3(256), 0, s, a);
  }
  if (delta) hipLaunchKernelGGL((chunk_kernel<MODE_OUT, true>), grid, dim3(NTHR), 0, s, a);
  else hipLaunchKernelGGL((chunk_kernel<MODE_OUT, false>), grid, dim3(NTHR), 0, s, a);
  return hipGetLastError();
}

}  // namespace la
