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
// gfx950 layout choices.  All chunk tiles live in LDS row-major ([token][d]); operands
// that contract over tokens (K^T, V^T) are read straight from those tiles with the
// CDNA4 transpose read ds_read_b64_tr_b16, so no transposed copies are built.  L (fp32)
// is kept transposed in the strict upper triangle of the same buffer whose lower
// triangle receives T.  A workgroup (4 waves) uses at most ~80 KB of LDS, so two
// workgroups share a CU and overlap their latency-bound phases (the triangular solve,
// barriers) with each other's MFMA phases.  The next chunk's inputs are prefetched into
// registers while the current chunk is processed.
//
// Sequence parallelism.  One workgroup owns the whole 128 x 128 state of one (b, h),
// split over its 4 waves (32 state rows each, in registers), and streams chunks with
// no inter-workgroup traffic.  A long sequence is split into segments so that
// B*H*segments fills the chip, in three passes:
//   pass 1 (MODE_MAP)  every segment from a zero start: its end state B_seg, and for the
//                      delta rule its d_k x d_k transition M_seg (the same chunk
//                      recurrence run on the identity, by a second workgroup per
//                      segment), or the scalar log decay
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
constexpr int NW = 4;     // waves per workgroup
constexpr int NTHR = NW * 64;
constexpr int RPW = DV / NW;  // state rows per wave (two 16-row column tiles)
#ifndef LA_CHUNK_WG_PER_CU
#define LA_CHUNK_WG_PER_CU 2
#endif
#ifndef LA_CHUNK_PREFETCH
#define LA_CHUNK_PREFETCH 0
#endif
// Two workgroups per CU hide each other's load latency and latency-bound phases; with
// one, the next chunk is prefetched into registers instead.
constexpr int WG_PER_CU = LA_CHUNK_WG_PER_CU;
// Keeps the scheduler from hoisting every operand load of a fully unrolled loop (which
// would raise register pressure past what two workgroups per CU allow).
#define LA_FENCE() __builtin_amdgcn_sched_barrier(0)
constexpr bool PREFETCH = LA_CHUNK_PREFETCH != 0;

constexpr int LDK = DK + 8;  // row-major bf16 tiles [C][DK]: K, Q, V, W, O staging
constexpr int LDA = C + 8;   // bf16 [C][C]: decay-masked Q K^T
constexpr int LDL = C + 4;   // fp32 [C][C]: L^T (strict upper) and T (lower)

constexpr int SZ_ROW = C * LDK * 2;
constexpr int SZ_LT = C * LDL * 4;
constexpr int SZ_A = C * LDA * 2;
constexpr int SZ_VEC = 5 * C * 4;
static_assert(SZ_ROW <= SZ_LT, "O staging fits the L/T buffer");
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

typedef short v4i16 __attribute__((ext_vector_type(4)));

// A operand with k along the columns of a row-major tile: row `row`, 32-wide k-step at
// col0; lane group g supplies columns col0+4g..+3 and col0+16+4g..+3, the column order
// of two stacked 16x16 accumulator tiles (their rows 4g..4g+3).
__device__ __forceinline__ bf16x8 frag_pair(const bf16_t *base, int ld, int row, int col0, int g) {
  const uint2 lo = *reinterpret_cast<const uint2 *>(base + row * ld + col0 + 4 * g);
  const uint2 hi = *reinterpret_cast<const uint2 *>(base + row * ld + col0 + 16 + 4 * g);
  const u32x4 w = {lo.x, lo.y, hi.x, hi.y};
  return __builtin_bit_cast(bf16x8, w);
}

// Operand with k along the ROWS (tokens) of a row-major [token][d] tile: lane (g, i)
// receives column 16 nt + i at tokens 32 s + 4 g + 0..3 and 32 s + 16 + 4 g + 0..3 (the
// same token order as frag_pair's columns).  ds_read_b64_tr_b16 hands lane i of each
// 16-lane group element (i & 3) of the 8-byte chunks addressed by lanes 4 e + (i >> 2),
// e = 0..3; lane j therefore addresses row tbase + (j >> 2), columns 16 nt + 4 (j & 3).
__device__ __forceinline__ bf16x8 col_frag(const bf16_t *tile, int ld, int nt, int s, int lane) {
  const int g = lane >> 4, i = lane & 15;
  const bf16_t *p0 = tile + (32 * s + 4 * g + (i >> 2)) * ld + 16 * nt + 4 * (i & 3);
  typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(p0));
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(p0 + 16 * ld));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

__device__ __forceinline__ bf16x8 pack_pair(f32x4 a, f32x4 b) {
  return pack8(a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]);
}

__device__ __forceinline__ f32x4 ld4(const float *p) { return *reinterpret_cast<const f32x4 *>(p); }

__device__ __forceinline__ void tri_index(int idx, int &ti, int &tj) {
  ti = idx >= 6 ? 3 : (idx >= 3 ? 2 : (idx >= 1 ? 1 : 0));
  tj = idx - ti * (ti + 1) / 2;
}

// Row t of T restricted to tokens perm(s, g), with the upper triangle (which holds L^T)
// masked to zero, scaled per token by sc and packed as a bf16 A operand.
__device__ __forceinline__ bf16x8 t_frag(const float *LT, const float *sc, int t, int s, int g) {
  f32x4 a = ld4(LT + t * LDL + 32 * s + 4 * g);
  f32x4 b = ld4(LT + t * LDL + 32 * s + 16 + 4 * g);
  const f32x4 sa = ld4(sc + 32 * s + 4 * g), sb = ld4(sc + 32 * s + 16 + 4 * g);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    a[e] = (32 * s + 4 * g + e) > t ? 0.0f : a[e] * sa[e];
    b[e] = (32 * s + 16 + 4 * g + e) > t ? 0.0f : b[e] * sb[e];
  }
  return pack_pair(a, b);
}

// Waves per workgroup: 4 (32 state rows each), or 8 for the delta-rule map pass, whose
// workgroup carries both the 128 B rows (waves 0-3) and the 128 M rows (waves 4-7) so
// that the state-independent work of a chunk is done once for both.
template <int MODE, bool DELTA> struct Waves {
  static constexpr int value = (MODE == MODE_MAP && DELTA) ? 8 : NW;
};

template <int MODE, bool DELTA>
__global__ __launch_bounds__((Waves<MODE, DELTA>::value * 64), (WG_PER_CU * NW / 4)) void chunk_kernel(const Args a) {
  constexpr bool OUT = MODE == MODE_OUT;
  constexpr int NWT = Waves<MODE, DELTA>::value;  // waves in this workgroup
  constexpr int NT = NWT * 64;
  constexpr int NLD = C * (DK / 8) / NT;           // 16-byte tile loads per thread
  constexpr int MAPROWS = DELTA ? 2 * DV : DV;
  constexpr int OFF_K = 0;
  constexpr int OFF_Q = SZ_ROW;  // MODE_OUT only
  constexpr int OFF_VW = OUT ? 2 * SZ_ROW : SZ_ROW;
  constexpr int OFF_LT = OFF_VW + SZ_ROW;
  constexpr int OFF_A = OFF_LT + SZ_LT;  // MODE_OUT only
  constexpr int OFF_VEC = OUT ? OFF_A + SZ_A : OFF_LT + SZ_LT;
  constexpr int SMEM = OFF_VEC + SZ_VEC;
  __shared__ __attribute__((aligned(16))) unsigned char smem[SMEM];
  bf16_t *sK = reinterpret_cast<bf16_t *>(smem + OFF_K);
  bf16_t *sQ = reinterpret_cast<bf16_t *>(smem + OFF_Q);
  bf16_t *sV = reinterpret_cast<bf16_t *>(smem + OFF_VW);   // V, then -W (delta rule)
  bf16_t *sW = sV;
  float *sLT = reinterpret_cast<float *>(smem + OFF_LT);
  bf16_t *sO = reinterpret_cast<bf16_t *>(smem + OFF_LT);  // O staging after T is used
  bf16_t *sA = reinterpret_cast<bf16_t *>(smem + OFF_A);
  float *sG = reinterpret_cast<float *>(smem + OFF_VEC);
  float *sBeta = sG + C;
  float *sGam = sG + 2 * C;
  float *sDec = sG + 3 * C;
  float *sBG = sG + 4 * C;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l16 = lane & 15, g = lane >> 4;
  // in the delta-rule map pass, waves 4-7 carry the transition (M) rows
  const bool m_kind = (MODE == MODE_MAP) && DELTA && wave >= NW;
  const int seg = (int)blockIdx.x;
  const size_t bh = (size_t)blockIdx.z * a.H + blockIdx.y;
  const int64_t T = a.T;
  const int row0 = wave * RPW;  // first state row owned by this wave

  // ---- state: lane holds S^T[d = 16 m + 4 g + e][row0 + 16 c + l16] in st[m][c][e]
  f32x4 st[DK / 16][2];
  {
    const float *src = nullptr;
    if (OUT) src = a.nseg > 1 ? a.starts + (bh * a.nseg + seg) * DV * DK : (a.S0 ? a.S0 + bh * DV * DK : nullptr);
#pragma unroll
    for (int m = 0; m < DK / 16; ++m)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int r = row0 + 16 * c + l16;
        if (src) {
          st[m][c] = ld4(src + (size_t)r * DK + 16 * m + 4 * g);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)  // identity for the transition rows, zero otherwise
            st[m][c][e] = (m_kind && r - DV == 16 * m + 4 * g + e) ? 1.0f : 0.0f;
        }
      }
  }

  // ---- register prefetch of one chunk: 4 x 16 bytes of K (and Q, V) per thread
  u32x4 pk[4], pq[4], pv[4];
  float pal = 1.0f, pbe = 0.0f;
  const bool load_v = true;
#define LA_LD1(i)                                                                                \
  do {                                                                                           \
    const int id = tid + NT * (i), r = id >> 4, cv = id & 15;                                    \
    const u32x4 z = {0u, 0u, 0u, 0u};                                                            \
    pk[i] = r < pn ? *reinterpret_cast<const u32x4 *>(a.k + (prb + r) * DK + cv * 8) : z;       \
    if (OUT) pq[i] = r < pn ? *reinterpret_cast<const u32x4 *>(a.q + (prb + r) * DK + cv * 8) : z; \
    if (load_v) pv[i] = r < pn ? *reinterpret_cast<const u32x4 *>(a.v + (prb + r) * DV + cv * 8) : z; \
  } while (0)
#define LA_PREFETCH(T0)                                                                          \
  do {                                                                                           \
    const int64_t pt0 = (T0);                                                                    \
    const int pn = (int)((T - pt0) < C ? (T - pt0) : C);                                         \
    const size_t prb = bh * (size_t)T + pt0;                                                     \
    LA_LD1(0);                                                                                   \
    if (NLD > 1) LA_LD1(1);                                                                      \
    if (NLD > 2) { LA_LD1(2); LA_LD1(3); }                                                       \
    if (wave == 0) {                                                                             \
      pal = 1.0f;                                                                                \
      pbe = 0.0f;                                                                                \
      if (lane < pn) {                                                                           \
        if (a.variant != V_ADDITIVE) pal = bf16_to_f32(a.alpha[prb + lane]);                     \
        pbe = (a.variant == V_GATED_DELTA || (a.variant == V_GATED && a.has_beta))               \
                  ? bf16_to_f32(a.beta[prb + lane]) : 1.0f;                                      \
      }                                                                                          \
    }                                                                                            \
  } while (0)

  float gseg = 0.0f;  // log decay over the segment (scalar-gated map)
  int64_t prev_t0 = -1;
  int prev_n = 0;
  const int64_t first = (int64_t)seg * a.seg_chunks * C;
  int nchunks = a.seg_chunks;
  if (first + (int64_t)nchunks * C > T) nchunks = (int)((T - first + C - 1) / C);
  if (PREFETCH && nchunks > 0) LA_PREFETCH(first);

  for (int ci = 0; ci < nchunks; ++ci) {
    const int64_t t0 = first + (int64_t)ci * C;
    const int n = (int)((T - t0) < C ? (T - t0) : C);
    // An opaque copy of the lane index: LDS addresses derived from it are recomputed per
    // chunk (a few integer ops) instead of being hoisted out of the loop, where dozens
    // of them would occupy registers for the whole kernel.
    int lane_v = lane;
    asm volatile("" : "+v"(lane_v));
    const int l16 = lane_v & 15, g = lane_v >> 4;

    // ---- phase A: write out the previous chunk's O, move the prefetched chunk to LDS,
    // gate prefix sums
    if (OUT && prev_t0 >= 0) {
      for (int id = tid; id < prev_n * (DV / 8); id += NT) {
        const int r = id / (DV / 8), cv = id % (DV / 8);
        gst16(a.o + (bh * (size_t)T + prev_t0 + r) * DV + cv * 8,
              *reinterpret_cast<const u32x4 *>(sO + r * LDK + cv * 8));
      }
    }
    if (!PREFETCH) LA_PREFETCH(t0);
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int id = tid + NT * i, r = id >> 4, cv = id & 15;
      *reinterpret_cast<u32x4 *>(sK + r * LDK + cv * 8) = pk[i];
      if (OUT) *reinterpret_cast<u32x4 *>(sQ + r * LDK + cv * 8) = pq[i];
      if (load_v) *reinterpret_cast<u32x4 *>(sV + r * LDK + cv * 8) = pv[i];
    }
    if (wave == 0) {
      float x = (a.variant == V_ADDITIVE) ? 0.0f : logf(pal);
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
      }
      const float gC = __shfl(x, 63, 64);
      const float gam = expf(x);
      sG[lane] = x;
      sBeta[lane] = pbe;
      sGam[lane] = gam;
      sDec[lane] = expf(gC - x);
      sBG[lane] = pbe * gam;
    }
    __syncthreads();

    // ---- phase B: start loading the next chunk; Gram tiles K K^T (-> L^T) and Q K^T (-> A)
    if (PREFETCH && ci + 1 < nchunks) LA_PREFETCH(t0 + C);
    if (OUT) {
      // Row-tile ownership: wave w computes the K K^T tiles of row tile w and the Q K^T
      // tiles of row tile 3 - w (five tiles per wave); the A fragments of both row tiles
      // are loaded once and each K row tile (the B fragments) once per wave.
      const int tk = wave, tq = 3 - wave;
      bf16x8 ak[DK / 32], aq[DK / 32];
#pragma unroll
      for (int s = 0; s < DK / 32; ++s) {
        if (DELTA) ak[s] = *reinterpret_cast<const bf16x8 *>(sK + (16 * tk + l16) * LDK + 32 * s + 8 * g);
        aq[s] = *reinterpret_cast<const bf16x8 *>(sQ + (16 * tq + l16) * LDK + 32 * s + 8 * g);
      }
#pragma unroll
      for (int tj = 0; tj < 4; ++tj) {
        LA_FENCE();
        const bool do_kk = DELTA && tj <= tk;
        const bool do_qk = tj <= tq;
        if (!(do_kk || do_qk)) continue;
        bf16x8 b[DK / 32];
#pragma unroll
        for (int s = 0; s < DK / 32; ++s)
          b[s] = *reinterpret_cast<const bf16x8 *>(sK + (16 * tj + l16) * LDK + 32 * s + 8 * g);
        const int j = 16 * tj + l16;
        const float gj = sG[j];
        if (do_kk) {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < DK / 32; ++s) acc = mfma_bf16(ak[s], b[s], acc);
          f32x4 lv;  // L_tj at the transposed position [j][t]
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int t = 16 * tk + 4 * g + e;
            lv[e] = (t > j) ? sBeta[t] * expf(sG[t] - gj) * acc[e] : 0.0f;
          }
          *reinterpret_cast<f32x4 *>(sLT + j * LDL + 16 * tk + 4 * g) = lv;
        }
        if (do_qk) {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < DK / 32; ++s) acc = mfma_bf16(aq[s], b[s], acc);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int t = 16 * tq + 4 * g + e;
            sA[t * LDA + j] = f32_to_bf16((t >= j) ? expf(sG[t] - gj) * acc[e] : 0.0f);
          }
        }
      }
    } else if (DELTA) {
      // K K^T tiles only, (ti, tj) with tj <= ti, dealt round robin over the waves
      for (int job = wave; job < 10; job += NWT) {
        int ti, tj;
        tri_index(job, ti, tj);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < DK / 32; ++s) {
          const bf16x8 fa = *reinterpret_cast<const bf16x8 *>(sK + (16 * ti + l16) * LDK + 32 * s + 8 * g);
          const bf16x8 fb = *reinterpret_cast<const bf16x8 *>(sK + (16 * tj + l16) * LDK + 32 * s + 8 * g);
          acc = mfma_bf16(fa, fb, acc);
        }
        const int j = 16 * tj + l16;
        const float gj = sG[j];
        f32x4 lv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = 16 * ti + 4 * g + e;
          lv[e] = (t > j) ? sBeta[t] * expf(sG[t] - gj) * acc[e] : 0.0f;
        }
        *reinterpret_cast<f32x4 *>(sLT + j * LDL + 16 * ti + 4 * g) = lv;
      }
    }
    {
      if (OUT) {  // the two above-diagonal tiles read by the A U products
        for (int id = tid; id < 512; id += NT) {
          const int tile = id >> 8, e = id & 255;
          sA[(32 * tile + (e >> 4)) * LDA + 32 * tile + 16 + (e & 15)] = 0;
        }
      }
    }
    __syncthreads();

    f32x4 Ut[4][2];  // U~ tiles of this wave's rows (delta rule, B rows)
    if (DELTA) {
      // ---- phase C: inverses of the four 16 x 16 diagonal blocks of (I + L), written
      // to the lower triangle of the diagonal blocks (column-by-column forward
      // substitution, one lane per column)
      if (wave == 0) {
        const int bi = lane >> 4, c = lane & 15;
        float col[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          LA_FENCE();
          float acc = 0.0f;
#pragma unroll
          for (int kq = 0; kq < r; ++kq) acc += sLT[(16 * bi + kq) * LDL + 16 * bi + r] * col[kq];
          col[r] = (r == c) ? 1.0f : (r > c ? -acc : 0.0f);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (r >= c) sLT[(16 * bi + r) * LDL + 16 * bi + c] = col[r];
      }
      __syncthreads();
      // ---- phase D: off-diagonal blocks T_ij = -T_ii sum_{k=j}^{i-1} L_ik T_kj, by
      // sub-diagonal level, on fp32 MFMA (16x16x4)
#pragma unroll
      for (int level = 1; level <= 3; ++level) {
        LA_FENCE();
        if (wave < 4 - level) {
          const int j = wave, i = wave + level;
          f32x4 x = {0.f, 0.f, 0.f, 0.f};
          for (int kb = j; kb < i; ++kb) {
#pragma unroll
            for (int s = 0; s < 4; ++s) {
              const int kr = 4 * s + g;  // row of the k-block
              const float fa = sLT[(16 * kb + kr) * LDL + 16 * i + l16];
              float fb = sLT[(16 * kb + kr) * LDL + 16 * j + l16];
              if (kb == j && l16 > kr) fb = 0.0f;  // upper part of a diagonal block
              x = __builtin_amdgcn_mfma_f32_16x16x4f32(fa, fb, x, 0, 0, 0);
            }
          }
          f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < 4; ++s) {  // inner index 4 g + s: x's own rows serve as B
            float fa = sLT[(16 * i + l16) * LDL + 16 * i + 4 * g + s];
            if (4 * g + s > l16) fa = 0.0f;
            y = __builtin_amdgcn_mfma_f32_16x16x4f32(fa, x[s], y, 0, 0, 0);
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) sLT[(16 * i + 4 * g + e) * LDL + 16 * j + l16] = -y[e];
        }
        __syncthreads();
      }
      // ---- phase E1: U~ = T diag(beta) V for this wave's own state rows (registers)
      if (!m_kind) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          LA_FENCE();
          Ut[mt][0] = {0.f, 0.f, 0.f, 0.f};
          Ut[mt][1] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            if (s == 1 && mt < 2) continue;  // T is lower triangular
            const bf16x8 fa = t_frag(sLT, sBeta, 16 * mt + l16, s, g);
#pragma unroll
            for (int c = 0; c < 2; ++c)
              Ut[mt][c] = mfma_bf16(fa, col_frag(sV, LDK, 2 * wave + c, s, lane_v), Ut[mt][c]);
          }
        }
      }
      __syncthreads();
      // ---- phase E2: W = T diag(beta gamma) K, stored negated (bf16) over V
      constexpr int WPT = 8 / NWT;  // W column tiles per wave
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        LA_FENCE();
        f32x4 accw[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          if (s == 1 && mt < 2) continue;
          const bf16x8 fa = t_frag(sLT, sBG, 16 * mt + l16, s, g);
#pragma unroll
          for (int c = 0; c < WPT; ++c) accw[c] = mfma_bf16(fa, col_frag(sK, LDK, WPT * wave + c, s, lane_v), accw[c]);
        }
#pragma unroll
        for (int c = 0; c < WPT; ++c)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            sW[(16 * mt + 4 * g + e) * LDK + 16 * (WPT * wave + c) + l16] = f32_to_bf16(-accw[c][e]);
      }
      __syncthreads();
    }

    // ---- phase F: the state-dependent part, per wave on its own 32 state rows
    f32x4 U[4][2], O[4][2];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        U[mt][c] = (DELTA && !m_kind) ? Ut[mt][c] : f32x4{0.f, 0.f, 0.f, 0.f};
        O[mt][c] = {0.f, 0.f, 0.f, 0.f};
      }
    if (DELTA || OUT) {  // U = U~ - W S^T and O = Q S^T, sharing the S^T operands
#pragma unroll
      for (int s = 0; s < DK / 32; ++s) {
        bf16x8 sfr[2];
#pragma unroll
        for (int c = 0; c < 2; ++c) sfr[c] = pack_pair(st[2 * s][c], st[2 * s + 1][c]);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          LA_FENCE();
          if (DELTA) {
            const bf16x8 wf = frag_pair(sW, LDK, 16 * mt + l16, 32 * s, g);
#pragma unroll
            for (int c = 0; c < 2; ++c) U[mt][c] = mfma_bf16(wf, sfr[c], U[mt][c]);
          }
          if (OUT) {
            const bf16x8 qf = frag_pair(sQ, LDK, 16 * mt + l16, 32 * s, g);
#pragma unroll
            for (int c = 0; c < 2; ++c) O[mt][c] = mfma_bf16(qf, sfr[c], O[mt][c]);
          }
        }
      }
    }
    LA_FENCE();
    bf16x8 ufr[2][2], dufr[2][2];  // U and diag(decay) U as operands with k = tokens
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const f32x4 d0 = ld4(sDec + 32 * s2 + 4 * g), d1 = ld4(sDec + 32 * s2 + 16 + 4 * g);
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        f32x4 u0, u1;
        if (DELTA) {
          u0 = U[2 * s2][c];
          u1 = U[2 * s2 + 1][c];
        } else {  // U = diag(beta) V, read along tokens from the V tile
          const bf16x8 vf = col_frag(sV, LDK, 2 * wave + c, s2, lane_v);
          const f32x4 b0 = ld4(sBeta + 32 * s2 + 4 * g), b1 = ld4(sBeta + 32 * s2 + 16 + 4 * g);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            u0[e] = (float)vf[e] * b0[e];
            u1[e] = (float)vf[4 + e] * b1[e];
          }
        }
        ufr[c][s2] = pack_pair(u0, u1);
        dufr[c][s2] = pack_pair(u0 * d0, u1 * d1);
      }
    }
    if (OUT) {  // O = diag(gamma) Q S^T + A U  -> bf16 staging for coalesced stores
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        LA_FENCE();
        const f32x4 gam = ld4(sGam + 16 * mt + 4 * g);
#pragma unroll
        for (int c = 0; c < 2; ++c) O[mt][c] = O[mt][c] * gam;
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          if (s2 == 1 && mt < 2) continue;  // A is causal
          const bf16x8 af = frag_pair(sA, LDA, 16 * mt + l16, 32 * s2, g);
#pragma unroll
          for (int c = 0; c < 2; ++c) O[mt][c] = mfma_bf16(af, ufr[c][s2], O[mt][c]);
        }
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            sO[(16 * mt + 4 * g + e) * LDK + row0 + 16 * c + l16] = f32_to_bf16(O[mt][c][e]);
      }
    }
    {  // S^T <- gamma_C S^T + K^T diag(decay) U
      const float gC = sGam[C - 1];
      gseg += sG[C - 1];
#pragma unroll
      for (int m = 0; m < DK / 16; ++m) {
        LA_FENCE();
        const bf16x8 k0 = col_frag(sK, LDK, m, 0, lane_v), k1 = col_frag(sK, LDK, m, 1, lane_v);
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          f32x4 acc = st[m][c] * gC;
          acc = mfma_bf16(k0, dufr[c][0], acc);
          acc = mfma_bf16(k1, dufr[c][1], acc);
          st[m][c] = acc;
        }
      }
    }
    __syncthreads();
    prev_t0 = t0;
    prev_n = n;
  }

  if (OUT) {
    if (prev_t0 >= 0) {
      for (int id = tid; id < prev_n * (DV / 8); id += NT) {
        const int r = id / (DV / 8), cv = id % (DV / 8);
        gst16(a.o + (bh * (size_t)T + prev_t0 + r) * DV + cv * 8,
              *reinterpret_cast<const u32x4 *>(sO + r * LDK + cv * 8));
      }
    }
    if (a.nseg == 1 && a.S_T) {
#pragma unroll
      for (int m = 0; m < DK / 16; ++m)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const int r = row0 + 16 * c + l16;
          *reinterpret_cast<f32x4 *>(a.S_T + (bh * DV + r) * DK + 16 * m + 4 * g) = st[m][c];
        }
    }
  } else {
    float *dst = a.maps + (bh * a.nseg + seg) * (size_t)MAPROWS * DK;
#pragma unroll
    for (int m = 0; m < DK / 16; ++m)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int r = row0 + 16 * c + l16;
        *reinterpret_cast<f32x4 *>(dst + (size_t)r * DK + 16 * m + 4 * g) = st[m][c];
      }
    if (!DELTA && tid == 0) a.gsum[bh * a.nseg + seg] = gseg;
  }
#undef LA_PREFETCH
#undef LA_LD1
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

void chunk_segments(int B, int H, int64_t T, int *nseg, int *seg_chunks) {
  const gdn::Plan p = gdn::make_plan(B, H, T);
  *nseg = p.nseg;
  *seg_chunks = p.seg_chunks;
}

hipError_t launch_chunk_prefill(int variant, int B, int H, int64_t T, int d_k, int d_v,
                                const void *q, const void *k, const void *v, const void *alpha,
                                const void *beta, const float *S0, void *o, float *S_T,
                                void *workspace, int pass_mask, hipStream_t s) {
  using namespace gdn;
  if (d_k != DK || d_v != DV) {  // other widths: the token-recurrent kernel (fp32 arithmetic)
    if (!(pass_mask & PASS_REPLAY)) return hipSuccess;
    return launch_recurrent_rows(variant, T_BF16, B, H, T, d_k, d_v, q, k, v, alpha, beta, S0, o, S_T, s);
  }
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
  if (p.nseg > 1 && (pass_mask & PASS_MAPS)) {
    if (delta) hipLaunchKernelGGL((chunk_kernel<MODE_MAP, true>), grid, dim3(Waves<MODE_MAP, true>::value * 64), 0, s, a);
    else hipLaunchKernelGGL((chunk_kernel<MODE_MAP, false>), grid, dim3(NTHR), 0, s, a);
  }
  if (p.nseg > 1 && (pass_mask & PASS_SCAN)) {
    if (delta) hipLaunchKernelGGL((scan_kernel<true>), dim3(DV / 4, H, B), dim3(256), 0, s, a);
    else hipLaunchKernelGGL((scan_kernel<false>), dim3(DV / 4, H, B), dim3(256), 0, s, a);
  }
  if (pass_mask & PASS_REPLAY) {
    if (delta) hipLaunchKernelGGL((chunk_kernel<MODE_OUT, true>), grid, dim3(NTHR), 0, s, a);
    else hipLaunchKernelGGL((chunk_kernel<MODE_OUT, false>), grid, dim3(NTHR), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace la
