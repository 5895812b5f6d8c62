// based_chunk.hip -- chunkwise bf16 prefill for BASED Taylor linear attention (d' = 16,
// d_v = 64; states in the full D = 273 or the compact D = 153 feature layout).
//
// What is computed ("Simple linear attention language models balance the
// recall-throughput tradeoff", reading notes Sec. 2.2-2.3, paper Eqs. (1)-(4)):
//   phi(x) = [1, x, vec(x x^T)/sqrt 2],  s_t = s_{t-1} + phi(k_t) v_t^T,
//   z_t = z_{t-1} + phi(k_t),  o_t = s_t^T phi(q_t) / (z_t^T phi(q_t) + eps).
// Blockwise (the notes' Sec. 2.5 form U_b = (M_b . Phi_Q Phi_K^T) V_b + Phi_Q S_{<b}, and
// its normaliser), for a chunk of C = 64 tokens entering with (s, z):
//   A_tj = 1 + q_t.k_j + (q_t.k_j)^2 / 2 for j <= t, else 0   (= phi(q_t).phi(k_j))
//   num  = Phi_Q s + A V,   den = Phi_Q z + A 1,   o = num / (den + eps)
//   s   += Phi_K^T V,       z  += Phi_K^T 1
// The in-chunk term uses the closed form of the kernel, so phi is never multiplied out
// there; Phi_Q and Phi_K^T enter only the products with the state, and their entries are
// generated in registers from q and k while the MFMA operands are built (the feature
// expansion never touches LDS or HBM, which is the point the notes make about the
// IO-aware kernel).
//
// gfx950 layout.  x x^T is symmetric, so phi(q).phi(k) only needs each unordered pair
// {a, b} once: internally the order-2 block is kept as 9 "circulant diagonal" tiles.
// Row r of tile d (d = 0..8) stands for the pair (r, (r + d) mod 16); for d = 1..7, and
// rows r < 8 of d = 8, the state row is the sum of the two ABI rows (a, b) and (b, a),
// and the key feature carries weight sqrt 2 instead of 1/sqrt 2 (both orders at once).
// Row 8 of tile 8 is the constant feature, rows 9..15 are zero, tile 9 is x_0..x_15:
// 160 internal features (10 tiles) instead of 273 (18 tiles with padding).  The ABI
// layout [1, x, x (x) x] is restored when states are written: the antisymmetric part of
// a start state never changes (every update is symmetric in (a, b)) and is added back.
// In the replay, four waves each own one 16-column tile of s (10 x 4 fp32 accumulator
// tiles); the normaliser z lives in LDS in fp32: its increment is a one-row MFMA operand,
// its product with phi(q) is formed on the VALU from the fp32 features.  The map pass,
// which has no numerator to form, deals the same 40 accumulator tiles out by feature
// tile instead, so that no phi(k) fragment has to be shared between waves.  The state products are
// v_mfma_f32_16x16x32_bf16 (q.k: 16x16x16) with fp32 accumulation; token-contraction
// operands of k and v are read with ds_read_b64_tr_b16.
//
// Sequence parallelism: as for the gated recurrences, long sequences are split into
// segments; since A_t = I here, a segment's map is a plain sum (delta s, delta z), so
// pass 1 computes the sums from a zero state, pass 2 takes exclusive prefix sums over
// segments, and pass 3 replays every segment from its start state.
#include <utility>

#include "la_device.h"
#include "la_launch.h"

namespace la {
namespace based {

constexpr int C = 64;    // tokens per chunk
constexpr int DP = 16;   // q/k width d'
constexpr int DV = 64;   // value width
constexpr int D = 1 + DP + DP * DP;  // 273 features (ABI)
constexpr int ND = DP / 2 + 1;  // order-2 tiles: circulant diagonals d = 0..8
constexpr int T_LIN = ND;       // tile of the linear features x_0..x_15
constexpr int NF = 16 * (ND + 1);  // internal features (10 tiles)
constexpr int NFT = NF / 16;
constexpr int NW = 4;
constexpr int NTHR = NW * 64;

constexpr int LDQ = DP + 8;  // bf16 [C][DP] row-major k tile (48-byte rows)
constexpr int LDQ2 = 2 * DP + 8;  // bf16 [C][2 DP] q tile, each row holding q_t twice
constexpr int LDV = DV + 8;  // bf16 [C][DV] row-major v tile
constexpr int LDA = C + 8;   // bf16 [C][C] kernel matrix (transposed)

struct Args {
  const bf16_t *q, *k, *v;
  const float *s0, *z0;  // ABI layout; start state of segment 0 (may be NULL = zero)
  bf16_t *o;
  float *s_T, *z_T;      // ABI layout; written by the last segment's replay
  float *dsum;           // [BH][nseg][NF][DV + 1] per-segment sums (internal order; col DV = z)
  float *starts;         // [BH][nseg][NF][DV + 1] segment start states (internal order)
  int64_t T;
  int H, nseg, seg_chunks;
  int compact;           // ABI state layout: 0 = full (D = 273), 1 = compact (D = 153)
  int Dabi;              // ABI feature count, 273 or 153
  float eps;
};

typedef short v4i16 __attribute__((ext_vector_type(4)));

// Compact ABI index of the pair a <= b (row-major upper triangle after [1, x]).
__device__ __forceinline__ int compact_index(int a, int b) { return 1 + DP + a * DP - a * (a - 1) / 2 + (b - a); }

// The ABI rows behind internal feature fi: internal = w (row f1 + row f2), f1, f2 = -1 for
// none.  Full layout: f2 >= 0 only for the symmetrised pairs, whose ABI rows (a, b) = f1
// and (b, a) = f2 are both written back from the one internal row (w = 1).  Compact
// layout (LA_BASED_COMPACT): one ABI row per pair; for a < b the internal row holds
// sqrt 2 times it (its key feature is sqrt 2 k_a k_b against the compact map's k_a k_b),
// so w = sqrt 2; the squares, x and the constant map one to one.
__device__ __forceinline__ void abi_pair(int fi, bool compact, int &f1, int &f2, float &w) {
  const int t = fi >> 4, r = fi & 15;
  f1 = -1;
  f2 = -1;
  w = 1.0f;
  if (t == T_LIN) {
    f1 = 1 + r;
  } else if (t == ND - 1 && r >= DP / 2) {
    if (r == DP / 2) f1 = 0;  // the constant
  } else {
    const int b = (r + t) & 15;
    if (compact) {
      f1 = compact_index(r < b ? r : b, r < b ? b : r);
      if (t != 0) w = 1.41421356237309505f;
    } else {
      f1 = 1 + DP + DP * r + b;
      if (t != 0) f2 = 1 + DP + DP * b + r;
    }
  }
}

// Internal feature fi of a state read in ABI layout (NULL = zero state).
__device__ __forceinline__ float abi_load(const float *src, bool compact, int fi, int stride, int col) {
  if (!src) return 0.0f;
  int f1, f2;
  float w;
  abi_pair(fi, compact, f1, f2, w);
  float x = f1 >= 0 ? src[(size_t)f1 * stride + col] : 0.0f;
  if (f2 >= 0) x += src[(size_t)f2 * stride + col];
  return w * x;
}

// Internal feature fi with value x written back in ABI layout; src is the start state
// the symmetrised rows began from (NULL = zero), whose antisymmetric part is restored.
__device__ __forceinline__ void abi_store(float *dst, const float *src, bool compact, int fi, int stride,
                                          int col, float x) {
  int f1, f2;
  float w;
  abi_pair(fi, compact, f1, f2, w);
  if (f1 < 0) return;
  if (f2 < 0) {
    dst[(size_t)f1 * stride + col] = w == 1.0f ? x : x * 0.70710678118654752f;
    return;
  }
  const float asym = src ? src[(size_t)f1 * stride + col] - src[(size_t)f2 * stride + col] : 0.0f;
  dst[(size_t)f1 * stride + col] = 0.5f * (x + asym);
  dst[(size_t)f2 * stride + col] = 0.5f * (x - asym);
}

__device__ __forceinline__ bf16x8 pack_pair(f32x4 a, f32x4 b) {
  return pack8(a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]);
}

// Four floats to bf16 in two pairs (two v_cvt_pk_bf16_f32, no byte permutes)
__device__ __forceinline__ u32x2 pk4u(f32x4 x) {
  const bf16x2 a = {(__bf16)x[0], (__bf16)x[1]}, b = {(__bf16)x[2], (__bf16)x[3]};
  return u32x2{__builtin_bit_cast(unsigned, a), __builtin_bit_cast(unsigned, b)};
}

__device__ __forceinline__ f32x4 u16x4_to_f32(uint2 u) {
  f32x4 r;
  r[0] = __uint_as_float(u.x << 16);
  r[1] = __uint_as_float(u.x & 0xffff0000u);
  r[2] = __uint_as_float(u.y << 16);
  r[3] = __uint_as_float(u.y & 0xffff0000u);
  return r;
}

// Column 16 nt + (lane & 15) of a row-major [token][*] tile at tokens 32 s + 4 g + 0..3 and
// 32 s + 16 + 4 g + 0..3 (g = lane >> 4), via the CDNA4 transpose read (see chunk.hip).
__device__ __forceinline__ bf16x8 col_frag(const bf16_t *tile, int ld, int nt, int s, int lane) {
  const int g = lane >> 4, i = lane & 15;
  const bf16_t *p0 = tile + (32 * s + 4 * g + (i >> 2)) * ld + 16 * nt + 4 * (i & 3);
  typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(p0));
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(p0 + 16 * ld));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}


// x as held by lane M of this lane's row of 16 (DPP row broadcast; folded into the VALU
// instruction that consumes it)
template <int M> __device__ __forceinline__ float row_bcast(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x150 + M, 0xF, 0xF, true));
}
// x as held by lane (i - N) mod 16 of this lane's row of 16, i = lane % 16 (DPP row rotation)
template <int N> __device__ __forceinline__ float row_ror(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x120 + N, 0xF, 0xF, true));
}

// f(std::integral_constant<int, 0>{}), ..., f(std::integral_constant<int, N - 1>{})
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F> __device__ __forceinline__ void static_for(F &&f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Pass 3: every segment replayed from its start state, the outputs written; the last
// segment writes the end state.  Three workgroups per CU (49 KB of LDS, at most 168
// registers each).
__global__ __launch_bounds__(NTHR, 3) void based_replay_kernel(const Args a) {
  __shared__ __attribute__((aligned(16))) bf16_t sQ[C * LDQ2];
  __shared__ __attribute__((aligned(16))) bf16_t sK[C * LDQ];
  __shared__ __attribute__((aligned(16))) bf16_t sV[C * LDV];
  __shared__ __attribute__((aligned(16))) bf16_t sA[C * LDA];  // kernel matrix, transposed
  __shared__ __attribute__((aligned(16))) float sZ[NF];        // z, internal order
  __shared__ __attribute__((aligned(16))) float sZinc[NF + 64];  // this chunk's Phi_K^T 1 (+ spare slots)
  __shared__ __attribute__((aligned(16))) float sDen[C];  // 1 / (den + eps) per token
  // phi(q) as MFMA B-operand fragments, [token tile][feature step][lane] (16 bytes each):
  // each wave builds its token tile's once per chunk, every wave reads all four
  __shared__ __attribute__((aligned(16))) bf16x8 sPhi[4 * (NFT / 2) * 64];
  // phi(k)^T of the 9 order-2 feature tiles as MFMA A-operand fragments, [tile][token
  // step][lane], built once per chunk (two or three tiles per wave), kept in sPhi's space
  // once the numerator is done with phi(q)
  bf16x8 *const phik = sPhi;
  static_assert(ND * 2 <= 4 * (NFT / 2), "phi(k) fragments must fit in sPhi");

  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int seg = blockIdx.x;
  const size_t bh = (size_t)blockIdx.z * a.H + blockIdx.y;
  const int64_t T = a.T;
  const int n_col = wave;  // value-column tile owned by this wave
  const float rs2 = 0.70710678118654752f;

  // ---- state: lane holds s[feature 16 m + 4 g + e][16 n_col + l16] in st[m][e]
  f32x4 st[NFT];
  {
    const int l16 = lane & 15, g = lane >> 4;
    // with several segments the replay starts every segment from the scan's start states
    // (segment 0's is S0 in internal order, so no replay workgroup reads S0 while the last
    // one writes S_T, which may be the same buffer); with one segment it starts from S0
    // (ABI layout); the map pass starts from zero
    const float *src_i = a.nseg > 1 ? a.starts + (bh * a.nseg + seg) * (size_t)NF * (DV + 1) : nullptr;
    const float *src_a = (a.nseg == 1 && a.s0) ? a.s0 + bh * (size_t)a.Dabi * DV : nullptr;
#pragma unroll
    for (int m = 0; m < NFT; ++m)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int fi = 16 * m + 4 * g + e, col = 16 * n_col + l16;
        st[m][e] = src_i ? src_i[(size_t)fi * (DV + 1) + col] : abi_load(src_a, a.compact, fi, DV, col);
      }
    for (int fi = tid; fi < NF; fi += NTHR) {
      sZ[fi] = src_i ? src_i[(size_t)fi * (DV + 1) + DV]
                     : abi_load(a.nseg == 1 && a.z0 ? a.z0 + bh * a.Dabi : nullptr, a.compact, fi, 1, 0);
    }
  }

  const int64_t first = (int64_t)seg * a.seg_chunks * C;
  int nchunks = a.seg_chunks;
  if (first + (int64_t)nchunks * C > T) nchunks = (int)((T - first + C - 1) / C);

  // one chunk's q, k, v in registers (loaded while the previous chunk is processed):
  // two 16-byte pieces of v per thread, one of k (threads 0-127) or q (threads 128-255)
  u32x4 pv[2], pkq;
#define LA_BLOAD(T0)                                                                               \
  do {                                                                                             \
    const int64_t lt0 = (T0);                                                                      \
    const uint32_t ln = (uint32_t)((T - lt0) < C ? (T - lt0) : C);                                 \
    const size_t rb = bh * (size_t)T + lt0;                                                        \
    const rsrc_t rv = make_rsrc(a.v + rb * DV, ln * DV * 2);                                       \
    pv[0] = bld16(rv, 16u * (uint32_t)tid);                                                        \
    pv[1] = bld16(rv, 16u * (uint32_t)(tid + NTHR));                                               \
    if (tid < 2 * C) pkq = bld16(make_rsrc(a.k + rb * DP, ln * DP * 2), 16u * (uint32_t)tid);      \
    else pkq = bld16(make_rsrc(a.q + rb * DP, ln * DP * 2), 16u * (uint32_t)(tid - 2 * C)); \
  } while (0)
  if (nchunks > 0) LA_BLOAD(first);
  // one-row operand (row 0): 1 at every token, for A 1 and sum_t k_t.  Past T (a partial
  // last chunk) the loaded q, k, v are zero and A is causal, so an output row t < T never
  // meets a token j > t, and the keys past T add nothing to the sums
  const bf16x8 ones = (lane & 15) == 0 ? pack8(1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f)
                                       : pack8(0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f);
  if (tid < 128) {  // the above-diagonal tiles read by the A V products, A (0,1) and
                           // (2,3): zero for every chunk (visible after the first barrier)
    const int tile = tid >> 6, e = tid & 63;
    *reinterpret_cast<uint2 *>(sA + (32 * tile + 16 + (e >> 2)) * LDA + 32 * tile + 4 * (e & 3)) = make_uint2(0u, 0u);
  }

  for (int ci = 0; ci < nchunks; ++ci) {
    const int64_t t0 = first + (int64_t)ci * C;
    const int n = (int)((T - t0) < C ? (T - t0) : C);
    int lane_v = lane;  // opaque: keeps per-fragment LDS addresses inside the loop
    asm volatile("" : "+v"(lane_v));
    const int l16 = lane_v & 15, g = lane_v >> 4;

    // ---- phase A: this chunk's q, k, v to LDS
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int id = tid + NTHR * i, r = id >> 3, cv = id & 7;
      *reinterpret_cast<u32x4 *>(sV + r * LDV + cv * 8) = pv[i];
    }
    if (tid < 2 * C) {
      const int r = tid >> 1, cv = tid & 1;
      *reinterpret_cast<u32x4 *>(sK + r * LDQ + cv * 8) = pkq;
    } else {
      const int id = tid - 2 * C, r = id >> 1, cv = id & 1;
      *reinterpret_cast<u32x4 *>(sQ + r * LDQ2 + cv * 8) = pkq;
      *reinterpret_cast<u32x4 *>(sQ + r * LDQ2 + DP + cv * 8) = pkq;
    }
    __syncthreads();
    if (ci + 1 < nchunks) LA_BLOAD(t0 + C);

    // ---- phase B: kernel matrix A = 1 + QK^T + (QK^T)^2/2, causal, stored transposed
    // (row j, column t) in bf16; the 10 lower tiles (ti >= tj) dealt round robin, 3, 3, 2
    // and 2 a wave, with the wave index a constant in each branch so that tile addresses
    // are immediates and only diagonal tiles are masked.  q.k over d' = 16 is one
    // v_mfma_f32_16x16x16_bf16 per tile: lane (g, i) supplies elements 4 g..4 g + 3 of row
    // i; the operand reads are issued before the first product.
    float zq = 0.0f;  // z . phi(q_t) for token 16 wave + lane % 16
    {
      static_for<NW>([&](auto wc) {
        constexpr int W = decltype(wc)::value, NJ = W < 2 ? 3 : 2;
        if (wave == W) {
          v4i16 fa[NJ], fb[NJ];
          static_for<NJ>([&](auto mc) {
            constexpr int job = W + NW * decltype(mc)::value;
            constexpr int ti = job >= 6 ? 3 : (job >= 3 ? 2 : (job >= 1 ? 1 : 0)), tj = job - ti * (ti + 1) / 2;
            fa[decltype(mc)::value] = *reinterpret_cast<const v4i16 *>(sQ + (16 * ti + l16) * LDQ2 + 4 * g);
            fb[decltype(mc)::value] = *reinterpret_cast<const v4i16 *>(sK + (16 * tj + l16) * LDQ + 4 * g);
          });
          static_for<NJ>([&](auto mc) {
            constexpr int job = W + NW * decltype(mc)::value;
            constexpr int ti = job >= 6 ? 3 : (job >= 3 ? 2 : (job >= 1 ? 1 : 0)), tj = job - ti * (ti + 1) / 2;
            const f32x4 acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(fa[decltype(mc)::value], fb[decltype(mc)::value],
                                                                      f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
            f32x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float x = acc[e];
              v[e] = __builtin_fmaf(x, __builtin_fmaf(0.5f, x, 1.0f), 1.0f);
              if constexpr (ti == tj) v[e] = 4 * g + e >= l16 ? v[e] : 0.0f;
            }
            *reinterpret_cast<u32x2 *>(sA + (16 * tj + l16) * LDA + 16 * ti + 4 * g) = pk4u(v);
          });
        }
      });
      {  // phi(q_t) for this wave's token tile mt = wave, t = 16 mt + l16: the B operand of
         // feature step s holds rows 4 g + e of tiles 2 s and 2 s + 1.  With w[j] =
         // q_t[(4 g + j) mod 16] (three 8-byte reads of the doubled row), row r = 4 g + e of
         // diagonal tile d is w[e] w[e + d] / sqrt 2 -- every index a constant.  The same
         // fp32 values give the normaliser's state term z . phi(q_t) (40 features per lane,
         // then summed over the four lanes of the token).
        const int t = 16 * wave + l16;
        float w[12];
#pragma unroll
        for (int h = 0; h < 3; ++h) {
          const f32x4 x = u16x4_to_f32(*reinterpret_cast<const uint2 *>(sQ + t * LDQ2 + 4 * g + 4 * h));
#pragma unroll
          for (int e = 0; e < 4; ++e) w[4 * h + e] = x[e];
        }
        float ws[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) ws[e] = w[e] * rs2;
#pragma unroll
        for (int s = 0; s < NFT / 2; ++s) {
          f32x4 bt[2];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int d = 2 * s + h;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float pr = ws[e] * w[e + (d < ND ? d : 0)];
              if (d == T_LIN) bt[h][e] = w[e];
              else if (d == ND - 1) bt[h][e] = g < 2 ? pr : (g == 2 && e == 0 ? 1.0f : 0.0f);
              else bt[h][e] = pr;
            }
          }
          sPhi[(wave * (NFT / 2) + s) * 64 + lane] = pack_pair(bt[0], bt[1]);
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const f32x4 zz = *reinterpret_cast<const f32x4 *>(sZ + 16 * (2 * s + h) + 4 * g);
#pragma unroll
            for (int e = 0; e < 4; ++e) zq += bt[h][e] * zz[e];
          }
        }
        zq += __shfl_xor(zq, 16, 64);
        zq += __shfl_xor(zq, 32, 64);
      }
      __syncthreads();
    }

    // ---- phase C: numerator and denominator on the entering state (transposed, so a
    // lane holds four consecutive outputs of one token), then the carry
    const bf16x8 vf0 = col_frag(sV, LDV, n_col, 0, lane_v), vf1 = col_frag(sV, LDV, n_col, 1, lane_v);
    f32x4 num[4];
    {
      // num^T[c][t] = sum_f s[f][c] phi_f(q_t) + sum_j v_j[c] A[t][j]: the state is the A
      // operand (rows = value columns, k = features), phi(q_t) (from LDS) the B operand;
      // the transposed product leaves four consecutive outputs of one token in each lane.
      bf16x8 sfr[NFT / 2];
#pragma unroll
      for (int s = 0; s < NFT / 2; ++s) sfr[s] = pack_pair(st[2 * s], st[2 * s + 1]);
      // feature steps outer, token tiles inner (four independent accumulators), the phi(q)
      // fragments of the next step read one step ahead
      bf16x8 ph[2][4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        num[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        ph[0][mt] = sPhi[(mt * (NFT / 2)) * 64 + lane_v];
      }
#pragma unroll
      for (int s = 0; s < NFT / 2; ++s) {
        if (s + 1 < NFT / 2) {
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) ph[(s + 1) & 1][mt] = sPhi[(mt * (NFT / 2) + s + 1) * 64 + lane_v];
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) num[mt] = mfma_bf16(sfr[s], ph[s & 1][mt], num[mt]);
      }
#pragma unroll
      for (int it = 0; it < 6; ++it) {  // A V: (mt, s2) with s2 = 1 only for mt >= 2 (causal)
        const int mt = it < 2 ? it : 2 + (it - 2) / 2, s2 = it < 2 ? 0 : (it - 2) % 2;
        num[mt] = mfma_bf16(s2 == 0 ? vf0 : vf1, col_frag(sA, LDA, mt, s2, lane_v), num[mt]);
      }
      {  // den = z . phi(q_t) + the row sums of A (valid-token row), for token tile mt = wave
        const int mt = wave;
        f32x4 dacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          if (s2 == 1 && mt < 2) continue;
          dacc = mfma_bf16(ones, col_frag(sA, LDA, mt, s2, lane_v), dacc);
        }
        if (g == 0) sDen[16 * mt + l16] = __builtin_amdgcn_rcpf(dacc[0] + zq + a.eps);  // 1 / (den + eps)
      }
    }
    __syncthreads();  // every wave is done with phi(q) before sPhi is overwritten
    {
      // phi(k)^T fragments of the order-2 tiles (A operand: rows = features, k = tokens),
      // shared through LDS.  Row i of diagonal tile d is k_t[i] k_t[(i + d) mod 16] times
      // 1/sqrt 2 (d = 0) or sqrt 2 (both orders of the pair); tile 8 keeps rows i < 8 and
      // holds the constant 1 in row 8.  The K^T fragment
      // holds k_t[i] for i = lane % 16 at the lane's 8 tokens, so k_t[(i + d) mod 16] at the
      // same tokens is a DPP rotation of the 16-lane row, folded into the multiply (d must
      // be a constant, hence the uniform branch on the wave index).
      const bf16x8 kj[2] = {col_frag(sK, LDQ, 0, 0, lane_v), col_frag(sK, LDQ, 0, 1, lane_v)};
      f32x4 kf[2][2], kw[2][2];  // [s2][lo/hi]: k_t[i] and sqrt 2 k_t[i], fp32
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            kf[s2][h][e] = (float)kj[s2][4 * h + e];
            kw[s2][h][e] = kf[s2][h][e] * (2.0f * rs2);
          }
      // the fragment of diagonal tile d for token step s2
      auto build = [&](auto dc, int s2) {
        constexpr int d = decltype(dc)::value;
        f32x4 f[2];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if constexpr (d == 0) f[h][e] = kf[s2][h][e] * kf[s2][h][e] * rs2;
            else f[h][e] = kw[s2][h][e] * row_ror<16 - d>(kf[s2][h][e]);
            if constexpr (d == ND - 1)
              if (l16 >= DP / 2) f[h][e] = l16 == DP / 2 ? 1.0f : 0.0f;
          }
        phik[(d * 2 + s2) * 64 + lane] = pack_pair(f[0], f[1]);
      };
      // wave w: tiles w and w + 4, and waves 0 and 1 one token step each of tile 8
      static_for<NW>([&](auto wc) {
        constexpr int W = decltype(wc)::value;
        if (wave == W) {
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) {
            build(std::integral_constant<int, W>{}, s2);
            build(std::integral_constant<int, W + NW>{}, s2);
          }
          if constexpr (W < 2) build(std::integral_constant<int, ND - 1>{}, W);
        }
      });
      static_assert(ND - 1 == 2 * NW, "tiles 0..7 two a wave, tile 8 split between waves 0 and 1");
      // z's increment phi(K)^T 1, written before the barrier and off the carry's path: the
      // order-2 part from the key Gram G = sum_t k_t k_t^T (waves 2 and 3, half its rows
      // each; entry (a, b) lands in row a of diagonal tile (b - a) mod 16 when that is a kept
      // row), the linear part sum_t k_t, the constant sum_t 1 and tile 8's zero rows (wave
      // 3): every internal feature written once
      if (wave >= 2) {  // both form G; wave 2 scatters its rows 4 g, 4 g + 1, wave 3 the other two
        f32x4 zg = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) zg = mfma_bf16(kj[s2], kj[s2], zg);
        auto scatter = [&](auto e0c) {  // G[a][b], a = 4 g + e, b = l16; unkept entries to a spare slot
#pragma unroll
          for (int e = decltype(e0c)::value; e < decltype(e0c)::value + 2; ++e) {
            const int ra = 4 * g + e, d = (l16 - ra) & 15;
            const bool keep = d < ND - 1 || (d == ND - 1 && ra < DP / 2);
            sZinc[keep ? 16 * d + ra : NF + lane] = zg[e] * (d == 0 ? rs2 : 2.0f * rs2);
          }
        };
        if (wave == 2) scatter(std::integral_constant<int, 0>{});
        else scatter(std::integral_constant<int, 2>{});
      }
      if (wave == 3) {
        f32x4 zs = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) zs = mfma_bf16(ones, kj[s2], zs);  // row 0: sum_t k_t[l16]
        if (g == 0) {
          sZinc[16 * T_LIN + l16] = zs[0];
          // the constant feature counts the valid tokens
          if (l16 >= DP / 2) sZinc[16 * (ND - 1) + l16] = l16 == DP / 2 ? (float)n : 0.0f;
        }
      }
      __syncthreads();
    }
    {
      // carry.  Order-2 tile d (with the constant in tile 8): s += phi(K)_d^T V with the shared
      // phi(K)_d^T fragments, read one tile ahead.  Linear tile: K^T V.
      const bf16x8 kj[2] = {col_frag(sK, LDQ, 0, 0, lane_v), col_frag(sK, LDQ, 0, 1, lane_v)};
      bf16x8 pkb[2][2];
      pkb[0][0] = phik[0 * 64 + lane_v];
      pkb[0][1] = phik[1 * 64 + lane_v];
#pragma unroll
      for (int m = 0; m < ND; ++m) {
        if (m + 1 < ND) {
          pkb[(m + 1) & 1][0] = phik[((m + 1) * 2 + 0) * 64 + lane_v];
          pkb[(m + 1) & 1][1] = phik[((m + 1) * 2 + 1) * 64 + lane_v];
        }
        __builtin_amdgcn_sched_barrier(0);
        f32x4 acc = st[m];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) acc = mfma_bf16(pkb[m & 1][s2], s2 == 0 ? vf0 : vf1, acc);
        st[m] = acc;
      }
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) st[T_LIN] = mfma_bf16(kj[s2], s2 == 0 ? vf0 : vf1, st[T_LIN]);
    }
    __syncthreads();

    // ---- phase D: o = num / (den + eps) straight to HBM; z += this chunk's Phi_K^T 1
    {
      const rsrc_t ro = make_rsrc(a.o + (bh * (size_t)T + t0) * DV, (uint32_t)n * DV * 2);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const float r = sDen[16 * mt + l16];
        const f32x4 x = num[mt] * r;
        bst8(ro, 2u * (uint32_t)((16 * mt + l16) * DV + 16 * n_col + 4 * g), pk4u(x));
      }
    }
    for (int fi = tid; fi < NF; fi += NTHR) sZ[fi] += sZinc[fi];
  }
#undef LA_BLOAD

  if (seg == a.nseg - 1 && a.s_T) {  // the last segment's end state is S_T
    __syncthreads();
    const int l16 = lane & 15, g = lane >> 4;
    const float *s0 = a.s0 ? a.s0 + bh * (size_t)a.Dabi * DV : nullptr;
    const float *z0 = a.z0 ? a.z0 + bh * a.Dabi : nullptr;
#pragma unroll
    for (int m = 0; m < NFT; ++m)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        abi_store(a.s_T + bh * (size_t)a.Dabi * DV, s0, a.compact, 16 * m + 4 * g + e, DV, 16 * n_col + l16,
                  st[m][e]);
    for (int fi = tid; fi < NF; fi += NTHR) abi_store(a.z_T + bh * a.Dabi, z0, a.compact, fi, 1, 0, sZ[fi]);
  }
}

// Pass 1: each segment's sums (delta s, delta z) from a zero state.  A segment with a
// map never holds the sequence's last chunk (the plan gives the remainder to the last
// segment), so its chunks are whole; loads past T would read zeros all the same, and the
// constant feature's count is taken from T.  Here the waves own (feature tile,
// value-column tile) pairs instead of column tiles: wave w keeps the order-2 tiles 2 w
// and 2 w + 1 over all four column tiles and half of tile 8 + w / 2 (tile 8, or the
// linear tile 9), ten accumulator tiles each, so every wave builds only the phi(k)
// fragments it multiplies and none crosses LDS.  The normaliser's increment is kept as
// the key Gram sum_t k_t k_t^T (wave 2) and sum_t k_t (wave 3), accumulated in registers
// over the segment and scattered onto the diagonal tiles once at the end.  K and V are
// staged through registers two chunks ahead into two LDS buffers: one barrier a chunk.
__global__ __launch_bounds__(NTHR, 3) void based_map_kernel(const Args a) {
  __shared__ __attribute__((aligned(16))) bf16_t sK[2][C * LDQ];
  __shared__ __attribute__((aligned(16))) bf16_t sV[2][C * LDV];
  __shared__ __attribute__((aligned(16))) float sZf[NF];
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int seg = blockIdx.x;
  const size_t bh = (size_t)blockIdx.z * a.H + blockIdx.y;
  const int64_t T = a.T;
  const float rs2 = 0.70710678118654752f;
  const int64_t first = (int64_t)seg * a.seg_chunks * C;
  const int nchunks = a.seg_chunks;

  f32x4 sf[2][4], sx[2], zg = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    sx[i] = zg;
#pragma unroll
    for (int c = 0; c < 4; ++c) sf[i][c] = zg;
  }
  // row 0 of a one-row operand: 1 at every token (A operand of sum_t k_t)
  const bf16x8 ones = (lane & 15) == 0 ? pack8(1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f)
                                       : pack8(0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f);

  auto load = [&](u32x4(&pv)[2], u32x4 &pk, int64_t t0) {
    const uint32_t ln = (uint32_t)((T - t0) < C ? (T - t0) : C);
    const size_t rb = bh * (size_t)T + t0;
    const rsrc_t rv = make_rsrc(a.v + rb * DV, ln * DV * 2);
    pv[0] = bld16(rv, 16u * (uint32_t)tid);
    pv[1] = bld16(rv, 16u * (uint32_t)(tid + NTHR));
    if (tid < 2 * C) pk = bld16(make_rsrc(a.k + rb * DP, ln * DP * 2), 16u * (uint32_t)tid);
  };
  auto chunk = [&](int ci, u32x4(&pv)[2], u32x4 &pk, bf16_t *sKb, bf16_t *sVb) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int id = tid + NTHR * i;
      *reinterpret_cast<u32x4 *>(sVb + (id >> 3) * LDV + (id & 7) * 8) = pv[i];
    }
    if (tid < 2 * C) *reinterpret_cast<u32x4 *>(sKb + (tid >> 1) * LDQ + (tid & 1) * 8) = pk;
    // the buffer was last read two chunks ago, before every wave reached the previous
    // chunk's barrier
    __syncthreads();
    if (ci + 2 < nchunks) load(pv, pk, first + (int64_t)(ci + 2) * C);
    int lane_v = lane;  // opaque: keeps per-fragment LDS addresses inside the loop
    asm volatile("" : "+v"(lane_v));
    const int l16 = lane_v & 15;
    const bf16x8 kj[2] = {col_frag(sKb, LDQ, 0, 0, lane_v), col_frag(sKb, LDQ, 0, 1, lane_v)};
    bf16x8 vf[4][2];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) vf[c][s2] = col_frag(sVb, LDV, c, s2, lane_v);
    f32x4 kf[2][2], kw[2][2];  // [s2][lo/hi]: k_t[i] and sqrt 2 k_t[i], i = lane % 16
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          kf[s2][h][e] = (float)kj[s2][4 * h + e];
          kw[s2][h][e] = kf[s2][h][e] * (2.0f * rs2);
        }
    // phi(k)^T fragments of diagonal tile d (rows = features, k = the lane's tokens)
    auto phi = [&](auto dc, bf16x8(&p)[2]) {
      constexpr int d = decltype(dc)::value;
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        f32x4 f[2];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if constexpr (d == 0) f[h][e] = kf[s2][h][e] * kf[s2][h][e] * rs2;
            else f[h][e] = kw[s2][h][e] * row_ror<16 - d>(kf[s2][h][e]);
            if constexpr (d == ND - 1)
              if (l16 >= DP / 2) f[h][e] = l16 == DP / 2 ? 1.0f : 0.0f;
          }
        p[s2] = pack_pair(f[0], f[1]);
      }
    };
    static_for<NW>([&](auto wc) {
      constexpr int W = decltype(wc)::value;
      if (wave == W) {
        static_for<2>([&](auto ic) {
          constexpr int I = decltype(ic)::value;
          bf16x8 p[2];
          phi(std::integral_constant<int, 2 * W + I>{}, p);
#pragma unroll
          for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) sf[I][c] = mfma_bf16(p[s2], vf[c][s2], sf[I][c]);
        });
        constexpr int c0 = 2 * (W & 1);
        bf16x8 p[2];
        if constexpr (W < 2) phi(std::integral_constant<int, ND - 1>{}, p);
        else {
          p[0] = kj[0];
          p[1] = kj[1];
        }
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) sx[c] = mfma_bf16(p[s2], vf[c0 + c][s2], sx[c]);
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          if constexpr (W == 2) zg = mfma_bf16(kj[s2], kj[s2], zg);  // G[a][b], a = row, b = column
          if constexpr (W == 3) zg = mfma_bf16(ones, kj[s2], zg);    // row 0: sum_t k_t[b]
        }
      }
    });
  };

  u32x4 pva[2], pka, pvb[2], pkb;
  if (nchunks > 0) load(pva, pka, first);
  if (nchunks > 1) load(pvb, pkb, first + C);
  for (int ci = 0; ci < nchunks; ci += 2) {
    chunk(ci, pva, pka, sK[0], sV[0]);
    if (ci + 1 < nchunks) chunk(ci + 1, pvb, pkb, sK[1], sV[1]);
  }

  // z: the Gram's kept entries (G[a][b] is pair (a, b) on diagonal (b - a) mod 16), the
  // linear sums, the constant's count and tile 8's zero rows: every feature once
  const int l16 = lane & 15, g = lane >> 4;
  if (wave == 2) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int ra = 4 * g + e, d = (l16 - ra) & 15;
      if (d < ND - 1 || (d == ND - 1 && ra < DP / 2)) sZf[16 * d + ra] = zg[e] * (d == 0 ? rs2 : 2.0f * rs2);
    }
  } else if (wave == 3 && g == 0) {
    sZf[16 * T_LIN + l16] = zg[0];
    const int64_t cnt = (T - first) < (int64_t)nchunks * C ? (T - first) : (int64_t)nchunks * C;
    if (l16 >= DP / 2) sZf[16 * (ND - 1) + l16] = l16 == DP / 2 ? (float)cnt : 0.0f;
  }
  __syncthreads();
  float *dst = a.dsum + (bh * a.nseg + seg) * (size_t)NF * (DV + 1);
  const int c0 = 2 * (wave & 1), fx = ND - 1 + (wave >> 1);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int c = 0; c < 4; ++c) dst[(size_t)(16 * (2 * wave + i) + 4 * g + e) * (DV + 1) + 16 * c + l16] = sf[i][c][e];
#pragma unroll
    for (int c = 0; c < 2; ++c) dst[(size_t)(16 * fx + 4 * g + e) * (DV + 1) + 16 * (c0 + c) + l16] = sx[c][e];
  }
  for (int fi = tid; fi < NF; fi += NTHR) dst[(size_t)fi * (DV + 1) + DV] = sZf[fi];
}

// Pass 2: the start states of all segments in internal order: segment 0's is the
// (ABI-layout) start state, the others prefix sums of the per-segment sums of segments
// 0..nseg-2 from it (the last segment's replay writes the end state).  One thread per
// state element and (b, h), up to 16 segments' sums loaded at once.
__global__ __launch_bounds__(256) void based_scan_kernel(const Args a) {
  const size_t bh = (size_t)blockIdx.z * a.H + blockIdx.y;
  constexpr int NE = NF * (DV + 1);
  constexpr int UNR = 16;  // segments whose sums are loaded together
  for (int id = blockIdx.x * 256 + threadIdx.x; id < NE; id += gridDim.x * 256) {
    const int fi = id / (DV + 1), col = id % (DV + 1);
    // the start state and the end state's ABI place of this element: s[f][col] or z[f]
    const float *src = col < DV ? (a.s0 ? a.s0 + bh * (size_t)a.Dabi * DV : nullptr) : (a.z0 ? a.z0 + bh * a.Dabi : nullptr);
    const int stride = col < DV ? DV : 1, c = col < DV ? col : 0;
    float x = abi_load(src, a.compact, fi, stride, c);
    a.starts[(bh * a.nseg) * (size_t)NE + id] = x;
    const int nmap = a.nseg - 1;  // segments with a map
    for (int i0 = 0; i0 < nmap; i0 += UNR) {
      float d[UNR];
#pragma unroll
      for (int u = 0; u < UNR; ++u) d[u] = i0 + u < nmap ? a.dsum[(bh * a.nseg + i0 + u) * (size_t)NE + id] : 0.0f;
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        x += d[u];
        if (i0 + u < nmap) a.starts[(bh * a.nseg + i0 + u + 1) * (size_t)NE + id] = x;
      }
    }
  }
}

struct Plan {
  int nseg, seg_chunks;
};

// At most `nseg` segments of equal whole-chunk length over nch chunks.
Plan plan_of(int64_t nch, int64_t nseg) {
  if (nseg > nch) nseg = nch;
  if (nseg < 1) nseg = 1;
  const int64_t sc = (nch + nseg - 1) / nseg;
  return Plan{(int)((nch + sc - 1) / sc), (int)sc};
}

size_t ws_bytes(int B, int H, const Plan &p) {
  return p.nseg > 1 ? 2 * (size_t)B * H * p.nseg * NF * (DV + 1) * sizeof(float) : 0;
}

// About three workgroups per CU in all, split only when the heads alone cannot fill it;
// fewer segments when the workspace must stay within `cap` bytes (one segment needs none).
Plan make_plan(int B, int H, int64_t T, size_t cap) {
  const int64_t nch = (T + C - 1) / C;
  const int64_t bhn = (int64_t)B * H;
  Plan p = plan_of(nch, bhn < 384 ? (768 + bhn - 1) / bhn : 1);
  while (p.nseg > 1 && ws_bytes(B, H, p) > cap) p = plan_of(nch, p.nseg / 2);
  return p;
}

}  // namespace based

size_t based_chunk_workspace_bytes(int B, int H, int64_t T, size_t cap) {
  return based::ws_bytes(B, H, based::make_plan(B, H, T, cap));
}

void based_chunk_segments(int B, int H, int64_t T, int *nseg, int *seg_chunks) {
  const based::Plan p = based::make_plan(B, H, T, SIZE_MAX);
  *nseg = p.nseg;
  *seg_chunks = p.seg_chunks;
}

hipError_t launch_based_chunk_prefill(bool compact, int B, int H, int64_t T, float eps,
                                      const void *q, const void *k, const void *v,
                                      const float *s0, const float *z0, void *o, float *s_T,
                                      float *z_T, void *workspace, size_t ws_cap, int pass_mask,
                                      hipStream_t s) {
  using namespace based;
  const Plan p = make_plan(B, H, T, ws_cap);
  Args a;
  a.q = (const bf16_t *)q;
  a.k = (const bf16_t *)k;
  a.v = (const bf16_t *)v;
  a.s0 = s0;
  a.z0 = z0;
  a.o = (bf16_t *)o;
  a.s_T = s_T;
  a.z_T = z_T;
  const size_t half = (size_t)B * H * p.nseg * NF * (DV + 1);
  a.dsum = p.nseg > 1 ? (float *)workspace : nullptr;
  a.starts = p.nseg > 1 ? (float *)workspace + half : nullptr;
  a.T = T;
  a.H = H;
  a.nseg = p.nseg;
  a.seg_chunks = p.seg_chunks;
  a.compact = compact ? 1 : 0;
  a.Dabi = compact ? 1 + DP + DP * (DP + 1) / 2 : D;
  a.eps = eps;
  const dim3 grid(p.nseg, H, B);
  if (p.nseg > 1 && (pass_mask & PASS_MAPS))  // every segment but the last
    hipLaunchKernelGGL(based_map_kernel, dim3(p.nseg - 1, H, B), dim3(NTHR), 0, s, a);
  if (p.nseg > 1 && (pass_mask & PASS_SCAN))
    hipLaunchKernelGGL(based_scan_kernel, dim3((NF * (DV + 1) + 255) / 256, H, B), dim3(256), 0, s, a);
  if (pass_mask & PASS_REPLAY)
    hipLaunchKernelGGL(based_replay_kernel, grid, dim3(NTHR), 0, s, a);
  return hipGetLastError();
}

}  // namespace la
