// la_abi.hip -- the C ABI declared in include/la.h: argument validation, aliasing and
// alignment checks, workspace sizing and dispatch to the kernels.  Validation always
// completes before anything is enqueued, so a rejected call touches no memory.
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "../../include/la.h"
#include "la_launch.h"

namespace la {

__global__ void copy_or_zero_kernel(const float *__restrict__ src, float *__restrict__ dst, size_t n) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    dst[i] = src ? src[i] : 0.0f;
}

hipError_t launch_copy_or_zero(const float *src, float *dst, size_t n, hipStream_t s) {
  if (n == 0 || src == dst) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(copy_or_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s, src, dst, n);
  return hipGetLastError();
}

// dst = lambda * src (lambda = 0: zeros, src not read); 16 bytes per thread and step, the
// n % 4 tail elementwise.
__global__ void scale_kernel(const float *__restrict__ src, float *dst, size_t n, float lambda) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  const size_t n4 = n / 4;
  const size_t i0 = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (size_t i = i0; i < n4; i += stride) {
    float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
    if (lambda != 0.0f) {
      x = reinterpret_cast<const float4 *>(src)[i];
      x = make_float4(lambda * x.x, lambda * x.y, lambda * x.z, lambda * x.w);
    }
    reinterpret_cast<float4 *>(dst)[i] = x;
  }
  for (size_t i = 4 * n4 + i0; i < n; i += stride) dst[i] = lambda != 0.0f ? lambda * src[i] : 0.0f;
}

namespace {

struct Range {
  const void *p;
  size_t n;
};

bool overlap(Range a, Range b) {
  if (!a.p || !b.p || a.n == 0 || b.n == 0) return false;
  const uintptr_t a0 = (uintptr_t)a.p, b0 = (uintptr_t)b.p;
  return a0 < b0 + b.n && b0 < a0 + a.n;
}

bool misaligned(const void *p, uintptr_t align = 16) { return p && ((uintptr_t)p & (align - 1)) != 0; }

bool is_based(int variant) { return variant == LA_BASED || variant == LA_BASED_COMPACT; }
int based_D(int dp, bool compact) { return compact ? 1 + dp + dp * (dp + 1) / 2 : 1 + dp + dp * dp; }

// Shared shape checks for prefill; returns LA_OK or an error.
int check_prefill_shape(int variant, int dtype, int B, int H, int64_t T, int dk, int dv) {
  if (variant < LA_ADDITIVE || variant > LA_BASED_COMPACT) return LA_ERR_INVALID;
  if (dtype != LA_F32 && dtype != LA_BF16) return LA_ERR_INVALID;
  if (B <= 0 || H <= 0 || T < 0 || dk <= 0 || dv <= 0) return LA_ERR_INVALID;
  if ((int64_t)B * H > (int64_t)INT32_MAX / 4) return LA_ERR_UNSUPPORTED;
  // at most 2^37 token-heads (2^31 chunks of 64: chunk and segment counts stay in 32 bits);
  // the inputs of a larger problem would not fit in any device's memory
  if (T > 0 && (int64_t)B * H > ((int64_t)1 << 37) / T) return LA_ERR_UNSUPPORTED;
  if (is_based(variant)) {
    if (dk != 16 || dv != 64) return LA_ERR_UNSUPPORTED;
    return LA_OK;
  }
  if (dtype == LA_BF16) {
    if (!(dk == dv && (dk == 64 || dk == 128 || dk == 256))) return LA_ERR_UNSUPPORTED;
  } else {
    if (dk != 64 && dk != 128 && dk != 256) return LA_ERR_UNSUPPORTED;
  }
  return LA_OK;
}

// Workspace bytes of a prefill whose segment plan keeps them within `cap` (SIZE_MAX: the
// plan depends on the shape alone); more than `cap` when even one segment needs more.
size_t prefill_ws(int variant, int dtype, int B, int H, int64_t T, int dk, int dv, size_t cap = SIZE_MAX) {
  if (T == 0) return 0;
  if (dtype != LA_BF16) {  // fp32: only the short chunk form uses one (without it, another fp32 path runs)
    const size_t need = is_based(variant) ? 0 : fp32_chunk_workspace_bytes(variant, B, H, T, dk, dv);
    return need <= cap ? need : 0;
  }
  if (is_based(variant)) return based_chunk_workspace_bytes(B, H, T, cap);
  return chunk_workspace_bytes(variant, B, H, T, dk, dv, cap);
}

}  // namespace

// Scratch of la_prefill_noalloc: the prefill workspace for callers that cannot allocate.
// One copy per device (a code-object global), held until the process ends.  Host code uses
// it only through the device address hipGetSymbolAddress returns (the array's name is a
// host-side stand-in, not a device address).
static __device__ __align__(256) unsigned char scratch[LA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[MAX_DEVICES];

// The scratch's device address on the current device, looked up once per device with that
// device current.
int scratch_for_current_device(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return LA_ERR_HIP;
  if (dev < 0 || dev >= MAX_DEVICES) return LA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return LA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return LA_OK;
}

}  // namespace
}  // namespace la

using namespace la;

extern "C" {

int la_abi_version(void) { return 1; }

const char *la_status_string(int status) {
  switch (status) {
    case LA_OK: return "LA_OK";
    case LA_ERR_NULL: return "LA_ERR_NULL: a required pointer is NULL";
    case LA_ERR_INVALID: return "LA_ERR_INVALID: invalid argument";
    case LA_ERR_UNSUPPORTED: return "LA_ERR_UNSUPPORTED: shape or dtype not supported";
    case LA_ERR_ALIGN: return "LA_ERR_ALIGN: pointer not 16-byte aligned";
    case LA_ERR_WORKSPACE: return "LA_ERR_WORKSPACE: workspace missing or too small";
    case LA_ERR_ALIAS: return "LA_ERR_ALIAS: buffers overlap";
    case LA_ERR_HIP: return "LA_ERR_HIP: a HIP launch failed";
    default: return "unknown la_status";
  }
}

int la_prefill_workspace_size(int variant, int dtype, int batch, int heads, int64_t seq_len,
                              int d_k, int d_v, size_t *bytes) {
  if (!bytes) return LA_ERR_NULL;
  const int st = check_prefill_shape(variant, dtype, batch, heads, seq_len, d_k, d_v);
  if (st != LA_OK) return st;
  *bytes = prefill_ws(variant, dtype, batch, heads, seq_len, d_k, d_v);
  return LA_OK;
}

static int prefill_impl(int pass_mask, int variant, int dtype, int batch, int heads,
                        int64_t seq_len, int d_k, int d_v, float eps, const void *q,
                        const void *k, const void *v, const void *alpha, const void *beta,
                        const float *S0, const float *z0, void *o, float *S_T, float *z_T,
                        void *workspace, size_t workspace_bytes, void *stream,
                        size_t ws_cap = SIZE_MAX) {
  if (pass_mask <= 0 || pass_mask > PASS_ALL) return LA_ERR_INVALID;
  int st = check_prefill_shape(variant, dtype, batch, heads, seq_len, d_k, d_v);
  if (st != LA_OK) return st;
  const int B = batch, H = heads;
  const int64_t T = seq_len;
  const bool based = is_based(variant), compact = variant == LA_BASED_COMPACT;
  // variant-specific pointer rules
  if (variant == LA_ADDITIVE || based) {
    if (alpha || beta) return LA_ERR_INVALID;
  } else if (variant == LA_GATED) {
    if (!alpha && T > 0) return LA_ERR_NULL;
  } else {
    if ((!alpha || !beta) && T > 0) return LA_ERR_NULL;
  }
  if (based) {
    if ((S0 == nullptr) != (z0 == nullptr)) return LA_ERR_INVALID;
    if ((S_T == nullptr) != (z_T == nullptr)) return LA_ERR_INVALID;
  } else if (z0 || z_T) {
    return LA_ERR_INVALID;
  }
  if (T > 0 && (!q || !k || !v || !o)) return LA_ERR_NULL;
  const size_t es = dtype == LA_F32 ? 4 : 2;
  // q, k, v, o and the states are moved in 16-byte vectors; alpha and beta per element
  const void *ptrs[] = {q, k, v, S0, z0, o, S_T, z_T, workspace};
  for (const void *p : ptrs)
    if (misaligned(p)) return LA_ERR_ALIGN;
  if (misaligned(alpha, es) || misaligned(beta, es)) return LA_ERR_ALIGN;

  const size_t BH = (size_t)B * H;
  const size_t D = based ? (size_t)based_D(d_k, compact) : 0;
  const size_t state_n = based ? BH * D * d_v : BH * d_v * d_k;
  const Range rq{q, BH * T * d_k * es}, rk{k, BH * T * d_k * es}, rv{v, BH * T * d_v * es};
  const Range ra{alpha, BH * T * es}, rb{beta, BH * T * es};
  const Range rS0{S0, state_n * 4}, rz0{z0, BH * D * 4};
  const Range ro{o, BH * T * d_v * es}, rST{S_T, state_n * 4}, rzT{z_T, BH * D * 4};
  const size_t need_ws = prefill_ws(variant, dtype, B, H, T, d_k, d_v, ws_cap);
  if (need_ws > 0 && (!workspace || workspace_bytes < need_ws)) return LA_ERR_WORKSPACE;
  const Range rw{workspace, need_ws};
  const Range outs[] = {ro, rST, rzT, rw};
  const Range ins[] = {rq, rk, rv, ra, rb, rS0, rz0};
  for (int i = 0; i < 4; ++i) {
    for (int j = i + 1; j < 4; ++j)
      if (overlap(outs[i], outs[j])) return LA_ERR_ALIAS;
    for (int j = 0; j < 7; ++j) {
      const bool same_state = (i == 1 && j == 5 && S_T == S0) || (i == 2 && j == 6 && z_T == z0);
      if (!same_state && overlap(outs[i], ins[j])) return LA_ERR_ALIAS;
    }
  }

  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipSuccess;
  if (T == 0) {  // empty sequence: the end state is the start state
    if (!(pass_mask & PASS_REPLAY)) return LA_OK;
    if (S_T) e = launch_copy_or_zero(S0, S_T, state_n, s);
    if (e == hipSuccess && z_T) e = launch_copy_or_zero(z0, z_T, BH * D, s);
    return e == hipSuccess ? LA_OK : LA_ERR_HIP;
  }
  if (based) {
    if (dtype == LA_BF16)
      e = launch_based_chunk_prefill(compact, B, H, T, eps, q, k, v, S0, z0, o, S_T, z_T, workspace,
                                     ws_cap, pass_mask, s);
    else if (pass_mask & PASS_REPLAY)
      e = launch_recurrent_based(dtype, compact, B, H, T, eps, q, k, v, S0, z0, o, S_T, z_T, s);
  } else if (dtype == LA_BF16) {
    e = launch_chunk_prefill(variant, B, H, T, d_k, d_v, q, k, v, alpha, beta, S0, o, S_T, workspace,
                             ws_cap, pass_mask, s);
  } else if (pass_mask & PASS_REPLAY) {
    e = launch_recurrent_rows(variant, dtype, B, H, T, d_k, d_v, q, k, v, alpha, beta, S0, o, S_T,
                              need_ws ? workspace : nullptr, need_ws, s);
  }
  return e == hipSuccess ? LA_OK : LA_ERR_HIP;
}

int la_prefill(int variant, int dtype, int batch, int heads, int64_t seq_len, int d_k, int d_v,
               float eps, const void *q, const void *k, const void *v, const void *alpha,
               const void *beta, const float *S0, const float *z0, void *o, float *S_T,
               float *z_T, void *workspace, size_t workspace_bytes, void *stream) {
  return prefill_impl(PASS_ALL, variant, dtype, batch, heads, seq_len, d_k, d_v, eps, q, k, v,
                      alpha, beta, S0, z0, o, S_T, z_T, workspace, workspace_bytes, stream);
}

int la_prefill_noalloc(int variant, int dtype, int batch, int heads, int64_t seq_len, int d_k,
                       int d_v, float eps, const void *q, const void *k, const void *v,
                       const void *alpha, const void *beta, const float *S0, const float *z0,
                       void *o, float *S_T, float *z_T, void *stream) {
  // shape first: a problem whose workspace exceeds the scratch even with one segment is
  // rejected before any HIP call
  const int st = check_prefill_shape(variant, dtype, batch, heads, seq_len, d_k, d_v);
  if (st != LA_OK) return st;
  if (prefill_ws(variant, dtype, batch, heads, seq_len, d_k, d_v, LA_NOALLOC_SCRATCH_BYTES) >
      LA_NOALLOC_SCRATCH_BYTES)
    return LA_ERR_WORKSPACE;
  void *ws = nullptr;
  const int sst = scratch_for_current_device(&ws);
  if (sst != LA_OK) return sst;
  return prefill_impl(PASS_ALL, variant, dtype, batch, heads, seq_len, d_k, d_v, eps, q, k, v, alpha,
                      beta, S0, z0, o, S_T, z_T, ws, LA_NOALLOC_SCRATCH_BYTES, stream,
                      LA_NOALLOC_SCRATCH_BYTES);
}

int la_prefill_pass(int pass, int variant, int dtype, int batch, int heads, int64_t seq_len,
                    int d_k, int d_v, float eps, const void *q, const void *k, const void *v,
                    const void *alpha, const void *beta, const float *S0, const float *z0,
                    void *o, float *S_T, float *z_T, void *workspace, size_t workspace_bytes,
                    void *stream) {
  int mask;
  switch (pass) {
    case LA_PASS_TRANSFORM: mask = PASS_TRANSFORM; break;
    case LA_PASS_MAPS: mask = PASS_MAPS; break;
    case LA_PASS_SCAN: mask = PASS_SCAN; break;
    case LA_PASS_REPLAY: mask = PASS_REPLAY; break;
    default: return LA_ERR_INVALID;
  }
  return prefill_impl(mask, variant, dtype, batch, heads, seq_len, d_k, d_v, eps, q, k, v, alpha,
                      beta, S0, z0, o, S_T, z_T, workspace, workspace_bytes, stream);
}

int la_prefill_segments(int variant, int dtype, int batch, int heads, int64_t seq_len, int d_k,
                        int d_v, int *n_segments, int *chunks_per_segment) {
  if (!n_segments || !chunks_per_segment) return LA_ERR_NULL;
  const int st = check_prefill_shape(variant, dtype, batch, heads, seq_len, d_k, d_v);
  if (st != LA_OK) return st;
  *n_segments = 1;
  *chunks_per_segment = 0;
  if (dtype != LA_BF16 || seq_len == 0) return LA_OK;
  if (is_based(variant))
    based_chunk_segments(batch, heads, seq_len, n_segments, chunks_per_segment);
  else if (d_k == d_v && (d_k == 128 || d_k == 256))
    chunk_segments(variant, batch, heads, seq_len, d_k, n_segments, chunks_per_segment);
  return LA_OK;
}


int la_decode_step(int variant, int dtype, int n, int d_k, int d_v, float eps, const float *S_in,
                   const float *z_in, float *S_out, float *z_out, const void *q, const void *k,
                   const void *v, const void *alpha, const void *beta, void *o, void *stream) {
  if (variant < LA_ADDITIVE || variant > LA_BASED_COMPACT) return LA_ERR_INVALID;
  if (dtype != LA_F32 && dtype != LA_BF16) return LA_ERR_INVALID;
  if (n <= 0 || d_k <= 0 || d_v <= 0) return LA_ERR_INVALID;
  const bool based = is_based(variant), compact = variant == LA_BASED_COMPACT;
  if (based) {
    if (d_k != 16 || d_v != 64) return LA_ERR_UNSUPPORTED;
  } else if (d_k != 64 && d_k != 128 && d_k != 256) {
    return LA_ERR_UNSUPPORTED;
  }
  if (variant == LA_ADDITIVE || based) {
    if (alpha || beta) return LA_ERR_INVALID;
  } else if (variant == LA_GATED) {
    if (!alpha) return LA_ERR_NULL;
  } else if (!alpha || !beta) {
    return LA_ERR_NULL;
  }
  if (!S_in || !S_out || !q || !k || !v || !o) return LA_ERR_NULL;
  if (based && (!z_in || !z_out)) return LA_ERR_NULL;
  if (!based && (z_in || z_out)) return LA_ERR_INVALID;
  const size_t es = dtype == LA_F32 ? 4 : 2;
  // states are moved in 16-byte vectors; the per-state token vectors element by element
  const void *sp[] = {S_in, z_in, S_out, z_out};
  for (const void *p : sp)
    if (misaligned(p)) return LA_ERR_ALIGN;
  const void *tp[] = {q, k, v, alpha, beta, o};
  for (const void *p : tp)
    if (misaligned(p, es)) return LA_ERR_ALIGN;
  const size_t D = based ? (size_t)based_D(d_k, compact) : 0;
  const size_t state_n = based ? (size_t)n * D * d_v : (size_t)n * d_v * d_k;
  const Range rSi{S_in, state_n * 4}, rzi{z_in, (size_t)n * D * 4};
  const Range rSo{S_out, state_n * 4}, rzo{z_out, (size_t)n * D * 4};
  const Range rq{q, (size_t)n * d_k * es}, rk{k, (size_t)n * d_k * es}, rv{v, (size_t)n * d_v * es};
  const Range ra{alpha, (size_t)n * es}, rb{beta, (size_t)n * es}, ro{o, (size_t)n * d_v * es};
  const Range outs[] = {rSo, rzo, ro};
  const Range ins[] = {rSi, rzi, rq, rk, rv, ra, rb};
  for (int i = 0; i < 3; ++i) {
    for (int j = i + 1; j < 3; ++j)
      if (overlap(outs[i], outs[j])) return LA_ERR_ALIAS;
    for (int j = 0; j < 7; ++j) {
      const bool same_state = (i == 0 && j == 0 && S_out == S_in) || (i == 1 && j == 1 && z_out == z_in);
      if (!same_state && overlap(outs[i], ins[j])) return LA_ERR_ALIAS;
    }
  }
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if (based)
    e = launch_decode_based(dtype, compact, n, eps, S_in, z_in, S_out, z_out, q, k, v, o, s);
  else
    e = launch_decode_rows(variant, dtype, n, d_k, d_v, S_in, S_out, q, k, v, alpha, beta, o, s);
  return e == hipSuccess ? LA_OK : LA_ERR_HIP;
}

int la_write_scores(int dtype, int batch, int heads, int64_t seq_len, int d_k, int chunk,
                    const void *k, float *d_head, float *d_mean, void *stream) {
  if (dtype != LA_F32 && dtype != LA_BF16) return LA_ERR_INVALID;
  if (batch <= 0 || heads <= 0 || seq_len < 0 || d_k <= 0 || chunk <= 0) return LA_ERR_INVALID;
  if (d_k != 64 && d_k != 128 && d_k != 256) return LA_ERR_UNSUPPORTED;
  if (batch > 65535 || heads > 65535 || (seq_len + chunk - 1) / chunk > INT32_MAX) return LA_ERR_UNSUPPORTED;
  if (seq_len == 0) return LA_OK;
  if (!k || !d_head) return LA_ERR_NULL;
  if (misaligned(k) || misaligned(d_head, 4) || misaligned(d_mean, 4)) return LA_ERR_ALIGN;
  const size_t es = dtype == LA_F32 ? 4 : 2, BHT = (size_t)batch * heads * seq_len;
  const Range rk{k, BHT * d_k * es}, rd{d_head, BHT * 4}, rm{d_mean, (size_t)batch * seq_len * 4};
  if (overlap(rk, rd) || overlap(rk, rm) || overlap(rd, rm)) return LA_ERR_ALIAS;
  const hipError_t e = launch_write_scores(dtype, batch, heads, seq_len, d_k, chunk, k, d_head, d_mean,
                                           (hipStream_t)stream);
  return e == hipSuccess ? LA_OK : LA_ERR_HIP;
}

int la_write_windows(int batch, int64_t seq_len, int chunk, int window, int tail,
                     const float *d_mean, int64_t *best_start, float *best_sum, void *stream) {
  if (batch <= 0 || seq_len < 0 || chunk <= 0 || window <= 0 || tail < 0 || tail > chunk)
    return LA_ERR_INVALID;
  if (batch > 65535 || seq_len / chunk > INT32_MAX) return LA_ERR_UNSUPPORTED;
  const int64_t nc = seq_len / chunk;
  if (nc == 0) return LA_OK;
  if (!d_mean || !best_start) return LA_ERR_NULL;
  if (misaligned(d_mean, 4) || misaligned(best_start, 8) || misaligned(best_sum, 4)) return LA_ERR_ALIGN;
  const Range rm{d_mean, (size_t)batch * seq_len * 4}, rs{best_start, (size_t)batch * nc * 8},
      rv{best_sum, (size_t)batch * nc * 4};
  if (overlap(rm, rs) || overlap(rm, rv) || overlap(rs, rv)) return LA_ERR_ALIAS;
  const hipError_t e = launch_write_windows(batch, seq_len, chunk, window, tail, d_mean, best_start, best_sum,
                                            (hipStream_t)stream);
  return e == hipSuccess ? LA_OK : LA_ERR_HIP;
}

int la_note_addresses(int dtype, int batch, int heads, int64_t seq_len, int d_k, int n_notes,
                      int d_rho, const float *d_head, const void *q, const int64_t *spans,
                      const int32_t *coords, int64_t *t_star, void *rho, void *stream) {
  if (dtype != LA_F32 && dtype != LA_BF16) return LA_ERR_INVALID;
  if (batch <= 0 || heads <= 0 || seq_len <= 0 || d_k <= 0 || n_notes < 0 || d_rho <= 0) return LA_ERR_INVALID;
  if (heads > 16 || d_rho > d_k || batch > 65535) return LA_ERR_UNSUPPORTED;
  if (n_notes == 0) return LA_OK;
  if (!d_head || !q || !spans || !coords || !t_star || !rho) return LA_ERR_NULL;
  const size_t es = dtype == LA_F32 ? 4 : 2;
  if (misaligned(d_head, 4) || misaligned(q, es) || misaligned(spans, 8) || misaligned(coords, 4) ||
      misaligned(t_star, 8) || misaligned(rho, es))
    return LA_ERR_ALIGN;
  const size_t BN = (size_t)batch * n_notes, BHT = (size_t)batch * heads * seq_len;
  const Range rt{t_star, BN * heads * 8}, rr{rho, BN * heads * d_rho * es};
  const Range ins[] = {{d_head, BHT * 4}, {q, BHT * d_k * es}, {spans, BN * 16}, {coords, (size_t)heads * d_rho * 4}};
  if (overlap(rt, rr)) return LA_ERR_ALIAS;
  for (const Range &r : ins)
    if (overlap(rt, r) || overlap(rr, r)) return LA_ERR_ALIAS;
  const hipError_t e = launch_note_addresses(dtype, batch, heads, seq_len, d_k, n_notes, d_rho, d_head, q, spans,
                                             coords, t_star, rho, (hipStream_t)stream);
  return e == hipSuccess ? LA_OK : LA_ERR_HIP;
}

int la_address_votes(int dtype, int n_notes, int channels, int n_query, int d_rho,
                     const void *rho, const void *u, int R, const int64_t *positions, float *score,
                     int32_t *choice, int32_t *votes, int32_t *selected, void *stream) {
  if (dtype != LA_F32 && dtype != LA_BF16) return LA_ERR_INVALID;
  if (n_notes <= 0 || channels <= 0 || n_query <= 0 || d_rho <= 0 || R <= 0) return LA_ERR_INVALID;
  if ((d_rho != 8 && d_rho != 16 && d_rho != 32) || n_query > 1024 || R > 64 || channels > 65535 ||
      n_notes > 16384)
    return LA_ERR_UNSUPPORTED;
  if (!rho || !u || !positions || !choice || !votes || !selected) return LA_ERR_NULL;
  const size_t es = dtype == LA_F32 ? 4 : 2;
  if (misaligned(rho, es) || misaligned(u, es) || misaligned(positions, 8) || misaligned(score, 4) ||
      misaligned(choice, 4) || misaligned(votes, 4) || misaligned(selected, 4))
    return LA_ERR_ALIGN;
  const size_t N = n_notes, J = channels;
  const Range outs[] = {{score, J * N * 4}, {choice, J * 4}, {votes, N * 4}, {selected, (size_t)R * 4}};
  const Range ins[] = {{rho, N * J * d_rho * es}, {u, (size_t)n_query * J * d_rho * es}, {positions, N * 8}};
  for (int i = 0; i < 4; ++i) {
    for (int j = i + 1; j < 4; ++j)
      if (overlap(outs[i], outs[j])) return LA_ERR_ALIAS;
    for (const Range &r : ins)
      if (overlap(outs[i], r)) return LA_ERR_ALIAS;
  }
  const hipError_t e = launch_address_votes(dtype, n_notes, channels, n_query, d_rho, rho, u, R, positions, score,
                                            choice, votes, selected, (hipStream_t)stream);
  return e == hipSuccess ? LA_OK : LA_ERR_HIP;
}

}  // extern "C"

int la_state_scale(int64_t n, float lambda, const float *S_in, float *S_out, void *stream) {
  if (n < 0 || !(lambda >= 0.0f && lambda <= 1.0f)) return LA_ERR_INVALID;
  if (n == 0) return LA_OK;
  if (!S_out || (!S_in && lambda != 0.0f)) return LA_ERR_NULL;
  if (misaligned(S_in) || misaligned(S_out)) return LA_ERR_ALIGN;
  const size_t bytes = (size_t)n * 4;
  if (S_in != S_out && overlap(Range{S_in, bytes}, Range{S_out, bytes})) return LA_ERR_ALIAS;
  size_t blocks = ((size_t)n / 4 + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(scale_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, S_in, S_out,
                     (size_t)n, lambda);
  return hipGetLastError() == hipSuccess ? LA_OK : LA_ERR_HIP;
}
