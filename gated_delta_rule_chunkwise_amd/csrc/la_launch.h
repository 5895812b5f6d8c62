// la_launch.h -- private host-side launchers implemented by the kernel files.  All
// arguments have been validated by the ABI layer (la_abi.hip) before these are called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace la {

enum { V_ADDITIVE = 0, V_BASED = 1, V_GATED = 2, V_GATED_DELTA = 3 };
enum { T_F32 = 0, T_BF16 = 1 };

// decode.hip
hipError_t launch_decode_rows(int variant, int dtype, int n, int d_k, int d_v, const float *S_in,
                              float *S_out, const void *q, const void *k, const void *v,
                              const void *alpha, const void *beta, void *o, hipStream_t s);
// compact: the 153-feature map of LA_BASED_COMPACT instead of the 273-feature one
hipError_t launch_decode_based(int dtype, bool compact, int n, float eps, const float *S_in,
                               const float *z_in, float *S_out, float *z_out, const void *q,
                               const void *k, const void *v, void *o, hipStream_t s);

// recurrent.hip (token-recurrent prefill; fp32 path)
// fp32 ADDITIVE / GATED problems of at most 2048 tokens (and small B H) take a chunk form
// whose per-chunk state sums live in the workspace: it runs when the workspace holds
// fp32_chunk_workspace_bytes() (non-zero), else the token walk or the attention form runs.
size_t fp32_chunk_workspace_bytes(int variant, int B, int H, int64_t T, int d_k, int d_v);
hipError_t launch_recurrent_rows(int variant, int dtype, int B, int H, int64_t T, int d_k, int d_v,
                                 const void *q, const void *k, const void *v, const void *alpha,
                                 const void *beta, const float *S0, void *o, float *S_T,
                                 void *workspace, size_t ws_bytes, hipStream_t s);
hipError_t launch_recurrent_based(int dtype, bool compact, int B, int H, int64_t T, float eps,
                                  const void *q, const void *k, const void *v, const float *s0,
                                  const float *z0, void *o, float *s_T, float *z_T, hipStream_t s);

// chunk.hip (chunkwise bf16 prefill for ADDITIVE / GATED / GATED_DELTA)
// ws_cap: the segment plan keeps the workspace within this many bytes (SIZE_MAX: no limit;
// the plan then depends on the shape alone, as la_prefill_segments reports it)
size_t chunk_workspace_bytes(int variant, int B, int H, int64_t T, int d_k, int d_v, size_t ws_cap);
// pass_mask: PASS_TRANSFORM | PASS_MAPS | PASS_SCAN | PASS_REPLAY (see la_prefill_pass in la.h)
enum { PASS_MAPS = 1, PASS_SCAN = 2, PASS_REPLAY = 4, PASS_TRANSFORM = 8, PASS_ALL = 15 };
hipError_t launch_chunk_prefill(int variant, int B, int H, int64_t T, int d_k, int d_v,
                                const void *q, const void *k, const void *v, const void *alpha,
                                const void *beta, const float *S0, void *o, float *S_T,
                                void *workspace, size_t ws_cap, int pass_mask, hipStream_t s);
void chunk_segments(int variant, int B, int H, int64_t T, int d, int *nseg, int *seg_chunks);

// based_chunk.hip (chunkwise bf16 BASED prefill)
size_t based_chunk_workspace_bytes(int B, int H, int64_t T, size_t ws_cap);
hipError_t launch_based_chunk_prefill(bool compact, int B, int H, int64_t T, float eps,
                                      const void *q, const void *k, const void *v,
                                      const float *s0, const float *z0, void *o, float *s_T,
                                      float *z_T, void *workspace, size_t ws_cap, int pass_mask,
                                      hipStream_t s);
void based_chunk_segments(int B, int H, int64_t T, int *nseg, int *seg_chunks);

// notebank.hip (NoteBank write and address steps)
hipError_t launch_write_scores(int dtype, int B, int H, int64_t T, int d_k, int chunk, const void *k,
                               float *d_head, float *d_mean, hipStream_t s);
hipError_t launch_write_windows(int B, int64_t T, int chunk, int window, int tail, const float *d_mean,
                                int64_t *best_start, float *best_sum, hipStream_t s);
hipError_t launch_note_addresses(int dtype, int B, int H, int64_t T, int d_k, int N, int d_rho,
                                 const float *d_head, const void *q, const int64_t *spans, const int *coords,
                                 int64_t *t_star, void *rho, hipStream_t s);
hipError_t launch_address_votes(int dtype, int N, int J, int nQ, int d_rho, const void *rho, const void *u,
                                int R, const int64_t *positions, float *score, int *choice, int *votes,
                                int *selected, hipStream_t s);

// util (la_abi.hip): copy or zero-fill n floats with a kernel (capture-safe, no memset nodes)
hipError_t launch_copy_or_zero(const float *src, float *dst, size_t n, hipStream_t s);

}  // namespace la
