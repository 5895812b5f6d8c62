// based_chunk.hip -- chunkwise bf16 BASED prefill (bring-up stub: token-recurrent path).
#include "la_device.h"
#include "la_launch.h"

namespace la {

size_t based_chunk_workspace_bytes(int, int, int64_t) { return 0; }

void based_chunk_segments(int, int, int64_t, int *nseg, int *seg_chunks) {
  *nseg = 1;
  *seg_chunks = 0;
}

hipError_t launch_based_chunk_prefill(int B, int H, int64_t T, float eps, const void *q,
                                      const void *k, const void *v, const float *s0,
                                      const float *z0, void *o, float *s_T, float *z_T, void *,
                                      int pass_mask, hipStream_t s) {
  if (!(pass_mask & PASS_REPLAY)) return hipSuccess;
  return launch_recurrent_based(T_BF16, B, H, T, eps, q, k, v, s0, z0, o, s_T, z_T, s);
}

}  // namespace la
