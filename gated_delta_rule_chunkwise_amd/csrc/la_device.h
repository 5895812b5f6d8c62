// la_device.h -- small device helpers shared by the gfx950 kernels of libla.
//
// Element types: fp32 inputs are `float`; bf16 inputs are raw 16-bit patterns
// (`uint16_t`) so that the same templates serve both.  Conversions are exact on the
// way in (bf16 -> fp32 is a shift) and round-to-nearest-even on the way out
// (v_cvt_pk_bf16_f32).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace la {

typedef uint16_t bf16_t;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));

// 16-byte (and 8-byte) global-memory load/store through an explicit global (address space 1)
// pointer, so the compiler emits global_load/global_store rather than flat accesses.
__device__ __forceinline__ u32x4 gld16(const void *p) {
  return *(const __attribute__((address_space(1))) u32x4 *)(p);
}
__device__ __forceinline__ void gst16(void *p, u32x4 v) {
  *(__attribute__((address_space(1))) u32x4 *)(p) = v;
}
__device__ __forceinline__ void gst8(void *p, u32x2 v) {
  *(__attribute__((address_space(1))) u32x2 *)(p) = v;
}

// Raw buffer access (CDNA "buffer" instructions): a descriptor holds a wave-uniform base
// address and a size in bytes; lanes pass 32-bit byte offsets.  Loads beyond the size
// return zero and stores beyond it are dropped, which is how partial tiles are handled.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 bld16(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
__device__ __forceinline__ void bst16(rsrc_t r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, 0);
}
__device__ __forceinline__ void bst8(rsrc_t r, uint32_t off, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, (int)off, 0, 0);
}
__device__ __forceinline__ uint16_t bld2(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
}

// 2^x with the hardware instruction alone (no denormal range reduction, so results below
// 2^-126 may come out as zero).  Used for decay factors 2^(g_t - g_j) <= 1, where a
// factor that small contributes nothing at the precision of the result.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float bf16_to_f32(bf16_t u) { return __uint_as_float(((uint32_t)u) << 16); }

__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  __bf16 b = (__bf16)f;  // round to nearest even
  return __builtin_bit_cast(bf16_t, b);
}

template <typename T> struct io;
template <> struct io<float> {
  static __device__ __forceinline__ float ld(const float *p, size_t i) { return p[i]; }
  static __device__ __forceinline__ void st(float *p, size_t i, float x) { p[i] = x; }
};
template <> struct io<bf16_t> {
  static __device__ __forceinline__ float ld(const bf16_t *p, size_t i) { return bf16_to_f32(p[i]); }
  static __device__ __forceinline__ void st(bf16_t *p, size_t i, float x) { p[i] = f32_to_bf16(x); }
};

// 16x16x32 bf16 MFMA, fp32 accumulate.  Operand layout (one 64-lane wave):
//   A (16 x 32): lane l holds row (l % 16), eight k values of group (l / 16)
//   B (32 x 16): lane l holds column (l % 16), the same eight k values of group (l / 16)
//   C (16 x 16): lane l holds rows 4 (l / 16) + i, i = 0..3, of column (l % 16)
// Which eight k values a group covers only has to agree between A and B; the kernels
// choose that assignment explicitly wherever an operand is built from registers.
__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u16x8 u) { return __builtin_bit_cast(bf16x8, u); }

__device__ __forceinline__ bf16x8 pack8(float a0, float a1, float a2, float a3, float a4, float a5,
                                        float a6, float a7) {
  bf16x8 r;
  r[0] = (__bf16)a0; r[1] = (__bf16)a1; r[2] = (__bf16)a2; r[3] = (__bf16)a3;
  r[4] = (__bf16)a4; r[5] = (__bf16)a5; r[6] = (__bf16)a6; r[7] = (__bf16)a7;
  return r;
}

// Sum over aligned groups of `W` lanes (W a power of two, W <= 64) with xor shuffles;
// the reduction order is fixed, so results are bitwise reproducible.
template <int W> __device__ __forceinline__ float group_sum(float x) {
#pragma unroll
  for (int off = W / 2; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

}  // namespace la
