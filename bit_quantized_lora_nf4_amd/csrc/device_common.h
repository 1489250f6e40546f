// Device helpers shared by the gfx950 kernels: vector types, bf16 packing, MFMA
// wrappers and the two-level constant decode.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qlora {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// Two floats -> packed bf16 pair (round to nearest even; v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint16_t to_bf16(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t v) {
  return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

// 32x32x16 bf16 MFMA, fp32 accumulate.  Operand lane layout (both A and B):
// lane l supplies row/column (l % 32) and 8 contraction elements of group (l / 32).
// The accumulator of lane l holds column (l % 32), rows 8*(i/4) + 4*(l/32) + (i%4).
__device__ __forceinline__ f32x16_t mfma32x32x16(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
// 16x16x32 bf16 MFMA: lane l supplies row/column (l % 16), contraction group (l / 16);
// the accumulator of lane l holds column (l % 16), rows 4*(l/16) + i.
__device__ __forceinline__ f32x4_t mfma16x16x32(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Decoded first-level constant of flat block b: c' = fma(c8, s[g], o[g]), g = b / 256,
// rounded once ([Digest] "数学公式与关键细节" item 3: dequant(c1, c2)).
__device__ __forceinline__ float decode_constant(const int8_t *absmax_q, const float *s,
                                                 const float *o, int64_t b) {
  const int64_t g = b >> 8;
  return __builtin_fmaf(static_cast<float>(absmax_q[b]), s[g], o[g]);
}

// Eight codes of one u32 (element e in bits 4e..4e+3) -> four packed bf16 pairs of
// bf16_rne(q[code] * c).  `lut` is the 16-entry fp32 codebook in LDS.
__device__ __forceinline__ u32x4_t decode8(uint32_t w, float c, const float *lut) {
  u32x4_t r;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const float a = lut[(w >> (8 * p)) & 15u] * c;
    const float b = lut[(w >> (8 * p + 4)) & 15u] * c;
    r[p] = pack_bf16x2(a, b);
  }
  return r;
}

// Raw buffer resources: loads at byte offsets >= `bytes` return zeros, which gives
// branch-free bounds handling for tile edges.  Offsets are 32-bit.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, bytes, 0x00020000);
}
__device__ __forceinline__ u32x4_t buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ u32x2_t buf_load8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
__device__ __forceinline__ uint32_t buf_load4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
constexpr uint32_t kOOB = 0xFFFFFFF0u;  // an offset past any buffer: reads as zero

// Pack the low halves / high halves of two dwords: (lo(a), lo(b)) and (hi(a), hi(b)).
__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}
__device__ __forceinline__ float wave_min(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fminf(v, __shfl_xor(v, m, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

}  // namespace qlora
