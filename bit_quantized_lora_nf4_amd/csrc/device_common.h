// Device helpers shared by the gfx950 kernels: vector types, bf16 packing, MFMA
// wrappers and the two-level constant decode.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qlora_internal.h"

namespace qlora {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef short v4i16_t __attribute__((ext_vector_type(4)));  // transposing LDS read result

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

// Exact value of an FP8 E4M3 byte (sign, 4 exponent bits with bias 7, 3 mantissa
// bits; exponent field 0 holds the subnormals m 2^-9).  The normal values are made
// by moving the byte into an fp32 bit pattern and re-biasing the exponent.
__device__ __forceinline__ float e4m3_value(uint32_t u) {
  const uint32_t mag = u & 0x7Fu;
  const float normal = __uint_as_float((mag << 20) + (120u << 23));
  const float sub = static_cast<float>(mag & 7u) * 0x1p-9f;
  const float v = (mag >> 3) ? normal : sub;
  return __uint_as_float(__float_as_uint(v) | ((u & 0x80u) << 24));
}

// The second-level code of a block constant as a float: a sign-extended int8, or an
// E4M3 value for the FP8-coded double quantization.
template <int CT>
__device__ __forceinline__ float c8_value(uint32_t byte) {
  if constexpr (CT == kConstDqFp8) return e4m3_value(byte);
  return static_cast<float>(static_cast<int>(byte << 24) >> 24);
}

// Decoded first-level constant of flat block b ([Digest] "数学公式与关键细节" item 3:
// dequant(c1, c2)): c' = fma(c8, s[b / 256], o[b / 256]), rounded once, for the
// double-quantized types; the stored fp32 constant for kConstF32.
template <int CT>
__device__ __forceinline__ float decode_constant(const WeightView &w, int64_t b) {
  if constexpr (CT == kConstF32) return w.absmax[b];
  const int64_t g = b >> 8;
  return __builtin_fmaf(c8_value<CT>(static_cast<uint8_t>(w.absmax_q[b])), w.dq_scale[g], w.dq_offset[g]);
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

// Buffer resources over the constant arrays of a quantized weight: the 8-bit codes,
// group scales and offsets of the double-quantized types, or (kConstF32) the fp32
// block constants in `s`.
struct ConstRsrc {
  __amdgpu_buffer_rsrc_t q8, s, o;
};
template <int CT>
__device__ __forceinline__ ConstRsrc make_const_rsrc(const WeightView &w, uint32_t n_blocks) {
  if constexpr (CT == kConstF32) {
    const __amdgpu_buffer_rsrc_t s = make_rsrc(w.absmax, n_blocks * 4u);
    return {s, s, s};
  }
  const uint32_t n_groups = (n_blocks + 255u) / 256u;
  return {make_rsrc(w.absmax_q, n_blocks), make_rsrc(w.dq_scale, n_groups * 4u),
          make_rsrc(w.dq_offset, n_groups * 4u)};
}
// Raw pieces of the constant of flat block b (zeros when !ok), loaded branch-free;
// c' is formed later by const_value, so that a prefetch does not force a wait on its
// own loads.  kConstF32 loads the one fp32 constant (into s).
struct ConstRaw {
  uint32_t c8, s, o;
};
template <int CT>
__device__ __forceinline__ ConstRaw fetch_constant(const ConstRsrc &r, uint32_t b, bool ok) {
  if constexpr (CT == kConstF32)
    return {0u, __builtin_amdgcn_raw_buffer_load_b32(r.s, ok ? b * 4u : kOOB, 0, 0), 0u};
  const uint32_t ob = ok ? b : kOOB;
  const uint32_t og = ok ? (b >> 8) * 4u : kOOB;
  return {__builtin_amdgcn_raw_buffer_load_b8(r.q8, ob, 0, 0),
          __builtin_amdgcn_raw_buffer_load_b32(r.s, og, 0, 0),
          __builtin_amdgcn_raw_buffer_load_b32(r.o, og, 0, 0)};
}
template <int CT>
__device__ __forceinline__ float const_value(const ConstRaw &c) {
  if constexpr (CT == kConstF32) return __uint_as_float(c.s);
  // The empty asm hides the loaded byte from instruction selection: otherwise the
  // sign extension is folded into a sign-extending load that is re-issued next to
  // this use, which then waits for every load in flight.
  uint32_t u = c.c8;
  asm("" : "+v"(u));
  return __builtin_fmaf(c8_value<CT>(u), __uint_as_float(c.s), __uint_as_float(c.o));
}

// Pack the low halves / high halves of two dwords: (lo(a), lo(b)) and (hi(a), hi(b)).
__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// ---- the last pass of a split reduction (FinalizeJob) -------------------------------
// Element i (of four floats) of the splits' partial sums added in split order,
// P_0 + P_1 + ...  The loads of four splits are issued before any is used: a split
// index past the last re-reads the last split and its value is not added, so the loads
// are straight-line code and the compiler does not wait for each before issuing the next.
__device__ __forceinline__ f32x4_t split_sum(const float *__restrict__ P, int splits, int64_t count, int64_t i) {
  const f32x4_t *P4 = reinterpret_cast<const f32x4_t *>(P);
  const int64_t c4 = count / 4;
  f32x4_t s = P4[i];
  for (int k = 1; k < splits; k += 4) {
    f32x4_t t[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) t[u] = P4[min(k + u, splits - 1) * c4 + i];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (k + u < splits) s += t[u];
  }
  return s;
}
// Group i of four values of the job: bf16(scale * sum) to its place in OUT.
__device__ __forceinline__ void finalize_one(const FinalizeJob &j, int64_t i) {
  const f32x4_t s = split_sum(j.P, j.splits, j.count, i);
  const u32x2_t o = {pack_bf16x2(s[0] * j.scale, s[1] * j.scale), pack_bf16x2(s[2] * j.scale, s[3] * j.scale)};
  const int64_t e = 4 * i, row = e / j.cols, col = e % j.cols;
  *reinterpret_cast<u32x2_t *>(j.OUT + row * j.ldout + col) = o;
}
// Workgroup wg of wgs (256 threads each) does groups wg 256 + t, then every wgs 256 on.
__device__ __forceinline__ void finalize_part(const FinalizeJob &j, int64_t wg, int64_t wgs) {
  const int64_t n4 = j.count / 4;
  for (int64_t i = wg * 256 + threadIdx.x; i < n4; i += wgs * 256) finalize_one(j, i);
}

// ---- register-only NF4 decode -------------------------------------------------------
// For one block constant c, the 16 possible decoded weights T[j] = bf16_rne(q[j] * c)
// are kept as byte planes: L[p] holds the low bytes of T[4p..4p+3], H[p] the high bytes.
struct Planes {
  uint32_t L[4], H[4];
};

__device__ __forceinline__ Planes make_planes(float c, const LevelTable &lv) {
  uint32_t t[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) t[i] = pack_bf16x2(lv.q[2 * i] * c, lv.q[2 * i + 1] * c);
  Planes P;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    P.L[p] = __builtin_amdgcn_perm(t[2 * p + 1], t[2 * p], 0x06040200u);
    P.H[p] = __builtin_amdgcn_perm(t[2 * p + 1], t[2 * p], 0x07050301u);
  }
  return P;
}

// Half h of make_planes: the byte planes of T[8h .. 8h + 7] (L[2h], L[2h + 1], H[2h],
// H[2h + 1]), so that the work of one block constant can be spread over two places.
__device__ __forceinline__ void make_planes_half(float c, const LevelTable &lv, int h, Planes &P) {
  uint32_t t[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) t[i] = pack_bf16x2(lv.q[8 * h + 2 * i] * c, lv.q[8 * h + 2 * i + 1] * c);
#pragma unroll
  for (int pp = 0; pp < 2; ++pp) {
    P.L[2 * h + pp] = __builtin_amdgcn_perm(t[2 * pp + 1], t[2 * pp], 0x06040200u);
    P.H[2 * h + pp] = __builtin_amdgcn_perm(t[2 * pp + 1], t[2 * pp], 0x07050301u);
  }
}

__device__ __forceinline__ uint32_t bitsel(uint32_t m, uint32_t a, uint32_t b) {
  return (m & a) | (~m & b);  // v_bfi_b32
}

// Eight codes (element e in bits 4e..4e+3 of w) -> four bf16 pairs in element order,
// T[code] looked up with byte permutes: the low three code bits select a byte among
// eight table bytes, the fourth picks between the two eight-entry halves through a
// byte mask made by v_perm's sign-replicate selectors (8..11 copy bit 15/31/47/63).
__device__ __forceinline__ u32x4_t lookup8(uint32_t w, const Planes &P) {
  const uint32_t se = w & 0x07070707u;         // elements 0, 2, 4, 6
  const uint32_t so = (w >> 4) & 0x07070707u;  // elements 1, 3, 5, 7
  const uint32_t me = __builtin_amdgcn_perm(w << 12, w << 4, 0x090B080Au);
  const uint32_t mo = __builtin_amdgcn_perm(w << 8, w, 0x090B080Au);
  const uint32_t Le = bitsel(me, __builtin_amdgcn_perm(P.L[3], P.L[2], se),
                             __builtin_amdgcn_perm(P.L[1], P.L[0], se));
  const uint32_t He = bitsel(me, __builtin_amdgcn_perm(P.H[3], P.H[2], se),
                             __builtin_amdgcn_perm(P.H[1], P.H[0], se));
  const uint32_t Lo = bitsel(mo, __builtin_amdgcn_perm(P.L[3], P.L[2], so),
                             __builtin_amdgcn_perm(P.L[1], P.L[0], so));
  const uint32_t Ho = bitsel(mo, __builtin_amdgcn_perm(P.H[3], P.H[2], so),
                             __builtin_amdgcn_perm(P.H[1], P.H[0], so));
  const uint32_t LL0 = __builtin_amdgcn_perm(Lo, Le, 0x05010400u);  // low bytes e0..e3
  const uint32_t LL1 = __builtin_amdgcn_perm(Lo, Le, 0x07030602u);  // low bytes e4..e7
  const uint32_t HH0 = __builtin_amdgcn_perm(Ho, He, 0x05010400u);
  const uint32_t HH1 = __builtin_amdgcn_perm(Ho, He, 0x07030602u);
  u32x4_t r;
  r[0] = __builtin_amdgcn_perm(HH0, LL0, 0x05010400u);
  r[1] = __builtin_amdgcn_perm(HH0, LL0, 0x07030602u);
  r[2] = __builtin_amdgcn_perm(HH1, LL1, 0x05010400u);
  r[3] = __builtin_amdgcn_perm(HH1, LL1, 0x07030602u);
  return r;
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
