// Blockwise NF4 quantization with fused double quantization (gfx950).
//
// One workgroup per double-quantization group: 256 blocks of 64 weights
// ([Ch. 11.3] "核心创新二": 64 weights share one constant; [Digest]
// "数学公式与关键细节" item 2: the constants are quantized again to 8 bits in
// groups of 256).  Eight lanes cover one block (8 weights each, one 16-byte
// load per lane for bf16), so a wave reads 1 KB of contiguous bf16 per pass
// and writes 256 contiguous bytes of packed codes.
//
// Per block: c = max |w| (a three-step lane reduction), inv = RN(1/c),
// x = RN(w * inv), code = #{j : x > T_j} through a 129-entry bucket table
// (one compare per weight), codes packed low nibble first.  A block with
// c < 2^-126 gets the zero code.  Per group (after a barrier): o = RN(min+max)
// * 0.5, h = max |RN(c - o)|, s = RN(h/127), c8 = clamp(rint(RN(RN(c-o)/s))).
// HBM-bound: 2.516 B per bf16 weight (4.516 for fp32 input).
//
// Variants of the pages' data-type comparison ([Digest] "6. 实验结果与分析",
// "核心结果分析" item 2; [Digest] "数学公式与关键细节" item 2 writes the second-level
// codes as FP8): the FP4 level table replaces the NF4 one through the bucket table;
// the FP8-coded double quantization uses s = RN(h / 448) and the E4M3 code of
// RN(RN(c - o) / s) (nearest, ties to the even code, saturated at 448); the fp32
// constant type keeps c itself (written to the absmax output) and skips the group pass.

#include "device_common.h"
#include "qlora_internal.h"

namespace qlora {
namespace {

constexpr int kThreads = 256;
constexpr float kTiny = 1.17549435e-38f;  // 2^-126

__device__ __forceinline__ float block_reduce_max(float v, float *red) {
  v = wave_max(v);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) red[wave] = v;
  __syncthreads();
  v = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  return v;
}
__device__ __forceinline__ float block_reduce_min(float v, float *red) {
  v = wave_min(v);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) red[wave] = v;
  __syncthreads();
  v = fminf(fminf(red[0], red[1]), fminf(red[2], red[3]));
  __syncthreads();
  return v;
}

// E4M3 code of x: the nearest value to |x| (saturated at 448), ties to the even code;
// the sign bit is set for x < 0.  Magnitudes below 2^-6 are the subnormal codes
// rint(|x| 2^9) (0 .. 8, where 8 is 2^-6 itself); above, the fp32 pattern is re-biased
// and its mantissa rounded to 3 bits, a carry moving into the exponent.
__device__ __forceinline__ uint32_t e4m3_encode(float x) {
  const float a = fminf(fabsf(x), 448.0f);
  uint32_t code;
  if (a < 0x1p-6f) {
    code = static_cast<uint32_t>(rintf(a * 512.0f));
  } else {
    const uint32_t bits = __float_as_uint(a);
    code = (bits + 0x7FFFFu + ((bits >> 20) & 1u) - (120u << 23)) >> 20;
  }
  return code | (x < 0.0f ? 0x80u : 0u);
}

template <bool IN_BF16>
__global__ __launch_bounds__(kThreads) void quantize_kernel(
    const void *__restrict__ W, int64_t n_blocks, uint32_t *__restrict__ codes,
    int8_t *__restrict__ absmax_q, float *__restrict__ dq_scale, float *__restrict__ dq_offset,
    float *__restrict__ absmax_out, int const_type, QuantTable tab) {
  __shared__ float2 s_tab[kBuckets];
  __shared__ float s_c[kGroup];
  __shared__ float s_red[4];

  const int tid = threadIdx.x;
  for (int i = tid; i < kBuckets; i += kThreads)
    s_tab[i] = make_float2(tab.thr[i], __int_as_float(tab.base[i]));

  const int64_t g = blockIdx.x;
  const int64_t b0 = g * kGroup;
  const int nbg = static_cast<int>(min<int64_t>(kGroup, n_blocks - b0));
  const int wave = tid >> 6, lane = tid & 63;
  const int sub = lane >> 3, part = lane & 7;

  // Issue every load of this lane first (8 passes of 8 blocks per wave), all in flight
  // at once: the loads are straight-line buffer loads over this group's bytes, and the
  // blocks past the last one (a partial final group) read as zero.
  constexpr uint32_t kEsz = IN_BF16 ? 2u : 4u;
  constexpr int kV = IN_BF16 ? 1 : 2;  // 16-byte loads per lane and pass
  const __amdgpu_buffer_rsrc_t rw =
      make_rsrc(static_cast<const char *>(W) + b0 * kBlock * kEsz, static_cast<uint32_t>(nbg) * kBlock * kEsz);
  u32x4_t raw[8][kV];
#pragma unroll
  for (int pass = 0; pass < 8; ++pass) {
    const uint32_t off = static_cast<uint32_t>((wave * 64 + pass * 8 + sub) * kBlock + part * 8) * kEsz;
#pragma unroll
    for (int v = 0; v < kV; ++v) raw[pass][v] = buf_load16(rw, off + 16u * v);
  }
  __syncthreads();  // bucket table ready

#pragma unroll
  for (int pass = 0; pass < 8; ++pass) {
    const int lb = wave * 64 + pass * 8 + sub;
    float w[8];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      if (IN_BF16) {
        w[2 * p] = bf16_lo(raw[pass][0][p]);
        w[2 * p + 1] = bf16_hi(raw[pass][0][p]);
      } else {
        w[p] = __uint_as_float(raw[pass][0][p]);
        w[4 + p] = __uint_as_float(raw[pass][kV - 1][p]);
      }
    }
    float m = 0.0f;
#pragma unroll
    for (int p = 0; p < 8; ++p) m = fmaxf(m, fabsf(w[p]));
    m = fmaxf(m, __shfl_xor(m, 1, 64));
    m = fmaxf(m, __shfl_xor(m, 2, 64));
    m = fmaxf(m, __shfl_xor(m, 4, 64));

    uint32_t word = 0x77777777u;  // zero code everywhere
    if (m >= kTiny) {
      const float inv = 1.0f / m;  // correctly rounded (no fast-math)
      word = 0;
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        const float x = w[p] * inv;
        // x * 64 is exact, so fma(x, 64, 64) equals RN(x * 64 + 64)
        int idx = static_cast<int>(fmaf(x, 64.0f, 64.0f));
        idx = min(max(idx, 0), kBuckets - 1);
        const float2 t = s_tab[idx];
        const uint32_t code = static_cast<uint32_t>(__float_as_int(t.y)) + (x > t.x ? 1u : 0u);
        word |= code << (4 * p);
      }
    }
    if (lb < nbg) {
      const int64_t blk = b0 + lb;
      codes[blk * 8 + part] = word;
      if (part == 0) {
        s_c[lb] = m;
        if (absmax_out) absmax_out[blk] = m;
      }
    }
  }
  __syncthreads();

  if (const_type == kConstF32) return;  // uniform: the constants went to absmax_out

  // ---- double quantization of this group's 256 constants --------------------
  const bool valid = tid < nbg;
  const float c = valid ? s_c[tid] : 0.0f;
  const float mn = block_reduce_min(valid ? c : INFINITY, s_red);
  const float mx = block_reduce_max(valid ? c : -INFINITY, s_red);
  const float o = (mn + mx) * 0.5f;
  const float d = c - o;
  const float h = block_reduce_max(valid ? fabsf(d) : 0.0f, s_red);
  uint32_t q8 = 0;
  float s = 0.0f;
  if (h != 0.0f) {
    if (const_type == kConstDqFp8) {
      s = h / 448.0f;  // correctly rounded
      q8 = e4m3_encode(d / s);
    } else {
      s = h / 127.0f;
      const float r = rintf(d / s);
      q8 = static_cast<uint32_t>(static_cast<int>(fminf(fmaxf(r, -127.0f), 127.0f))) & 0xFFu;
    }
  }
  if (valid) absmax_q[b0 + tid] = static_cast<int8_t>(static_cast<uint8_t>(q8));
  if (tid == 0) {
    dq_scale[g] = s;
    dq_offset[g] = o;
  }
}

}  // namespace

hipError_t launch_quantize(const void *W, bool w_bf16, int64_t n_rows, int64_t n_cols, int quant_type,
                           int const_type, uint8_t *codes, int8_t *absmax_q, float *dq_scale,
                           float *dq_offset, float *absmax_f32, hipStream_t stream) {
  if (const_type == kConstF32 && !absmax_f32) return hipErrorInvalidValue;
  const Codebook &cb = codebook(quant_type);
  QuantTable tab;
  for (int i = 0; i < kBuckets; ++i) {
    tab.thr[i] = cb.bucket_thr[i];
    tab.base[i] = cb.bucket_base[i];
  }
  const int64_t n_blocks = n_rows * n_cols / kBlock;
  const int64_t n_groups = (n_blocks + kGroup - 1) / kGroup;
  if (n_groups > 0x7fffffff) return hipErrorInvalidValue;
  dim3 grid(static_cast<unsigned>(n_groups)), block(kThreads);
  if (w_bf16)
    hipLaunchKernelGGL(quantize_kernel<true>, grid, block, 0, stream, W, n_blocks,
                       reinterpret_cast<uint32_t *>(codes), absmax_q, dq_scale, dq_offset,
                       absmax_f32, const_type, tab);
  else
    hipLaunchKernelGGL(quantize_kernel<false>, grid, block, 0, stream, W, n_blocks,
                       reinterpret_cast<uint32_t *>(codes), absmax_q, dq_scale, dq_offset,
                       absmax_f32, const_type, tab);
  return hipGetLastError();
}

}  // namespace qlora
