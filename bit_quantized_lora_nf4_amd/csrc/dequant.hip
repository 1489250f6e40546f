// Standalone doubleDequant of an NF4 + DQ weight (gfx950).
//
// out = RN(q[code] * c') (fp32) or bf16_rne of it, with c' = fma(c8, s, o)
// ([Digest] "数学公式与关键细节" item 3, doubleDequant equation), or the stored fp32
// constant c' = c for the constant type without double quantization.  Each thread
// decodes 32 weights (16 bytes of codes, half a block, one constant) per
// iteration; a wave therefore reads 1 KB of codes and writes 4 KB of bf16.
// HBM-bound: reads 0.516 B and writes 2 (bf16) or 4 (fp32) bytes per weight.

#include "device_common.h"
#include "qlora_internal.h"

namespace qlora {
namespace {

constexpr int kThreads = 256;

template <bool OUT_BF16, int CT>
__global__ __launch_bounds__(kThreads) void dequant_kernel(WeightView wv, int64_t n_chunks,
                                                           void *__restrict__ out, LevelTable lv) {
  const u32x4_t *__restrict__ codes = reinterpret_cast<const u32x4_t *>(wv.codes);
  __shared__ float lut[16];
  if (threadIdx.x < 16) lut[threadIdx.x] = lv.q[threadIdx.x];
  __syncthreads();
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
  for (int64_t ch = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; ch < n_chunks;
       ch += stride) {
    const u32x4_t w = codes[ch];
    const float c = decode_constant<CT>(wv, ch >> 1);  // 2 chunks per block
    if (OUT_BF16) {
      u32x4_t *dst = reinterpret_cast<u32x4_t *>(static_cast<uint16_t *>(out) + ch * 32);
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[i] = decode8(w[i], c, lut);
    } else {
      f32x4_t *dst = reinterpret_cast<f32x4_t *>(static_cast<float *>(out) + ch * 32);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f32x4_t a, b;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a[e] = lut[(w[i] >> (4 * e)) & 15u] * c;
          b[e] = lut[(w[i] >> (4 * e + 16)) & 15u] * c;
        }
        dst[2 * i] = a;
        dst[2 * i + 1] = b;
      }
    }
  }
}

}  // namespace

hipError_t launch_dequantize(const WeightView &w, void *out, bool out_bf16, hipStream_t stream) {
  const LevelTable lv = level_table(w.quant_type);
  const int64_t n_chunks = w.n_rows * w.n_cols / 32;
  int64_t blocks = (n_chunks + kThreads - 1) / kThreads;
  if (blocks > 256 * 16) blocks = 256 * 16;
  dim3 grid(static_cast<unsigned>(blocks)), block(kThreads);
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, block, 0, stream, w, n_chunks, out, lv);
    return hipGetLastError();
  };
  switch (w.const_type * 2 + (out_bf16 ? 1 : 0)) {
    case 0: return go(dequant_kernel<false, kConstDqInt8>);
    case 1: return go(dequant_kernel<true, kConstDqInt8>);
    case 2: return go(dequant_kernel<false, kConstDqFp8>);
    case 3: return go(dequant_kernel<true, kConstDqFp8>);
    case 4: return go(dequant_kernel<false, kConstF32>);
    case 5: return go(dequant_kernel<true, kConstF32>);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qlora
