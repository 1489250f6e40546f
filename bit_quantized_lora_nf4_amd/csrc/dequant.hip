// Standalone doubleDequant of an NF4 + DQ weight (gfx950).
//
// out = RN(q[code] * c') (fp32) or bf16_rne of it, with c' = fma(c8, s, o)
// ([Digest] "数学公式与关键细节" item 3, doubleDequant equation), or the stored fp32
// constant c' = c for the constant type without double quantization.
// HBM-bound: reads 0.516 B and writes 2 (bf16) or 4 (fp32) bytes per weight, so the
// writes set the pace.  A wave takes a span of 256 code dwords (2048 weights); in pass
// u = 0..3 lane l decodes dword 64 u + l of it (eight weights of one block) and
// writes them next to its neighbours' (bf16: one 16-byte store per lane, so every
// store instruction covers 1 KB of output contiguously).

#include "device_common.h"
#include "qlora_internal.h"

namespace qlora {
namespace {

constexpr int kThreads = 256;
constexpr int kSpanDwords = 4 * 64;  // four passes of the wave's 64 lanes

template <bool OUT_BF16, int CT>
__global__ __launch_bounds__(kThreads) void dequant_kernel(WeightView wv, int64_t n_dwords,
                                                           void *__restrict__ out, LevelTable lv) {
  const uint32_t *__restrict__ codes = reinterpret_cast<const uint32_t *>(wv.codes);
  __shared__ float lut[16];
  if (threadIdx.x < 16) lut[threadIdx.x] = lv.q[threadIdx.x];
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t n_spans = (n_dwords + kSpanDwords - 1) / kSpanDwords;
  const int64_t wstride = static_cast<int64_t>(gridDim.x) * (kThreads / 64);
  for (int64_t sp = static_cast<int64_t>(blockIdx.x) * (kThreads / 64) + wave; sp < n_spans; sp += wstride) {
    uint32_t w[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t d = sp * kSpanDwords + 64 * u + lane;
      w[u] = d < n_dwords ? codes[d] : 0u;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t d = sp * kSpanDwords + 64 * u + lane;  // weights 8 d .. 8 d + 7, block d / 8
      if (d >= n_dwords) continue;
      const float c = decode_constant<CT>(wv, d >> 3);
      if (OUT_BF16) {
        reinterpret_cast<u32x4_t *>(out)[d] = decode8(w[u], c, lut);
      } else {
        f32x4_t a, b;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a[e] = lut[(w[u] >> (4 * e)) & 15u] * c;
          b[e] = lut[(w[u] >> (4 * e + 16)) & 15u] * c;
        }
        f32x4_t *dst = reinterpret_cast<f32x4_t *>(out) + 2 * d;
        dst[0] = a;
        dst[1] = b;
      }
    }
  }
}

}  // namespace

hipError_t launch_dequantize(const WeightView &w, void *out, bool out_bf16, hipStream_t stream) {
  const LevelTable lv = level_table(w.quant_type);
  const int64_t n_dwords = w.n_rows * w.n_cols / 8;
  const int64_t spans = (n_dwords + kSpanDwords - 1) / kSpanDwords;
  int64_t blocks = (spans + kThreads / 64 - 1) / (kThreads / 64);
  if (blocks > 256 * 16) blocks = 256 * 16;
  dim3 grid(static_cast<unsigned>(blocks)), block(kThreads);
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, block, 0, stream, w, n_dwords, out, lv);
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
