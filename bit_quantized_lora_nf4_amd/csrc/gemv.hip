// Small-M forward (M <= 16): a bandwidth-oriented dequant-GEMV (gfx950).
//
// Y[m, n] = bf16(sum_k X[m, k] W'[n, k] + sum_j U[m, j] Bl[n, j]) for M <= 16.  At
// such M the layer is bound by the weight stream (0.516 B per weight), so each
// wave streams one weight row with 16-byte coalesced loads of packed codes,
// decodes them to W' = bf16_rne(q[code] * c') ([Digest] "数学公式与关键细节"
// item 3) and accumulates in fp32; a wave reduction finishes the row.

#include "device_common.h"
#include "qlora_internal.h"

namespace qlora {
namespace {

constexpr int NT = 256;

__global__ __launch_bounds__(NT) void gemv_kernel(WeightView w, const uint16_t *__restrict__ X,
                                                  int M, const uint16_t *__restrict__ U,
                                                  const uint16_t *__restrict__ Bl, int r,
                                                  uint16_t *__restrict__ Y, LevelTable lvl) {
  __shared__ float lut[16];
  if (threadIdx.x < 16) lut[threadIdx.x] = lvl.q[threadIdx.x];
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t n = static_cast<int64_t>(blockIdx.x) * 4 + wave;
  const int64_t N = w.n_rows, K = w.n_cols;
  if (n >= N) return;
  float acc[16];
#pragma unroll
  for (int m = 0; m < 16; ++m) acc[m] = 0.0f;
  const int64_t chunks = K / 32;  // 16 bytes of codes = 32 weights
  const u32x4_t *crow = reinterpret_cast<const u32x4_t *>(w.codes + n * (K / 2));
  for (int64_t ch = lane; ch < chunks; ch += 64) {
    const u32x4_t code = crow[ch];
    const float c = decode_constant(w.absmax_q, w.dq_scale, w.dq_offset, (n * K) / 64 + ch / 2);
    float v[32];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u32x4_t d = decode8(code[i], c, lut);
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        v[i * 8 + 2 * p] = bf16_lo(d[p]);
        v[i * 8 + 2 * p + 1] = bf16_hi(d[p]);
      }
    }
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      if (m >= M) break;
      const u32x4_t *xr = reinterpret_cast<const u32x4_t *>(X + m * K + ch * 32);
      float s = acc[m];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const u32x4_t xv = xr[q];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          s = __builtin_fmaf(bf16_lo(xv[p]), v[q * 8 + 2 * p], s);
          s = __builtin_fmaf(bf16_hi(xv[p]), v[q * 8 + 2 * p + 1], s);
        }
      }
      acc[m] = s;
    }
  }
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    if (m >= M) break;
    float s = wave_sum(acc[m]);
    if (lane == 0) {
      for (int j = 0; j < r; ++j) s += bf16_to_f32(U[m * r + j]) * bf16_to_f32(Bl[n * r + j]);
      Y[m * N + n] = to_bf16(s);
    }
  }
}

}  // namespace

hipError_t launch_gemv_fwd(const WeightView &w, const uint16_t *X, int64_t M, const uint16_t *U,
                           const uint16_t *Bl, int r, uint16_t *Y, hipStream_t stream) {
  if (M < 1 || M > 16) return hipErrorInvalidValue;
  LevelTable lvl;
  for (int i = 0; i < 16; ++i) lvl.q[i] = codebook().q[i];
  dim3 grid(static_cast<unsigned>((w.n_rows + 3) / 4)), block(NT);
  hipLaunchKernelGGL(gemv_kernel, grid, block, 0, stream, w, X, static_cast<int>(M), U, Bl, r, Y,
                     lvl);
  return hipGetLastError();
}

}  // namespace qlora
