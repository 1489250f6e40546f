// Skinny LoRA products (gfx950): the rank-r down-projections U_s, V and the two
// reductions over tokens that give dB and dA.
//
//   U_s = bf16((alpha/r) X A^T)   and   V = bf16((alpha/r) dY B)      (lora_down)
//   dB  = bf16(dY^T U_s)          and   dA = bf16(V^T X)              (reduce_m)
//
// ([Paper note] "关键设计 3" equation and listing; [Repro] "LoRA 的公式和张量形状":
// scaling = lora_alpha / r; [Digest] "方法步骤与流程" step 4: only the adapter
// receives gradients.)  All products run on the 32x32x16 bf16 MFMA with fp32
// accumulation.  The reductions over M are split over workgroups; each writes fp32
// partial sums to caller workspace and a second pass adds the partials in a fixed
// order, so results are bitwise reproducible (no floating-point atomics).

#include "device_common.h"
#include "qlora_internal.h"

namespace qlora {
namespace {

constexpr int NT = 256;

__device__ __forceinline__ u32x4_t load8(const uint16_t *p, int64_t rows, int64_t cols, int64_t row,
                                         int64_t col, bool vec_ok) {
  u32x4_t v = {0u, 0u, 0u, 0u};
  if (row >= rows || col >= cols) return v;
  const uint16_t *src = p + row * cols + col;
  if (vec_ok && col + 8 <= cols) return *reinterpret_cast<const u32x4_t *>(src);
  uint16_t t[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) t[e] = (col + e < cols) ? src[e] : uint16_t(0);
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = uint32_t(t[2 * e]) | (uint32_t(t[2 * e + 1]) << 16);
  return v;
}

// OUT[M, r] = bf16(scale * IN[M, Kc] . WT[r, Kc]^T).  Each wave owns 32 rows of IN and
// all RT * 32 >= r output columns; a workgroup covers 128 rows.
template <int RT>
__global__ __launch_bounds__(NT) void lora_down_kernel(const uint16_t *__restrict__ IN, int64_t M,
                                                       int64_t Kc, const uint16_t *__restrict__ WT,
                                                       int r, float scale,
                                                       uint16_t *__restrict__ OUT) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 128 + wave * 32 + (lane & 31);
  const bool vec = (Kc % 8) == 0;
  f32x16_t acc[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[t][e] = 0.0f;
  for (int64_t k = 0; k < Kc; k += 16) {
    const int64_t kk = k + (lane >> 5) * 8;
    const u32x4_t a = load8(IN, M, Kc, row, kk, vec);
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      const u32x4_t b = load8(WT, r, Kc, t * 32 + (lane & 31), kk, vec);
      acc[t] = mfma32x32x16(a, b, acc[t]);
    }
  }
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    const int col = t * 32 + (lane & 31);
    if (col >= r) continue;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int64_t orow = static_cast<int64_t>(blockIdx.x) * 128 + wave * 32 + (e >> 2) * 8 +
                           (lane >> 5) * 4 + (e & 3);
      if (orow < M) OUT[orow * r + col] = to_bf16(acc[t][e] * scale);
    }
  }
}

__global__ __launch_bounds__(NT) void transpose_kernel(const uint16_t *__restrict__ IN, int64_t R,
                                                       int64_t C, uint16_t *__restrict__ OUT) {
  __shared__ uint16_t tile[64][65];
  const int64_t r0 = static_cast<int64_t>(blockIdx.y) * 64, c0 = static_cast<int64_t>(blockIdx.x) * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int i = ty; i < 64; i += 4) {
    const int64_t r = r0 + i, c = c0 + tx;
    tile[i][tx] = (r < R && c < C) ? IN[r * C + c] : uint16_t(0);
  }
  __syncthreads();
  for (int i = ty; i < 64; i += 4) {
    const int64_t c = c0 + i, r = r0 + tx;
    if (r < R && c < C) OUT[c * R + r] = tile[tx][i];
  }
}

// Partial reduction over a split of MS = 256 rows:
//   P[s][no][j] = sum_{m in split s} IN[m][no] * S[m][j]
// IN [M, No] and S [M, r] are staged 32 rows at a time in LDS (row-major) and read
// column-wise into MFMA fragments (8 consecutive m per lane).  A workgroup covers 128
// columns of IN (one 32-column tile per wave) and all RT * 32 >= r columns of S.
constexpr int MS = 256;
constexpr int RM_COLS = 128;

template <int RT>
__global__ __launch_bounds__(NT) void reduce_m_partial_kernel(const uint16_t *__restrict__ IN,
                                                              int64_t M, int64_t No,
                                                              const uint16_t *__restrict__ S, int r,
                                                              float *__restrict__ P) {
  __shared__ uint16_t sIn[32][RM_COLS + 2];
  __shared__ uint16_t sS[32][RT * 32 + 2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t c0 = static_cast<int64_t>(blockIdx.x) * RM_COLS;
  const int64_t s_idx = blockIdx.y;
  const int64_t mbeg = s_idx * MS, mend = min<int64_t>(M, mbeg + MS);
  f32x16_t acc[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[t][e] = 0.0f;

  for (int64_t mb = mbeg; mb < mend; mb += 32) {
    __syncthreads();
    for (int i = tid; i < 32 * RM_COLS; i += NT) {
      const int rr = i / RM_COLS, cc = i % RM_COLS;
      const int64_t m = mb + rr, c = c0 + cc;
      sIn[rr][cc] = (m < mend && c < No) ? IN[m * No + c] : uint16_t(0);
    }
    for (int i = tid; i < 32 * RT * 32; i += NT) {
      const int rr = i / (RT * 32), cc = i % (RT * 32);
      const int64_t m = mb + rr;
      sS[rr][cc] = (m < mend && cc < r) ? S[m * r + cc] : uint16_t(0);
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int mm = ks * 16 + (lane >> 5) * 8;
      u32x4_t a;
      const int ac = wave * 32 + (lane & 31);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        a[e] = uint32_t(sIn[mm + 2 * e][ac]) | (uint32_t(sIn[mm + 2 * e + 1][ac]) << 16);
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        const int bc = t * 32 + (lane & 31);
        u32x4_t b;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          b[e] = uint32_t(sS[mm + 2 * e][bc]) | (uint32_t(sS[mm + 2 * e + 1][bc]) << 16);
        acc[t] = mfma32x32x16(a, b, acc[t]);
      }
    }
  }
  // acc[t] holds rows = IN columns (no), columns = S columns (j)
  float *dst = P + s_idx * No * r;
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    const int j = t * 32 + (lane & 31);
    if (j >= r) continue;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int64_t no = c0 + wave * 32 + (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3);
      if (no < No) dst[no * r + j] = acc[t][e];
    }
  }
}

__global__ __launch_bounds__(NT) void reduce_m_final_kernel(const float *__restrict__ P,
                                                            int64_t splits, int64_t No, int r,
                                                            uint16_t *__restrict__ OUT,
                                                            bool trans_out) {
  const int64_t total = No * r;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * NT + threadIdx.x; i < total;
       i += static_cast<int64_t>(gridDim.x) * NT) {
    float s = 0.0f;
    for (int64_t k = 0; k < splits; ++k) s += P[k * total + i];
    const int64_t no = i / r, j = i % r;
    if (trans_out)
      OUT[j * No + no] = to_bf16(s);
    else
      OUT[i] = to_bf16(s);
  }
}

}  // namespace

hipError_t launch_lora_down(const uint16_t *IN, int64_t M, int64_t Kc, const uint16_t *WT, int r,
                            float scale, uint16_t *OUT, hipStream_t stream) {
  const int64_t blocks = (M + 127) / 128;
  dim3 grid(static_cast<unsigned>(blocks)), block(NT);
  const int rt = (r + 31) / 32;
  switch (rt) {
#define QLORA_CASE(T)                                                                        \
  case T:                                                                                    \
    hipLaunchKernelGGL(lora_down_kernel<T>, grid, block, 0, stream, IN, M, Kc, WT, r, scale, \
                       OUT);                                                                 \
    break;
    QLORA_CASE(1) QLORA_CASE(2) QLORA_CASE(3) QLORA_CASE(4)
    QLORA_CASE(5) QLORA_CASE(6) QLORA_CASE(7) QLORA_CASE(8)
#undef QLORA_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_transpose_bf16(const uint16_t *IN, int64_t R, int64_t C, uint16_t *OUT,
                                 hipStream_t stream) {
  dim3 grid(static_cast<unsigned>((C + 63) / 64), static_cast<unsigned>((R + 63) / 64)), block(NT);
  hipLaunchKernelGGL(transpose_kernel, grid, block, 0, stream, IN, R, C, OUT);
  return hipGetLastError();
}

size_t reduce_m_workspace(int64_t M, int64_t No, int r) {
  const int64_t splits = (M + MS - 1) / MS;
  return static_cast<size_t>(splits) * No * r * sizeof(float);
}

hipError_t launch_reduce_m(const uint16_t *IN, int64_t M, int64_t No, const uint16_t *S, int r,
                           float *partials, uint16_t *OUT, bool trans_out, hipStream_t stream) {
  const int64_t splits = (M + MS - 1) / MS;
  dim3 grid(static_cast<unsigned>((No + RM_COLS - 1) / RM_COLS), static_cast<unsigned>(splits));
  dim3 block(NT);
  const int rt = (r + 31) / 32;
  switch (rt) {
#define QLORA_CASE(T)                                                                            \
  case T:                                                                                        \
    hipLaunchKernelGGL(reduce_m_partial_kernel<T>, grid, block, 0, stream, IN, M, No, S, r,      \
                       partials);                                                                \
    break;
    QLORA_CASE(1) QLORA_CASE(2) QLORA_CASE(3) QLORA_CASE(4)
    QLORA_CASE(5) QLORA_CASE(6) QLORA_CASE(7) QLORA_CASE(8)
#undef QLORA_CASE
    default:
      return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  int64_t fb = (No * r + NT - 1) / NT;
  if (fb > 4096) fb = 4096;
  hipLaunchKernelGGL(reduce_m_final_kernel, dim3(static_cast<unsigned>(fb)), dim3(NT), 0, stream,
                     partials, splits, No, r, OUT, trans_out);
  return hipGetLastError();
}

}  // namespace qlora
