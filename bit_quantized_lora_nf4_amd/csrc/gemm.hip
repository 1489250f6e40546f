// Fused NF4-decode GEMMs on bf16 MFMA (gfx950): the forward Y = X W'^T + U Bl^T
// and the input gradient dX = dY W' + V At^T.
//
// W' is never written to HBM: each workgroup streams packed codes plus int8 block
// constants, decodes them to bf16 in registers ([Digest] "方法步骤与流程" step 3 and
// [QLoRA note] "5. QLoRA 训练方式本身": the 4-bit weight is decoded to BF16 inside
// the operator) and stages the decoded tile in LDS next to the bf16 activation tile.
// The LoRA product (U . Bl^T or V . At^T) is added to the same fp32 accumulators as
// r extra contraction steps before the single bf16 rounding of the output.
//
// Tiling: a 256-thread workgroup computes a 256 x 256 output tile with four waves in
// a 2 x 2 arrangement (128 x 128 per wave: 4 x 4 tiles of the 32x32x16 MFMA).  The
// contraction advances 64 at a time through double-buffered LDS (row pitch 72 bf16,
// which keeps 16-byte fragment reads of 16 consecutive rows on distinct banks).
// Each weight element is decoded once per workgroup tile.
//
// Forward:  output [M, N], contraction over K.  Thread t decodes weight row n0 + t,
//           one 64-block (32 bytes of codes, one constant) per step: LDS layout [n][k].
// Backward: output [M, K], contraction over N.  Thread t decodes rows kt + 2p and
//           kt + 2p + 1 (p = t % 32) over 32 columns, and writes the two rows as bf16
//           pairs into LDS transposed, [k][n], so the MFMA reads 8 consecutive n.

#include "device_common.h"
#include "qlora_internal.h"

namespace qlora {
namespace {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int PITCH = BK + 8;  // bf16 elements per LDS row
constexpr int NT = 256;

struct GemmParams {
  const uint16_t *A;  // fwd: X [M, K]; bwd: dY [M, N]; pitch Kc
  WeightView w;
  const uint16_t *A2;  // U or V [M, r]
  const uint16_t *B2;  // fwd: Bl [N, r]; bwd: At [K, r]
  uint16_t *C;         // [M, No]
  int64_t M, No, Kc;
  int r;
  LevelTable lvl;  // NF4 codebook
};

// Load 8 consecutive bf16 of row `row` starting at column `col` of a [rows, cols]
// matrix with pitch `cols`; zero outside the matrix.  `vec_ok` = rows are 16-byte
// aligned (cols % 8 == 0).
__device__ __forceinline__ u32x4_t load8_bf16(const uint16_t *p, int64_t rows, int64_t cols,
                                              int64_t row, int64_t col, bool vec_ok) {
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

struct Prefetch {
  u32x4_t a[8];       // activation tile chunks
  u32x4_t code[2];    // packed codes
  float c[2];         // decoded block constants
};

template <bool BWD>
__device__ __forceinline__ void load_tile(const GemmParams &p, int64_t m0, int64_t n0, int64_t kt,
                                          bool a_vec, Prefetch &f) {
  const int tid = threadIdx.x;
  // activation tile [BM rows, BK cols]: 8 lanes per 128-byte row
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int ch = tid + i * NT;
    const int row = ch >> 3, c8 = ch & 7;
    f.a[i] = load8_bf16(p.A, p.M, p.Kc, m0 + row, kt + c8 * 8, a_vec);
  }
  const int64_t K = p.w.n_cols, N = p.w.n_rows;
  if (!BWD) {
    const int64_t n = n0 + tid;
    if (n < N) {
      const u32x4_t *src = reinterpret_cast<const u32x4_t *>(p.w.codes + n * (K / 2) + kt / 2);
      f.code[0] = src[0];
      f.code[1] = src[1];
      f.c[0] = decode_constant(p.w.absmax_q, p.w.dq_scale, p.w.dq_offset, (n * K + kt) >> 6);
    } else {
      f.code[0] = f.code[1] = u32x4_t{0u, 0u, 0u, 0u};
      f.c[0] = 0.0f;
    }
  } else {
    const int pr = tid & 31, kc = tid >> 5;
    const int64_t k = n0 + kc * 32;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int64_t n = kt + 2 * pr + h;
      if (n < N && k < K) {
        f.code[h] = *reinterpret_cast<const u32x4_t *>(p.w.codes + n * (K / 2) + k / 2);
        f.c[h] = decode_constant(p.w.absmax_q, p.w.dq_scale, p.w.dq_offset, (n * K + k) >> 6);
      } else {
        f.code[h] = u32x4_t{0u, 0u, 0u, 0u};
        f.c[h] = 0.0f;
      }
    }
  }
}

template <bool BWD>
__device__ __forceinline__ void store_tile(const Prefetch &f, uint16_t *sA, uint16_t *sB,
                                           const float *lut) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int ch = tid + i * NT;
    const int row = ch >> 3, c8 = ch & 7;
    *reinterpret_cast<u32x4_t *>(sA + row * PITCH + c8 * 8) = f.a[i];
  }
  if (!BWD) {
    uint16_t *dst = sB + tid * PITCH;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<u32x4_t *>(dst + (h * 4 + i) * 8) = decode8(f.code[h][i], f.c[0], lut);
  } else {
    const int pr = tid & 31, kc = tid >> 5;
    uint32_t *dst = reinterpret_cast<uint32_t *>(sB + (kc * 32) * PITCH) + pr;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t wa = f.code[0][i], wb = f.code[1][i];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float va = lut[(wa >> (4 * e)) & 15u] * f.c[0];
        const float vb = lut[(wb >> (4 * e)) & 15u] * f.c[1];
        dst[(i * 8 + e) * (PITCH / 2)] = pack_bf16x2(va, vb);
      }
    }
  }
}

template <bool BWD>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_kernel(
    GemmParams p) {
  __shared__ uint16_t sA[2][BM * PITCH];
  __shared__ uint16_t sB[2][BN * PITCH];
  __shared__ float lut[16];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t m0 = static_cast<int64_t>(blockIdx.x) * BM;
  const int64_t n0 = static_cast<int64_t>(blockIdx.y) * BN;
  if (tid < 16) lut[tid] = p.lvl.q[tid];

  const bool a_vec = (p.Kc % 8) == 0;
  const int nk = static_cast<int>((p.Kc + BK - 1) / BK);

  f32x16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  Prefetch f;
  load_tile<BWD>(p, m0, n0, 0, a_vec, f);
  __syncthreads();  // codebook in LDS
  store_tile<BWD>(f, sA[0], sB[0], lut);
  __syncthreads();

  for (int it = 0; it < nk; ++it) {
    const int cur = it & 1;
    if (it + 1 < nk) load_tile<BWD>(p, m0, n0, static_cast<int64_t>(it + 1) * BK, a_vec, f);
    const uint16_t *a_base = sA[cur] + (wm * 128 + (lane & 31)) * PITCH + (lane >> 5) * 8;
    const uint16_t *b_base = sB[cur] + (wn * 128 + (lane & 31)) * PITCH + (lane >> 5) * 8;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      u32x4_t a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a[i] = *reinterpret_cast<const u32x4_t *>(a_base + i * 32 * PITCH + ks * 16);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        b[j] = *reinterpret_cast<const u32x4_t *>(b_base + j * 32 * PITCH + ks * 16);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma32x32x16(a[i], b[j], acc[i][j]);
    }
    if (it + 1 < nk) store_tile<BWD>(f, sA[cur ^ 1], sB[cur ^ 1], lut);
    __syncthreads();
  }

  // LoRA up-projection as r extra contraction steps: acc += A2 . B2^T
  if (p.r > 0) {
    const bool r_vec = (p.r % 8) == 0;
    for (int rk = 0; rk < p.r; rk += 16) {
      const int64_t j0 = rk + (lane >> 5) * 8;
      u32x4_t a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a[i] = load8_bf16(p.A2, p.M, p.r, m0 + wm * 128 + i * 32 + (lane & 31), j0, r_vec);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        b[j] = load8_bf16(p.B2, p.No, p.r, n0 + wn * 128 + j * 32 + (lane & 31), j0, r_vec);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma32x32x16(a[i], b[j], acc[i][j]);
    }
  }

  // epilogue: one bf16 rounding per output element
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t col = n0 + wn * 128 + j * 32 + (lane & 31);
      if (col >= p.No) continue;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t row = m0 + wm * 128 + i * 32 + (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3);
        if (row < p.M) p.C[row * p.No + col] = to_bf16(acc[i][j][e]);
      }
    }
}

}  // namespace

static hipError_t launch_gemm(bool bwd, const GemmParams &p, hipStream_t stream) {
  const int64_t tm = (p.M + BM - 1) / BM, tn = (p.No + BN - 1) / BN;
  if (tm > 0x7fffffff || tn > 65535) return hipErrorInvalidValue;
  dim3 grid(static_cast<unsigned>(tm), static_cast<unsigned>(tn)), block(NT);
  if (bwd)
    hipLaunchKernelGGL(gemm_kernel<true>, grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL(gemm_kernel<false>, grid, block, 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_gemm_fwd(const WeightView &w, const uint16_t *X, int64_t M, const uint16_t *U,
                           const uint16_t *Bl, int r, uint16_t *Y, hipStream_t stream) {
  GemmParams p{X, w, U, Bl, Y, M, w.n_rows, w.n_cols, r, {}};
  for (int i = 0; i < 16; ++i) p.lvl.q[i] = codebook().q[i];
  return launch_gemm(false, p, stream);
}

hipError_t launch_gemm_dx(const WeightView &w, const uint16_t *dY, int64_t M, const uint16_t *V,
                          const uint16_t *At, int r, uint16_t *dX, hipStream_t stream) {
  GemmParams p{dY, w, V, At, dX, M, w.n_cols, w.n_rows, r, {}};
  for (int i = 0; i < 16; ++i) p.lvl.q[i] = codebook().q[i];
  return launch_gemm(true, p, stream);
}

}  // namespace qlora
