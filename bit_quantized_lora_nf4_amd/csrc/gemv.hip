// Small-M forward (M <= 16): a bandwidth-oriented dequant-GEMV (gfx950).
//
// Y[m, n] = bf16(sum_k X[m, k] W'[n, k] + sum_j U_s[m, j] Bl[n, j]),
// U_s = bf16(scale * X . A^T)  ([Paper note] "关键设计 3"; [Repro] "LoRA 的公式和张量形状").
//
// At such M the layer is bound by the weight stream (0.516 B per weight), so the work
// is cut into many independent pieces, each of which issues all of its loads at once:
//
//   stream kernel   workgroup (row group g, contraction slice s): 64 weight rows x
//                   1024 columns.  The slice of X (M rows, pre-permuted, see below) is
//                   staged in LDS once; each wave owns 16 rows, and lane l decodes the
//                   whole 64-weight blocks s * 16 + 4 i + l / 16 (i = 0..3) of row
//                   l % 16: one block constant, 32 bytes of codes, eight register
//                   lookups ([Digest] "数学公式与关键细节" item 3: w' = bf16(q[code] c')).
//                   The dot products run on 16x16x32 bf16 MFMA (tokens padded to 16),
//                   fp32 partial sums P[s][n][m] go to the workspace.  Extra workgroups
//                   of the same launch compute the LoRA down-projection partials
//                   UP[s][m][j] over the same slices.
//   finalize        per weight row: U_s from UP (summed in slice order, scaled, rounded
//                   once), then Y = bf16(sum_s P + U_s . Bl^T), one rounding.
//
// Decoded weights come out of the byte-permute lookup as bf16 pairs (e0,e2), (e4,e6),
// (e1,e3), (e5,e7) of each 8-element group; the X slice is staged with the same
// permutation inside every 8-element group, so the contraction pairs the right
// elements without re-interleaving the decoded weights.

#include <mutex>

#include "device_common.h"
#include "qlora_internal.h"

namespace qlora {
namespace {

constexpr int GT = 256;                  // threads per workgroup (4 waves)
constexpr int GROWS = 64;                // weight rows per workgroup, 16 per wave
#ifndef GEMV_GIT
#define GEMV_GIT 4
#endif
constexpr int GIT = GEMV_GIT;            // 64-blocks per lane and workgroup
constexpr int GSLICE = 4 * GIT * 64;     // contraction elements per workgroup (1024)
constexpr int XPITCH = GSLICE * 2 + 16;  // bytes per staged token row (padded)
constexpr int GMAXM = 16;

struct GemvArgs {
  WeightView w;
  const uint16_t *X;  // [M, K]
  const uint16_t *A;  // [r, K] (unused when r = 0)
  float *P;           // [S][N][M]
  float *UP;          // [S][M][r]
  int M, r, S;
  LevelTable lvl;
};

// Eight codes (element e in bits 4e..4e+3 of w) -> bf16 pairs (e0,e2), (e4,e6),
// (e1,e3), (e5,e7): the lookup of lookup8 without its final re-interleave.
__device__ __forceinline__ u32x4_t lookup8_pairs(uint32_t w, const Planes &P) {
  const uint32_t se = w & 0x07070707u;
  const uint32_t so = (w >> 4) & 0x07070707u;
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
  u32x4_t r;
  r[0] = __builtin_amdgcn_perm(He, Le, 0x05010400u);
  r[1] = __builtin_amdgcn_perm(He, Le, 0x07030602u);
  r[2] = __builtin_amdgcn_perm(Ho, Lo, 0x05010400u);
  r[3] = __builtin_amdgcn_perm(Ho, Lo, 0x07030602u);
  return r;
}

// An 8-element bf16 group x0..x7 in the element order of lookup8_pairs.
__device__ __forceinline__ u32x4_t permute8(u32x4_t d) {
  return u32x4_t{pack_lo(d[0], d[1]), pack_lo(d[2], d[3]), pack_hi(d[0], d[1]), pack_hi(d[2], d[3])};
}

// LDS of the stream kernel (one dynamic object): per wave its 16 rows x 512 bytes of
// codes (16-byte chunk cr of row r at slot cr ^ (r & 15)), per wave 16 rows x 16
// 8-bit block constants (or 16 fp32 constants for the type without double
// quantization), then the staged X slice (M rows of XPITCH bytes).
constexpr int CROW = 4 * GIT * 32;   // code bytes per row and slice (512)
constexpr int WCODE = 16 * CROW;     // code bytes per wave (8 KB)
constexpr int SC_BYTES = 4 * WCODE;  // 32 KB
constexpr int sq_wave(int ct) { return ct == kConstF32 ? 1024 : 256; }  // constant bytes per wave
int gemv_xl(int M) { return M <= 2 ? 1 : M <= 4 ? 2 : M <= 8 ? 4 : 8; }
// staged X rows = XL * 256 * 8 / GSLICE = 2 XL (rows past M hold zeros)
size_t gemv_lds_bytes(int M, int ct) {
  return SC_BYTES + 4 * sq_wave(ct) + static_cast<size_t>(2 * gemv_xl(M)) * XPITCH;
}

// XL: 16-byte X loads per thread (M * 128 / 256 rounded up to a power of two);
// C8W: the rows' int8 constants are dword aligned (K % 256 == 0).
template <int XL, bool C8W, int CT>
__global__ __launch_bounds__(GT) void gemv_stream_kernel(GemvArgs a) {
  constexpr int SQW = sq_wave(CT);
  extern __shared__ __attribute__((aligned(16))) char lds[];
  char *const sc = lds;
  char *const sq = lds + SC_BYTES;
  char *const sx = lds + SC_BYTES + 4 * SQW;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int N = static_cast<int>(a.w.n_rows), K = static_cast<int>(a.w.n_cols), KB = K / 64;
  const int lora_wgs = a.r > 0 ? a.S : 0;
  const int bid = blockIdx.x;
  const bool lora = bid < lora_wgs;
  const int s = lora ? bid : (bid - lora_wgs) % a.S;
  const int rg = lora ? 0 : (bid - lora_wgs) / a.S;
  const int k0 = s * GSLICE;
  const int ml = lane & 15, g = lane >> 4;
  const int row0 = rg * GROWS + wave * 16;  // first weight row of this wave

  // ---- issue every global load of the workgroup up front ----
  // X slice, tokens < M only (16-byte chunks; columns past K read as zero)
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.X, static_cast<uint32_t>(a.M) * K * 2);
  u32x4_t xs[XL];
#pragma unroll
  for (int j = 0; j < XL; ++j) {
    const int c = tid + j * GT;
    const int m = c / (GSLICE / 8), k = k0 + (c % (GSLICE / 8)) * 8;
    xs[j] = buf_load16(rx, (m < a.M && k < K) ? (static_cast<uint32_t>(m) * K + k) * 2 : kOOB);
  }
  uint32_t c8w = 0, sv[2] = {0u, 0u}, ov[2] = {0u, 0u}, cf[4] = {0u, 0u, 0u, 0u};
  uint8_t c8b[4] = {0, 0, 0, 0};
  int gfirst = 0;
  {
    // Straight-line for every workgroup (the LoRA ones read nothing: all offsets out of
    // range), so that the compiler's waits stay exact counts.  Order: constants, then
    // the codes block group by block group, so that decoding can follow the arrivals.
    const int nlim = lora ? 0 : N;
    const ConstRsrc rq = make_const_rsrc<CT>(a.w, static_cast<uint32_t>(uint64_t(N) * KB));
    // group scale and offset: the slice of one row spans at most two groups
    if constexpr (CT != kConstF32) {
      const int n = row0 + ml;
      const uint32_t bfirst = static_cast<uint32_t>(n) * KB + s * 16;
      gfirst = static_cast<int>(bfirst >> 8);
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const uint32_t og = n < nlim ? (bfirst / 256 + e) * 4u : kOOB;
        sv[e] = __builtin_amdgcn_raw_buffer_load_b32(rq.s, og, 0, 0);
        ov[e] = __builtin_amdgcn_raw_buffer_load_b32(rq.o, og, 0, 0);
      }
    }
    // 8-bit constants: lane l loads blocks s * 16 + 4 (l % 4) .. + 3 of row l / 4
    // (fp32 constants: the same blocks, one dword each)
    {
      const int n = row0 + (lane >> 2);
      const uint32_t b = static_cast<uint32_t>(n) * KB + s * 16 + 4 * (lane & 3);
      if constexpr (CT == kConstF32) {
#pragma unroll
        for (int e = 0; e < 4; ++e) cf[e] = __builtin_amdgcn_raw_buffer_load_b32(rq.s, n < nlim ? (b + e) * 4u : kOOB, 0, 0);
      } else if constexpr (C8W) {
        c8w = __builtin_amdgcn_raw_buffer_load_b32(rq.q8, n < nlim ? b : kOOB, 0, 0);
      } else {  // rows not dword aligned: four byte loads, stored to LDS one by one
#pragma unroll
        for (int e = 0; e < 4; ++e) c8b[e] = __builtin_amdgcn_raw_buffer_load_b8(rq.q8, n < nlim ? b + e : kOOB, 0, 0);
      }
    }
    // codes: for block group i (blocks 4 i .. 4 i + 3 of the slice, 128 bytes per row)
    // two 1 KB direct-to-LDS loads of 8 rows each; lane l fills slot l % 8 of row
    // 8 h + l / 8 with the row's 16-byte chunk (l % 8) ^ f(row), f(r) = (r / 2) % 8
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(a.w.codes, static_cast<uint32_t>(uint64_t(N) * K / 2));
    char *const wc = sc + wave * WCODE;
#pragma unroll
    for (int i = 0; i < GIT; ++i)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int rl = 8 * h + (lane >> 3);
        const int chunk = (lane & 7) ^ ((rl >> 1) & 7);
        const int n = row0 + rl;
        const int kbyte = s * CROW + i * 128 + chunk * 16;
        const uint32_t off = (n < nlim && kbyte < K / 2) ? static_cast<uint32_t>(n) * (K / 2) + kbyte : kOOB;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rc, (__attribute__((address_space(3))) void *)(wc + i * 2048 + h * 1024), 16, off, 0, 0, 0);
      }
    __builtin_amdgcn_sched_barrier(0);  // keep the issue order that the waits below count on
  }
  // ---- stage X (permuted per 8-element group) and the int8 constants in LDS ----
#pragma unroll
  for (int j = 0; j < XL; ++j) {  // staged rows past M (up to the power of two) are zero
    const int c = tid + j * GT;
    const int m = c / (GSLICE / 8), q = c % (GSLICE / 8);
    *reinterpret_cast<u32x4_t *>(sx + m * XPITCH + q * 16) = permute8(xs[j]);
  }
  if constexpr (CT == kConstF32) {
    *reinterpret_cast<u32x4_t *>(sq + wave * SQW + lane * 16) = u32x4_t{cf[0], cf[1], cf[2], cf[3]};
  } else if constexpr (C8W) {
    *reinterpret_cast<uint32_t *>(sq + wave * 256 + lane * 4) = c8w;
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) sq[wave * 256 + lane * 4 + e] = static_cast<char>(c8b[e]);
  }
  // the X slice is shared by the four waves; the codes are per wave and are waited
  // for block group by block group below
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

  const int xrow = ml < a.M ? ml : a.M - 1;  // tokens past M only feed unused outputs
  auto xfrag = [&](int kk) {  // B operand: token xrow, 8 elements at slice column kk
    return *reinterpret_cast<const u32x4_t *>(sx + xrow * XPITCH + kk * 2);
  };

  if (!lora) {
    // ---- weight stream: lane = (row ml of this wave's 16, lane group g) ----
    const char *const wc = sc + wave * WCODE + ml * 128;
    const u32x4_t q8 = *reinterpret_cast<const u32x4_t *>(sq + wave * SQW + ml * (SQW / 16));
    const int n = row0 + ml;
    f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int i = 0; i < GIT; ++i) {
      // block group i of this wave has landed: 2 (GIT - 1 - i) code loads remain
      static_assert(GIT == 4, "the waits below count two code loads per block group of four");
      if (i == 0) asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
      if (i == 1) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
      if (i == 2) asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
      if (i == 3) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      const int blk = 4 * i + g;  // block of the slice
      u32x4_t code[2];
#pragma unroll
      for (int h = 0; h < 2; ++h)
        code[h] = *reinterpret_cast<const u32x4_t *>(wc + i * 2048 + (((2 * g + h) ^ ((ml >> 1) & 7)) << 4));
      const int kk = blk * 64;
      u32x4_t xb[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) xb[t] = xfrag(kk + 8 * t);
      float cval;
      if constexpr (CT == kConstF32) {  // fp32 constant blk of the row's 16
        cval = *reinterpret_cast<const float *>(sq + wave * SQW + ml * 64 + blk * 4);
      } else {  // constant of block blk: byte g of dword i of the row's 16 bytes
        const int gi = static_cast<int>((static_cast<uint32_t>(n) * KB + s * 16 + blk) >> 8) - gfirst;
        const ConstRaw cr{(q8[i] >> (8 * g)) & 0xFFu, gi ? sv[1] : sv[0], gi ? ov[1] : ov[0]};
        cval = const_value<CT>(cr);
      }
      const Planes pl = make_planes(cval, a.lvl);
#pragma unroll
      for (int t = 0; t < 8; ++t) acc = mfma16x16x32(lookup8_pairs(code[t >> 2][t & 3], pl), xb[t], acc);
    }
    // lane holds rows 4 g + e of the wave's 16, token ml
    if (ml < a.M) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int nn = row0 + 4 * g + e;
        if (nn < N) a.P[(static_cast<int64_t>(s) * N + nn) * a.M + ml] = acc[e];
      }
    }
  } else {
    // ---- LoRA down-projection partials over this slice: wave w takes rank tiles w, w + 4, ...
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(a.A, static_cast<uint32_t>(a.r) * K * 2);
    for (int jt = wave; jt * 16 < a.r; jt += 4) {
      const int j = jt * 16 + ml;
      const bool jok = j < a.r;
      f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 4
      for (int st = 0; st < GSLICE / 32; ++st) {
        const int kk = st * 32 + 8 * g;
        const int k = k0 + kk;
        const u32x4_t av = buf_load16(ra, (jok && k < K) ? (static_cast<uint32_t>(j) * K + k) * 2 : kOOB);
        acc = mfma16x16x32(permute8(av), xfrag(kk), acc);
      }
      if (ml < a.M) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int jj = jt * 16 + 4 * g + e;
          if (jj < a.r) a.UP[(static_cast<int64_t>(s) * a.M + ml) * a.r + jj] = acc[e];
        }
      }
    }
  }
}

// Sum of x[0], x[stride], ..., x[(S - 1) stride] in that order, with the loads of
// eight terms in flight at a time (the additions stay in slice order).
__device__ __forceinline__ float ordered_sum(const float *__restrict__ x, int64_t stride, int S) {
  float sum = 0.0f;
  for (int s0 = 0; s0 < S; s0 += 8) {
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (s0 + e < S) ? x[(s0 + e) * stride] : 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (s0 + e < S) sum += v[e];
  }
  return sum;
}

constexpr int FT = 64;  // finalize threads per workgroup

// Y[m, n] = bf16(sum_s P[s][n][m] + sum_j U_s[m, q r + j] Bl[n, j]); U_s = bf16(scale * sum_s UP)
// over the R stacked ranks; q = n / part_rows is the part of a fused linear (0 for one).
__global__ __launch_bounds__(FT) void gemv_finalize_kernel(const float *__restrict__ P,
                                                           const float *__restrict__ UP, int S, int N,
                                                           int M, const uint16_t *__restrict__ Bl,
                                                           int r, int R, int part_rows, float scale,
                                                           uint16_t *__restrict__ Y,
                                                           uint16_t *__restrict__ U_saved) {
  __shared__ float us[GMAXM * kMaxRank];
  if (R > 0) {
    for (int e = threadIdx.x; e < M * R; e += FT) {
      const int m = e / R, j = e % R;
      const uint16_t u = to_bf16(scale * ordered_sum(UP + m * R + j, static_cast<int64_t>(M) * R, S));
      us[e] = bf16_to_f32(u);
      if (U_saved && blockIdx.x == 0) U_saved[m * R + j] = u;
    }
    __syncthreads();
  }
  const int n = blockIdx.x * FT + threadIdx.x;
  if (n >= N) return;
  const uint16_t *brow = Bl + static_cast<int64_t>(n) * r;
  const float *uq = us + (part_rows > 0 ? (n / part_rows) * r : 0);
  for (int m = 0; m < M; ++m) {
    float y = ordered_sum(P + static_cast<int64_t>(n) * M + m, static_cast<int64_t>(N) * M, S);
    if ((r & 7) == 0) {
      for (int j0 = 0; j0 < r; j0 += 8) {
        const u32x4_t bv = *reinterpret_cast<const u32x4_t *>(brow + j0);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          y = __builtin_fmaf(uq[m * R + j0 + 2 * e], bf16_lo(bv[e]), y);
          y = __builtin_fmaf(uq[m * R + j0 + 2 * e + 1], bf16_hi(bv[e]), y);
        }
      }
    } else {
      for (int j = 0; j < r; ++j) y = __builtin_fmaf(uq[m * R + j], bf16_to_f32(brow[j]), y);
    }
    Y[static_cast<int64_t>(m) * N + n] = to_bf16(y);
  }
}

}  // namespace

int gemv_slices(int64_t K) { return static_cast<int>((K + GSLICE - 1) / GSLICE); }

namespace {
size_t up256(size_t b) { return (b + 255) & ~size_t(255); }
float *gemv_p(void *ws) { return static_cast<float *>(ws); }
float *gemv_up(void *ws, int64_t M, int64_t K, int64_t N) {
  return reinterpret_cast<float *>(static_cast<char *>(ws) +
                                   up256(size_t(gemv_slices(K)) * size_t(N) * size_t(M) * 4));
}
}  // namespace

size_t gemv_workspace(int64_t M, int64_t K, int64_t N, int r) {
  const size_t S = static_cast<size_t>(gemv_slices(K));
  return up256(S * size_t(N) * size_t(M) * 4) + up256(S * size_t(M) * size_t(r) * 4);
}

bool gemv_supported(const WeightView &w, int64_t M, int r) {
  const int64_t N = w.n_rows, K = w.n_cols;
  return M >= 1 && M <= GMAXM && r >= 0 && r <= kMaxRank && N <= 0x7fffffff &&
         uint64_t(N) * K / 2 <= 0xFFFFFFF0ull && uint64_t(M) * K * 2 <= 0xFFFFFFF0ull &&
         uint64_t(r) * K * 2 <= 0xFFFFFFF0ull;
}

namespace {
// Dynamic LDS above 64 KB (M > 8) has to be allowed once per kernel instantiation
// (and per device); the flag is per instantiation and thread-safe.
template <int XL, bool C8W, int CT>
hipError_t allow_lds() {
  static std::once_flag once[64];
  static hipError_t err[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::call_once(once[dev], [&] {
    err[dev] = hipFuncSetAttribute(reinterpret_cast<const void *>(gemv_stream_kernel<XL, C8W, CT>),
                                   hipFuncAttributeMaxDynamicSharedMemorySize,
                                   static_cast<int>(gemv_lds_bytes(GMAXM, CT)));
  });
  return err[dev];
}

template <int XL, bool C8W, int CT>
hipError_t go_stream(const GemvArgs &a, unsigned grid, hipStream_t stream) {
  if (XL == 8) {
    const hipError_t e = allow_lds<XL, C8W, CT>();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((gemv_stream_kernel<XL, C8W, CT>), dim3(grid), dim3(GT), gemv_lds_bytes(a.M, CT), stream, a);
  return hipGetLastError();
}

template <int CT>
hipError_t launch_stream(const GemvArgs &a, unsigned grid, bool c8w, hipStream_t stream) {
  switch (gemv_xl(a.M) * 2 + (c8w ? 1 : 0)) {
    case 3: return go_stream<1, true, CT>(a, grid, stream);
    case 2: return go_stream<1, false, CT>(a, grid, stream);
    case 5: return go_stream<2, true, CT>(a, grid, stream);
    case 4: return go_stream<2, false, CT>(a, grid, stream);
    case 9: return go_stream<4, true, CT>(a, grid, stream);
    case 8: return go_stream<4, false, CT>(a, grid, stream);
    case 17: return go_stream<8, true, CT>(a, grid, stream);
    default: return go_stream<8, false, CT>(a, grid, stream);
  }
}
}  // namespace

hipError_t launch_gemv_stream(const WeightView &w, const uint16_t *X, int64_t M, const uint16_t *A,
                              int r, void *ws, hipStream_t stream) {
  if (!gemv_supported(w, M, r)) return hipErrorInvalidValue;
  const int64_t N = w.n_rows, K = w.n_cols;
  GemvArgs a;
  a.w = w;
  a.X = X;
  a.A = A;
  a.M = static_cast<int>(M);
  a.r = r;
  a.S = gemv_slices(K);
  a.P = gemv_p(ws);
  a.UP = gemv_up(ws, M, K, N);
  a.lvl = level_table(w.quant_type);
  const unsigned groups = static_cast<unsigned>((N + GROWS - 1) / GROWS);
  const unsigned grid = groups * static_cast<unsigned>(a.S) + (r > 0 ? static_cast<unsigned>(a.S) : 0u);
  const bool c8w = (K / 64) % 4 == 0;
  switch (w.const_type) {
    case kConstDqInt8: return launch_stream<kConstDqInt8>(a, grid, c8w, stream);
    case kConstDqFp8: return launch_stream<kConstDqFp8>(a, grid, c8w, stream);
    case kConstF32: return launch_stream<kConstF32>(a, grid, c8w, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemv_finalize(const WeightView &w, int64_t M, const uint16_t *Bl, int r, int R,
                                int64_t part_rows, float scale, uint16_t *Y, uint16_t *U_saved,
                                void *ws, hipStream_t stream) {
  if (!gemv_supported(w, M, R) || R < r || (part_rows > 0 && w.n_rows % part_rows != 0))
    return hipErrorInvalidValue;
  const int64_t N = w.n_rows, K = w.n_cols;
  hipLaunchKernelGGL(gemv_finalize_kernel, dim3(static_cast<unsigned>((N + FT - 1) / FT)), dim3(FT), 0,
                     stream, gemv_p(ws), gemv_up(ws, M, K, N), gemv_slices(K), static_cast<int>(N),
                     static_cast<int>(M), Bl, r, R, static_cast<int>(part_rows), scale, Y, U_saved);
  return hipGetLastError();
}

}  // namespace qlora
