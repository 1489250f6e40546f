// LoRA merge / unmerge into a bf16 weight (gfx950).
//
// [Repro] "官方代码阅读路线": after training, the scaled low-rank update B A can be
// folded into the frozen weight and taken out again; [QLoRA note] (error added by
// merging): the target is a higher-precision copy of the base, here the bf16
// decode of the NF4 weight.  Per element, with scale = alpha / r:
//     merge:    out[n, k] = bf16_rne(W'[n, k] + RN(scale * D[n, k]))
//     unmerge:  out[n, k] = bf16_rne(Wm[n, k] - RN(scale * D[n, k]))
// where D = B A is accumulated in fp32 on the matrix cores and W' = bf16_rne(q * c')
// is the weight decode of the forward GEMM.
//
// HBM-bound (0.52 + 2 bytes per weight for the merge, 2 + 2 for the unmerge), so the
// kernel is laid out for bytes in flight.  A workgroup owns a 256-column strip of
// the output and walks 32-row tiles of it; wave w owns the strip's columns
// 64 w .. 64 w + 63.  At the start the strip of A (all r rows) is staged through LDS
// once and kept in registers as MFMA fragments (read with the transposing
// ds_read_b64_tr_b16).  Per tile a wave then
//   - runs the 32x32x16 MFMAs of this tile's D = B A (32 rows x 64 columns) on the
//     B fragments (rows n0 .. n0 + 31, all ranks) fetched two tiles earlier,
//   - passes D through its private LDS region so that each lane holds 8 consecutive
//     columns of a row, and adds it to the base decoded from codes (or Wm) fetched
//     two tiles earlier,
//   - issues the B fragments and the codes and constants of the tile after next,
//   - writes its 16 bytes per lane and pass.
// Every load and store is a buffer access at a straight-line position (offsets past
// the data read as zero and drop stores), so the wait counts stay exact and two
// tiles of loads and of stores stay in flight per wave.
//
// With r <= 64 and r % 8 == 0 (one rank chunk, 16-byte aligned B rows) the operands
// that every wave of a workgroup shares go through a shared stage instead: the tile's
// B rows, its block constants and (merge) the strip's codes are fetched by the whole
// workgroup in whole rows, one 16-byte piece per thread two tiles ahead, written to
// LDS at the start of the tile, and read back as MFMA fragments and per-lane codes
// after a barrier; a second barrier frees the stage for the next tile.  Per wave
// these loads had touched 32 rows each, and B and the constants were fetched by all
// four waves.

#include <type_traits>

#include "device_common.h"
#include "qlora_internal.h"

namespace qlora {
namespace {

constexpr int NT = 256;
constexpr int TR = 32;                 // rows per tile
constexpr int TC = 256;                // columns per strip (64 per wave)
constexpr int JC = 64;                 // ranks per staged chunk of A
constexpr int PA = TC * 2 + 64;        // A chunk pitch (bytes): rows 16 banks apart
constexpr int SA_BYTES = JC * PA;      // 36864
constexpr int PD = 64 * 4 + 16;        // per-wave D pitch (fp32 row of 64 columns)
constexpr int SD_WAVE = TR * PD;       // 8704
constexpr int SMEM = SA_BYTES > 4 * SD_WAVE ? SA_BYTES : 4 * SD_WAVE;
constexpr int PASSES = 4;              // 32 x 64 outputs per wave = 4 passes of 8 per lane
// Shared stage (r <= 64, r % 8 == 0): the tile's B rows (32 rows of 128 bytes, 16-byte
// chunks swizzled per row), its block constants (one word per row and wave) and, for
// the merge, the codes of the strip (32 rows of 128 bytes), loaded once per workgroup
// in whole rows after the four D regions
constexpr int SB_OFF = 4 * SD_WAVE;
constexpr int SB_BYTES = TR * 128;
constexpr int SC_OFF = SB_OFF + SB_BYTES;
constexpr int SC_BYTES = NT * 4;
constexpr int SK_OFF = SC_OFF + SC_BYTES;
constexpr int SK_BYTES = TR * 128;
constexpr int SMEM_LB = SA_BYTES > SK_OFF + SK_BYTES ? SA_BYTES : SK_OFF + SK_BYTES;


// Keeps the memory operations on each side where they are: the empty asm with a
// memory clobber orders them for the IR and instruction-selection passes, the
// scheduling barrier for the machine scheduler.
__device__ __forceinline__ void issue_fence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

struct MergeArgs {
  const uint8_t *codes;
  const int8_t *absmax_q;
  const float *dq_scale;
  const float *dq_offset;
  const float *absmax;  // fp32 block constants (weights without double quantization)
  const uint16_t *Wm;  // unmerge input (bf16 [N, K])
  const uint16_t *A;   // [r, K]
  const uint16_t *B;   // [N, r]
  uint16_t *out;       // [N, K]
  int64_t N, K;
  int r;
  int strips;          // ceil(K / 256)
  int tiles;           // ceil(N / 32)
  int per_strip;       // workgroups per strip
  float scale;
  LevelTable lvl;
};

// Per-tile buffer resources over rows n0 .. min(n0 + 32, N) - 1: offsets inside a
// tile fit 32 bits for any K, and rows past N (or a tile past the last) read zero.
struct TileRsrc {
  __amdgpu_buffer_rsrc_t codes, c8, s, o, wm, b, out;
};

template <int CT = kConstDqInt8>
__device__ __forceinline__ TileRsrc tile_rsrc(const MergeArgs &a, int tile, bool unmerge) {
  const int64_t n0 = static_cast<int64_t>(tile) * TR;
  const int64_t left = a.N - n0;
  // rows of the tile, 0 past the last one (32-bit selects keep this branch-free)
  const uint32_t rows = tile < a.tiles ? static_cast<uint32_t>(left < TR ? left : TR) : 0u;
  const int64_t e0 = n0 * a.K;  // first element of the tile
  const uint32_t kb = static_cast<uint32_t>(a.K);  // K < 2^26 is checked on the host
  TileRsrc t;
  if (unmerge) {
    t.wm = make_rsrc(a.Wm + e0, rows * kb * 2u);
    t.codes = t.c8 = t.s = t.o = t.wm;
  } else {
    const int64_t b0 = e0 >> 6, g0 = b0 >> 8;
    const uint32_t nb = rows * (kb / 64u);
    const uint32_t ng = nb == 0u ? 0u : ((static_cast<uint32_t>(b0 & 255) + nb + 255u) >> 8);
    t.codes = make_rsrc(a.codes + e0 / 2, rows * (kb / 2u));
    if constexpr (CT == kConstF32) {  // the tile's fp32 block constants
      t.c8 = t.s = t.o = make_rsrc(a.absmax + b0, nb * 4u);
    } else {
      t.c8 = make_rsrc(a.absmax_q + b0, nb);
      t.s = make_rsrc(a.dq_scale + g0, ng * 4u);
      t.o = make_rsrc(a.dq_offset + g0, ng * 4u);
    }
    t.wm = t.codes;
  }
  t.b = make_rsrc(a.B + n0 * a.r, rows * static_cast<uint32_t>(a.r) * 2u);
  t.out = make_rsrc(a.out + e0, rows * kb * 2u);
  return t;
}

// Base operands of one tile for this lane: pass p covers row 8 p + lane / 8 and
// columns c0 + 8 (lane % 8) .. + 7 of the strip (c0 = 64 wave + strip start), which
// lie in one 64-weight block.  The block's 8-bit constant is fetched as the aligned
// dword holding it (a 32-bit load keeps the value out of sub-dword extensions that
// the compiler would otherwise place, with a wait, at the top of the loop).
struct BaseStage {
  uint32_t code[PASSES];
  uint32_t c8w[PASSES], s[PASSES], o[PASSES];
  u32x4_t wm[PASSES];
};

// Per-lane offsets of the base operands inside any tile (the same for every tile, so
// they stay in registers across the tile loop): element e = (8 p + lane / 8) K + col.
struct LaneOffsets {
  uint32_t code[PASSES];  // byte offset of the 4 code bytes, or kOOB
  uint32_t wm[PASSES];    // byte offset of the 16 Wm bytes, or kOOB
  uint32_t blk[PASSES];   // block of e relative to the tile's first block
};

__device__ __forceinline__ LaneOffsets lane_offsets(const MergeArgs &a, int64_t col, bool col_ok) {
  const int lane = threadIdx.x & 63;
  LaneOffsets lo;
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int64_t e = static_cast<int64_t>(8 * p + (lane >> 3)) * a.K + col;
    lo.code[p] = col_ok ? static_cast<uint32_t>(e / 2) : kOOB;
    lo.wm[p] = col_ok ? static_cast<uint32_t>(e * 2) : kOOB;
    lo.blk[p] = static_cast<uint32_t>(e >> 6);
  }
  return lo;
}

template <bool UNMERGE, int CT>
__device__ __forceinline__ void issue_base(const MergeArgs &a, const TileRsrc &t, int tile,
                                           const LaneOffsets &lo, bool col_ok, BaseStage &st) {
  if (UNMERGE) {
#pragma unroll
    for (int p = 0; p < PASSES; ++p) st.wm[p] = buf_load16(t.wm, lo.wm[p]);
    return;
  }
  if constexpr (CT == kConstF32) {  // codes and the block's fp32 constant
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      st.code[p] = buf_load4(t.codes, lo.code[p]);
      st.s[p] = __builtin_amdgcn_raw_buffer_load_b32(t.s, col_ok ? lo.blk[p] * 4u : kOOB, 0, 0);
    }
    return;
  }
  // The 8-bit constants are read as the aligned dword holding each one (the tile's
  // first block is a multiple of 4).  Such a dword lies on the byte's own page, so
  // the read is safe even where the array ends mid-dword; lanes past the last block
  // (rows past the weight, whose outputs are dropped) read the last dword instead,
  // and a tile past the end reads the first.
  const int64_t total = a.N * a.K / 64;
  const int64_t b0 = (static_cast<int64_t>(tile) * TR * a.K) >> 6;  // tile's first block
  const bool live = b0 < total;
  const int8_t *cbase = a.absmax_q + (live ? b0 : 0);
  const uint32_t last = live ? static_cast<uint32_t>((total - 1 - b0) & ~int64_t(3)) : 0u;
  const uint32_t gb = static_cast<uint32_t>(b0 & 255);  // tile's first block inside its group
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const uint32_t g = (gb + lo.blk[p]) >> 8;  // group relative to the tile's first group
    st.code[p] = buf_load4(t.codes, lo.code[p]);
    st.c8w[p] = *reinterpret_cast<const uint32_t *>(cbase + min(lo.blk[p] & ~3u, last));
    st.s[p] = __builtin_amdgcn_raw_buffer_load_b32(t.s, col_ok ? g * 4 : kOOB, 0, 0);
    st.o[p] = __builtin_amdgcn_raw_buffer_load_b32(t.o, col_ok ? g * 4 : kOOB, 0, 0);
  }
}

// c' = fma(c8, s, o) of pass p; the constant's byte sits at byte (block % 4) of c8w,
// and tiles start on a multiple of four blocks, so the position depends on the lane only.
// Weights without double quantization hold c' itself in s.
template <int CT>
__device__ __forceinline__ float stage_constant(const BaseStage &st, int p, int byte) {
  if constexpr (CT == kConstF32) return __uint_as_float(st.s[p]);
  float c8;
  if constexpr (CT == kConstDqFp8)
    c8 = e4m3_value(st.c8w[p] >> (8 * byte));
  else
    c8 = static_cast<float>(static_cast<int>(st.c8w[p] << (24 - 8 * byte)) >> 24);
  return __builtin_fmaf(c8, __uint_as_float(st.s[p]), __uint_as_float(st.o[p]));
}

// The merge's base operands of one tile for this lane: row lane / 2, the 32 columns
// c0 + 32 (lane % 2) .. + 31 (c0 = 64 wave + strip start), half of one 64-weight block:
// one 16-byte code load and one constant per lane and tile (four passes of the per-pass
// layout would take sixteen small loads, and the loads' issue limited the kernel).
struct MergeStage {
  u32x4_t code;
  uint32_t c8w, s, o;
};
// LB: the codes and the block constant come from the workgroup's shared stage
// (issue_shared), so only the group scale and offset (double quantization) are loaded here.
template <int CT, bool LB>
__device__ __forceinline__ void issue_merge_base(const MergeArgs &a, const TileRsrc &t, int tile, uint32_t code16,
                                                 uint32_t blk16, bool col_ok, MergeStage &st) {
  if constexpr (!LB) st.code = buf_load16(t.codes, code16);
  if constexpr (CT == kConstF32) {
    if constexpr (!LB) st.s = __builtin_amdgcn_raw_buffer_load_b32(t.s, col_ok ? blk16 * 4u : kOOB, 0, 0);
    return;
  }
  if constexpr (LB) {
    const int64_t b0 = (static_cast<int64_t>(tile) * TR * a.K) >> 6;
    const uint32_t g = (static_cast<uint32_t>(b0 & 255) + blk16) >> 8;
    st.s = __builtin_amdgcn_raw_buffer_load_b32(t.s, col_ok ? g * 4 : kOOB, 0, 0);
    st.o = __builtin_amdgcn_raw_buffer_load_b32(t.o, col_ok ? g * 4 : kOOB, 0, 0);
    return;
  }
  // as in issue_base: the aligned dword holding the 8-bit constant, clamped to the array
  const int64_t total = a.N * a.K / 64;
  const int64_t b0 = (static_cast<int64_t>(tile) * TR * a.K) >> 6;
  const bool live = b0 < total;
  const int8_t *cbase = a.absmax_q + (live ? b0 : 0);
  const uint32_t last = live ? static_cast<uint32_t>((total - 1 - b0) & ~int64_t(3)) : 0u;
  const uint32_t g = (static_cast<uint32_t>(b0 & 255) + blk16) >> 8;
  st.c8w = *reinterpret_cast<const uint32_t *>(cbase + min(blk16 & ~3u, last));
  st.s = __builtin_amdgcn_raw_buffer_load_b32(t.s, col_ok ? g * 4 : kOOB, 0, 0);
  st.o = __builtin_amdgcn_raw_buffer_load_b32(t.o, col_ok ? g * 4 : kOOB, 0, 0);
}
// The block constant c' from the shared stage's word w (the fp32 constant, or the
// zero-extended 8-bit code) and the lane's group scale and offset.
template <int CT>
__device__ __forceinline__ float shared_constant(const MergeStage &st, uint32_t w) {
  if constexpr (CT == kConstF32) return __uint_as_float(w);
  return __builtin_fmaf(c8_value<CT>(w), __uint_as_float(st.s), __uint_as_float(st.o));
}
template <int CT>
__device__ __forceinline__ float merge_constant(const MergeStage &st, int byte) {
  if constexpr (CT == kConstF32) return __uint_as_float(st.s);
  float c8;
  if constexpr (CT == kConstDqFp8)
    c8 = e4m3_value(st.c8w >> (8 * byte));
  else
    c8 = static_cast<float>(static_cast<int>(st.c8w << (24 - 8 * byte)) >> 24);
  return __builtin_fmaf(c8, __uint_as_float(st.s), __uint_as_float(st.o));
}
constexpr int PO = 64 * 2 + 16;  // per-wave bf16 output tile pitch (bytes), in the D region
static_assert(TR * PO <= SD_WAVE, "output tile in the D region");

// B fragments of one tile: sub-step s (ranks 16 s .. 16 s + 15) of lane l holds
// B[n0 + l % 32][16 s + 8 (l / 32) .. + 7]; ranks past r read as zero.
template <int NCH, bool RVEC>
__device__ __forceinline__ void issue_b(const MergeArgs &a, const TileRsrc &t, u32x4_t (&bf)[4 * NCH]) {
  const int lane = threadIdx.x & 63;
  const uint32_t row = static_cast<uint32_t>(lane & 31) * a.r * 2;
#pragma unroll
  for (int s = 0; s < 4 * NCH; ++s) {
    const int j = 16 * s + 8 * (lane >> 5);
    if (RVEC) {
      bf[s] = buf_load16(t.b, j < a.r ? row + j * 2 : kOOB);
    } else {
      uint32_t h[8];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        h[e] = __builtin_amdgcn_raw_buffer_load_b16(t.b, j + e < a.r ? row + (j + e) * 2 : kOOB, 0, 0);
#pragma unroll
      for (int e = 0; e < 4; ++e) bf[s][e] = h[2 * e] | (h[2 * e + 1] << 16);
    }
  }
}

// Shared stage of one tile, one piece per thread: 16 bytes of the tile's B rows (chunk
// `tid` of the contiguous 32 r bf16, zero past the weight's last row or the tile) and,
// for the merge, the block constant of (row tid / 4, wave tid % 4), the 8-bit code or
// the fp32 constant (zero for tid >= 128 or columns past K), and 16 bytes of the strip's
// codes (row tid / 8, columns k0 + 32 (tid % 8) ..).  Every wave of the workgroup needs
// all of B's rows and all its rows' constants; loading them per wave took four times the
// loads, each touching 32 rows, where these touch whole rows; the codes, which each
// wave loaded as 32 rows x 32 bytes, now come in rows of 128 bytes.
template <int CT>
struct SharedStage {
  u32x4_t b, code;
  typename std::conditional<CT == kConstF32, uint32_t, uint8_t>::type c;  // 8-bit code kept 8-bit
};
template <bool UNMERGE, int CT>
__device__ __forceinline__ void issue_shared(const MergeArgs &a, const TileRsrc &t, int tile, int64_t k0,
                                             SharedStage<CT> &sh) {
  const int tid = threadIdx.x;
  sh.b = buf_load16(t.b, static_cast<uint32_t>(tid) * 16u);
  if constexpr (!UNMERGE) {
    const int64_t kc = k0 + 32 * (tid & 7);
    sh.code = buf_load16(t.codes, kc < a.K ? static_cast<uint32_t>(((tid >> 3) * a.K + kc) / 2) : kOOB);
    const int wv = tid & 3;
    const bool ok = tid < 4 * TR && k0 + 64 * wv < a.K;
    // the block relative to the tile's first block
    const uint32_t blk = static_cast<uint32_t>((static_cast<int64_t>(tid >> 2) * a.K + k0) >> 6) + wv;
    if constexpr (CT == kConstF32)
      sh.c = __builtin_amdgcn_raw_buffer_load_b32(t.s, ok ? blk * 4u : kOOB, 0, 0);
    else
      sh.c = __builtin_amdgcn_raw_buffer_load_b8(t.c8, ok ? blk : kOOB, 0, 0);
  }
  (void)tile;
}

// A fragment of sub-step s for the 32 columns starting at `cb` of a staged chunk:
// lane l receives column cb + l % 32 of rank rows 16 s + 8 (l / 32) .. + 7.  Within a
// 16-lane group, lane i reads row base + i / 4 at column 4 (i % 4) of its 16-column
// half and receives column i of four rows.
__device__ __forceinline__ u32x4_t afrag(const char *sa, int s, int cb) {
  const int lane = threadIdx.x & 63;
  const int i = lane & 15, g = lane >> 4;
  const int col = cb + (g & 1) * 16 + 4 * (i & 3);
  u32x4_t v;
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int row = 16 * s + 8 * (g >> 1) + 4 * e + (i >> 2);
    const v4i16_t t = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16_t *)(sa + row * PA + col * 2));
    const u32x2_t u = __builtin_bit_cast(u32x2_t, t);
    v[2 * e] = u[0];
    v[2 * e + 1] = u[1];
  }
  return v;
}

template <bool UNMERGE, bool RVEC, int NCH, int CT>
__global__ __launch_bounds__(NT) void merge_kernel(MergeArgs a) {
  // B rows of 16-byte aligned length and one rank chunk: B and the block constants go
  // through the workgroup's shared stage
  constexpr bool LB = RVEC && NCH == 1;
  __shared__ __attribute__((aligned(16))) char smem[LB ? SMEM_LB : SMEM];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int strip = blockIdx.x % a.strips;
  const int first = blockIdx.x / a.strips;  // this workgroup's tiles: first + i * per_strip
  const int64_t k0 = static_cast<int64_t>(strip) * TC;

  // ---- A strip -> register fragments, 64 ranks at a time ---------------------------
  u32x4_t af[4 * NCH][2];
  {
    const int kk = 8 * (tid & 31);
    const bool ok = k0 + kk < a.K;
    // A from column k0 on: r K - k0 elements (r K < 2^31 is checked on the host)
    const uint32_t a_bytes = __builtin_amdgcn_readfirstlane(
        a.r == 0 ? 0u : static_cast<uint32_t>((static_cast<int64_t>(a.r) * a.K - k0) * 2));
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(a.A + k0, a_bytes);
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      if (c > 0) __syncthreads();
#pragma unroll
      for (int q = 0; q < JC / 8; ++q) {
        const int jr = 8 * q + (tid >> 5);
        const int j = JC * c + jr;
        const uint32_t off = (ok && j < a.r) ? static_cast<uint32_t>((int64_t(j) * a.K + kk) * 2) : kOOB;
        *reinterpret_cast<u32x4_t *>(smem + jr * PA + kk * 2) = buf_load16(ra, off);
      }
      __syncthreads();
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int t = 0; t < 2; ++t) af[4 * c + s][t] = afrag(smem, s, 64 * wave + 32 * t);
    }
    __syncthreads();  // the staging area becomes the per-wave D regions
  }
  char *sd = smem + wave * SD_WAVE;

  // columns of this lane in the decode passes (strip-relative: c0 + 8 (lane % 8))
  const int64_t col = k0 + 64 * wave + 8 * (lane & 7);
  const bool col_ok = col < a.K;  // K % 64 == 0: a wave's 64 columns are all in or all out
  const int count = (a.tiles - first + a.per_strip - 1) / a.per_strip;

  auto tile_of = [&](int i) { return first + i * a.per_strip; };  // >= tiles: empty

  const LaneOffsets lo = lane_offsets(a, col, col_ok);
  // the merge's base layout: row lane / 2, columns colm .. colm + 31
  const int64_t colm = k0 + 64 * wave + 32 * (lane & 1);
  const int64_t em = static_cast<int64_t>(lane >> 1) * a.K + colm;
  const uint32_t code16 = col_ok ? static_cast<uint32_t>(em / 2) : kOOB;
  const uint32_t blk16 = static_cast<uint32_t>(em >> 6);
  using Stage = std::conditional_t<UNMERGE, BaseStage, MergeStage>;
  auto load_base = [&](const TileRsrc &t, int tile, Stage &st) {
    if constexpr (UNMERGE)
      issue_base<true, CT>(a, t, tile, lo, col_ok, st);
    else
      issue_merge_base<CT, LB>(a, t, tile, code16, blk16, col_ok, st);
  };
  Stage st0, st1;
  u32x4_t bf0[4 * NCH], bf1[4 * NCH];
  SharedStage<CT> sh0, sh1;
  // the shared stage: this thread's slot in the swizzled B tile (row x at x * 128,
  // chunk c at slot c ^ (x % 8), so that the 16-byte fragment reads of eight
  // consecutive rows fall in distinct banks); threads past the 4 r chunks write none
  const int rpc = a.r / 8;  // 16-byte chunks per B row
  const bool b_writer = LB && rpc > 0 && tid < 4 * a.r;
  const int bx = rpc > 0 ? tid / rpc : 0, bc = rpc > 0 ? tid - bx * rpc : 0;
  const int b_slot = SB_OFF + bx * 128 + ((bc ^ (bx & 7)) << 4);
  auto issue_stage = [&](const TileRsrc &t, int tile, u32x4_t (&bf)[4 * NCH], SharedStage<CT> &sh) {
    if constexpr (LB)
      issue_shared<UNMERGE, CT>(a, t, tile, k0, sh);
    else
      issue_b<NCH, RVEC>(a, t, bf);
  };
  {
    const TileRsrc t0 = tile_rsrc<CT>(a, tile_of(0), UNMERGE);
    const TileRsrc t1 = tile_rsrc<CT>(a, tile_of(1), UNMERGE);
    // same order as inside the loop (B, then base), so that the wait counts the
    // compiler derives for the loop entry match the steady state
    issue_stage(t0, tile_of(0), bf0, sh0);
    issue_fence();
    load_base(t0, tile_of(0), st0);
    issue_fence();
    issue_stage(t1, tile_of(1), bf1, sh1);
    issue_fence();
    load_base(t1, tile_of(1), st1);
    issue_fence();
  }

  // One tile i with the operands fetched two tiles earlier (st, bf).  Vector-memory
  // completions are counted in issue order, stores included, so a wait for a load
  // also waits for every store issued before it: the loads of tile i + 2 therefore go
  // out before the stores of tile i, which leaves two tiles of stores in flight per
  // wave.  The fences keep each group where it is issued.
  auto step = [&](int i, Stage &st, u32x4_t (&bf)[4 * NCH], SharedStage<CT> &sh) {
    uint32_t cword = 0;  // the lane's block constant from the shared stage (merge)
    if constexpr (LB) {
      // Publish the shared stage of tile i (fetched two tiles earlier); every wave has
      // read the previous tile's out of LDS (second barrier of the previous tile).
      if (b_writer) *reinterpret_cast<u32x4_t *>(smem + b_slot) = sh.b;
      if constexpr (!UNMERGE) {
        if constexpr (CT == kConstF32)
          *reinterpret_cast<uint32_t *>(smem + SC_OFF + 4 * tid) = sh.c;
        else
          *reinterpret_cast<uint8_t *>(smem + SC_OFF + tid) = sh.c;
        // row x = tid / 8 at x * 128, chunk c at slot c ^ (x & 6): the readers' eight
        // lanes (four rows, two chunks each) fall in distinct banks
        *reinterpret_cast<u32x4_t *>(smem + SK_OFF + (tid >> 3) * 128 + (((tid & 7) ^ ((tid >> 3) & 6)) << 4)) =
            sh.code;
      }
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      // B fragments: row l % 32, chunk 2 s + l / 32 (ranks 16 s + 8 (l / 32) ..); chunks
      // at or past r / 8 are zero
      const int x = lane & 31;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = 2 * q + (lane >> 5);
        const u32x4_t v = *reinterpret_cast<const u32x4_t *>(smem + SB_OFF + x * 128 + ((c ^ (x & 7)) << 4));
        bf[q] = c < rpc ? v : u32x4_t{0u, 0u, 0u, 0u};
      }
      if constexpr (!UNMERGE) {
        const int ci = 4 * (lane >> 1) + wave;  // (row lane / 2, this wave's block)
        if constexpr (CT == kConstF32)
          cword = *reinterpret_cast<const uint32_t *>(smem + SC_OFF + 4 * ci);
        else
          cword = *reinterpret_cast<const uint8_t *>(smem + SC_OFF + ci);
        // this lane's 32 codes: row lane / 2, chunk 2 wave + lane % 2
        const int kx = lane >> 1, kcn = 2 * wave + (lane & 1);
        st.code = *reinterpret_cast<const u32x4_t *>(smem + SK_OFF + kx * 128 + ((kcn ^ (kx & 6)) << 4));
      }
      // every wave holds its fragments and constant before the stage is replaced
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }
    f32x16_t acc[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[t][e] = 0.0f;
#pragma unroll
    for (int s = 0; s < 4 * NCH; ++s)
#pragma unroll
      for (int t = 0; t < 2; ++t) acc[t] = mfma32x32x16(af[s][t], bf[s], acc[t]);
    issue_fence();
    const TileRsrc tn = tile_rsrc<CT>(a, tile_of(i + 2), UNMERGE);
    issue_stage(tn, tile_of(i + 2), bf, sh);
    issue_fence();
    // acc[t][4 q + e]: row l % 32, wave column 32 t + 8 q + 4 (l / 32) + e
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = 32 * t + 8 * q + 4 * (lane >> 5);
        const f32x4_t v = {acc[t][4 * q], acc[t][4 * q + 1], acc[t][4 * q + 2], acc[t][4 * q + 3]};
        *reinterpret_cast<f32x4_t *>(sd + (lane & 31) * PD + c * 4) = v;
      }
    u32x4_t o[PASSES];
    if constexpr (UNMERGE) {
#pragma unroll
      for (int p = 0; p < PASSES; ++p) {
        const int row = 8 * p + (lane >> 3);
        const f32x4_t d0 = *reinterpret_cast<const f32x4_t *>(sd + row * PD + (lane & 7) * 32);
        const f32x4_t d1 = *reinterpret_cast<const f32x4_t *>(sd + row * PD + (lane & 7) * 32 + 16);
        const float d[8] = {d0[0], d0[1], d0[2], d0[3], d1[0], d1[1], d1[2], d1[3]};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const float t0 = a.scale * d[2 * h], t1 = a.scale * d[2 * h + 1];
          const float w0 = bf16_lo(st.wm[p][h]), w1 = bf16_hi(st.wm[p][h]);
          o[p][h] = pack_bf16x2(w0 - t0, w1 - t1);
        }
      }
    } else {
      // this lane's 32 columns of row lane / 2: the base from one plane table, D from
      // the D region; the bf16 results go back to the region (rows of PO bytes) and are
      // read out in the per-pass layout of the stores (8 rows x 128 bytes a pass)
      const int row = lane >> 1, half = lane & 1;
      const float cc =
          LB ? shared_constant<CT>(st, cword) : merge_constant<CT>(st, static_cast<int>(blk16 & 3u));
      const Planes pl = make_planes(cc, a.lvl);
      u32x4_t r4[4];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const f32x4_t d0 = *reinterpret_cast<const f32x4_t *>(sd + row * PD + (32 * half + 8 * w) * 4);
        const f32x4_t d1 = *reinterpret_cast<const f32x4_t *>(sd + row * PD + (32 * half + 8 * w) * 4 + 16);
        const float d[8] = {d0[0], d0[1], d0[2], d0[3], d1[0], d1[1], d1[2], d1[3]};
        const u32x4_t base = lookup8(st.code[w], pl);
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const float t0 = a.scale * d[2 * h], t1 = a.scale * d[2 * h + 1];
          r4[w][h] = pack_bf16x2(bf16_lo(base[h]) + t0, bf16_hi(base[h]) + t1);
        }
      }
      // the results overwrite D rows that other lanes read above: keep every read first
      // (one wave's LDS accesses complete in issue order)
      issue_fence();
#pragma unroll
      for (int w = 0; w < 4; ++w) *reinterpret_cast<u32x4_t *>(sd + row * PO + 64 * half + 16 * w) = r4[w];
#pragma unroll
      for (int p = 0; p < PASSES; ++p)
        o[p] = *reinterpret_cast<const u32x4_t *>(sd + (8 * p + (lane >> 3)) * PO + 16 * (lane & 7));
    }
    issue_fence();
    load_base(tn, tile_of(i + 2), st);
    issue_fence();
    const TileRsrc tc = tile_rsrc<CT>(a, tile_of(i), UNMERGE);
#pragma unroll
    for (int p = 0; p < PASSES; ++p) __builtin_amdgcn_raw_buffer_store_b128(o[p], tc.out, lo.wm[p], 0, 0);
    issue_fence();
  };

  for (int i = 0; i < count; i += 2) {
    step(i, st0, bf0, sh0);
    step(i + 1, st1, bf1, sh1);  // past the last tile: zero loads, dropped stores
  }
}

template <bool UNMERGE, bool RVEC, int NCH, int CT>
hipError_t launch_one(MergeArgs args, hipStream_t stream) {
  static int per_cu = -1;
  if (per_cu < 0) {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, merge_kernel<UNMERGE, RVEC, NCH, CT>, NT, 0) !=
            hipSuccess ||
        nb < 1)
      nb = 1;
    per_cu = nb;
  }
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    cus = 256;
  const int64_t slots = static_cast<int64_t>(per_cu) * cus;
  int64_t per_strip = (slots + args.strips - 1) / args.strips;
  if (per_strip > args.tiles) per_strip = args.tiles;
  if (per_strip < 1) per_strip = 1;
  args.per_strip = static_cast<int>(per_strip);
  const int64_t grid = per_strip * args.strips;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL((merge_kernel<UNMERGE, RVEC, NCH, CT>), dim3(static_cast<unsigned>(grid)), dim3(NT), 0,
                     stream, args);
  return hipGetLastError();
}

template <bool UNMERGE, int CT>
hipError_t launch(MergeArgs args, hipStream_t stream) {
  args.strips = static_cast<int>((args.K + TC - 1) / TC);
  args.tiles = static_cast<int>((args.N + TR - 1) / TR);
  const int nch = args.r == 0 ? 1 : (args.r + JC - 1) / JC;
  const bool rvec = args.r % 8 == 0;
#define QLORA_MERGE_CASE(C)                                                                        \
  case C:                                                                                          \
    return rvec ? launch_one<UNMERGE, true, C, CT>(args, stream) : launch_one<UNMERGE, false, C, CT>(args, stream);
  switch (nch) {
    QLORA_MERGE_CASE(1)
    QLORA_MERGE_CASE(2)
    QLORA_MERGE_CASE(3)
    QLORA_MERGE_CASE(4)
    default: return hipErrorInvalidValue;
  }
#undef QLORA_MERGE_CASE
}

}  // namespace

hipError_t launch_lora_merge(const WeightView &w, const uint16_t *A, const uint16_t *B, int r,
                             float scale, uint16_t *out, hipStream_t stream) {
  MergeArgs args{};
  args.codes = w.codes;
  args.absmax_q = w.absmax_q;
  args.dq_scale = w.dq_scale;
  args.dq_offset = w.dq_offset;
  args.absmax = w.absmax;
  args.A = A;
  args.B = B;
  args.out = out;
  args.N = w.n_rows;
  args.K = w.n_cols;
  args.r = r;
  args.scale = scale;
  args.lvl = level_table(w.quant_type);
  switch (w.const_type) {
    case kConstDqInt8: return launch<false, kConstDqInt8>(args, stream);
    case kConstDqFp8: return launch<false, kConstDqFp8>(args, stream);
    case kConstF32: return launch<false, kConstF32>(args, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_lora_unmerge(const uint16_t *Wm, int64_t n_rows, int64_t n_cols, const uint16_t *A,
                               const uint16_t *B, int r, float scale, uint16_t *out,
                               hipStream_t stream) {
  MergeArgs args{};
  args.Wm = Wm;
  args.A = A;
  args.B = B;
  args.out = out;
  args.N = n_rows;
  args.K = n_cols;
  args.r = r;
  args.scale = scale;
  return launch<true, kConstDqInt8>(args, stream);
}

}  // namespace qlora
