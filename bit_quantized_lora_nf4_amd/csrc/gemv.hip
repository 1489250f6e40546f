// Small-M forward (M <= 16): a bandwidth-oriented dequant-GEMV in one launch (gfx950).
//
// Y[m, n] = bf16(sum_k X[m, k] W'[n, k] + sum_j U_s[m, q r + j] Bl[n, j]),
// U_s = bf16(scale * X . A^T)  ([Paper note] "关键设计 3"; [Repro] "LoRA 的公式和张量形状")
// with q the part of row n for horizontally fused linears (0 for one linear).
//
// At such M the layer is bound by the weight stream (0.516 B per weight) and by the VALU
// work of decoding it (about fifteen byte permutes per eight weights), so the launch is
// shaped to keep both busy from start to end:
//
//   weight waves      a row group per 16 weight rows, covering all of K; its W weight
//                     waves split K into contiguous block ranges of at most 4 T blocks
//                     (T steps).  Per step a wave decodes 16 rows x 4 blocks of 64: lane
//                     (row l % 16, group l / 16) loads the 32 bytes of codes of its block
//                     with two 16-byte loads straight into registers, forms
//                     c' = fma(c8, s, o) and the 16 table entries bf16(q[j] c') as byte
//                     planes, and turns each code dword into an MFMA operand with register
//                     byte-permute lookups ([Digest] "数学公式与关键细节" item 3).  The dot
//                     products run on 16x16x32 bf16 MFMA with tokens as the 16 columns
//                     (columns past M are never stored).  A workgroup holds one row group,
//                     or RG of them (one workgroup per CU) when X would not fit in LDS
//                     beside several workgroups; when X fits neither way and the grid
//                     is one workgroup per CU, each weight wave stages its own steps' X
//                     slices (two LDS stages per wave, loaded in whole 128-byte rows).
//                     It first stages X and its rows of the
//                     LoRA B in LDS, then each wave issues the loads of its first D steps
//                     (a register ring), so that decoding starts as soon as the first step
//                     has landed and the weight stream never drains; the compiler derives
//                     every wait from the register dependencies (for the per-wave X stages,
//                     from the LDS object each stage is).  W, T and RG are chosen on
//                     the host so that the busiest SIMD of the launch runs as few
//                     wave-steps as possible.  At the end each group adds its waves'
//                     partial sums in a fixed order through LDS, and the LoRA up-projection
//                     is one more MFMA per 32 ranks on the same accumulator, before the
//                     single bf16 rounding.
//   LoRA wave         one more wave per workgroup (R > 0) computes pieces of the
//                     down-projection X . A^T: 16 ranks over a slice of LB blocks of K,
//                     with X from the staged copy, and stores the piece's partial sums.
//                     U_s then reaches the weight waves one of two ways.  Counter
//                     hand-over (few partial sums): each piece counts itself on every
//                     workgroup's counter, and the LoRA wave of each workgroup waits for
//                     its own counter, adds the slices in order, rounds its part's U_s
//                     and puts it in LDS before the reduction barrier.  Ticket hand-over:
//                     the last piece of a rank tile to finish (an agent-scope ticket) adds
//                     the slices in order, rounds U_s and publishes it in copies; the last
//                     rank tile raises a flag per workgroup, which the weight waves poll
//                     in their epilogue.  The pieces live in the lowest workgroups of the
//                     grid, which are dispatched first, so that no wait is for a workgroup
//                     that cannot start.  Every counter and flag is returned to zero by
//                     its last user.
//
// Data handed between workgroups (the partial sums, U_s, the counters) is only ever
// written and read with agent-coherent accesses (the SC1 cache policy: the L2 of one XCD
// is not coherent with the others), and each hand-over waits for the writes to complete
// before the counter that publishes them is bumped.
//
// Decoded weights come out of the byte-permute lookup as bf16 pairs (e0,e2), (e4,e6),
// (e1,e3), (e5,e7) of each 8-element group; X is used with the same permutation inside
// every 8-element group, so the contraction pairs the right elements without
// re-interleaving the decoded weights.

#include <algorithm>
#include <mutex>
#include <type_traits>

#include "device_common.h"
#include "qlora_internal.h"

namespace qlora {
namespace {

constexpr int GMAXM = 16;
constexpr int kMaxWaves = 16;
// X from memory with one workgroup per CU (XDMA): each weight wave stages its own steps'
// X slices (M tokens x the step's 4 blocks, at most 8 KB) in two LDS stages of its own,
// loaded in whole 128-byte rows; at most kXdmaWaves weight waves per workgroup
constexpr int kXdmaWaves = 8;
constexpr int kXdmaStage = GMAXM * 4 * 128;
// LDS bytes of one token's staged X row: 128 per 64-element block plus 16 of padding, so
// that the rows of consecutive tokens start 16 bytes apart modulo 256 and the 16-byte
// reads of the sixteen token lanes fall in distinct banks
__host__ __device__ constexpr int xrow_bytes(int KB) { return KB * 128 + 16; }
constexpr uint32_t kSpinLimit = 1u << 20;
constexpr int kSC1 = 16;             // buffer cache policy: SC1 (agent-coherent access)
// counter words at the start of the workspace
constexpr int kSyncTiles = 1;        // rank tiles of U_s done
constexpr int kSyncTile0 = 2;        // per rank tile: slices done
constexpr int kMaxRankTiles = (kMaxRank + 15) / 16;
// then one "U_s is complete" word per workgroup, kFlagStride bytes apart: the LoRA wave
// that completes U_s raises all of them, and each workgroup polls its own and clears it
// once it has seen it, so that no address takes the polls or the updates of the whole
// grid (accesses to one address are served one after another)
constexpr int kFlagBase = 256, kFlagStride = 16, kMaxFlagWGs = 4096;
static_assert((kSyncTile0 + kMaxRankTiles) * 4 <= kFlagBase, "counter header");
static_assert(kFlagBase + kMaxFlagWGs * kFlagStride <= static_cast<int>(kGemvSyncBytes), "flags");
constexpr int kMaxUCopies = 64;
// DIRECT hand-over: slices of partial sums a LoRA wave loads at once, and the most
// memory round trips (element passes of 64 lanes x slice chunks) it may take
constexpr int kGatherChunk = 16, kGatherTrips = 2;
// with several row groups per workgroup a call runs longer, and the gather may take more
constexpr int kGatherTripsRG = 4;
// U_s is published in several copies too (at most this many bytes in all)
constexpr size_t kUCopyBudget = 128 * 1024;

struct GemvArgs {
  WeightView w;
  const uint16_t *X;    // [M, K]
  const uint16_t *A;    // [R, K] stacked adapters (R = 0: none)
  const uint16_t *Bl;   // [N, r]
  uint16_t *Y;          // [M, N]
  uint16_t *U_saved;    // [M, R] or NULL
  uint32_t *sync;       // counter words (see kSync*)
  uint16_t *Uc;         // NC copies of U_s, bf16 [M][16 PT] each, UCE elements apart
  float *PU;            // LoRA partial sums [PT][S][M][16]
  int NC, UCE;
  float scale;
  int M, R, r, part_rows;
  int W, T;             // weight waves per row group, steps of 4 blocks per weight wave
  int RG;               // row groups (16-row tiles) per workgroup, sharing the staged X
  int PT, SP, LB, G;    // rank tiles, pieces per rank tile and their 64-blocks, workgroups
  LevelTable lvl;
};

__device__ __forceinline__ u32x4_t load16_sc1(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kSC1));
}
__device__ __forceinline__ void store16_sc1(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4_t v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned int, v),
                                         r, off, 0, kSC1);
}
__device__ __forceinline__ void store8_sc1(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x2_t v) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(__attribute__((ext_vector_type(2))) unsigned int, v),
                                        r, off, 0, kSC1);
}

// Eight codes (element e in bits 4e..4e+3 of w) -> bf16 pairs (e0,e2), (e4,e6),
// (e1,e3), (e5,e7): the lookup of lookup8 without its final re-interleave.  The two
// eight-entry halves are merged with v_bitop3 (a full-rate operation on gfx950).
__device__ __forceinline__ u32x4_t lookup8_pairs(uint32_t w, const Planes &P) {
  const uint32_t se = w & 0x07070707u;
  const uint32_t so = (w >> 4) & 0x07070707u;
  const uint32_t me = __builtin_amdgcn_perm(w << 12, w << 4, 0x090B080Au);
  const uint32_t mo = __builtin_amdgcn_perm(w << 8, w, 0x090B080Au);
  const uint32_t Le = __builtin_amdgcn_bitop3_b32(me, __builtin_amdgcn_perm(P.L[3], P.L[2], se),
                                                   __builtin_amdgcn_perm(P.L[1], P.L[0], se), 0xCA);
  const uint32_t He = __builtin_amdgcn_bitop3_b32(me, __builtin_amdgcn_perm(P.H[3], P.H[2], se),
                                                   __builtin_amdgcn_perm(P.H[1], P.H[0], se), 0xCA);
  const uint32_t Lo = __builtin_amdgcn_bitop3_b32(mo, __builtin_amdgcn_perm(P.L[3], P.L[2], so),
                                                   __builtin_amdgcn_perm(P.L[1], P.L[0], so), 0xCA);
  const uint32_t Ho = __builtin_amdgcn_bitop3_b32(mo, __builtin_amdgcn_perm(P.H[3], P.H[2], so),
                                                   __builtin_amdgcn_perm(P.H[1], P.H[0], so), 0xCA);
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

// One wave step of the weight stream: the loads of one lane's block, and its eight X
// fragments when X is not staged in LDS.  The group scale and offset of the
// double-quantized constants are loaded once per wave (GroupConsts).
template <int CT, bool XLDS>
struct StepLoads {
  u32x4_t c0, c1;            // 32 bytes of codes
  // the block constant: the 8-bit code (kept 8-bit: a wider type is zero-extended where
  // the loads are issued, waiting for them), or the fp32 constant of kConstF32
  typename std::conditional<CT == kConstF32, uint32_t, uint8_t>::type q;
  u32x4_t x[XLDS ? 1 : 8];   // X[token][64 b + 8 u ..] (natural order)
};

// The group scale and offset of the first and of the last block of a wave's range (the
// range is at most 64 blocks, so it spans at most two groups of 256 blocks).
struct GroupConsts {
  uint32_t g0;               // group of the first block
  uint32_t s0, o0, s1, o1;
};
template <int CT>
__device__ __forceinline__ GroupConsts load_groups(const ConstRsrc &rq, uint32_t first, uint32_t last, bool ok) {
  GroupConsts gc{first >> 8, 0u, 0u, 0u, 0u};
  if constexpr (CT != kConstF32) {
    gc.s0 = __builtin_amdgcn_raw_buffer_load_b32(rq.s, ok ? (first >> 8) * 4u : kOOB, 0, 0);
    gc.o0 = __builtin_amdgcn_raw_buffer_load_b32(rq.o, ok ? (first >> 8) * 4u : kOOB, 0, 0);
    gc.s1 = __builtin_amdgcn_raw_buffer_load_b32(rq.s, ok ? (last >> 8) * 4u : kOOB, 0, 0);
    gc.o1 = __builtin_amdgcn_raw_buffer_load_b32(rq.o, ok ? (last >> 8) * 4u : kOOB, 0, 0);
  }
  return gc;
}

// The block-constant load of flat block b (zero when !ok).
template <int CT, bool XLDS>
__device__ __forceinline__ void load_constant(const ConstRsrc &rq, uint32_t b, bool ok, StepLoads<CT, XLDS> &st) {
  if constexpr (CT == kConstF32)
    st.q = __builtin_amdgcn_raw_buffer_load_b32(rq.s, ok ? b * 4u : kOOB, 0, 0);
  else
    st.q = __builtin_amdgcn_raw_buffer_load_b8(rq.q8, ok ? b : kOOB, 0, 0);
}

// c' of flat block b from its loaded pieces: fma(c8, s, o) rounded once ([Digest]
// "数学公式与关键细节" item 3), or the stored fp32 constant; 0 when !ok (blocks past the
// wave's range and rows past N add nothing).  The int8 code is sign-extended in floating
// point, (float)(byte ^ 0x80) - 128, which the compiler cannot fold into a sign-extending
// load placed next to this use.
template <int CT, bool XLDS>
__device__ __forceinline__ float constant_of(const StepLoads<CT, XLDS> &st, const GroupConsts &gc, uint32_t b,
                                             bool ok) {
  if constexpr (CT == kConstF32) return __uint_as_float(st.q);
  const bool first = (b >> 8) == gc.g0;
  const float s = __uint_as_float(first ? gc.s0 : gc.s1), o = __uint_as_float(first ? gc.o0 : gc.o1);
  float c8;
  if constexpr (CT == kConstDqFp8)
    c8 = e4m3_value(st.q);
  else
    c8 = static_cast<float>(static_cast<int>(st.q ^ 0x80u)) - 128.0f;
  return ok ? __builtin_fmaf(c8, s, o) : 0.0f;
}

// LDS layout (one dynamic object): the weight waves' partial sums [RG W][64 lanes][4]
// fp32, then (R > 0) the workgroup's 16 RG rows of Bl (bf16, row pitch r8 = r rounded up
// to 8, zeros past r), then, when X is staged, X [M] rows of xrow_bytes(KB) (each 64-element block
// permuted per 8-element group), then (DIRECT hand-over) the part's U_s
// [M][r8] bf16 (zeros past r).  The padded rows let every LoRA operand of the epilogue be
// one 16-byte read (a lane whose 8 ranks start past r reads nothing).
struct LdsPlan {
  int red, bt, x, u, total;
};
__host__ __device__ inline int up16(int b) { return (b + 15) & ~15; }
__host__ __device__ inline LdsPlan lds_plan(int nW, int M, int R, int r, int KB, bool xlds, bool direct, int RG) {
  LdsPlan p;
  p.red = 0;
  const int r8 = (r + 7) & ~7;
  p.bt = nW * 1024;
  p.x = p.bt + (R > 0 ? 32 * r8 * RG : 0);
  p.u = p.x + (xlds ? M * xrow_bytes(KB) : 0);
  p.total = p.u + (direct ? up16(2 * M * r8) : 0);
  return p;
}

// The f32x4 accumulators (this lane's) of waves 0 .. W - 1 added in wave order through
// LDS (one barrier).  The sum is valid in wave 0 (callers let the other waves return
// right after).
__device__ __forceinline__ f32x4_t reduce_waves(char *red, f32x4_t acc, int W, int wave, int lane) {
  *reinterpret_cast<f32x4_t *>(red + (wave * 64 + lane) * 16) = acc;
  __syncthreads();
  f32x4_t s = *reinterpret_cast<const f32x4_t *>(red + lane * 16);
  if (wave == 0) {
    for (int v = 1; v < W; ++v) {
      const f32x4_t t = *reinterpret_cast<const f32x4_t *>(red + (v * 64 + lane) * 16);
#pragma unroll
      for (int e = 0; e < 4; ++e) s[e] += t[e];
    }
  }
  return s;
}

// The LoRA wave of a workgroup: for each of its pieces p (rank tile t = p / SP, slice
// s = p % SP of LB 64-blocks of K) the partial sums of X . A^T for ranks [16 t, 16 t + 16),
// stored for the rank tile; the last piece of a tile to finish (an agent-scope ticket)
// adds the SP slices in order, rounds U_s = bf16(scale * sum) and publishes it in NC
// copies; the last tile raises every copy of the flag.  A lane (rank l % 16, group g)
// takes block b_lo + 4 i + g of step i, as a weight wave does; X comes from the
// workgroup's staged copy (then A is permuted like it) or from memory.
template <bool XLDS>
struct LoraLoads {
  static constexpr int STEPS = XLDS ? 2 : 1;  // steps of 4 blocks per piece (LB <= 4 STEPS)
  u32x4_t av[STEPS][8];
  u32x4_t xv[XLDS ? 1 : STEPS][8];
};

template <bool XLDS>
__device__ __forceinline__ LoraLoads<XLDS> lora_issue(const GemvArgs &a, int KB, int p) {
  constexpr int STEPS = LoraLoads<XLDS>::STEPS;
  const int lane = threadIdx.x & 63;
  const int ml = lane & 15, g = lane >> 4;
  const int K = KB * 64;
  const bool tok_ok = ml < a.M;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(a.A, static_cast<uint32_t>(a.R) * K * 2);
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.X, static_cast<uint32_t>(a.M) * K * 2);
  const int t = p / a.SP, s = p % a.SP;
  const int j = t * 16 + ml;  // rank (A row) of this lane's operand
  const int b_lo = s * a.LB, b_hi = min(KB, b_lo + a.LB);
  LoraLoads<XLDS> ll;
#pragma unroll
  for (int i = 0; i < STEPS; ++i) {
    const int b = b_lo + 4 * i + g;
    const bool ok = b < b_hi;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      ll.av[i][u] = buf_load16(ra, (ok && j < a.R) ? (static_cast<uint32_t>(j) * K + b * 64 + 8 * u) * 2 : kOOB);
      if constexpr (!XLDS)
        ll.xv[i][u] = buf_load16(rx, (ok && tok_ok) ? (static_cast<uint32_t>(ml) * K + b * 64 + 8 * u) * 2 : kOOB);
    }
  }
  return ll;
}

template <bool XLDS, bool DIRECT>
__device__ void lora_finish(const GemvArgs &a, const char *sx, int KB, int p, const LoraLoads<XLDS> &ll) {
  constexpr int STEPS = LoraLoads<XLDS>::STEPS;
  const int lane = threadIdx.x & 63;
  const int ml = lane & 15, g = lane >> 4;
  const bool tok_ok = ml < a.M;
  const int tok = tok_ok ? ml : 0;
  const uint32_t pu_bytes = static_cast<uint32_t>(a.PT) * a.SP * a.M * 64;
  const __amdgpu_buffer_rsrc_t rp = make_rsrc(a.PU, pu_bytes);
  const int RP = 16 * a.PT;
  const __amdgpu_buffer_rsrc_t ru = make_rsrc(a.Uc, static_cast<uint32_t>(a.NC) * a.UCE * 2);
  const int t = p / a.SP, s = p % a.SP;
  const int b_lo = s * a.LB, b_hi = min(KB, b_lo + a.LB);
  f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int i = 0; i < STEPS; ++i) {
    const int b = b_lo + 4 * i + g;
    const bool ok = b < b_hi;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if constexpr (XLDS) {
        // the staged X is permuted per 8-element group: permute A the same way
        const u32x4_t x = *reinterpret_cast<const u32x4_t *>(sx + tok * xrow_bytes(KB) + (ok ? b : 0) * 128 + u * 16);
        acc = mfma16x16x32(permute8(ll.av[i][u]), x, acc);
      } else {
        acc = mfma16x16x32(ll.av[i][u], ll.xv[i][u], acc);
      }
    }
  }
  // lane: token ml, ranks 16 t + 4 g + e; the piece's partial sums, then the ticket once
  // they have completed (agent-coherent loads of any workgroup then see them)
  if (tok_ok) store16_sc1(rp, (((t * a.SP + s) * a.M + ml) * 16 + 4 * g) * 4, __builtin_bit_cast(u32x4_t, acc));
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if constexpr (DIRECT) {
    // every workgroup's counter counts this piece once its partial sums have completed
    for (int w = lane; w < static_cast<int>(gridDim.x); w += 64)
      __hip_atomic_fetch_add(a.sync + (kFlagBase + w * kFlagStride) / 4, 1u, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  uint32_t ticket = 0;
  if (lane == 0)
    ticket = __hip_atomic_fetch_add(a.sync + kSyncTile0 + t, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  ticket = __builtin_amdgcn_readfirstlane(ticket);
  if (ticket != static_cast<uint32_t>(a.SP - 1)) return;
  // the last piece of the tile: add the slices in order
  float u4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int s0 = 0; s0 < a.SP; s0 += 8) {
    u32x4_t v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      v[i] = load16_sc1(rp, (tok_ok && s0 + i < a.SP) ? (((t * a.SP + s0 + i) * a.M + ml) * 16 + 4 * g) * 4 : kOOB);
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) u4[e] += __uint_as_float(v[i][e]);
  }
  if (tok_ok) {
    uint16_t ub[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) ub[e] = to_bf16(a.scale * u4[e]);
    const u32x2_t uv{ub[0] | (static_cast<uint32_t>(ub[1]) << 16), ub[2] | (static_cast<uint32_t>(ub[3]) << 16)};
    for (int c = 0; c < a.NC; ++c) store8_sc1(ru, (c * a.UCE + ml * RP + t * 16 + 4 * g) * 2, uv);
    if (a.U_saved) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int jj = t * 16 + 4 * g + e;
        if (jj < a.R) a.U_saved[ml * a.R + jj] = ub[e];
      }
    }
  }
  // count the tile done once every store of this wave (U_s, the reset counter) has
  // completed; the last tile raises the flags
  if (lane == 0) __hip_atomic_store(a.sync + kSyncTile0 + t, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  uint32_t tiles_done = 0;
  if (a.PT > 1) {
    if (lane == 0)
      tiles_done = __hip_atomic_fetch_add(a.sync + kSyncTiles, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    tiles_done = __builtin_amdgcn_readfirstlane(tiles_done);
  }
  if (tiles_done == static_cast<uint32_t>(a.PT - 1)) {
    // every rank tile is published: raise each workgroup's flag (the counter of done
    // tiles has no other user left in this call)
    if (a.PT > 1 && lane == 0) __hip_atomic_store(a.sync + kSyncTiles, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int w = lane; w < static_cast<int>(gridDim.x); w += 64)
      __hip_atomic_store(a.sync + (kFlagBase + w * kFlagStride) / 4, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// DIRECT hand-over (small M r SP): the LoRA wave of every workgroup waits until its own
// counter has counted all PT SP pieces, clears it for the next call, and forms the U_s
// columns of its part itself: U_s[m, j] = bf16(scale * sum over the slices, in slice
// order, of the partial sums), the same value the ticket path publishes.  It writes them
// to LDS ([M][r8] bf16, zeros past r) for the epilogue, and the first workgroup of the
// part also stores them to U_saved.
__device__ void gather_u(const GemvArgs &a, uint16_t *su, int n0) {
  const int lane = threadIdx.x & 63;
  uint32_t *cnt = a.sync + (kFlagBase + blockIdx.x * kFlagStride) / 4;
  const uint32_t want = static_cast<uint32_t>(a.PT * a.SP);
  for (uint32_t it = 0; it < kSpinLimit; ++it) {
    if (__hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= want) break;
    __builtin_amdgcn_s_sleep(1);
  }
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  if (lane == 0) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int q = a.part_rows > 0 ? n0 / a.part_rows : 0;
  const bool saver = a.U_saved && (a.part_rows > 0 ? n0 % a.part_rows == 0 : blockIdx.x == 0);
  const __amdgpu_buffer_rsrc_t rp = make_rsrc(a.PU, static_cast<uint32_t>(a.PT) * a.SP * a.M * 64);
  const int r8 = (a.r + 7) & ~7;
  const int n = a.M * r8;
  for (int e0 = 0; e0 < n; e0 += 64) {
    const int e = e0 + lane;
    const int m = e / r8, jr = e % r8;
    const bool ok = e < n && jr < a.r;
    const int j = q * a.r + (ok ? jr : 0);
    const int t = j >> 4, jj = j & 15;
    // the loads of up to kGatherChunk slices at once: one memory round trip per chunk
    float sum = 0.0f;
    for (int s0 = 0; s0 < a.SP; s0 += kGatherChunk) {
      uint32_t v[kGatherChunk];
#pragma unroll
      for (int i = 0; i < kGatherChunk; ++i)
        v[i] = __builtin_amdgcn_raw_buffer_load_b32(
            rp, (ok && s0 + i < a.SP) ? (((t * a.SP + s0 + i) * a.M + m) * 16 + jj) * 4 : kOOB, 0, kSC1);
#pragma unroll
      for (int i = 0; i < kGatherChunk; ++i)
        if (s0 + i < a.SP) sum += __uint_as_float(v[i]);
    }
    if (e < n) su[e] = ok ? to_bf16(a.scale * sum) : static_cast<uint16_t>(0);
    if (ok && saver) a.U_saved[m * a.R + j] = su[e];
  }
}

// One 16-byte piece per lane from a buffer straight into LDS (lane l at dst + 16 l).  A
// named function: called from a lambda of the kernel template, the builtin kept the host
// compilation from emitting those instantiations' launch stubs.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, char *dst, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)dst, 16, off, 0, 0, 0);
}

template <int CT, bool XLDS, bool MULTI, bool DIRECT, bool XDMA = false>
__global__ __launch_bounds__(kMaxWaves * 64) void gemv_kernel(GemvArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  // XDMA: the two X stages of every weight wave, separate objects so that the waits the
  // compiler derives for a stage's reads cover only that stage's loads
  __shared__ __attribute__((aligned(16))) char xst0[XDMA ? kXdmaWaves * kXdmaStage : 16];
  __shared__ __attribute__((aligned(16))) char xst1[XDMA ? kXdmaWaves * kXdmaStage : 16];
  static_assert(!(XLDS && XDMA), "X is staged for the workgroup or per wave, not both");
  constexpr int D = XLDS ? 4 : 2;  // steps whose loads are in flight (the register ring)
  constexpr bool XREG = !XLDS && !XDMA;  // X fragments loaded into registers with every step
  using Loads = StepLoads<CT, !XREG>;
  // RG row groups of W weight waves each; wave RG W (R > 0) is the LoRA wave
  const int W = a.W, RG = a.RG, nW = RG * W;
  const int N = static_cast<int>(a.w.n_rows), KB = static_cast<int>(a.w.n_cols / 64), K = KB * 64;
  const LdsPlan lp = lds_plan(nW, a.M, a.R, a.r, KB, XLDS, DIRECT, RG);
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ml = lane & 15, g = lane >> 4;
  const int grp = wave / W, wv = wave - grp * W;  // row group and wave within it
  const int n0w = static_cast<int>(blockIdx.x) * RG * 16;  // first row of the workgroup
  const int n0 = n0w + grp * 16;
  const int n = n0 + ml;  // weight row of this lane's operand
  const bool row_ok = n < N;
  const int tok = ml < a.M ? ml : 0;
  const bool tok_ok = ml < a.M;
  const int kb0 = (KB * wv) / W, kb1 = (KB * (wv + 1)) / W;
  const int Tw = (kb1 - kb0 + 3) / 4;  // this wave's steps (at most T)

  const uint32_t n_blocks = static_cast<uint32_t>(uint64_t(N) * KB);
  const __amdgpu_buffer_rsrc_t rc = make_rsrc(a.w.codes, static_cast<uint32_t>(uint64_t(N) * K / 2));
  const ConstRsrc rq = make_const_rsrc<CT>(a.w, n_blocks);
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.X, static_cast<uint32_t>(a.M) * K * 2);
  const uint32_t row_code = static_cast<uint32_t>(n) * (K / 2);
  const uint32_t row_blk = static_cast<uint32_t>(n) * KB;
  char *const sx = lds + lp.x;
  uint16_t *const sb = reinterpret_cast<uint16_t *>(lds + lp.bt);

  // 16-byte pieces staged into LDS: X (when staged) and the 16 rows of Bl (R > 0; a
  // contiguous 32 r bytes; Bl is read to its last element's whole dword).  They are
  // staged before the first weight load is issued: a load issued behind the weight
  // stream of the whole chip would arrive only when that stream has drained.
  if (wave == nW) {
    // The LoRA wave: it takes no part in the staging and issues the loads of its first
    // piece at once, ahead of the weight stream.  It passes the same two barriers as the
    // weight waves (the staging barrier and the one of the final reduction).
    const int npieces = a.PT * a.SP;
    LoraLoads<XLDS> ll;
    if (static_cast<int>(blockIdx.x) < npieces) ll = lora_issue<XLDS>(a, KB, blockIdx.x);
    __syncthreads();
    if (static_cast<int>(blockIdx.x) < npieces) lora_finish<XLDS, DIRECT>(a, lds + lp.x, KB, blockIdx.x, ll);
    if constexpr (MULTI) {
      // more pieces than workgroups (few output rows): the later ones one after another
      // (a separate instantiation: the loop costs the kernel about 35 registers)
      for (int p = blockIdx.x + gridDim.x; p < npieces; p += gridDim.x) {
        const LoraLoads<XLDS> lp2 = lora_issue<XLDS>(a, KB, p);
        lora_finish<XLDS, DIRECT>(a, lds + lp.x, KB, p, lp2);
      }
    }
    // DIRECT: U_s for the epilogue, in LDS before the reduction barrier
    if constexpr (DIRECT) gather_u(a, reinterpret_cast<uint16_t *>(lds + lp.u), n0w);
    __syncthreads();
    return;
  }
  const int nthr = 64 * nW, tid = threadIdx.x;
  const int xpieces = XLDS ? a.M * KB * 8 : 0;
  // Bl rows: 16-byte pieces when the rows are (r a multiple of 8), else element by element
  // into rows padded to r8
  const int r8 = (a.r + 7) & ~7;
  const int bpieces = (a.R > 0 && r8 == a.r) ? 2 * a.r * RG : 0;
  const uint32_t b_bytes = static_cast<uint32_t>((uint64_t(N) * a.r * 2 + 3) & ~uint64_t(3));
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(a.Bl, b_bytes);
  const uint32_t b_base = static_cast<uint32_t>(n0w) * a.r * 2;
  auto x_lds = [&](int c) { return sx + (c / (KB * 8)) * xrow_bytes(KB) + (c % (KB * 8)) * 16; };
  u32x4_t xs[2], bs[2];
  if constexpr (XLDS) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + i * nthr;
      xs[i] = buf_load16(rx, c < xpieces ? static_cast<uint32_t>(c) * 16 : kOOB);
    }
  }
  auto load_b = [&](int c) {
    const uint32_t off = b_base + static_cast<uint32_t>(c) * 16;
    if (c >= bpieces || off >= b_bytes) return u32x4_t{0u, 0u, 0u, 0u};
    if (off + 16 <= b_bytes) return buf_load16(rb, off);
    // the piece that runs past the end of Bl: dword by dword (each past the end reads 0)
    u32x4_t v;
#pragma unroll
    for (int h = 0; h < 4; ++h) v[h] = buf_load4(rb, off + 4 * h);
    return v;
  };
  if (bpieces > 0) {
#pragma unroll
    for (int i = 0; i < 2; ++i) bs[i] = load_b(tid + i * nthr);
  }
  const GroupConsts gc = load_groups<CT>(rq, row_blk + kb0, row_blk + kb1 - 1, row_ok);
  __builtin_amdgcn_sched_barrier(0);

  // the loads of step t (blocks past the wave's range, or rows past N, read zeros: their
  // constant decodes to c' = 0, so they add nothing)
  auto load = [&](int t) {
    Loads s;
    const int b = kb0 + 4 * t + g;
    const bool ok = row_ok && b < kb1;
    const uint32_t off = ok ? row_code + b * 32 : kOOB;
    s.c0 = buf_load16(rc, off);
    s.c1 = buf_load16(rc, ok ? off + 16 : kOOB);
    load_constant<CT, !XREG>(rq, row_blk + b, ok, s);
    if constexpr (XREG) {
      const uint32_t xo = (static_cast<uint32_t>(tok) * K + b * 64) * 2;
#pragma unroll
      for (int u = 0; u < 8; ++u) s.x[u] = buf_load16(rx, (tok_ok && b < kb1) ? xo + u * 16 : kOOB);
    }
    return s;
  };
  // XDMA: the wave's X slice of step t goes to its stage as rows (blk M + tok) of 128
  // bytes, the 16-byte chunk c of a row at slot c ^ (tok % 8) (the eight token lanes of a
  // read then fall in distinct banks); load q of the eight writes rows 8 q .. 8 q + 7,
  // lane l row 8 q + l / 8 and slot l % 8, so each covers eight whole 128-byte rows of X
  // (rows past 4 M and blocks past the wave's range read zero)
  uint32_t xq_off[XDMA ? 8 : 1];
  int xq_blk[XDMA ? 8 : 1];
  uint32_t xr_off[XDMA ? 8 : 1];
  if constexpr (XDMA) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int row = 8 * q + (lane >> 3);
      const int tk = row % a.M, c = (lane & 7) ^ (tk & 7);
      xq_off[q] = row < 4 * a.M ? (static_cast<uint32_t>(tk) * K + c * 8) * 2 : kOOB;
      xq_blk[q] = row / a.M;
    }
    // this lane's reads: token tok, block g of the step, chunk u
#pragma unroll
    for (int u = 0; u < 8; ++u)
      xr_off[u] = static_cast<uint32_t>(wave * kXdmaStage + (g * a.M + tok) * 128 + ((u ^ (tok & 7)) << 4));
  }
  auto issue_x = [&](int t, char *stage) {
    const int bp = kb0 + 4 * t;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const bool ok = xq_off[q] != kOOB && bp + xq_blk[q] < kb1;
      dma16(rx, stage + wave * kXdmaStage + q * 1024, ok ? xq_off[q] + static_cast<uint32_t>(bp + xq_blk[q]) * 128 : kOOB);
    }
  };
  f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
  auto compute = [&](const Loads &s, int t, const char *stage) {
    const int b = kb0 + 4 * t + g;
    const Planes pl = make_planes(constant_of<CT, !XREG>(s, gc, row_blk + b, row_ok && b < kb1), a.lvl);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint32_t cw = u < 4 ? s.c0[u] : s.c1[u - 4];
      u32x4_t xv;
      if constexpr (XLDS)
        xv = *reinterpret_cast<const u32x4_t *>(sx + tok * xrow_bytes(KB) + (b < kb1 ? b : kb0) * 128 + u * 16);
      else if constexpr (XDMA)
        xv = permute8(*reinterpret_cast<const u32x4_t *>(stage + xr_off[u]));
      else
        xv = permute8(s.x[u]);
      acc = mfma16x16x32(lookup8_pairs(cw, pl), xv, acc);
    }
  };

  // Each step's loads are issued together and in step order, after the staging barrier
  // and in the loop alike (the scheduling barriers keep the compiler from interleaving two steps'
  // loads), so every path into the loop head has the same D steps in flight and the
  // waits the compiler derives leave the later steps' loads in flight.
  if constexpr (XLDS) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + i * nthr;
      if (c < xpieces) *reinterpret_cast<u32x4_t *>(x_lds(c)) = permute8(xs[i]);
    }
    for (int c = tid + 2 * nthr; c < xpieces; c += nthr)
      *reinterpret_cast<u32x4_t *>(x_lds(c)) = permute8(buf_load16(rx, static_cast<uint32_t>(c) * 16));
  }
  if (bpieces > 0) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + i * nthr;
      if (c < bpieces) *reinterpret_cast<u32x4_t *>(sb + 8 * c) = bs[i];
    }
    for (int c = tid + 2 * nthr; c < bpieces; c += nthr) *reinterpret_cast<u32x4_t *>(sb + 8 * c) = load_b(c);
  } else if (a.R > 0) {
    for (int e = tid; e < 16 * RG * r8; e += nthr) {
      const int row = e / r8, j = e % r8;
      const bool ok = j < a.r && n0w + row < N;
      sb[e] = ok ? static_cast<uint16_t>(__builtin_amdgcn_raw_buffer_load_b16(
                       rb, static_cast<uint32_t>((n0w + row) * a.r + j) * 2, 0, 0))
                 : static_cast<uint16_t>(0);
    }
  }
  __syncthreads();
  Loads st[D];
  // XDMA: ring slot j's X stage (D = 2 there; j is a constant once the loops are unrolled)
  auto stage_of = [&](int j) -> char * { return j == 0 ? xst0 : xst1; };
#pragma unroll
  for (int j = 0; j < D; ++j) {
    st[j] = load(j);
    if constexpr (XDMA) issue_x(j, stage_of(j));
    __builtin_amdgcn_sched_barrier(0);
  }

  int t0 = 0;
  for (; t0 + D < Tw; t0 += D) {
#pragma unroll
    for (int j = 0; j < D; ++j) {
      compute(st[j], t0 + j, stage_of(j));
      __builtin_amdgcn_sched_barrier(0);
      st[j] = load(t0 + j + D);
      if constexpr (XDMA) issue_x(t0 + j + D, stage_of(j));
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int j = 0; j < D; ++j)
    if (t0 + j < Tw) compute(st[j], t0 + j, stage_of(j));

  f32x4_t y = reduce_waves(lds + lp.red + grp * W * 1024, acc, W, wv, lane);
  if (wv != 0) return;
  // lane: token ml, weight rows n0 + 4 g + e

  if (DIRECT && a.R > 0) {
    // U_s of this part is in LDS (the LoRA wave put it there before the barrier)
    const uint16_t *urow = reinterpret_cast<const uint16_t *>(lds + lp.u) + tok * r8;
    const uint16_t *brow = sb + (grp * 16 + ml) * r8;
    for (int c = 0; c < a.r; c += 32) {
      const int j0 = c + 8 * g;
      const bool in = j0 < a.r;
      u32x4_t bf = *reinterpret_cast<const u32x4_t *>(brow + (in ? j0 : 0));
      u32x4_t uf = *reinterpret_cast<const u32x4_t *>(urow + (in ? j0 : 0));
      if (!in) bf = u32x4_t{0u, 0u, 0u, 0u};
      if (!(in && tok_ok)) uf = u32x4_t{0u, 0u, 0u, 0u};
      y = mfma16x16x32(bf, uf, y);
    }
  } else if (a.R > 0) {
    // U_s from the LoRA waves: poll this workgroup's flag (and clear it for the next
    // call), then read this workgroup's copy of U_s (one row group per workgroup on this
    // path: the host takes several only with the DIRECT hand-over)
    uint32_t *flag = a.sync + (kFlagBase + blockIdx.x * kFlagStride) / 4;
    for (uint32_t it = 0; it < kSpinLimit; ++it) {
      if (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) break;
      __builtin_amdgcn_s_sleep(1);
    }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if (lane == 0) __hip_atomic_store(flag, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int RP = 16 * a.PT;
    const __amdgpu_buffer_rsrc_t ru = make_rsrc(a.Uc, static_cast<uint32_t>(a.NC) * a.UCE * 2);
    // Y += U_s[:, q r : q r + r] . Bl[rows]^T on the same accumulator: rows (the A
    // operand) from the staged Bl tile, tokens (the B operand) from U_s
    const int q = a.part_rows > 0 ? n0 / a.part_rows : 0;
    const bool aligned = (a.r & 7) == 0;
    const uint16_t *brow = sb + (grp * 16 + ml) * r8;
    const uint32_t ubase = static_cast<uint32_t>((blockIdx.x % a.NC) * a.UCE + tok * RP + q * a.r);
    for (int c = 0; c < a.r; c += 32) {
      const int j0 = c + 8 * g;
      u32x4_t bf = *reinterpret_cast<const u32x4_t *>(brow + (j0 < a.r ? j0 : 0));
      if (j0 >= a.r) bf = u32x4_t{0u, 0u, 0u, 0u};
      u32x4_t uf = u32x4_t{0u, 0u, 0u, 0u};
      if (tok_ok && j0 < a.r) {
        if (aligned) {
          uf = load16_sc1(ru, (ubase + j0) * 2);
        } else {
#pragma unroll
          for (int h = 0; h < 4; ++h) {
            const int j = j0 + 2 * h;
            const uint32_t lo = j < a.r ? __builtin_amdgcn_raw_buffer_load_b16(ru, (ubase + j) * 2, 0, kSC1) : 0u;
            const uint32_t hi =
                j + 1 < a.r ? __builtin_amdgcn_raw_buffer_load_b16(ru, (ubase + j + 1) * 2, 0, kSC1) : 0u;
            uf[h] = lo | (hi << 16);
          }
        }
      }
      y = mfma16x16x32(bf, uf, y);
    }
  }
  if (tok_ok) {
    const int nb = n0 + 4 * g;
    uint16_t *yr = a.Y + static_cast<int64_t>(ml) * N;
    if (nb + 3 < N && (N & 3) == 0) {
      *reinterpret_cast<u32x2_t *>(yr + nb) = u32x2_t{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (nb + e < N) yr[nb + e] = to_bf16(y[e]);
    }
  }
}

// Weight waves per workgroup (W) and steps per weight wave (T).  A launch of G tiles puts
// at most c = ceil(G / 256) workgroups on one CU; its busiest SIMD runs ceil(c W / 4)
// weight waves of T = ceil(ceil(KB / W) / 4) steps each, the decode time of the launch.
// W minimises that product (a lone wave per SIMD counts 30% more: it cannot hide its own
// dependency chains), within the waves a CU holds at once (`max_cu_waves`, counting the
// LoRA wave of each workgroup, `extra`), preferring fewer steps.
struct GemvShape {
  int W, T;
};
GemvShape gemv_shape(int64_t N, int64_t K, int max_cu_waves, int extra) {
  const int64_t tiles = (N + 15) / 16, KB = K / 64;
  const int64_t c = (tiles + 255) / 256;
  GemvShape best{1, static_cast<int>((KB + 3) / 4)};
  double best_cost = 1e30;
  for (int W = 1; W + extra <= kMaxWaves; ++W) {
    if (W > 1 && (c * (W + extra) > max_cu_waves || W > KB)) break;
    const int64_t T = ((KB + W - 1) / W + 3) / 4;
    const int64_t per_simd = (c * W + 3) / 4;
    const double cost = double(per_simd * T) * (per_simd == 1 ? 1.3 : 1.0);
    if (cost < best_cost - 1e-9 || (cost < best_cost + 1e-9 && T < best.T)) {
      best_cost = cost;
      best = {W, static_cast<int>(T)};
    }
  }
  return best;
}

// Row groups of W weight waves in workgroups of RG tiles, one workgroup per CU: W
// minimises the busiest SIMD's wave-steps within the 16 waves of a workgroup.
GemvShape gemv_shape_rg(int64_t K, int RG, int extra) {
  const int64_t KB = K / 64;
  GemvShape best{1, static_cast<int>((KB + 3) / 4)};
  double best_cost = 1e30;
  for (int W = 1; RG * W + extra <= kMaxWaves && W <= KB; ++W) {
    const int64_t T = ((KB + W - 1) / W + 3) / 4;
    const int64_t per_simd = (RG * W + 3) / 4;
    const double cost = double(per_simd * T) * (per_simd == 1 ? 1.3 : 1.0);
    if (cost < best_cost - 1e-9 || (cost < best_cost + 1e-9 && T < best.T)) {
      best_cost = cost;
      best = {W, static_cast<int>(T)};
    }
  }
  return best;
}

// LDS bytes a workgroup may use: the 160 KB of a CU shared among the workgroups that one
// round of the grid (of `wgs` workgroups) puts on it.
int lds_budget(int64_t wgs) {
  const int64_t per_cu = (wgs + 255) / 256;
  return static_cast<int>((160 * 1024) / (per_cu < 1 ? 1 : per_cu));
}

// The launch configuration: shape, whether X is staged in LDS, LDS bytes, and the LoRA
// pieces: about 16 slices of LB 64-blocks per rank tile (LB at most 8 with X staged,
// 4 without: the blocks whose loads a LoRA wave keeps in flight at once).
struct GemvPlan {
  GemvShape sh;
  int RG;       // row groups per workgroup
  bool xlds;
  bool xdma;    // X not staged for the workgroup: each weight wave stages its own steps' X
  bool direct;  // U_s handed over through per-workgroup counters (gather_u)
  int lds_bytes;
  int LB, SP;
};
// LoRA pieces: about 16 slices of LB 64-blocks per rank tile.
void lora_slices(GemvPlan &p, int KB) {
  const int lb_max = p.xlds ? 8 : 4;
  p.LB = (KB + 15) / 16;
  if (p.LB > lb_max) p.LB = lb_max;
  p.SP = (KB + p.LB - 1) / p.LB;
}
// In the DIRECT hand-over the LoRA wave of every workgroup loads its part's M r SP
// partial sums (r <= R): taken when that costs at most `trips` memory round trips; else
// the last piece of each rank tile publishes U_s once.
bool gather_ok(int64_t M, int R, int SP, int trips) {
  const int64_t passes = (M * ((R + 7) & ~7) + 63) / 64, chunks = (SP + kGatherChunk - 1) / kGatherChunk;
  return R > 0 && passes * chunks <= trips;
}
// Depends on (M, K, N, R) alone (and on whether several row groups may share a
// workgroup), so that the workspace size is known before the call (the Bl tile is taken
// at its largest, r = R, for the choice of staging X).
GemvPlan gemv_plan(int64_t M, int64_t K, int64_t N, int R, bool allow_rg = true) {
  const int KB = static_cast<int>(K / 64);
  const int extra = R > 0 ? 1 : 0;
  const int64_t tiles = (N + 15) / 16;
  GemvPlan p;
  p.RG = 1;
  p.xdma = false;
  // staged X: about 100 VGPRs (5 waves per SIMD); X from memory: about 130 (4)
  p.sh = gemv_shape(N, K, 20, extra);
  p.xlds = lds_plan(p.sh.W, static_cast<int>(M), R, R, KB, true, true, 1).total <= lds_budget(tiles);
  // X too large to stage beside several workgroups per CU: workgroups of RG tiles, one
  // per CU, share one staged copy (they need the DIRECT hand-over: the ticket path polls
  // a flag per workgroup from each row group's leader)
  const int rg = static_cast<int>((tiles + 255) / 256);
  if (!p.xlds && allow_rg && rg > 1 && rg <= 4) {
    GemvPlan q = p;
    q.RG = rg;
    q.sh = gemv_shape_rg(K, rg, extra);
    q.xlds = true;
    lora_slices(q, KB);
    if (lds_plan(rg * q.sh.W, static_cast<int>(M), R, R, KB, true, true, rg).total <= 160 * 1024 &&
        (R == 0 || gather_ok(M, R, q.SP, kGatherTripsRG)))
      p = q;
  }
  // X from memory: with one workgroup per CU (at most 256 tiles) and two or more tokens,
  // each of at most kXdmaWaves weight waves stages its own X slices in LDS (the X
  // fragment loads of the other layout touch 64 rows of X each)
  p.xdma = !p.xlds && tiles <= 256 && M >= 2;
  if (!p.xlds) p.sh = gemv_shape(N, K, p.xdma ? kXdmaWaves + extra : 16, extra);
  lora_slices(p, KB);
  p.direct = gather_ok(M, R, p.SP, p.RG > 1 ? kGatherTripsRG : kGatherTrips);
  p.lds_bytes = lds_plan(p.RG * p.sh.W, static_cast<int>(M), R, R, KB, p.xlds, p.direct, p.RG).total;
  return p;
}

size_t up256(size_t b) { return (b + 255) & ~size_t(255); }

// Copies of U_s [M][16 PT] bf16 published by the LoRA waves.
int gemv_u_copies(int64_t M, int R) {
  const size_t ub = static_cast<size_t>(M) * ((R + 15) / 16) * 32;
  if (ub == 0) return 1;
  const size_t c = kUCopyBudget / ub;
  return static_cast<int>(c < 1 ? 1 : c > kMaxUCopies ? kMaxUCopies : c);
}

}  // namespace

// Layout: the counter / flag header, the NC copies of U_s, the LoRA partial sums.
size_t gemv_workspace(int64_t M, int64_t K, int64_t N, int r) {
  const size_t PT = static_cast<size_t>((r + 15) / 16);
  // a fused call whose parts do not align with the row groups falls back to one group
  const size_t SP = static_cast<size_t>(std::max(gemv_plan(M, K, N, r).SP, gemv_plan(M, K, N, r, false).SP));
  const size_t NC = static_cast<size_t>(gemv_u_copies(M, r));
  return kGemvSyncBytes + NC * up256(static_cast<size_t>(M) * PT * 16 * 2) + up256(PT * SP * M * 16 * 4);
}

bool gemv_supported(const WeightView &w, int64_t M, int r) {
  const int64_t N = w.n_rows, K = w.n_cols;
  return gemv_shape_ok(M, N) && M <= GMAXM && r >= 0 && r <= kMaxRank && (N + 15) / 16 <= kMaxFlagWGs &&
         uint64_t(N) * K / 2 <= 0xFFFFFFF0ull && uint64_t(M) * K * 2 <= 0xFFFFFFF0ull &&
         uint64_t(r) * K * 2 <= 0xFFFFFFF0ull && uint64_t(N) * (K / 64) <= 0xFFFFFFF0ull &&
         uint64_t(N) * r * 2 + 4 <= 0xFFFFFFF0ull;
}

namespace {
template <int CT, bool XLDS, bool MULTI, bool DIRECT, bool XDMA = false>
hipError_t go_gemv1(const GemvArgs &a, int lds_bytes, hipStream_t stream) {
  if (lds_bytes > 64 * 1024) {
    static std::once_flag once[64];
    static hipError_t err[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::call_once(once[dev], [&] {
      err[dev] = hipFuncSetAttribute(reinterpret_cast<const void *>(gemv_kernel<CT, XLDS, MULTI, DIRECT, XDMA>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    });
    if (err[dev] != hipSuccess) return err[dev];
  }
  hipLaunchKernelGGL((gemv_kernel<CT, XLDS, MULTI, DIRECT, XDMA>), dim3(static_cast<unsigned>(a.G)),
                     dim3(64 * (a.RG * a.W + (a.R > 0 ? 1 : 0))),
                     static_cast<size_t>(lds_bytes), stream, a);
  return hipGetLastError();
}
template <int CT, bool XLDS>
hipError_t go_gemv(const GemvArgs &a, bool direct, bool xdma, int lds_bytes, hipStream_t stream) {
  const bool multi = a.PT * a.SP > a.G;
  if constexpr (!XLDS) {
    // the XDMA layout with one row group and at most kXdmaWaves weight waves
    if (xdma && a.RG == 1 && a.W <= kXdmaWaves) {
      if (direct)
        return multi ? go_gemv1<CT, false, true, true, true>(a, lds_bytes, stream)
                     : go_gemv1<CT, false, false, true, true>(a, lds_bytes, stream);
      return multi ? go_gemv1<CT, false, true, false, true>(a, lds_bytes, stream)
                   : go_gemv1<CT, false, false, false, true>(a, lds_bytes, stream);
    }
  }
  if (direct)
    return multi ? go_gemv1<CT, XLDS, true, true>(a, lds_bytes, stream)
                 : go_gemv1<CT, XLDS, false, true>(a, lds_bytes, stream);
  return multi ? go_gemv1<CT, XLDS, true, false>(a, lds_bytes, stream)
               : go_gemv1<CT, XLDS, false, false>(a, lds_bytes, stream);
}
}  // namespace

hipError_t launch_gemv(const WeightView &w, const uint16_t *X, int64_t M, const uint16_t *A, int R,
                       const uint16_t *Bl, int r, int64_t part_rows, float scale, uint16_t *Y,
                       uint16_t *U_saved, void *ws, hipStream_t stream) {
  if (!gemv_supported(w, M, R) || R < r || (part_rows > 0 && (w.n_rows % part_rows != 0 || part_rows % 16 != 0)))
    return hipErrorInvalidValue;
  const int64_t N = w.n_rows, K = w.n_cols;
  GemvPlan p = gemv_plan(M, K, N, R);
  // the row groups of a workgroup must lie in one part (they share its U_s)
  if (p.RG > 1 && part_rows > 0 && part_rows % (16 * p.RG) != 0) p = gemv_plan(M, K, N, R, false);
  GemvArgs a;
  a.w = w;
  a.X = X;
  a.A = A;
  a.Bl = Bl;
  a.Y = Y;
  a.U_saved = U_saved;
  a.sync = static_cast<uint32_t *>(ws);
  a.PT = (R + 15) / 16;
  a.NC = gemv_u_copies(M, R);
  a.UCE = static_cast<int>(up256(size_t(M) * a.PT * 16 * 2) / 2);
  a.Uc = reinterpret_cast<uint16_t *>(static_cast<char *>(ws) + kGemvSyncBytes);
  a.PU = reinterpret_cast<float *>(static_cast<char *>(ws) + kGemvSyncBytes + size_t(a.NC) * a.UCE * 2);
  a.scale = scale;
  a.M = static_cast<int>(M);
  a.R = R;
  a.r = r;
  a.part_rows = static_cast<int>(part_rows);
  a.W = p.sh.W;
  a.RG = p.RG;
  a.T = p.sh.T;
  a.LB = p.LB;
  a.SP = R > 0 ? p.SP : 0;
  a.G = static_cast<int>(((N + 15) / 16 + p.RG - 1) / p.RG);
  a.lvl = level_table(w.quant_type);
  switch (w.const_type) {
    case kConstDqInt8:
      return p.xlds ? go_gemv<kConstDqInt8, true>(a, p.direct, false, p.lds_bytes, stream)
                    : go_gemv<kConstDqInt8, false>(a, p.direct, p.xdma, p.lds_bytes, stream);
    case kConstDqFp8:
      return p.xlds ? go_gemv<kConstDqFp8, true>(a, p.direct, false, p.lds_bytes, stream)
                    : go_gemv<kConstDqFp8, false>(a, p.direct, p.xdma, p.lds_bytes, stream);
    case kConstF32:
      return p.xlds ? go_gemv<kConstF32, true>(a, p.direct, false, p.lds_bytes, stream)
                    : go_gemv<kConstF32, false>(a, p.direct, p.xdma, p.lds_bytes, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qlora
