// Fused NF4-decode GEMMs on bf16 MFMA (gfx950): the forward Y = X W'^T + U Bl^T
// and the input gradient dX = dY W' + V At^T.
//
// W' is never written to HBM: the kernels stream packed 4-bit codes plus int8 block
// constants and decode them to bf16 on the fly ([Digest] "方法步骤与流程" step 3 and
// [QLoRA note] "5. QLoRA 训练方式本身": the 4-bit weight is decoded to BF16 inside
// the operator): w' = bf16_rne(q[code] * c'), c' = fma(c8, s, o).  The LoRA product
// is added to the same fp32 accumulators as r extra contraction steps (before the
// weight's) ahead of the single bf16 rounding of each output.
//
// Tile: a 256-thread workgroup (four waves, one per SIMD) computes a 256 x 256 output
// tile, 256 fp32 accumulators per lane.  In the forward, wave w owns all 256
// activation rows and output columns [64 w, 64 w + 64), i.e. 8 x 2 tiles of the
// 32x32x16 MFMA; in dX the waves split the tile 2 x 2 (4 x 4 MFMA tiles each).  The
// MFMA "A" operand is the weight side (rows = output columns) and "B" the activation
// side (columns = tokens), so each lane ends with 4 consecutive output columns of one
// token: 8-byte stores.  The contraction advances 64 at a time.
//
// Activation tiles (X or dY, 256 rows x 64) are staged in LDS (a three-deep ring in
// the forward, two stages in dX) with an XOR swizzle of the eight 16-byte chunks of
// each 128-byte row, chunk c of row r at slot c ^ f(r), f(r) = (r & 7) ^ ((r >> 3) & 1):
// the 16-byte fragment reads of 16 consecutive rows hit distinct banks for either 32
// or 64 LDS banks.
//
// Decode: per block constant c a lane builds the 16 possible outputs
// bf16_rne(q[j] * c) as byte planes in registers and looks codes up with byte
// permutes (no LDS table; about four VALU instructions per weight).
//
// Forward: the weight operand is decoded privately per lane straight into MFMA
// fragments (lane l of wave w: weight rows 64 w + 32 j + l % 32, contraction half
// l / 32 of each 64-step, i.e. one 16-byte code load and one block constant per row
// and step); no weight bytes touch LDS.  The contraction order inside a step is
// permuted identically on both operands (lane half h takes k in [32 h, 32 h + 32)).
// Backward: the contraction runs over weight rows, so the 64 x 256 weight tile is
// decoded cooperatively into LDS in its natural row-major layout (16-byte chunk c of
// row n at slot c ^ g(n), with g(n) = (n1, n0, n1 ^ n3, n2) in the bits of n) and read
// with the gfx950 transposing LDS read ds_read_b64_tr_b16, which hands each lane four
// consecutive weight rows of one column; the dY tiles come through LDS like the
// forward's activations, and the four waves split the output tile 2 x 2.

#include "device_common.h"
#include "qlora_internal.h"

namespace qlora {
namespace {

constexpr int NT = 256;
constexpr int TM = 256, TN = 256, TK = 64;
#ifndef LORA_RQ
#define LORA_RQ 4
#endif
constexpr int TILE_BYTES = TM * TK * 2;  // 32 KB per staged operand tile

struct GemmParams {
  const uint16_t *A;  // fwd: X [M, K]; bwd: dY [M, N]; row length Kc
  WeightView w;
  const uint16_t *A2;  // U or V [M, r]
  const uint16_t *B2;  // fwd: Bl [N, r]; bwd: At [K, r]
  uint16_t *C;         // [M, No]
  int M, No, Kc, r;
  LevelTable lvl;  // NF4 codebook
  int lda2;       // row pitch of A2 (r, or the stacked rank of fused linears)
  int part_rows;  // fused linears: output columns [q P, q P + P) use A2 columns
                  // [q r, q r + r); 0 = one linear (tiles never straddle parts)
  int tiles;         // dX: workgroups [0, tiles) compute output tiles; the fin_wgs after
  int fin_wgs;       // them do the finalize job `fin` (the dA pass of the same backward)
  FinalizeJob fin;
};

__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

// byte offset of 16-byte chunk c of row `row` in a swizzled 256 x 64 bf16 tile
__device__ __forceinline__ int tile_off(int row, int c) { return row * 128 + ((c ^ swz(row)) << 4); }

// ---- activation tile staging: 256 rows x 64 columns, 8 chunks of 16 B per thread ----
struct ActStage {
  u32x4_t v[8];
};

// thread t handles rows (t >> 3) + 32 i, chunk t & 7
__device__ __forceinline__ void act_load(__amdgpu_buffer_rsrc_t rs, int m0, int M, int Kc, int kt,
                                         bool vec, const uint16_t *base, ActStage &st) {
  const int tid = threadIdx.x;
  const int c = tid & 7;
  const int col = kt + c * 8;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = m0 + (tid >> 3) + 32 * i;
    if (vec) {
      const bool ok = row < M && col < Kc;
      st.v[i] = buf_load16(rs, ok ? (static_cast<uint32_t>(row) * Kc + col) * 2 : kOOB);
    } else {
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (row < M) {
        const uint16_t *src = base + static_cast<int64_t>(row) * Kc;
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const uint32_t lo = (col + e < Kc) ? src[col + e] : 0u;
          const uint32_t hi = (col + e + 1 < Kc) ? src[col + e + 1] : 0u;
          v[e / 2] = lo | (hi << 16);
        }
      }
      st.v[i] = v;
    }
  }
}

__device__ __forceinline__ void act_store(char *s, const ActStage &st) {
  const int tid = threadIdx.x;
  const int c = tid & 7;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = (tid >> 3) + 32 * i;
    *reinterpret_cast<u32x4_t *>(s + tile_off(row, c)) = st.v[i];
  }
}

__device__ __forceinline__ void zero_acc(f32x16_t (&acc)[8][2]) {
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
}

// One MFMA operand fragment of a LoRA matrix: 8 consecutive ranks j0 .. j0 + 7 of row
// `row` (row pitch ld elements); rows past `rows` and ranks past r read as zero.  With
// 16-byte aligned rows it is one 16-byte load, else eight 2-byte loads; both are
// straight-line buffer loads.
__device__ __forceinline__ u32x4_t lora_frag(__amdgpu_buffer_rsrc_t rs, bool vec, int row, int rows, int ld,
                                             int j0, int r) {
  const bool ok = row < rows;
  if (vec) return buf_load16(rs, (ok && j0 < r) ? (static_cast<uint32_t>(row) * ld + j0) * 2 : kOOB);
  u32x4_t v;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int j = j0 + 2 * e;
    const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(
        rs, (ok && j < r) ? (static_cast<uint32_t>(row) * ld + j) * 2 : kOOB, 0, 0);
    const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b16(
        rs, (ok && j + 1 < r) ? (static_cast<uint32_t>(row) * ld + j + 1) * 2 : kOOB, 0, 0);
    v[e] = lo | (hi << 16);
  }
  return v;
}

// LoRA steps: acc[i][j] += A2 rows (tokens) x B2 rows (output columns), r in steps of 16.
// LORA_RQ rank steps at a time: every fragment load of a chunk is issued before its
// first MFMA, so the chunk pays one memory latency instead of one per 16 ranks.
__device__ __forceinline__ void lora_steps(const GemmParams &p, int m0, int c0,
                                           f32x16_t (&acc)[8][2]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = p.r, lda2 = p.lda2;
  const bool vec = (r % 8) == 0 && (lda2 % 8) == 0;
  // fused linears: this tile's part picks its rank columns of A2
  const uint16_t *const A2 = p.A2 + (p.part_rows > 0 ? (c0 / p.part_rows) * r : 0);
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(A2, static_cast<uint32_t>(uint64_t(p.M) * lda2 * 2));
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.B2, static_cast<uint32_t>(uint64_t(p.No) * r * 2));
  constexpr int RQ = LORA_RQ;
  for (int r0 = 0; r0 < r; r0 += 16 * RQ) {
    u32x4_t wa[RQ][2], xb[RQ][8];
#pragma unroll
    for (int q = 0; q < RQ; ++q) {
      const int j0 = r0 + 16 * q + (lane >> 5) * 8;
#pragma unroll
      for (int j = 0; j < 2; ++j) wa[q][j] = lora_frag(rb, vec, c0 + wave * 64 + j * 32 + (lane & 31), p.No, r, j0, r);
#pragma unroll
      for (int i = 0; i < 8; ++i) xb[q][i] = lora_frag(ra, vec, m0 + i * 32 + (lane & 31), p.M, lda2, j0, r);
    }
#pragma unroll
    for (int q = 0; q < RQ; ++q) {
      if (r0 + 16 * q < r) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) acc[i][j] = mfma32x32x16(wa[q][j], xb[q][i], acc[i][j]);
      }
    }
  }
}

// Epilogue: lane holds token m = m0 + 32 i + l % 32 and output columns
// c0 + 64 w + 32 j + 8 g + 4 (l / 32) + 0..3 for g = 0..3.
__device__ __forceinline__ void store_out(const GemmParams &p, int m0, int c0,
                                          const f32x16_t (&acc)[8][2]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const bool vec = (p.No % 4) == 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int m = m0 + i * 32 + (lane & 31);
    if (m >= p.M) continue;
    uint16_t *row = p.C + static_cast<int64_t>(m) * p.No;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = c0 + wave * 64 + j * 32 + g * 8 + (lane >> 5) * 4;
        const f32x16_t &a = acc[i][j];
        if (vec) {
          if (col < p.No) {
            u32x2_t o = {pack_bf16x2(a[4 * g], a[4 * g + 1]), pack_bf16x2(a[4 * g + 2], a[4 * g + 3])};
            *reinterpret_cast<u32x2_t *>(row + col) = o;
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (col + e < p.No) row[col + e] = to_bf16(a[4 * g + e]);
        }
      }
  }
}

// The same epilogue through LDS, for outputs with 16-byte aligned rows (No % 8 == 0):
// each wave stages its 256 x 64 output block in two halves of 128 tokens (rows of 136
// bytes, so that the 32 token rows of a lane half's 8-byte writes fall in distinct
// banks) and writes it back 8 rows x 128 bytes per store instruction, where the
// register layout would give 32 pieces of 16 bytes.  `lds` holds 4 x 128 x 136 bytes
// that no wave reads any more.
constexpr int kOutPitch = 136;
__device__ __forceinline__ void store_out_lds(const GemmParams &p, int m0, int c0, const f32x16_t (&acc)[8][2],
                                              char *lds) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  char *const reg = lds + wave * (128 * kOutPitch);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int ii = 0; ii < 4; ++ii)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x16_t &a = acc[4 * h + ii][j];
          const int tok = ii * 32 + (lane & 31), col = j * 32 + g * 8 + (lane >> 5) * 4;
          const u32x2_t o = {pack_bf16x2(a[4 * g], a[4 * g + 1]), pack_bf16x2(a[4 * g + 2], a[4 * g + 3])};
          *reinterpret_cast<u32x2_t *>(reg + tok * kOutPitch + col * 2) = o;
        }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the wave's writes have landed
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int tok = 8 * q + (lane >> 3), ch = lane & 7;
      const u32x2_t lo = *reinterpret_cast<const u32x2_t *>(reg + tok * kOutPitch + ch * 16);
      const u32x2_t hi = *reinterpret_cast<const u32x2_t *>(reg + tok * kOutPitch + ch * 16 + 8);
      const int m = m0 + 128 * h + tok, col = c0 + wave * 64 + ch * 8;
      if (m < p.M && col < p.No)
        *reinterpret_cast<u32x4_t *>(p.C + static_cast<int64_t>(m) * p.No + col) = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // read back before the next half overwrites it
  }
}

// Map the linear workgroup id to (token tile, output tile): workgroups are dispatched
// round-robin over the 8 XCDs, so consecutive tiles of the grouped raster order are
// given to the same XCD (sharing its L2); groups of 4 token tiles sweep the outputs.
__device__ __forceinline__ void tile_coords(int tiles_m, int tiles_n, int &tm, int &tn) {
  const int T = tiles_m * tiles_n;
  int b = blockIdx.x;
  if ((T & 7) == 0) b = (b & 7) * (T >> 3) + (b >> 3);
  constexpr int G = 4;
  const int group = b / (G * tiles_n);
  const int first = group * G;
  const int gsize = min(tiles_m - first, G);
  const int in = b - group * G * tiles_n;
  tm = first + in % gsize;
  tn = in / gsize;
}

// ===================================== forward =====================================
// Per-lane code prefetch for one contraction step: two weight rows (j = 0, 1).
struct CodeStage {
  u32x4_t code[2];
  ConstRaw c[2];
};

template <int V>
struct Ic {
  static constexpr int v = V;
};

// X fragments (B operand) of contraction sub-step s from a staged tile: rows
// 32 i + l % 32, contraction half l / 32 -> chunk 4 (l / 32) + s.
__device__ __forceinline__ void read_xfrags_fwd(const char *sx, int s, u32x4_t (&xb)[8]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    xb[i] = *reinterpret_cast<const u32x4_t *>(sx + tile_off(i * 32 + (lane & 31), (lane >> 5) * 4 + s));
}

// Instruction-scheduling template for one forward sub-step (16 MFMAs), applied to a
// region fenced by sched_barrier: the 8 LDS fragment reads for the next sub-step go
// first, then each MFMA is followed by `NV` VALU instructions of decode work; the
// sub-step's `NG` global loads are spread evenly between the MFMAs, so that the four
// waves of a workgroup (which run in step) never queue all their loads at once.
template <int NV, int NG>
__device__ __forceinline__ void substep_schedule() {
  __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);  // DS reads
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    if constexpr (NG > 0)
      if (q % (16 / NG) == 0) __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);  // VMEM
    __builtin_amdgcn_sched_group_barrier(0x002, NV, 0);  // VALU
  }
}

// Global loads per wave and contraction step: per weight row (2) the codes and the
// constant's pieces (three, or one fp32 constant) of the step two ahead, then eight
// activation DMA loads, the last four after the step's barrier.  The barrier's wait
// leaves in flight the loads issued since the previous barrier and retires everything
// older, which includes the tile read right after it.  The last one or two steps of a
// launch issue no code loads (nothing would read them; left in the source, the
// compiler would delete them as dead and the count would no longer hold), so their
// barriers leave only their own DMA loads in flight.
constexpr int kDmaPerHalf = 4;  // DMA loads per wave and half tile (issue_dma)
template <int CT>
constexpr int code_loads_per_row() {
  return 1 + (CT == kConstF32 ? 1 : 3);  // issue_codes
}
template <int CT, bool CODES>
constexpr int loads_before_barrier() {
  return (CODES ? 2 * code_loads_per_row<CT>() : 0) + kDmaPerHalf;
}

// The forward is software-pipelined by contraction sub-step (16 of each 64-step):
// while the 16 MFMAs of sub-step s run, the weight fragments of sub-step s + 1 are
// decoded in registers and its activation fragments read from LDS.  Activation tiles
// rotate through three LDS buffers filled by direct buffer -> LDS loads: step i
// computes from buffer i % 3, issues the loads of tile i + 2 (into (i + 2) % 3, last
// read in step i - 1) during its second half, and reads the first fragments of tile
// i + 1 in its last sub-step, after a barrier that waits only for the loads of
// earlier steps.  Code stages and
// buffer indices are compile-time roles of a three-way unrolled loop, so no
// register copy ever waits for a load in flight.
constexpr int NBUF = 3;

template <int CT>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_fwd_kernel(
    GemmParams p) {
  __shared__ __attribute__((aligned(16))) char sX[NBUF * TILE_BYTES];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int tmi, tni;
  tile_coords((p.M + TM - 1) / TM, (p.No + TN - 1) / TN, tmi, tni);
  const int m0 = tmi * TM, n0 = tni * TN;

  const int K = p.Kc;
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(p.A, static_cast<uint32_t>(uint64_t(p.M) * K * 2));
  const __amdgpu_buffer_rsrc_t rc = make_rsrc(p.w.codes, static_cast<uint32_t>(uint64_t(p.No) * K / 2));
  const ConstRsrc rq = make_const_rsrc<CT>(p.w, static_cast<uint32_t>(uint64_t(p.No) * K / 64));
  const int nk = K / TK;
  const int last = nk - 1;

  // Per-lane load offsets; the contraction position enters as the scalar offset.
  // Rows past M and weight rows past N are clamped to the last valid one: they feed
  // only outputs that are never stored, and every load stays inside its buffer.
  // DMA: each wave-wide load writes 1 KB of LDS contiguously (lane l at byte 16 l),
  // so lane l fetches the chunk that belongs at that swizzled slot: tile row
  // r = 8 q + l / 8, slot l % 8 holds chunk (l % 8) ^ f(r); wave w issues q = 8 w + i.
  uint32_t xoff[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = (wave * 8 + i) * 8 + (lane >> 3);
    const int row = min(m0 + r, p.M - 1);
    xoff[i] = (static_cast<uint32_t>(row) * K + ((lane & 7) ^ swz(r)) * 8) * 2;
  }
  uint32_t coff[2], boff[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = min(n0 + wave * 64 + j * 32 + (lane & 31), p.No - 1);
    coff[j] = static_cast<uint32_t>(n) * (K / 2) + (lane >> 5) * 16;
    boff[j] = static_cast<uint32_t>(n) * (K / 64);
  }
  auto issue_codes = [&](int kt, int j, CodeStage &cs) {
    cs.code[j] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rc, coff[j], kt / 2, 0));
    if constexpr (CT == kConstF32) {
      cs.c[j] = {0u, __builtin_amdgcn_raw_buffer_load_b32(rq.s, boff[j] * 4u, kt / 16, 0), 0u};
    } else {
      cs.c[j].c8 = __builtin_amdgcn_raw_buffer_load_b8(rq.q8, boff[j], kt / 64, 0);
      const uint32_t g4 = ((boff[j] + kt / 64) >> 8) * 4u;
      cs.c[j].s = __builtin_amdgcn_raw_buffer_load_b32(rq.s, g4, 0, 0);
      cs.c[j].o = __builtin_amdgcn_raw_buffer_load_b32(rq.o, g4, 0, 0);
    }
  };
  auto issue_dma = [&](int kt, int h, char *buf) {
    char *dst = buf + wave * 8 * 1024;
#pragma unroll
    for (int i = kDmaPerHalf * h; i < kDmaPerHalf * (h + 1); ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (__attribute__((address_space(3))) void *)(dst + i * 1024),
                                               16, xoff[i], kt * 2, 0, 0);
  };

  f32x16_t acc[8][2];
  zero_acc(acc);

  CodeStage S0, S1, S2;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    issue_codes(0, h, S0);
    issue_codes(min(1, last) * TK, h, S1);
    issue_dma(0, h, sX);
    issue_dma(min(1, last) * TK, h, sX + TILE_BYTES);
  }
  // The LoRA term first, while the first tiles' loads are in flight.  Up to 64 ranks
  // with 16-byte aligned rows: the U_s tile of the 256 tokens (the rank columns of this
  // tile's part, zeros past r) is staged in the third activation buffer like one
  // contraction step of X and read with the same fragment reads, so every wave reads it
  // from LDS and loads only its own weight rows' B fragments (sub-step s: ranks
  // 8 s .. 8 s + 7 and 32 + 8 s .. in the two lane halves, as X's contraction order).
  // Otherwise the rank steps load both operands' fragments from memory.
  const bool lds_lora = p.r > 0 && p.r <= TK && (p.r % 8) == 0 && (p.lda2 % 8) == 0;
  u32x4_t wl[4][2];
  char *const sU = sX + 2 * TILE_BYTES;  // not written by the prologue's tile loads
  if (lds_lora) {
    const int qc = p.part_rows > 0 ? (n0 / p.part_rows) * p.r : 0;
    const __amdgpu_buffer_rsrc_t ru = make_rsrc(p.A2, static_cast<uint32_t>(uint64_t(p.M) * p.lda2 * 2));
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.B2, static_cast<uint32_t>(uint64_t(p.No) * p.r * 2));
    char *dst = sU + wave * 8 * 1024;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int rr = (wave * 8 + i) * 8 + (lane >> 3);
      const int row = min(m0 + rr, p.M - 1);
      const int c = (lane & 7) ^ swz(rr);
      const uint32_t off = c * 8 < p.r ? (static_cast<uint32_t>(row) * p.lda2 + qc + c * 8) * 2 : kOOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ru, (__attribute__((address_space(3))) void *)(dst + i * 1024), 16,
                                               off, 0, 0, 0);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        wl[s][j] = lora_frag(rb, true, n0 + wave * 64 + j * 32 + (lane & 31), p.No, p.r,
                             32 * (lane >> 5) + 8 * s, p.r);
  } else if (p.r > 0) {
    lora_steps(p, m0, n0, acc);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (lds_lora) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (8 * s < p.r) {
        u32x4_t xu[8];
        read_xfrags_fwd(sU, s, xu);
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) acc[i][j] = mfma32x32x16(wl[s][j], xu[i], acc[i][j]);
      }
    }
    __syncthreads();  // no wave reads the U_s tile any more when step 0 loads tile 2 there
  }

  Planes pl[2], pln[2];
  u32x4_t wa[2], xb[8];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    pl[j] = make_planes(const_value<CT>(S0.c[j]), p.lvl);
    wa[j] = lookup8(S0.code[j][0], pl[j]);
  }
  read_xfrags_fwd(sX, 0, xb);

  auto mfmas = [&]() {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = mfma32x32x16(wa[j], xb[i], acc[i][j]);
  };

  // One contraction step; B is the LDS buffer of the step's tile (it % 3); CODES says
  // whether the codes of step it + 2 are loaded (every step but the last one or two).
  auto step = [&](auto B, auto CODES, int it, CodeStage &cur, CodeStage &nxt, CodeStage &nn) {
    constexpr int b = decltype(B)::v;
    constexpr bool codes = decltype(CODES)::v != 0;
    const char *sx = sX + b * TILE_BYTES;
    const char *sxn = sX + ((b + 1) % NBUF) * TILE_BYTES;
    char *sxw = sX + ((b + 2) % NBUF) * TILE_BYTES;
    const int ktn = min(it + 2, last) * TK;
    float cn0, cn1;  // block constants of the next step's two rows
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4_t wan[2], xbn[8];
      if (codes && s < 2) issue_codes(ktn, s, nn);  // codes first: they are needed soonest
      // the next step's planes, half a row per sub-step (row 1's last half is needed
      // by this step's last sub-step)
      if (s == 0) {
        cn0 = const_value<CT>(nxt.c[0]);
        make_planes_half(cn0, p.lvl, 0, pln[0]);
      }
      if (s == 1) make_planes_half(cn0, p.lvl, 1, pln[0]);
      if (s == 2) {
        cn1 = const_value<CT>(nxt.c[1]);
        make_planes_half(cn1, p.lvl, 0, pln[1]);
      }
      if (s == 3) make_planes_half(cn1, p.lvl, 1, pln[1]);
      if (s == 2) issue_dma(ktn, 0, sxw);
      if (s == 3) {
        // tile it + 1 (issued a step ago) must have landed for every wave, and no wave
        // may still read the buffer that the next step's loads will overwrite
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(loads_before_barrier<CT, codes>())
                     : "memory");
        issue_dma(ktn, 1, sxw);
        read_xfrags_fwd(sxn, 0, xbn);
#pragma unroll
        for (int j = 0; j < 2; ++j) wan[j] = lookup8(nxt.code[j][0], pln[j]);
      } else {
        read_xfrags_fwd(sx, s + 1, xbn);
#pragma unroll
        for (int j = 0; j < 2; ++j) wan[j] = lookup8(cur.code[j][s + 1], pl[j]);
      }
      mfmas();
#pragma unroll
      for (int j = 0; j < 2; ++j) wa[j] = wan[j];
#pragma unroll
      for (int i = 0; i < 8; ++i) xb[i] = xbn[i];
      substep_schedule<5, 4>();
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) pl[j] = pln[j];
  };

  int it = 0;
  for (; it + 3 <= nk; it += 3) {
    step(Ic<0>{}, Ic<1>{}, it, S0, S1, S2);
    step(Ic<1>{}, Ic<1>{}, it + 1, S1, S2, S0);
    step(Ic<2>{}, Ic<1>{}, it + 2, S2, S0, S1);
  }
  // the last one or two steps: the codes of steps past the end are not loaded
  if (it < nk) step(Ic<0>{}, Ic<0>{}, it, S0, S1, S2);
  if (it + 1 < nk) step(Ic<1>{}, Ic<0>{}, it + 1, S1, S2, S0);
  // drain the clamped prefetches of the last steps before the epilogue
  __builtin_amdgcn_s_waitcnt(0);
  if (p.No % 8 == 0) {
    static_assert(4 * 128 * kOutPitch <= NBUF * TILE_BYTES, "output staging");
    __syncthreads();  // every wave is done reading the activation buffers
    store_out_lds(p, m0, n0, acc, sX);
  } else {
    store_out(p, m0, n0, acc);
  }
}

// ===================================== backward ====================================
// Weight tile for contraction rows [kt, kt + 64) and output columns [k0, k0 + 256),
// natural layout: 64 rows of 512 bytes, 16-byte chunk c of row n at slot c ^ g(n).
// Thread t decodes row kt + (t % 64), columns k0 + 64 (t / 64) .. + 64: one block
// constant, 32 bytes of codes, eight 16-byte LDS stores.  With n = (n3 n2 n1 n0) in
// binary, g(n) = (n1, n0, n1 ^ n3, n2): the 8 (16) consecutive rows of one store
// hit 8 (16) distinct 16-byte bank groups of a 128-byte (256-byte) bank cycle, and
// the 4 rows x 2 (4) chunks of a transposing read's 16 (32) lanes do too.
__device__ __forceinline__ int gswz(int n) {
  return ((n & 3) << 2) | ((((n >> 1) ^ (n >> 3)) & 1) << 1) | ((n >> 2) & 1);
}
__device__ __forceinline__ int wtile_off(int n, int col) {
  return n * 512 + ((((col >> 3) ^ gswz(n)) & 31) << 4) + (col & 7) * 2;
}

struct CodeStageB {
  u32x4_t code[2];
  ConstRaw c;
};

template <int CT>
__device__ __forceinline__ void code_load_bwd(const GemmParams &p, __amdgpu_buffer_rsrc_t rc,
                                              const ConstRsrc &rq, int k0, int kt, CodeStageB &cs) {
  const int tid = threadIdx.x;
  const int K = p.No, N = p.Kc;  // output columns are weight columns; contraction over rows
  const int n = kt + (tid & 63);
  const int k = k0 + (tid >> 6) * 64;
  const bool ok = n < N && k < K;
  const uint32_t off = static_cast<uint32_t>(n) * (K / 2) + k / 2;
  cs.code[0] = buf_load16(rc, ok ? off : kOOB);
  cs.code[1] = buf_load16(rc, ok ? off + 16 : kOOB);
  cs.c = fetch_constant<CT>(rq, static_cast<uint32_t>(n) * (K / 64) + k / 64, ok);
}

template <int CT>
__device__ __forceinline__ void code_store_bwd(const GemmParams &p, const CodeStageB &cs, char *sw) {
  const int tid = threadIdx.x;
  const int n = tid & 63, c0 = (tid >> 6) * 64;
  const Planes pl = make_planes(const_value<CT>(cs.c), p.lvl);
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<u32x4_t *>(sw + wtile_off(n, c0 + h * 32 + i * 8)) = lookup8(cs.code[h][i], pl);
}


// Weight-side MFMA fragment for contraction step s (16 rows) and output-column tile
// j of this wave: two transposing reads of 4 rows each.  Within a 16-lane group, lane
// i reads row nbase + i / 4 at column cbase + 4 (i % 4) and receives column cbase + i
// of rows nbase .. nbase + 3.
__device__ __forceinline__ u32x4_t wfrag_tr(const char *sw, int s, int j) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i = lane & 15, g = lane >> 4;
  const int cbase = wave * 64 + j * 32 + (g & 1) * 16;
  const int col = cbase + 4 * (i & 3);
  u32x4_t r;
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int n = 16 * s + 8 * (g >> 1) + 4 * e + (i >> 2);
    const v4i16_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16_t *)(sw + wtile_off(n, col)));
    const u32x2_t u = __builtin_bit_cast(u32x2_t, v);
    r[2 * e] = u[0];
    r[2 * e + 1] = u[1];
  }
  return r;
}

template <bool VEC, int CT>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_dx_kernel(
    GemmParams p) {
  __shared__ __attribute__((aligned(16))) char sX[2][TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char sW[2][TILE_BYTES];
  if (static_cast<int>(blockIdx.x) >= p.tiles) {
    finalize_part(p.fin, blockIdx.x - p.tiles, p.fin_wgs);
    return;
  }
  const int tid = threadIdx.x, lane = tid & 63;
  int tmi, tni;
  tile_coords((p.M + TM - 1) / TM, (p.No + TN - 1) / TN, tmi, tni);
  const int m0 = tmi * TM, k0 = tni * TN;

  const int N = p.Kc, K = p.No;
  const __amdgpu_buffer_rsrc_t rdy = make_rsrc(p.A, static_cast<uint32_t>(uint64_t(p.M) * N * 2));
  const __amdgpu_buffer_rsrc_t rc = make_rsrc(p.w.codes, static_cast<uint32_t>(uint64_t(N) * K / 2));
  const ConstRsrc rq = make_const_rsrc<CT>(p.w, static_cast<uint32_t>(uint64_t(N) * K / 64));
  const int nk = (N + TK - 1) / TK;
  const int last = nk - 1;

  f32x16_t acc[8][2];
  zero_acc(acc);

  ActStage st;
  CodeStageB cs;
  act_load(rdy, m0, p.M, N, 0, VEC, p.A, st);
  code_load_bwd<CT>(p, rc, rq, k0, 0, cs);
  act_store(sX[0], st);
  code_store_bwd<CT>(p, cs, sW[0]);
  __syncthreads();

  auto step = [&](int it, const char *sx, const char *sw, char *sx_next, char *sw_next) {
    const int nt = min(it + 1, last) * TK;
    act_load(rdy, m0, p.M, N, nt, VEC, p.A, st);
    code_load_bwd<CT>(p, rc, rq, k0, nt, cs);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4_t wa[2], xb[8];
      const int chunk = 2 * s + (lane >> 5);
#pragma unroll
      for (int j = 0; j < 2; ++j) wa[j] = wfrag_tr(sw, s, j);
#pragma unroll
      for (int i = 0; i < 8; ++i)
        xb[i] = *reinterpret_cast<const u32x4_t *>(sx + tile_off(i * 32 + (lane & 31), chunk));
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32x32x16(wa[j], xb[i], acc[i][j]);
    }
    act_store(sx_next, st);
    code_store_bwd<CT>(p, cs, sw_next);
    __syncthreads();
  };
  int it = 0;
  for (; it + 1 < nk; it += 2) {
    step(it, sX[0], sW[0], sX[1], sW[1]);
    step(it + 1, sX[1], sW[1], sX[0], sW[0]);
  }
  if (it < nk) step(it, sX[0], sW[0], sX[1], sW[1]);
  if (p.r > 0) lora_steps(p, m0, k0, acc);
  store_out(p, m0, k0, acc);
}

// Pipelined dX for dY rows of whole 16-byte chunks (N % 8 == 0).
//
// Layout: 2 x 2 waves; wave w owns tokens m0 + 128 (w / 2) .. + 128 (four 32-token
// MFMA tiles) and output columns k0 + 128 (w % 2) .. + 128 (four 32-column tiles),
// acc[i][j], so per sub-step it reads 4 weight and 4 dY fragments for 16 MFMAs.  Each
// step's 256 x 64 dY slice is fetched one step ahead by direct buffer -> LDS loads
// into one of two stages, wave w loading rows 64 w .. + 64 (whole 128-byte row
// segments per load, in the swizzled row layout of tile_off); the MFMA fragments are
// read back with ds_read_b128 (lane l: token 32 i + l % 32, 8 contraction rows at
// 16 s + 8 (l / 32)).  The step's barrier, after each wave's own load wait,
// publishes the next stage.  The decoded weight tile (64 rows x 256 columns) is
// shared through LDS (each wave reads its 128 columns) with the transposing
// ds_read_b64_tr_b16.  During step i
// every thread decodes its 64 weights of step i + 1 (one block constant, eight
// lookups) into the other of two weight tiles, spread over the first three
// sub-steps; the single barrier per step, before the last sub-step, publishes that
// tile, whose first fragments the last sub-step then reads.  dY columns past N read
// as zero and weight rows past N decode to zero, so the contraction tail adds nothing.

// Weight-side fragment for contraction sub-step s and output-column tile j (32
// columns) of the block: two transposing reads of 4 rows each.  Within a 16-lane
// group, lane i reads row nbase + i / 4 at column cbase + 4 (i % 4) and receives
// column cbase + i of rows nbase .. nbase + 3.  The swizzle g(n) depends on the row
// only through n % 16, and j / 4 moves the chunk index by 16, past the bits that
// g(n) touches, so a lane's read addresses are eight per-lane bases trb[e][j % 4]
// (sub-step 0, j < 4) plus the constants 8192 s + 256 (j / 4).
__device__ __forceinline__ void wfrag_bases(uint32_t (&trb)[2][4]) {
  const int lane = threadIdx.x & 63;
  const int i = lane & 15, g = lane >> 4;
#pragma unroll
  for (int e = 0; e < 2; ++e)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
      trb[e][jj] = wtile_off(8 * (g >> 1) + 4 * e + (i >> 2), jj * 32 + (g & 1) * 16 + 4 * (i & 3));
}
__device__ __forceinline__ u32x4_t wfrag_tr_all(const char *sw, const uint32_t (&trb)[2][4], int s, int j) {
  u32x4_t r;
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const v4i16_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16_t *)(sw + trb[e][j & 3] + (8192 * s + 256 * (j >> 2))));
    const u32x2_t u = __builtin_bit_cast(u32x2_t, v);
    r[2 * e] = u[0];
    r[2 * e + 1] = u[1];
  }
  return r;
}

// Epilogue of the dX layout: lane holds tokens tb + 32 i + l % 32 and output columns
// cb + 32 j + 8 g + 4 (l / 32) + 0..3 (g = 0..3) of acc[i][j].
template <int NI, int NJ>
__device__ __forceinline__ void store_out_dx(const GemmParams &p, int tb, int cb,
                                             const f32x16_t (&acc)[NI][NJ]) {
  const int lane = threadIdx.x & 63;
  const bool vec = (p.No % 4) == 0;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int m = tb + i * 32 + (lane & 31);
    if (m >= p.M) continue;
    uint16_t *row = p.C + static_cast<int64_t>(m) * p.No;
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = cb + j * 32 + g * 8 + (lane >> 5) * 4;
        const f32x16_t &a = acc[i][j];
        if (vec) {
          if (col < p.No) {
            u32x2_t o = {pack_bf16x2(a[4 * g], a[4 * g + 1]), pack_bf16x2(a[4 * g + 2], a[4 * g + 3])};
            *reinterpret_cast<u32x2_t *>(row + col) = o;
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (col + e < p.No) row[col + e] = to_bf16(a[4 * g + e]);
        }
      }
  }
}

// The dX epilogue through LDS, for 16-byte aligned output rows (No % 8 == 0): each
// wave stages its 128 x 128 output block in its own 32 KB buffer `reg`, in two halves
// of 64 tokens (rows of 264 bytes, so that a lane half's 32 token rows fall in
// distinct banks), and writes it back 4 rows x 256 bytes per store instruction.
constexpr int kOutPitchDx = 264;
__device__ __forceinline__ void store_out_dx_lds(const GemmParams &p, int tb, int cb, const f32x16_t (&acc)[4][4],
                                                 char *reg) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int ii = 0; ii < 2; ++ii)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x16_t &a = acc[2 * h + ii][j];
          const int tok = ii * 32 + (lane & 31), col = j * 32 + g * 8 + (lane >> 5) * 4;
          const u32x2_t o = {pack_bf16x2(a[4 * g], a[4 * g + 1]), pack_bf16x2(a[4 * g + 2], a[4 * g + 3])};
          *reinterpret_cast<u32x2_t *>(reg + tok * kOutPitchDx + col * 2) = o;
        }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the wave's writes have landed
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int tok = 4 * q + (lane >> 4), ch = lane & 15;
      const u32x2_t lo = *reinterpret_cast<const u32x2_t *>(reg + tok * kOutPitchDx + ch * 16);
      const u32x2_t hi = *reinterpret_cast<const u32x2_t *>(reg + tok * kOutPitchDx + ch * 16 + 8);
      const int m = tb + 64 * h + tok, col = cb + ch * 8;
      if (m < p.M && col < p.No)
        *reinterpret_cast<u32x4_t *>(p.C + static_cast<int64_t>(m) * p.No + col) = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // read back before the next half overwrites it
  }
}

// LoRA steps of the dX layout: acc[i][j] += A2 rows (tokens tb + 32 i + ..) x B2 rows
// (output columns cb + 32 j + ..), rank in steps of 16.
template <int NI, int NJ>
__device__ __forceinline__ void lora_steps_dx(const GemmParams &p, int tb, int cb, f32x16_t (&acc)[NI][NJ]) {
  const int lane = threadIdx.x & 63;
  const int r = p.r;
  const bool vec = (r % 8) == 0;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.A2, static_cast<uint32_t>(uint64_t(p.M) * r * 2));
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.B2, static_cast<uint32_t>(uint64_t(p.No) * r * 2));
  constexpr int RQ = LORA_RQ;  // rank steps per chunk, all loads before the MFMAs
  for (int r0 = 0; r0 < r; r0 += 16 * RQ) {
    u32x4_t wa[RQ][NJ], vb[RQ][NI];
#pragma unroll
    for (int q = 0; q < RQ; ++q) {
      const int j0 = r0 + 16 * q + (lane >> 5) * 8;
#pragma unroll
      for (int j = 0; j < NJ; ++j) wa[q][j] = lora_frag(rb, vec, cb + j * 32 + (lane & 31), p.No, r, j0, r);
#pragma unroll
      for (int i = 0; i < NI; ++i) vb[q][i] = lora_frag(ra, vec, tb + i * 32 + (lane & 31), p.M, r, j0, r);
    }
#pragma unroll
    for (int q = 0; q < RQ; ++q) {
      if (r0 + 16 * q < r) {
#pragma unroll
        for (int i = 0; i < NI; ++i)
#pragma unroll
          for (int j = 0; j < NJ; ++j) acc[i][j] = mfma32x32x16(wa[q][j], vb[q][i], acc[i][j]);
      }
    }
  }
}

template <int NR, int NV, int NG, int NW>
__device__ __forceinline__ void dx_schedule() {
  __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);  // DS reads
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    if constexpr (NG > 0)
      if (q % (16 / NG) == 0) __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);  // VMEM
    if constexpr (NW > 0)
      if (q % (16 / NW) == (16 / NW) - 1) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // DS write
    __builtin_amdgcn_sched_group_barrier(0x002, NV, 0);  // VALU
  }
}

// dY rows that one wave loads per step: 64 tokens x 64 contraction rows (8 KB); a stage
// holds the four waves' slices.
constexpr int YWAVE_BYTES = 64 * TK * 2;

template <int CT>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_dx_pipe_kernel(
    GemmParams p) {
  // two weight tiles and two dY stages, 128 KB; separate objects, so that the
  // compiler can tell reads of one stage or tile from the loads into the other stage
  __shared__ __attribute__((aligned(16))) char sW0[TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char sW1[TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char sY0[TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char sY1[TILE_BYTES];
  // the workgroups after the tiles (dispatched last, so in CUs the tiles have left) do
  // the finalize job that rides in this launch
  if (static_cast<int>(blockIdx.x) >= p.tiles) {
    finalize_part(p.fin, blockIdx.x - p.tiles, p.fin_wgs);
    return;
  }
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // 2 x 2 waves: wave w computes tokens 128 (w / 2) .. + 128 and output columns
  // 128 (w % 2) .. + 128; it loads the dY rows 64 w .. + 64 of the block
  const int wr = wave >> 1, wc = wave & 1;
  char *const sYw[2] = {sY0 + wave * YWAVE_BYTES, sY1 + wave * YWAVE_BYTES};
  int tmi, tni;
  tile_coords((p.M + TM - 1) / TM, (p.No + TN - 1) / TN, tmi, tni);
  const int m0 = tmi * TM, k0 = tni * TN;

  const int N = p.Kc, K = p.No;  // contraction over weight rows, outputs are weight columns
  const __amdgpu_buffer_rsrc_t rdy = make_rsrc(p.A, static_cast<uint32_t>(uint64_t(p.M) * N * 2));
  const __amdgpu_buffer_rsrc_t rc = make_rsrc(p.w.codes, static_cast<uint32_t>(uint64_t(N) * K / 2));
  const ConstRsrc rq = make_const_rsrc<CT>(p.w, static_cast<uint32_t>(uint64_t(N) * K / 64));
  const int nk = (N + TK - 1) / TK;
  const int last = nk - 1;

  // dY loads: load q of a step writes rows 8 q .. 8 q + 7 of the wave's slice (1 KB,
  // lane l at byte 16 l), so lane l fetches the chunk that belongs at slot l % 8 of
  // row r = 8 q + l / 8: chunk (l % 8) ^ swz(r), which depends on q only through its
  // parity.  Rows past M are clamped to the last one; they feed only outputs that are
  // never stored.
  const int ych[2] = {(lane & 7) ^ (lane >> 3), (lane & 7) ^ (lane >> 3) ^ 1};
  uint32_t yoff[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int row = min(m0 + wave * 64 + 8 * q + (lane >> 3), p.M - 1);
    yoff[q] = (static_cast<uint32_t>(row) * N + ych[q & 1] * 8) * 2;
  }
  // CHK: the step may reach past N (the last one); chunks at or past N read as zero
  auto issue_y = [&](auto CHK, int kt, char *dst) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      auto *d = (__attribute__((address_space(3))) void *)(dst + q * 1024);
      if constexpr (decltype(CHK)::v) {
        const uint32_t off = kt + ych[q & 1] * 8 < N ? yoff[q] + kt * 2 : kOOB;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rdy, d, 16, off, 0, 0, 0);
      } else {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rdy, d, 16, yoff[q], kt * 2, 0, 0);
      }
    }
  };
  // dY fragments of sub-step s from a stage: token 128 wr + 32 i + l % 32 is row
  // 32 (i % 2) + l % 32 of the slice loaded by wave 2 wr + i / 2; swz() sees only the
  // row's low five bits, so token tile i adds the constant 4096 i to one base per
  // sub-step
  uint32_t yrb[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) yrb[s] = wr * 2 * YWAVE_BYTES + tile_off(lane & 31, 2 * s + (lane >> 5));
  auto read_y = [&](const char *sy, int s, u32x4_t (&yb)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) yb[i] = *reinterpret_cast<const u32x4_t *>(sy + yrb[s] + 4096 * i);
  };
  // weight fragments of this wave's column tiles j = 0..3 (block tiles 4 wc + j)
  uint32_t trb[2][4];
  wfrag_bases(trb);
#pragma unroll
  for (int e = 0; e < 2; ++e)
#pragma unroll
    for (int j = 0; j < 4; ++j) trb[e][j] += 256 * wc;
  // Weight decode: thread t owns tile row t % 64 and columns 64 (t / 64) .. + 64.
  const int dn = tid & 63, dc = (tid >> 6) * 64;
  const bool col_ok = k0 + dc < K;
  auto issue_codes = [&](int kt, CodeStageB &cs) {
    const int n = kt + dn;
    const bool ok = col_ok && n < N;
    const uint32_t off = static_cast<uint32_t>(n) * (K / 2) + (k0 + dc) / 2;
    cs.code[0] = buf_load16(rc, ok ? off : kOOB);
    cs.code[1] = buf_load16(rc, ok ? off + 16 : kOOB);
    cs.c = fetch_constant<CT>(rq, static_cast<uint32_t>(n) * (K / 64) + (k0 + dc) / 64, ok);
  };
  // global loads of one issue_codes: two code chunks and the constant's pieces
  constexpr int CODE_LOADS = 2 + (CT == kConstF32 ? 1 : 3);
  // lookups q0 .. q1 - 1 of the eight (q = 4 h + i: 16-byte code half h, word i)
  auto decode_part = [&](const CodeStageB &cs, const Planes &pd, char *sw, int q0, int q1) {
#pragma unroll
    for (int q = q0; q < q1; ++q)
      *reinterpret_cast<u32x4_t *>(sw + wtile_off(dn, dc + q * 8)) = lookup8(cs.code[q >> 2][q & 3], pd);
  };

  f32x16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  CodeStageB S0, S1;
  issue_codes(0, S0);
  issue_codes(min(1, last) * TK, S1);
  issue_y(Ic<1>{}, 0, sYw[0]);
  // The LoRA term first, while the first tiles' loads are in flight.  Up to 64 ranks
  // with 16-byte aligned rows: the V tile of the 256 tokens (zeros past r) is loaded
  // into the second dY stage laid out like a dY stage and read with the same fragment
  // reads (sub-step s: ranks 16 s .. 16 s + 15); each wave loads only its own output
  // columns' At fragments.  Otherwise the rank steps load both operands from memory.
  const bool lds_lora = p.r > 0 && p.r <= TK && (p.r % 8) == 0;
  u32x4_t wl[4][4];
  if (lds_lora) {
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.A2, static_cast<uint32_t>(uint64_t(p.M) * p.r * 2));
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.B2, static_cast<uint32_t>(uint64_t(p.No) * p.r * 2));
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int row = min(m0 + wave * 64 + 8 * q + (lane >> 3), p.M - 1);
      const int c = ych[q & 1];
      const uint32_t off = c * 8 < p.r ? (static_cast<uint32_t>(row) * p.r + c * 8) * 2 : kOOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (__attribute__((address_space(3))) void *)(sYw[1] + q * 1024), 16,
                                               off, 0, 0, 0);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        wl[s][j] = lora_frag(rb, true, k0 + 128 * wc + j * 32 + (lane & 31), p.No, p.r, 16 * s + (lane >> 5) * 8, p.r);
  } else if (p.r > 0) {
    lora_steps_dx(p, m0 + 128 * wr, k0 + 128 * wc, acc);
  }
  {
    const Planes pd = make_planes(const_value<CT>(S0.c), p.lvl);
    decode_part(S0, pd, sW0, 0, 8);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (lds_lora) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (16 * s < p.r) {
        u32x4_t vb[4];
        read_y(sY1, s, vb);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = mfma32x32x16(wl[s][j], vb[i], acc[i][j]);
      }
    }
    __syncthreads();  // no wave reads the V tile any more when step 0 loads dY step 1 there
  }

  u32x4_t wa[4], yb[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) wa[j] = wfrag_tr_all(sW0, trb, 0, j);
  read_y(sY0, 0, yb);

  // Step it: weight tile and dY stage b2 = it % 2 are this step's; the other stage
  // receives the dY slice of step it + 1, `dec` holds the codes of step it + 1
  // (decoded now into the other weight tile), `ld` receives those of step it + 2.
  // In the main loop (CHK = 0) the barrier leaves the code loads of step it + 2 in
  // flight.  In the last one to three steps (CHK = 1) some of those loads feed nothing,
  // and the compiler may delete them on some paths, so the count of loads in flight
  // would not hold there: those steps wait for all of their loads at the barrier.
  auto step = [&](auto B2, auto CHK, int it, CodeStageB &dec, CodeStageB &ld) {
    constexpr int b2 = decltype(B2)::v;
    constexpr bool tail = decltype(CHK)::v != 0;
    const char *sw = b2 ? sW1 : sW0;
    char *swn = b2 ? sW0 : sW1;
    const char *sy = b2 ? sY1 : sY0;
    const char *syn = b2 ? sY0 : sY1;
    const int kt1 = min(it + 1, last) * TK, kt2 = min(it + 2, last) * TK;
    Planes pd;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4_t wan[4], ybn[4];
      if (s == 0) {
        pd = make_planes(const_value<CT>(dec.c), p.lvl);
        // the other stage was last read two sub-steps ago, and every LDS read has
        // completed at the previous step's barrier
        issue_y(CHK, kt1, sYw[1 - b2]);
        decode_part(dec, pd, swn, 0, 2);
      }
      if (s == 1) {
        issue_codes(kt2, ld);
        decode_part(dec, pd, swn, 2, 5);
      }
      if (s == 2) decode_part(dec, pd, swn, 5, 8);
      if (s == 3) {
        // this wave's dY slice of step it + 1 has landed (only the code loads of
        // sub-step 1 were issued after it), and after the barrier every wave's has;
        // every thread's part of the next weight tile is written; no wave still
        // reads the tile or stage that the next step overwrites
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(tail ? 0 : CODE_LOADS) : "memory");
#pragma unroll
        for (int j = 0; j < 4; ++j) wan[j] = wfrag_tr_all(swn, trb, 0, j);
        read_y(syn, 0, ybn);
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) wan[j] = wfrag_tr_all(sw, trb, s + 1, j);
        read_y(sy, s + 1, ybn);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma32x32x16(wa[j], yb[i], acc[i][j]);
#pragma unroll
      for (int j = 0; j < 4; ++j) wa[j] = wan[j];
#pragma unroll
      for (int i = 0; i < 4; ++i) yb[i] = ybn[i];
      if (s == 0)
        dx_schedule<12, 5, 8, 2>();
      else if (s == 1)
        dx_schedule<12, 4, CODE_LOADS, 3>();
      else if (s == 2)
        dx_schedule<12, 4, 0, 3>();
      else
        dx_schedule<12, 1, 0, 0>();
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Two steps per trip (stages, code stages and weight tiles alternate) while the
  // dY prefetch stays inside N; the last steps check the contraction tail.
  int it = 0;
  for (; it + 4 <= nk; it += 2) {
    step(Ic<0>{}, Ic<0>{}, it, S1, S0);
    step(Ic<1>{}, Ic<0>{}, it + 1, S0, S1);
  }
  if (it < nk) step(Ic<0>{}, Ic<1>{}, it, S1, S0);
  if (it + 1 < nk) step(Ic<1>{}, Ic<1>{}, it + 1, S0, S1);
  if (it + 2 < nk) step(Ic<0>{}, Ic<1>{}, it + 2, S1, S0);
  __builtin_amdgcn_s_waitcnt(0);
  if (p.No % 8 == 0) {
    static_assert(64 * kOutPitchDx <= TILE_BYTES, "output staging");
    __syncthreads();  // every wave is done reading the weight tiles and dY stages
    char *const reg = wave == 0 ? sW0 : wave == 1 ? sW1 : wave == 2 ? sY0 : sY1;
    store_out_dx_lds(p, m0 + 128 * wr, k0 + 128 * wc, acc, reg);
  } else {
    store_out_dx(p, m0 + 128 * wr, k0 + 128 * wc, acc);
  }
}

bool fits_32bit(int64_t M, int64_t N, int64_t K, int r) {
  const uint64_t lim = 0xFFFFFFF0ull;
  return uint64_t(M) * K * 2 <= lim && uint64_t(M) * N * 2 <= lim && uint64_t(N) * K / 2 <= lim &&
         uint64_t(M) * r * 2 <= lim && uint64_t(N) * r * 2 <= lim && uint64_t(K) * r * 2 <= lim;
}

GemmParams make_params(const uint16_t *A, const WeightView &w, const uint16_t *A2,
                       const uint16_t *B2, uint16_t *C, int64_t M, int64_t No, int64_t Kc, int r) {
  GemmParams p{A, w, A2, B2, C, static_cast<int>(M), static_cast<int>(No), static_cast<int>(Kc), r, {}, r, 0};
  p.lvl = level_table(w.quant_type);
  p.tiles = static_cast<int>(((M + TM - 1) / TM) * ((No + TN - 1) / TN));
  p.fin_wgs = 0;
  p.fin = FinalizeJob{nullptr, 0, 0, 0, 0, 0.0f, nullptr};
  return p;
}

unsigned grid_size(int64_t M, int64_t No) {
  return static_cast<unsigned>(((M + TM - 1) / TM) * ((No + TN - 1) / TN));
}

}  // namespace

bool gemm_supported(const WeightView &w, int64_t M, int r) {
  return M <= 0x7fffffff && fits_32bit(M, w.n_rows, w.n_cols, r);
}

hipError_t launch_gemm_fwd(const WeightView &w, const uint16_t *X, int64_t M, const uint16_t *U,
                           int ldu, const uint16_t *Bl, int r, int64_t part_rows, uint16_t *Y,
                           hipStream_t stream) {
  if (!fits_32bit(M, w.n_rows, w.n_cols, ldu) || M > 0x7fffffff) return hipErrorInvalidValue;
  if (part_rows > 0 && (part_rows % TN != 0 || w.n_rows % part_rows != 0)) return hipErrorInvalidValue;
  GemmParams p = make_params(X, w, U, Bl, Y, M, w.n_rows, w.n_cols, r);
  p.lda2 = ldu;
  p.part_rows = static_cast<int>(part_rows);
  const dim3 grid(grid_size(M, w.n_rows));
  switch (w.const_type) {
    case kConstDqInt8: hipLaunchKernelGGL(gemm_fwd_kernel<kConstDqInt8>, grid, dim3(NT), 0, stream, p); break;
    case kConstDqFp8: hipLaunchKernelGGL(gemm_fwd_kernel<kConstDqFp8>, grid, dim3(NT), 0, stream, p); break;
    case kConstF32: hipLaunchKernelGGL(gemm_fwd_kernel<kConstF32>, grid, dim3(NT), 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gemm_dx(const WeightView &w, const uint16_t *dY, int64_t M, const uint16_t *V,
                          const uint16_t *At, int r, uint16_t *dX, hipStream_t stream, const FinalizeJob *fin) {
  if (!fits_32bit(M, w.n_rows, w.n_cols, r) || M > 0x7fffffff) return hipErrorInvalidValue;
  GemmParams p = make_params(dY, w, V, At, dX, M, w.n_cols, w.n_rows, r);
  if (fin && fin->splits > 0) {
    p.fin = *fin;
    p.fin_wgs = static_cast<int>(finalize_workgroups(*fin));
  }
  if (int64_t(p.tiles) + p.fin_wgs > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(p.tiles + p.fin_wgs));
  const bool pipe = w.n_rows % 8 == 0;
  auto go = [&](auto pipe_kern, auto plain_kern) {
    if (pipe)
      hipLaunchKernelGGL(pipe_kern, grid, dim3(NT), 0, stream, p);
    else
      hipLaunchKernelGGL(plain_kern, grid, dim3(NT), 0, stream, p);
    return hipGetLastError();
  };
  switch (w.const_type) {
    case kConstDqInt8: return go(gemm_dx_pipe_kernel<kConstDqInt8>, gemm_dx_kernel<false, kConstDqInt8>);
    case kConstDqFp8: return go(gemm_dx_pipe_kernel<kConstDqFp8>, gemm_dx_kernel<false, kConstDqFp8>);
    case kConstF32: return go(gemm_dx_pipe_kernel<kConstF32>, gemm_dx_kernel<false, kConstF32>);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qlora
