// Skinny LoRA products (gfx950): the rank-r down-projections U_s, V and the two
// reductions over tokens that give dB and dA.
//
//   U_s = bf16((alpha/r) X A^T)   and   V = bf16((alpha/r) dY B)      (lora_down)
//   dB  = bf16(dY^T U_s)          and   dA = bf16(V^T X)              (reduce_m)
//
// ([Paper note] "关键设计 3" equation and listing; [Repro] "LoRA 的公式和张量形状":
// scaling = lora_alpha / r; [Digest] "方法步骤与流程" step 4: only the adapter
// receives gradients.)  All products run on the 32x32x16 bf16 MFMA with fp32
// accumulation.  These kernels are HBM-bound (they stream X or dY once), so they
// are split over many workgroups: each writes fp32 partial sums to caller
// workspace and a finalize pass adds the partials in a fixed order and rounds to
// bf16 once, so results are bitwise reproducible (no floating-point atomics).
//
// Fast paths need 16-byte aligned rows (row length % 8 == 0, r % 8 == 0) and
// tensors below 4 GiB (32-bit buffer offsets; out-of-range buffer reads return
// zero, which handles every tile edge without branches).  Other shapes take the
// generic kernels at the end of this file.

#include "device_common.h"
#include "qlora_internal.h"

namespace qlora {
namespace {

constexpr int NT = 256;
constexpr uint64_t k4G = 0xFFFFFFF0ull;
constexpr int64_t kDownWGs = 256;  // lora_down workgroups aimed at (one per CU)

// ---------------------------------------------------------------------------------
// lora_down: P[ks][m][j] = sum_{k in split ks} IN[m][k] WT[j][k]
// MFMA roles: A = WT fragment (rows j), B = IN fragment (columns m), so each lane
// ends with 4 consecutive j of one m: 16-byte partial stores.
//
// lora_down with LDS-staged operands: the same partial sums P[ks][m][j] over one K-split,
// with both operand tiles brought into LDS by direct buffer -> LDS loads.  A 64-wide
// contraction step stages IN rows m0 .. m0 + 63 and WT rows 0 .. 32 RT - 1, 128 bytes
// each; eight lanes read one whole row (the 16-byte chunk a lane fetches is the one that
// belongs at its slot of the swizzled tile, chunk c of row x at slot c ^ f(x), as in the
// forward GEMM), so every load instruction covers eight complete 128-byte lines.  NB
// buffers keep NB - 1 steps of loads in flight; one barrier per step publishes a step's
// tile and retires the buffer that the next loads overwrite.  Wave w owns output tiles
// w, w + 4, ... of the 2 x RT tiles of 32 x 32 and accumulates them over the whole split,
// so no cross-wave reduction is needed.
__device__ __forceinline__ int stile_off(int row, int c) { return row * 128 + ((c ^ ((row & 7) ^ ((row >> 3) & 1))) << 4); }

// LDS of the staged bodies: (64 + 32 RT) rows of 128 bytes per buffer, as many buffers
// (at most 4) as fit in the 160 KB of a workgroup
template <int RT>
constexpr int staged_nb() {
  return 4 * (64 + 32 * RT) * 128 <= 160 * 1024 ? 4 : 3 * (64 + 32 * RT) * 128 <= 160 * 1024 ? 3 : 2;
}
template <int RT>
constexpr int staged_bytes() {
  return staged_nb<RT>() * (64 + 32 * RT) * 128;
}

// Row-major tiles of 64 rows x 32 RT bf16 columns (64 RT bytes per row, the 16-byte
// chunks swizzled within the row when there are a power of two of them): the S tile of
// reduce_m and the B tile of lora_down over B [Kc, r].
template <int RT>
__device__ __forceinline__ int s_swz(int row) {
  // the S tile's rows hold 4 RT chunks; swizzle within the row when that is a power of two
  return ((4 * RT) & (4 * RT - 1)) == 0 ? (((row & 7) ^ ((row >> 3) & 1)) & (4 * RT - 1)) : 0;
}
// MFMA operand fragment of such a tile read with the transposing LDS read: column
// cb + (lane % 32) of rows 16 s + 8 (lane / 32) .. + 7 (within a 16-lane group, lane i
// reads 8 bytes of row base + i / 4 at column 4 (i % 4) of its 16-column half and
// receives column i of those four rows).
template <int RT>
__device__ __forceinline__ u32x4_t frag_rows(const char *tile, int s, int cb) {
  const int lane = threadIdx.x & 63;
  const int i = lane & 15, gq = lane >> 4;
  const int col = cb + (gq & 1) * 16 + 4 * (i & 3);
  u32x4_t v;
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int row = 16 * s + 8 * (gq >> 1) + 4 * e + (i >> 2);
    const int off = row * (64 * RT) + (((col >> 3) ^ s_swz<RT>(row)) << 4) + (col & 7) * 2;
    const v4i16_t t = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16_t *)(tile + off));
    const u32x2_t w = __builtin_bit_cast(u32x2_t, t);
    v[2 * e] = w[0];
    v[2 * e + 1] = w[1];
  }
  return v;
}

// The workgroup's AEXT x BEXT tile of fp32 partial sums, element (a, b) going to
// P[a pitch + b] for a < a_lim, b < b_lim.  Each wave holds tiles w, w + 4, ... of
// 32 x 32 in the MFMA accumulator layout (lane l: a = a0 + l % 32, four consecutive
// b from b0 + 8 g + 4 (l / 32)); tile_ab(t, a0, b0) gives tile t's corner.  The tile
// is staged through LDS (rows of BEXT floats plus 16 bytes) and written back row by
// row, BEXT / 4 lanes per row segment, so that a store instruction covers whole row
// segments instead of 32 pieces of 32 bytes.
template <int AEXT, int BEXT, int TPW, int TILES, typename TileAB>
__device__ __forceinline__ void store_partials(char *sbuf, const f32x16_t (&acc)[TPW], TileAB tile_ab, float *P,
                                               int64_t pitch, int a_lim, int b_lim) {
  constexpr int PB = BEXT * 4 + 16;
  constexpr int LPR = BEXT / 4;  // 16-byte pieces per row
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();  // no wave reads the staging buffers any more
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    const int tile = wave + 4 * u;
    if (TILES % 4 != 0 && tile >= TILES) continue;
    int a0, b0;
    tile_ab(tile, a0, b0);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int a = a0 + (lane & 31), b = b0 + 8 * g + 4 * (lane >> 5);
      *reinterpret_cast<f32x4_t *>(sbuf + a * PB + b * 4) =
          f32x4_t{acc[u][4 * g], acc[u][4 * g + 1], acc[u][4 * g + 2], acc[u][4 * g + 3]};
    }
  }
  __syncthreads();
#pragma unroll
  for (int q = static_cast<int>(threadIdx.x); q < AEXT * LPR; q += NT) {
    const int a = q / LPR, b = (q % LPR) * 4;
    if (a < a_lim && b < b_lim)
      *reinterpret_cast<f32x4_t *>(P + a * pitch + b) = *reinterpret_cast<const f32x4_t *>(sbuf + a * PB + b * 4);
  }
}

// BK: the adapter operand is given as B [Kc, r] (rows of the contraction, row pitch
// ldwt) instead of WT [r, Kc]; its step tile (64 contraction rows of r ranks) is staged
// row-major like reduce_m's S tile and read with the transposing LDS read, so the
// product V = dY B needs no transposed copy of B.
template <int RT, int NB, bool BK = false>
__device__ __forceinline__ void lora_down_dma_body(
    char *sbuf, int bx, int by, const uint16_t *__restrict__ IN, int M, int Kc, int ldin,
    const uint16_t *__restrict__ WT, int ldwt, int r, int KR, float *__restrict__ P) {
  constexpr int ROWS = 64 + 32 * RT;       // staged rows per step (IN then WT)
  constexpr int BUF = ROWS * 128;          // bytes per buffer
  constexpr int NLD = ROWS / 8;            // 1 KB loads per step
  constexpr int LPW = NLD / 4;             // loads per wave and step
  constexpr int TILES = 2 * RT, TPW = (TILES + 3) / 4;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int m0 = bx * 64;
  const int kbeg = by * KR, kend = min(Kc, kbeg + KR);
  const int nsteps = kend > kbeg ? (kend - kbeg + 63) / 64 : 0;
  const __amdgpu_buffer_rsrc_t rin = make_rsrc(IN, static_cast<uint32_t>(uint64_t(M) * ldin * 2));
  const __amdgpu_buffer_rsrc_t rwt =
      make_rsrc(WT, static_cast<uint32_t>(uint64_t(BK ? Kc : r) * ldwt * 2));

  // per-lane row byte offsets of this wave's loads (kOOB for rows past M or r) and the
  // 16-byte chunk each lane fetches; BK, loads of the B tile: the lane's tile row (a
  // contraction offset) in chk and its column's byte offset (kOOB past r) in roff
  uint32_t roff[LPW];
  int chk[LPW];
#pragma unroll
  for (int u = 0; u < LPW; ++u) {
    const int g = wave + 4 * u;            // load index: rows 8 g .. 8 g + 7 of the step tile
    const int x = 8 * g + (lane >> 3);     // staged row
    chk[u] = (lane & 7) ^ ((x & 7) ^ ((x >> 3) & 1));
    if (x < 64) {
      roff[u] = m0 + x < M ? static_cast<uint32_t>(m0 + x) * ldin * 2 : kOOB;
    } else if (!BK) {
      roff[u] = x - 64 < r ? static_cast<uint32_t>(x - 64) * ldwt * 2 : kOOB;
    } else {
      const int byte = (g - 8) * 1024 + lane * 16;
      const int bx = byte / (64 * RT), c = ((byte % (64 * RT)) / 16) ^ s_swz<RT>(bx);
      chk[u] = bx;
      roff[u] = c * 8 < r ? static_cast<uint32_t>(c) * 16 : kOOB;
    }
  }
  auto dma = [&](int step) {
    char *dst = sbuf + (step % NB) * BUF;
    const int kt = kbeg + step * 64;
#pragma unroll
    for (int u = 0; u < LPW; ++u) {
      const int g = wave + 4 * u;
      uint32_t off;
      if (BK && 8 * g >= 64) {
        const int k = kt + chk[u];
        off = (roff[u] != kOOB && k < kend) ? static_cast<uint32_t>(k) * ldwt * 2 + roff[u] : kOOB;
      } else {
        const int k = kt + chk[u] * 8;
        off = (roff[u] != kOOB && k < kend) ? roff[u] + k * 2 : kOOB;
      }
      __builtin_amdgcn_raw_ptr_buffer_load_lds(8 * g < 64 ? rin : rwt,
                                               (__attribute__((address_space(3))) void *)(dst + g * 1024), 16,
                                               off, 0, 0, 0);
    }
  };

  f32x16_t acc[TPW];
#pragma unroll
  for (int u = 0; u < TPW; ++u)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[u][e] = 0.0f;

#pragma unroll
  for (int s = 0; s < NB - 1; ++s) dma(s);
  for (int i = 0; i < nsteps; ++i) {
    // step i has landed for every wave, and no wave still reads buffer (i - 1) % NB
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"((NB - 2) * LPW) : "memory");
    dma(i + NB - 1);
    const char *sb = sbuf + (i % NB) * BUF;
    // all fragments of the step first, then the MFMAs (one LDS latency per step)
    u32x4_t fa[TPW][4], fb[TPW][4];
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const int tile = wave + 4 * u;
      if (TILES % 4 != 0 && tile >= TILES) continue;
      const int ti = tile & 1, tt = tile >> 1;  // row half of IN, rank tile of WT
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int c = 2 * s + (lane >> 5);
        if constexpr (BK)
          fa[u][s] = frag_rows<RT>(sb + 64 * 128, s, 32 * tt);
        else
          fa[u][s] = *reinterpret_cast<const u32x4_t *>(sb + stile_off(64 + 32 * tt + (lane & 31), c));
        fb[u][s] = *reinterpret_cast<const u32x4_t *>(sb + stile_off(32 * ti + (lane & 31), c));
      }
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of the MFMAs
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int u = 0; u < TPW; ++u) {
        const int tile = wave + 4 * u;
        if (TILES % 4 != 0 && tile >= TILES) continue;
        acc[u] = mfma32x32x16(fa[u][s], fb[u][s], acc[u]);
      }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no load may land after the kernel ends

  // partial sums [m][j] of rows m0 .. m0 + 63 (tile t: rows 32 (t & 1), ranks 32 (t >> 1))
  static_assert(64 * (32 * RT * 4 + 16) <= NB * BUF, "partial-sum staging");
  store_partials<64, 32 * RT, TPW, TILES>(
      sbuf, acc, [](int t, int &a0, int &b0) { a0 = 32 * (t & 1); b0 = 32 * (t >> 1); },
      P + static_cast<size_t>(by) * M * r + static_cast<size_t>(m0) * r, r, M - m0, r);
}

template <int RT>
__global__ __launch_bounds__(NT) void lora_down_partial_kernel(
    const uint16_t *__restrict__ IN, int M, int Kc, int ldin, const uint16_t *__restrict__ WT, int ldwt,
    int r, int KR, float *__restrict__ P) {
  __shared__ __attribute__((aligned(16))) char sbuf[staged_bytes<RT>()];
  lora_down_dma_body<RT, staged_nb<RT>()>(sbuf, blockIdx.x, blockIdx.y, IN, M, Kc, ldin, WT, ldwt, r, KR, P);
}

// ---------------------------------------------------------------------------------
// reduce_m: partial sums over a split of rows m of IN[m][no] * S[m][j].
//   JMAJOR = false: P[s][no][j]  (A = S rows j, B = IN columns no)   -> dB [N, r]
//   JMAJOR = true:  P[s][j][no]  (A = IN rows no, B = S columns j)   -> dA [r, K]
// reduce_m with LDS-staged operands: the same partial sums over one M-split, with
// row-major tiles of IN (64 rows m x 64 columns) and S (64 rows m x 32 RT columns)
// brought into LDS by direct buffer -> LDS loads (eight lanes per 128 bytes of a row,
// 16-byte chunks swizzled per row), and the MFMA operands, which need eight consecutive
// m per lane, read with the transposing LDS read: within a 16-lane group, lane i reads 8
// bytes of row base + i / 4 at column 4 (i % 4) of its 16-column half and receives
// column i of those four rows.  NB buffers, one barrier per 64-row step; wave w owns
// output tiles w, w + 4, ... of the 2 x RT tiles of 32 x 32.

template <int RT, bool JMAJOR, int NB>
__device__ __forceinline__ void reduce_m_dma_body(
    char *sbuf, int bx, int by, const uint16_t *__restrict__ IN, int M, int No, int ldin,
    const uint16_t *__restrict__ S, int lds, int r, int MR, float *__restrict__ P) {
  constexpr int INB = 64 * 128;        // IN tile bytes
  constexpr int SROW = 64 * RT;        // S tile row bytes
  constexpr int BUF = INB + 64 * SROW;
  constexpr int NLD = BUF / 1024;      // 1 KB loads per step (8 + 4 RT)
  constexpr int LPW = NLD / 4;
  constexpr int TILES = 2 * RT, TPW = (TILES + 3) / 4;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nb0 = bx * 64;
  const int mb = by * MR, me = min(M, mb + MR);
  const int nsteps = me > mb ? (me - mb + 63) / 64 : 0;
  const __amdgpu_buffer_rsrc_t rin = make_rsrc(IN, static_cast<uint32_t>(uint64_t(M) * ldin * 2));
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(S, static_cast<uint32_t>(uint64_t(M) * lds * 2));

  // per-lane tile row and global column of this wave's loads: load g < 8 covers IN rows
  // 8 g .. 8 g + 7; the others cover 1 KB of the S tile
  int lrow[LPW];
  uint32_t lcol[LPW];  // byte offset of the column inside the global row, kOOB if past the edge
#pragma unroll
  for (int u = 0; u < LPW; ++u) {
    const int g = wave + 4 * u;
    if (g < 8) {
      const int x = 8 * g + (lane >> 3);
      const int c = (lane & 7) ^ ((x & 7) ^ ((x >> 3) & 1));
      lrow[u] = x;
      lcol[u] = nb0 + c * 8 < No ? static_cast<uint32_t>(nb0 + c * 8) * 2 : kOOB;
    } else {
      const int byte = (g - 8) * 1024 + lane * 16;
      const int x = byte / SROW, slot = (byte % SROW) / 16;
      const int c = slot ^ s_swz<RT>(x);
      lrow[u] = x;
      lcol[u] = c * 8 < r ? static_cast<uint32_t>(c * 8) * 2 : kOOB;
    }
  }
  auto dma = [&](int step) {
    char *dst = sbuf + (step % NB) * BUF;
    const int m = mb + step * 64;
#pragma unroll
    for (int u = 0; u < LPW; ++u) {
      const int g = wave + 4 * u;
      const int mm = m + lrow[u];
      const uint32_t ld2 = static_cast<uint32_t>(g < 8 ? ldin : lds) * 2;
      const uint32_t off = (lcol[u] != kOOB && mm < me) ? static_cast<uint32_t>(mm) * ld2 + lcol[u] : kOOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(g < 8 ? rin : rs,
                                               (__attribute__((address_space(3))) void *)(dst + g * 1024), 16, off, 0,
                                               0, 0);
    }
  };
  // operand fragment: column cb + (lane % 32) of rows 16 s + 8 (lane / 32) .. + 7
  auto frag_in = [&](const char *sb, int s, int cb) {
    const int i = lane & 15, gq = lane >> 4;
    const int col = cb + (gq & 1) * 16 + 4 * (i & 3);
    u32x4_t v;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int row = 16 * s + 8 * (gq >> 1) + 4 * e + (i >> 2);
      const int off = row * 128 + (((col >> 3) ^ ((row & 7) ^ ((row >> 3) & 1))) << 4) + (col & 7) * 2;
      const v4i16_t t = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16_t *)(sb + off));
      const u32x2_t w = __builtin_bit_cast(u32x2_t, t);
      v[2 * e] = w[0];
      v[2 * e + 1] = w[1];
    }
    return v;
  };
  auto frag_s = [&](const char *sb, int s, int cb) { return frag_rows<RT>(sb + INB, s, cb); };

  f32x16_t acc[TPW];
#pragma unroll
  for (int u = 0; u < TPW; ++u)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[u][e] = 0.0f;

#pragma unroll
  for (int s = 0; s < NB - 1; ++s) dma(s);
  for (int i = 0; i < nsteps; ++i) {
    // step i has landed for every wave, and no wave still reads buffer (i - 1) % NB
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"((NB - 2) * LPW) : "memory");
    dma(i + NB - 1);
    const char *sb = sbuf + (i % NB) * BUF;
    u32x4_t fi[TPW][4], fs[TPW][4];
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const int tile = wave + 4 * u;
      if (TILES % 4 != 0 && tile >= TILES) continue;
      const int tn = tile & 1, tj = tile >> 1;  // IN column tile, S column (rank) tile
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        fi[u][s] = frag_in(sb, s, 32 * tn);
        fs[u][s] = frag_s(sb, s, 32 * tj);
      }
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of the MFMAs
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int u = 0; u < TPW; ++u) {
        const int tile = wave + 4 * u;
        if (TILES % 4 != 0 && tile >= TILES) continue;
        acc[u] = JMAJOR ? mfma32x32x16(fi[u][s], fs[u][s], acc[u]) : mfma32x32x16(fs[u][s], fi[u][s], acc[u]);
      }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no load may land after the kernel ends

  // tile t: columns 32 (t & 1) of the 64 no, ranks 32 (t >> 1)
  float *dst = P + static_cast<size_t>(by) * No * r;
  if constexpr (!JMAJOR) {  // partial sums [no][j]
    static_assert(64 * (32 * RT * 4 + 16) <= NB * BUF, "partial-sum staging");
    store_partials<64, 32 * RT, TPW, TILES>(
        sbuf, acc, [](int t, int &a0, int &b0) { a0 = 32 * (t & 1); b0 = 32 * (t >> 1); },
        dst + static_cast<size_t>(nb0) * r, r, No - nb0, r);
  } else {  // partial sums [j][no]
    static_assert(32 * RT * (64 * 4 + 16) <= NB * BUF, "partial-sum staging");
    store_partials<32 * RT, 64, TPW, TILES>(
        sbuf, acc, [](int t, int &a0, int &b0) { a0 = 32 * (t >> 1); b0 = 32 * (t & 1); }, dst + nb0, No, r,
        No - nb0);
  }
}

template <int RT, bool JMAJOR>
__global__ __launch_bounds__(NT) void reduce_m_partial_kernel(
    const uint16_t *__restrict__ IN, int M, int No, int ldin, const uint16_t *__restrict__ S, int lds,
    int r, int MR, float *__restrict__ P) {
  __shared__ __attribute__((aligned(16))) char sbuf[staged_bytes<RT>()];
  reduce_m_dma_body<RT, JMAJOR, staged_nb<RT>()>(sbuf, blockIdx.x, blockIdx.y, IN, M, No, ldin, S, lds, r, MR, P);
}

// Transposes of bf16 matrices: OUT[C, R] = IN[R, C]^T.  A workgroup moves one 64 x 64
// tile through LDS: 16-byte row loads when C % 8 == 0 and 16-byte stores when R % 8 == 0,
// element accesses otherwise.
struct TransposeJob {
  const uint16_t *in;
  uint16_t *out;
  int64_t R, C;
  int64_t tiles_c;  // ceil(C / 64)
};

// Tile b (row-major over the 64 x 64 tiles of IN) of job jb, through `tile` (64 rows of
// 72 elements in LDS: 16-byte aligned rows).
__device__ __forceinline__ void transpose_tile(const TransposeJob &jb, int64_t b, uint16_t (*tile)[72]) {
  const int64_t r0 = (b / jb.tiles_c) * 64, c0 = (b % jb.tiles_c) * 64;
  const int tid = threadIdx.x, ch = tid & 7;
  const bool vin = jb.C % 8 == 0, vout = jb.R % 8 == 0;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int rr = (tid >> 3) + 32 * i;
    const int64_t row = r0 + rr, col = c0 + ch * 8;
    u32x4_t v = {0u, 0u, 0u, 0u};
    if (row < jb.R && col < jb.C) {
      const uint16_t *src = jb.in + row * jb.C + col;
      if (vin) {
        v = *reinterpret_cast<const u32x4_t *>(src);
      } else {
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const uint32_t lo = col + e < jb.C ? src[e] : 0u;
          const uint32_t hi = col + e + 1 < jb.C ? src[e + 1] : 0u;
          v[e / 2] = lo | (hi << 16);
        }
      }
    }
    *reinterpret_cast<u32x4_t *>(&tile[rr][ch * 8]) = v;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int cc = (tid >> 3) + 32 * i;  // output row = input column c0 + cc
    const int64_t orow = c0 + cc, ocol = r0 + ch * 8;
    if (orow >= jb.C || ocol >= jb.R) continue;
    uint16_t *dst = jb.out + orow * jb.R + ocol;
    u32x4_t v;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      v[e] = uint32_t(tile[ch * 8 + 2 * e][cc]) | (uint32_t(tile[ch * 8 + 2 * e + 1][cc]) << 16);
    if (vout) {
      *reinterpret_cast<u32x4_t *>(dst) = v;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (ocol + e < jb.R) dst[e] = static_cast<uint16_t>(v[e / 2] >> (16 * (e & 1)));
    }
  }
}

// Two transposes in one launch (workgroups [0, n0) take matrix 0).
__global__ __launch_bounds__(NT) void transpose2_kernel(TransposeJob j0, TransposeJob j1, int64_t n0) {
  __shared__ uint16_t tile[64][72];
  const bool second = blockIdx.x >= n0;
  transpose_tile(second ? j1 : j0, second ? blockIdx.x - n0 : blockIdx.x, tile);
}

// The two products of the backward that read only dY, in one launch: workgroups
// [0, nd) compute the V partials (lora_down over dY and B, read untransposed), the next
// nq the dB partials (reduce over tokens of dY and U_s); the rest transpose A into the
// A^T that the dX GEMM reads afterwards.  Same partial sums as the separate kernels.
struct DownArgs {
  const uint16_t *IN;
  int M, Kc, ldin;
  const uint16_t *WT;
  int ldwt, r, KR;
  float *P;
  int gx;  // row-tile count (first grid dimension of the separate kernel)
};
struct ReduceArgs {
  const uint16_t *IN;
  int M, No, ldin;
  const uint16_t *S;
  int lds, r, MR;
  float *P;
  int gx;
};
template <int RT>
__global__ __launch_bounds__(NT) void down_reduce_partial_kernel(DownArgs d, ReduceArgs q, int nd, int nq,
                                                                 TransposeJob tj) {
  __shared__ __attribute__((aligned(16))) char sbuf[staged_bytes<RT>()];  // used by every body
  static_assert(staged_bytes<RT>() >= 64 * 72 * 2, "transpose tile");
  const int b = blockIdx.x;
  if (b < nd) {
    lora_down_dma_body<RT, staged_nb<RT>(), true>(sbuf, b % d.gx, b / d.gx, d.IN, d.M, d.Kc, d.ldin, d.WT, d.ldwt,
                                                   d.r, d.KR, d.P);
  } else if (b < nd + nq) {
    const int c = b - nd;
    reduce_m_dma_body<RT, false, staged_nb<RT>()>(sbuf, c % q.gx, c / q.gx, q.IN, q.M, q.No, q.ldin, q.S, q.lds,
                                                   q.r, q.MR, q.P);
  } else {
    transpose_tile(tj, b - nd - nq, reinterpret_cast<uint16_t(*)[72]>(sbuf));
  }
}

// OUT = bf16(scale * sum_s P[s]) for the `count` partial sums (count % 4 == 0) laid out
// as rows of `cols` values (cols % 4 == 0), written with row pitch ldout; fixed order
// (split_sum in device_common.h).
__global__ __launch_bounds__(NT) void finalize_kernel(const float *__restrict__ P, int splits,
                                                      int64_t count, int64_t cols, int64_t ldout,
                                                      float scale, uint16_t *__restrict__ OUT) {
  const int64_t n4 = count / 4;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * NT + threadIdx.x; i < n4;
       i += static_cast<int64_t>(gridDim.x) * NT) {
    const f32x4_t s = split_sum(P, splits, count, i);
    u32x2_t o = {pack_bf16x2(s[0] * scale, s[1] * scale), pack_bf16x2(s[2] * scale, s[3] * scale)};
    const int64_t e = 4 * i, row = e / cols, col = e % cols;
    *reinterpret_cast<u32x2_t *>(OUT + row * ldout + col) = o;
  }
}

// Two finalize passes in one launch (the same fixed order and rounding as finalize_kernel).
using FinJob = FinalizeJob;
__global__ __launch_bounds__(NT) void finalize2_kernel(FinJob a, FinJob b) {
  const int64_t na = a.count / 4, n = na + b.count / 4;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * NT + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * NT) {
    if (i < na)
      finalize_one(a, i);
    else
      finalize_one(b, i - na);
  }
}

// ---------------------------------------------------------------------------------
// Generic kernels (any row length or rank): simple and unvectorized.
__device__ __forceinline__ u32x4_t load8(const uint16_t *p, int64_t rows, int64_t cols, int64_t ld,
                                         int64_t row, int64_t col) {
  u32x4_t v = {0u, 0u, 0u, 0u};
  if (row >= rows || col >= cols) return v;
  const uint16_t *src = p + row * ld + col;
  uint16_t t[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) t[e] = (col + e < cols) ? src[e] : uint16_t(0);
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = uint32_t(t[2 * e]) | (uint32_t(t[2 * e + 1]) << 16);
  return v;
}

// OUT[M, r] = bf16(scale * IN[M, Kc] . WT[r, Kc]^T); one wave per 32 rows.
template <int RT>
__global__ __launch_bounds__(NT) void lora_down_generic_kernel(
    const uint16_t *__restrict__ IN, int64_t M, int64_t Kc, int64_t ldin, const uint16_t *__restrict__ WT,
    int64_t ldwt, int r, float scale, uint16_t *__restrict__ OUT, int64_t ldout) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 128 + wave * 32 + (lane & 31);
  f32x16_t acc[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[t][e] = 0.0f;
  for (int64_t k = 0; k < Kc; k += 16) {
    const int64_t kk = k + (lane >> 5) * 8;
    const u32x4_t a = load8(IN, M, Kc, ldin, row, kk);
#pragma unroll
    for (int t = 0; t < RT; ++t)
      acc[t] = mfma32x32x16(a, load8(WT, r, Kc, ldwt, t * 32 + (lane & 31), kk), acc[t]);
  }
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    const int col = t * 32 + (lane & 31);
    if (col >= r) continue;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int64_t orow = static_cast<int64_t>(blockIdx.x) * 128 + wave * 32 + (e >> 2) * 8 +
                           (lane >> 5) * 4 + (e & 3);
      if (orow < M) OUT[orow * ldout + col] = to_bf16(acc[t][e] * scale);
    }
  }
}

// P[s][no][j] over splits of 256 rows, staged element-wise through LDS.
constexpr int GMS = 256;
template <int RT>
__global__ __launch_bounds__(NT) void reduce_m_generic_kernel(
    const uint16_t *__restrict__ IN, int64_t M, int64_t No, int64_t ldin, const uint16_t *__restrict__ S,
    int64_t lds, int r, float *__restrict__ P) {
  __shared__ uint16_t sIn[32][128 + 2];
  __shared__ uint16_t sS[32][RT * 32 + 2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t c0 = static_cast<int64_t>(blockIdx.x) * 128;
  const int64_t s_idx = blockIdx.y;
  const int64_t mbeg = s_idx * GMS, mend = min<int64_t>(M, mbeg + GMS);
  f32x16_t acc[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[t][e] = 0.0f;
  for (int64_t mb = mbeg; mb < mend; mb += 32) {
    __syncthreads();
    for (int i = tid; i < 32 * 128; i += NT) {
      const int rr = i / 128, cc = i % 128;
      const int64_t m = mb + rr, c = c0 + cc;
      sIn[rr][cc] = (m < mend && c < No) ? IN[m * ldin + c] : uint16_t(0);
    }
    for (int i = tid; i < 32 * RT * 32; i += NT) {
      const int rr = i / (RT * 32), cc = i % (RT * 32);
      const int64_t m = mb + rr;
      sS[rr][cc] = (m < mend && cc < r) ? S[m * lds + cc] : uint16_t(0);
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int mm = ks * 16 + (lane >> 5) * 8;
      const int ac = wave * 32 + (lane & 31);
      u32x4_t a;
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

__global__ __launch_bounds__(NT) void reduce_m_generic_final_kernel(
    const float *__restrict__ P, int64_t splits, int64_t No, int r, uint16_t *__restrict__ OUT,
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

// ---- split selection (shared by the workspace queries and the launches) -----------
struct DownSplit {
  int ksplit, KR;
};
DownSplit down_split(int64_t M, int64_t Kc) {
  const int64_t row_tiles = (M + 63) / 64;
  int64_t ks = (kDownWGs + row_tiles - 1) / row_tiles;
  const int64_t kmax = (Kc + 255) / 256;
  if (ks > kmax) ks = kmax;
  if (ks < 1) ks = 1;
  int64_t KR = ((Kc + ks - 1) / ks + 63) / 64 * 64;
  ks = (Kc + KR - 1) / KR;
  return {static_cast<int>(ks), static_cast<int>(KR)};
}

struct MSplit {
  int splits, MR;
};
MSplit m_split(int64_t M, int64_t No) {
  const int64_t tiles = (No + 63) / 64;
  int64_t sp = (512 + tiles - 1) / tiles;
  const int64_t smax = (M + 63) / 64;
  if (sp > smax) sp = smax;
  if (sp < 1) sp = 1;
  int64_t MR = ((M + sp - 1) / sp + 31) / 32 * 32;
  sp = (M + MR - 1) / MR;
  return {static_cast<int>(sp), static_cast<int>(MR)};
}

bool down_fast(int64_t M, int64_t Kc, int64_t ldin, int64_t ldwt, int r, int64_t ldout) {
  return Kc % 8 == 0 && r % 8 == 0 && ldin % 8 == 0 && ldwt % 8 == 0 && ldout % 4 == 0 &&
         uint64_t(M) * ldin * 2 <= k4G && uint64_t(r) * ldwt * 2 <= k4G && M < (int64_t(1) << 30) &&
         ldin < (int64_t(1) << 30) && ldwt < (int64_t(1) << 30);
}
bool reduce_fast(int64_t M, int64_t No, int64_t ldin, int64_t lds, int r) {
  return No % 8 == 0 && r % 8 == 0 && ldin % 8 == 0 && lds % 8 == 0 && uint64_t(M) * ldin * 2 <= k4G &&
         uint64_t(M) * lds * 2 <= k4G && No < (int64_t(1) << 30) && ldin < (int64_t(1) << 30) &&
         lds < (int64_t(1) << 30);
}

hipError_t launch_finalize(const float *P, int splits, int64_t count, int64_t cols, int64_t ldout,
                           float scale, uint16_t *OUT, hipStream_t stream) {
  int64_t blocks = (count / 4 + NT - 1) / NT;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(finalize_kernel, dim3(static_cast<unsigned>(blocks)), dim3(NT), 0, stream, P,
                     splits, count, cols, ldout, scale, OUT);
  return hipGetLastError();
}

}  // namespace

// Sized for dense operands: any strided call that takes the fast path is also fast
// dense (the pitches only add conditions), so the same bound holds for slices.
size_t lora_down_workspace(int64_t M, int64_t Kc, int r) {
  if (r <= 0 || !down_fast(M, Kc, Kc, Kc, r, r)) return 0;
  return static_cast<size_t>(down_split(M, Kc).ksplit) * M * r * sizeof(float);
}

hipError_t launch_lora_down(const uint16_t *IN, int64_t M, int64_t Kc, int64_t ldin, const uint16_t *WT,
                            int64_t ldwt, int r, float scale, uint16_t *OUT, int64_t ldout, float *ws,
                            hipStream_t stream) {
  const int rt = (r + 31) / 32;
  if (rt < 1 || rt > 8) return hipErrorInvalidValue;
  if (down_fast(M, Kc, ldin, ldwt, r, ldout)) {
    const DownSplit sp = down_split(M, Kc);
    dim3 grid(static_cast<unsigned>((M + 63) / 64), static_cast<unsigned>(sp.ksplit)), block(NT);
    switch (rt) {
#define QLORA_CASE(T)                                                                            \
  case T:                                                                                        \
    hipLaunchKernelGGL(lora_down_partial_kernel<T>, grid, block, 0, stream, IN,                  \
                       static_cast<int>(M), static_cast<int>(Kc), static_cast<int>(ldin), WT,     \
                       static_cast<int>(ldwt), r, sp.KR, ws);                                     \
    break;
      QLORA_CASE(1) QLORA_CASE(2) QLORA_CASE(3) QLORA_CASE(4)
      QLORA_CASE(5) QLORA_CASE(6) QLORA_CASE(7) QLORA_CASE(8)
#undef QLORA_CASE
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_finalize(ws, sp.ksplit, M * r, r, ldout, scale, OUT, stream);
  }
  dim3 grid(static_cast<unsigned>((M + 127) / 128)), block(NT);
  switch (rt) {
#define QLORA_CASE(T)                                                                         \
  case T:                                                                                     \
    hipLaunchKernelGGL(lora_down_generic_kernel<T>, grid, block, 0, stream, IN, M, Kc, ldin, WT, \
                       ldwt, r, scale, OUT, ldout);                                              \
    break;
    QLORA_CASE(1) QLORA_CASE(2) QLORA_CASE(3) QLORA_CASE(4)
    QLORA_CASE(5) QLORA_CASE(6) QLORA_CASE(7) QLORA_CASE(8)
#undef QLORA_CASE
  }
  return hipGetLastError();
}

hipError_t launch_transpose2_bf16(const uint16_t *IN0, int64_t R0, int64_t C0, uint16_t *OUT0, const uint16_t *IN1,
                                  int64_t R1, int64_t C1, uint16_t *OUT1, hipStream_t stream) {
  TransposeJob j0{IN0, OUT0, R0, C0, (C0 + 63) / 64}, j1{IN1, OUT1, R1, C1, (C1 + 63) / 64};
  const int64_t n0 = IN0 ? ((R0 + 63) / 64) * j0.tiles_c : 0;
  const int64_t n1 = IN1 ? ((R1 + 63) / 64) * j1.tiles_c : 0;
  if (n0 + n1 == 0) return hipSuccess;
  if (n0 + n1 > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(transpose2_kernel, dim3(static_cast<unsigned>(n0 + n1)), dim3(NT), 0, stream, j0, j1, n0);
  return hipGetLastError();
}

size_t reduce_m_workspace(int64_t M, int64_t No, int r) {
  if (r <= 0) return 0;
  if (reduce_fast(M, No, No, r, r)) return static_cast<size_t>(m_split(M, No).splits) * No * r * sizeof(float);
  const int64_t splits = (M + GMS - 1) / GMS;
  return static_cast<size_t>(splits) * No * r * sizeof(float);
}

hipError_t launch_reduce_m(const uint16_t *IN, int64_t M, int64_t No, int64_t ldin, const uint16_t *S,
                           int64_t lds, int r, float *partials, uint16_t *OUT, bool trans_out,
                           hipStream_t stream, FinalizeJob *defer) {
  if (defer) defer->splits = 0;
  const int rt = (r + 31) / 32;
  if (rt < 1 || rt > 8) return hipErrorInvalidValue;
  if (reduce_fast(M, No, ldin, lds, r)) {
    const MSplit sp = m_split(M, No);
    dim3 grid(static_cast<unsigned>((No + 63) / 64), static_cast<unsigned>(sp.splits)), block(NT);
    const int Mi = static_cast<int>(M), Noi = static_cast<int>(No);
    const int Ldi = static_cast<int>(ldin), Lds = static_cast<int>(lds);
    switch (rt * 2 + (trans_out ? 1 : 0)) {
#define QLORA_CASE(T)                                                                              \
  case 2 * T:                                                                                      \
    hipLaunchKernelGGL((reduce_m_partial_kernel<T, false>), grid, block, 0, stream, IN, Mi, Noi,    \
                       Ldi, S, Lds, r, sp.MR, partials);                                           \
    break;                                                                                         \
  case 2 * T + 1:                                                                                  \
    hipLaunchKernelGGL((reduce_m_partial_kernel<T, true>), grid, block, 0, stream, IN, Mi, Noi,     \
                       Ldi, S, Lds, r, sp.MR, partials);                                           \
    break;
      QLORA_CASE(1) QLORA_CASE(2) QLORA_CASE(3) QLORA_CASE(4)
      QLORA_CASE(5) QLORA_CASE(6) QLORA_CASE(7) QLORA_CASE(8)
#undef QLORA_CASE
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // [No, r] (or [r, No] for trans_out) dense rows
    if (defer) {
      *defer = FinalizeJob{partials, sp.splits, No * r, No * r, No * r, 1.0f, OUT};
      return hipSuccess;
    }
    return launch_finalize(partials, sp.splits, No * r, No * r, No * r, 1.0f, OUT, stream);
  }
  const int64_t splits = (M + GMS - 1) / GMS;
  dim3 grid(static_cast<unsigned>((No + 127) / 128), static_cast<unsigned>(splits)), block(NT);
  switch (rt) {
#define QLORA_CASE(T)                                                                            \
  case T:                                                                                        \
    hipLaunchKernelGGL(reduce_m_generic_kernel<T>, grid, block, 0, stream, IN, M, No, ldin, S, \
                       lds, r, partials);                                                        \
    break;
    QLORA_CASE(1) QLORA_CASE(2) QLORA_CASE(3) QLORA_CASE(4)
    QLORA_CASE(5) QLORA_CASE(6) QLORA_CASE(7) QLORA_CASE(8)
#undef QLORA_CASE
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  int64_t fb = (No * r + NT - 1) / NT;
  if (fb > 4096) fb = 4096;
  hipLaunchKernelGGL(reduce_m_generic_final_kernel, dim3(static_cast<unsigned>(fb)), dim3(NT), 0,
                     stream, partials, splits, No, r, OUT, trans_out);
  return hipGetLastError();
}

bool vdb_fast(int64_t M, int64_t Np, int64_t ldy, int64_t ldu, int r) {
  // B [Np, r] is read with row pitch r (its part of a stacked B)
  return down_fast(M, Np, ldy, r, r, ldu) && reduce_fast(M, Np, ldy, ldu, r) && uint64_t(Np) * r * 2 <= k4G;
}

size_t vdb_workspace_v(int64_t M, int64_t Np, int r) {
  return static_cast<size_t>(down_split(M, Np).ksplit) * M * r * sizeof(float);
}
size_t vdb_workspace_db(int64_t M, int64_t Np, int r) {
  return static_cast<size_t>(m_split(M, Np).splits) * Np * r * sizeof(float);
}

hipError_t launch_vdb(const uint16_t *dY, int64_t M, int64_t Np, int64_t ldy, const uint16_t *B, const uint16_t *U,
                      int64_t ldu, int r, float scale, uint16_t *V, uint16_t *dB, float *ws_v, float *ws_db,
                      const uint16_t *A, int64_t RA, int64_t KA, uint16_t *At, hipStream_t stream) {
  const int rt = (r + 31) / 32;
  if (rt < 1 || rt > 8 || !vdb_fast(M, Np, ldy, ldu, r)) return hipErrorInvalidValue;
  const DownSplit sd = down_split(M, Np);
  const MSplit sq = m_split(M, Np);
  DownArgs d{dY, static_cast<int>(M), static_cast<int>(Np), static_cast<int>(ldy), B, r, r,
             sd.KR, ws_v, static_cast<int>((M + 63) / 64)};
  ReduceArgs q{dY, static_cast<int>(M), static_cast<int>(Np), static_cast<int>(ldy), U, static_cast<int>(ldu), r,
               sq.MR, ws_db, static_cast<int>((Np + 63) / 64)};
  const TransposeJob tj{A, At, RA, KA, (KA + 63) / 64};
  const int64_t nd = int64_t(d.gx) * sd.ksplit, nq = int64_t(q.gx) * sq.splits;
  const int64_t nt = (A && At) ? ((RA + 63) / 64) * tj.tiles_c : 0;
  if (nd + nq + nt > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(nd + nq + nt)), block(NT);
  switch (rt) {
#define QLORA_CASE(T)                                                                          \
  case T:                                                                                      \
    hipLaunchKernelGGL(down_reduce_partial_kernel<T>, grid, block, 0, stream, d, q, static_cast<int>(nd), \
                       static_cast<int>(nq), tj);                                              \
    break;
    QLORA_CASE(1) QLORA_CASE(2) QLORA_CASE(3) QLORA_CASE(4)
    QLORA_CASE(5) QLORA_CASE(6) QLORA_CASE(7) QLORA_CASE(8)
#undef QLORA_CASE
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // V = bf16(scale sum P_V) as [M, r] rows of pitch ldu; dB = bf16(sum P_dB) dense [Np, r]
  const FinJob fv{ws_v, sd.ksplit, M * r, r, ldu, scale, V};
  const FinJob fb{ws_db, sq.splits, Np * r, Np * r, Np * r, 1.0f, dB};
  int64_t blocks = ((fv.count + fb.count) / 4 + NT - 1) / NT;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(finalize2_kernel, dim3(static_cast<unsigned>(blocks)), dim3(NT), 0, stream, fv, fb);
  return hipGetLastError();
}

}  // namespace qlora
