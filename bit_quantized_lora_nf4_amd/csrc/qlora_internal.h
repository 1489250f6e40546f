// Internal declarations shared by the host API and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qlora {

constexpr int kBlock = 64;     // weights per first-level block
constexpr int kGroup = 256;    // block constants per double-quantization group
constexpr int kBuckets = 129;  // quantizer bucket table entries (x in [-1, 1])
constexpr int kMaxRank = 256;  // largest LoRA rank
// Bytes at the start of every workspace layout reserved for the small-M forward's
// cross-workgroup counters; no other kernel writes them.
constexpr size_t kGemvSyncBytes = 256 + 4096 * 16;  // QLORA_WORKSPACE_HEADER_BYTES

// Level tables of the 4-bit codes and encodings of the block constants (the values
// of the weight descriptor's quant_type and const_type).
enum : int { kQuantNF4 = 0, kQuantFP4 = 1 };
enum : int { kConstDqInt8 = 0, kConstDqFp8 = 1, kConstF32 = 2 };

struct Codebook {
  float q[16];                  // levels, ascending
  float thr[15];                // decision thresholds
  float bucket_thr[kBuckets];   // the threshold inside each bucket window (2.0 if none)
  int bucket_base[kBuckets];    // thresholds below each bucket window
  bool bucket_ok;               // every window holds at most one threshold
};

// kQuantNF4 or kQuantFP4 (any other value: NF4).
const Codebook &codebook(int quant_type = kQuantNF4);

// Kernel arguments passed by value (kernarg segment).
struct QuantTable {
  float thr[kBuckets];
  int base[kBuckets];
};
struct LevelTable {
  float q[16];
};
LevelTable level_table(int quant_type);

// Device view of a quantized weight.  Double-quantized constants (kConstDqInt8,
// kConstDqFp8) use absmax_q / dq_scale / dq_offset; kConstF32 uses absmax.
struct WeightView {
  const uint8_t *codes;
  const int8_t *absmax_q;
  const float *dq_scale;
  const float *dq_offset;
  int64_t n_rows;  // N = d_out
  int64_t n_cols;  // K = d_in
  const float *absmax;
  int quant_type;
  int const_type;
};

// ---- launchers (each returns the HIP error of its launches) -----------------
// absmax_f32 receives the fp32 block constants (required for kConstF32, optional
// otherwise); absmax_q / dq_scale / dq_offset are written for the double-quantized types.
hipError_t launch_quantize(const void *W, bool w_bf16, int64_t n_rows, int64_t n_cols, int quant_type,
                           int const_type, uint8_t *codes, int8_t *absmax_q, float *dq_scale,
                           float *dq_offset, float *absmax_f32, hipStream_t stream);
hipError_t launch_dequantize(const WeightView &w, void *out, bool out_bf16, hipStream_t stream);

// OUT[M, r] (row pitch ldout, bf16) = bf16(scale * IN[M, Kc] . WT[r, Kc]^T);  IN rows
// have pitch ldin, WT rows pitch ldwt (column slices of wider matrices are allowed).
// `ws` holds lora_down_workspace(M, Kc, r) bytes of fp32 partial sums.
size_t lora_down_workspace(int64_t M, int64_t Kc, int r);
hipError_t launch_lora_down(const uint16_t *IN, int64_t M, int64_t Kc, int64_t ldin, const uint16_t *WT,
                            int64_t ldwt, int r, float scale, uint16_t *OUT, int64_t ldout, float *ws,
                            hipStream_t stream);
// OUT_q[C_q, R_q] = IN_q[R_q, C_q]^T for two bf16 matrices (dense row-major) in one
// launch; IN1 may be NULL (one transpose).
hipError_t launch_transpose2_bf16(const uint16_t *IN0, int64_t R0, int64_t C0, uint16_t *OUT0, const uint16_t *IN1,
                                  int64_t R1, int64_t C1, uint16_t *OUT1, hipStream_t stream);
// The last pass of a split reduction: OUT = bf16(scale * (P_0 + P_1 + ...)) for the
// `count` partial sums of each of `splits` splits (count % 4 == 0), laid out as rows of
// `cols` values written with row pitch ldout.  splits == 0: nothing to do.
struct FinalizeJob {
  const float *P;
  int splits;
  int64_t count, cols, ldout;
  float scale;
  uint16_t *OUT;
};
// Workgroups of 256 threads a finalize job is spread over when it rides in another
// launch (the dX GEMM's); finalize_part (device_common.h) does one workgroup's share.
inline int64_t finalize_workgroups(const FinalizeJob &j) {
  if (j.splits <= 0) return 0;
  const int64_t w = (j.count / 4 + 4 * 256 - 1) / (4 * 256);  // four groups of four values per thread
  return w < 1 ? 1 : w;
}

// P[s][No][r] fp32 partials of sum over m in split s of IN[m][no] * S[m][j]; then
// OUT = bf16(sum_s P) written as [No, r] (trans_out = false) or [r, No] (true).
// IN rows have pitch ldin, S rows pitch lds.  If `defer` is not NULL and the fast path
// runs, the finalize pass is not launched but described in *defer (else defer->splits
// is 0), for a later launch to do.
size_t reduce_m_workspace(int64_t M, int64_t No, int r);
hipError_t launch_reduce_m(const uint16_t *IN, int64_t M, int64_t No, int64_t ldin, const uint16_t *S,
                           int64_t lds, int r, float *partials, uint16_t *OUT, bool trans_out,
                           hipStream_t stream, FinalizeJob *defer = nullptr);

// The backward's two products over dY in one launch plus one finalize launch:
// V[M, r] (row pitch ldu) = bf16(scale dY B) and dB[Np, r] = bf16(dY^T U), where dY has
// row pitch ldy (a column slice of width Np), B is [Np, r] (dense rows) and U [M, r]
// with row pitch ldu.  If A and At are given, the same launch also writes At[KA, RA] =
// A[RA, KA]^T.  Needs the fast-path shapes (vdb_fast) and the two fp32 partial regions
// sized by vdb_workspace_v / vdb_workspace_db.
bool vdb_fast(int64_t M, int64_t Np, int64_t ldy, int64_t ldu, int r);
size_t vdb_workspace_v(int64_t M, int64_t Np, int r);
size_t vdb_workspace_db(int64_t M, int64_t Np, int r);
hipError_t launch_vdb(const uint16_t *dY, int64_t M, int64_t Np, int64_t ldy, const uint16_t *B, const uint16_t *U,
                      int64_t ldu, int r, float scale, uint16_t *V, uint16_t *dB, float *ws_v, float *ws_db,
                      const uint16_t *A, int64_t RA, int64_t KA, uint16_t *At, hipStream_t stream);

// AdamW step (fp32 parameter and moments, bf16 gradient, optional bf16 parameter copy).
struct AdamConsts {
  float decay, b1, ob1, b2, ob2, step_size, bc2s, eps;
};
hipError_t launch_adamw(float *p, uint16_t *pb, const uint16_t *g, float *m, float *v, int64_t n,
                        const AdamConsts &c, hipStream_t stream);

// LoRA merge / unmerge of one adapter into a bf16 weight [N, K]:
// out = bf16(W' + scale . B A) from the NF4 weight, or bf16(Wm - scale . B A).
hipError_t launch_lora_merge(const WeightView &w, const uint16_t *A, const uint16_t *B, int r,
                             float scale, uint16_t *out, hipStream_t stream);
hipError_t launch_lora_unmerge(const uint16_t *Wm, int64_t n_rows, int64_t n_cols, const uint16_t *A,
                               const uint16_t *B, int r, float scale, uint16_t *out,
                               hipStream_t stream);

// Whether the fused GEMMs take this shape: X or dY, Y or dX, the codes and the LoRA
// operands (rank or row pitch r) below 0xFFFFFFF0 bytes each (32-bit buffer offsets).
bool gemm_supported(const WeightView &w, int64_t M, int r);
// Y[M, N] = bf16(X . W'^T + U . Bl^T)  (U [M, r] pitch ldu, Bl [N, r]); r may be 0.
// part_rows > 0 (a multiple of 256 dividing N): output rows of part q = n / part_rows
// use U columns [q r, q r + r) (horizontally fused linears with stacked adapters).
hipError_t launch_gemm_fwd(const WeightView &w, const uint16_t *X, int64_t M, const uint16_t *U,
                           int ldu, const uint16_t *Bl, int r, int64_t part_rows, uint16_t *Y,
                           hipStream_t stream);
// Small-M forward (M <= 16) in one launch: Y = bf16(X W'^T + U_s Bl^T) and
// U_s = bf16(scale X A^T) (written to U_saved if not NULL) over the R stacked ranks of
// A; output row n uses U_s columns [q r, q r + r), q = n / part_rows (part_rows = 0:
// one linear, R = r).  `ws` holds gemv_workspace bytes: a kGemvSyncBytes header of
// counters and flags that must be zero when the call starts (every call leaves it
// zero), then copies of U_s and the partial sums of the down-projection.
// The small-M forward runs for M <= 16 and up to 4096 tiles of 16 output rows (one flag
// word per workgroup in the header); other shapes take the fused GEMM.
inline bool gemv_shape_ok(int64_t M, int64_t N) { return M >= 1 && M <= 16 && (N + 15) / 16 <= 4096; }
size_t gemv_workspace(int64_t M, int64_t K, int64_t N, int r);
bool gemv_supported(const WeightView &w, int64_t M, int r);
hipError_t launch_gemv(const WeightView &w, const uint16_t *X, int64_t M, const uint16_t *A, int R,
                       const uint16_t *Bl, int r, int64_t part_rows, float scale, uint16_t *Y,
                       uint16_t *U_saved, void *ws, hipStream_t stream);
// dX[M, K] = bf16(dY . W' + V . At^T)  (V [M, r], At [K, r]); r may be 0.  A finalize
// job (NULL or splits == 0: none) runs in extra workgroups after the GEMM's tiles.
hipError_t launch_gemm_dx(const WeightView &w, const uint16_t *dY, int64_t M, const uint16_t *V,
                          const uint16_t *At, int r, uint16_t *dX, hipStream_t stream,
                          const FinalizeJob *fin = nullptr);

}  // namespace qlora
