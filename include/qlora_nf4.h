/*
 * qlora_nf4.h -- C ABI of the MI355X (gfx950) QLoRA linear library.
 *
 * The library computes the frozen-base QLoRA linear layer
 *
 *     Y = X . W'^T + (alpha / r) . (X . A^T) . B^T
 *
 * where W' is the bf16 decode of a weight stored as blockwise NF4 codes with
 * 8-bit double-quantized block constants.  Pages cited below:
 *   [QLoRA note]  "1. 啥是 QLoRA" (p19e99.github.io/posts/note/qlora)
 *   [Ch. 11.3]    "11.3 QLoRA：单卡微调大模型" (gheillcoat.github.io)
 *   [Paper note]  "QLoRA — 让 65B 大模型微调落到单张 48GB GPU 上" (awesome.papernotes.org)
 *   [Digest]      "QLoRA: 高效微调量化大语言模型" (aipaper.cc)
 *   [Repro]       "LoRA / QLoRA低秩更新、量化和显存预算" (mhpn.cn)
 *
 * Conventions (all entry points):
 *   - Shapes follow [Repro] "LoRA 的公式和张量形状": the weight is W[N = d_out,
 *     K = d_in] row-major (K contiguous); A is [r, K], B is [N, r], X is
 *     [M, K], Y and dY are [M, N].  All matrices are dense row-major.
 *   - bf16 tensors are passed as uint16_t bit patterns.
 *   - Every tensor pointer is a DEVICE pointer owned by the caller, 16-byte
 *     aligned.  The library never allocates or frees memory; scratch memory
 *     comes from the caller's workspace (qlora_linear_fwd_noalloc alone uses a
 *     fixed scratch array of the library instead).
 *   - Workspaces: the first QLORA_WORKSPACE_HEADER_BYTES bytes of every
 *     workspace hold counters and flags that the small-M forward's workgroups
 *     use to hand U_s to each other.  They must be zero when a workspace is
 *     first used (clear it once after allocating); every call leaves them
 *     zero, and no other call writes them, so one workspace can serve calls of
 *     any shape.  Calls that share a workspace must not overlap.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Each call checks
 *     its arguments on the host, then enqueues its kernels asynchronously on
 *     `stream` and returns.  Kernel faults surface at the caller's next
 *     synchronisation.  Host code never synchronises.
 *   - Return value: QLORA_OK (0) or a negative qlora_status; on error nothing
 *     was enqueued (except QLORA_ERR_LAUNCH, where an earlier kernel of the
 *     same call may already be queued).  qlora_last_error() gives a
 *     thread-local message for the last failing call of this thread.
 *   - Outputs must not alias inputs.  Inputs must be finite.
 *   - K (= n_cols) must be a multiple of 64; M >= 1; 0 <= r <= 256 (r = 0
 *     means no adapter: A, B may be NULL).
 */
#ifndef QLORA_NF4_H
#define QLORA_NF4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QLORA_OK = 0,
  QLORA_ERR_NULL = -1,      /* a required pointer is NULL                        */
  QLORA_ERR_SHAPE = -2,     /* M < 1, n_rows < 1, n_cols % 64 != 0, size overflow */
  QLORA_ERR_RANK = -3,      /* r outside [0, 256] or alpha not finite             */
  QLORA_ERR_DTYPE = -4,     /* unsupported dtype enum                             */
  QLORA_ERR_WORKSPACE = -5, /* workspace smaller than qlora_workspace_bytes()     */
  QLORA_ERR_ALIGN = -6,     /* a pointer is not 16-byte aligned                   */
  QLORA_ERR_DEVICE = -7,    /* no usable gfx950 device                            */
  QLORA_ERR_LAUNCH = -8,    /* the HIP runtime refused a kernel launch            */
  QLORA_ERR_VALUE = -9      /* a scalar argument is out of range                  */
} qlora_status;

typedef enum { QLORA_F32 = 0, QLORA_BF16 = 1 } qlora_dtype;

/* Data-type variants of the stored weight, after the data-type comparison of [Digest]
 * "6. 实验结果与分析" ("核心结果分析" item 2: Float4, NF4, NF4 with double quantization)
 * and the FP8 notation of the second-level codes in [Digest] "数学公式与关键细节" item 2.
 * The pages fix neither value set; the library's readings:
 *   QLORA_QUANT_FP4      the E2M1 float (magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6, signed)
 *                        divided by 6; levels -1, -2/3, -1/2, -1/3, -1/4, -1/6, -1/12, 0,
 *                        0, 1/12, 1/6, 1/4, 1/3, 1/2, 2/3, 1 (each rounded once to fp32)
 *   QLORA_CONST_DQ_FP8   the double quantization with E4M3 second-level codes (bias 7, 3
 *                        mantissa bits, subnormals, largest value 448): s = RN(h / 448),
 *                        code = E4M3 nearest to RN(RN(c - o) / s) (ties to the even code,
 *                        saturated at 448; sign bit set for a negative value),
 *                        c' = fma(e4m3(code), s, o)
 *   QLORA_CONST_FP32     no double quantization: c' = c, stored as fp32 */
typedef enum { QLORA_QUANT_NF4 = 0, QLORA_QUANT_FP4 = 1 } qlora_quant_type;
typedef enum { QLORA_CONST_DQ_INT8 = 0, QLORA_CONST_DQ_FP8 = 1, QLORA_CONST_FP32 = 2 } qlora_const_type;

enum { QLORA_BLOCK = 64, QLORA_GROUP = 256, QLORA_MAX_RANK = 256, QLORA_MAX_PARTS = 8 };

/* A quantized weight W[n_rows = d_out, n_cols = d_in] ([Digest] "数学公式与关键细节"
 * items 1-2; [Ch. 11.3] "核心创新二").  Block b holds the 64 consecutive elements
 * [64 b, 64 b + 64) of the row-major weight; group g holds blocks [256 g, 256 g + 256).
 *   codes      [n_rows * n_cols / 2]   byte i = code(2i) | code(2i+1) << 4
 *   absmax_q   [n_blocks]              8-bit double-quantized block constant: int8
 *                                      (QLORA_CONST_DQ_INT8) or an E4M3 byte (_DQ_FP8)
 *   dq_scale   [n_groups]              fp32 group scale s        (double-quantized types)
 *   dq_offset  [n_groups]              fp32 group offset o       (double-quantized types)
 *   absmax     [n_blocks]              fp32 block constant c     (QLORA_CONST_FP32 only)
 *   quant_type                         level table q: QLORA_QUANT_NF4 or QLORA_QUANT_FP4
 *   const_type                         QLORA_CONST_DQ_INT8, _DQ_FP8 or _FP32
 * Arrays a type does not use may be NULL.  A zero tail (types 0, absmax NULL) is the
 * NF4 weight with int8 double quantization.  fp32 arrays must be 4-byte aligned.
 * Block constant decode: c' = fma(absmax_q[b], s[g], o[g]) (int8; one rounding),
 *                        c' = fma(e4m3(absmax_q[b]), s[g], o[g]) (FP8), c' = absmax[b].
 * Weight decode:          W'  = bf16_rne(q[code] * c')   (fp32 product, RN). */
typedef struct {
  const uint8_t *codes;
  const int8_t *absmax_q;
  const float *dq_scale;
  const float *dq_offset;
  int64_t n_rows;
  int64_t n_cols;
  const float *absmax;
  int32_t quant_type;
  int32_t const_type;
} qlora_nf4_weight;

/* ---- host-only helpers (no GPU needed) ------------------------------------ */

/* Storage sizes of an n_rows x n_cols weight.  Any output pointer may be NULL.
 * Returns QLORA_ERR_SHAPE unless n_rows >= 1 and n_cols is a positive multiple of 64. */
int qlora_nf4_sizes(int64_t n_rows, int64_t n_cols, size_t *code_bytes, int64_t *n_blocks,
                    int64_t *n_groups);

/* The NF4 codebook q[0..15] (ascending; q[0] = -1, q[7] = 0, q[15] = +1) and the 15
 * decision thresholds T[j] = largest fp32 <= (q[j] + q[j+1]) / 2, computed by the
 * library in double precision from N(0,1) quantiles ([QLoRA note] "2. NF4";
 * [Paper note] "关键设计 1", quantile-midpoint equation; [Digest] item 1, "特点":
 * exact zero through asymmetric halves).  Either pointer may be NULL. */
void qlora_nf4_codebook(float q[16], float thresholds[15]);

/* The level table and thresholds of quant_type (QLORA_QUANT_NF4: as qlora_nf4_codebook;
 * QLORA_QUANT_FP4: the E2M1 / 6 levels above, thresholds by the same rule, the one
 * between the two zeros being 0).  QLORA_ERR_DTYPE for another quant_type. */
int qlora_codebook(int quant_type, float q[16], float thresholds[15]);

/* Bytes of caller workspace needed by qlora_linear_fwd (op = 0) or qlora_linear_bwd
 * (op = 1) for the given shapes; 0 for invalid arguments. */
size_t qlora_workspace_bytes(int op, int64_t M, int64_t K, int64_t N, int r);

/* Bytes of caller workspace for qlora_linear_fwd_fused (op = 0) or
 * qlora_linear_bwd_fused (op = 1): N is the fused row count, r the rank of each part. */
size_t qlora_workspace_bytes_fused(int op, int64_t M, int64_t K, int64_t N, int r, int n_parts);

const char *qlora_status_string(int status);
const char *qlora_last_error(void);

/* Timing hook for measurement tools.  Arms the calling thread so that its next
 * fused NF4 GEMM launch (the main kernel of qlora_linear_fwd or of the dX part of
 * qlora_linear_bwd) is bracketed by hipEventRecord(start) and hipEventRecord(stop)
 * on that call's stream; the hook then disarms itself.  The events are hipEvent_t
 * handles owned by the caller; passing NULL disarms.  No effect on results. */
void qlora_time_next_gemm(void *start_event, void *stop_event);

/* ---- device entry points ---------------------------------------------------- */

/* Blockwise NF4 quantization plus double quantization of the block constants
 * ([QLoRA note] "2. NF4", "3. 双重量化"; [Digest] "数学公式与关键细节" items 1-2).
 *   W         [n_rows, n_cols] fp32 (w_dtype = QLORA_F32) or bf16 (QLORA_BF16)
 *   per block: c = max |w|; x = RN(w * RN(1/c)); code = #{j : x > T[j]}
 *              (ties go to the lower code; a block with c < 2^-126 gets code 7);
 *   per group: o = RN(min c + max c) * 0.5; h = max |RN(c - o)|; s = RN(h / 127);
 *              absmax_q = clamp(rint_even(RN(RN(c - o) / s)), -127, 127) (0 if h = 0).
 * Outputs are the four arrays of qlora_nf4_weight; absmax_f32 (nullable, [n_blocks])
 * receives the first-level constants c. */
int qlora_quantize_nf4(const void *W, int w_dtype, int64_t n_rows, int64_t n_cols, uint8_t *codes,
                       int8_t *absmax_q, float *dq_scale, float *dq_offset, float *absmax_f32,
                       void *stream);

/* Blockwise quantization with a chosen level table and block-constant type (the
 * variants of the data-type comparison; see qlora_quant_type / qlora_const_type).
 * Codes as in qlora_quantize_nf4 with the quant_type's thresholds.  Constants:
 * QLORA_CONST_DQ_INT8 as qlora_quantize_nf4; QLORA_CONST_DQ_FP8 writes E4M3 bytes to
 * absmax_q and s = RN(h / 448), o to dq_scale, dq_offset; QLORA_CONST_FP32 writes c to
 * absmax (required) and leaves absmax_q, dq_scale, dq_offset untouched (may be NULL).
 * For the double-quantized types absmax (nullable) receives c as well. */
int qlora_quantize(const void *W, int w_dtype, int64_t n_rows, int64_t n_cols, int quant_type, int const_type,
                   uint8_t *codes, int8_t *absmax_q, float *dq_scale, float *dq_offset, float *absmax,
                   void *stream);

/* doubleDequant ([Digest] item 3, doubleDequant equation): out[n_rows, n_cols] =
 * RN(q[code] * c') as fp32 (out_dtype = QLORA_F32) or its bf16 rounding (QLORA_BF16). */
int qlora_dequantize(const qlora_nf4_weight *w, void *out, int out_dtype, void *stream);

/* Forward ([Paper note] "关键设计 3" equation and qlora_linear listing; [Digest]
 * "方法步骤与流程" step 3; [Repro] "LoRA 的公式和张量形状", scaling alpha / r):
 *   U_s = bf16((alpha / r) . X . A^T)                 [M, r]
 *   Y   = bf16(X . W'^T + U_s . B^T)                  [M, N], fp32 accumulation
 * X bf16 [M, K]; A bf16 [r, K]; B bf16 [N, r]; Y bf16 [M, N].
 * U_saved (nullable) receives U_s for the backward.  The decode of W' happens inside
 * the GEMM; no bf16 copy of the weight is written.  The call needs
 * qlora_workspace_bytes(0, M, K, N, r) bytes of workspace: for M <= 16 and N <= 65536
 * (the small-M path, one launch)
 * the counter header, copies of U_s and the partial sums of the down-projection
 * (the header alone when r = 0); otherwise the header, the fp32
 * partial sums of the down-projection plus U_s when U_saved is NULL, and none when
 * r = 0.  The kernels use 32-bit buffer offsets: QLORA_ERR_SHAPE, before anything is
 * launched, when X, Y, the codes or a LoRA operand exceed 0xFFFFFFF0 bytes. */
int qlora_linear_fwd(const qlora_nf4_weight *w, const uint16_t *X, int64_t M, const uint16_t *A,
                     const uint16_t *B, int r, float alpha, uint16_t *Y, uint16_t *U_saved,
                     void *workspace, size_t workspace_bytes, void *stream);

/* For callers that cannot allocate (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): qlora_linear_fwd with the workspace taken
 * from a fixed scratch array that the library holds in device memory, 16 MiB per GPU
 * it runs on (QLORA_NOALLOC_SCRATCH_BYTES), kept until the process ends.  Same
 * arguments, results and kernels as qlora_linear_fwd without workspace / workspace_bytes;
 * the call allocates nothing.  QLORA_ERR_WORKSPACE, before anything is launched, when
 * qlora_workspace_bytes(0, M, K, N, r) (U_saved == NULL adds the M x r U_s) exceeds the
 * scratch.  Every call on one GPU uses that GPU's one scratch array: calls that can
 * overlap on one GPU (different streams, different host threads) race and must be
 * serialised by the caller. */
#define QLORA_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
/* Leading workspace bytes that must be zero at first use (see Conventions). */
#define QLORA_WORKSPACE_HEADER_BYTES ((size_t)65792)
int qlora_linear_fwd_noalloc(const qlora_nf4_weight *w, const uint16_t *X, int64_t M, const uint16_t *A,
                             const uint16_t *B, int r, float alpha, uint16_t *Y, uint16_t *U_saved,
                             void *stream);

/* Backward ([Digest] "方法步骤与流程" step 4; [QLoRA note] "5. QLoRA 训练方式本身":
 * gradients flow through W' into the adapter only; no gradient for W):
 *   V  = bf16((alpha / r) . dY . B)                   [M, r]
 *   dX = bf16(dY . W' + V . A)                        [M, K]  (skipped if dX == NULL)
 *   dB = bf16(dY^T . U_s)                             [N, r]
 *   dA = bf16(V^T . X)                                [r, K]
 * U_saved is the forward's U_s; if NULL it is recomputed from X and A.  When r > 0 the
 * call needs qlora_workspace_bytes(1, M, K, N, r) bytes of workspace.
 * dY bf16 [M, N]; X bf16 [M, K] (needed for dA, and for U_s when U_saved is NULL).
 * QLORA_ERR_SHAPE, before anything is launched, when dX is requested and dY, dX, the
 * codes or a LoRA operand exceed 0xFFFFFFF0 bytes (32-bit buffer offsets). */
int qlora_linear_bwd(const qlora_nf4_weight *w, const uint16_t *dY, const uint16_t *X, int64_t M,
                     const uint16_t *A, const uint16_t *B, int r, float alpha,
                     const uint16_t *U_saved, uint16_t *dX, uint16_t *dA, uint16_t *dB,
                     void *workspace, size_t workspace_bytes, void *stream);

/* Horizontal fusion of linears that read the same X (the query, key and value
 * projections, or the gate and up projections, of a decoder layer; [Ch. 11.3] and
 * [Paper note] apply LoRA to all linear layers of the block, so each of them has its
 * own adapter).  The fused weight stacks n_parts weights of equal shape along rows
 * (qlora_nf4_concat_rows), the adapters are stacked too:
 *   A  bf16 [n_parts r, K]  rows [q r, q r + r) are part q's A
 *   B  bf16 [N, r]          rows [q P, q P + P) are part q's B  (P = N / n_parts)
 * and one call computes, for every part q at once (one weight stream, one GEMM),
 *   Y[:, qP .. qP + P) = bf16(X W_q'^T + U_q B_q^T),  U_q = bf16((alpha/r) X A_q^T)
 * which is bit-for-bit the output of qlora_linear_fwd on part q alone.  U_saved (if
 * not NULL) receives the stacked [M, n_parts r] U.  Requirements: N % n_parts == 0,
 * 1 <= n_parts <= QLORA_MAX_PARTS, n_parts r <= 256, and P % 256 == 0 when r > 0.
 * Workspace: qlora_workspace_bytes_fused(0, M, K, N, r, n_parts). */
int qlora_linear_fwd_fused(const qlora_nf4_weight *w, int n_parts, const uint16_t *X, int64_t M,
                           const uint16_t *A, const uint16_t *B, int r, float alpha, uint16_t *Y,
                           uint16_t *U_saved, void *workspace, size_t workspace_bytes, void *stream);

/* Backward of qlora_linear_fwd_fused: dY bf16 [M, N] holds the parts' output
 * gradients side by side.  dA [n_parts r, K] and dB [N, r] are stacked like A and B
 * and equal, part by part, what qlora_linear_bwd gives for that part; dX [M, K] is the
 * gradient of X through all parts together, bf16(sum_q (dY_q W_q' + V_q A_q)), rounded
 * once.  Workspace: qlora_workspace_bytes_fused(1, M, K, N, r, n_parts). */
int qlora_linear_bwd_fused(const qlora_nf4_weight *w, int n_parts, const uint16_t *dY, const uint16_t *X,
                           int64_t M, const uint16_t *A, const uint16_t *B, int r, float alpha,
                           const uint16_t *U_saved, uint16_t *dX, uint16_t *dA, uint16_t *dB,
                           void *workspace, size_t workspace_bytes, void *stream);

/* Concatenate quantized weights along rows into `out` (device copies on `stream`):
 * codes, block constants and group constants are appended part after part.  With
 * double-quantized constants every part but the last must hold a multiple of 256
 * blocks (of 16384 weights), so that its double-quantization groups end with it; the
 * result is then exactly the quantization of the row-concatenated matrix.  All parts
 * share n_cols, quant_type and const_type with out; out must be [sum n_rows, n_cols]
 * with arrays sized by qlora_nf4_sizes. */
int qlora_nf4_concat_rows(const qlora_nf4_weight *parts, int n_parts, const qlora_nf4_weight *out,
                          void *stream);

/* AdamW step on adapter parameters ([Digest] "方法步骤与流程" step 5: only the LoRA
 * matrices are updated, by an optimizer such as Adam; the pages give no formula, so
 * this is AdamW with decoupled weight decay and bias correction).  For i < n:
 *   g = grad[i] (bf16);  p = param[i] * fp32(1 - lr * weight_decay)
 *   m = b1 * m + (1 - b1) * g;  v = b2 * v + (1 - b2) * g * g
 *   param[i] = p - fp32(lr / (1 - b1^step)) * m / (sqrt(v) / fp32(sqrt(1 - b2^step)) + eps)
 * every operation one fp32 rounding (no fused multiply-add); the factors are formed in
 * double from the double hyper-parameters and rounded once.
 *   param, exp_avg, exp_avg_sq  fp32 [n], updated in place (exp_avg = m, exp_avg_sq = v)
 *   grad                        bf16 [n] (e.g. dA or dB of qlora_linear_bwd)
 *   param_bf16                  nullable bf16 [n]: receives bf16_rne(param) after the step
 * step >= 1 counts the steps taken including this one; 0 <= beta1, beta2 < 1; eps > 0;
 * lr and weight_decay finite and >= 0 (else QLORA_ERR_VALUE).  All pointers 16-byte
 * aligned. */
int qlora_adamw_step(float *param, uint16_t *param_bf16, const uint16_t *grad, float *exp_avg,
                     float *exp_avg_sq, int64_t n, double lr, double beta1, double beta2, double eps,
                     double weight_decay, int64_t step, void *stream);

/* LoRA merge ([Repro] "官方代码阅读路线": the scaled update B A can be folded into
 * the frozen weight for inference and removed again; [QLoRA note], on the error that
 * merging adds: merge into a higher-precision copy of the base, here bf16).
 *   out[n, k] = bf16_rne(W'[n, k] + RN(scale * D[n, k])),  D = B A,  scale = alpha / r
 * W' the bf16 weight decode (as qlora_dequantize with QLORA_BF16); D is accumulated
 * in fp32 (its summation order is unspecified).  r = 0 writes W' itself.
 *   A bf16 [r, K];  B bf16 [N, r];  out bf16 [N, K] (must not alias the weight arrays)
 * Merge exactly once ([Repro] "失败排查清单" item 4): a second merge adds B A again.
 * Check a merge by comparing the logits of qlora_linear_fwd with those of the merged
 * weight on the same input (item 6 of that list). */
int qlora_lora_merge(const qlora_nf4_weight *w, const uint16_t *A, const uint16_t *B, int r,
                     float alpha, uint16_t *out, void *stream);

/* LoRA unmerge, the inverse of qlora_lora_merge on a bf16 weight:
 *   out[n, k] = bf16_rne(W_merged[n, k] - RN(scale * D[n, k]))
 * W_merged, out bf16 [n_rows, n_cols]; out may equal W_merged (in place: each element
 * is read before it is written by the same thread).  A bf16 [r, n_cols], B bf16
 * [n_rows, r].  Merge then unmerge returns W' to within two bf16 roundings. */
int qlora_lora_unmerge(const uint16_t *W_merged, int64_t n_rows, int64_t n_cols, const uint16_t *A,
                       const uint16_t *B, int r, float alpha, uint16_t *out, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* QLORA_NF4_H */
