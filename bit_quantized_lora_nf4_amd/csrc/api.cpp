// C ABI of the library: argument checks, workspace layout and kernel dispatch.
// Every check runs on the host before anything is enqueued; the kernels then run
// asynchronously on the caller's stream.  No device memory is allocated here.

#include "../../include/qlora_nf4.h"
#include "qlora_internal.h"

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

namespace {

thread_local std::string g_last_error;
thread_local hipEvent_t g_ev_start = nullptr, g_ev_stop = nullptr;

// Launch through the timing hook: bracket with the armed events, then disarm.
template <typename F>
hipError_t timed_launch(hipStream_t st, F launch) {
  if (!g_ev_start || !g_ev_stop) return launch();
  hipEvent_t a = g_ev_start, b = g_ev_stop;
  g_ev_start = g_ev_stop = nullptr;
  hipError_t e = hipEventRecord(a, st);
  if (e != hipSuccess) return e;
  e = launch();
  if (e != hipSuccess) return e;
  return hipEventRecord(b, st);
}

int fail(int status, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int64_t kMaxDim = int64_t(1) << 40;

size_t align_up(size_t x) { return (x + 255) & ~size_t(255); }

int check_weight_shape(int64_t n_rows, int64_t n_cols) {
  if (n_rows < 1 || n_cols < 1 || n_cols % qlora::kBlock != 0)
    return fail(QLORA_ERR_SHAPE, "weight shape [%lld, %lld]: need n_rows >= 1 and n_cols a positive multiple of 64",
                (long long)n_rows, (long long)n_cols);
  if (n_rows > kMaxDim || n_cols > kMaxDim || n_rows > kMaxDim / n_cols)
    return fail(QLORA_ERR_SHAPE, "weight shape [%lld, %lld] too large", (long long)n_rows,
                (long long)n_cols);
  return QLORA_OK;
}

bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

int check_types(int quant_type, int const_type) {
  if (quant_type != QLORA_QUANT_NF4 && quant_type != QLORA_QUANT_FP4)
    return fail(QLORA_ERR_DTYPE, "quant_type %d: expected QLORA_QUANT_NF4 or QLORA_QUANT_FP4", quant_type);
  if (const_type != QLORA_CONST_DQ_INT8 && const_type != QLORA_CONST_DQ_FP8 && const_type != QLORA_CONST_FP32)
    return fail(QLORA_ERR_DTYPE, "const_type %d: expected QLORA_CONST_DQ_INT8, _DQ_FP8 or _FP32", const_type);
  return QLORA_OK;
}

int check_weight(const qlora_nf4_weight *w) {
  if (!w) return fail(QLORA_ERR_NULL, "weight descriptor is NULL");
  int s = check_weight_shape(w->n_rows, w->n_cols);
  if (s == QLORA_OK) s = check_types(w->quant_type, w->const_type);
  if (s != QLORA_OK) return s;
  if (w->const_type == QLORA_CONST_FP32) {
    if (!w->codes || !w->absmax)
      return fail(QLORA_ERR_NULL, "weight descriptor (fp32 constants) needs codes and absmax");
    if (!aligned4(w->absmax)) return fail(QLORA_ERR_ALIGN, "absmax must be 4-byte aligned");
  } else {
    if (!w->codes || !w->absmax_q || !w->dq_scale || !w->dq_offset)
      return fail(QLORA_ERR_NULL, "weight descriptor has a NULL array");
    if (!aligned4(w->dq_scale) || !aligned4(w->dq_offset))
      return fail(QLORA_ERR_ALIGN, "dq_scale and dq_offset must be 4-byte aligned");
  }
  if (!aligned16(w->codes))
    return fail(QLORA_ERR_ALIGN, "weight codes must be 16-byte aligned");
  return QLORA_OK;
}

int check_rank(int r, float alpha) {
  if (r < 0 || r > QLORA_MAX_RANK) return fail(QLORA_ERR_RANK, "r = %d outside [0, 256]", r);
  if (r > 0 && !std::isfinite(alpha)) return fail(QLORA_ERR_RANK, "alpha is not finite");
  return QLORA_OK;
}

int check_m(int64_t M) {
  if (M < 1 || M > kMaxDim) return fail(QLORA_ERR_SHAPE, "M = %lld must be >= 1", (long long)M);
  return QLORA_OK;
}

// The library runs on gfx950 only; the answer is cached per device ordinal.
int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return fail(QLORA_ERR_DEVICE, "no HIP device available");
  }
  static std::mutex mu;
  static int known[64] = {0};  // 0 unknown, 1 ok, 2 not gfx950
  std::lock_guard<std::mutex> lock(mu);
  if (dev < 64 && known[dev] == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      (void)hipGetLastError();
      return fail(QLORA_ERR_DEVICE, "hipGetDeviceProperties failed on device %d", dev);
    }
    known[dev] = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
  }
  if (dev >= 64 || known[dev] != 1)
    return fail(QLORA_ERR_DEVICE, "device %d is not a gfx950 (MI355X) GPU", dev);
  return QLORA_OK;
}

int launched(hipError_t e, const char *what) {
  if (e != hipSuccess)
    return fail(QLORA_ERR_LAUNCH, "%s: %s", what, hipGetErrorString(e));
  return QLORA_OK;
}

qlora::WeightView view(const qlora_nf4_weight *w) {
  return qlora::WeightView{w->codes,  w->absmax_q, w->dq_scale,   w->dq_offset,  w->n_rows,
                           w->n_cols, w->absmax,   w->quant_type, w->const_type};
}

// ---- fixed scratch of qlora_linear_fwd_noalloc ------------------------------
// One array per GPU, zero at load, kept until the process ends.  In host code the
// name `scratch` only stands for the symbol: kernels get the device address that
// hipGetSymbolAddress returns for the current device, looked up once per device.
constexpr size_t kScratchBytes = QLORA_NOALLOC_SCRATCH_BYTES;
static_assert(qlora::kGemvSyncBytes == QLORA_WORKSPACE_HEADER_BYTES, "workspace header size");
static __device__ __align__(256) char scratch[kScratchBytes];

int scratch_address(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return fail(QLORA_ERR_DEVICE, "linear_fwd_noalloc: no usable current device");
  }
  static std::once_flag once[64];
  static void *addr[64];
  static hipError_t err[64];
  std::call_once(once[dev], [dev] {
    void *p = nullptr;
    err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    addr[dev] = p;
  });
  if (err[dev] != hipSuccess || !addr[dev])
    return fail(QLORA_ERR_DEVICE, "linear_fwd_noalloc: hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                hipGetErrorString(err[dev]));
  *out = addr[dev];
  return QLORA_OK;
}

// ---- workspace layouts ------------------------------------------------------
struct FwdLayout {
  size_t u = 0, part = 0, total = 0;
};
// Every layout starts with the kGemvSyncBytes header of the small-M forward's counters
// and flags, which only that kernel touches (so one workspace can serve calls of any
// shape).  Small M (gemv_shape_ok): the whole GEMV workspace.  Otherwise U_s (when the
// caller does not keep it) then the fp32 partial sums of lora_down; nothing when r = 0.
FwdLayout fwd_layout(int64_t M, int64_t K, int64_t N, int r, bool need_u) {
  FwdLayout L;
  if (qlora::gemv_shape_ok(M, N)) {
    L.total = qlora::gemv_workspace(M, K, N, r);
    return L;
  }
  if (r == 0) return L;
  size_t off = qlora::kGemvSyncBytes;
  L.u = off;
  if (need_u) off += align_up(size_t(M) * r * 2);
  L.part = off;
  off += align_up(qlora::lora_down_workspace(M, K, r));
  L.total = off;
  return L;
}

struct BwdLayout {
  size_t u, bt, v, at, part, part2, total;
};
// U_s [M, R], B^T [r, N], V [M, R], A^T [K, R] (R = parts r), then the fp32 partial sums
// of the largest LoRA reduction, then those of dB (live together with V's partials when
// V and dB run in one launch).
BwdLayout bwd_layout(int64_t M, int64_t K, int64_t N, int r, int parts) {
  BwdLayout L{};
  if (r == 0) return L;
  const int R = r * parts;
  const int64_t Np = N / parts;
  size_t off = qlora::kGemvSyncBytes;
  L.u = off;
  off += align_up(size_t(M) * R * 2);
  L.bt = off;
  off += align_up(size_t(N) * r * 2);
  L.v = off;
  off += align_up(size_t(M) * R * 2);
  L.at = off;
  off += align_up(size_t(K) * R * 2);
  L.part = off;
  size_t p = qlora::reduce_m_workspace(M, Np, r);
  const size_t others[] = {qlora::reduce_m_workspace(M, K, R), qlora::lora_down_workspace(M, K, R),
                           qlora::lora_down_workspace(M, Np, r)};
  for (size_t o : others) p = o > p ? o : p;
  off += align_up(p);
  L.part2 = off;
  off += align_up(qlora::vdb_workspace_db(M, Np, r));
  L.total = off;
  return L;
}

// Horizontally fused linears: `parts` linears of N / parts weight rows each share X;
// their adapters are stacked (A [parts r, K], B [N, r]).  parts = 1 is one linear.
int check_parts(const char *who, int64_t N, int r, int parts) {
  if (parts < 1 || parts > QLORA_MAX_PARTS)
    return fail(QLORA_ERR_SHAPE, "%s: n_parts = %d outside [1, %d]", who, parts, QLORA_MAX_PARTS);
  if (N % parts != 0)
    return fail(QLORA_ERR_SHAPE, "%s: %lld weight rows do not split into %d equal parts", who,
                (long long)N, parts);
  if (int64_t(r) * parts > QLORA_MAX_RANK)
    return fail(QLORA_ERR_RANK, "%s: stacked rank %d x %d exceeds %d", who, parts, r, QLORA_MAX_RANK);
  if (parts > 1 && r > 0 && (N / parts) % 256 != 0)
    return fail(QLORA_ERR_SHAPE, "%s: part rows %lld must be a multiple of 256", who,
                (long long)(N / parts));
  return QLORA_OK;
}

int fwd_impl(const char *who, const qlora_nf4_weight *w, int parts, const uint16_t *X, int64_t M,
             const uint16_t *A, const uint16_t *B, int r, float alpha, uint16_t *Y, uint16_t *U_saved,
             void *workspace, size_t workspace_bytes, void *stream) {
  int s = check_weight(w);
  if (s == QLORA_OK) s = check_m(M);
  if (s == QLORA_OK) s = check_rank(r, alpha);
  if (s == QLORA_OK) s = check_parts(who, w->n_rows, r, parts);
  if (s != QLORA_OK) return s;
  if (!X || !Y) return fail(QLORA_ERR_NULL, "%s: X and Y are required", who);
  if (r > 0 && (!A || !B)) return fail(QLORA_ERR_NULL, "%s: A and B are required when r > 0", who);
  if (!aligned16(X) || !aligned16(Y) || (r > 0 && (!aligned16(A) || !aligned16(B))) ||
      (U_saved && !aligned16(U_saved)))
    return fail(QLORA_ERR_ALIGN, "%s: tensors must be 16-byte aligned", who);
  const int64_t K = w->n_cols, N = w->n_rows;
  const int R = r * parts;
  // per-part rank offsets only matter with an adapter; without one the fused weight is
  // a single linear to the kernels (part heights need not be multiples of 256)
  const int64_t part_rows = (parts > 1 && r > 0) ? N / parts : 0;
  const FwdLayout L = fwd_layout(M, K, N, R, !U_saved);
  const bool need_ws = L.total > 0;
  if (need_ws && (!workspace || workspace_bytes < L.total))
    return fail(QLORA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", who, L.total,
                workspace_bytes);
  if (need_ws && !aligned16(workspace))
    return fail(QLORA_ERR_ALIGN, "%s: workspace must be 16-byte aligned", who);
  const qlora::WeightView wv = view(w);
  const bool small = qlora::gemv_shape_ok(M, wv.n_rows);
  if (small ? !qlora::gemv_supported(wv, M, R) : !qlora::gemm_supported(wv, M, R))
    return fail(QLORA_ERR_SHAPE, "%s: a tensor of %lld x %lld x %lld exceeds 32-bit buffer offsets", who,
                (long long)M, (long long)K, (long long)N);
  s = check_device();
  if (s != QLORA_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const float scale = r > 0 ? alpha / static_cast<float>(r) : 0.0f;
  if (small)
    return launched(timed_launch(st, [&] {
                      return qlora::launch_gemv(wv, X, M, A, R, B, r, part_rows, scale, Y, U_saved, workspace, st);
                    }),
                    "gemv");
  uint16_t *U = nullptr;
  if (r > 0) {
    char *ws = static_cast<char *>(workspace);
    U = U_saved ? U_saved : reinterpret_cast<uint16_t *>(ws + L.u);
    s = launched(qlora::launch_lora_down(X, M, K, K, A, K, R, scale, U, R,
                                         reinterpret_cast<float *>(ws + L.part), st),
                 "lora_down");
    if (s != QLORA_OK) return s;
  }
  return launched(
      timed_launch(st, [&] { return qlora::launch_gemm_fwd(wv, X, M, U, R, B, r, part_rows, Y, st); }),
      "gemm_fwd");
}

int bwd_impl(const char *who, const qlora_nf4_weight *w, int parts, const uint16_t *dY,
             const uint16_t *X, int64_t M, const uint16_t *A, const uint16_t *B, int r, float alpha,
             const uint16_t *U_saved, uint16_t *dX, uint16_t *dA, uint16_t *dB, void *workspace,
             size_t workspace_bytes, void *stream) {
  int s = check_weight(w);
  if (s == QLORA_OK) s = check_m(M);
  if (s == QLORA_OK) s = check_rank(r, alpha);
  if (s == QLORA_OK) s = check_parts(who, w->n_rows, r, parts);
  if (s != QLORA_OK) return s;
  if (!dY) return fail(QLORA_ERR_NULL, "%s: dY is required", who);
  if (r > 0 && (!A || !B || !X || !dA || !dB))
    return fail(QLORA_ERR_NULL, "%s: X, A, B, dA and dB are required when r > 0", who);
  if (r == 0 && !dX) return fail(QLORA_ERR_NULL, "%s: nothing to compute (r = 0, dX NULL)", who);
  const void *ptrs[] = {dY, X, A, B, U_saved, dX, dA, dB};
  for (const void *p : ptrs)
    if (p && !aligned16(p)) return fail(QLORA_ERR_ALIGN, "%s: tensors must be 16-byte aligned", who);
  const int64_t K = w->n_cols, N = w->n_rows;
  const int R = r * parts;
  const int64_t Np = N / parts;
  const BwdLayout L = bwd_layout(M, K, N, r, parts);
  if (r > 0 && (!workspace || workspace_bytes < L.total))
    return fail(QLORA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", who, L.total,
                workspace_bytes);
  if (r > 0 && !aligned16(workspace))
    return fail(QLORA_ERR_ALIGN, "%s: workspace must be 16-byte aligned", who);
  if (dX && !qlora::gemm_supported(view(w), M, R))
    return fail(QLORA_ERR_SHAPE, "%s: a tensor of %lld x %lld x %lld exceeds 32-bit buffer offsets", who,
                (long long)M, (long long)K, (long long)N);
  s = check_device();
  if (s != QLORA_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const qlora::WeightView wv = view(w);
  char *ws = static_cast<char *>(workspace);
  const uint16_t *V = nullptr, *At = nullptr;
  qlora::FinalizeJob fin_da{nullptr, 0, 0, 0, 0, 0.0f, nullptr};
  if (r > 0) {
    const float scale = alpha / static_cast<float>(r);
    float *part = reinterpret_cast<float *>(ws + L.part);
    const uint16_t *U = U_saved;
    if (!U) {
      uint16_t *Uw = reinterpret_cast<uint16_t *>(ws + L.u);
      s = launched(qlora::launch_lora_down(X, M, K, K, A, K, R, scale, Uw, R, part, st), "lora_down(U)");
      if (s != QLORA_OK) return s;
      U = Uw;
    }
    uint16_t *Bt = reinterpret_cast<uint16_t *>(ws + L.bt);
    uint16_t *Vw = reinterpret_cast<uint16_t *>(ws + L.v);
    uint16_t *Atw = reinterpret_cast<uint16_t *>(ws + L.at);
    // part q: V[:, q r ..] = bf16(scale dY_q B_q) and dB_q = bf16(dY_q^T U_q), where dY_q is
    // columns [q Np, (q + 1) Np) of dY, B_q rows [q Np, (q + 1) Np) of B and U_q columns
    // [q r, (q + 1) r) of U_s; both products in one launch (and one finalize launch)
    // where the shapes allow, which reads B as it is and also writes A^T for the dX
    // GEMM's rank steps (when dX is wanted).  Otherwise B^T and A^T come from a
    // transpose launch first.
    const bool vdb = qlora::vdb_fast(M, Np, N, R, r);
    if (!vdb)
      s = launched(qlora::launch_transpose2_bf16(B, N, r, Bt, dX ? A : nullptr, R, K, Atw, st), "transpose(B, A)");
    float *part2 = reinterpret_cast<float *>(ws + L.part2);
    for (int q = 0; q < parts && s == QLORA_OK; ++q) {
      if (vdb) {
        const bool at = dX && q == 0;
        s = launched(qlora::launch_vdb(dY + q * Np, M, Np, N, B + q * Np * r, U + q * r, R, r, scale, Vw + q * r,
                                       dB + q * Np * r, part, part2, at ? A : nullptr, R, K, at ? Atw : nullptr, st),
                     "lora(V, dB)");
        continue;
      }
      s = launched(qlora::launch_lora_down(dY + q * Np, M, Np, N, Bt + q * Np, N, r, scale, Vw + q * r, R,
                                           part, st),
                   "lora_down(V)");
      if (s == QLORA_OK)
        s = launched(qlora::launch_reduce_m(dY + q * Np, M, Np, N, U + q * r, R, r, part, dB + q * Np * r,
                                            false, st),
                     "reduce(dB)");
    }
    // dA's finalize pass rides in the dX GEMM's launch when there is one
    if (s == QLORA_OK)
      s = launched(qlora::launch_reduce_m(X, M, K, K, Vw, R, R, part, dA, true, st, dX ? &fin_da : nullptr),
                   "reduce(dA)");
    if (s != QLORA_OK) return s;
    V = Vw;
    At = Atw;
  }
  if (dX)
    return launched(timed_launch(st, [&] { return qlora::launch_gemm_dx(wv, dY, M, V, At, R, dX, st, &fin_da); }),
                    "gemm_dx");
  return QLORA_OK;
}

}  // namespace

extern "C" {

const char *qlora_status_string(int status) {
  switch (status) {
    case QLORA_OK: return "ok";
    case QLORA_ERR_NULL: return "null pointer";
    case QLORA_ERR_SHAPE: return "invalid shape";
    case QLORA_ERR_RANK: return "invalid rank or alpha";
    case QLORA_ERR_DTYPE: return "unsupported dtype";
    case QLORA_ERR_WORKSPACE: return "workspace too small";
    case QLORA_ERR_VALUE: return "scalar argument out of range";
    case QLORA_ERR_ALIGN: return "pointer not 16-byte aligned";
    case QLORA_ERR_DEVICE: return "no usable gfx950 device";
    case QLORA_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

const char *qlora_last_error(void) { return g_last_error.c_str(); }

void qlora_time_next_gemm(void *start_event, void *stop_event) {
  g_ev_start = static_cast<hipEvent_t>(start_event);
  g_ev_stop = static_cast<hipEvent_t>(stop_event);
}

int qlora_nf4_sizes(int64_t n_rows, int64_t n_cols, size_t *code_bytes, int64_t *n_blocks,
                    int64_t *n_groups) {
  int s = check_weight_shape(n_rows, n_cols);
  if (s != QLORA_OK) return s;
  const int64_t n = n_rows * n_cols;
  const int64_t nb = n / qlora::kBlock;
  if (code_bytes) *code_bytes = static_cast<size_t>(n / 2);
  if (n_blocks) *n_blocks = nb;
  if (n_groups) *n_groups = (nb + qlora::kGroup - 1) / qlora::kGroup;
  return QLORA_OK;
}

size_t qlora_workspace_bytes(int op, int64_t M, int64_t K, int64_t N, int r) {
  return qlora_workspace_bytes_fused(op, M, K, N, r, 1);
}

size_t qlora_workspace_bytes_fused(int op, int64_t M, int64_t K, int64_t N, int r, int n_parts) {
  if (M < 1 || K < 1 || N < 1 || K % 64 != 0 || r < 0 || n_parts < 1 || n_parts > QLORA_MAX_PARTS ||
      N % n_parts != 0 || int64_t(r) * n_parts > QLORA_MAX_RANK)
    return 0;
  if (op == 0) return fwd_layout(M, K, N, r * n_parts, true).total;
  if (op == 1) return bwd_layout(M, K, N, r, n_parts).total;
  return 0;
}

int qlora_quantize(const void *W, int w_dtype, int64_t n_rows, int64_t n_cols, int quant_type, int const_type,
                   uint8_t *codes, int8_t *absmax_q, float *dq_scale, float *dq_offset, float *absmax,
                   void *stream) {
  int s = check_weight_shape(n_rows, n_cols);
  if (s == QLORA_OK) s = check_types(quant_type, const_type);
  if (s != QLORA_OK) return s;
  if (w_dtype != QLORA_F32 && w_dtype != QLORA_BF16)
    return fail(QLORA_ERR_DTYPE, "w_dtype %d: expected QLORA_F32 or QLORA_BF16", w_dtype);
  if (!W || !codes) return fail(QLORA_ERR_NULL, "quantize: NULL input or codes");
  if (const_type == QLORA_CONST_FP32 ? !absmax : (!absmax_q || !dq_scale || !dq_offset))
    return fail(QLORA_ERR_NULL, "quantize: NULL constant output for const_type %d", const_type);
  if (!aligned16(W) || !aligned16(codes))
    return fail(QLORA_ERR_ALIGN, "quantize: W and codes must be 16-byte aligned");
  if (!aligned4(absmax) || !aligned4(dq_scale) || !aligned4(dq_offset))
    return fail(QLORA_ERR_ALIGN, "quantize: fp32 outputs must be 4-byte aligned");
  if (!qlora::codebook(quant_type).bucket_ok) return fail(QLORA_ERR_DEVICE, "internal: bucket table");
  s = check_device();
  if (s != QLORA_OK) return s;
  return launched(qlora::launch_quantize(W, w_dtype == QLORA_BF16, n_rows, n_cols, quant_type, const_type,
                                         codes, absmax_q, dq_scale, dq_offset, absmax,
                                         static_cast<hipStream_t>(stream)),
                  "quantize");
}

int qlora_quantize_nf4(const void *W, int w_dtype, int64_t n_rows, int64_t n_cols, uint8_t *codes,
                       int8_t *absmax_q, float *dq_scale, float *dq_offset, float *absmax_f32,
                       void *stream) {
  return qlora_quantize(W, w_dtype, n_rows, n_cols, QLORA_QUANT_NF4, QLORA_CONST_DQ_INT8, codes, absmax_q,
                        dq_scale, dq_offset, absmax_f32, stream);
}

int qlora_dequantize(const qlora_nf4_weight *w, void *out, int out_dtype, void *stream) {
  int s = check_weight(w);
  if (s != QLORA_OK) return s;
  if (out_dtype != QLORA_F32 && out_dtype != QLORA_BF16)
    return fail(QLORA_ERR_DTYPE, "out_dtype %d: expected QLORA_F32 or QLORA_BF16", out_dtype);
  if (!out) return fail(QLORA_ERR_NULL, "dequantize: out is NULL");
  if (!aligned16(out)) return fail(QLORA_ERR_ALIGN, "dequantize: out must be 16-byte aligned");
  s = check_device();
  if (s != QLORA_OK) return s;
  return launched(qlora::launch_dequantize(view(w), out, out_dtype == QLORA_BF16,
                                           static_cast<hipStream_t>(stream)),
                  "dequantize");
}

int qlora_linear_fwd(const qlora_nf4_weight *w, const uint16_t *X, int64_t M, const uint16_t *A,
                     const uint16_t *B, int r, float alpha, uint16_t *Y, uint16_t *U_saved,
                     void *workspace, size_t workspace_bytes, void *stream) {
  return fwd_impl("linear_fwd", w, 1, X, M, A, B, r, alpha, Y, U_saved, workspace, workspace_bytes,
                  stream);
}

int qlora_linear_fwd_noalloc(const qlora_nf4_weight *w, const uint16_t *X, int64_t M, const uint16_t *A,
                             const uint16_t *B, int r, float alpha, uint16_t *Y, uint16_t *U_saved,
                             void *stream) {
  int s = check_weight(w);
  if (s == QLORA_OK) s = check_m(M);
  if (s == QLORA_OK) s = check_rank(r, alpha);
  if (s != QLORA_OK) return s;
  const size_t need = fwd_layout(M, w->n_cols, w->n_rows, r, !U_saved).total;
  if (need > kScratchBytes)
    return fail(QLORA_ERR_WORKSPACE,
                "linear_fwd_noalloc: these shapes need %zu bytes of scratch; the fixed scratch holds %zu",
                need, kScratchBytes);
  s = check_device();
  if (s != QLORA_OK) return s;
  void *ws = nullptr;
  s = scratch_address(&ws);
  if (s != QLORA_OK) return s;
  return fwd_impl("linear_fwd_noalloc", w, 1, X, M, A, B, r, alpha, Y, U_saved, ws, kScratchBytes, stream);
}

int qlora_linear_fwd_fused(const qlora_nf4_weight *w, int n_parts, const uint16_t *X, int64_t M,
                           const uint16_t *A, const uint16_t *B, int r, float alpha, uint16_t *Y,
                           uint16_t *U_saved, void *workspace, size_t workspace_bytes, void *stream) {
  return fwd_impl("linear_fwd_fused", w, n_parts, X, M, A, B, r, alpha, Y, U_saved, workspace,
                  workspace_bytes, stream);
}

int qlora_linear_bwd(const qlora_nf4_weight *w, const uint16_t *dY, const uint16_t *X, int64_t M,
                     const uint16_t *A, const uint16_t *B, int r, float alpha,
                     const uint16_t *U_saved, uint16_t *dX, uint16_t *dA, uint16_t *dB,
                     void *workspace, size_t workspace_bytes, void *stream) {
  return bwd_impl("linear_bwd", w, 1, dY, X, M, A, B, r, alpha, U_saved, dX, dA, dB, workspace,
                  workspace_bytes, stream);
}

int qlora_linear_bwd_fused(const qlora_nf4_weight *w, int n_parts, const uint16_t *dY, const uint16_t *X,
                           int64_t M, const uint16_t *A, const uint16_t *B, int r, float alpha,
                           const uint16_t *U_saved, uint16_t *dX, uint16_t *dA, uint16_t *dB,
                           void *workspace, size_t workspace_bytes, void *stream) {
  return bwd_impl("linear_bwd_fused", w, n_parts, dY, X, M, A, B, r, alpha, U_saved, dX, dA, dB,
                  workspace, workspace_bytes, stream);
}

int qlora_nf4_concat_rows(const qlora_nf4_weight *parts, int n_parts, const qlora_nf4_weight *out,
                          void *stream) {
  if (!parts || !out) return fail(QLORA_ERR_NULL, "nf4_concat_rows: parts and out are required");
  if (n_parts < 1 || n_parts > QLORA_MAX_PARTS)
    return fail(QLORA_ERR_SHAPE, "nf4_concat_rows: n_parts = %d outside [1, %d]", n_parts, QLORA_MAX_PARTS);
  int64_t rows = 0;
  const int64_t K = parts[0].n_cols;
  const bool dq = out->const_type != QLORA_CONST_FP32;
  for (int i = 0; i < n_parts; ++i) {
    int s = check_weight(&parts[i]);
    if (s != QLORA_OK) return s;
    if (parts[i].n_cols != K)
      return fail(QLORA_ERR_SHAPE, "nf4_concat_rows: part %d has %lld columns, part 0 %lld", i,
                  (long long)parts[i].n_cols, (long long)K);
    if (parts[i].quant_type != out->quant_type || parts[i].const_type != out->const_type)
      return fail(QLORA_ERR_DTYPE, "nf4_concat_rows: part %d has types (%d, %d), out (%d, %d)", i,
                  parts[i].quant_type, parts[i].const_type, out->quant_type, out->const_type);
    // the double-quantization groups of a part must end on a group boundary for the
    // concatenated arrays to be the quantization of the concatenated matrix
    if (dq && i + 1 < n_parts && (parts[i].n_rows * K / qlora::kBlock) % qlora::kGroup != 0)
      return fail(QLORA_ERR_SHAPE,
                  "nf4_concat_rows: part %d holds %lld blocks, not a multiple of %d (its last "
                  "double-quantization group would straddle the next part)",
                  i, (long long)(parts[i].n_rows * K / qlora::kBlock), qlora::kGroup);
    rows += parts[i].n_rows;
  }
  int s = check_weight(out);
  if (s != QLORA_OK) return s;
  if (out->n_rows != rows || out->n_cols != K)
    return fail(QLORA_ERR_SHAPE, "nf4_concat_rows: out is [%lld, %lld], the parts make [%lld, %lld]",
                (long long)out->n_rows, (long long)out->n_cols, (long long)rows, (long long)K);
  s = check_device();
  if (s != QLORA_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  size_t oc = 0, ob = 0, og = 0;
  for (int i = 0; i < n_parts; ++i) {
    const int64_t nb = parts[i].n_rows * K / qlora::kBlock;
    const int64_t ng = (nb + qlora::kGroup - 1) / qlora::kGroup;
    const size_t cb = static_cast<size_t>(parts[i].n_rows * K / 2);
    // the descriptor's arrays are declared const for the compute entries; here they
    // are the caller's destination
    auto dst = [](const void *p, size_t off) { return static_cast<char *>(const_cast<void *>(p)) + off; };
    hipError_t e = hipMemcpyAsync(dst(out->codes, oc), parts[i].codes, cb, hipMemcpyDeviceToDevice, st);
    if (!dq) {
      if (e == hipSuccess)
        e = hipMemcpyAsync(dst(out->absmax, ob * 4), parts[i].absmax, nb * 4, hipMemcpyDeviceToDevice, st);
    } else {
      if (e == hipSuccess)
        e = hipMemcpyAsync(dst(out->absmax_q, ob), parts[i].absmax_q, nb, hipMemcpyDeviceToDevice, st);
      if (e == hipSuccess)
        e = hipMemcpyAsync(dst(out->dq_scale, og * 4), parts[i].dq_scale, ng * 4, hipMemcpyDeviceToDevice, st);
      if (e == hipSuccess)
        e = hipMemcpyAsync(dst(out->dq_offset, og * 4), parts[i].dq_offset, ng * 4, hipMemcpyDeviceToDevice, st);
    }
    s = launched(e, "nf4_concat_rows");
    if (s != QLORA_OK) return s;
    oc += cb;
    ob += nb;
    og += ng;
  }
  return QLORA_OK;
}

int qlora_lora_merge(const qlora_nf4_weight *w, const uint16_t *A, const uint16_t *B, int r,
                     float alpha, uint16_t *out, void *stream) {
  int s = check_weight(w);
  if (s == QLORA_OK) s = check_rank(r, alpha);
  if (s != QLORA_OK) return s;
  if (!out) return fail(QLORA_ERR_NULL, "lora_merge: out is NULL");
  if (r > 0 && (!A || !B)) return fail(QLORA_ERR_NULL, "lora_merge: A and B are required when r > 0");
  if (!aligned16(out) || (r > 0 && (!aligned16(A) || !aligned16(B))))
    return fail(QLORA_ERR_ALIGN, "lora_merge: tensors must be 16-byte aligned");
  s = check_device();
  if (s != QLORA_OK) return s;
  const float scale = r > 0 ? alpha / static_cast<float>(r) : 0.0f;
  return launched(qlora::launch_lora_merge(view(w), A, B, r, scale, out,
                                           static_cast<hipStream_t>(stream)),
                  "lora_merge");
}

int qlora_lora_unmerge(const uint16_t *W_merged, int64_t n_rows, int64_t n_cols, const uint16_t *A,
                       const uint16_t *B, int r, float alpha, uint16_t *out, void *stream) {
  int s = check_weight_shape(n_rows, n_cols);
  if (s == QLORA_OK) s = check_rank(r, alpha);
  if (s != QLORA_OK) return s;
  if (!W_merged || !out) return fail(QLORA_ERR_NULL, "lora_unmerge: W_merged and out are required");
  if (r > 0 && (!A || !B)) return fail(QLORA_ERR_NULL, "lora_unmerge: A and B are required when r > 0");
  if (!aligned16(W_merged) || !aligned16(out) || (r > 0 && (!aligned16(A) || !aligned16(B))))
    return fail(QLORA_ERR_ALIGN, "lora_unmerge: tensors must be 16-byte aligned");
  s = check_device();
  if (s != QLORA_OK) return s;
  const float scale = r > 0 ? alpha / static_cast<float>(r) : 0.0f;
  return launched(qlora::launch_lora_unmerge(W_merged, n_rows, n_cols, A, B, r, scale, out,
                                             static_cast<hipStream_t>(stream)),
                  "lora_unmerge");
}

}  // extern "C"

int qlora_adamw_step(float *param, uint16_t *param_bf16, const uint16_t *grad, float *exp_avg,
                     float *exp_avg_sq, int64_t n, double lr, double beta1, double beta2, double eps,
                     double weight_decay, int64_t step, void *stream) {
  if (!param || !grad || !exp_avg || !exp_avg_sq)
    return fail(QLORA_ERR_NULL, "adamw_step: param, grad, exp_avg and exp_avg_sq are required");
  if (n < 1 || n > (int64_t(1) << 40)) return fail(QLORA_ERR_SHAPE, "adamw_step: n = %lld", (long long)n);
  if (step < 1) return fail(QLORA_ERR_VALUE, "adamw_step: step = %lld must be >= 1", (long long)step);
  if (!(beta1 >= 0.0 && beta1 < 1.0) || !(beta2 >= 0.0 && beta2 < 1.0) || !(eps > 0.0) ||
      !std::isfinite(eps) || !(lr >= 0.0) || !std::isfinite(lr) || !(weight_decay >= 0.0) ||
      !std::isfinite(weight_decay))
    return fail(QLORA_ERR_VALUE, "adamw_step: hyper-parameter out of range");
  if (!aligned16(param) || !aligned16(grad) || !aligned16(exp_avg) || !aligned16(exp_avg_sq) ||
      (param_bf16 && !aligned16(param_bf16)))
    return fail(QLORA_ERR_ALIGN, "adamw_step: pointers must be 16-byte aligned");
  int s = check_device();
  if (s != QLORA_OK) return s;
  const double t = static_cast<double>(step);
  qlora::AdamConsts c;
  c.decay = static_cast<float>(1.0 - lr * weight_decay);
  c.b1 = static_cast<float>(beta1);
  c.ob1 = static_cast<float>(1.0 - beta1);
  c.b2 = static_cast<float>(beta2);
  c.ob2 = static_cast<float>(1.0 - beta2);
  c.step_size = static_cast<float>(lr / (1.0 - std::pow(beta1, t)));
  c.bc2s = static_cast<float>(std::sqrt(1.0 - std::pow(beta2, t)));
  c.eps = static_cast<float>(eps);
  if (!std::isfinite(c.step_size) || !(c.bc2s > 0.0f))
    return fail(QLORA_ERR_VALUE, "adamw_step: bias correction underflows at this step");
  return launched(qlora::launch_adamw(param, param_bf16, grad, exp_avg, exp_avg_sq, n, c,
                                      static_cast<hipStream_t>(stream)),
                  "adamw");
}
