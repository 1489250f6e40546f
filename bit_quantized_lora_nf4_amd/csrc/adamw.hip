// AdamW step on the LoRA parameters ([Digest] "方法步骤与流程" step 5: after the
// backward an optimizer such as Adam updates only the adapter matrices).
//
// One pass over HBM (28 bytes per parameter: fp32 parameter and both moments read
// and written, the bf16 gradient read and the bf16 parameter copy written); four
// parameters per thread with 16-byte accesses.  Every element follows this exact
// sequence of fp32 operations (compiled without contraction into fma, with correctly
// rounded division and square root):
//     p1 = p * decay;  m1 = b1 * m + ob1 * g;  v1 = b2 * v + ob2 * (g * g)
//     p2 = p1 - step_size * (m1 / (sqrt(v1) / bc2s + eps));  p_bf16 = bf16_rne(p2)

#include "device_common.h"
#include "qlora_internal.h"

namespace qlora {
namespace {

__device__ __forceinline__ float adam_elem(float p, float g, float &m, float &v, const AdamConsts &c) {
  const float p1 = p * c.decay;
  const float m1 = c.b1 * m + c.ob1 * g;
  const float v1 = c.b2 * v + c.ob2 * (g * g);
  const float denom = __builtin_sqrtf(v1) / c.bc2s + c.eps;
  m = m1;
  v = v1;
  return p1 - c.step_size * (m1 / denom);
}

constexpr int AT = 256;

__global__ __launch_bounds__(AT) void adamw_kernel(float *__restrict__ p, uint16_t *__restrict__ pb,
                                                   const uint16_t *__restrict__ g, float *__restrict__ m,
                                                   float *__restrict__ v, int64_t n, AdamConsts c) {
  const int64_t base = (static_cast<int64_t>(blockIdx.x) * AT + threadIdx.x) * 4;
  if (base + 4 <= n) {
    f32x4_t pv = *reinterpret_cast<const f32x4_t *>(p + base);
    f32x4_t mv = *reinterpret_cast<const f32x4_t *>(m + base);
    f32x4_t vv = *reinterpret_cast<const f32x4_t *>(v + base);
    const u32x2_t gv = *reinterpret_cast<const u32x2_t *>(g + base);
    const float gf[4] = {bf16_lo(gv[0]), bf16_hi(gv[0]), bf16_lo(gv[1]), bf16_hi(gv[1])};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float me = mv[e], ve = vv[e];
      pv[e] = adam_elem(pv[e], gf[e], me, ve, c);
      mv[e] = me;
      vv[e] = ve;
    }
    *reinterpret_cast<f32x4_t *>(p + base) = pv;
    *reinterpret_cast<f32x4_t *>(m + base) = mv;
    *reinterpret_cast<f32x4_t *>(v + base) = vv;
    if (pb)
      *reinterpret_cast<u32x2_t *>(pb + base) = u32x2_t{pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3])};
  } else {
    for (int64_t i = base; i < n; ++i) {
      float me = m[i], ve = v[i];
      const float pn = adam_elem(p[i], bf16_to_f32(g[i]), me, ve, c);
      p[i] = pn;
      m[i] = me;
      v[i] = ve;
      if (pb) pb[i] = to_bf16(pn);
    }
  }
}

}  // namespace

hipError_t launch_adamw(float *p, uint16_t *pb, const uint16_t *g, float *m, float *v, int64_t n,
                        const AdamConsts &c, hipStream_t stream) {
  const int64_t threads = (n + 3) / 4;
  const int64_t blocks = (threads + AT - 1) / AT;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(adamw_kernel, dim3(static_cast<unsigned>(blocks)), dim3(AT), 0, stream, p, pb, g, m, v,
                     n, c);
  return hipGetLastError();
}

}  // namespace qlora
