// 32-bit AdamW step of the LoRA matrices (the paged optimiser's update),
// gfx950.
//
// Day-25 notes 3.4 (Adam's momentum and variance kept in float32, paged out
// to CPU RAM under memory pressure); QLoRA glossary, "QLoRA 的工作原理",
// paged-optimiser bullet; "如何利用QLoRA在消费级GPU上实现大模型的高效微调",
// sections 3 and 4 (paged_adamw_32bit). The update rule is AdamW as
// published (bias-corrected moments, decoupled weight decay); per element,
// each float32 operation rounded once (IEEE division and square root):
//   m' = b1 m + c1 g,  v' = b2 v + c2 (g g),
//   p' = p - lr ((m'/bc1) / (sqrt(v'/bc2) + eps) + wd p),  out = bf16(p').
// HBM-bound: 14 bytes read and 14 written per element. A lane updates two
// groups of four consecutive elements (16-byte float32 and 8-byte bf16
// accesses, all loads issued before the first update);
// the state may be device memory or device-mapped page-locked host memory
// (paged out), which the same loads and stores reach over the host link.
#include "kernels.h"

namespace {

// Correctly rounded float32 square root of x >= 0: the hardware root (within
// one ulp), then the neighbour whose product with it brackets x is taken
// (the residual x - c * s, formed by an fma, changes sign at the midpoint
// between adjacent candidates up to a term below the resolution of x).
QL_DEV float sqrt_rn(float x) {
  const float s = __builtin_sqrtf(x);
  if (!(x > 0.0f) || !(s < __builtin_inff())) return s;   // 0, NaN, inf
  const float sm = __uint_as_float(__float_as_uint(s) - 1u);
  const float sp = __uint_as_float(__float_as_uint(s) + 1u);
  float r = s;
  if (__builtin_fmaf(-sm, s, x) <= 0.0f) r = sm;
  if (__builtin_fmaf(-sp, s, x) > 0.0f) r = sp;
  return r;
}

QL_DEV void adam1(float &p, float &m, float &v, float g, const AdamScalars &s) {
  m = __fadd_rn(__fmul_rn(s.b1, m), __fmul_rn(s.c1, g));
  v = __fadd_rn(__fmul_rn(s.b2, v), __fmul_rn(s.c2, __fmul_rn(g, g)));
  const float mh = __fdiv_rn(m, s.bc1);
  const float vh = __fdiv_rn(v, s.bc2);
  const float u = __fdiv_rn(mh, __fadd_rn(sqrt_rn(vh), s.eps));
  p = __fsub_rn(p, __fmul_rn(s.lr, __fadd_rn(u, __fmul_rn(s.wd, p))));
}

constexpr int AV = 2;   // float4 groups per lane, loads issued together

__global__ __launch_bounds__(256) void adamw_kernel(float *__restrict__ p, float *__restrict__ m,
                                                    float *__restrict__ v,
                                                    const uint16_t *__restrict__ g,
                                                    uint16_t *__restrict__ out, int64_t n,
                                                    AdamScalars s) {
  // lane j of workgroup b: groups (b * AV + a) * 256 + j, a < AV, 4 elements each
  const int64_t gbase = (int64_t)blockIdx.x * AV * 256 + threadIdx.x;
  if ((gbase + (AV - 1) * 256) * 4 + 4 <= n) {
    float4 pv[AV], mv[AV], vv[AV];
    uint2 gw[AV];
#pragma unroll
    for (int a = 0; a < AV; ++a) {
      const int64_t i0 = (gbase + a * 256) * 4;
      pv[a] = *(const float4 *)(p + i0);
      mv[a] = *(const float4 *)(m + i0);
      vv[a] = *(const float4 *)(v + i0);
      gw[a] = *(const uint2 *)(g + i0);
    }
#pragma unroll
    for (int a = 0; a < AV; ++a) {
      const int64_t i0 = (gbase + a * 256) * 4;
      adam1(pv[a].x, mv[a].x, vv[a].x, ql::bf16lo(gw[a].x), s);
      adam1(pv[a].y, mv[a].y, vv[a].y, ql::bf16hi(gw[a].x), s);
      adam1(pv[a].z, mv[a].z, vv[a].z, ql::bf16lo(gw[a].y), s);
      adam1(pv[a].w, mv[a].w, vv[a].w, ql::bf16hi(gw[a].y), s);
      *(float4 *)(p + i0) = pv[a];
      *(float4 *)(m + i0) = mv[a];
      *(float4 *)(v + i0) = vv[a];
      *(uint2 *)(out + i0) =
          make_uint2(ql::pack_bf16x2(pv[a].x, pv[a].y), ql::pack_bf16x2(pv[a].z, pv[a].w));
    }
  } else {
    // the workgroup holding the end: element by element
    for (int a = 0; a < AV; ++a) {
      const int64_t i0 = (gbase + a * 256) * 4;
      for (int64_t i = i0; i < i0 + 4 && i < n; ++i) {
        float pe = p[i], me = m[i], ve = v[i];
        adam1(pe, me, ve, ql::bf16_to_f(g[i]), s);
        p[i] = pe;
        m[i] = me;
        v[i] = ve;
        out[i] = ql::f_to_bf16(pe);
      }
    }
  }
}

}  // namespace

qlora_status launch_adamw(float *p, float *m, float *v, const uint16_t *g, uint16_t *out,
                          int64_t n, const AdamScalars &s, hipStream_t st) {
  const int64_t blocks = ql_cdiv(ql_cdiv(n, 4), 256 * AV);
  if (blocks > 0x7fffffff) return QLORA_ERR_UNSUPPORTED;
  QlProf prof(QLORA_K_ADAMW, st);
  adamw_kernel<<<(unsigned)blocks, 256, 0, st>>>(p, m, v, g, out, n, s);
  QL_LAUNCH_CHECK();
  return QLORA_OK;
}
