// Standalone NF4 dequantisation to bf16 for gfx950 (QLoRA glossary,
// Ultralytics, "QLoRA 的工作原理": frozen weights are dequantised to bfloat16
// before the matmul; LLM tutorial ch. 3, 3.8: a 4-bit base is dequantised to
// bf16 before merging).
//
// w' = bf16_rne(fl(level[code] * a')), a' = fl(fl(q * s2) + mu) or absmax.
// One lane per 8 codes (4 bytes in, 16 bytes out), 8 lanes per block;
// levels come from a 16-entry LDS table. Memory-bound: 2.516 bytes moved per
// weight (0.5 code + block scale share in, 2 out).
#include <algorithm>

#include "kernels.h"
#include "nf4_tables.h"

namespace {

constexpr int DT = 256;
__constant__ uint32_t c_levels[16] = NF4_LEVEL_BITS;

__global__ __launch_bounds__(DT) void dequant_kernel(const uint32_t *__restrict__ codes,
                                                     ql::ScaleSrc sc, int64_t nchunks,
                                                     uint4 *__restrict__ out) {
  __shared__ float lv[16];
  if (threadIdx.x < 16) lv[threadIdx.x] = __uint_as_float(c_levels[threadIdx.x]);
  __syncthreads();
  const float mu = sc.dq ? sc.mu[0] : 0.0f;
  const int64_t stride = (int64_t)gridDim.x * DT;
  for (int64_t ch = (int64_t)blockIdx.x * DT + threadIdx.x; ch < nchunks; ch += stride) {
    const uint32_t c = codes[ch];
    const float ap = ql::block_scale(sc, ch >> 3, mu);
    float f[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int sh = 8 * (e >> 1) + ((e & 1) ? 0 : 4);
      f[e] = lv[(c >> sh) & 15u] * ap;
    }
    uint4 o;
    o.x = ql::pack_bf16x2(f[0], f[1]);
    o.y = ql::pack_bf16x2(f[2], f[3]);
    o.z = ql::pack_bf16x2(f[4], f[5]);
    o.w = ql::pack_bf16x2(f[6], f[7]);
    out[ch] = o;
  }
}

}  // namespace

qlora_status launch_dequantize(const uint8_t *codes, ql::ScaleSrc sc, int64_t n,
                               uint16_t *out, hipStream_t st) {
  const int64_t nchunks = n / 8;
  const int grid = (int)std::min<int64_t>(ql_cdiv(nchunks, DT), 8192);
  QlProf prof(QLORA_K_DEQUANTIZE, st);
  dequant_kernel<<<grid, DT, 0, st>>>((const uint32_t *)codes, sc, nchunks, (uint4 *)out);
  QL_LAUNCH_CHECK();
  return QLORA_OK;
}
