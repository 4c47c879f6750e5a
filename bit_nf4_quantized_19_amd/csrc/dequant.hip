// Standalone NF4 dequantisation to bf16 for gfx950 (QLoRA glossary,
// Ultralytics, "QLoRA 的工作原理": frozen weights are dequantised to bfloat16
// before the matmul; LLM tutorial ch. 3, 3.8: a 4-bit base is dequantised to
// bf16 before merging).
//
// w' = bf16_rne(fl(level[code] * a')), a' = fl(fl(q * s2) + mu) or absmax.
// Memory-bound: 2.516 bytes moved per weight (0.5 code + block scale share in,
// 2 out). A lane owns 4-byte code words (8 weights, one 16-byte output store);
// a wave's load and store instructions each cover one contiguous run (256
// bytes of codes, 1 KB of output), and every lane issues all its loads (DU
// code words and one block's scale inputs) before the first use: the 64
// blocks of a wave's words get their a' from one lane each and reach the
// lanes that need them by lane shuffles. Levels come from a 16-entry LDS
// table (any lookup pattern is conflict-free).
#include <algorithm>

#include "kernels.h"
#include "nf4_tables.h"

namespace {

constexpr int DT = 256;  // threads per workgroup
constexpr int DU = 8;    // code words per lane
__constant__ uint32_t c_levels[16] = NF4_LEVEL_BITS;

template <bool DQ>
__global__ __launch_bounds__(DT) void dequant_kernel(const uint32_t *__restrict__ codes,
                                                     ql::ScaleSrc sc, int64_t nchunks,
                                                     uint4 *__restrict__ out) {
  __shared__ float lv[16];
  if (threadIdx.x < 16) lv[threadIdx.x] = __uint_as_float(c_levels[threadIdx.x]);
  const int lane = threadIdx.x & 63;
  const int64_t w0 = ((int64_t)blockIdx.x * (DT / 64) + (threadIdx.x >> 6)) * (64 * DU);
  // loads: code words, then their scale inputs; indices past the end are
  // clamped (their results are not stored)
  uint32_t cw[DU];
  int64_t idx[DU];
#pragma unroll
  for (int i = 0; i < DU; ++i) {
    idx[i] = w0 + 64 * i + lane;
    cw[i] = codes[min(idx[i], nchunks - 1)];
  }
  // block scales: the wave's code words cover the 64 consecutive blocks
  // w0 / 8 ..; lane l derives a' of block w0 / 8 + l (one load of each scale
  // input), and the lane holding word i of block 8 i + lane / 8 takes it
  // from lane 8 i + lane / 8
  const int64_t nb = nchunks >> 3;
  const int64_t blk = min((w0 >> 3) + lane, nb - 1);
  float a_l;
  if (DQ) {
    const float qv = (float)sc.q[blk];
    const float s2 = sc.s2[blk >> 8];
    const float prod = qv * s2;
    a_l = prod + sc.mu[0];
  } else {
    a_l = sc.absmax[blk];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < DU; ++i) {
    const float ap = __shfl(a_l, 8 * i + (lane >> 3));
    const uint32_t c = cw[i];
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
    if (idx[i] < nchunks) out[idx[i]] = o;
  }
}

}  // namespace

qlora_status launch_dequantize(const uint8_t *codes, ql::ScaleSrc sc, int64_t n,
                               uint16_t *out, hipStream_t st) {
  const int64_t nchunks = n / 8;
  const int64_t grid = ql_cdiv(nchunks, (int64_t)DT * DU);
  if (grid > 0x7fffffff) return QLORA_ERR_UNSUPPORTED;
  QlProf prof(QLORA_K_DEQUANTIZE, st);
  if (sc.dq)
    dequant_kernel<true><<<(unsigned)grid, DT, 0, st>>>((const uint32_t *)codes, sc, nchunks,
                                                       (uint4 *)out);
  else
    dequant_kernel<false><<<(unsigned)grid, DT, 0, st>>>((const uint32_t *)codes, sc, nchunks,
                                                        (uint4 *)out);
  QL_LAUNCH_CHECK();
  return QLORA_OK;
}
