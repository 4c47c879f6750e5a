// Merge of the LoRA update into the dequantised base, gfx950.
//
// Day-25 notes 2.6 (W_merged = W0 + B A) and 6.2 (scale alpha/r); LLM
// tutorial ch. 3, 3.8 and QLoRA glossary "权衡": a 4-bit base is dequantised
// to 16 bits before merging. Here
//     W_m = bf16(fl(w' + fl(s * sum_t B[j][t] A[t][c])))
// with w' the bf16 dequantised weight and the rank-r sum in float32 (FMA,
// t ascending). Workgroup tile: 32 rows x 64 columns; the A columns and B
// rows of the tile are staged in LDS; each lane produces 8 consecutive
// outputs from one 4-byte code word.
#include "kernels.h"
#include "nf4_tables.h"

namespace {

constexpr int MR = 32, MC = 64, MAXR = 128;
__constant__ uint32_t c_levels_m[16] = NF4_LEVEL_BITS;

__global__ __launch_bounds__(256) void merge_kernel(const uint8_t *__restrict__ codes,
                                                    ql::ScaleSrc sc, int64_t d, int64_t k,
                                                    const uint16_t *__restrict__ A,
                                                    const uint16_t *__restrict__ B, int r,
                                                    float s, uint16_t *__restrict__ Wm) {
  __shared__ float As[MAXR][MC];  // A[t][c0..c0+63]
  __shared__ float Bs[MR][MAXR];  // B[j0..j0+31][t]
  __shared__ float lv[16];
  const int tid = threadIdx.x;
  const int64_t j0 = (int64_t)blockIdx.y * MR, c0 = (int64_t)blockIdx.x * MC;
  if (tid < 16) lv[tid] = __uint_as_float(c_levels_m[tid]);
  for (int e = tid; e < r * MC; e += 256) {
    const int t = e / MC, c = e % MC;
    As[t][c] = (c0 + c < k) ? ql::bf16_to_f(A[(int64_t)t * k + c0 + c]) : 0.0f;
  }
  for (int e = tid; e < MR * r; e += 256) {
    const int jj = e / r, t = e % r;
    Bs[jj][t] = (j0 + jj < d) ? ql::bf16_to_f(B[(j0 + jj) * r + t]) : 0.0f;
  }
  __syncthreads();
  const int jj = tid >> 3, cg = (tid & 7) * 8;
  const int64_t j = j0 + jj, c = c0 + cg;
  if (j >= d || c >= k) return;
  const float mu = sc.dq ? sc.mu[0] : 0.0f;
  const int64_t e0 = j * k + c;
  const uint32_t cw = *(const uint32_t *)(codes + (e0 >> 1));
  const float ap = ql::block_scale(sc, e0 >> 6, mu);
  float ba[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) ba[i] = 0.0f;
  for (int t = 0; t < r; ++t) {
    const float bv = Bs[jj][t];
#pragma unroll
    for (int i = 0; i < 8; ++i) ba[i] = fmaf(bv, As[t][cg + i], ba[i]);
  }
  float o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int sh = 8 * (i >> 1) + ((i & 1) ? 0 : 4);
    const float wq = ql::bf16_to_f(ql::f_to_bf16(lv[(cw >> sh) & 15u] * ap));
    o[i] = wq + s * ba[i];
  }
  uint4 out;
  out.x = ql::pack_bf16x2(o[0], o[1]);
  out.y = ql::pack_bf16x2(o[2], o[3]);
  out.z = ql::pack_bf16x2(o[4], o[5]);
  out.w = ql::pack_bf16x2(o[6], o[7]);
  *(uint4 *)(Wm + e0) = out;
}

}  // namespace

qlora_status launch_merge(const uint8_t *codes, ql::ScaleSrc sc, int64_t d, int64_t k,
                          const uint16_t *A, const uint16_t *B, int r, float s, uint16_t *Wm,
                          hipStream_t st) {
  dim3 grid((unsigned)ql_cdiv(k, MC), (unsigned)ql_cdiv(d, MR));
  QlProf prof(QLORA_K_MERGE, st);
  merge_kernel<<<grid, 256, 0, st>>>(codes, sc, d, k, A, B, r, s, Wm);
  QL_LAUNCH_CHECK();
  return QLORA_OK;
}
