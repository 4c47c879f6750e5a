// Rank-r LoRA contractions and layout helpers, gfx950.
//
// The LoRA branch (Day-25 notes 2.1 and 6.2; QLoRA glossary, "QLoRA 的工作原理"):
//   forward   H  = X A^T                 (M x r, float32)
//   backward  G  = dY B                  (M x r, float32)
//             dB = s dY^T H              (d x r, bf16)
//             dA = s G^T X               (r x k, bf16)
// Each reads one M x C activation once (X or dY); they are memory-bound.
//   * skinny: out[m][t] = sum_c In[m][c] P[t][c] on MFMA 16x16x32 (the row
//     of In and of P are both contiguous in c), split over c into a fixed
//     number of partial sums that a second kernel adds in order; the second
//     kernel also emits s*out as bf16 hi/lo parts for the fused GEMM epilogue.
//   * colacc: out[c][t] = s sum_m In[m][c] Q[m][t] on float32 FMA, one lane
//     per two columns, Q rows read by scalar loads, 4 waves per workgroup on
//     disjoint token ranges reduced in LDS, split over tokens into partial
//     sums added in a fixed order by a second kernel.
// r is padded to rp (a multiple of 16) with zero rows/columns.
#include <algorithm>

#include "kernels.h"

namespace {

__global__ void pad_copy_kernel(const uint16_t *__restrict__ src, int64_t rows, int64_t cols,
                                uint16_t *__restrict__ dst, int64_t drows, int64_t dcols,
                                int transpose) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= drows * dcols) return;
  const int64_t i = idx / dcols, j = idx % dcols;
  uint16_t v = 0;
  if (!transpose) {
    if (i < rows && j < cols) v = src[i * cols + j];
  } else {
    if (j < rows && i < cols) v = src[j * cols + i];
  }
  dst[idx] = v;
}

constexpr int SK_MAXSPLIT = 64;

// grid: x = wave items (m-block, t-block) / 4 per workgroup, y = split
__global__ __launch_bounds__(256) void skinny_kernel(const uint16_t *__restrict__ In, int64_t M,
                                                     int64_t C, const uint16_t *__restrict__ P,
                                                     int rp, int64_t cps,
                                                     float *__restrict__ part) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t item = (int64_t)blockIdx.x * 4 + wave;
  const int64_t tb = rp / 16;
  const int64_t mb = item / tb, tbi = item % tb;
  if (mb * 16 >= M) return;
  const int64_t split = blockIdx.y;
  const int64_t c_lo = split * cps, c_hi = min(C, c_lo + cps);
  const int r16 = lane & 15, kq = lane >> 4;
  const int64_t m = mb * 16 + r16;
  const bool m_ok = m < M;
  const uint16_t *inr = In + (m_ok ? m : 0) * C;
  const uint16_t *pr = P + (tbi * 16 + r16) * C;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int64_t c = c_lo; c < c_hi; c += 32) {
    const int64_t cc = c + 8 * kq;
    uint4 a = ql::zero4(), b = ql::zero4();
    if (cc < c_hi) {
      if (m_ok) a = *(const uint4 *)(inr + cc);
      b = *(const uint4 *)(pr + cc);
    }
    acc = ql::mfma16(a, b, acc);
  }
  // lane holds D[4kq + i][r16] = out[m-block row 4kq+i][t = tbi*16 + r16]
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t mm = mb * 16 + 4 * kq + i;
    if (mm < M) part[(split * M + mm) * rp + tbi * 16 + r16] = acc[i];
  }
}

__global__ __launch_bounds__(256) void skinny_reduce_kernel(
    const float *__restrict__ part, int S, int64_t M, int rp, float *__restrict__ out,
    float *__restrict__ out2, int out2_ld, float s, uint16_t *__restrict__ hi,
    uint16_t *__restrict__ lo) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= M * rp) return;
  const int64_t m = idx / rp, t = idx % rp;
  float v = 0.0f;
  for (int sp = 0; sp < S; ++sp) v += part[(sp * M + m) * rp + t];
  out[idx] = v;
  if (out2 && t < out2_ld) out2[m * out2_ld + t] = v;
  if (hi) {
    const float sv = s * v;
    const uint16_t h = ql::f_to_bf16(sv);
    hi[idx] = h;
    lo[idx] = ql::f_to_bf16(sv - ql::bf16_to_f(h));
  }
}

// colacc: grid x = column groups of 128, y = t groups of 16, z = token splits
constexpr int CA_COLS = 128;
__global__ __launch_bounds__(256) void colacc_kernel(const uint16_t *__restrict__ In, int64_t M,
                                                     int64_t C, const float *__restrict__ Q,
                                                     int rp, int64_t mps,
                                                     float *__restrict__ part) {
  __shared__ float red[3][64][32];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t c0 = (int64_t)blockIdx.x * CA_COLS + 2 * lane;
  const int t0 = blockIdx.y * 16;
  const int64_t split = blockIdx.z;
  const int64_t m_lo = split * mps, m_hi = min(M, m_lo + mps);
  // this wave's token sub-range
  const int64_t span = m_hi - m_lo;
  const int64_t w_lo = m_lo + (span * wave) / 4, w_hi = m_lo + (span * (wave + 1)) / 4;
  float acc[2][16];
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int t = 0; t < 16; ++t) acc[c][t] = 0.0f;
  const bool c_ok = c0 < C;  // C % 8 == 0, so c0 + 1 < C as well
  for (int64_t m = w_lo; m < w_hi; ++m) {
    // Q row m is wave-uniform: scalar loads, broadcast to the FMAs
    const float *qrow = Q + m * rp + t0;
    const uint32_t v = c_ok ? *(const uint32_t *)(In + m * C + c0) : 0u;
    const float x0 = ql::bf16lo(v), x1 = ql::bf16hi(v);
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const float qv = qrow[t];
      acc[0][t] = fmaf(x0, qv, acc[0][t]);
      acc[1][t] = fmaf(x1, qv, acc[1][t]);
    }
  }
  // reduce the 4 waves in fixed order: wave 0 + 1 + 2 + 3
  if (wave > 0) {
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int t = 0; t < 16; ++t) red[wave - 1][lane][c * 16 + t] = acc[c][t];
  }
  __syncthreads();
  if (wave == 0 && c_ok) {
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const float v = ((acc[c][t] + red[0][lane][c * 16 + t]) + red[1][lane][c * 16 + t]) +
                        red[2][lane][c * 16 + t];
        part[(split * C + c0 + c) * rp + t0 + t] = v;
      }
  }
}

__global__ __launch_bounds__(256) void colacc_reduce_kernel(const float *__restrict__ part, int S,
                                                            int64_t C, int rp, int r, float s,
                                                            uint16_t *__restrict__ out,
                                                            int transpose_out) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= C * r) return;
  int64_t c, t;
  if (transpose_out) {
    t = idx / C;
    c = idx % C;
  } else {
    c = idx / r;
    t = idx % r;
  }
  float v = 0.0f;
  for (int sp = 0; sp < S; ++sp) v += part[(sp * C + c) * rp + t];
  out[idx] = ql::f_to_bf16(s * v);
}

int64_t colacc_split(int64_t M, int64_t C, int rp) {
  const int64_t wgs = ql_cdiv(C, CA_COLS) * (rp / 16);
  int64_t S = ql_cdiv(1024, wgs);
  S = std::min<int64_t>(S, std::max<int64_t>(1, M / 64));
  return std::max<int64_t>(S, 1);
}

int64_t host_skinny_split(int64_t M, int64_t C, int rp) {
  const int64_t items = ql_cdiv(M, 16) * (rp / 16);
  int64_t S = ql_cdiv(2048, items);
  S = std::min<int64_t>(S, std::max<int64_t>(1, C / 256));
  return std::min<int64_t>(std::max<int64_t>(S, 1), SK_MAXSPLIT);
}

}  // namespace

qlora_status launch_pad_copy(const uint16_t *src, int64_t rows, int64_t cols, uint16_t *dst,
                             int64_t drows, int64_t dcols, int transpose, hipStream_t st) {
  const int64_t n = drows * dcols;
  QlProf prof(QLORA_K_LAYOUT, st);
  pad_copy_kernel<<<(unsigned)ql_cdiv(n, 256), 256, 0, st>>>(src, rows, cols, dst, drows, dcols,
                                                              transpose);
  QL_LAUNCH_CHECK();
  return QLORA_OK;
}

size_t skinny_part_bytes(int64_t M, int64_t C, int rp) {
  return (size_t)(host_skinny_split(M, C, rp) * M * rp * 4);
}

qlora_status launch_skinny(const uint16_t *In, int64_t M, int64_t C, const uint16_t *P, int rp,
                           float *part, float *out, int64_t out_ld, float *out2, int out2_ld,
                           float s, uint16_t *hi, uint16_t *lo, hipStream_t st) {
  (void)out_ld;
  const int64_t S0 = host_skinny_split(M, C, rp);
  const int64_t cps = ql_rup(ql_cdiv(C, S0), 32);
  const int64_t S = ql_cdiv(C, cps);
  const int64_t items = ql_cdiv(M, 16) * (rp / 16);
  dim3 grid((unsigned)ql_cdiv(items, 4), (unsigned)S);
  {
    QlProf prof(QLORA_K_LORA_DOWN, st);
    skinny_kernel<<<grid, 256, 0, st>>>(In, M, C, P, rp, cps, part);
  }
  QlProf prof(QLORA_K_LORA_REDUCE, st);
  skinny_reduce_kernel<<<(unsigned)ql_cdiv(M * rp, 256), 256, 0, st>>>(part, (int)S, M, rp, out,
                                                                       out2, out2_ld, s, hi, lo);
  QL_LAUNCH_CHECK();
  return QLORA_OK;
}

size_t colacc_part_bytes(int64_t M, int64_t C, int rp) {
  return (size_t)(colacc_split(M, C, rp) * C * rp * 4);
}

qlora_status launch_colacc(const uint16_t *In, int64_t M, int64_t C, const float *Q, int rp,
                           int r, float s, float *part, uint16_t *out, int transpose_out,
                           hipStream_t st) {
  const int64_t S0 = colacc_split(M, C, rp);
  const int64_t mps = ql_cdiv(M, S0);
  const int64_t S = ql_cdiv(M, mps);
  dim3 grid((unsigned)ql_cdiv(C, CA_COLS), (unsigned)(rp / 16), (unsigned)S);
  {
    QlProf prof(QLORA_K_LORA_COLACC, st);
    colacc_kernel<<<grid, 256, 0, st>>>(In, M, C, Q, rp, mps, part);
  }
  QlProf prof(QLORA_K_LORA_COLACC_REDUCE, st);
  colacc_reduce_kernel<<<(unsigned)ql_cdiv(C * r, 256), 256, 0, st>>>(part, (int)S, C, rp, r, s,
                                                                      out, transpose_out);
  QL_LAUNCH_CHECK();
  return QLORA_OK;
}
