// Memory-bound NF4 forward for few tokens (M <= 16), gfx950.
//
// Same layer as the fused GEMM (QLoRA glossary, Ultralytics, "QLoRA 的工作原理",
// forward paragraph): Y = X W'^T + s H B^T. With M <= 16 the time is the HBM
// read of the packed codes (0.5 byte per weight), so the kernel moves as few
// bytes and issues as few VALU operations per weight as it can:
//   * The per-block scale is factored out of each 64-wide partial sum,
//     sum_b a'_b * sum_{c in b} level[code_c] x_c; the 64-term inner sums run
//     on MFMA (16x16x32 bf16, tokens padded to 16) with the levels as bf16
//     operands looked up two at a time from a 256-entry byte -> (level, level)
//     LDS table. This equals X W'^T up to float32/bf16 rounding (the weights
//     are rounded to bf16 at the level instead of after the product).
//   * Each wave streams 16 weight rows; a workgroup covers 64 rows and one of
//     S contraction splits; partial sums go to a small float32 buffer and a
//     second kernel adds the splits in a fixed order, the rank-r LoRA term in
//     float32, and rounds to bf16.
#include <algorithm>

#include "kernels.h"
#include "nf4_tables.h"

namespace {

constexpr int GT = 256;
__constant__ uint32_t c_levels_v[16] = NF4_LEVEL_BITS;

struct GemvArgs {
  const uint8_t *codes;
  ql::ScaleSrc sc;
  int64_t d, k;
  const uint16_t *X;
  int64_t M;
  int64_t blocks_per_split;
  float *part;  // [S][M][d]
};

__global__ __launch_bounds__(GT) void nf4_gemv_kernel(GemvArgs g) {
  __shared__ uint32_t lut[256];
  {
    const int b = threadIdx.x;
    const float hi = __uint_as_float(c_levels_v[b >> 4]);
    const float lo = __uint_as_float(c_levels_v[b & 15]);
    lut[b] = ql::pack_bf16x2(hi, lo);  // element 2j (high nibble) first
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t j0 = (int64_t)blockIdx.x * 64 + 16 * wave;
  const int64_t split = blockIdx.y;
  const int64_t nbr = g.k >> 6;  // blocks per row
  const int64_t b_lo = split * g.blocks_per_split;
  const int64_t b_hi = min(nbr, b_lo + g.blocks_per_split);
  if (j0 >= g.d) return;  // whole wave idle (d % 16 == 0)

  const int r16 = lane & 15, kq = lane >> 4;
  const int64_t arow = j0 + r16;            // weight row this lane feeds (A operand)
  const bool arow_ok = arow < g.d;
  const int64_t xrow = r16;                 // token row this lane feeds (B operand)
  const bool xrow_ok = xrow < g.M;
  // rows of the accumulator this lane holds: j0 + 4*kq + i
  const float mu = g.sc.dq ? g.sc.mu[0] : 0.0f;
  int64_t grow[4];
  float s2lo[4], s2hi[4];
  int64_t glo[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    grow[i] = j0 + 4 * kq + i;
    const int64_t r = grow[i] < g.d ? grow[i] : (g.d - 1);
    grow[i] = r;
    if (g.sc.dq) {
      glo[i] = (r * nbr + b_lo) >> 8;
      const int64_t ghi = (r * nbr + max(b_hi - 1, b_lo)) >> 8;
      s2lo[i] = g.sc.s2[glo[i]];
      s2hi[i] = g.sc.s2[ghi];
    }
  }

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  const uint8_t *crow = g.codes + ((arow_ok ? arow : 0) * g.k >> 1);
  const uint16_t *xr = g.X + (xrow_ok ? xrow : 0) * g.k;

#pragma unroll 4
  for (int64_t b = b_lo; b < b_hi; ++b) {
    const int64_t kb = b << 6;
    uint32_t c0 = 0, c1 = 0;
    if (arow_ok) {
      c0 = *(const uint32_t *)(crow + ((kb + 8 * kq) >> 1));
      c1 = *(const uint32_t *)(crow + ((kb + 32 + 8 * kq) >> 1));
    }
    uint4 x0 = ql::zero4(), x1 = ql::zero4();
    if (xrow_ok) {
      x0 = *(const uint4 *)(xr + kb + 8 * kq);
      x1 = *(const uint4 *)(xr + kb + 32 + 8 * kq);
    }
    uint4 a0, a1;
    a0.x = lut[c0 & 255]; a0.y = lut[(c0 >> 8) & 255];
    a0.z = lut[(c0 >> 16) & 255]; a0.w = lut[c0 >> 24];
    a1.x = lut[c1 & 255]; a1.y = lut[(c1 >> 8) & 255];
    a1.z = lut[(c1 >> 16) & 255]; a1.w = lut[c1 >> 24];
    f32x4 p = ql::mfma16(a0, x0, zero);
    p = ql::mfma16(a1, x1, p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t blk = grow[i] * nbr + b;
      float ap;
      if (g.sc.dq) {
        const float s2 = ((blk >> 8) == glo[i]) ? s2lo[i] : s2hi[i];
        ap = (float)g.sc.q[blk] * s2 + mu;
      } else {
        ap = g.sc.absmax[blk];
      }
      acc[i] = fmaf(ap, p[i], acc[i]);
    }
  }
  // lane holds D[4*kq + i][r16] = partial Y[token r16][row j0 + 4kq + i]
  if (r16 < g.M) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t row = j0 + 4 * kq + i;
      if (row < g.d) g.part[(split * g.M + r16) * g.d + row] = acc[i];
    }
  }
}

__global__ __launch_bounds__(256) void gemv_epilogue_kernel(
    const float *__restrict__ part, int S, int64_t M, int64_t d,
    const uint16_t *__restrict__ Bp, const float *__restrict__ H, int rp, float s,
    uint16_t *__restrict__ Y) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= M * d) return;
  const int64_t m = idx / d, j = idx % d;
  float acc = 0.0f;
  for (int sp = 0; sp < S; ++sp) acc += part[(sp * M + m) * d + j];
  float l = 0.0f;
  for (int t = 0; t < rp; ++t) l = fmaf(H[m * rp + t], ql::bf16_to_f(Bp[j * rp + t]), l);
  Y[idx] = ql::f_to_bf16(acc + s * l);
}

}  // namespace

static int64_t gemv_splits(int64_t d, int64_t k) {
  const int64_t nbr = k >> 6;
  const int64_t wgs = ql_cdiv(d, 64);
  int64_t S = ql_cdiv(1024, wgs);
  S = std::min<int64_t>(S, std::max<int64_t>(1, nbr / 8));  // >= 8 blocks per wave
  S = std::max<int64_t>(S, ql_cdiv(nbr, 256));              // <= 256 blocks per split
  return std::max<int64_t>(S, 1);
}

size_t gemv_part_bytes(int64_t d, int64_t k, int64_t M) {
  return (size_t)(gemv_splits(d, k) * M * d * 4);
}

qlora_status launch_gemv_fwd(const uint8_t *codes, ql::ScaleSrc sc, int64_t d, int64_t k,
                             const uint16_t *X, int64_t M, const uint16_t *Bp,
                             const float *H, int rp, float s, float *part, uint16_t *Y,
                             hipStream_t st) {
  const int64_t nbr = k >> 6;
  const int64_t S = gemv_splits(d, k);
  const int64_t bps = ql_cdiv(nbr, S);
  GemvArgs g{codes, sc, d, k, X, M, bps, part};
  dim3 grid((unsigned)ql_cdiv(d, 64), (unsigned)ql_cdiv(nbr, bps));
  {
    QlProf prof(QLORA_K_GEMV, st);
    nf4_gemv_kernel<<<grid, GT, 0, st>>>(g);
  }
  {
    QlProf prof(QLORA_K_GEMV_EPILOGUE, st);
    gemv_epilogue_kernel<<<(unsigned)ql_cdiv(M * d, 256), 256, 0, st>>>(
        part, (int)grid.y, M, d, Bp, H, rp, s, Y);
  }
  QL_LAUNCH_CHECK();
  return QLORA_OK;
}
