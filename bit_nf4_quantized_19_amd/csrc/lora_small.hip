// Rank-r LoRA contractions and layout helpers, gfx950.
//
// The LoRA branch (Day-25 notes 2.1 and 6.2; QLoRA glossary, "QLoRA 的工作原理"):
//   forward   H  = X A^T                 (M x r, float32)
//   backward  G  = dY B                  (M x r, float32)
//             dB = s dY^T H              (d x r, bf16)
//             dA = s G^T X               (r x k, bf16)
// Each reads one M x C activation once (X or dY) and is memory-bound; the
// aim is to keep enough loads in flight and few launches.
//   * skinny: out[m][t] = sum_c In[m][c] P[t][c] on MFMA 16x16x32 (the rows
//     of In and of P are both contiguous in c). A wave owns a 16-token x
//     16-t block over a contiguous range of c and issues the loads of eight
//     32-wide K-slices before their MFMAs; the c range is split S ways
//     (S <= 8) into partial sums that a second kernel adds in a fixed order,
//     also emitting s*out as bf16 hi/lo parts for the fused GEMM epilogue.
//   * colacc: out[c][t] = s sum_m In[m][c] Q[m][t] on float32 FMA, one lane
//     per two columns, the Q rows of four tokens at a time read by scalar
//     loads; eight waves per workgroup on disjoint token ranges, reduced in
//     LDS in a fixed order; the token range is split S ways into partial sums
//     that a second kernel adds in a fixed order. dB and dA run as two
//     problems of one launch, and their reductions as one launch.
//   * layout: the zero-padded and transposed copies of A and B the other
//     kernels read (A^T for the dX epilogue, B^T for G), in one launch.
// r is padded to rp (a multiple of 16) with zero rows/columns.
#include <algorithm>

#include "kernels.h"

namespace {

// ---- layout ------------------------------------------------------------------
struct LayoutJob {
  const uint16_t *src;
  int64_t rows, cols;    // source shape (row-major)
  uint16_t *dst;
  int64_t drows, dcols;  // destination shape
  int transpose;         // dst[i][j] = src[j][i] instead of src[i][j]
  int64_t n;             // drows * dcols (0: unused)
};
struct LayoutJobs {
  LayoutJob j[4];
};

__global__ __launch_bounds__(256) void layout_kernel(LayoutJobs jobs) {
  int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const LayoutJob &J = jobs.j[q];
    if (idx < J.n) {
      const int64_t i = idx / J.dcols, jj = idx % J.dcols;
      uint16_t v = 0;
      if (!J.transpose) {
        if (i < J.rows && jj < J.cols) v = J.src[i * J.cols + jj];
      } else {
        if (jj < J.rows && i < J.cols) v = J.src[jj * J.cols + i];
      }
      J.dst[idx] = v;
      return;
    }
    idx -= J.n;
  }
}

// ---- skinny -----------------------------------------------------------------
constexpr int SK_MAXSPLIT = 8;
constexpr int SK_UNROLL = 8;   // K-slices of 32 whose loads are issued together

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
  const uint16_t *inr = In + (m_ok ? m : 0) * C + 8 * kq;
  const uint16_t *pr = P + (tbi * 16 + r16) * C + 8 * kq;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int64_t c = c_lo; c < c_hi; c += 32 * SK_UNROLL) {
    uint4 a[SK_UNROLL], b[SK_UNROLL];
#pragma unroll
    for (int u = 0; u < SK_UNROLL; ++u) {
      const int64_t cc = c + 32 * u;
      a[u] = ql::zero4();
      b[u] = ql::zero4();
      if (cc + 8 * kq < c_hi) {   // C % 8 == 0: a chunk is all in or all out
        if (m_ok) a[u] = *(const uint4 *)(inr + cc);
        b[u] = *(const uint4 *)(pr + cc);
      }
    }
#pragma unroll
    for (int u = 0; u < SK_UNROLL; ++u) acc = ql::mfma16(a[u], b[u], acc);
  }
  // lane holds D[4kq + i][r16] = out[m-block row 4kq+i][t = tbi*16 + r16]
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t mm = mb * 16 + 4 * kq + i;
    if (mm < M) part[(split * M + mm) * rp + tbi * 16 + r16] = acc[i];
  }
}

// one thread per 4 consecutive t of one token
__global__ __launch_bounds__(256) void skinny_reduce_kernel(
    const float *__restrict__ part, int S, int64_t M, int rp, float *__restrict__ out,
    float *__restrict__ out2, int out2_ld, float s, uint16_t *__restrict__ hi,
    uint16_t *__restrict__ lo) {
  const int64_t idx4 = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx4 * 4 >= M * rp) return;
  const int64_t idx = idx4 * 4;
  const int64_t m = idx / rp, t = idx % rp;
  float4 p[SK_MAXSPLIT];
#pragma unroll
  for (int sp = 0; sp < SK_MAXSPLIT; ++sp)
    if (sp < S) p[sp] = *(const float4 *)(part + sp * M * rp + idx);
  float v[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int sp = 0; sp < SK_MAXSPLIT; ++sp)
    if (sp < S) {
      v[0] += p[sp].x;
      v[1] += p[sp].y;
      v[2] += p[sp].z;
      v[3] += p[sp].w;
    }
  *(float4 *)(out + idx) = make_float4(v[0], v[1], v[2], v[3]);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if (out2 && t + e < out2_ld) out2[m * out2_ld + t + e] = v[e];
    if (hi) {
      const float sv = s * v[e];
      const uint16_t hb = ql::f_to_bf16(sv);
      hi[idx + e] = hb;
      lo[idx + e] = ql::f_to_bf16(sv - ql::bf16_to_f(hb));
    }
  }
}

// ---- colacc -------------------------------------------------------------------
constexpr int CA_COLS = 128;     // columns per wave (two per lane)
constexpr int CA_MAXSPLIT = 16;
constexpr int CA_TOK = 4;        // tokens per inner batch
constexpr int CA_W = 8;          // waves per workgroup

struct ColaccProb {
  const uint16_t *In;  // M x C
  int64_t C;
  const float *Q;      // M x rp
  float *part;         // S x C x rp
  int64_t groups;      // column groups of CA_COLS
};

// grid: x = column groups of problem 0 then problem 1 (times rp/16 t-blocks),
// y = token split. The waves of a workgroup split the split's tokens.
__global__ __launch_bounds__(64 * CA_W) void colacc_kernel(ColaccProb p0, ColaccProb p1,
                                                           int64_t M, int rp, int64_t mps) {
  __shared__ float red[CA_W - 1][64][32];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t tbs = rp / 16;
  int64_t gx = blockIdx.x;
  const bool second = gx >= p0.groups * tbs;
  const ColaccProb &P = second ? p1 : p0;
  if (second) gx -= p0.groups * tbs;
  const int64_t cg = gx / tbs, tb = gx % tbs;
  const int64_t c0 = cg * CA_COLS + 2 * lane;
  const int t0 = (int)tb * 16;
  const int64_t split = blockIdx.y;
  const int64_t m_lo = split * mps, m_hi = min(M, m_lo + mps);
  const int64_t span = m_hi - m_lo;
  const int64_t w_lo = m_lo + (span * wave) / CA_W, w_hi = m_lo + (span * (wave + 1)) / CA_W;
  float acc[2][16];
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int t = 0; t < 16; ++t) acc[c][t] = 0.0f;
  const bool c_ok = c0 < P.C;  // C % 8 == 0, so c0 + 1 < C as well
  const uint16_t *inc = P.In + (c_ok ? c0 : 0);
  int64_t m = w_lo;
  for (; m + CA_TOK <= w_hi; m += CA_TOK) {
    uint32_t v[CA_TOK];
#pragma unroll
    for (int u = 0; u < CA_TOK; ++u) v[u] = c_ok ? *(const uint32_t *)(inc + (m + u) * P.C) : 0u;
#pragma unroll
    for (int u = 0; u < CA_TOK; ++u) {
      // Q row m+u is wave-uniform: scalar loads, broadcast to the FMAs
      const float *qrow = P.Q + (m + u) * rp + t0;
      const float x0 = ql::bf16lo(v[u]), x1 = ql::bf16hi(v[u]);
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const float qv = qrow[t];
        acc[0][t] = fmaf(x0, qv, acc[0][t]);
        acc[1][t] = fmaf(x1, qv, acc[1][t]);
      }
    }
  }
  for (; m < w_hi; ++m) {
    const uint32_t v = c_ok ? *(const uint32_t *)(inc + m * P.C) : 0u;
    const float *qrow = P.Q + m * rp + t0;
    const float x0 = ql::bf16lo(v), x1 = ql::bf16hi(v);
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const float qv = qrow[t];
      acc[0][t] = fmaf(x0, qv, acc[0][t]);
      acc[1][t] = fmaf(x1, qv, acc[1][t]);
    }
  }
  // reduce the waves in a fixed order: ((wave 0 + 1) + 2) + ...
  if (wave > 0) {
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int t = 0; t < 16; ++t) red[wave - 1][lane][c * 16 + t] = acc[c][t];
  }
  __syncthreads();
  if (wave == 0 && c_ok) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      float o[16];
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        o[t] = acc[c][t];
#pragma unroll
        for (int w = 0; w < CA_W - 1; ++w) o[t] += red[w][lane][c * 16 + t];
      }
      float *dst = P.part + (split * P.C + c0 + c) * rp + t0;
#pragma unroll
      for (int t = 0; t < 16; t += 4) *(float4 *)(dst + t) = make_float4(o[t], o[t + 1], o[t + 2], o[t + 3]);
    }
  }
}

struct ColaccOut {
  const float *part;  // S x C x rp
  int64_t C;
  uint16_t *out;
  int transpose_out;  // 0: out is C x r; 1: out is r x C
  int64_t n;          // C * r
};

// one thread per output element of problem 0 then problem 1
__global__ __launch_bounds__(256) void colacc_reduce_kernel(ColaccOut o0, ColaccOut o1, int S,
                                                            int rp, int r, float s) {
  int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const bool second = idx >= o0.n;
  const ColaccOut &O = second ? o1 : o0;
  if (second) idx -= o0.n;
  if (idx >= O.n) return;
  int64_t c, t;
  if (O.transpose_out) {
    t = idx / O.C;
    c = idx % O.C;
  } else {
    c = idx / r;
    t = idx % r;
  }
  float p[CA_MAXSPLIT];
#pragma unroll
  for (int sp = 0; sp < CA_MAXSPLIT; ++sp)
    if (sp < S) p[sp] = O.part[(sp * O.C + c) * rp + t];
  float v = 0.0f;
#pragma unroll
  for (int sp = 0; sp < CA_MAXSPLIT; ++sp)
    if (sp < S) v += p[sp];
  O.out[idx] = ql::f_to_bf16(s * v);
}

int64_t colacc_split(int64_t M, int64_t C, int rp) {
  // about 256 workgroups of CA_W waves, each wave with at least 64 tokens
  const int64_t wgs = ql_cdiv(C, CA_COLS) * (rp / 16);
  int64_t S = ql_cdiv(256, wgs);
  S = std::min<int64_t>(S, std::max<int64_t>(1, M / (64 * CA_W)));
  return std::min<int64_t>(std::max<int64_t>(S, 1), CA_MAXSPLIT);
}

int64_t host_skinny_split(int64_t M, int64_t C, int rp) {
  // about 2048 waves in all, each with at least 8 K-slices of 32
  const int64_t items = ql_cdiv(M, 16) * (rp / 16);
  int64_t S = ql_cdiv(2048, items);
  S = std::min<int64_t>(S, std::max<int64_t>(1, C / (32 * SK_UNROLL)));
  return std::min<int64_t>(std::max<int64_t>(S, 1), SK_MAXSPLIT);
}

}  // namespace

qlora_status launch_layout(const LayoutReq *req, int nreq, hipStream_t st) {
  LayoutJobs jobs{};
  int64_t total = 0;
  for (int q = 0; q < 4; ++q) {
    if (q < nreq && req[q].dst) {
      const LayoutReq &R = req[q];
      jobs.j[q] = LayoutJob{R.src, R.rows, R.cols, R.dst, R.drows, R.dcols, R.transpose,
                            R.drows * R.dcols};
      total += R.drows * R.dcols;
    } else {
      jobs.j[q] = LayoutJob{nullptr, 0, 0, nullptr, 0, 1, 0, 0};
    }
  }
  if (total == 0) return QLORA_OK;
  QlProf prof(QLORA_K_LAYOUT, st);
  layout_kernel<<<(unsigned)ql_cdiv(total, 256), 256, 0, st>>>(jobs);
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
  skinny_reduce_kernel<<<(unsigned)ql_cdiv(M * rp / 4, 256), 256, 0, st>>>(
      part, (int)S, M, rp, out, out2, out2_ld, s, hi, lo);
  QL_LAUNCH_CHECK();
  return QLORA_OK;
}

size_t colacc_part_bytes(int64_t M, int64_t C0, int64_t C1, int rp) {
  const int64_t S = colacc_split(M, C0 + C1, rp);
  return (size_t)(S * (C0 + C1) * rp * 4);
}

qlora_status launch_colacc2(const ColaccReq &a, const ColaccReq &b, int64_t M, int rp, int r,
                            float s, float *part, hipStream_t st) {
  const int64_t S0 = colacc_split(M, a.C + b.C, rp);
  const int64_t mps = ql_cdiv(M, S0);
  const int64_t S = ql_cdiv(M, mps);
  ColaccProb p0{a.In, a.C, a.Q, part, ql_cdiv(a.C, CA_COLS)};
  ColaccProb p1{b.In, b.C, b.Q, part + S * a.C * rp, ql_cdiv(b.C, CA_COLS)};
  const int64_t tbs = rp / 16;
  dim3 grid((unsigned)((p0.groups + p1.groups) * tbs), (unsigned)S);
  {
    QlProf prof(QLORA_K_LORA_COLACC, st);
    colacc_kernel<<<grid, 64 * CA_W, 0, st>>>(p0, p1, M, rp, mps);
  }
  ColaccOut o0{p0.part, a.C, a.out, a.transpose_out, a.C * r};
  ColaccOut o1{p1.part, b.C, b.out, b.transpose_out, b.C * r};
  QlProf prof(QLORA_K_LORA_COLACC_REDUCE, st);
  colacc_reduce_kernel<<<(unsigned)ql_cdiv(o0.n + o1.n, 256), 256, 0, st>>>(o0, o1, (int)S, rp,
                                                                           r, s);
  QL_LAUNCH_CHECK();
  return QLORA_OK;
}
