// Rank-r LoRA contractions and layout helpers, gfx950.
//
// The LoRA branch (Day-25 notes 2.1 and 6.2; QLoRA glossary, "QLoRA 的工作原理"):
//   forward   H  = X A^T                 (M x r, float32)
//   backward  G  = dY B                  (M x r, float32)
//             dB = s dY^T H              (d x r, bf16)
//             dA = s G^T X               (r x k, bf16)
// Each reads one M x C activation once (X or dY) and is memory-bound; the
// aim is to keep enough loads in flight and few launches.
//   * skinny: out[m][t] = sum_c In[m][c] P[t][c] on MFMA 16x16x32, one
//     launch: a workgroup owns an 8-token x 16-t block (the MFMA tile's
//     other 8 rows stay zero, so 2048 tokens fill the chip), its 16 waves split
//     the c range and issue the loads of eight 32-wide K-slices before their
//     MFMAs, and the waves' sums are added in LDS in a fixed order; it also
//     emits s*out as bf16 hi/lo parts for the fused GEMM epilogue. P is A
//     (rows contiguous in c) or B read in place (columns contiguous in t),
//     transposed per K-slice through LDS.
//   * colacc: out[c][t] = s sum_m In[m][c] Q[m][t] on float32 FMA, one lane
//     per four columns and 16 t, rows streamed 16 tokens per batch with the
//     next batch in flight, the batch's Q block broadcast from LDS; eight
//     waves per workgroup on disjoint token ranges, reduced in LDS in a fixed
//     order; the token range is split S ways into partial sums that a second
//     kernel adds in a fixed order. dB and dA run as two problems of one
//     launch, and their reductions as one launch.
//   * layout: the zero-padded and transposed copies of A and B the other
//     kernels read (A^T for the dX epilogue, B^T for G), in one launch.
// r is padded to rp (a multiple of 16) with zero rows/columns.
#include <algorithm>

#include "kernels.h"
#include "philox.h"

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
constexpr int SK_W = 16;       // waves per workgroup (column ranges of one token block)
constexpr int SK_UNROLL = 8;   // K-slices of 32 whose loads are issued together

// out[m][t] = sum_c In[m][c] P[t][c] for the SK_TOK tokens of block blockIdx.x and
// t = 16 blockIdx.y + 0..15 (t < r; the rest are zero). P[t][c] is
// Pm[t * C + c] (PCOL = false: A, r x C) or Pm[c * r + t] (PCOL = true: B,
// C x r, r % 16 == 0). Wave w contracts columns [w cpw, (w+1) cpw) on
// MFMA 16x16x32; for PCOL each K-slice's 8 x 16 block of B per lane group
// is transposed through the wave's own LDS slot. The 16 waves' sums are
// added in LDS in a fixed order and written as out (M x rp), out2 (M x r,
// optional) and s*out as bf16 hi + lo parts (optional).
// Up to four contractions of the same In (sibling projections): grid row y
// = weight * (rp / 16) + t-block.
struct SkW {
  const uint16_t *P;
  float *out, *out2;
  uint16_t *hi, *lo;
  DropParams dp;   // dropout of In's elements (row form only)
};
struct SkinnyArgs {
  SkW w[4];
  const uint16_t *In;
  int64_t M, C, cpw;
  int r, rp, tbw, out2_ld;
  float s;
};
template <class T>
QL_DEV T pick4s(int i, T a0, T a1, T a2, T a3) {
  return i == 0 ? a0 : i == 1 ? a1 : i == 2 ? a2 : a3;
}
#define QL_SKPICK(f) pick4s(wi, a.w[0].f, a.w[1].f, a.w[2].f, a.w[3].f)

constexpr int SK_TOK = 8;   // tokens per workgroup (of the 16 MFMA rows)
template <bool PCOL>
__global__ __launch_bounds__(64 * SK_W) void skinny_kernel(SkinnyArgs a) {
  const int wi = (int)blockIdx.y / a.tbw;   // uniform: fields picked by selects
  const uint16_t *__restrict__ In = a.In;
  const uint16_t *__restrict__ Pm = QL_SKPICK(P);
  float *__restrict__ out = QL_SKPICK(out);
  float *__restrict__ out2 = QL_SKPICK(out2);
  uint16_t *__restrict__ hi = QL_SKPICK(hi);
  uint16_t *__restrict__ lo = QL_SKPICK(lo);
  const int64_t M = a.M, C = a.C, cpw = a.cpw;
  const int r = a.r, rp = a.rp, out2_ld = a.out2_ld;
  const float s = a.s;
  DropParams dp;
  dp.k0 = QL_SKPICK(dp.k0);
  dp.k1 = QL_SKPICK(dp.k1);
  dp.thr = QL_SKPICK(dp.thr);
  dp.inv_keep = QL_SKPICK(dp.inv_keep);
  dp.on = !PCOL && QL_SKPICK(dp.on);
  dp.mask_write = QL_SKPICK(dp.mask_write);
  dp.mask = QL_SKPICK(dp.mask);
  constexpr int PQ = 272;   // bytes per lane group in the transposition slot (256 + pad)
  __shared__ f32x4 red[SK_W][64];
  __shared__ __align__(16) unsigned char pst[PCOL ? SK_W : 1][4 * PQ];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, kq = lane >> 4;
  const int64_t mb = blockIdx.x;
  const int t0 = 16 * ((int)blockIdx.y % a.tbw);
  const int64_t m = mb * SK_TOK + r16;
  const bool m_ok = r16 < SK_TOK && m < M;   // MFMA rows past SK_TOK stay zero
  const uint16_t *inr = In + (m_ok ? m : 0) * C + 8 * kq;
  const int64_t c_lo = wave * cpw, c_hi = min(C, c_lo + cpw);
  const bool t_ok = t0 + r16 < r;
  const uint16_t *prow = Pm + (t_ok ? t0 + r16 : 0) * C + 8 * kq;          // !PCOL
  const int rho = (lane >> 1) & 7, hf = lane & 1;                           // PCOL raw piece
  unsigned char *slot = pst[PCOL ? wave : 0];
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int64_t c = c_lo; c < c_hi; c += 32 * SK_UNROLL) {
    uint4 a[SK_UNROLL], b[SK_UNROLL];
#pragma unroll
    for (int u = 0; u < SK_UNROLL; ++u) {
      const int64_t cc = c + 32 * u;
      a[u] = ql::zero4();
      b[u] = ql::zero4();
      if (cc + 8 * kq < c_hi) {   // c_hi % 8 == 0: a chunk is all in or all out
        if (m_ok) a[u] = *(const uint4 *)(inr + cc);
        if (!PCOL && t_ok) b[u] = *(const uint4 *)(prow + cc);
      }
      if (dp.on) {   // dropped elements of X (token m, columns cc + 8kq ..) read as 0
        const uint64_t e = (uint64_t)(m_ok ? m : 0) * (uint64_t)C + (uint64_t)(cc + 8 * kq);
        const uint32_t k8 = keep4(dp, e) | (keep4(dp, e + 4) << 4);
        a[u] = mask_bf16x8(a[u], k8);
        // stored for the backward once (first rank block), by the lanes whose
        // chunk lies in the row
        if (dp.mask_write && dp.mask && t0 == 0 && m_ok && cc + 8 * kq < c_hi)
          *(uint16_t *)(dp.mask + (e >> 2)) = (uint16_t)((k8 & 15u) | ((k8 >> 4) << 8));
      }
      if (PCOL) {
        const int64_t row = cc + 8 * kq + rho;   // B row, t = t0 + 8 hf .. +7
        if (row < c_hi) b[u] = *(const uint4 *)(Pm + row * r + t0 + 8 * hf);
      }
    }
    if (PCOL) {
      // lane (t = r16, kq) needs B rows cc + 8kq .. +7 of column t: write the
      // raw pieces (group kq, row rho, half hf) and read them back by column
#pragma unroll
      for (int u = 0; u < SK_UNROLL; ++u) {
        *(uint4 *)(slot + kq * PQ + rho * 32 + hf * 16) = b[u];
        uint32_t w[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t e0 = *(const uint16_t *)(slot + kq * PQ + (2 * q) * 32 + 2 * r16);
          const uint32_t e1 = *(const uint16_t *)(slot + kq * PQ + (2 * q + 1) * 32 + 2 * r16);
          w[q] = e0 | (e1 << 16);
        }
        b[u] = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
#pragma unroll
    for (int u = 0; u < SK_UNROLL; ++u) acc = ql::mfma16(a[u], b[u], acc);
  }
  // lane holds D[4kq + i][r16] = out[token 4kq+i of the block][t0 + r16]
  red[wave][lane] = acc;
  __syncthreads();
  if (wave != 0) return;
  f32x4 v = red[0][lane];
#pragma unroll
  for (int w = 1; w < SK_W; ++w) {
    const f32x4 x = red[w][lane];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] += x[i];
  }
  const int t = t0 + r16;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t mm = mb * SK_TOK + 4 * kq + i;
    if (4 * kq + i >= SK_TOK || mm >= M) continue;
    if (dp.on) v[i] *= dp.inv_keep;   // inverted dropout: kept elements scaled by 1/(1-p)
    out[mm * rp + t] = v[i];
    if (out2 && t < out2_ld) out2[mm * out2_ld + t] = v[i];
    if (hi) {
      const float sv = s * v[i];
      const uint16_t hb = ql::f_to_bf16(sv);
      hi[mm * rp + t] = hb;
      lo[mm * rp + t] = ql::f_to_bf16(sv - ql::bf16_to_f(hb));
    }
  }
}

// ---- colacc -------------------------------------------------------------------
constexpr int CA_COLS = 256;     // columns per workgroup (four per lane)
constexpr int CA_MAXSPLIT = 16;
constexpr int CA_TOK = 16;       // tokens per batch
constexpr int CA_W = 8;          // waves per workgroup (token ranges)

struct ColaccProb {
  const uint16_t *In;  // M x C
  int64_t C;
  const float *Q;      // M x rp
  float *part;         // S x C x rp
  int64_t groups;      // column groups of CA_COLS
  DropParams dp;       // dropout of In's elements (dp.on == 0: none)
  uint8_t *keep;       // M x C/4 keep nibbles written when dropping (or NULL)
};

// Batch of CA_TOK tokens of one wave: this lane's 4 columns of each token
// row and its float4 of the batch's Q block (token l/4, t = t0 + 4(l%4)..);
// tokens past the wave's range read as zero.
template <bool MK>
struct CaBatch {
  uint2 v[CA_TOK];
  float4 q;
  uint32_t kb[MK ? CA_TOK / 4 : 1];   // stored keep nibbles of the batch's tokens (4 per word)
};

template <bool MK>
QL_DEV void ca_load(CaBatch<MK> &b, const uint16_t *inc, int64_t C, bool c_ok, const float *Q,
                    int rp, int t0, int64_t m, int64_t m_hi, int lane, const uint8_t *mk) {
#pragma unroll
  for (int u = 0; u < CA_TOK; ++u) {
    const int64_t mm = m + u < m_hi ? m + u : m_hi - 1;  // clamped; not accumulated
    b.v[u] = c_ok ? *(const uint2 *)(inc + mm * C) : make_uint2(0u, 0u);
  }
  // with a stored mask, its bytes travel with the batch's loads (mk: the
  // lane's column byte of row 0, or NULL)
#pragma unroll
  for (int j = 0; j < (MK ? CA_TOK / 4 : 1); ++j) b.kb[j] = 0u;
  if (MK && mk) {
#pragma unroll
    for (int u = 0; u < CA_TOK; ++u) {
      const int64_t mm = m + u < m_hi ? m + u : m_hi - 1;
      b.kb[u >> 2] |= (uint32_t)mk[mm * (C >> 2)] << (8 * (u & 3));
    }
  }
  const int64_t mq = m + (lane >> 2);
  b.q = mq < m_hi ? *(const float4 *)(Q + mq * rp + t0 + 4 * (lane & 3))
                  : make_float4(0.f, 0.f, 0.f, 0.f);
}

// Dropout of the batch's first n tokens: their dropped elements become 0,
// and the keep bits (4 per lane and token) are stored for the dX epilogue.
template <bool MK>
QL_DEV void ca_drop(CaBatch<MK> &b, const DropParams &dp, int64_t m, int n, int64_t C, int64_t c0,
                    uint8_t *keep) {
#pragma unroll
  for (int u = 0; u < CA_TOK; ++u) {
    if (u >= n) continue;  // wave-uniform
    // the bits the forward stored (loaded with the batch), or drawn here
    const uint32_t bits = MK ? (b.kb[MK ? u >> 2 : 0] >> (8 * (u & 3))) & 15u
                             : keep4(dp, (uint64_t)(m + u) * (uint64_t)C + (uint64_t)c0);
    b.v[u].x &= ((bits & 1u) ? 0x0000FFFFu : 0u) | ((bits & 2u) ? 0xFFFF0000u : 0u);
    b.v[u].y &= ((bits & 4u) ? 0x0000FFFFu : 0u) | ((bits & 8u) ? 0xFFFF0000u : 0u);
    if (keep) keep[(m + u) * (C >> 2) + (c0 >> 2)] = (uint8_t)bits;
  }
}

// acc[c][t] += x[token][c] * Q[token][t] over the batch's tokens (the first
// n of them when PART)
template <bool PART, bool MK>
QL_DEV void ca_batch(float (&acc)[4][16], const CaBatch<MK> &b, const float4 *qs, int n) {
#pragma unroll
  for (int u = 0; u < CA_TOK; ++u) {
    if (PART && u >= n) continue;  // wave-uniform
    float q[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 f = qs[4 * u + i];   // same address in every lane
      q[4 * i] = f.x; q[4 * i + 1] = f.y; q[4 * i + 2] = f.z; q[4 * i + 3] = f.w;
    }
    const float x[4] = {ql::bf16lo(b.v[u].x), ql::bf16hi(b.v[u].x), ql::bf16lo(b.v[u].y),
                        ql::bf16hi(b.v[u].y)};
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int t = 0; t < 16; ++t) acc[c][t] = fmaf(x[c], q[t], acc[c][t]);
  }
}

// grid: x = column groups of problem 0 then problem 1 (times rp/16 t-blocks),
// y = token split. The eight waves of a workgroup take the same 256 columns
// over disjoint token ranges, each streaming its rows in batches of 16
// tokens with the next batch's loads in flight; the Q block of a batch is
// staged in the wave's own LDS slot and read back as broadcasts. The waves'
// sums are added in LDS in a fixed order.
template <bool MK>
__global__ __launch_bounds__(64 * CA_W) void colacc_kernel(ColaccProb p0, ColaccProb p1,
                                                           int64_t M, int rp, int64_t mps) {
  __shared__ float4 qst[CA_W][64];
  __shared__ float4 red[CA_W][16][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t tbs = rp / 16;
  int64_t gx = blockIdx.x;
  const bool second = gx >= p0.groups * tbs;
  const ColaccProb &P = second ? p1 : p0;
  if (second) gx -= p0.groups * tbs;
  const int64_t cg = gx / tbs, tb = gx % tbs;
  const int64_t c0 = cg * CA_COLS + 4 * lane;
  const int t0 = (int)tb * 16;
  const int64_t split = blockIdx.y;
  const int64_t m_lo = split * mps, m_hi = min(M, m_lo + mps);
  const int64_t span = m_hi - m_lo;
  const int64_t w_lo = m_lo + (span * wave) / CA_W, w_hi = m_lo + (span * (wave + 1)) / CA_W;
  float acc[4][16];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int t = 0; t < 16; ++t) acc[c][t] = 0.0f;
  const bool c_ok = c0 < P.C;  // C % 64 == 0: the 4 columns are all in or all out
  const uint16_t *inc = P.In + (c_ok ? c0 : 0);
  // only the problem that drops (the adapter input) has a mask; the other
  // problem of the launch (dY for dB) reads none
  const uint8_t *mk = (MK && P.dp.on && P.dp.mask && !P.dp.mask_write && c_ok)
                          ? P.dp.mask + (c0 >> 2)
                          : nullptr;
  if (w_lo < w_hi) {
    CaBatch<MK> cur, nxt;
    ca_load(nxt, inc, P.C, c_ok, P.Q, rp, t0, w_lo, w_hi, lane, mk);
    for (int64_t m = w_lo; m < w_hi; m += CA_TOK) {
      cur = nxt;
      if (m + CA_TOK < w_hi)
        ca_load(nxt, inc, P.C, c_ok, P.Q, rp, t0, m + CA_TOK, w_hi, lane, mk);
      qst[wave][lane] = cur.q;   // this wave's previous reads of the slot precede (in order)
      if (P.dp.on && c_ok)
        ca_drop(cur, P.dp, m, (int)min<int64_t>(CA_TOK, w_hi - m), P.C, c0,
                tb == 0 ? P.keep : nullptr);
      if (m + CA_TOK <= w_hi)
        ca_batch<false, MK>(acc, cur, qst[wave], CA_TOK);
      else
        ca_batch<true, MK>(acc, cur, qst[wave], (int)(w_hi - m));
    }
  }
  // the waves' sums in a fixed order: ((wave 0 + 1) + 2) + ... ; thread p of
  // the workgroup finishes float4 entries p and p + 512 of the 64 x 16 grid
#pragma unroll
  for (int i = 0; i < 16; ++i)
    red[wave][i][lane] = make_float4(acc[i >> 2][4 * (i & 3)], acc[i >> 2][4 * (i & 3) + 1],
                                     acc[i >> 2][4 * (i & 3) + 2], acc[i >> 2][4 * (i & 3) + 3]);
  __syncthreads();
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int e = (int)threadIdx.x + 512 * h;
    const int l = e & 63, i = e >> 6;
    float4 o = red[0][i][l];
#pragma unroll
    for (int w = 1; w < CA_W; ++w) {
      const float4 v = red[w][i][l];
      o.x += v.x; o.y += v.y; o.z += v.z; o.w += v.w;
    }
    const int64_t c = cg * CA_COLS + 4 * l + (i >> 2);
    if (c < P.C) *(float4 *)(P.part + (split * P.C + c) * rp + t0 + 4 * (i & 3)) = o;
  }
}

struct ColaccOut {
  const float *part;  // S x C x rp
  int64_t C;
  uint16_t *out;
  int transpose_out;  // 0: out is C x r; 1: out is r x C
  int64_t n;          // C * r
  float scale;        // s, times 1/(1-p) for a dropped input
};

// one thread per output element of problem 0 then problem 1
__global__ __launch_bounds__(256) void colacc_reduce_kernel(ColaccOut o0, ColaccOut o1, int S,
                                                            int rp, int r) {
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
  O.out[idx] = ql::f_to_bf16(O.scale * v);
}

int64_t colacc_split(int64_t M, int64_t C, int rp) {
  // about 256 workgroups of CA_W waves, each wave with at least 16 tokens
  const int64_t wgs = ql_cdiv(C, CA_COLS) * (rp / 16);
  int64_t S = ql_cdiv(256, wgs);
  S = std::min<int64_t>(S, std::max<int64_t>(1, M / (CA_TOK * CA_W)));
  return std::min<int64_t>(std::max<int64_t>(S, 1), CA_MAXSPLIT);
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

qlora_status launch_skinny(const uint16_t *In, int64_t M, int64_t C, int nw, const SkinnyOut *o,
                           bool p_col, int r, int rp, int out2_ld, float s, hipStream_t st) {
  if (nw < 1 || nw > 4) return QLORA_ERR_INVALID_ARG;
  if (p_col && (r % 16 != 0 || r != rp)) return QLORA_ERR_UNSUPPORTED;
  SkinnyArgs a{};
  for (int i = 0; i < 4; ++i) {
    const SkinnyOut &x = o[i < nw ? i : 0];   // unused slots: never selected
    a.w[i] = SkW{x.P, x.out, x.out2, x.hi, x.lo, x.dp};
  }
  a.In = In;
  a.M = M;
  a.C = C;
  a.cpw = ql_rup(ql_cdiv(C, SK_W), 32);
  a.r = r;
  a.rp = rp;
  a.tbw = rp / 16;
  a.out2_ld = out2_ld;
  a.s = s;
  const int64_t mbs = ql_cdiv(M, SK_TOK);
  if (mbs > 0x7fffffff || (int64_t)nw * a.tbw > 65535) return QLORA_ERR_UNSUPPORTED;
  dim3 grid((unsigned)mbs, (unsigned)(nw * a.tbw));
  QlProf prof(QLORA_K_LORA_DOWN, st);
  if (p_col)
    skinny_kernel<true><<<grid, 64 * SK_W, 0, st>>>(a);
  else
    skinny_kernel<false><<<grid, 64 * SK_W, 0, st>>>(a);
  QL_LAUNCH_CHECK();
  return QLORA_OK;
}

qlora_status launch_skinny(const uint16_t *In, int64_t M, int64_t C, const uint16_t *P,
                           bool p_col, int r, int rp, float *out, float *out2, int out2_ld,
                           float s, uint16_t *hi, uint16_t *lo, hipStream_t st) {
  const SkinnyOut o{P, out, out2, hi, lo, DropParams{0u, 0u, 0u, 1.0f, 0}};
  return launch_skinny(In, M, C, 1, &o, p_col, r, rp, out2_ld, s, st);
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
  ColaccProb p0{a.In, a.C, a.Q, part, ql_cdiv(a.C, CA_COLS), a.dp, a.keep};
  ColaccProb p1{b.In, b.C, b.Q, part + S * a.C * rp, ql_cdiv(b.C, CA_COLS), b.dp, b.keep};
  const int64_t tbs = rp / 16;
  dim3 grid((unsigned)((p0.groups + p1.groups) * tbs), (unsigned)S);
  {
    QlProf prof(QLORA_K_LORA_COLACC, st);
    // MK: the adapter input's keep bits come from the mask the forward stored
    if (p1.dp.on && p1.dp.mask && !p1.dp.mask_write)
      colacc_kernel<true><<<grid, 64 * CA_W, 0, st>>>(p0, p1, M, rp, mps);
    else
      colacc_kernel<false><<<grid, 64 * CA_W, 0, st>>>(p0, p1, M, rp, mps);
  }
  ColaccOut o0{p0.part, a.C, a.out, a.transpose_out, a.C * r, a.dp.on ? s * a.dp.inv_keep : s};
  ColaccOut o1{p1.part, b.C, b.out, b.transpose_out, b.C * r, b.dp.on ? s * b.dp.inv_keep : s};
  QlProf prof(QLORA_K_LORA_COLACC_REDUCE, st);
  colacc_reduce_kernel<<<(unsigned)ql_cdiv(o0.n + o1.n, 256), 256, 0, st>>>(o0, o1, (int)S, rp,
                                                                           r);
  QL_LAUNCH_CHECK();
  return QLORA_OK;
}
