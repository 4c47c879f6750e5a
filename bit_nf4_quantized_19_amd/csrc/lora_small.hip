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
//     (rows contiguous in c, loaded as 64-byte row segments) or B read in
//     place (columns contiguous in t); either is re-laid out into the MFMA
//     operand order per K-slice through the wave's LDS slot.
//   * colacc: out[c][t] = s sum_m In[m][c] Q[m][t] on MFMA 16x16x32 with the
//     tokens as the contraction (Q as bf16 hi + lo parts); a workgroup owns 64
//     columns and one of S token ranges, streams token chunks through LDS with
//     the next chunks' loads in flight, and writes its partial sums; the last
//     workgroup of a column block to finish adds the S partials in split
//     order and rounds them. dB and dA run as two problems of one launch.
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
  int *zero;        // counters a later launch of the same call needs zeroed (or NULL)
  int64_t nzero;
};
template <class T>
QL_DEV T pick4s(int i, T a0, T a1, T a2, T a3) {
  return i == 0 ? a0 : i == 1 ? a1 : i == 2 ? a2 : a3;
}
#define QL_SKPICK(f) pick4s(wi, a.w[0].f, a.w[1].f, a.w[2].f, a.w[3].f)

constexpr int SK_TOK = 8;   // tokens per workgroup (of the 16 MFMA rows)
template <bool PCOL>
__global__ __launch_bounds__(64 * SK_W) void skinny_kernel(SkinnyArgs a) {
  if (a.zero && blockIdx.x == 0 && blockIdx.y == 0)
    for (int64_t i = threadIdx.x; i < a.nzero; i += 64 * SK_W) a.zero[i] = 0;
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
  // per-wave slot for re-laying out the P pieces of one K-slice: B's raw
  // pieces (PCOL) or A's 16 rows of 64 bytes at a stride of 80 (!PCOL)
  constexpr int AST = 80;
  __shared__ __align__(16) unsigned char pst[SK_W][PCOL ? 4 * PQ : 16 * AST];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, kq = lane >> 4;
  const int64_t mb = blockIdx.x;
  const int t0 = 16 * ((int)blockIdx.y % a.tbw);
  const int64_t m = mb * SK_TOK + r16;
  const bool m_ok = r16 < SK_TOK && m < M;   // MFMA rows past SK_TOK stay zero
  const uint16_t *inr = In + (m_ok ? m : 0) * C + 8 * kq;
  const int64_t c_lo = wave * cpw, c_hi = min(C, c_lo + cpw);
  // !PCOL: A rows are loaded whole (lane -> row ra = lane / 4, 16-byte piece
  // pa = lane % 4 of the slice's 64 bytes, so a quarter-wave reads 4 rows of
  // 64 contiguous bytes) and re-laid out through the slot; rows past r read 0
  const int ra = lane >> 2, pa = lane & 3;
  const bool ta_ok = t0 + ra < r;
  const uint16_t *prow = Pm + (ta_ok ? t0 + ra : 0) * C + 8 * pa;           // !PCOL
  const int rho = (lane >> 1) & 7, hf = lane & 1;                           // PCOL raw piece
  unsigned char *slot = pst[wave];
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
      }
      if (!PCOL && ta_ok && cc + 8 * pa < c_hi) b[u] = *(const uint4 *)(prow + cc);
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
    if (!PCOL) {
      // lane (t = r16, kq) needs A[t][cc + 8kq .. +7]: row ra's piece pa in,
      // row r16's piece kq out
#pragma unroll
      for (int u = 0; u < SK_UNROLL; ++u) {
        *(uint4 *)(slot + ra * AST + pa * 16) = b[u];
        b[u] = *(const uint4 *)(slot + r16 * AST + kq * 16);
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
  // all the waves' partials read first (one LDS latency), then added in wave order
  f32x4 x[SK_W];
#pragma unroll
  for (int w = 0; w < SK_W; ++w) x[w] = red[w][lane];
  __builtin_amdgcn_sched_barrier(0);
  f32x4 v = x[0];
#pragma unroll
  for (int w = 1; w < SK_W; ++w)
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] += x[w][i];
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
// out^T[t][c] = sum_m Q[m][t] In[m][c] on MFMA 16x16x32 with the tokens as
// the contraction: A = Q^T (rows t, 8 consecutive tokens per lane), B = In
// (8 consecutive tokens of one column per lane). In is token-major, so each
// 32-token x 64-column chunk is staged in LDS row by row (16 coalesced bytes
// per thread) and read back down the columns; Q is staged transposed and
// split into bf16 hi + lo parts (two MFMAs per chunk, ~16 significant bits).
// A workgroup (four waves, one 16-column tile each) owns 64 columns of one
// problem, every rank block of them, and one of S token ranges; its partial
// sums go to part[split][c][t]. The last workgroup of a column block to
// finish (a counter per block, zero at launch) adds the S partials in split
// order, scales and rounds them: dB and dA with one launch and no second
// pass.
constexpr int CM_COLS = 64;      // columns per workgroup
constexpr int CM_MAXSPLIT = 16;
constexpr int CM_MAXRP = 128;
constexpr int CM_INS = CM_COLS / 2 + 1;   // dwords per staged In row (one pad dword)
// A chunk is KS MFMA contraction steps of 32 tokens; a staged Q^T row holds
// the chunk's 32 KS tokens plus a 16-byte pad.
template <int KS> constexpr int cm_qs() { return 32 * KS + 8; }

struct ColaccProb {
  const uint16_t *In;  // M x C
  int64_t C;
  const float *Q;      // M x rp
  float *part;         // S x C x rp
  int64_t blocks;      // column blocks of CM_COLS
  uint16_t *out;
  int transpose_out;   // 0: out is C x r (ld r); 1: out is r x C (ld C)
  float scale;         // s, times 1/(1-p) for a dropped input
  DropParams dp;       // dropout of In's elements (dp.on == 0: none)
  uint8_t *keep;       // M x C/4 keep nibbles written when drawing them (or NULL)
};

// Chunk staged through registers: this thread's 8 columns of one token row
// (and their keep bits) and up to four float4 of the chunk's Q block.
template <int RPM, int KS>
struct CmRegs {
  uint4 x[KS];
  float4 q[RPM * KS / 32 > 0 ? RPM * KS / 32 : 1];
};

// Rows at or past M (here: the end of this workgroup's token range) read as 0.
template <bool MK, int RPM, int KS>
QL_DEV void cm_load(CmRegs<RPM, KS> &R, const ColaccProb &P, int64_t M, int rp, int64_t m0, int64_t c0,
                    int tid) {
#pragma unroll
  for (int j = 0; j < KS; ++j) {
    const int64_t m = m0 + 32 * j + (tid >> 3), c = c0 + 8 * (tid & 7);
    const bool ok = m < M && c < P.C;   // C % 8 == 0: the 8 columns are all in or all out
    R.x[j] = ok ? *(const uint4 *)(P.In + m * P.C + c) : ql::zero4();
    if (P.dp.on && ok) {
      const uint64_t e = (uint64_t)m * (uint64_t)P.C + (uint64_t)c;
      uint32_t k8;
      if (MK && P.dp.mask && !P.dp.mask_write) {
        const uint32_t b2 = *(const uint16_t *)(P.dp.mask + (e >> 2));   // the forward's bits
        k8 = (b2 & 15u) | (((b2 >> 8) & 15u) << 4);
      } else {
        k8 = keep4(P.dp, e) | (keep4(P.dp, e + 4) << 4);
        if (P.keep) *(uint16_t *)(P.keep + (e >> 2)) = (uint16_t)((k8 & 15u) | ((k8 >> 4) << 8));
      }
      R.x[j] = mask_bf16x8(R.x[j], k8);
    }
  }
  const int nq = 8 * KS * rp;   // float4 in the chunk's Q block
#pragma unroll
  for (int u = 0; u < (RPM * KS + 31) / 32; ++u) {
    const int f = tid + 256 * u;
    if (f >= nq) break;
    const int64_t mq = m0 + f / (rp / 4);
    R.q[u] = mq < M ? *(const float4 *)(P.Q + mq * rp + 4 * (f % (rp / 4)))
                    : make_float4(0.f, 0.f, 0.f, 0.f);
  }
}

template <int RPM, int KS>
QL_DEV void cm_store(const CmRegs<RPM, KS> &R, uint32_t *sin, uint16_t *sqh, uint16_t *sql, int rp,
                     int tid) {
#pragma unroll
  for (int j = 0; j < KS; ++j) {
    uint32_t *row = sin + (32 * j + (tid >> 3)) * CM_INS + 4 * (tid & 7);
    row[0] = R.x[j].x; row[1] = R.x[j].y; row[2] = R.x[j].z; row[3] = R.x[j].w;
  }
  const int nq = 8 * KS * rp;
#pragma unroll
  for (int u = 0; u < (RPM * KS + 31) / 32; ++u) {
    const int f = tid + 256 * u;
    if (f >= nq) break;
    const int tok = f / (rp / 4), t = 4 * (f % (rp / 4));
    const float v[4] = {R.q[u].x, R.q[u].y, R.q[u].z, R.q[u].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint16_t hb = ql::f_to_bf16(v[i]);
      sqh[(t + i) * cm_qs<KS>() + tok] = hb;
      sql[(t + i) * cm_qs<KS>() + tok] = ql::f_to_bf16(v[i] - ql::bf16_to_f(hb));
    }
  }
}

// One chunk from LDS buffer `buf`: B = tokens 8g .. 8g+7 of column
// 16 wave + cl, A = Q^T hi and lo of each rank block.
template <int RPM, int KS>
QL_DEV void cm_compute(f32x4 (&acc)[RPM / 16], const uint32_t *sin, const uint16_t *sqh,
                       const uint16_t *sql, int tbs, int wave, int cl, int g) {
  const unsigned char *colp = (const unsigned char *)sin + 2 * (16 * wave + cl);
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    uint32_t h[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      h[i] = *(const uint16_t *)(colp + (32 * ks + 8 * g + i) * CM_INS * 4);
    const uint4 bop = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                                 h[6] | (h[7] << 16));
#pragma unroll
    for (int b = 0; b < RPM / 16; ++b) {
      if (b >= tbs) break;
      const int qo = (16 * b + cl) * cm_qs<KS>() + 32 * ks + 8 * g;
      const uint4 ah = *(const uint4 *)&sqh[qo];
      const uint4 al = *(const uint4 *)&sql[qo];
      acc[b] = ql::mfma16(ah, bop, acc[b]);
      acc[b] = ql::mfma16(al, bop, acc[b]);
    }
  }
}

// Chunks in flight per thread, and the target workgroup count from which
// the token split S is derived. Measured at 4096x4096, 2048 tokens, r = 16
// (dA + dB launch, us): target 256 / 512 / 640 / 768 / 896 / 1024 ->
// 18.8 / 16.4 / 15.9 / 15.7 / 15.6 / 17.5; three chunks in flight no better.
#ifndef QL_CM_PF
#define QL_CM_PF 2
#endif
#ifndef QL_CM_WGS
#define QL_CM_WGS 768
#endif
constexpr int CM_PF = QL_CM_PF;   // chunks whose loads are in flight per thread

// Dynamic LDS: two buffers of the In chunk (32 KS x CM_INS dwords) and of
// Q^T hi and lo (rp x cm_qs bf16 each).
template <int KS>
size_t cm_lds_bytes(int rp) {
  return 2 * 32 * KS * CM_INS * 4 + 2 * 2 * (size_t)rp * cm_qs<KS>() * 2;
}

// RPM: the largest padded rank this instance handles (32, 64 or 128), which
// sizes its registers.
template <bool MK, int RPM, int KS>
__global__ __launch_bounds__(256) void colacc_kernel(ColaccProb p0, ColaccProb p1, int64_t M,
                                                     int rp, int r, int64_t mps, int S,
                                                     int *cnt) {
  extern __shared__ __align__(16) unsigned char cm_lds[];
  constexpr int TOK = 32 * KS, QS = cm_qs<KS>();
  uint32_t *s_in0 = (uint32_t *)cm_lds, *s_in1 = s_in0 + TOK * CM_INS;
  uint16_t *s_q = (uint16_t *)(s_in1 + TOK * CM_INS);
  uint16_t *s_qh0 = s_q, *s_ql0 = s_q + rp * QS, *s_qh1 = s_q + 2 * rp * QS,
           *s_ql1 = s_q + 3 * rp * QS;
  __shared__ int s_last;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cl = lane & 15, g = lane >> 4;
  int64_t bx = blockIdx.x;
  const bool second = bx >= p0.blocks;
  const ColaccProb &P = second ? p1 : p0;
  if (second) bx -= p0.blocks;
  const int64_t c0 = bx * CM_COLS;
  const int split = blockIdx.y;
  const int64_t m_lo = split * mps, m_hi = min(M, m_lo + mps);
  const int tbs = rp / 16;
  f32x4 acc[RPM / 16];
#pragma unroll
  for (int b = 0; b < RPM / 16; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[b][i] = 0.0f;
  const int nch = (int)ql_cdiv(m_hi - m_lo, TOK);
  // a ring of CM_PF register sets, the loop unrolled by CM_PF so every set is
  // named at compile time: chunk ch + CM_PF - 1 is loaded while chunk ch is
  // stored to LDS and computed
  CmRegs<RPM, KS> R[CM_PF];
#pragma unroll
  for (int i = 0; i < CM_PF - 1; ++i)
    if (i < nch) cm_load<MK, RPM, KS>(R[i], P, m_hi, rp, m_lo + (int64_t)i * TOK, c0, tid);
  for (int ch0 = 0; ch0 < nch; ch0 += CM_PF) {
#pragma unroll
    for (int u = 0; u < CM_PF; ++u) {
      const int ch = ch0 + u;
      if (ch >= nch) break;
      if (ch + CM_PF - 1 < nch)
        cm_load<MK, RPM, KS>(R[(u + CM_PF - 1) % CM_PF], P, m_hi, rp,
                             m_lo + (int64_t)(ch + CM_PF - 1) * TOK, c0, tid);
      uint32_t *sin = (u & 1) ? s_in1 : s_in0;
      uint16_t *sqh = (u & 1) ? s_qh1 : s_qh0, *sql = (u & 1) ? s_ql1 : s_ql0;
      cm_store<RPM, KS>(R[u], sin, sqh, sql, rp, tid);
      __syncthreads();
      cm_compute<RPM, KS>(acc, sin, sqh, sql, tbs, wave, cl, g);
    }
  }
  // lane holds out^T[16 b + 4 g + i][c0 + 16 wave + cl]. The partials are
  // published with agent-scope stores (written through to the level every
  // XCD sees), so no L2 write-back or invalidation is needed: the barrier
  // below waits for this workgroup's stores to complete before the counter
  // moves, and the last workgroup reads them back with agent-scope loads.
  const int64_t c = c0 + 16 * wave + cl;
  if (c < P.C) {
#pragma unroll
    for (int b = 0; b < RPM / 16; ++b) {
      if (b >= tbs) break;
      // four consecutive ranks: two 8-byte stores (the offset is a multiple of 16 bytes)
      uint64_t *dst = (uint64_t *)(P.part + ((int64_t)split * P.C + c) * rp + 16 * b + 4 * g);
      const uint64_t w0 = (uint64_t)__float_as_uint(acc[b][0]) |
                          ((uint64_t)__float_as_uint(acc[b][1]) << 32);
      const uint64_t w1 = (uint64_t)__float_as_uint(acc[b][2]) |
                          ((uint64_t)__float_as_uint(acc[b][3]) << 32);
      __hip_atomic_store(dst, w0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(dst + 1, w1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  // the last workgroup of this column block adds the S partials in order
  int *ctr = cnt + (second ? p0.blocks : 0) + bx;
  __builtin_amdgcn_s_waitcnt(0);   // this thread's stores have completed
  __syncthreads();
  if (tid == 0)
    s_last = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == S - 1;
  __syncthreads();
  if (!s_last) return;
  // thread (col = tid / 4, q = tid % 4) adds ranks 16 b + 4 q .. +3 of column
  // c0 + col over the S splits in split order; each split's four values are
  // two 8-byte agent-scope loads from a clamped (always valid) split, four
  // splits' loads in flight before their sums
  {
    const int col = tid >> 2, q4 = tid & 3;
    const int64_t cc = c0 + col;
    const bool cok = cc < P.C;
    const int64_t ccl = cok ? cc : c0;
    for (int b = 0; b < tbs; ++b) {
      float v[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      for (int s0 = 0; s0 < S; s0 += 4) {
        // addresses first (all live at once), then the eight loads back to back
        const uint64_t *src[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int sp = s0 + u < S ? s0 + u : s0;
          src[u] = (const uint64_t *)(P.part + ((int64_t)sp * P.C + ccl) * rp + 16 * b + 4 * q4);
        }
        __builtin_amdgcn_sched_barrier(0);
        uint64_t w[4][2];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          w[u][0] = __hip_atomic_load(src[u], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          w[u][1] = __hip_atomic_load(src[u] + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (s0 + u >= S) break;
          v[0] += __uint_as_float((uint32_t)w[u][0]);
          v[1] += __uint_as_float((uint32_t)(w[u][0] >> 32));
          v[2] += __uint_as_float((uint32_t)w[u][1]);
          v[3] += __uint_as_float((uint32_t)(w[u][1] >> 32));
        }
      }
      // all four results first, then the stores (one 8-byte store when the
      // four ranks are consecutive and aligned in out)
      uint32_t ob[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) ob[i] = ql::f_to_bf16(P.scale * v[i]);
      const int t4 = 16 * b + 4 * q4;
      if (cok && !P.transpose_out && (r & 3) == 0 && t4 < r) {
        *(uint2 *)(P.out + cc * r + t4) = make_uint2(ob[0] | (ob[1] << 16), ob[2] | (ob[3] << 16));
      } else if (cok) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (t4 + i < r)
            P.out[P.transpose_out ? (int64_t)(t4 + i) * P.C + cc : cc * r + t4 + i] = (uint16_t)ob[i];
      }
    }
  }
  if (tid == 0)   // left clear for the next call on this workspace
    __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

int64_t colacc_split(int64_t M, int64_t C0, int64_t C1) {
  // about three workgroups per compute unit, each split at least one chunk
  const int64_t blocks = ql_cdiv(C0, CM_COLS) + ql_cdiv(C1, CM_COLS);
  int64_t S = ql_cdiv(QL_CM_WGS, blocks);
  S = std::min<int64_t>(S, ql_cdiv(M, 128));
  return std::min<int64_t>(std::max<int64_t>(S, 1), CM_MAXSPLIT);
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
                           bool p_col, int r, int rp, int out2_ld, float s, hipStream_t st,
                           int *zero, int64_t nzero) {
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
  a.zero = zero;
  a.nzero = nzero;
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
                           float s, uint16_t *hi, uint16_t *lo, hipStream_t st, int *zero,
                           int64_t nzero) {
  const SkinnyOut o{P, out, out2, hi, lo, DropParams{0u, 0u, 0u, 1.0f, 0}};
  return launch_skinny(In, M, C, 1, &o, p_col, r, rp, out2_ld, s, st, zero, nzero);
}

size_t colacc_part_bytes(int64_t M, int64_t C0, int64_t C1, int rp) {
  const int64_t S = colacc_split(M, C0, C1);
  return (size_t)ql_rup(S * (C0 + C1) * rp * 4, 256) + colacc_counter_count(C0, C1) * 4;
}

int64_t colacc_counter_count(int64_t C0, int64_t C1) {
  return ql_cdiv(C0, CM_COLS) + ql_cdiv(C1, CM_COLS);
}

int *colacc_counters(float *part, int64_t M, int64_t C0, int64_t C1, int rp) {
  const int64_t S = colacc_split(M, C0, C1);
  return (int *)((char *)part + ql_rup(S * (C0 + C1) * rp * 4, 256));
}

qlora_status launch_colacc2(const ColaccReq &a, const ColaccReq &b, int64_t M, int rp, int r,
                            float s, float *part, hipStream_t st) {
  if (rp % 16 || rp > CM_MAXRP) return QLORA_ERR_UNSUPPORTED;
  const int64_t S0 = colacc_split(M, a.C, b.C);
  const int64_t mps = ql_rup(ql_cdiv(M, S0), 128);   // a multiple of every chunk size
  const int64_t S = ql_cdiv(M, mps);
  const int64_t pbytes = ql_rup(S0 * (a.C + b.C) * rp * 4, 256);
  int *cnt = (int *)((char *)part + pbytes);   // zeroed by the launch before (launch_skinny)
  ColaccProb p0{a.In, a.C, a.Q, part, ql_cdiv(a.C, CM_COLS), a.out, a.transpose_out,
                a.dp.on ? s * a.dp.inv_keep : s, a.dp, a.keep};
  ColaccProb p1{b.In, b.C, b.Q, part + S * a.C * rp, ql_cdiv(b.C, CM_COLS), b.out,
                b.transpose_out, b.dp.on ? s * b.dp.inv_keep : s, b.dp, b.keep};
  dim3 grid((unsigned)(p0.blocks + p1.blocks), (unsigned)S);
  QlProf prof(QLORA_K_LORA_COLACC, st);
  // MK: the adapter input's keep bits come from the mask the forward stored
  const bool mk = p1.dp.on && p1.dp.mask && !p1.dp.mask_write;
  // chunk depth per rank bound: the LDS of two chunks stays within 64 KB
#define QL_CM(RPV, KSV)                                                                   \
  {                                                                                       \
    const size_t lds = cm_lds_bytes<KSV>(rp);                                             \
    if (mk)                                                                               \
      colacc_kernel<true, RPV, KSV><<<grid, 256, lds, st>>>(p0, p1, M, rp, r, mps, (int)S, cnt); \
    else                                                                                  \
      colacc_kernel<false, RPV, KSV><<<grid, 256, lds, st>>>(p0, p1, M, rp, r, mps, (int)S, cnt); \
  }
  if (rp <= 16) QL_CM(16, 4)
  else if (rp <= 32) QL_CM(32, 2)
  else if (rp <= 64) QL_CM(64, 2)
  else QL_CM(128, 1)
#undef QL_CM
  QL_LAUNCH_CHECK();
  return QLORA_OK;
}
