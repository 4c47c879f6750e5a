// Fused NF4 dequant-GEMM with the LoRA rank-r epilogue, gfx950 MFMA.
//
// Forward (QLoRA glossary, Ultralytics, "QLoRA 的工作原理", forward paragraph;
// Day-25 notes 2.1 and 6.2):      Y  = X W'^T + (s H) B^T
// Input gradient (chain rule of the same; only A and B are trained):
//                                 dX = dY W' + (s G) A
// W' = bf16(level[code] * a') is decoded on the fly from the packed codes;
// it is never materialised in HBM.
//
// One kernel computes Out[m][n] = sum_K Wop[n][K] In[m][K] + sum_t L[n][t] S[m][t]
// as the transposed product Out^T = Wop In^T on MFMA, so each lane ends with
// 4 consecutive n of one token row (8-byte stores):
//   forward: n = output feature (d), K = k, Wop = W' rows,  In = X,  L = B,   S = sH
//   dX:      n = input feature (k),  K = d, Wop = W' cols,  In = dY, L = A^T, S = sG
// S is passed as bf16 hi + lo parts (two K-chunks) so the rank-r term keeps
// ~16 significant bits.
//
// Tiling: workgroup tile 128 (n) x 256 (m), K-step 64 = one NF4 block per W'
// row (forward) or per 8-row column strip (dX). 4 waves in a 2 x 2 grid, each
// 64 x 128 with v_mfma_f32_32x32x16_bf16 (8 accumulator tiles). W' and In
// tiles are double-buffered in LDS (96 KB) with an XOR swizzle of the 16-byte
// chunks (chunk ^ row%8) so the MFMA operand reads are bank-conflict free.
// The next step's global loads are issued before this step's MFMAs and its
// codes are decoded after them, so VALU decode overlaps the matrix cores.
// Workgroups are mapped XCD-aware: consecutive tiles of one token block land
// on the same XCD (its L2 then holds that X/dY block).
#include "kernels.h"
#include "nf4_tables.h"

namespace {

constexpr int BN = 128, BM = 256, BK = 64, NT = 256;
__constant__ uint32_t c_levels_g[16] = NF4_LEVEL_BITS;

struct GemmArgs {
  const uint8_t *codes;
  ql::ScaleSrc sc;
  int64_t d, k;          // weight shape
  const uint16_t *In;    // M x Ktot
  int64_t M;
  int64_t Ntot, Ktot;    // output columns, contraction length
  const uint16_t *L;     // Ntot x rp
  const uint16_t *Shi, *Slo;  // M x rp
  int rp;
  uint16_t *Out;         // M x Ntot
};

QL_DEV int swz(int row, int chunk) { return row * 8 + (chunk ^ (row & 7)); }

template <int MODE>
struct Stage {
  uint4 x[8];
  // MODE 0: one 16-byte code chunk + one block scale
  // MODE 1: eight 2-byte code pieces (8 rows) + eight block scales
  uint4 c0;
  uint32_t c1[8];
  float ap[8];
};

template <int MODE>
QL_DEV void stage_load(const GemmArgs &g, Stage<MODE> &st, int64_t m0, int64_t n0,
                       int64_t kk, float mu, int tid) {
  // In tile: 256 rows x 64 (8 chunks of 8 bf16)
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int ci = tid + NT * i;
    const int row = ci >> 3, c = ci & 7;
    const int64_t m = m0 + row;
    const int64_t kc = kk + 8 * c;
    if (m < g.M && kc < g.Ktot)
      st.x[i] = *(const uint4 *)(g.In + m * g.Ktot + kc);
    else
      st.x[i] = ql::zero4();
  }
  if (MODE == 0) {
    const int n = tid >> 1, half = tid & 1;
    const int64_t row = n0 + n;
    if (row < g.d) {
      const int64_t e0 = row * g.k + kk + 32 * half;  // first element
      st.c0 = *(const uint4 *)(g.codes + (e0 >> 1));
      st.ap[0] = ql::block_scale(g.sc, e0 >> 6, mu);
    } else {
      st.c0 = ql::zero4();
      st.ap[0] = 0.0f;
    }
  } else {
    const int jg = tid & 7, kg = tid >> 3;
    const int64_t col = n0 + 4 * kg;  // input-feature column (k index)
#pragma unroll
    for (int rr = 0; rr < 8; ++rr) {
      const int64_t row = kk + 8 * jg + rr;  // output-feature row (d index)
      if (row < g.d && col < g.k) {
        const int64_t e0 = row * g.k + col;
        st.c1[rr] = *(const uint16_t *)(g.codes + (e0 >> 1));
        st.ap[rr] = ql::block_scale(g.sc, e0 >> 6, mu);
      } else {
        st.c1[rr] = 0u;
        st.ap[rr] = 0.0f;
      }
    }
  }
}

template <int MODE>
QL_DEV void stage_commit(const Stage<MODE> &st, uint4 *Wl, uint4 *Xl, const float *lv,
                         int tid) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int ci = tid + NT * i;
    Xl[swz(ci >> 3, ci & 7)] = st.x[i];
  }
  if (MODE == 0) {
    const int n = tid >> 1, half = tid & 1;
    const uint32_t w4[4] = {st.c0.x, st.c0.y, st.c0.z, st.c0.w};
    const float a = st.ap[0];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t c = w4[i];  // 8 codes: bytes b0..b3, high nibble first
      uint4 o;
      o.x = ql::pack_bf16x2(lv[(c >> 4) & 15] * a, lv[c & 15] * a);
      o.y = ql::pack_bf16x2(lv[(c >> 12) & 15] * a, lv[(c >> 8) & 15] * a);
      o.z = ql::pack_bf16x2(lv[(c >> 20) & 15] * a, lv[(c >> 16) & 15] * a);
      o.w = ql::pack_bf16x2(lv[(c >> 28) & 15] * a, lv[(c >> 24) & 15] * a);
      Wl[swz(n, 4 * half + i)] = o;
    }
  } else {
    const int jg = tid & 7, kg = tid >> 3;
    float f[8][4];
#pragma unroll
    for (int rr = 0; rr < 8; ++rr) {
      const uint32_t c = st.c1[rr];  // bytes: (e0,e1), (e2,e3)
      const float a = st.ap[rr];
      f[rr][0] = lv[(c >> 4) & 15] * a;
      f[rr][1] = lv[c & 15] * a;
      f[rr][2] = lv[(c >> 12) & 15] * a;
      f[rr][3] = lv[(c >> 8) & 15] * a;
    }
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      uint4 o;
      o.x = ql::pack_bf16x2(f[0][cc], f[1][cc]);
      o.y = ql::pack_bf16x2(f[2][cc], f[3][cc]);
      o.z = ql::pack_bf16x2(f[4][cc], f[5][cc]);
      o.w = ql::pack_bf16x2(f[6][cc], f[7][cc]);
      Wl[swz(4 * kg + cc, jg)] = o;
    }
  }
}

template <int MODE>
__global__ __launch_bounds__(NT, 1) void nf4_gemm_kernel(GemmArgs g) {
  __shared__ uint4 Wl[2][BN * 8];
  __shared__ uint4 Xl[2][BM * 8];
  __shared__ float lv[16];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = wave & 1, wm = wave >> 1;
  if (tid < 16) lv[tid] = __uint_as_float(c_levels_g[tid]);

  // XCD-aware tile order
  const int64_t ntn = ql_cdiv(g.Ntot, BN), ntm = ql_cdiv(g.M, BM);
  const int64_t total = ntn * ntm;
  int64_t tile = blockIdx.x;
  if ((total & 7) == 0) tile = (int64_t)(blockIdx.x & 7) * (total >> 3) + (blockIdx.x >> 3);
  const int64_t tm = tile / ntn, tn = tile % ntn;
  const int64_t m0 = tm * BM, n0 = tn * BN;
  const float mu = g.sc.dq ? g.sc.mu[0] : 0.0f;
  __syncthreads();

  f32x16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  const int64_t nk = ql_cdiv(g.Ktot, BK);
  Stage<MODE> st;
  stage_load<MODE>(g, st, m0, n0, 0, mu, tid);
  stage_commit<MODE>(st, Wl[0], Xl[0], lv, tid);
  __syncthreads();

  const int r32 = lane & 31, hk = lane >> 5;
  for (int64_t s = 0; s < nk; ++s) {
    const int buf = (int)(s & 1);
    const bool more = (s + 1) < nk;
    if (more) stage_load<MODE>(g, st, m0, n0, (s + 1) * BK, mu, tid);
    const uint4 *W = Wl[buf];
    const uint4 *Xs = Xl[buf];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int chunk = 2 * ks + hk;
      uint4 a[2], b[4];
#pragma unroll
      for (int i = 0; i < 2; ++i) a[i] = W[swz(wn * 64 + 32 * i + r32, chunk)];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Xs[swz(wm * 128 + 32 * j + r32, chunk)];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = ql::mfma32(a[i], b[j], acc[i][j]);
    }
    if (more) stage_commit<MODE>(st, Wl[buf ^ 1], Xl[buf ^ 1], lv, tid);
    __syncthreads();
  }

  // LoRA rank-r term: two extra K-chunks per 16 of rp (hi and lo parts of S)
  for (int t0 = 0; t0 < g.rp; t0 += 16) {
#pragma unroll
    for (int part = 0; part < 2; ++part) {
      const uint16_t *S = part ? g.Slo : g.Shi;
      uint4 a[2], b[4];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int64_t n = n0 + wn * 64 + 32 * i + r32;
        a[i] = (n < g.Ntot) ? *(const uint4 *)(g.L + n * g.rp + t0 + 8 * hk) : ql::zero4();
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t m = m0 + wm * 128 + 32 * j + r32;
        b[j] = (m < g.M) ? *(const uint4 *)(S + m * g.rp + t0 + 8 * hk) : ql::zero4();
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = ql::mfma32(a[i], b[j], acc[i][j]);
    }
  }

  // store: lane holds D[8(e/4) + 4(l/32) + e%4][l%32] = Out[m][n]
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t m = m0 + wm * 128 + 32 * j + r32;
      if (m >= g.M) continue;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int64_t n = n0 + wn * 64 + 32 * i + 8 * q4 + 4 * hk;
        if (n >= g.Ntot) continue;
        uint2 o;
        o.x = ql::pack_bf16x2(acc[i][j][4 * q4 + 0], acc[i][j][4 * q4 + 1]);
        o.y = ql::pack_bf16x2(acc[i][j][4 * q4 + 2], acc[i][j][4 * q4 + 3]);
        *(uint2 *)(g.Out + m * g.Ntot + n) = o;
      }
    }
}

}  // namespace

static qlora_status launch_gemm(int mode, GemmArgs g, hipStream_t st) {
  const int64_t tiles = ql_cdiv(g.Ntot, BN) * ql_cdiv(g.M, BM);
  QlProf prof(mode == 0 ? QLORA_K_GEMM_FWD : QLORA_K_GEMM_DX, st);
  if (mode == 0)
    nf4_gemm_kernel<0><<<(unsigned)tiles, NT, 0, st>>>(g);
  else
    nf4_gemm_kernel<1><<<(unsigned)tiles, NT, 0, st>>>(g);
  QL_LAUNCH_CHECK();
  return QLORA_OK;
}

qlora_status launch_gemm_fwd(const uint8_t *codes, ql::ScaleSrc sc, int64_t d, int64_t k,
                             const uint16_t *X, int64_t M, const uint16_t *Bp,
                             const uint16_t *Hs_hi, const uint16_t *Hs_lo, int rp,
                             uint16_t *Y, hipStream_t st) {
  GemmArgs g{codes, sc, d, k, X, M, d, k, Bp, Hs_hi, Hs_lo, rp, Y};
  return launch_gemm(0, g, st);
}

qlora_status launch_gemm_dx(const uint8_t *codes, ql::ScaleSrc sc, int64_t d, int64_t k,
                            const uint16_t *dY, int64_t M, const uint16_t *At,
                            const uint16_t *Gs_hi, const uint16_t *Gs_lo, int rp,
                            uint16_t *dX, hipStream_t st) {
  GemmArgs g{codes, sc, d, k, dY, M, k, d, At, Gs_hi, Gs_lo, rp, dX};
  return launch_gemm(1, g, st);
}
