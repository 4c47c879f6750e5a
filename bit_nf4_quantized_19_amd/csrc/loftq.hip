// LoftQ initialisation (LLM-train tutorial ch. 3, jwzheng96.github.io,
// section 3.10): alternate a rank-r SVD of the gap between the 16-bit weight
// and its 4-bit base with the quantisation of W - s B A, so that the base
// plus the LoRA branch approximates the 16-bit weight.
//
// Iteration t: R = W - W'_{t-1} (float32; W'_0 = 0, so the first SVD is of W);
// a rank-p SVD of R by randomized subspace iteration (Halko, Martinsson and
// Tropp, SIAM Review 2011: range finder Y = R Omega, q power iterations with
// an orthonormalisation after every product, then the SVD of Q^T R) with
// p = r padded to 16 columns; A = sqrt(S) V^T, B = U sqrt(S) / s (bf16);
// W~ = bf16(W - s B A) (float32, products summed in rank order); the base is
// the NF4 quantisation of W~.
//
// Kernels:
//   mul_right  Y_part = R[:, chunk] Z[chunk, :]   (fp32 MFMA 16x16x4, split over k)
//   mul_left   Z_part = R[chunk, :]^T Y[chunk, :] (fp32 MFMA 16x16x4, split over d)
//   reduce     sum of the split partials in a fixed order
//   gram       float64 partial Gram matrices Y^T Y over 256-row chunks
//   chol       one wave: Cholesky of the Gram matrix (float64) and L^{-T}
//              (CholeskyQR; run twice per orthonormalisation)
//   eig        one wave: cyclic Jacobi on (Q^T R)(Q^T R)^T (float64) giving
//              the small SVD; writes the p x p maps to A^T and B
//   apply      row-wise product with a p x p matrix (fp32 out, or bf16 A^T / B)
//   residual_f32, residual_bf16, pad: elementwise.
// Every kernel is deterministic (fixed summation orders, no atomics).

#include "kernels.h"

namespace {

constexpr int kKC = 512;   // k columns per workgroup of mul_right
constexpr int kDC = 256;   // rows per workgroup of mul_left
constexpr int kGramRows = 256;

QL_DEV f32x4 mfma_f32(float a, float b, f32x4 c) {
  // 16x16x4 fp32: lane l supplies A[l%16][l/16] and B[l/16][l%16];
  // it holds D[4(l/16) + i][l%16].
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// ---- elementwise ------------------------------------------------------------
// R = fl32(W - Wq) (Wq may be null: R = W), 8 elements per thread.
__global__ __launch_bounds__(256) void residual_f32_kernel(const uint16_t *__restrict__ W,
                                                           const uint16_t *__restrict__ Wq,
                                                           int64_t n8, float *__restrict__ R) {
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < n8;
       e += (int64_t)gridDim.x * 256) {
    const uint4 w = ((const uint4 *)W)[e];
    uint4 q = ql::zero4();
    if (Wq) q = ((const uint4 *)Wq)[e];
    const uint32_t wv[4] = {w.x, w.y, w.z, w.w}, qv[4] = {q.x, q.y, q.z, q.w};
    f32x4 o0, o1;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      o0[2 * i] = ql::bf16lo(wv[i]) - ql::bf16lo(qv[i]);
      o0[2 * i + 1] = ql::bf16hi(wv[i]) - ql::bf16hi(qv[i]);
      o1[2 * i] = ql::bf16lo(wv[i + 2]) - ql::bf16lo(qv[i + 2]);
      o1[2 * i + 1] = ql::bf16hi(wv[i + 2]) - ql::bf16hi(qv[i + 2]);
    }
    ((f32x4 *)R)[2 * e] = o0;
    ((f32x4 *)R)[2 * e + 1] = o1;
  }
}

// Zero-padded copy of the test matrix: Op (k x P) <- Omega (k x r).
__global__ __launch_bounds__(256) void pad_kernel(const float *__restrict__ Om, int64_t k, int r,
                                                  int P, float *__restrict__ Op) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= k * P) return;
  const int64_t c = e / P;
  const int j = (int)(e % P);
  Op[e] = j < r ? Om[c * r + j] : 0.0f;
}

// W~ = bf16(W - s B A): per element acc = 0; acc = fma(b_j, a_j, acc) for
// j = 0..r-1 in order (each product of two bf16 values is exact in float32,
// so this is the rounded sum acc + b_j a_j); t = fl(s acc); fl(w - t) rounded
// to bf16 (nearest even). A workgroup covers 16 rows x 1024 columns; a thread
// 16 rows x 4 columns; B's 16 rows are staged in LDS.
constexpr int kRbRows = 16, kRbCols = 1024;
__global__ __launch_bounds__(256) void residual_bf16_kernel(
    const uint16_t *__restrict__ W, const uint16_t *__restrict__ A, const uint16_t *__restrict__ B,
    int64_t d, int64_t k, int r, float s, uint16_t *__restrict__ out) {
  __shared__ float Bs[kRbRows][64];
  const int64_t i0 = (int64_t)blockIdx.y * kRbRows;
  for (int e = threadIdx.x; e < kRbRows * r; e += 256) {
    const int row = e / r, j = e % r;
    Bs[row][j] = (i0 + row < d) ? ql::bf16_to_f(B[(i0 + row) * r + j]) : 0.0f;
  }
  __syncthreads();
  const int64_t c = (int64_t)blockIdx.x * kRbCols + threadIdx.x * 4;
  if (c >= k) return;
  float acc[kRbRows][4];
#pragma unroll
  for (int i = 0; i < kRbRows; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[i][e] = 0.0f;
  for (int j = 0; j < r; ++j) {
    const uint2 av = *(const uint2 *)(A + (int64_t)j * k + c);
    const float a[4] = {ql::bf16lo(av.x), ql::bf16hi(av.x), ql::bf16lo(av.y), ql::bf16hi(av.y)};
#pragma unroll
    for (int i = 0; i < kRbRows; ++i) {
      const float b = Bs[i][j];
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[i][e] = __builtin_fmaf(b, a[e], acc[i][e]);
    }
  }
#pragma unroll
  for (int i = 0; i < kRbRows; ++i) {
    if (i0 + i >= d) break;
    const uint2 wv = *(const uint2 *)(W + (i0 + i) * k + c);
    const float w[4] = {ql::bf16lo(wv.x), ql::bf16hi(wv.x), ql::bf16lo(wv.y), ql::bf16hi(wv.y)};
    float o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float t = s * acc[i][e];
      o[e] = w[e] - t;
    }
    *(uint2 *)(out + (i0 + i) * k + c) = make_uint2(ql::pack_bf16x2(o[0], o[1]),
                                                    ql::pack_bf16x2(o[2], o[3]));
  }
}

// ---- products with the tall operands ----------------------------------------
// part[ks] (d x P) = R[:, ks*kKC .. +kKC) Z[same rows of Z, :], Z k x P.
// Wave = 16 rows of R; lane (m = l%16, q = l/16) loads R[row m][k0+4q..+3]
// and MFMA j takes element j, pairing it with Z[k0 + 4q + j][column].
template <int NB>
__global__ __launch_bounds__(256) void mul_right_kernel(const float *__restrict__ R, int64_t d,
                                                        int64_t k, const float *__restrict__ Z,
                                                        float *__restrict__ part) {
  constexpr int P = 16 * NB;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t i0 = ((int64_t)blockIdx.x * 4 + wave) * 16;
  if (i0 >= d) return;
  const int64_t kb = (int64_t)blockIdx.y * kKC;
  const int64_t ke = kb + kKC < k ? kb + kKC : k;
  const int m = lane & 15, q = lane >> 4;
  const int64_t row = i0 + m < d ? i0 + m : d - 1;
  const float *Rp = R + row * k + 4 * q;
  const float *Zp = Z + (int64_t)(4 * q) * P + m;
  f32x4 acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
  for (int64_t k0 = kb; k0 < ke; k0 += 16) {
    const f32x4 a = *(const f32x4 *)(Rp + k0);
    float b[4][NB];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) b[j][nb] = Zp[(k0 + j) * P + nb * 16];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[nb] = mfma_f32(a[j], b[j][nb], acc[nb]);
  }
  float *out = part + (int64_t)blockIdx.y * d * P;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t ro = i0 + 4 * q + v;
      if (ro < d) out[ro * P + nb * 16 + m] = acc[nb][v];
    }
}

// part[ds] (k x P) = R[ds*kDC .. +kDC, :]^T Y[same rows, :], Y d x P.
// Wave = 64 columns of R; lane (m, q) loads R[r0 + q][c0 + 4m..+3]; MFMA j
// covers the 16 columns c0 + 4m' + j (m' = 0..15), paired with Y[r0 + q][:].
template <int NB>
__global__ __launch_bounds__(256) void mul_left_kernel(const float *__restrict__ R, int64_t d,
                                                       int64_t k, const float *__restrict__ Y,
                                                       float *__restrict__ part) {
  constexpr int P = 16 * NB;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t c0 = ((int64_t)blockIdx.x * 4 + wave) * 64;
  if (c0 >= k) return;
  const int64_t rb = (int64_t)blockIdx.y * kDC;
  const int64_t re = rb + kDC < d ? rb + kDC : d;
  const int m = lane & 15, q = lane >> 4;
  f32x4 acc[4][NB];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[j][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
  for (int64_t r0 = rb; r0 < re; r0 += 4) {
    const bool ok = r0 + q < re;
    const int64_t row = ok ? r0 + q : re - 1;
    f32x4 a = *(const f32x4 *)(R + row * k + c0 + 4 * m);
    float y[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) y[nb] = Y[row * P + nb * 16 + m];
    if (!ok) {
      a = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) y[nb] = 0.0f;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[j][nb] = mfma_f32(a[j], y[nb], acc[j][nb]);
  }
  float *out = part + (int64_t)blockIdx.y * k * P;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        out[(c0 + 4 * (4 * q + v) + j) * P + nb * 16 + m] = acc[j][nb][v];
}

// out[e] = sum over s < ns of part[s * stride + e] (in order), 4 per thread.
__global__ __launch_bounds__(256) void reduce_kernel(const float *__restrict__ part, int ns,
                                                     int64_t stride4, float *__restrict__ out) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= stride4) return;
  f32x4 acc = ((const f32x4 *)part)[e];
  for (int s = 1; s < ns; ++s) acc += ((const f32x4 *)part)[(int64_t)s * stride4 + e];
  ((f32x4 *)out)[e] = acc;
}

// ---- small dense algebra -----------------------------------------------------
// gpart[b] (P x P, float64) = sum over rows i of chunk b of Y[i][a] Y[i][c].
template <int P>
__global__ __launch_bounds__(256) void gram_kernel(const float *__restrict__ Y, int64_t n,
                                                   double *__restrict__ gpart) {
  __shared__ float ys[kGramRows][P];
  const int64_t r0 = (int64_t)blockIdx.x * kGramRows;
  const int t = threadIdx.x;
  for (int e = t; e < kGramRows * P / 4; e += 256) {
    const int row = e / (P / 4), c4 = e % (P / 4);
    f32x4 v = f32x4{0.f, 0.f, 0.f, 0.f};
    if (r0 + row < n) v = ((const f32x4 *)(Y + (r0 + row) * P))[c4];
    *(f32x4 *)&ys[row][4 * c4] = v;
  }
  __syncthreads();
  for (int e = t; e < P * P; e += 256) {
    const int a = e / P, c = e % P;
    double s = 0.0;
    for (int i = 0; i < kGramRows; ++i) s = fma((double)ys[i][a], (double)ys[i][c], s);
    gpart[(int64_t)blockIdx.x * P * P + e] = s;
  }
}

// Sum of nch partial Gram matrices in chunk order.
template <int P>
QL_DEV void load_gram(const double *gpart, int nch, double (*G)[P]) {
  for (int e = threadIdx.x; e < P * P; e += 64) {
    double s = 0.0;
    for (int c = 0; c < nch; ++c) s += gpart[(int64_t)c * P * P + e];
    G[e / P][e % P] = s;
  }
  __syncthreads();
}

// One wave: G = L L^T (float64, left-looking by columns); a pivot not above
// 1e-12 of its diagonal entry marks a dependent column, whose L column is
// zero (its Q column comes out zero). Writes M = L^{-T} (fp32) so that
// Q = Y M has orthonormal columns.
template <int P>
__global__ __launch_bounds__(64) void chol_kernel(const double *__restrict__ gpart, int nch,
                                                  float *__restrict__ M) {
  __shared__ double G[P][P];
  __shared__ double L[P][P];
  __shared__ double piv;
  const int lane = threadIdx.x;
  load_gram<P>(gpart, nch, G);
  for (int e = lane; e < P * P; e += 64) L[e / P][e % P] = 0.0;
  __syncthreads();
  for (int j = 0; j < P; ++j) {
    double v = 0.0;
    if (lane < P && lane >= j) {
      v = G[lane][j];
      for (int t = 0; t < j; ++t) v -= L[lane][t] * L[j][t];
    }
    if (lane == j) piv = v;
    __syncthreads();
    const double pj = piv;
    const bool dead = !(pj > 1e-12 * G[j][j]);
    if (lane < P && lane >= j) L[lane][j] = dead ? 0.0 : v / sqrt(pj);
    __syncthreads();
  }
  // column j of L^{-1} by forward substitution (lane j); stored in G
  if (lane < P) {
    const int j = lane;
    for (int i = 0; i < P; ++i) {
      double x = 0.0;
      if (i >= j) {
        double s = (i == j) ? 1.0 : 0.0;
        for (int t = j; t < i; ++t) s -= L[i][t] * G[t][j];
        x = L[i][i] != 0.0 ? s / L[i][i] : 0.0;
      }
      G[i][j] = x;
    }
  }
  __syncthreads();
  for (int e = lane; e < P * P; e += 64) M[e] = (float)G[e % P][e / P];   // M[a][c] = Linv[c][a]
}

// One wave: eigen-decomposition of the symmetric P x P matrix C C^T (sum of
// the partial Gram matrices of Z = R^T Q, so C = Q^T R) by cyclic Jacobi in
// float64; eigenvalues sorted descending, sigma_j = sqrt(lambda_j). Writes
// MA = U_c diag(sigma^{-1/2}) (A^T = Z MA) and MB = U_c diag(sigma^{1/2}) / s
// (B = Q MB); directions with lambda_j <= 1e-24 lambda_0 get zero columns.
template <int P>
__global__ __launch_bounds__(64) void eig_kernel(const double *__restrict__ gpart, int nch,
                                                 int r, float s, float *__restrict__ MA,
                                                 float *__restrict__ MB,
                                                 float *__restrict__ sigma) {
  __shared__ double Am[P][P];
  __shared__ double V[P][P];
  __shared__ int order[P];
  __shared__ int used[P];
  __shared__ int done;
  const int lane = threadIdx.x;
  load_gram<P>(gpart, nch, Am);
  for (int e = lane; e < P * P; e += 64) V[e / P][e % P] = (e / P == e % P) ? 1.0 : 0.0;
  __syncthreads();
  for (int sweep = 0; sweep < 60; ++sweep) {
    if (lane == 0) {
      double off = 0.0, dg = 0.0;
      for (int p = 0; p < P; ++p)
        for (int c = 0; c < P; ++c) {
          const double x = Am[p][c] * Am[p][c];
          if (p == c) dg += x; else off += x;
        }
      done = !(off > 1e-30 * dg);
    }
    __syncthreads();
    if (done) break;
    for (int p = 0; p < P - 1; ++p)
      for (int q = p + 1; q < P; ++q) {
        const double apq = Am[p][q], app = Am[p][p], aqq = Am[q][q];
        __syncthreads();
        if (apq == 0.0) continue;
        const double tau = (aqq - app) / (2.0 * apq);
        const double t = (tau >= 0.0 ? 1.0 : -1.0) / (fabs(tau) + sqrt(1.0 + tau * tau));
        const double c = 1.0 / sqrt(1.0 + t * t), sn = t * c;
        if (lane < P) {
          const double tp = Am[lane][p], tq = Am[lane][q];
          Am[lane][p] = c * tp - sn * tq;
          Am[lane][q] = sn * tp + c * tq;
          const double vp = V[lane][p], vq = V[lane][q];
          V[lane][p] = c * vp - sn * vq;
          V[lane][q] = sn * vp + c * vq;
        }
        __syncthreads();
        if (lane < P) {
          const double tp = Am[p][lane], tq = Am[q][lane];
          Am[p][lane] = c * tp - sn * tq;
          Am[q][lane] = sn * tp + c * tq;
        }
        __syncthreads();
      }
  }
  if (lane < P) used[lane] = 0;
  __syncthreads();
  if (lane == 0) {
    // selection order by descending eigenvalue (lower index first on ties)
    for (int j = 0; j < P; ++j) {
      int best = -1;
      for (int c = 0; c < P; ++c)
        if (!used[c] && (best < 0 || Am[c][c] > Am[best][best])) best = c;
      used[best] = 1;
      order[j] = best;
    }
  }
  __syncthreads();
  const double lmax = Am[order[0]][order[0]];
  for (int e = lane; e < P * P; e += 64) {
    const int a = e / P, j = e % P;
    const double lam = Am[order[j]][order[j]];
    const bool alive = lmax > 0.0 && lam > 1e-24 * lmax;
    const double sg = alive ? sqrt(lam) : 0.0;
    const double u = V[a][order[j]];
    MA[e] = alive ? (float)(u / sqrt(sg)) : 0.0f;
    MB[e] = alive ? (float)(u * sqrt(sg) / (double)s) : 0.0f;
  }
  if (sigma && lane < r) {
    const double lam = Am[order[lane]][order[lane]];
    sigma[lane] = lam > 0.0 ? (float)sqrt(lam) : 0.0f;
  }
}

// out = In (n x P) M (P x P): MODE 0 fp32 n x P; MODE 1 bf16 n x r (row i,
// column j < r); MODE 2 bf16 r x n (the transpose). Thread = one row and one
// 16-column block.
template <int P, int MODE>
__global__ __launch_bounds__(256) void apply_kernel(const float *__restrict__ In, int64_t n,
                                                    const float *__restrict__ M, int r,
                                                    void *__restrict__ out) {
  constexpr int NB = P / 16;
  __shared__ float Ms[P][P];
  for (int e = threadIdx.x; e < P * P; e += 256) Ms[e / P][e % P] = M[e];
  __syncthreads();
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t i = g / NB;
  const int cb = (int)(g % NB);
  if (i >= n) return;
  float x[P];
#pragma unroll
  for (int a4 = 0; a4 < P / 4; ++a4) {
    const f32x4 v = ((const f32x4 *)(In + i * P))[a4];
    x[4 * a4] = v[0]; x[4 * a4 + 1] = v[1]; x[4 * a4 + 2] = v[2]; x[4 * a4 + 3] = v[3];
  }
#pragma unroll
  for (int jj = 0; jj < 16; ++jj) {
    const int j = cb * 16 + jj;
    float acc = 0.0f;
#pragma unroll
    for (int a = 0; a < P; ++a) acc = __builtin_fmaf(x[a], Ms[a][j], acc);
    if (MODE == 0) {
      ((float *)out)[i * P + j] = acc;
    } else if (j < r) {
      const uint16_t b = ql::f_to_bf16(acc);
      if (MODE == 1) ((uint16_t *)out)[i * r + j] = b;
      else ((uint16_t *)out)[(int64_t)j * n + i] = b;
    }
  }
}

// ---- host side -----------------------------------------------------------------
struct LoftqWs {
  float *R, *Op, *Yd, *Td, *Zk, *Tk, *part, *MA, *MB, *Mc;
  double *gpart;
  uint16_t *Wb;      // W~ (and the dequantised base W' before it)
  void *qws;         // quantiser workspace
  int64_t bytes;
};

constexpr int64_t kAl = 256;
template <class T>
T *carve(char *base, int64_t &off, int64_t bytes) {
  T *p = base ? (T *)(base + off) : nullptr;
  off += ql_rup(bytes, kAl);
  return p;
}

LoftqWs loftq_layout(char *base, int64_t d, int64_t k, int r, int dq) {
  const int64_t P = ql_rup(r, 16);
  const int64_t ks = ql_cdiv(k, kKC), ds = ql_cdiv(d, kDC);
  const int64_t nch = ql_cdiv(d > k ? d : k, kGramRows);
  int64_t off = 0;
  LoftqWs L{};
  L.R = carve<float>(base, off, 4 * d * k);
  L.Wb = carve<uint16_t>(base, off, 2 * d * k);
  L.qws = carve<char>(base, off, (int64_t)quantize_ws_bytes(d * k, dq));
  L.Op = carve<float>(base, off, 4 * k * P);
  L.Yd = carve<float>(base, off, 4 * d * P);
  L.Td = carve<float>(base, off, 4 * d * P);
  L.Zk = carve<float>(base, off, 4 * k * P);
  L.Tk = carve<float>(base, off, 4 * k * P);
  L.part = carve<float>(base, off, 4 * P * (ks * d > ds * k ? ks * d : ds * k));
  L.gpart = carve<double>(base, off, 8 * nch * P * P);
  L.MA = carve<float>(base, off, 4 * P * P);
  L.MB = carve<float>(base, off, 4 * P * P);
  L.Mc = carve<float>(base, off, 4 * P * P);
  L.bytes = off;
  return L;
}

template <int NB>
struct Loftq {
  static constexpr int P = 16 * NB;
  const LoftqWs &L;
  int64_t d, k;
  hipStream_t st;

  qlora_status right(const float *Z, float *Y) {   // Y (d x P) = R Z
    {
      QlProf pf(QLORA_K_LOFTQ_PRODUCT, st);
      mul_right_kernel<NB><<<dim3((unsigned)ql_cdiv(d, 64), (unsigned)ql_cdiv(k, kKC)), 256, 0, st>>>(
          L.R, d, k, Z, L.part);
    }
    QL_LAUNCH_CHECK();
    return reduce(L.part, (int)ql_cdiv(k, kKC), d, Y);
  }
  qlora_status left(const float *Y, float *Z) {    // Z (k x P) = R^T Y
    {
      QlProf pf(QLORA_K_LOFTQ_PRODUCT, st);
      mul_left_kernel<NB><<<dim3((unsigned)ql_cdiv(k, 256), (unsigned)ql_cdiv(d, kDC)), 256, 0, st>>>(
          L.R, d, k, Y, L.part);
    }
    QL_LAUNCH_CHECK();
    return reduce(L.part, (int)ql_cdiv(d, kDC), k, Z);
  }
  qlora_status reduce(const float *part, int ns, int64_t n, float *out) {
    const int64_t n4 = n * P / 4;
    QlProf pf(QLORA_K_LOFTQ_SMALL, st);
    reduce_kernel<<<(unsigned)ql_cdiv(n4, 256), 256, 0, st>>>(part, ns, n4, out);
    QL_LAUNCH_CHECK();
    return QLORA_OK;
  }
  qlora_status gram(const float *Y, int64_t n) {
    QlProf pf(QLORA_K_LOFTQ_SMALL, st);
    gram_kernel<P><<<(unsigned)ql_cdiv(n, kGramRows), 256, 0, st>>>(Y, n, L.gpart);
    QL_LAUNCH_CHECK();
    return QLORA_OK;
  }
  // CholeskyQR2: the orthonormal basis of Y's columns ends in Y (T: scratch)
  qlora_status orth(float *Y, float *T, int64_t n) {
    qlora_status s;
    float *src = Y, *dst = T;
    for (int pass = 0; pass < 2; ++pass) {
      if ((s = gram(src, n)) != QLORA_OK) return s;
      {
        QlProf pf(QLORA_K_LOFTQ_SMALL, st);
        chol_kernel<P><<<1, 64, 0, st>>>(L.gpart, (int)ql_cdiv(n, kGramRows), L.Mc);
        QL_LAUNCH_CHECK();
        apply_kernel<P, 0><<<(unsigned)ql_cdiv(n * NB, 256), 256, 0, st>>>(src, n, L.Mc, P, dst);
        QL_LAUNCH_CHECK();
      }
      float *t = src; src = dst; dst = t;
    }
    return QLORA_OK;
  }
  // rank-P SVD of R; writes A (r x k), B (d x r) bf16 and sigma (r)
  qlora_status svd(int power_iters, int r, float s, uint16_t *A, uint16_t *B, float *sigma) {
    qlora_status e;
    if ((e = right(L.Op, L.Yd)) != QLORA_OK) return e;
    if ((e = orth(L.Yd, L.Td, d)) != QLORA_OK) return e;
    for (int it = 0; it < power_iters; ++it) {
      if ((e = left(L.Yd, L.Zk)) != QLORA_OK) return e;
      if ((e = orth(L.Zk, L.Tk, k)) != QLORA_OK) return e;
      if ((e = right(L.Zk, L.Yd)) != QLORA_OK) return e;
      if ((e = orth(L.Yd, L.Td, d)) != QLORA_OK) return e;
    }
    if ((e = left(L.Yd, L.Zk)) != QLORA_OK) return e;   // Z = R^T Q = C^T
    if ((e = gram(L.Zk, k)) != QLORA_OK) return e;
    QlProf pf(QLORA_K_LOFTQ_SMALL, st);
    eig_kernel<P><<<1, 64, 0, st>>>(L.gpart, (int)ql_cdiv(k, kGramRows), r, s, L.MA, L.MB, sigma);
    QL_LAUNCH_CHECK();
    apply_kernel<P, 2><<<(unsigned)ql_cdiv(k * NB, 256), 256, 0, st>>>(L.Zk, k, L.MA, r, A);
    QL_LAUNCH_CHECK();
    apply_kernel<P, 1><<<(unsigned)ql_cdiv(d * NB, 256), 256, 0, st>>>(L.Yd, d, L.MB, r, B);
    QL_LAUNCH_CHECK();
    return QLORA_OK;
  }
};

qlora_status residual_f32(const uint16_t *W, const uint16_t *Wq, int64_t n, float *R,
                          hipStream_t st) {
  const int64_t n8 = n / 8;
  const int64_t grid = ql_cdiv(n8, 256) < 8192 ? ql_cdiv(n8, 256) : 8192;
  QlProf pf(QLORA_K_RESIDUAL, st);
  residual_f32_kernel<<<(unsigned)grid, 256, 0, st>>>(W, Wq, n8, R);
  QL_LAUNCH_CHECK();
  return QLORA_OK;
}

template <int NB>
qlora_status loftq_run(const uint16_t *W, const float *omega, int64_t d, int64_t k, int r,
                       float s, int iters, int power_iters, const QuantOut &qo, uint16_t *A,
                       uint16_t *B, float *sigma, const LoftqWs &L, hipStream_t st) {
  Loftq<NB> lq{L, d, k, st};
  constexpr int P = 16 * NB;
  qlora_status e;
  pad_kernel<<<(unsigned)ql_cdiv(k * P, 256), 256, 0, st>>>(omega, k, r, P, L.Op);
  QL_LAUNCH_CHECK();
  for (int t = 0; t < iters; ++t) {
    if (t > 0) {
      if ((e = launch_dequantize(qo.codes, qo.sc, d * k, L.Wb, st)) != QLORA_OK) return e;
    }
    if ((e = residual_f32(W, t > 0 ? L.Wb : nullptr, d * k, L.R, st)) != QLORA_OK) return e;
    if ((e = lq.svd(power_iters, r, s, A, B, sigma)) != QLORA_OK) return e;
    if ((e = launch_residual_quantize(W, A, B, d, k, r, s, qo, L.Wb, L.qws, st)) != QLORA_OK)
      return e;
  }
  return QLORA_OK;
}

}  // namespace

size_t loftq_ws_bytes(int64_t d, int64_t k, int r, int dq) {
  return (size_t)loftq_layout(nullptr, d, k, r, dq).bytes;
}

size_t residual_quantize_ws_bytes(int64_t d, int64_t k, int dq) {
  return (size_t)(ql_rup(2 * d * k, kAl) + (int64_t)quantize_ws_bytes(d * k, dq));
}

qlora_status launch_residual_quantize(const uint16_t *W, const uint16_t *A, const uint16_t *B,
                                      int64_t d, int64_t k, int r, float s, const QuantOut &qo,
                                      uint16_t *Wt, void *qws, hipStream_t st) {
  {
    QlProf pf(QLORA_K_RESIDUAL, st);
    residual_bf16_kernel<<<dim3((unsigned)ql_cdiv(k, kRbCols), (unsigned)ql_cdiv(d, kRbRows)), 256,
                           0, st>>>(W, A, B, d, k, r, s, Wt);
  }
  QL_LAUNCH_CHECK();
  return launch_quantize(Wt, d * k, qo.codes, qo.absmax, qo.sc.dq, qo.q, qo.s2, qo.mu, qws, st);
}

qlora_status launch_residual_quantize_ws(const uint16_t *W, const uint16_t *A, const uint16_t *B,
                                         int64_t d, int64_t k, int r, float s, const QuantOut &qo,
                                         void *ws, hipStream_t st) {
  uint16_t *Wt = (uint16_t *)ws;
  void *qws = (char *)ws + ql_rup(2 * d * k, kAl);
  return launch_residual_quantize(W, A, B, d, k, r, s, qo, Wt, qws, st);
}

qlora_status launch_loftq(const uint16_t *W, const float *omega, int64_t d, int64_t k, int r,
                          float s, int iters, int power_iters, const QuantOut &qo, uint16_t *A,
                          uint16_t *B, float *sigma, void *ws, hipStream_t st) {
  const LoftqWs L = loftq_layout((char *)ws, d, k, r, qo.sc.dq);
  switch (ql_cdiv(r, 16)) {
    case 1: return loftq_run<1>(W, omega, d, k, r, s, iters, power_iters, qo, A, B, sigma, L, st);
    case 2: return loftq_run<2>(W, omega, d, k, r, s, iters, power_iters, qo, A, B, sigma, L, st);
    case 3: return loftq_run<3>(W, omega, d, k, r, s, iters, power_iters, qo, A, B, sigma, L, st);
    case 4: return loftq_run<4>(W, omega, d, k, r, s, iters, power_iters, qo, A, B, sigma, L, st);
    default: return QLORA_ERR_UNSUPPORTED;
  }
}
