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
//   reduce_gram  sum of the split partials in a fixed order, with the
//              float64 partial Gram matrices Y^T Y of 256-row chunks
//   orth_apply CholeskyQR: every workgroup sums the partial Gram matrices
//              (all threads, one entry each), factors the sum in one wave
//              (float64, registers) and applies L^{-T} to its rows,
//              optionally with the partial Gram matrices of its output (run
//              twice per orthonormalisation: CholeskyQR2)
//   eig        one wave: Jacobi (round-robin, float64) on (Q^T R)(Q^T R)^T
//              giving the small SVD; writes the p x p maps to A^T and B
//   apply      row-wise product with a p x p matrix (bf16 A^T / B)
//   residual_f32, residual_bf16, pad: elementwise.
// Every kernel is deterministic (fixed summation orders, no atomics).

#include <type_traits>

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
constexpr int kU = 4;   // 16-column (mul_right) or 4-row (mul_left) steps per load batch

// part[ks] (d x P) = R[:, ks*kKC .. +kKC) Z[same rows of Z, :], Z k x P.
// Workgroup = 16 rows of R; its 4 waves take the chunk's 64-column batches
// in turn and add their sums in LDS (in wave order). Lane (m = l%16,
// q = l/16) loads R[row m][k0+4q..+3] and MFMA j takes element j, pairing it
// with Z[k0 + 4q + j][column]; a batch issues its kU loads before its MFMAs.
template <int NB>
__global__ __launch_bounds__(256) void mul_right_kernel(const float *__restrict__ R, int64_t d,
                                                        int64_t k, const float *__restrict__ Z,
                                                        float *__restrict__ part) {
  constexpr int P = 16 * NB;
  __shared__ f32x4 red[4][NB][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t i0 = (int64_t)blockIdx.x * 16;
  const int64_t kb = (int64_t)blockIdx.y * kKC;
  const int64_t ke = kb + kKC < k ? kb + kKC : k;   // ke - kb: a multiple of 64 = 16 kU
  const int m = lane & 15, q = lane >> 4;
  const int64_t row = i0 + m < d ? i0 + m : d - 1;
  const float *Rp = R + row * k + 4 * q;
  const float *Zp = Z + (int64_t)(4 * q) * P + m;
  f32x4 acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int64_t k0 = kb + 16 * kU * wave; k0 < ke; k0 += 4 * 16 * kU) {
    f32x4 a[kU];
    float b[kU][4][NB];
#pragma unroll
    for (int u = 0; u < kU; ++u) a[u] = *(const f32x4 *)(Rp + k0 + 16 * u);
#pragma unroll
    for (int u = 0; u < kU; ++u)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) b[u][j][nb] = Zp[(k0 + 16 * u + j) * P + nb * 16];
#pragma unroll
    for (int u = 0; u < kU; ++u)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[nb] = mfma_f32(a[u][j], b[u][j][nb], acc[nb]);
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) red[wave][nb][lane] = acc[nb];
  __syncthreads();
  if (wave != 0) return;
  float *out = part + (int64_t)blockIdx.y * d * P;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const f32x4 t = red[0][nb][lane] + red[1][nb][lane] + red[2][nb][lane] + red[3][nb][lane];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t ro = i0 + 4 * q + v;
      if (ro < d) out[ro * P + nb * 16 + m] = t[v];
    }
  }
}

// part[ds] (k x P) = R[ds*kDC .. +kDC, :]^T Y[same rows, :], Y d x P.
// Workgroup = 64 columns of R; its 4 waves take the chunk's 16-row batches
// in turn and add their sums in LDS (in wave order). Lane (m, q) loads
// R[r0 + q][c0 + 4m..+3]; MFMA j covers the 16 columns c0 + 4m' + j
// (m' = 0..15), paired with Y[r0 + q][:]. Rows past the chunk read as zero.
template <int NB>
__global__ __launch_bounds__(256) void mul_left_kernel(const float *__restrict__ R, int64_t d,
                                                       int64_t k, const float *__restrict__ Y,
                                                       float *__restrict__ part) {
  constexpr int P = 16 * NB;
  __shared__ f32x4 red[4][4][NB][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t c0 = (int64_t)blockIdx.x * 64;
  const int64_t rb = (int64_t)blockIdx.y * kDC;
  const int64_t re = rb + kDC < d ? rb + kDC : d;
  const int m = lane & 15, q = lane >> 4;
  f32x4 acc[4][NB];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[j][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int64_t r0 = rb + 4 * kU * wave; r0 < re; r0 += 4 * 4 * kU) {
    f32x4 a[kU];
    float y[kU][NB];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t rr = r0 + 4 * u + q;
      const int64_t row = rr < re ? rr : re - 1;
      a[u] = *(const f32x4 *)(R + row * k + c0 + 4 * m);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) y[u][nb] = Y[row * P + nb * 16 + m];
    }
#pragma unroll
    for (int u = 0; u < kU; ++u)
      if (r0 + 4 * u + q >= re) {
        a[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) y[u][nb] = 0.0f;
      }
#pragma unroll
    for (int u = 0; u < kU; ++u)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[j][nb] = mfma_f32(a[u][j], y[u][nb], acc[j][nb]);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) red[wave][j][nb][lane] = acc[j][nb];
  __syncthreads();
  // wave w writes the outputs of MFMA j = w
  const int j = wave;
  float *out = part + (int64_t)blockIdx.y * k * P;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const f32x4 t = red[0][j][nb][lane] + red[1][j][nb][lane] + red[2][j][nb][lane] +
                    red[3][j][nb][lane];
#pragma unroll
    for (int v = 0; v < 4; ++v) out[(c0 + 4 * (4 * q + v) + j) * P + nb * 16 + m] = t[v];
  }
}

// ---- small dense algebra -----------------------------------------------------
// Partial Gram matrix of the rows staged in ys (rows x P, zero past n):
// g[a][c] = sum_i ys[i][a] ys[i][c] in float64, written to gout.
// rows is a multiple of 4; four partial sums over rows i % 4, added in order.
// T is the staging type: float, or the same values already widened to
// double (one conversion per element instead of two per product; the
// products and sums are the same).
template <int P, class T>
QL_DEV void gram_rows(const T (*ys)[P], int rows, double *gout) {
  for (int e = threadIdx.x; e < P * P; e += 256) {
    const int a = e / P, c = e % P;
    double s0 = 0.0, s1 = 0.0, s2 = 0.0, s3 = 0.0;
    for (int i = 0; i < rows; i += 4) {
      s0 = fma((double)ys[i][a], (double)ys[i][c], s0);
      s1 = fma((double)ys[i + 1][a], (double)ys[i + 1][c], s1);
      s2 = fma((double)ys[i + 2][a], (double)ys[i + 2][c], s2);
      s3 = fma((double)ys[i + 3][a], (double)ys[i + 3][c], s3);
    }
    gout[e] = (s0 + s1) + (s2 + s3);
  }
}

// Y (n x P) = sum over s < ns of part[s] (in order), and the partial Gram
// matrix of each 256-row chunk (gout[block], float64). The chunk is staged in
// LDS as double for P = 16 (32 KB), as float for wider P.
template <int P>
__global__ __launch_bounds__(256) void reduce_gram_kernel(const float *__restrict__ part, int ns,
                                                          int64_t n, float *__restrict__ Y,
                                                          double *__restrict__ gout) {
  using T = typename std::conditional<P == 16, double, float>::type;
  __shared__ T ys[kGramRows][P];
  const int64_t r0 = (int64_t)blockIdx.x * kGramRows;
  const int64_t n4 = n * P / 4;
  for (int e = threadIdx.x; e < kGramRows * P / 4; e += 256) {
    const int row = e / (P / 4), c4 = e % (P / 4);
    const int64_t g = (r0 + row) * (P / 4) + c4;
    f32x4 v = f32x4{0.f, 0.f, 0.f, 0.f};
    if (r0 + row < n) {
      v = ((const f32x4 *)part)[g];
      // eight splits' loads in flight (clamped split index), then their sums
      // in split order
      for (int s0 = 1; s0 < ns; s0 += 8) {
        f32x4 t[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          t[u] = ((const f32x4 *)part)[(int64_t)min(s0 + u, ns - 1) * n4 + g];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (s0 + u < ns) v += t[u];
      }
      ((f32x4 *)Y)[g] = v;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) ys[row][4 * c4 + i] = (T)v[i];
  }
  __syncthreads();
  gram_rows<P, T>(ys, kGramRows, gout + (int64_t)blockIdx.x * P * P);
}

// 1/sqrt(x) for x > 0: the hardware estimate refined by two Newton steps
// (relative error at the float64 rounding level).
QL_DEV double rsqrt_f64(double x) {
  double y = __builtin_amdgcn_rsq(x);
  y = y * fma(-0.5 * x * y, y, 1.5);
  y = y * fma(-0.5 * x * y, y, 1.5);
  return y;
}

QL_DEV double bcast(double x, int l) {
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)u, l);
  const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(u >> 32), l);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Every thread of the workgroup: G = sum of the nch partial Gram matrices
// (float64, in partial order), entry e summed by thread e % 256, into Gs.
template <int P>
QL_DEV void gram_sum(const double *__restrict__ gin, int nch, double (*Gs)[P]) {
  for (int e = threadIdx.x; e < P * P; e += 256) {
    double sum = 0.0;
    // eight partials' loads in flight (clamped index), then their sums in order
    for (int b0 = 0; b0 < nch; b0 += 8) {
      double t[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) t[u] = gin[(int64_t)min(b0 + u, nch - 1) * P * P + e];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (b0 + u < nch) sum += t[u];
    }
    Gs[e / P][e % P] = sum;
  }
}

// One wave (all 64 lanes active), after gram_sum: G = L L^T by columns with
// lane i holding row i of L in registers (other rows by readlane); a pivot
// not above 1e-12 of its diagonal entry marks a dependent column, whose L
// column is zero (its Q column comes out zero). Lane j then computes column
// j of L^{-1}; Ms = L^{-T} (fp32), so that Q = Y Ms has orthonormal columns.
template <int P>
QL_DEV void chol_wave(const double (*Gs)[P], float (*Ms)[P]) {
  const int lane = threadIdx.x & 63;
  double L[P];
#pragma unroll
  for (int c = 0; c < P; ++c) L[c] = lane < P ? Gs[lane][c] : 0.0;
  // L[c] holds G[lane][c] until column c is computed; ri[j] = 1 / L[j][j]
  // (0 for a dependent column)
  double ri[P];
#pragma unroll
  for (int j = 0; j < P; ++j) {
    double v = L[j];
#pragma unroll
    for (int t = 0; t < j; ++t) v = fma(-L[t], bcast(L[t], j), v);
    const double piv = bcast(v, j);
    const double gjj = bcast(L[j], j);
    const bool dead = !(piv > 1e-12 * gjj);
    const double rs = dead ? 0.0 : rsqrt_f64(piv);
    ri[j] = rs;
    L[j] = lane >= j ? v * rs : 0.0;
  }
  double x[P];
#pragma unroll
  for (int i = 0; i < P; ++i) {
    double s = (lane == i) ? 1.0 : 0.0;
#pragma unroll
    for (int t = 0; t < i; ++t) s = fma(-bcast(L[t], i), x[t], s);
    x[i] = s * ri[i];
  }
  if (lane < P)
#pragma unroll
    for (int c = 0; c < P; ++c) Ms[lane][c] = (float)x[c];   // Ms[a][c] = Linv[c][a]
}

// Q = Y L^{-T} with L from the partial Gram matrices gin (each workgroup
// sums them with all its threads and factors the P x P result in its first
// wave); with GRAM the partial Gram
// matrix of the workgroup's output rows goes to gout[block]. A thread owns
// one row and one 16-column block; a workgroup orth_rows(NB) rows (a multiple
// of 4 with rows x NB <= 256; the other threads only take part in the
// barriers and the Gram sums).
constexpr int orth_rows(int nb) { return nb == 1 ? 256 : (nb == 2 ? 128 : 64); }
template <int P, bool GRAM>
__global__ __launch_bounds__(256) void orth_apply_kernel(const float *__restrict__ In, int64_t n,
                                                         const double *__restrict__ gin, int nch,
                                                         float *__restrict__ Out,
                                                         double *__restrict__ gout) {
  constexpr int NB = P / 16, RPB = orth_rows(NB);
  static_assert(RPB % 4 == 0 && RPB * NB <= 256, "rows per workgroup");
  __shared__ float Ms[P][P];
  __shared__ double Gs[P][P];
  __shared__ double ys[GRAM ? RPB : 1][P];
  gram_sum<P>(gin, nch, Gs);
  __syncthreads();
  if (threadIdx.x < 64) chol_wave<P>(Gs, Ms);
  __syncthreads();
  const int lr = threadIdx.x / NB, cb = threadIdx.x % NB;
  const bool own = lr < RPB;
  const int64_t i = (int64_t)blockIdx.x * RPB + lr;
  float o[16];
#pragma unroll
  for (int jj = 0; jj < 16; ++jj) o[jj] = 0.0f;
  if (own && i < n) {
    float x[P];
#pragma unroll
    for (int a4 = 0; a4 < P / 4; ++a4) {
      const f32x4 v = ((const f32x4 *)(In + i * P))[a4];
      x[4 * a4] = v[0]; x[4 * a4 + 1] = v[1]; x[4 * a4 + 2] = v[2]; x[4 * a4 + 3] = v[3];
    }
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) {
      float acc = 0.0f;
#pragma unroll
      for (int a = 0; a < P; ++a) acc = __builtin_fmaf(x[a], Ms[a][cb * 16 + jj], acc);
      o[jj] = acc;
    }
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4)
      ((f32x4 *)(Out + i * P + cb * 16))[j4] =
          f32x4{o[4 * j4], o[4 * j4 + 1], o[4 * j4 + 2], o[4 * j4 + 3]};
  }
  if (GRAM) {
    if (own)
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) ys[lr][cb * 16 + jj] = (double)o[jj];
    __syncthreads();
    gram_rows<P, double>(ys, RPB, gout + (int64_t)blockIdx.x * P * P);
  }
}

// One wave: eigen-decomposition of the symmetric P x P matrix C C^T (sum of
// the partial Gram matrices of Z = R^T Q, so C = Q^T R) by Jacobi in float64
// with the round-robin ordering: each of the P-1 steps of a sweep applies
// P/2 disjoint rotations at once (their angles from the matrix at the start
// of the step, which is exact since they touch disjoint rows and columns).
// Eigenvalues sorted descending, sigma_j = sqrt(lambda_j). Writes
// MA = U_c diag(sigma^{-1/2}) (A^T = Z MA) and MB = U_c diag(sigma^{1/2}) / s
// (B = Q MB); directions with lambda_j <= 1e-24 lambda_0 get zero columns.
template <int P>
__global__ __launch_bounds__(64) void eig_kernel(const double *__restrict__ gpart, int nch,
                                                 int r, float s, float *__restrict__ MA,
                                                 float *__restrict__ MB,
                                                 float *__restrict__ sigma) {
  constexpr int G = 64 / P;          // lane groups sharing the pairs of a step
  constexpr int PPL = P / 2 / G;     // pairs per lane
  __shared__ double Am[P][P + 1];
  __shared__ double V[P][P + 1];
  __shared__ double rc[P / 2], rs[P / 2];
  __shared__ int rp[P / 2], rq[P / 2];
  __shared__ double offp[P], dgp[P];
  __shared__ int order[P];
  const int lane = threadIdx.x;
  for (int e = lane; e < P * P; e += 64) {
    double sum = 0.0;
#pragma unroll 8
    for (int b = 0; b < nch; ++b) sum += gpart[(int64_t)b * P * P + e];
    Am[e / P][e % P] = sum;
    V[e / P][e % P] = (e / P == e % P) ? 1.0 : 0.0;
  }
  __syncthreads();
  const int row = lane % P, grp = lane / P;
  for (int sweep = 0; sweep < 60; ++sweep) {
    if (lane < P) {   // squares of row `lane`, off the diagonal and on it
      double off = 0.0;
#pragma unroll
      for (int c = 0; c < P; ++c) off += (c == lane) ? 0.0 : Am[lane][c] * Am[lane][c];
      offp[lane] = off;
      dgp[lane] = Am[lane][lane] * Am[lane][lane];
    }
    __syncthreads();
    double off = 0.0, dg = 0.0;
#pragma unroll
    for (int c = 0; c < P; ++c) { off += offp[c]; dg += dgp[c]; }
    if (!(off > 1e-30 * dg)) break;   // uniform: every lane sums the same values
    for (int step = 0; step < P - 1; ++step) {
      if (lane < P / 2) {
        // circle method: player 0 meets 1 + step; the others pair around it
        int p, q;
        if (lane == 0) {
          p = 0;
          q = 1 + step;
        } else {
          p = 1 + (step + lane) % (P - 1);
          q = 1 + (step + P - 1 - lane) % (P - 1);
        }
        if (p > q) { const int t = p; p = q; q = t; }
        const double apq = Am[p][q], dd = Am[q][q] - Am[p][p];
        double c = 1.0, sn = 0.0;
        if (apq != 0.0) {
          // t = tan(theta) of the rotation that zeroes A[p][q] (smaller root)
          const double t = (dd >= 0.0 ? 2.0 * apq : -2.0 * apq) /
                           (fabs(dd) + sqrt(fma(dd, dd, 4.0 * apq * apq)));
          c = rsqrt_f64(fma(t, t, 1.0));
          sn = t * c;
        }
        rp[lane] = p; rq[lane] = q; rc[lane] = c; rs[lane] = sn;
      }
      __syncthreads();
      if (grp < G) {   // A <- A J and V <- V J: row `row`, columns p, q of this lane's pairs
        double ap[PPL], aq[PPL], vp[PPL], vq[PPL];
#pragma unroll
        for (int h = 0; h < PPL; ++h) {
          const int hh = grp * PPL + h;
          ap[h] = Am[row][rp[hh]]; aq[h] = Am[row][rq[hh]];
          vp[h] = V[row][rp[hh]]; vq[h] = V[row][rq[hh]];
        }
#pragma unroll
        for (int h = 0; h < PPL; ++h) {
          const int hh = grp * PPL + h;
          const double c = rc[hh], sn = rs[hh];
          Am[row][rp[hh]] = c * ap[h] - sn * aq[h];
          Am[row][rq[hh]] = sn * ap[h] + c * aq[h];
          V[row][rp[hh]] = c * vp[h] - sn * vq[h];
          V[row][rq[hh]] = sn * vp[h] + c * vq[h];
        }
      }
      __syncthreads();
      if (grp < G) {   // A <- J^T A: column `row`, rows p, q of this lane's pairs
        double ap[PPL], aq[PPL];
#pragma unroll
        for (int h = 0; h < PPL; ++h) {
          const int hh = grp * PPL + h;
          ap[h] = Am[rp[hh]][row]; aq[h] = Am[rq[hh]][row];
        }
#pragma unroll
        for (int h = 0; h < PPL; ++h) {
          const int hh = grp * PPL + h;
          const double c = rc[hh], sn = rs[hh];
          Am[rp[hh]][row] = c * ap[h] - sn * aq[h];
          Am[rq[hh]][row] = sn * ap[h] + c * aq[h];
        }
      }
      __syncthreads();
    }
  }
  if (lane < P) {   // rank by descending eigenvalue, lower index first on ties
    const double lj = Am[lane][lane];
    int rank = 0;
#pragma unroll
    for (int c = 0; c < P; ++c) {
      const double lc = Am[c][c];
      rank += (lc > lj || (lc == lj && c < lane)) ? 1 : 0;
    }
    order[rank] = lane;
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

// out = In (n x P) M (P x P) as bf16: MODE 1 n x r (row i, column j < r);
// MODE 2 r x n (the transpose). Thread = one row and one 16-column block.
template <int P, int MODE>
__global__ __launch_bounds__(256) void apply_kernel(const float *__restrict__ In, int64_t n,
                                                    const float *__restrict__ M, int r,
                                                    uint16_t *__restrict__ out) {
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
    if (j < r) {
      const uint16_t b = ql::f_to_bf16(acc);
      if (MODE == 1) out[i * r + j] = b;
      else out[(int64_t)j * n + i] = b;
    }
  }
}

// ---- host side -----------------------------------------------------------------
struct LoftqWs {
  float *R, *Op, *Yd, *Td, *Zk, *Tk, *part, *MA, *MB;
  double *g1, *g2;
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
  const int64_t P = ql_rup(r, 16), NB = P / 16;
  const int64_t ks = ql_cdiv(k, kKC), ds = ql_cdiv(d, kDC);
  const int64_t nmax = d > k ? d : k;
  const int64_t nch1 = ql_cdiv(nmax, kGramRows), nch2 = ql_cdiv(nmax, orth_rows((int)NB));
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
  L.g1 = carve<double>(base, off, 8 * nch1 * P * P);
  L.g2 = carve<double>(base, off, 8 * nch2 * P * P);
  L.MA = carve<float>(base, off, 4 * P * P);
  L.MB = carve<float>(base, off, 4 * P * P);
  L.bytes = off;
  return L;
}

template <int NB>
struct Loftq {
  static constexpr int P = 16 * NB;
  const LoftqWs &L;
  int64_t d, k;
  hipStream_t st;

  // Y (n x P) from the split partial products, and its partial Gram matrices
  qlora_status reduce_gram(int ns, int64_t n, float *Y) {
    QlProf pf(QLORA_K_LOFTQ_SMALL, st);
    reduce_gram_kernel<P><<<(unsigned)ql_cdiv(n, kGramRows), 256, 0, st>>>(L.part, ns, n, Y, L.g1);
    QL_LAUNCH_CHECK();
    return QLORA_OK;
  }
  qlora_status right(const float *Z, float *Y) {   // Y (d x P) = R Z
    {
      QlProf pf(QLORA_K_LOFTQ_PRODUCT, st);
      mul_right_kernel<NB><<<dim3((unsigned)ql_cdiv(d, 16), (unsigned)ql_cdiv(k, kKC)), 256, 0, st>>>(
          L.R, d, k, Z, L.part);
    }
    QL_LAUNCH_CHECK();
    return reduce_gram((int)ql_cdiv(k, kKC), d, Y);
  }
  qlora_status left(const float *Y, float *Z) {    // Z (k x P) = R^T Y
    {
      QlProf pf(QLORA_K_LOFTQ_PRODUCT, st);
      mul_left_kernel<NB><<<dim3((unsigned)(k / 64), (unsigned)ql_cdiv(d, kDC)), 256, 0, st>>>(
          L.R, d, k, Y, L.part);
    }
    QL_LAUNCH_CHECK();
    return reduce_gram((int)ql_cdiv(d, kDC), k, Z);
  }
  // CholeskyQR2 of Y (whose partial Gram matrices are in g1): the orthonormal
  // basis ends in Y (T: scratch)
  qlora_status orth(float *Y, float *T, int64_t n) {
    const unsigned grid = (unsigned)ql_cdiv(n, orth_rows(NB));
    QlProf pf(QLORA_K_LOFTQ_SMALL, st);
    orth_apply_kernel<P, true><<<grid, 256, 0, st>>>(Y, n, L.g1, (int)ql_cdiv(n, kGramRows), T, L.g2);
    QL_LAUNCH_CHECK();
    orth_apply_kernel<P, false><<<grid, 256, 0, st>>>(T, n, L.g2, (int)grid, Y, nullptr);
    QL_LAUNCH_CHECK();
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
    if ((e = left(L.Yd, L.Zk)) != QLORA_OK) return e;   // Z = R^T Q = C^T, Gram C C^T in g1
    QlProf pf(QLORA_K_LOFTQ_SMALL, st);
    eig_kernel<P><<<1, 64, 0, st>>>(L.g1, (int)ql_cdiv(k, kGramRows), r, s, L.MA, L.MB, sigma);
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
