// NF4 blockwise quantiser and double quantisation of the block absmax values
// for gfx950.
//
// Method (QLoRA glossary, Ultralytics, "QLoRA 的工作原理": NF4 bullet, snippet
// and double-quantisation bullet; Day-25 notes 3.3): per block of 64
// consecutive bf16 weights a = max|w|, each weight gets the code of the level
// nearest to fl32(w / a) (float32 distance, lower code on equal distance);
// then the absmax values are themselves quantised to 8 bits in groups of 256.
//
// Kernel design
//  * quantize_kernel: one lane per 16-byte chunk (8 weights), 8 lanes per
//    block, coalesced 16-byte loads and 4-byte code stores; each lane takes
//    QU chunks 256 lanes apart and issues their loads together. The block absmax
//    is a DPP max over the 8 lanes on the bf16 magnitude bits. The code
//    decision is division-free and bit-exact: the chunk's x is located in
//    one of 65 cells (approximate reciprocal), the cell's single candidate
//    threshold T_j is tested exactly through the sign of
//    fma(-H_j, a, fma(-T_j, a, w)) (H_j = half the gap to the next float32;
//    see gen_tables.py for why this equals fl32(w/a) > T_j for bf16 inputs).
//    Blocks with a < 2^-90 are rescaled by 2^100 first (exact) so no fma
//    underflows.
//  * With double quantisation the kernel also accumulates an exact integer
//    histogram of the bf16 absmax values by exponent (sum of 8-bit
//    significands per exponent): the exact sum of all absmax values, needed
//    for the mean, independent of summation order. Each wave first adds the
//    significands of its blocks per distinct exponent (few: the absmax values
//    of one tensor span few octaves), so the LDS atomics are per wave, not
//    per block; each workgroup then adds its histogram to one of NHC global
//    copies (spreading the atomics over more addresses).
//  * dq_mean_kernel (one workgroup) adds the histogram copies, places them
//    into 384-bit limb sums with LDS atomics (one lane per exponent) and
//    turns the sum into mu = round_f32(sum / nb) by exact long division.
//  * dq_encode_kernel: one workgroup per group of 256 blocks: s2 and the
//    int8 codes of its group.
#include <cstring>

#include <algorithm>

#include "kernels.h"
#include "nf4_tables.h"

namespace {

constexpr int QT = 256;
constexpr int QU = 2;      // chunks per lane (measured: 8 -> 19.0 us, 4 -> 16.4, 2 -> 15.6, 1 -> 17.5 at 4096x4096)
constexpr int NHC = 64;    // global histogram copies (workgroup b adds to copy b % NHC)

// Cell table entry: the candidate threshold T_j and the bits of H_j with j in
// the low four mantissa bits (every H_j is a power of two, so those bits are
// zero in H_j itself): 8 bytes, one ds_read_b64 per weight.
struct __align__(8) Cell {
  float T;
  uint32_t Hj;
};

__constant__ uint32_t c_thresh[15] = NF4_THRESH_BITS;
__constant__ uint32_t c_halfgap[15] = NF4_HALFGAP_BITS;
__constant__ uint8_t c_cell[NF4_NCELL] = NF4_CELL_THRESH;

QL_DEV uint32_t max8_dpp(uint32_t v) {
  // quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror: max over 8 lanes
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));
  return v;
}

// Codes of 8 bf16 weights (u[0] low half = first weight) of a block with
// absmax a, packed as 4 bytes (even element in the high nibble).
template <bool RESCALE>
QL_DEV uint32_t encode8(const uint32_t u[4], float a, const Cell *cell) {
  float aa = (a == 0.0f) ? 1.0f : a;
  float sw = 1.0f;
  if (RESCALE && a < 0x1p-90f) {
    aa = a * 0x1p100f;
    sw = 0x1p100f;
  }
  // 32 / aa as the reciprocal of aa / 32 (exact scaling), which stays a
  // normal float32 for aa up to the largest bf16
  const float r32 = __builtin_amdgcn_rcpf(aa * 0x1p-5f);
  uint32_t packed = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t word = u[e >> 1];
    float w = (e & 1) ? ql::bf16hi(word) : ql::bf16lo(word);
    if (RESCALE) w *= sw;
    const float qx = fmaf(w, r32, 32.0f);
    int c = (int)qx;
    c = min(max(c, 0), NF4_NCELL - 1);
    const Cell ce = cell[c];
    const float dd = fmaf(-ce.T, aa, w);
    const float ee = fmaf(-__uint_as_float(ce.Hj & ~15u), aa, dd);
    const uint32_t code = (ce.Hj & 15u) + (ee > 0.0f ? 1u : 0u);
    packed |= code << (8 * (e >> 1) + ((e & 1) ? 0 : 4));
  }
  return (a == 0.0f) ? 0x77777777u : packed;
}

template <bool DQ>
__global__ __launch_bounds__(QT) void quantize_kernel(
    const uint4 *__restrict__ W, uint32_t *__restrict__ codes,
    float *__restrict__ absmax_out, unsigned long long *__restrict__ hist,
    int64_t nchunks) {
  __shared__ Cell cell[NF4_NCELL];
  // 8 private 32-bit copies of the histogram, one per block-leader slot of a
  // wave (lanes 0, 8, .., 56), so the LDS atomics rarely collide; a copy
  // receives at most 16 significands (< 2^12) per workgroup
  __shared__ uint32_t lh8[8][256];
  const int tid = threadIdx.x;
  if (tid < NF4_NCELL) {
    const int j = c_cell[tid];
    cell[tid].T = __uint_as_float(c_thresh[j]);
    cell[tid].Hj = c_halfgap[j] | (uint32_t)j;
  }
  if (DQ)
#pragma unroll
    for (int i = 0; i < 8; ++i) lh8[i][tid] = 0u;
  const int64_t base = (int64_t)blockIdx.x * (QT * QU) + tid;
  // the QU chunks of this lane, loads first; n % 64 == 0, so the 8 lanes of
  // a block agree on validity
  uint4 v[QU];
#pragma unroll
  for (int u = 0; u < QU; ++u) {
    const int64_t ch = base + u * QT;
    v[u] = ch < nchunks ? W[ch] : make_uint4(0u, 0u, 0u, 0u);
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < QU; ++u) {
    const int64_t ch = base + u * QT;
    const uint32_t w4[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) m = max(m, max(w4[i] & 0x7fffu, (w4[i] >> 16) & 0x7fffu));
    const uint32_t mb = max8_dpp(m);
    const float a = __uint_as_float(mb << 16);
    uint32_t packed;
    if (__builtin_expect(__any(a < 0x1p-90f && a > 0.0f), 0))
      packed = encode8<true>(w4, a, cell);
    else
      packed = encode8<false>(w4, a, cell);
    const bool ok = ch < nchunks;
    if (ok) codes[ch] = packed;
    const bool leader = ok && (ch & 7) == 0;
    if (leader) absmax_out[ch >> 3] = a;
    if (DQ) {
      const uint32_t t = mb >> 7, man = mb & 0x7fu;
      const uint32_t sig = t ? (man | 0x80u) : man;
      if (leader && sig) atomicAdd(&lh8[(tid >> 3) & 7][t ? t : 1u], sig);
    }
  }
  if (DQ) {
    __syncthreads();
    unsigned long long h = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) h += lh8[i][tid];
    if (h) atomicAdd(&hist[(blockIdx.x % NHC) * 256 + tid], h);
  }
}

// one thread per word
__global__ void zero_u64_kernel(unsigned long long *p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0ull;
}

// mu = nearest float32 (ties to even) of N / nb, N the numerator in units of
// 2^-197 scaled by 2^64, held as 12 32-bit limbs whose sums `limb` still lack
// their carries. Executed by one lane. The long division goes 16 bits at a
// time in fp64: each partial dividend r * 2^16 + d (r < nb < 2^32) is below
// 2^48 and exact, the quotient is below 2^16, and an integer quotient k - e
// (e >= 1/nb) sits more than 2^-48 relatively below k, so the correctly
// rounded fp64 quotient never reaches k: its floor is the integer quotient.
QL_DEV float mean_from_limbs(const unsigned long long *limb, uint32_t *sq, uint32_t nb) {
  uint32_t N[12];
  unsigned long long carry = 0;
  bool nonzero = false;
#pragma unroll
  for (int i = 0; i < 12; ++i) {
    const unsigned long long s = limb[i] + carry;
    N[i] = (uint32_t)s;
    carry = s >> 32;
    nonzero |= N[i] != 0u;
  }
  if (!nonzero || nb == 0) return 0.0f;
  const double dn = (double)nb;
  uint32_t Q[12];
  unsigned long long rem = 0;
#pragma unroll
  for (int i = 11; i >= 0; --i) {
    uint32_t qw = 0;
    if (rem != 0 || N[i] != 0u) {
      const double c1 = (double)((rem << 16) | (N[i] >> 16));
      const double q1 = floor(c1 / dn);
      const double c2 = (c1 - q1 * dn) * 65536.0 + (double)(N[i] & 0xFFFFu);
      const double q2 = floor(c2 / dn);
      rem = (unsigned long long)(c2 - q2 * dn);
      qw = ((uint32_t)q1 << 16) | (uint32_t)q2;
    }
    Q[i] = qw;
    sq[i] = qw;
  }
  int top = 0;
#pragma unroll
  for (int i = 1; i < 12; ++i) if (Q[i]) top = i;
  const int p = 32 * top + 31 - __builtin_clz(sq[top]);
  const int E = p - 197;
  int e_eff = E < -126 ? -126 : E;
  const int sh = e_eff - 23 + 197;  // bit of Q holding the float32 ulp (>= 48)
  const int li = sh >> 5, lb = sh & 31;
  const unsigned long long win = (unsigned long long)sq[li] |
                                 ((unsigned long long)sq[li + 1] << 32);  // li <= 10
  uint32_t mant = (uint32_t)((win >> lb) & 0xFFFFFFull);
  const int g = sh - 1, gl = g >> 5, gb = g & 31;
  const uint32_t gw = sq[gl];
  const uint32_t guard = (gw >> gb) & 1u;
  bool sticky = rem != 0 || (gw & ((1u << gb) - 1u)) != 0u;
#pragma unroll
  for (int i = 0; i < 12; ++i) sticky |= (i < gl) && Q[i] != 0u;
  if (guard && (sticky || (mant & 1u))) ++mant;
  uint32_t bits;
  if (E >= -126) {
    if (mant >> 24) {
      mant >>= 1;
      ++e_eff;
    }
    bits = (e_eff > 127) ? 0x7f800000u
                         : ((uint32_t)(e_eff + 127) << 23) | (mant & 0x7FFFFFu);
  } else {
    bits = mant;  // subnormal (or the smallest normal after rounding up)
  }
  return __uint_as_float(bits);
}

// One workgroup: lane t adds the NHC copies of bucket t (sum of 8-bit
// significands of the absmax values with bf16 exponent field t, subnormals in
// bucket 1) and adds h * 2^(t-1+64) into the limb sums with LDS atomics.
__global__ __launch_bounds__(256) void dq_mean_kernel(const unsigned long long *__restrict__ hist,
                                                     uint32_t nb, float *__restrict__ mu_out) {
  __shared__ unsigned long long limb[12];
  __shared__ uint32_t sq[12];
  const int tid = threadIdx.x;
  if (tid < 12) limb[tid] = 0ull;
  unsigned long long hc[NHC];
#pragma unroll
  for (int c = 0; c < NHC; ++c) hc[c] = hist[c * 256 + tid];
  unsigned long long h = 0;
#pragma unroll
  for (int c = 0; c < NHC; ++c) h += hc[c];
  __syncthreads();
  if (tid >= 1 && h != 0ull) {
    // h < 2^48, shift <= 318: three limbs, the last one <= 11
    const int sh = tid - 1 + 64, li = sh >> 5, bit = sh & 31;
    const unsigned long long lo = h << bit;
    atomicAdd(&limb[li], lo & 0xFFFFFFFFull);
    atomicAdd(&limb[li + 1], lo >> 32);
    if (bit) atomicAdd(&limb[li + 2], h >> (64 - bit));
  }
  __syncthreads();
  if (tid == 0) mu_out[0] = mean_from_limbs(limb, sq, nb);
}

__global__ __launch_bounds__(256) void dq_encode_kernel(
    const float *__restrict__ absmax, int64_t nb, const float *__restrict__ mu_p,
    int8_t *__restrict__ q, float *__restrict__ s2) {
  __shared__ uint32_t wmax[4];
  const int tid = threadIdx.x;
  const int64_t b = (int64_t)blockIdx.x * 256 + tid;
  const float mu = mu_p[0];
  float d = 0.0f;
  if (b < nb) d = absmax[b] - mu;
  uint32_t m = __float_as_uint(fabsf(d));
  for (int off = 32; off > 0; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
  if ((tid & 63) == 0) wmax[tid >> 6] = m;
  __syncthreads();
  const uint32_t gm = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
  const float sc = __uint_as_float(gm) / 127.0f;
  if (tid == 0) s2[blockIdx.x] = sc;
  if (b < nb) {
    int qi = 0;
    if (sc != 0.0f) {
      float r = rintf(d / sc);
      r = fminf(fmaxf(r, -127.0f), 127.0f);
      qi = (int)r;
    }
    q[b] = (int8_t)qi;
  }
}

}  // namespace

size_t quantize_ws_bytes(int64_t n, int dq) {
  if (!dq) return 0;
  const int64_t nb = n / 64;
  return (size_t)(ql_rup(4 * nb, 256) + NHC * 256 * 8);
}

qlora_status launch_quantize(const uint16_t *W0, int64_t n, uint8_t *codes,
                             float *absmax_out, int dq, int8_t *q, float *s2,
                             float *mu, void *ws, hipStream_t st) {
  const int64_t nchunks = n / 8, nb = n / 64;
  const int64_t grid = ql_cdiv(nchunks, QT * QU);
  if (!dq) {
    QlProf prof(QLORA_K_QUANTIZE, st);
    quantize_kernel<false><<<(unsigned)grid, QT, 0, st>>>((const uint4 *)W0, (uint32_t *)codes,
                                                 absmax_out, nullptr, nchunks);
    QL_LAUNCH_CHECK();
    return QLORA_OK;
  }
  float *amax = (float *)ws;
  unsigned long long *hist = (unsigned long long *)((char *)ws + ql_rup(4 * nb, 256));
  zero_u64_kernel<<<NHC, 256, 0, st>>>(hist, NHC * 256);
  {
    QlProf prof(QLORA_K_QUANTIZE, st);
    quantize_kernel<true><<<(unsigned)grid, QT, 0, st>>>((const uint4 *)W0, (uint32_t *)codes, amax,
                                                hist, nchunks);
  }
  {
    QlProf prof(QLORA_K_DOUBLE_QUANT, st);
    dq_mean_kernel<<<1, 256, 0, st>>>(hist, (uint32_t)nb, mu);
    dq_encode_kernel<<<(unsigned)ql_cdiv(nb, 256), 256, 0, st>>>(amax, nb, mu, q, s2);
  }
  QL_LAUNCH_CHECK();
  return QLORA_OK;
}

void host_codebook(float levels[16], float thresholds[15]) {
  static const uint32_t lv[16] = NF4_LEVEL_BITS;
  static const uint32_t th[15] = NF4_THRESH_BITS;
  for (int i = 0; i < 16; ++i) std::memcpy(&levels[i], &lv[i], 4);
  for (int i = 0; i < 15; ++i) std::memcpy(&thresholds[i], &th[i], 4);
}
