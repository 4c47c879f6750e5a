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
//    block, coalesced 16-byte loads and 4-byte code stores. The block absmax
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
//    for the mean, independent of summation order.
//  * dq_mean_kernel turns the histogram into mu = round_f32(sum / nb) with a
//    384-bit integer division (one lane; the kernel is tiny).
//  * dq_encode_kernel: one workgroup per group of 256 blocks.
#include <cstring>

#include <algorithm>

#include "kernels.h"
#include "nf4_tables.h"

namespace {

constexpr int QT = 256;
constexpr int kMaxQuantGrid = 2048;

struct __align__(16) Cell {
  float T, H;
  uint32_t base, pad;
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
  const float r32 = 32.0f * __builtin_amdgcn_rcpf(aa);
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
    const float ee = fmaf(-ce.H, aa, dd);
    const uint32_t code = ce.base + (ee > 0.0f ? 1u : 0u);
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
  __shared__ unsigned long long lhist[256];
  const int tid = threadIdx.x;
  if (tid < NF4_NCELL) {
    const int j = c_cell[tid];
    cell[tid].T = __uint_as_float(c_thresh[j]);
    cell[tid].H = __uint_as_float(c_halfgap[j]);
    cell[tid].base = (uint32_t)j;
    cell[tid].pad = 0;
  }
  if (DQ) lhist[tid] = 0;
  __syncthreads();

  const int64_t stride = (int64_t)gridDim.x * QT;
  for (int64_t base = (int64_t)blockIdx.x * QT; base < nchunks; base += stride) {
    const int64_t ch = base + tid;
    if (ch < nchunks) {  // n % 64 == 0: the 8 lanes of a block agree
      const uint4 v = W[ch];
      const uint32_t u[4] = {v.x, v.y, v.z, v.w};
      uint32_t m = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        m = max(m, max(u[i] & 0x7fffu, (u[i] >> 16) & 0x7fffu));
      const uint32_t mb = max8_dpp(m);
      const float a = __uint_as_float(mb << 16);
      uint32_t packed;
      if (__builtin_expect(__any(a < 0x1p-90f && a > 0.0f), 0))
        packed = encode8<true>(u, a, cell);
      else
        packed = encode8<false>(u, a, cell);
      codes[ch] = packed;
      if ((ch & 7) == 0) {
        absmax_out[ch >> 3] = a;
        if (DQ) {
          const uint32_t t = mb >> 7, man = mb & 0x7fu;
          const uint32_t sig = t ? (man | 0x80u) : man;
          if (sig) atomicAdd(&lhist[t ? t : 1], (unsigned long long)sig);
        }
      }
    }
  }
  if (DQ) {
    __syncthreads();
    const unsigned long long h = lhist[tid];
    if (h) atomicAdd(&hist[tid], h);
  }
}

__global__ void zero_u64_kernel(unsigned long long *p, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0ull;
}

// mu = nearest float32 (ties to even) of sum_t hist[t] * 2^(t-134) / nb.
__global__ void dq_mean_kernel(const unsigned long long *__restrict__ hist,
                               uint32_t nb, float *__restrict__ mu_out) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  // numerator N * 2^64 in 2^-197 units, 384 bits in 32-bit limbs
  uint32_t N[12];
  for (int i = 0; i < 12; ++i) N[i] = 0u;
  for (int t = 1; t < 256; ++t) {
    const unsigned long long h = hist[t];
    if (!h) continue;
    const int sh = t - 1 + 64;
    int li = sh >> 5;
    const int bit = sh & 31;
    // h < 2^48; h << bit spans at most 3 limbs
    unsigned long long lo = h << bit;
    uint32_t part[3] = {(uint32_t)lo, (uint32_t)(lo >> 32),
                        (uint32_t)(bit ? (h >> (64 - bit)) : 0ull)};
    unsigned long long carry = 0;
    for (int j = 0; li + j < 12; ++j) {
      const unsigned long long add = (j < 3 ? part[j] : 0u);
      if (j >= 3 && carry == 0) break;
      const unsigned long long s = (unsigned long long)N[li + j] + add + carry;
      N[li + j] = (uint32_t)s;
      carry = s >> 32;
    }
  }
  bool nonzero = false;
  for (int i = 0; i < 12; ++i) nonzero |= (N[i] != 0u);
  if (!nonzero || nb == 0) {
    mu_out[0] = 0.0f;
    return;
  }
  uint32_t Q[12];
  unsigned long long rem = 0;
  for (int i = 11; i >= 0; --i) {
    const unsigned long long cur = (rem << 32) | N[i];
    Q[i] = (uint32_t)(cur / nb);
    rem = cur % nb;
  }
  int p = -1;
  for (int i = 11; i >= 0 && p < 0; --i)
    if (Q[i]) p = 32 * i + 31 - __builtin_clz(Q[i]);
  const int E = p - 197;
  int e_eff = E < -126 ? -126 : E;
  const int sh = e_eff - 23 + 197;  // bit of Q holding the float32 ulp (>= 9)
  auto bit_at = [&](int b) -> uint32_t { return (Q[b >> 5] >> (b & 31)) & 1u; };
  const int li = sh >> 5, lb = sh & 31;
  unsigned long long win = (unsigned long long)Q[li] |
                           ((li + 1 < 12) ? ((unsigned long long)Q[li + 1] << 32) : 0ull);
  uint32_t mant = (uint32_t)((win >> lb) & 0xFFFFFFull);
  const uint32_t guard = bit_at(sh - 1);
  bool sticky = rem != 0;
  for (int b = 0; b < sh - 1 && !sticky; ++b) sticky = bit_at(b) != 0u;
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
  mu_out[0] = __uint_as_float(bits);
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
  return (size_t)(ql_rup(4 * nb, 256) + 256 * 8);
}

qlora_status launch_quantize(const uint16_t *W0, int64_t n, uint8_t *codes,
                             float *absmax_out, int dq, int8_t *q, float *s2,
                             float *mu, void *ws, hipStream_t st) {
  const int64_t nchunks = n / 8, nb = n / 64;
  const int grid = (int)std::min<int64_t>(ql_cdiv(nchunks, QT), kMaxQuantGrid);
  if (!dq) {
    QlProf prof(QLORA_K_QUANTIZE, st);
    quantize_kernel<false><<<grid, QT, 0, st>>>((const uint4 *)W0, (uint32_t *)codes,
                                                 absmax_out, nullptr, nchunks);
    QL_LAUNCH_CHECK();
    return QLORA_OK;
  }
  float *amax = (float *)ws;
  unsigned long long *hist = (unsigned long long *)((char *)ws + ql_rup(4 * nb, 256));
  zero_u64_kernel<<<1, 256, 0, st>>>(hist, 256);
  {
    QlProf prof(QLORA_K_QUANTIZE, st);
    quantize_kernel<true><<<grid, QT, 0, st>>>((const uint4 *)W0, (uint32_t *)codes, amax,
                                                hist, nchunks);
  }
  {
    QlProf prof(QLORA_K_DOUBLE_QUANT, st);
    dq_mean_kernel<<<1, 64, 0, st>>>(hist, (uint32_t)nb, mu);
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
