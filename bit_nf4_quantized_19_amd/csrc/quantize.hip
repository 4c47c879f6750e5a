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
//    QU chunks 256 lanes apart per tile, and a workgroup (8 per CU) loops over
//    tiles with the next tile's loads issued before the current tile is
//    coded, so the table and the LDS histogram are set up once per
//    workgroup and the loads stream without gaps. The block absmax
//    is a DPP max over the 8 lanes on the bf16 magnitude bits. The code
//    decision is division-free and bit-exact: the chunk's x is located in
//    one of 65 cells (approximate reciprocal), the cell's single candidate
//    threshold T_j is tested exactly through the sign of
//    fma(-H_j, a, fma(-T_j, a, w)) (H_j = half the gap to the next float32;
//    see gen_tables.py for why this equals fl32(w/a) > T_j for bf16 inputs).
//    Blocks with a < 2^-90 are rescaled by 2^100 first (exact) so no fma
//    underflows; they and blocks with an infinite or NaN absmax take a form
//    that also clamps the cell index, which the others do not need.
//  * With double quantisation the kernel also accumulates an exact integer
//    histogram of the bf16 absmax values by exponent (sum of 8-bit
//    significands per exponent): the exact sum of all absmax values, needed
//    for the mean, independent of summation order. Each wave first adds the
//    significands of its blocks per distinct exponent (few: the absmax values
//    of one tensor span few octaves), so the LDS atomics are per wave, not
//    per block; each workgroup then adds its histogram to one of NHC global
//    copies (spreading the atomics over more addresses).
//  * dq_encode_kernel: every workgroup adds the histogram copies, places
//    them into 384-bit limb sums with LDS atomics (one lane per exponent),
//    turns the sum into mu = round_f32(sum / nb) by exact long division (the
//    same value in every workgroup), then computes s2 and the int8 codes of
//    its GPW groups of 256 blocks: the double quantisation is one launch
//    after the quantiser (plus the histogram clear before it).
#include <cstring>

#include <algorithm>

#include "kernels.h"
#include "nf4_tables.h"

namespace {

constexpr int QT = 256;
// Tile = QU chunks per lane (QT QU chunks); QWPC workgroups per CU loop over
// the tiles with the next tile's loads in flight. Measured quantise + DQ call
// (4096x4096 / 22016x8192, us): one workgroup per tile, QU = 2: 24.1 / 131;
// persistent QU = 2, 8 per CU: 23.2 / 121 (4 per CU 23.5 / 124, 2 per CU
// 25.5 / 149; QU = 1 or 4 within 2% at 8 per CU).
constexpr int QU = 2;
constexpr int QWPC = 8;
constexpr int NHC = 8;     // global histogram copies (workgroup b adds to copy b % NHC)
constexpr int GPW = 8;     // double-quant groups per encode workgroup

// Cell table entry: the candidate threshold T_j and the bits of H_j with j in
// the low four mantissa bits (every H_j is a power of two, so those bits are
// zero in H_j itself): 8 bytes, one ds_read_b64 per weight. (A 16-byte entry
// with j apart, two masking operations fewer per weight, measured 8% slower:
// the table reads, not the ALU, set the pace.)
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
// absmax a, packed as 4 bytes (even element in the high nibble). For a
// finite block with a >= 2^-90 every |w| <= a, so fl(w r32 + 32) lies in
// [0, 65) (r32 is within one ulp of 32 / a) and the cell index needs no
// clamp; the SAFE form (blocks with tiny, infinite or NaN absmax) rescales
// tiny blocks and clamps the index.
template <bool SAFE>
QL_DEV uint32_t encode8(const uint32_t u[4], float a, const Cell *cell) {
  float aa = (a == 0.0f) ? 1.0f : a;
  float sw = 1.0f;
  if (SAFE && a < 0x1p-90f) {
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
    if (SAFE) w *= sw;
    const float qx = fmaf(w, r32, 32.0f);
    int c = (int)qx;
    if (SAFE) c = min(max(c, 0), NF4_NCELL - 1);
    const Cell ce = cell[c];
    const float dd = fmaf(-ce.T, aa, w);
    const float ee = fmaf(-__uint_as_float(ce.Hj & ~15u), aa, dd);
    const uint32_t code = (ce.Hj & 15u) + (ee > 0.0f ? 1u : 0u);
    packed |= code << (8 * (e >> 1) + ((e & 1) ? 0 : 4));
  }
  return (a == 0.0f) ? 0x77777777u : packed;
}

// Loads of tile t: chunk t * QT * QU + tid + u * QT for u < QU, at a clamped
// index (a chunk past the end is never stored).
QL_DEV void load_tile(const uint4 *__restrict__ W, int64_t nchunks, int64_t t, int tid,
                      uint4 (&v)[QU]) {
  const int64_t base = t * (QT * QU) + tid;
#pragma unroll
  for (int u = 0; u < QU; ++u) v[u] = W[min(base + u * QT, nchunks - 1)];
}

template <bool DQ>
__global__ __launch_bounds__(QT) void quantize_kernel(
    const uint4 *__restrict__ W, uint32_t *__restrict__ codes,
    float *__restrict__ absmax_out, unsigned long long *__restrict__ hist,
    int64_t nchunks, int64_t ntiles) {
  __shared__ Cell cell[NF4_NCELL];
  // 8 private 32-bit copies of the histogram, one per block-leader slot of a
  // wave (lanes 0, 8, .., 56), so the LDS atomics rarely collide; an entry
  // receives at most 4 QU significands (< 2^8 each) per tile, so it holds the
  // sums of up to 2^20 tiles per workgroup
  __shared__ uint32_t lh8[8][256];
  const int tid = threadIdx.x;
  // the first tile's loads go out before the table is set up
  int64_t t = blockIdx.x;
  uint4 v[QU];
  load_tile(W, nchunks, t, tid, v);
  if (tid < NF4_NCELL) {
    const int j = c_cell[tid];
    cell[tid].T = __uint_as_float(c_thresh[j]);
    cell[tid].Hj = c_halfgap[j] | (uint32_t)j;
  }
  if (DQ)
#pragma unroll
    for (int i = 0; i < 8; ++i) lh8[i][tid] = 0u;
  __syncthreads();
  // tiles t, t + G, ...: the next tile's loads are in flight while this one
  // is coded (in the last round they re-read this tile, from cache)
  for (; t < ntiles; t += gridDim.x) {
    uint4 vn[QU];
    load_tile(W, nchunks, t + gridDim.x < ntiles ? t + gridDim.x : t, tid, vn);
    const int64_t base = t * (QT * QU) + tid;
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
      if (__builtin_expect(__any((a < 0x1p-90f && a > 0.0f) || !(a < __builtin_inff())), 0))
        packed = encode8<true>(w4, a, cell);
      else
        packed = encode8<false>(w4, a, cell);
      // n % 64 == 0, so the 8 lanes of a block agree on validity
      const bool ok = ch < nchunks;
      if (ok) codes[ch] = packed;
      const bool leader = ok && (ch & 7) == 0;
      if (leader) absmax_out[ch >> 3] = a;
      if (DQ) {
        const uint32_t e = mb >> 7, man = mb & 0x7fu;
        const uint32_t sig = e ? (man | 0x80u) : man;
        if (leader && sig) atomicAdd(&lh8[(tid >> 3) & 7][e ? e : 1u], sig);
      }
    }
#pragma unroll
    for (int u = 0; u < QU; ++u) v[u] = vn[u];
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
// their carries. Executed by one lane; sq is LDS scratch for the quotient
// limbs (read at run-time positions).
// Long division, 16 quotient bits per step, in fp64: each partial dividend
// c = r * 2^16 + d (r < nb < 2^32) is an integer below 2^48, held exactly.
// The digit is floor(c * (1/nb)) corrected once: the product's relative error
// is below 2^-52 and c / nb < 2^16, so it is within 2^-36 of c / nb and its
// floor is the digit or one off; r' = c - q nb (exact: an integer below
// 2^49) outside [0, nb) moves q by one.
// Only the quotient limbs down to the one holding the guard bit are formed:
// below it the rest of the quotient is nonzero exactly when the running
// remainder or a lower limb of N is, which is all the sticky bit needs.
QL_DEV uint32_t div_digit16(double c, double dn, double inv, double &r) {
  double q = floor(c * inv);
  double rr = fma(-q, dn, c);
  if (rr < 0.0) {
    q -= 1.0;
    rr += dn;
  } else if (rr >= dn) {
    q += 1.0;
    rr -= dn;
  }
  r = rr;
  return (uint32_t)q;
}

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
  const double dn = (double)nb, inv = 1.0 / dn;
  double rem = 0.0;
  bool started = false, done = false, lower = false;
  int E = 0, e_eff = 0, sh = 0, gl = 0;
#pragma unroll
  for (int i = 11; i >= 0; --i) {
    uint32_t qw = 0;
    if (done) {
      lower |= N[i] != 0u;   // a limb below the stop
    } else if (rem != 0.0 || N[i] != 0u) {
      double r1;
      const uint32_t q1 = div_digit16(rem * 65536.0 + (double)(N[i] >> 16), dn, inv, r1);
      const uint32_t q2 = div_digit16(r1 * 65536.0 + (double)(N[i] & 0xFFFFu), dn, inv, rem);
      qw = (q1 << 16) | q2;
    }
    sq[i] = qw;
    if (!done) {
      if (!started && qw != 0u) {
        started = true;
        const int p = 32 * i + 31 - __builtin_clz(qw);
        E = p - 197;
        e_eff = E < -126 ? -126 : E;
        sh = e_eff - 23 + 197;  // bit of the quotient holding the float32 ulp (>= 48)
        gl = (sh - 1) >> 5;     // limb of the guard bit
      }
      if (started && i <= gl) done = true;
    }
  }
  if (!started) return 0.0f;  // N < nb: below 2^-197 (not reachable from bf16 inputs)
  // the stop was at limb gl, or at limb 0 below it (a quotient whose top limb
  // lies under the guard's): formed limbs below the guard's count as they are
  lower |= rem != 0.0;
  for (int j = 0; j < gl; ++j) lower |= sq[j] != 0u;
  const int li = sh >> 5, lb = sh & 31;
  const unsigned long long win = (unsigned long long)sq[li] |
                                 ((unsigned long long)sq[li + 1] << 32);  // li <= 10
  uint32_t mant = (uint32_t)((win >> lb) & 0xFFFFFFull);
  const int gb = (sh - 1) & 31;
  const uint32_t gw = sq[gl];
  const uint32_t guard = (gw >> gb) & 1u;
  const bool sticky = lower || (gw & ((1u << gb) - 1u)) != 0u;
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

// max over the 64 lanes of a wave (every lane gets it): rows of 16 by DPP,
// then the four row maxima by readlane
QL_DEV uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));   // quad [1,0,3,2]
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));   // quad [2,3,0,1]
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));  // half-row mirror
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));  // row mirror
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
  const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return max(max(r0, r1), max(r2, r3));
}

// Double quantisation in one launch. Every workgroup first derives the exact
// mean itself: lane t adds the NHC histogram copies of bucket t (sum of
// 8-bit significands of the absmax values with bf16 exponent field t,
// subnormals in bucket 1) and adds h * 2^(t-1+64) into 384-bit limb sums with
// LDS atomics; lane 0 rounds sum / nb once to float32. Then it encodes GPW
// groups of 256 blocks (all their absmax loads issued first): per group
// s2 = fl(max|a - mu| / 127) and q = clamp(rne(fl((a - mu) / s2)), -127, 127).
__global__ __launch_bounds__(256) void dq_encode_kernel(
    const unsigned long long *__restrict__ hist, const float *__restrict__ absmax, int64_t nb,
    int64_t ng, int8_t *__restrict__ q, float *__restrict__ s2, float *__restrict__ mu_out) {
  __shared__ unsigned long long limb[12];
  __shared__ uint32_t sq[12];
  __shared__ float s_mu;
  __shared__ uint32_t wmax[GPW][4];
  const int tid = threadIdx.x;
  const int64_t g0 = (int64_t)blockIdx.x * GPW;
  // the group loads do not depend on the mean: issue them with the histogram's
  float av[GPW];
#pragma unroll
  for (int j = 0; j < GPW; ++j) {
    const int64_t b = (g0 + j) * 256 + tid;
    av[j] = b < nb ? absmax[b] : 0.0f;
  }
  unsigned long long hc[NHC];
#pragma unroll
  for (int c = 0; c < NHC; ++c) hc[c] = hist[c * 256 + tid];
  if (tid < 12) limb[tid] = 0ull;
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
  if (tid == 0) {
    const float m = mean_from_limbs(limb, sq, (uint32_t)nb);
    s_mu = m;
    if (blockIdx.x == 0) mu_out[0] = m;
  }
  __syncthreads();
  const float mu = s_mu;
  float dv[GPW];
#pragma unroll
  for (int j = 0; j < GPW; ++j) {
    // blocks past nb (the last group's tail) take no part in the group max
    dv[j] = (g0 + j) * 256 + tid < nb ? av[j] - mu : 0.0f;
    const uint32_t m = wave_max_u32(__float_as_uint(fabsf(dv[j])));
    if ((tid & 63) == 0) wmax[j][tid >> 6] = m;
  }
  __syncthreads();
  // group scales, then the codes of all groups (no early exit, so the
  // groups' divisions interleave); blocks past nb are not stored
  float sc[GPW];
#pragma unroll
  for (int j = 0; j < GPW; ++j)
    sc[j] = __uint_as_float(max(max(wmax[j][0], wmax[j][1]), max(wmax[j][2], wmax[j][3]))) / 127.0f;
  if (tid == 0) {
#pragma unroll
    for (int j = 0; j < GPW; ++j)
      if (g0 + j < ng) s2[g0 + j] = sc[j];
  }
#pragma unroll
  for (int j = 0; j < GPW; ++j) {
    int qi = 0;
    if (sc[j] != 0.0f) {
      float r = rintf(dv[j] / sc[j]);
      r = fminf(fmaxf(r, -127.0f), 127.0f);
      qi = (int)r;
    }
    const int64_t b = (g0 + j) * 256 + tid;
    if (b < nb) q[b] = (int8_t)qi;
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
  const int64_t ntiles = ql_cdiv(nchunks, QT * QU);
  const int64_t grid = std::min<int64_t>(ntiles, (int64_t)QWPC * ql_num_cus());
  if (!dq) {
    QlProf prof(QLORA_K_QUANTIZE, st);
    quantize_kernel<false><<<(unsigned)grid, QT, 0, st>>>((const uint4 *)W0, (uint32_t *)codes,
                                                 absmax_out, nullptr, nchunks, ntiles);
    QL_LAUNCH_CHECK();
    return QLORA_OK;
  }
  float *amax = (float *)ws;
  unsigned long long *hist = (unsigned long long *)((char *)ws + ql_rup(4 * nb, 256));
  zero_u64_kernel<<<NHC, 256, 0, st>>>(hist, NHC * 256);
  {
    QlProf prof(QLORA_K_QUANTIZE, st);
    quantize_kernel<true><<<(unsigned)grid, QT, 0, st>>>((const uint4 *)W0, (uint32_t *)codes, amax,
                                                hist, nchunks, ntiles);
  }
  {
    QlProf prof(QLORA_K_DOUBLE_QUANT, st);
    const int64_t ng = ql_cdiv(nb, 256);
    dq_encode_kernel<<<(unsigned)ql_cdiv(ng, GPW), 256, 0, st>>>(hist, amax, nb, ng, q, s2, mu);
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
