// Merge of the LoRA update into the dequantised base, gfx950.
//
// Day-25 notes 2.6 (W_merged = W0 + B A) and 6.2 (scale alpha/r); LLM
// tutorial ch. 3, 3.8 and QLoRA glossary "权衡": a 4-bit base is dequantised
// to 16 bits before merging. Here
//     W_m = bf16(fl(w' + fl(s * (B A)[j][c])))
// with w' the bf16 dequantised weight and the rank-r product summed in
// float32 (exact bf16 products, MFMA accumulation order).
//
// Workgroup tile: 4 waves x 32 rows, MC = 128 columns (256- and 64-column
// tiles measured 10% and 15% slower per call at 4096x4096).
//  * A^T of the tile's columns (all ranks, zero-padded to a multiple of 16)
//    is staged once in LDS, each thread writing rank pairs as 4-byte words;
//    the column pitch (2 rp + 16 bytes, an odd number of 16-byte slots) keeps
//    the operand reads conflict-free.
//  * Each wave keeps the B entries of its 32 rows in registers (one 16-byte
//    load per rank chunk when r % 8 == 0, as the whole-piece loads cut the
//    call by 8%) and walks the
//    tile in 32-column blocks: 32x32x16 bf16 MFMAs give D[c][j] = (B A)[j][c]
//    with lane (j, h) holding columns 8g + 4h .. 8g + 4h + 3 (g = 0..3) of
//    row j, exactly the columns whose code nibbles it reads, so the update is
//    applied straight from the accumulators: level lookup, block scale, bf16
//    rounding, add s (B A), round. The bf16 results pass through a per-wave
//    LDS staging area so that the global stores are whole 128-byte lines.
//  * All global loads of a wave (its rows' code words and block-scale
//    inputs for the whole tile, its B rows) are issued before the barrier.
// HBM traffic per weight: 0.5 code byte + scale share in, 2 bytes out; A is
// read once per 128 rows.
#include "kernels.h"
#include "nf4_tables.h"

namespace {

constexpr int MC = 128, MT = 256, MNB = MC / 32;  // tile columns, threads, column blocks
constexpr int MAXRP = 128;
__constant__ uint32_t c_levels_m[16] = NF4_LEVEL_BITS;

struct MergeArgs {
  const uint8_t *codes;
  ql::ScaleSrc sc;
  int64_t d, k;
  const uint16_t *A, *B;
  int r, rp;
  float s;
  uint16_t *Wm;
};

// MQ (double quantisation with k % 128 == 0): the tile's two 64-column
// blocks of a row have adjacent int8 codes at an even index (c0 / 64 is
// even), read as one 2-byte load, and share one s2 (an even block index is
// never the last of its 256-block group).
template <bool DQ, int NCH, bool MQ>
__global__ __launch_bounds__(MT) void merge_kernel(MergeArgs g) {
  constexpr int RP = 16 * NCH;            // padded rank
  constexpr int PITCH = 2 * RP + 16;      // bytes per A^T column
  __shared__ __align__(16) unsigned char s_at[MC * PITCH];
  __shared__ __align__(16) unsigned char s_stg[4 * 32 * 128];  // per-wave output staging
  __shared__ float s_lv[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int64_t c0 = (int64_t)blockIdx.x * MC;
  const int64_t j = (int64_t)blockIdx.y * 128 + 32 * wave + l32;  // this lane's row
  const int64_t jc = min(j, g.d - 1);
  if (tid < 16) s_lv[tid] = __uint_as_float(c_levels_m[tid]);

  // 1. A^T chunk loads, one 16-rank chunk per pass: thread (rank pair
  //    tp = tid % 8, 8-column segment tid / 8) loads ranks 16 ch + 2tp, +1 of
  //    columns 8 seg .. +7 (threads past MC repeat a segment; they write
  //    nothing)
  uint4 av[NCH][2];
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch) {
    const int t = 16 * ch + 2 * (tid & 7);
    const int64_t col = c0 + 8 * ((tid >> 3) & (MC / 8 - 1));
    av[ch][0] = ql::zero4();
    av[ch][1] = ql::zero4();
    if (col < g.k) {  // k % 64 == 0: the 8 columns are all in range
      const uint16_t *src = g.A + (int64_t)t * g.k + col;
      if (t < g.r) av[ch][0] = *(const uint4 *)src;
      if (t + 1 < g.r) av[ch][1] = *(const uint4 *)(src + g.k);
    }
  }
  // 2. this lane's code words: row j, 32-column block b = 16 bytes (clamped
  //    in range; results of rows past d or columns past k are not stored)
  const int64_t kb = g.k >> 1;  // code bytes per row
  uint4 cw[MNB];
#pragma unroll
  for (int b = 0; b < MNB; ++b)
    cw[b] = *(const uint4 *)(g.codes + jc * kb + min(c0 / 2 + 16 * b, kb - 16));
  // block scales: 32-column block b lies in 64-column block (c0 + 32 b) / 64
  float sa[MNB / 2], sb[MNB / 2];
  const int64_t nbr = g.k >> 6;
  if (DQ && MQ) {
    static_assert(MNB / 2 == 2, "two 64-column blocks per tile");
    const int64_t blk = jc * nbr + min(c0 / 64, nbr - 2);
    const uint32_t q2 = *(const uint16_t *)(g.sc.q + blk);
    sa[0] = (float)(int8_t)(q2 & 0xFFu);
    sa[1] = (float)(int8_t)(q2 >> 8);
    sb[0] = sb[1] = g.sc.s2[blk >> 8];
  } else {
#pragma unroll
    for (int b2 = 0; b2 < MNB / 2; ++b2) {
      const int64_t blk = jc * nbr + min(c0 / 64 + b2, nbr - 1);
      if (DQ) {
        sa[b2] = (float)g.sc.q[blk];
        sb[b2] = g.sc.s2[blk >> 8];
      } else {
        sa[b2] = g.sc.absmax[blk];
      }
    }
  }
  const float mu = DQ ? g.sc.mu[0] : 0.0f;
  // B entries of row j, ranks 16 ch + 8h .. +7 (ranks past r are zero)
  uint32_t bw[NCH][4];
  if (g.r % 8 == 0) {
    // whole 16-byte pieces: ranks 16 ch + 8h .. +7 of row j, one load each
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
      const int t = 16 * ch + 8 * h;
      const uint4 v = *(const uint4 *)(g.B + jc * g.r + (t < g.r ? t : g.r - 8));
      const bool ok = t < g.r;
      bw[ch][0] = ok ? v.x : 0u; bw[ch][1] = ok ? v.y : 0u;
      bw[ch][2] = ok ? v.z : 0u; bw[ch][3] = ok ? v.w : 0u;
    }
  } else {
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * ch + 8 * h + 2 * i;
        uint32_t lo = 0, hi = 0;
        if (t < g.r) lo = g.B[jc * g.r + t];
        if (t + 1 < g.r) hi = g.B[jc * g.r + t + 1];
        bw[ch][i] = lo | (hi << 16);
      }
  }
  // 3. A^T to LDS: column c at c * PITCH, rank t at byte 2t
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch) {
    if (tid >= MC) break;   // MC / 8 segments of 8 columns, 8 rank pairs each
    const int t = 16 * ch + 2 * (tid & 7), seg = tid >> 3;
    const uint32_t v0[4] = {av[ch][0].x, av[ch][0].y, av[ch][0].z, av[ch][0].w};
    const uint32_t v1[4] = {av[ch][1].x, av[ch][1].y, av[ch][1].z, av[ch][1].w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t lo = (v0[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
      const uint32_t hi = (v1[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
      *(uint32_t *)(s_at + (8 * seg + i) * PITCH + 2 * t) = lo | (hi << 16);
    }
  }
  __syncthreads();

  // 4. per pair of 32-column blocks: D[c][j] on MFMA, the merged outputs into
  //    the wave's staging rows (16-byte chunks XOR-swizzled by row), then
  //    read back as whole rows and stored 16 bytes per lane (a wave store =
  //    8 rows x 128 bytes). LDS accesses of a wave execute in order, so the
  //    staging needs no barrier.
  unsigned char *stg = s_stg + wave * (32 * 128);
  const int64_t jw = (int64_t)blockIdx.y * 128 + 32 * wave;  // first row of the wave
#pragma unroll
  for (int pb = 0; pb < MNB / 2; ++pb) {
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
      const int b = 2 * pb + bb;
      f32x16 acc;
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
      for (int ch = 0; ch < NCH; ++ch) {
        // A operand: A^T[c = 32 b + l32][ranks 16 ch + 8h ..]; B operand: B[j][same ranks]
        const uint4 aop = *(const uint4 *)(s_at + (32 * b + l32) * PITCH + 32 * ch + 16 * h);
        const uint4 bop = make_uint4(bw[ch][0], bw[ch][1], bw[ch][2], bw[ch][3]);
        acc = ql::mfma32(aop, bop, acc);
      }
      // lane (row l32, h) holds D[8 gq + 4h + e][l32], columns 32 b + 8 gq + 4h + e
      const float ap = DQ ? sa[pb] * sb[pb] + mu : sa[pb];
      const uint32_t cwords[4] = {cw[b].x, cw[b].y, cw[b].z, cw[b].w};
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        // code bytes 4 gq + 2h, +1: columns 8 gq + 4h .. +3 (even element high nibble)
        const uint32_t c16 = (cwords[gq] >> (16 * h)) & 0xFFFFu;
        float o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int sh = 8 * (e >> 1) + ((e & 1) ? 0 : 4);
          const float wq = ql::bf16_to_f(ql::f_to_bf16(s_lv[(c16 >> sh) & 15u] * ap));
          o[e] = wq + g.s * acc[4 * gq + e];
        }
        const int chunk = (4 * bb + gq) ^ (l32 & 7);
        *(uint2 *)(stg + l32 * 128 + 16 * chunk + 8 * h) =
            make_uint2(ql::pack_bf16x2(o[0], o[1]), ql::pack_bf16x2(o[2], o[3]));
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = 8 * i + (lane >> 3), c = lane & 7;
      const uint4 v = *(const uint4 *)(stg + rr * 128 + 16 * (c ^ (rr & 7)));
      const int64_t row = jw + rr, col = c0 + 64 * pb + 8 * c;
      if (row < g.d && col < g.k) *(uint4 *)(g.Wm + row * g.k + col) = v;
    }
  }
}

}  // namespace

qlora_status launch_merge(const uint8_t *codes, ql::ScaleSrc sc, int64_t d, int64_t k,
                          const uint16_t *A, const uint16_t *B, int r, float s, uint16_t *Wm,
                          hipStream_t st) {
  const int nch = (r + 15) / 16;
  if (nch < 1 || 16 * nch > MAXRP) return QLORA_ERR_UNSUPPORTED;
  const int64_t gx = ql_cdiv(k, MC), gy = ql_cdiv(d, 128);
  if (gy > 65535 || gx > 0x7fffffff) return QLORA_ERR_UNSUPPORTED;
  MergeArgs g{codes, sc, d, k, A, B, r, 16 * nch, s, Wm};
  dim3 grid((unsigned)gx, (unsigned)gy);
  QlProf prof(QLORA_K_MERGE, st);
#define QL_MERGE(NCHV)                                                 \
  if (sc.dq && mq)                                                     \
    merge_kernel<true, NCHV, true><<<grid, MT, 0, st>>>(g);            \
  else if (sc.dq)                                                      \
    merge_kernel<true, NCHV, false><<<grid, MT, 0, st>>>(g);           \
  else                                                                 \
    merge_kernel<false, NCHV, false><<<grid, MT, 0, st>>>(g);
  const bool mq = (k % 128) == 0;
  switch (nch) {
    case 1: QL_MERGE(1) break;
    case 2: QL_MERGE(2) break;
    case 3: QL_MERGE(3) break;
    case 4: QL_MERGE(4) break;
    case 5: QL_MERGE(5) break;
    case 6: QL_MERGE(6) break;
    case 7: QL_MERGE(7) break;
    default: QL_MERGE(8) break;
  }
#undef QL_MERGE
  QL_LAUNCH_CHECK();
  return QLORA_OK;
}
