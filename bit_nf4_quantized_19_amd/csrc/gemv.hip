// Memory-bound NF4 forward for few tokens (M <= 16), gfx950. Two kernels
// produce the same float32 partial sums: the MFMA kernel below (3 to 16
// tokens, or any count with adapter-input dropout) and a VALU kernel for one
// or two tokens (section "few-token forward on VALU" further down); one
// epilogue kernel finishes both.
//
// Same layer as the fused GEMM (QLoRA glossary, Ultralytics, "QLoRA 的工作原理",
// forward paragraph): Y = X W'^T + s H B^T. With M <= 16 the time is the HBM
// read of the packed codes (0.5 byte per weight), so the kernel reads them in
// whole 128-byte lines, keeps all of a wave's loads in flight at once, and
// spends little VALU per weight:
//   * The per-block scale is factored out of each 64-wide partial sum,
//     sum_b a'_b * sum_{c in b} level[code_c] x_c. The 64-term inner sums run
//     on MFMA (16x16x32 bf16). This equals X W'^T up to float32/bf16 rounding
//     (the weights are rounded to bf16 at the level instead of after the
//     product).
//   * Operand layout: lane (n, q) of a wave (n = lane % 16, q = lane / 16)
//     holds whole blocks 4c + q (c = 0..3) of weight row n, 32 bytes each,
//     read as two 16-byte loads; a pair of load instructions thus covers
//     full 128-byte lines of 16 rows. At MFMA step s the lane supplies codes
//     8s..8s+7 of its block as the B operand (column n). A row m = 4g + t
//     carries token 4 tp + t on the k-slots of lane group g only (zeros
//     elsewhere), so D[4q + t][n] is the partial sum of block 4c + q for that
//     token, held by the lane that owns the block and its scale. The four
//     lane groups of a row are added once at the end.
//   * Decoding: one code byte gives two bf16 levels through a 256-entry LDS
//     table replicated 32 times (entry e, copy c at byte e*256 + 4c). One
//     byte permute builds the address (code byte in bits 8-15, 4*(lane%32)
//     in bits 0-7), and each 32-lane half of a read hits 32 distinct banks.
//   * The X slice (up to 16 tokens x 1024 columns) lives in the upper halves
//     of the table rows, placed so that a lane's A operand for chunk c, step s
//     is at a per-lane base plus an immediate offset; lanes outside their
//     token group read a zero region at the same offsets. No VALU is spent on
//     A addresses.
//   * Work unit: 16 weight rows x one slice of 16 blocks (1024 columns).
//     About one workgroup of 8 waves per compute unit; each workgroup serves
//     one slice (table and X slice built once) and each wave takes up to two
//     units, whose MFMA chains are interleaved. Only their first code chunk
//     is loaded before the table is built; the others go out after the
//     workgroup barrier, one chunk ahead of the decode, so the decode runs
//     while the codes stream in. Partial sums per slice go to a float32
//     buffer; a second kernel adds the slices in a fixed order, the rank-r
//     LoRA term in float32, and rounds to bf16.
#include <algorithm>

#include "kernels.h"
#include "nf4_tables.h"
#include "philox.h"

namespace {

constexpr int GW = 8;            // waves per workgroup, one row group of 16 rows each
constexpr int GT = 64 * GW;
constexpr int GX = 2048 / GT;    // X chunks (16 tokens x 16 blocks x 8) per thread
constexpr int GB = 16;           // blocks per slice (1024 columns)
constexpr int GMAXW = 4;         // weights per grouped call
// Code-load order (see the kernel): GPRE chunks go out before the table is
// built, the rest GLA chunks ahead of the decode. Measured call times at
// 11008x4096 (M = 1 / 16): all four chunks before the table 15.5 / 21.6 us;
// GPRE = 1: 14.1 / 19.7 us (0 and 2 within 2%); GLA = 1: 14.0 / 19.0 us
// (2..3 within 3%).
constexpr int GPRE = 1;   // code chunks issued before the table is built (0..4)
constexpr int GLA = 1;    // chunks of code loads ahead of the chunk being decoded (>= 1)
// LDS: 256 rows of 256 bytes (table copies in bytes 0-127, X in 128-255),
// then the zero region read by lanes outside their token group
constexpr uint32_t ZBASE = 65536 + 64;
constexpr uint32_t ZBYTES = 15 * 256 + 64 + 16;
constexpr int LDS_BYTES = (int)(ZBASE + ZBYTES);
__constant__ uint32_t c_levels_v[16] = NF4_LEVEL_BITS;

// One weight of a grouped call (sibling projections that read the same X).
struct GemvW {
  const uint8_t *codes;
  ql::ScaleSrc sc;
  int64_t d;
  int64_t nb;      // blocks of the weight (d k / 64)
  int64_t gbase;   // first row group of this weight in the grouped numbering
  int64_t rbase;   // first column of this weight in the partial-sum rows
  const uint16_t *Ap;  // LoRA A, rp x k (ranks past r are zero rows)
  float *hpart;    // [S * GW][M][rp]: H = X A^T partial sums per slice and wave
  DropParams dp;   // dropout of X on this weight's adapter input
};

struct GemvArgs {
  GemvW w[GMAXW];
  int nw;          // weights in the call (1..GMAXW)
  int64_t k;
  const uint16_t *X;
  int64_t M;
  int64_t ngroups; // row groups of 16 rows, all weights
  int G;           // workgroups per slice
  int rpw;         // row groups per workgroup, <= 2 GW (the last ones may be past the end)
  float *part;     // [S][M][dtot]: slice partial sums, weights side by side
  int64_t dtot;
  int rp;
};

// Weight i of the call, field by field through uniform selects (a dynamic
// index into the argument block would copy it to scratch memory).
template <class T>
QL_DEV T pick4(int i, T a0, T a1, T a2, T a3) {
  return i == 0 ? a0 : i == 1 ? a1 : i == 2 ? a2 : a3;
}
#define QL_PICK(arr, i, f) pick4(i, arr[0].f, arr[1].f, arr[2].f, arr[3].f)
template <class Args>
QL_DEV GemvW wsel(const Args &g, int i) {
  GemvW W;
  W.codes = QL_PICK(g.w, i, codes);
  W.sc.absmax = QL_PICK(g.w, i, sc.absmax);
  W.sc.q = QL_PICK(g.w, i, sc.q);
  W.sc.s2 = QL_PICK(g.w, i, sc.s2);
  W.sc.mu = QL_PICK(g.w, i, sc.mu);
  W.sc.dq = QL_PICK(g.w, i, sc.dq);
  W.d = QL_PICK(g.w, i, d);
  W.nb = QL_PICK(g.w, i, nb);
  W.gbase = QL_PICK(g.w, i, gbase);
  W.rbase = QL_PICK(g.w, i, rbase);
  W.Ap = QL_PICK(g.w, i, Ap);
  W.hpart = QL_PICK(g.w, i, hpart);
  W.dp.k0 = QL_PICK(g.w, i, dp.k0);
  W.dp.k1 = QL_PICK(g.w, i, dp.k1);
  W.dp.thr = QL_PICK(g.w, i, dp.thr);
  W.dp.inv_keep = QL_PICK(g.w, i, dp.inv_keep);
  W.dp.on = QL_PICK(g.w, i, dp.on);
  W.dp.mask_write = 0;   // the decode path never stores the mask
  W.dp.mask = nullptr;
  return W;
}
template <class Args>
QL_DEV int weight_of(const Args &g, int64_t rg) {
  int i = 0;
#pragma unroll
  for (int j = 1; j < GMAXW; ++j) i += (j < g.nw && rg >= g.w[j].gbase) ? 1 : 0;
  return i;
}

// LDS byte offset of X[token 4 tp + t][slice block 4c + g][8s .. 8s+7]: row
// tp*64 + g*16 + c*4 + s/2, upper half, 16-byte slot (s%2)*4 + t
QL_DEV constexpr uint32_t xa_base(int tp, int g, int t) {
  return (uint32_t)((tp * 64 + g * 16) * 256 + 128 + t * 16);
}
QL_DEV constexpr uint32_t xa_imm(int c, int s) {
  return (uint32_t)((c * 4 + (s >> 1)) * 256 + (s & 1) * 64);
}

// Registers of one work unit (16 rows x one slice) of a wave.
struct GUnit {
  uint4 cw[4][2];   // lane (n, q): blocks 4c + q of row n, 32 bytes each
  uint32_t qw[5];   // int8 scale codes of the row's slice (aligned dwords; QA: qw[0] only)
  float araw[4];    // absmax of blocks 4c + q (no double quantisation)
  float s2lo, s2hi;
  float mu;         // the weight's DQ mean
  int64_t blk0;     // first block of the row's slice
  int64_t row0;     // first row of the unit (in its weight)
  int64_t dlim;     // rows of its weight
  int64_t rbase;    // its weight's first column in the partial-sum rows
  const uint8_t *crow;   // the lane's row codes of this slice
};

// QA: k % 256 == 0, so a row's slice codes start 4-byte aligned and lane
// (n, q) loads just the dword of blocks 4q .. 4q + 3 of its row; the lane
// that needs block 4c + q takes it from lane (n, c) by a shuffle.
template <bool DQ, bool FULL, bool GRP, bool QA>
QL_DEV void unit_load(const GemvArgs &g, GUnit &u, int64_t rg, int64_t b0, int nblk, int n,
                      int q) {
  const int64_t nbr = g.k >> 6;
  // grouped calls pick the unit's weight (rg is wave-uniform)
  const GemvW W = GRP ? wsel(g, weight_of(g, rg)) : g.w[0];
  u.row0 = (rg - W.gbase) * 16;
  u.dlim = W.d;
  u.rbase = W.rbase;
  const int64_t row = min(u.row0 + n, W.d - 1);
  u.blk0 = row * nbr + b0;
  if (DQ) {
    u.mu = W.sc.mu[0];
    u.s2lo = W.sc.s2[u.blk0 >> 8];
    u.s2hi = W.sc.s2[(u.blk0 + nblk - 1) >> 8];
    // the row's int8 codes from the 5 aligned dwords around them (the code
    // array has a multiple of 8 bytes, so a clamped dword index stays in it)
    const uint32_t *qp = (const uint32_t *)W.sc.q;
    const int64_t w0 = u.blk0 >> 2, wlast = (W.nb >> 2) - 1;
    if (QA) {
      u.qw[0] = qp[min(w0 + q, wlast)];
    } else {
#pragma unroll
      for (int j = 0; j < 5; ++j) u.qw[j] = qp[min(w0 + j, wlast)];
    }
  } else {
    u.mu = 0.0f;
#pragma unroll
    for (int c = 0; c < 4; ++c)
      u.araw[c] = W.sc.absmax[u.blk0 + (FULL ? 4 * c + q : min(4 * c + q, nblk - 1))];
  }
  // blocks past the end of a ragged slice re-read the last block; their X
  // chunks are zero
  u.crow = W.codes + row * (g.k >> 1) + b0 * 32;
}
// codes of chunk c (blocks 4c + q) of a unit
template <bool FULL>
QL_DEV void unit_codes(GUnit &u, int c, int nblk, int q) {
  const int bb = FULL ? 4 * c + q : min(4 * c + q, nblk - 1);
  u.cw[c][0] = *(const uint4 *)(u.crow + 32 * bb);
  u.cw[c][1] = *(const uint4 *)(u.crow + 32 * bb + 16);
}

// MFMA steps of NU units of a wave (same slice, so they share the A
// operand reads; their independent chains interleave). D[4q + t][n] = partial
// sum of block 4c + q for token 4tp + t. Writes the units' partial sums.
template <bool DQ, int TP, int NU, bool QA, class Issue>
QL_DEV void unit_compute(const GemvArgs &g, const GUnit *const (&us)[NU],
                         const unsigned char *smem, const uint32_t (&abase)[TP], uint32_t lcopy,
                         int n, int q, int64_t slice, Issue issue) {
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  f32x4 acc[NU][TP];
#pragma unroll
  for (int v = 0; v < NU; ++v)
#pragma unroll
    for (int tp = 0; tp < TP; ++tp) acc[v][tp] = zero;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    issue(c);   // the code loads of a later chunk go out before this chunk's decode
    __builtin_amdgcn_sched_barrier(0);
    f32x4 p[NU][TP];
#pragma unroll
    for (int v = 0; v < NU; ++v)
#pragma unroll
      for (int tp = 0; tp < TP; ++tp) p[v][tp] = zero;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      uint4 bop[NU];
#pragma unroll
      for (int v = 0; v < NU; ++v) {
        const uint4 &h = us[v]->cw[c][s >> 2];
        const uint32_t w = (s & 3) == 0 ? h.x : (s & 3) == 1 ? h.y : (s & 3) == 2 ? h.z : h.w;
        bop[v].x = *(const uint32_t *)(smem + __builtin_amdgcn_perm(w, lcopy, 0x0C0C0400u));
        bop[v].y = *(const uint32_t *)(smem + __builtin_amdgcn_perm(w, lcopy, 0x0C0C0500u));
        bop[v].z = *(const uint32_t *)(smem + __builtin_amdgcn_perm(w, lcopy, 0x0C0C0600u));
        bop[v].w = *(const uint32_t *)(smem + __builtin_amdgcn_perm(w, lcopy, 0x0C0C0700u));
      }
#pragma unroll
      for (int tp = 0; tp < TP; ++tp) {
        const uint4 aop = *(const uint4 *)(smem + abase[tp] + xa_imm(c, s));
#pragma unroll
        for (int v = 0; v < NU; ++v) p[v][tp] = ql::mfma16(aop, bop[v], p[v][tp]);
      }
    }
#pragma unroll
    for (int v = 0; v < NU; ++v) {
      // scale of block 4c + q of row n
      const GUnit &u = *us[v];
      float ap;
      if (DQ) {
        const float s2 = ((u.blk0 + 4 * c + q) >> 8) == (u.blk0 >> 8) ? u.s2lo : u.s2hi;
        const uint32_t win =
            QA ? (uint32_t)__shfl((int)u.qw[0], n + 16 * c)
               : __builtin_amdgcn_alignbyte(u.qw[c + 1], u.qw[c], (uint32_t)(u.blk0 & 3));
        const int qv = (int)(int8_t)(win >> (8 * q));
        ap = (float)qv * s2 + u.mu;
      } else {
        ap = u.araw[c];
      }
#pragma unroll
      for (int tp = 0; tp < TP; ++tp)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[v][tp][i] = fmaf(ap, p[v][tp][i], acc[v][tp][i]);
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the chunks' register sets apart
  }
#pragma unroll
  for (int v = 0; v < NU; ++v) {
    // add the four lane groups (blocks 4c + q) of each row
#pragma unroll
    for (int tp = 0; tp < TP; ++tp)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float x = acc[v][tp][i];
        x += __shfl_xor(x, 16);
        x += __shfl_xor(x, 32);
        acc[v][tp][i] = x;
      }
    const int64_t row0 = us[v]->row0;
    if (q == 0 && row0 + n < us[v]->dlim) {
      const int64_t col = us[v]->rbase + row0 + n;
#pragma unroll
      for (int tp = 0; tp < TP; ++tp)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = 4 * tp + i;
          if (t < g.M) g.part[(slice * g.M + t) * g.dtot + col] = acc[v][tp][i];
        }
    }
  }
}

// LoRA down projection H = X A^T (QLoRA glossary, forward paragraph), partial
// sums over the 128 columns of this slice that wave w covers, on 16x16x32
// MFMA: A operand = X rows (tokens), B operand = A rows (ranks 16 cb ..
// 16 cb + 15); D[4q + i][n] = partial H[token 4q + i][rank 16 cb + n]. One
// X read serves every weight of the call. The X chunk and the first 16 ranks
// of the first weight's A are loaded up front (HPre), before the code loads,
// so the partial costs no memory round trip after the main compute.
struct HPre {
  uint4 xa[4];   // X[n][c0 + 32 i + 8 q .. + 7], raw (masked where used)
  uint4 aa[4];   // A[n][...] of weight 0, ranks 0..15, raw
};

// Unconditional loads from clamped addresses (a branch around a load makes
// the compiler wait for it on the spot); lanes outside M or the slice read
// the first row of X or A and are zeroed where the values are used.
QL_DEV void lora_down_load(const GemvArgs &g, int64_t slice, int nblk, int wave, int n, int q,
                           HPre &h) {
  const int64_t c0 = slice * (64 * GB) + 128 * wave;  // first column of the wave
  const int ncol = 64 * nblk - 128 * wave;           // valid columns of the wave (may be <= 0)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bool ok = 32 * i + 8 * q < ncol;
    const int64_t col = c0 + 32 * i + 8 * q;
    h.xa[i] = *(const uint4 *)(g.X + (ok && n < g.M ? n * g.k + col : 0));
    h.aa[i] = *(const uint4 *)(g.w[0].Ap + (ok ? (int64_t)n * g.k + col : 0));
  }
}

template <bool GRP>
QL_DEV void lora_down_partial(const GemvArgs &g, int64_t slice, int nblk, int wave, int n,
                              int q, const HPre &h) {
  const int64_t c0 = slice * (64 * GB) + 128 * wave;
  const int ncol = 64 * nblk - 128 * wave;
  for (int wi = 0; wi < (GRP ? g.nw : 1); ++wi) {
    const GemvW W = GRP ? wsel(g, wi) : g.w[0];
    uint4 xm[4];   // X with this weight's adapter-input dropout applied
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      xm[i] = (32 * i + 8 * q < ncol && n < g.M) ? h.xa[i] : ql::zero4();
      if (W.dp.on) {
        const uint64_t e = (uint64_t)(n < g.M ? n : 0) * (uint64_t)g.k +
                           (uint64_t)(c0 + 32 * i + 8 * q);
        xm[i] = mask_bf16x8(xm[i], keep4(W.dp, e) | (keep4(W.dp, e + 4) << 4));
      }
    }
    for (int cb = 0; cb < g.rp / 16; ++cb) {
      uint4 aa[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = 32 * i + 8 * q < ncol;
        aa[i] = !ok ? ql::zero4()
                : (wi == 0 && cb == 0)
                    ? h.aa[i]
                    : *(const uint4 *)(W.Ap + (int64_t)(16 * cb + n) * g.k + c0 + 32 * i + 8 * q);
      }
      f32x4 hacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; ++i) hacc = ql::mfma16(xm[i], aa[i], hacc);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 4 * q + i;
        if (t < g.M) W.hpart[((slice * GW + wave) * g.M + t) * g.rp + 16 * cb + n] = hacc[i];
      }
    }
  }
}

// Workgroup (x, slice) takes row groups x, x + G, x + 2G, ... (at most 2 GW
// of them) of one slice; wave w takes the workgroup's row groups w and
// w + GW, both loaded before the table is built, then computed together. The
// table and the X slice are built once per workgroup.
template <bool DQ, int TP, bool FULL, bool GRP, bool QA>
__global__ __launch_bounds__(GT) void nf4_gemv_kernel(GemvArgs g) {
  __shared__ __align__(16) unsigned char smem[LDS_BYTES];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, q = lane >> 4;
  const int64_t nbr = g.k >> 6;
  const int64_t slice = blockIdx.y;
  const int64_t b0 = slice * GB;
  const int nblk = FULL ? GB : (int)min<int64_t>(GB, nbr - b0);
  auto rg_of = [&](int j) -> int64_t { return (int64_t)blockIdx.x + (int64_t)g.G * j; };

  // Global loads in the order they are used: table entry, X slice, first unit.
  // 1. table entry written by this lane: byte e -> (level[e >> 4], level[e & 15]);
  //    the levels are read with uniform (scalar) loads and picked per lane,
  //    so no vector-memory wait stands before the table is built
  const int te = tid & 255;
  uint32_t lv_hi = c_levels_v[0], lv_lo = c_levels_v[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) {
    const uint32_t v = c_levels_v[i];
    lv_hi = (te >> 4) == i ? v : lv_hi;
    lv_lo = (te & 15) == i ? v : lv_lo;
  }
  // 2. X slice: chunk idx -> token m, slice block b, 8-column chunk s
  uint4 xv[GX];
#pragma unroll
  for (int i = 0; i < GX; ++i) {
    const int idx = tid + GT * i;
    const int m = idx >> 7, b = (idx >> 3) & 15, sc8 = idx & 7;
    const bool ok = m < g.M && b < nblk;  // else read X[0][0..7], stored as zeros
    xv[i] = *(const uint4 *)(g.X + (ok ? m * g.k + (b0 + b) * 64 + 8 * sc8 : 0));
  }
  // the LoRA down-projection operands, in the workgroup that computes that
  // partial (the last one of the slice, which has the fewest units); issued
  // before the code loads so the waits for the codes count the same loads
  // in every workgroup
  const bool hwg = blockIdx.x == gridDim.x - 1;
  HPre hp;
  if (hwg) lora_down_load(g, slice, nblk, wave, n, q, hp);
  __builtin_amdgcn_sched_barrier(0);
  // 3. the wave's two units (row groups wave and wave + GW of this
  //    workgroup), loaded unconditionally (clamped) so every wait is exact
  const int64_t rga = rg_of(wave), rgb = rg_of(wave + GW);
  const bool has_a = wave < g.rpw && rga < g.ngroups;
  const bool has_b = wave + GW < g.rpw && rgb < g.ngroups;
  GUnit ua, ub;
  unit_load<DQ, FULL, GRP, QA>(g, ua, min(rga, g.ngroups - 1), b0, nblk, n, q);
  unit_load<DQ, FULL, GRP, QA>(g, ub, min(rgb, g.ngroups - 1), b0, nblk, n, q);
  // codes chunk by chunk, both units' chunk c before chunk c + 1: the
  // compute of chunk c waits only for the loads up to it. Only the first
  // GPRE chunks go out before the table is built: once the memory queues are
  // full a load instruction waits to issue, and a wave issues in order, so
  // loads placed before the barrier below would hold every wave of the
  // workgroup at it until nearly all of its data had streamed in, and no
  // decode would overlap the stream.
#pragma unroll
  for (int c = 0; c < GPRE; ++c) {
    unit_codes<FULL>(ua, c, nblk, q);
    unit_codes<FULL>(ub, c, nblk, q);
    __builtin_amdgcn_sched_barrier(0);
  }
  // 4. table (bf16 pair, even element in the low half), 32 copies per entry;
  //    X chunks; zero region
  {
    const uint32_t v = ql::pack_bf16x2(__uint_as_float(lv_hi), __uint_as_float(lv_lo));
    const uint4 v4 = make_uint4(v, v, v, v);
    constexpr int PER = 2048 / GT;  // 16-byte stores per lane
    unsigned char *t = smem + te * 256 + 16 * PER * (tid >> 8);
#pragma unroll
    for (int i = 0; i < PER; ++i) *(uint4 *)(t + 16 * i) = v4;
  }
#pragma unroll
  for (int i = 0; i < GX; ++i) {
    const int idx = tid + GT * i;
    const int m = idx >> 7, b = (idx >> 3) & 15, sc8 = idx & 7;
    const bool ok = m < g.M && b < nblk;
    *(uint4 *)(smem + xa_base(m >> 2, b & 3, m & 3) + xa_imm(b >> 2, sc8)) = ok ? xv[i] : ql::zero4();
  }
  if (tid < (int)(ZBYTES / 16)) *(uint4 *)(smem + ZBASE + 16 * tid) = ql::zero4();
  __syncthreads();
  // the rest of the code loads: chunks up to GLA - 1 now, chunk c + GLA just
  // before the decode of chunk c, so a wave held at a load issue has already
  // decoded what arrived
#pragma unroll
  for (int c = GPRE; c < GLA && c < 4; ++c) {
    unit_codes<FULL>(ua, c, nblk, q);
    unit_codes<FULL>(ub, c, nblk, q);
    __builtin_amdgcn_sched_barrier(0);
  }
  auto issue = [&](int c) {
    const int cn = c + GLA;
    if (cn >= GPRE && cn < 4) {
      unit_codes<FULL>(ua, cn, nblk, q);
      unit_codes<FULL>(ub, cn, nblk, q);
    }
  };

  const uint32_t lcopy = 4u * (uint32_t)(lane & 31);
  const bool a_on = (n >> 2) == q;  // lane group q carries token rows 4q..4q+3
  uint32_t abase[TP];
#pragma unroll
  for (int tp = 0; tp < TP; ++tp) abase[tp] = a_on ? xa_base(tp, q, n & 3) : ZBASE;
  if (has_b) {  // has_b implies has_a
    const GUnit *const both[2] = {&ua, &ub};
    unit_compute<DQ, TP, 2, QA>(g, both, smem, abase, lcopy, n, q, slice, issue);
  } else if (has_a) {
    const GUnit *const one[1] = {&ua};
    unit_compute<DQ, TP, 1, QA>(g, one, smem, abase, lcopy, n, q, slice, issue);
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c) issue(c);   // every code register gets its (clamped) load
  }
  // The second unit's loads were issued on every wave; keep their registers
  // live to here so that no instruction above reuses one while its load is
  // in flight (which would make the first wait of a one-unit wave cover
  // every load).
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int h = 0; h < 2; ++h)
      asm volatile("" ::"v"(ub.cw[c][h].x), "v"(ub.cw[c][h].y), "v"(ub.cw[c][h].z),
                   "v"(ub.cw[c][h].w));
  if (hwg) lora_down_partial<GRP>(g, slice, nblk, wave, n, q, hp);
}

// ---- few-token forward on VALU (M <= VMAXM, no adapter-input dropout) ----
// Same partial sums as above, organised for one or two tokens, where the
// 16x16x32 MFMA would run with 15 of 16 rows zero and every X operand would
// be an LDS read. A slice is 2048 columns: lane l owns columns 32 l .. 32 l
// + 31 (16 code bytes, half of block l / 2), keeps those X values in
// registers for every row it visits, and per code byte reads the pair of
// bf16 levels from the byte table (32 copies, as above) and adds both
// products with one v_dot2_f32_bf16 per token. The 32-weight partial is
// scaled by the block's a' once. A workgroup serves one slice: its threads
// load the slice of X once and pass it through LDS; each wave takes VR
// rows, and the per-row sums of its lanes are added by a butterfly that
// hands each lane group one (row, token) sum in a fixed order. The byte
// table is built first (it waits on nothing), then every load of a wave (X,
// block scales, the VR rows' code words) is issued before the barrier, so
// the whole record is requested at the start and each row is decoded as it
// arrives. H = X A^T partials come from one more workgroup per slice, weight
// and 16 ranks (ranks 2w, 2w + 1 of the 16 for wave w). Both go to the
// epilogue kernel below (one H partial per slice).
// Measured call times (graph replay, 16 rotated weights, us) against the
// MFMA kernel above at M = 1: 12.9 / 14.3 (11008x4096) and 14.0 / 16.4
// (4096x11008). The int8 block codes as one dword per lane (below) instead
// of a byte load per row took 0.5 us off each; with no block-scale loads at
// all (a timing copy) the call took 12.5 / 13.2 before that change, so the
// read of the record in this shape (plus the epilogue launch, ~3.5) sets
// the time more than the decode or the scales do. Measured and not
// kept: sixteen rows per wave (half the waves) 19.8 / 20.0; each wave
// reading its own X slice from L2 instead of through LDS, 14.4 / 14.8 (with
// the butterfly still spilling); this path for four tokens 21.0 / 21.8
// against 14.9 / 16.3 on MFMA (one workgroup per CU at 134 registers).
constexpr int VW = 8;          // waves per workgroup
constexpr int VCOL = 2048;     // columns per slice (64 lanes x 32)
constexpr int VR = 8;          // weight rows per wave
constexpr int VMAXM = 2;       // tokens served by this path

struct VArgs {
  GemvW w[GMAXW];   // gbase counts groups of VR rows
  int nw;
  int64_t k;
  const uint16_t *X;
  int64_t M;
  int64_t nunits;   // row groups of all weights x slices
  int S;            // slices
  int nrow_wg;      // workgroups of row units; the H workgroups follow
  float *part;      // [S][M][dtot]
  int64_t dtot;
  int rp;
};

// Sum v[i] over the 64 lanes of a wave for every i, in a fixed order: each
// butterfly step hands half of the entries to the lane partner that keeps
// them, so after the steps lane l holds the sum of entry l >> (6 - log2 N)
// in its return value (all lanes of a group of 64 / N hold the same bits).
template <int N>
QL_DEV float wave_transpose_sum(float (&v)[N], int lane) {
  static_assert(N >= 1 && N <= 64 && (N & (N - 1)) == 0, "N: power of two up to 64");
#pragma unroll
  for (int st = 0; st < 6; ++st) {
    const int mask = 32 >> st;
    const int half = N >> (st + 1);
    const bool up = (lane & mask) != 0;
    if (half >= 1) {
#pragma unroll
      for (int i = 0; i < half; ++i) {
        // the pair as opaque register values: otherwise the lane-dependent
        // selects become an indexed access to a scratch copy of v
        float lo = v[i], hi = v[i + half];
        asm("" : "+v"(lo), "+v"(hi));
        const float send = up ? lo : hi;
        const float keep = up ? hi : lo;
        v[i] = keep + __shfl_xor(send, mask);
      }
    } else {
      v[0] += __shfl_xor(v[0], mask);
    }
  }
  return v[0];
}

// X[m][col0 .. col0 + 31] of tokens m < MV as 16 bf16 pairs (token rows past
// M and lanes past k read clamped addresses; their sums are never stored or
// are zeroed)
template <int MV>
QL_DEV void valu_load_x(const VArgs &g, int64_t colc, uint32_t (&xw)[MV][16]) {
#pragma unroll
  for (int m = 0; m < MV; ++m) {
    const int64_t mr = m < g.M ? m : 0;
    const uint4 *src = (const uint4 *)(g.X + mr * g.k + colc);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 v = src[i];
      xw[m][4 * i] = v.x;
      xw[m][4 * i + 1] = v.y;
      xw[m][4 * i + 2] = v.z;
      xw[m][4 * i + 3] = v.w;
    }
  }
}

QL_DEV float dot2bf(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), c, false);
}

// H partials of one slice of one weight for one chunk of 16 ranks (one
// workgroup per weight, slice and chunk): wave w takes ranks 16 cb + 2 w, +1.
template <int MV, bool GRP>
QL_DEV void valu_lora_down(const VArgs &g, int hidx, int wave, int lane) {
  const int nrc = g.rp / 16;
  const int cb = hidx % nrc, ws = hidx / nrc;
  const int wi = ws / g.S, slice = ws % g.S;
  const GemvW W = GRP ? wsel(g, wi) : g.w[0];
  const int64_t col0 = (int64_t)slice * VCOL + 32 * lane;
  const bool lok = col0 < g.k;
  const int64_t colc = lok ? col0 : 0;
  uint32_t xw[MV][16];
  valu_load_x<MV>(g, colc, xw);
  float v[2 * MV];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const int t = 16 * cb + 2 * wave + tt;
    const uint4 *src = (const uint4 *)(W.Ap + (int64_t)t * g.k + colc);
    uint32_t aw[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 a = src[i];
      aw[4 * i] = a.x;
      aw[4 * i + 1] = a.y;
      aw[4 * i + 2] = a.z;
      aw[4 * i + 3] = a.w;
    }
#pragma unroll
    for (int m = 0; m < MV; ++m) {
      float p0 = 0.f, p1 = 0.f;
#pragma unroll
      for (int j = 0; j < 16; j += 2) {
        p0 = dot2bf(aw[j], xw[m][j], p0);
        p1 = dot2bf(aw[j + 1], xw[m][j + 1], p1);
      }
      v[tt * MV + m] = lok ? p0 + p1 : 0.f;
    }
  }
  const float sum = wave_transpose_sum<2 * MV>(v, lane);
  constexpr int LGH = MV == 1 ? 5 : MV == 2 ? 4 : 3;   // log2(64 / (2 MV))
  const int idx = lane >> LGH;
  const int tt = idx / MV, m = idx % MV;
  if ((lane & ((1 << LGH) - 1)) == 0 && m < g.M)
    W.hpart[((int64_t)slice * g.M + m) * g.rp + 16 * cb + 2 * wave + tt] = sum;
}

// QA (double quantisation with k % 256 == 0, so every row's int8 codes start
// 4-byte aligned): one dword load per lane brings the codes of all VR rows'
// slice blocks (lane l: row l / 8, blocks 4 (l % 8) .. + 3), handed to the
// lanes that need them by one shuffle per row; otherwise one byte load per
// row and lane.
template <bool DQ, int MV, bool GRP, bool QA>
__global__ __launch_bounds__(64 * VW) void nf4_gemv_valu_kernel(VArgs g) {
  __shared__ __align__(16) unsigned char lut[256 * 256];
  __shared__ __align__(16) uint4 xs[MV][256];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if ((int)blockIdx.x >= g.nrow_wg) {   // uniform per workgroup
    valu_lora_down<MV, GRP>(g, (int)blockIdx.x - g.nrow_wg, wave, lane);
    return;
  }
  // workgroup b: slice b % S, row groups (b / S) VW + wave (clamped; the
  // waves past the last row group write nothing)
  const int slice = (int)(blockIdx.x % g.S);
  const int64_t ngroups = g.nunits / g.S;
  const int64_t rg = ((int64_t)blockIdx.x / g.S) * VW + wave;
  const int64_t rgc = rg < ngroups ? rg : ngroups - 1;
  const GemvW W = GRP ? wsel(g, weight_of(g, rgc)) : g.w[0];
  const int64_t row0 = (rgc - W.gbase) * VR;
  const int64_t nbr = g.k >> 6;
  const int64_t col0 = (int64_t)slice * VCOL + 32 * lane;
  const bool lok = col0 < g.k;
  const int64_t colc = lok ? col0 : 0;
  // 1. byte table: entry e = (level[e >> 4], level[e & 15]) as a bf16 pair
  //    (even element low), 32 copies in bytes 0-127 of row e; built first,
  //    as it waits on no memory
  {
    const int te = tid & 255;
    uint32_t lv_hi = c_levels_v[0], lv_lo = c_levels_v[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) {
      const uint32_t v = c_levels_v[i];
      lv_hi = (te >> 4) == i ? v : lv_hi;
      lv_lo = (te & 15) == i ? v : lv_lo;
    }
    const uint32_t v = ql::pack_bf16x2(__uint_as_float(lv_hi), __uint_as_float(lv_lo));
    const uint4 v4 = make_uint4(v, v, v, v);
    unsigned char *t = lut + te * 256 + 64 * (tid >> 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) *(uint4 *)(t + 16 * i) = v4;
  }
  __builtin_amdgcn_sched_barrier(0);
  // 2. loads, in the order they are needed: the slice of X (8 columns per
  //    thread, clamped past k), then per row the block-scale inputs and the
  //    lane's code word
  uint4 xv[MV];
  {
    const int64_t xc = (int64_t)slice * VCOL + 8 * (tid & 255);
#pragma unroll
    for (int m = 0; m < MV; ++m)
      xv[m] = *(const uint4 *)(g.X + (m < g.M ? m : 0) * g.k + (xc < g.k ? xc : 0));
  }
  const float mu = DQ ? W.sc.mu[0] : 0.0f;
  static_assert(!QA || VR == 8, "one dword load per lane covers 8 rows");
  uint32_t qd = 0;
  if (DQ && QA) {   // clamped to the last row and the row's last 4 blocks
    const int64_t rq = min(row0 + (lane >> 3), W.d - 1);
    const int64_t off = min((int64_t)slice * (VCOL / 64) + 4 * (lane & 7), nbr - 4);
    qd = *(const uint32_t *)(W.sc.q + rq * nbr + off);
  }
  uint4 cw[VR];
  float sa[VR], sb[VR];
#pragma unroll
  for (int r = 0; r < VR; ++r) {
    const int64_t row = min(row0 + r, W.d - 1);
    const int64_t blk = row * nbr + (colc >> 6);
    if (DQ) {
      sa[r] = QA ? 0.0f : (float)W.sc.q[blk];
      sb[r] = W.sc.s2[blk >> 8];
    } else {
      sa[r] = W.sc.absmax[blk];
      sb[r] = 0.0f;
    }
    cw[r] = *(const uint4 *)(W.codes + row * (g.k >> 1) + (colc >> 1));
  }
  // 3. X through LDS: waits for the X loads only (issued first), then each
  //    lane takes its 32 columns into registers
  if (tid < 256) {
#pragma unroll
    for (int m = 0; m < MV; ++m) xs[m][tid] = xv[m];
  }
  __syncthreads();
  uint32_t xw[MV][16];
#pragma unroll
  for (int m = 0; m < MV; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 v = xs[m][4 * lane + i];
      xw[m][4 * i] = v.x;
      xw[m][4 * i + 1] = v.y;
      xw[m][4 * i + 2] = v.z;
      xw[m][4 * i + 3] = v.w;
    }
  // 4. rows in load order: 16 table reads and 16 MV dot products per lane
  const uint32_t lcopy = 4u * (uint32_t)(lane & 31);
  float acc[VR * MV];
#pragma unroll
  for (int r = 0; r < VR; ++r) {
    const uint32_t cws[4] = {cw[r].x, cw[r].y, cw[r].z, cw[r].w};
    float p0[MV], p1[MV];
#pragma unroll
    for (int m = 0; m < MV; ++m) p0[m] = p1[m] = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint32_t lv = *(const uint32_t *)(lut + __builtin_amdgcn_perm(
                                                       cws[j >> 2], lcopy, 0x0C0C0400u + ((j & 3) << 8)));
#pragma unroll
      for (int m = 0; m < MV; ++m) {
        if (j & 1) p1[m] = dot2bf(lv, xw[m][j], p1[m]);
        else p0[m] = dot2bf(lv, xw[m][j], p0[m]);
      }
    }
    if (DQ && QA) {   // this lane's block code of row r, from lane 8 r + l / 8
      const uint32_t w = (uint32_t)__shfl((int)qd, 8 * r + (lane >> 3));
      sa[r] = (float)(int8_t)(w >> (8 * ((lane >> 1) & 3)));
    }
    const float ap = DQ ? sa[r] * sb[r] + mu : sa[r];
#pragma unroll
    for (int m = 0; m < MV; ++m) acc[r * MV + m] = lok ? ap * (p0[m] + p1[m]) : 0.f;
  }
  // 5. per (row, token) sums over the lanes; lane group idx writes entry idx
  constexpr int N = VR * MV;
  const float sum = wave_transpose_sum<N>(acc, lane);
  constexpr int LG = N == 8 ? 3 : N == 16 ? 2 : N == 32 ? 1 : 0;   // log2(64 / N)
  const int idx = lane >> LG;
  const int r = idx / MV, m = idx % MV;
  if (rg < ngroups && (lane & ((1 << LG) - 1)) == 0 && m < g.M && row0 + r < W.d)
    g.part[((int64_t)slice * g.M + m) * g.dtot + W.rbase + row0 + r] = sum;
}

// Y[m][j] = bf16(sum_s part[s][m][j] + s_l * sum_t H[m][t] B[j][t]) with
// H[m][t] = sum_p hpart[p][m][t] (fixed orders), per weight of the call;
// workgroup (x, m) serves 256 columns of one weight and builds its H[m] in
// LDS (256 / rp lane groups of rp lanes, rp <= 128); the first workgroup of
// each weight also writes H_save (M x r).
struct EpiW {
  const uint16_t *Bp;   // d x rp
  const float *hpart;   // [nhp][M][rp]
  uint16_t *Y;          // M x d
  float *hsave;         // M x r or NULL
  int64_t d, rbase, ebase;   // rows, first partial-sum column, first workgroup
  float hscale;         // 1/(1-p) with adapter-input dropout, else 1
};
struct EpiArgs {
  EpiW w[GMAXW];
  int nw;
  const float *part;    // [S][M][dtot]
  int S;
  int64_t M, dtot;
  int nhp, rp, r;
  float s;
};
QL_DEV EpiW esel(const EpiArgs &e, int i) {
  EpiW W;
  W.Bp = QL_PICK(e.w, i, Bp);
  W.hpart = QL_PICK(e.w, i, hpart);
  W.Y = QL_PICK(e.w, i, Y);
  W.hsave = QL_PICK(e.w, i, hsave);
  W.d = QL_PICK(e.w, i, d);
  W.rbase = QL_PICK(e.w, i, rbase);
  W.ebase = QL_PICK(e.w, i, ebase);
  W.hscale = QL_PICK(e.w, i, hscale);
  return W;
}

__global__ __launch_bounds__(256) void gemv_epilogue_kernel(EpiArgs e) {
  __shared__ float hp[16][128];  // per lane-group sums of the H partials
  __shared__ float hs[128];
  const int64_t m = blockIdx.y;
  const int tid = threadIdx.x;
  int wi = 0;
#pragma unroll
  for (int j = 1; j < GMAXW; ++j) wi += (j < e.nw && (int64_t)blockIdx.x >= e.w[j].ebase) ? 1 : 0;
  const EpiW W = esel(e, wi);
  const int rp = e.rp;
  // the loads that do not depend on H go first (slice partials of output j
  // and the first 16 ranks of its B row), so one memory round trip covers
  // them and the H partials
  const int64_t xb = (int64_t)blockIdx.x - W.ebase;
  const int64_t j = xb * 256 + tid;
  const int64_t jc = j < W.d ? j : W.d - 1;
  const uint4 b0 = *(const uint4 *)(W.Bp + jc * rp), b1 = *(const uint4 *)(W.Bp + jc * rp + 8);
  // eight slices' loads in flight (clamped slice index), then their sums in
  // slice order: a loop unrolled over a run-time count would leave its tail
  // as one load and wait per slice
  float acc = 0.0f;
  for (int s0 = 0; s0 < e.S; s0 += 8) {
    float pv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      pv[u] = e.part[((int64_t)min(s0 + u, e.S - 1) * e.M + m) * e.dtot + W.rbase + jc];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (s0 + u < e.S) acc += pv[u];
  }
  // H[m][t]: lane group grp adds partials p = grp, grp + ng, ... of rank t
  // (ng = 256 / rp groups), then rank t adds the groups in order
  {
    const int ng = 256 / rp, t = tid % rp, grp = tid / rp;
    if (grp < ng) {
      float ha = 0.0f;
      for (int p0 = grp; p0 < e.nhp; p0 += 4 * ng) {   // four partials' loads, then their sums
        float hv[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
          hv[u] = W.hpart[((int64_t)min(p0 + u * ng, e.nhp - 1) * e.M + m) * rp + t];
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (p0 + u * ng < e.nhp) ha += hv[u];
      }
      hp[grp][t] = ha;
    }
    __syncthreads();
    if (tid < rp) {
      float ha = 0.0f;
      for (int gi = 0; gi < ng; ++gi) ha += hp[gi][tid];
      ha *= W.hscale;   // inverted dropout of the adapter input (exactly 1 without)
      hs[tid] = ha;
      if (W.hsave && xb == 0 && tid < e.r) W.hsave[m * e.r + tid] = ha;
    }
    __syncthreads();
  }
  if (j >= W.d) return;
  const uint32_t bw[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
  float l = 0.0f;
#pragma unroll
  for (int t = 0; t < 16; ++t)
    l = fmaf(hs[t], (t & 1) ? ql::bf16hi(bw[t >> 1]) : ql::bf16lo(bw[t >> 1]), l);
  for (int t = 16; t < rp; ++t) l = fmaf(hs[t], ql::bf16_to_f(W.Bp[j * rp + t]), l);
  W.Y[m * W.d + j] = ql::f_to_bf16(acc + e.s * l);
}

}  // namespace

static int64_t gemv_splits(int64_t k) { return ql_cdiv(k >> 6, GB); }

size_t gemv_part_bytes(int64_t dtot, int64_t k, int64_t M, int rp, int nw) {
  return (size_t)(gemv_splits(k) * M * dtot * 4 + nw * gemv_splits(k) * GW * M * rp * 4);
}

// The VALU path for M <= VMAXM without adapter-input dropout: S = k / 2048
// slices (the last may be ragged), one H partial per slice and weight; its
// partial sums fit in the workspace sized for the MFMA path (fewer slices,
// fewer H partials).
static qlora_status launch_gemv_valu(int nw, const GemvIn *in, int64_t k, const uint16_t *X,
                                     int64_t M, int r, int rp, float s, float *part,
                                     hipStream_t st) {
  const int64_t S = ql_cdiv(k, VCOL);
  int64_t dtot = 0, ngroups = 0, eblocks = 0;
  VArgs g{};
  EpiArgs e{};
  for (int i = 0; i < nw; ++i) {
    const int64_t d = in[i].d;
    g.w[i] = GemvW{in[i].codes, in[i].sc, d, d * (k >> 6), ngroups, dtot, in[i].Ap, nullptr,
                   in[i].dp};
    e.w[i] = EpiW{in[i].Bp, nullptr, in[i].Y, in[i].H_save, d, dtot, eblocks, 1.0f};
    ngroups += ql_cdiv(d, VR);
    eblocks += ql_cdiv(d, 256);
    dtot += d;
  }
  for (int i = 0; i < nw; ++i) {
    float *hpart = part + S * M * dtot + (int64_t)i * S * M * rp;
    g.w[i].hpart = hpart;
    e.w[i].hpart = hpart;
  }
  for (int i = nw; i < GMAXW; ++i) {  // unused slots: never selected
    g.w[i] = g.w[0];
    e.w[i] = e.w[0];
  }
  const int64_t nunits = ngroups * S;
  const int64_t nrow_wg = ql_cdiv(ngroups, VW) * S;
  const int64_t nh_wg = nw * S * (rp / 16);   // H: one workgroup per weight, slice, 16 ranks
  if (nrow_wg + nh_wg > 0x7fffffff || eblocks > 0x7fffffff) return QLORA_ERR_UNSUPPORTED;
  g.nw = nw;
  g.k = k;
  g.X = X;
  g.M = M;
  g.nunits = nunits;
  g.S = (int)S;
  g.nrow_wg = (int)nrow_wg;
  g.part = part;
  g.dtot = dtot;
  g.rp = rp;
  {
    QlProf prof(QLORA_K_GEMV, st);
    const unsigned grid = (unsigned)(nrow_wg + nh_wg);
#define QL_VGEMV(DQV, MVV, QAV)                                                  \
  if (nw > 1)                                                                    \
    nf4_gemv_valu_kernel<DQV, MVV, true, QAV><<<grid, 64 * VW, 0, st>>>(g);      \
  else                                                                           \
    nf4_gemv_valu_kernel<DQV, MVV, false, QAV><<<grid, 64 * VW, 0, st>>>(g);
    const bool qa = (k % 256) == 0;
    if (in[0].sc.dq && qa) {
      if (M == 1) { QL_VGEMV(true, 1, true) } else { QL_VGEMV(true, 2, true) }
    } else if (in[0].sc.dq) {
      if (M == 1) { QL_VGEMV(true, 1, false) } else { QL_VGEMV(true, 2, false) }
    } else {
      if (M == 1) { QL_VGEMV(false, 1, false) } else { QL_VGEMV(false, 2, false) }
    }
#undef QL_VGEMV
  }
  {
    e.nw = nw;
    e.part = part;
    e.S = (int)S;
    e.M = M;
    e.dtot = dtot;
    e.nhp = (int)S;
    e.rp = rp;
    e.r = r;
    e.s = s;
    QlProf prof(QLORA_K_GEMV_EPILOGUE, st);
    dim3 eg((unsigned)eblocks, (unsigned)M);
    gemv_epilogue_kernel<<<eg, 256, 0, st>>>(e);
  }
  QL_LAUNCH_CHECK();
  return QLORA_OK;
}

qlora_status launch_gemv_fwd(int nw, const GemvIn *in, int64_t k, const uint16_t *X, int64_t M,
                             int r, int rp, float s, float *part, hipStream_t st) {
  if (M < 1 || M > 16 || rp < 16 || rp > 128 || rp % 16) return QLORA_ERR_INVALID_ARG;
  if (nw < 1 || nw > GMAXW) return QLORA_ERR_INVALID_ARG;
  for (int i = 1; i < nw; ++i)
    if (in[i].sc.dq != in[0].sc.dq) return QLORA_ERR_INVALID_ARG;
  bool drop = false;
  for (int i = 0; i < nw; ++i) drop = drop || in[i].dp.on;
  if (M <= VMAXM && !drop) return launch_gemv_valu(nw, in, k, X, M, r, rp, s, part, st);
  const int ncu = ql_num_cus();
  const int64_t S = gemv_splits(k);
  int64_t dtot = 0, ngroups = 0, eblocks = 0;
  GemvArgs g{};
  EpiArgs e{};
  for (int i = 0; i < nw; ++i) {
    const int64_t d = in[i].d;
    g.w[i] = GemvW{in[i].codes, in[i].sc, d, d * (k >> 6), ngroups, dtot, in[i].Ap, nullptr,
                   in[i].dp};
    e.w[i] = EpiW{in[i].Bp, nullptr, in[i].Y, in[i].H_save, d, dtot, eblocks,
                  in[i].dp.on ? in[i].dp.inv_keep : 1.0f};
    ngroups += ql_cdiv(d, 16);
    eblocks += ql_cdiv(d, 256);
    dtot += d;
  }
  for (int i = 0; i < nw; ++i) {
    float *hpart = part + S * M * dtot + (int64_t)i * S * GW * M * rp;
    g.w[i].hpart = hpart;
    e.w[i].hpart = hpart;
  }
  for (int i = nw; i < GMAXW; ++i) {  // unused slots: never selected
    g.w[i] = g.w[0];
    e.w[i] = e.w[0];
  }
  // about one workgroup per compute unit, each slice served by G of them,
  // and at most two row groups per wave
  const int64_t G = std::min<int64_t>(
      ngroups, std::max<int64_t>(std::max<int64_t>(1, ncu / S), ql_cdiv(ngroups, 2 * GW)));
  const int64_t rpw = ql_cdiv(ngroups, G);
  if (S > 65535 || G > (int64_t(1) << 30) || eblocks > 0x7fffffff) return QLORA_ERR_UNSUPPORTED;
  g.nw = nw;
  g.k = k;
  g.X = X;
  g.M = M;
  g.ngroups = ngroups;
  g.G = (int)G;
  g.rpw = (int)rpw;
  g.part = part;
  g.dtot = dtot;
  g.rp = rp;
  dim3 grid((unsigned)G, (unsigned)S);
  {
    QlProf prof(QLORA_K_GEMV, st);
    const int tp = (int)ql_cdiv(M, 4);
    // every slice is full when k is a multiple of 1024
    const bool full = (k % (64 * GB)) == 0;
#define QL_GEMV5(DQV, TPV, FV, QAV)                                     \
  if (nw > 1)                                                           \
    nf4_gemv_kernel<DQV, TPV, FV, true, QAV><<<grid, GT, 0, st>>>(g);   \
  else                                                                  \
    nf4_gemv_kernel<DQV, TPV, FV, false, QAV><<<grid, GT, 0, st>>>(g);
#define QL_GEMV4(DQV, TPV, FV)                                          \
  if (DQV && (k % 256) == 0) {                                          \
    QL_GEMV5(DQV, TPV, FV, DQV)                                         \
  } else {                                                              \
    QL_GEMV5(DQV, TPV, FV, false)                                       \
  }
#define QL_GEMV3(DQV, TPV)                                              \
  if (full) {                                                           \
    QL_GEMV4(DQV, TPV, true)                                            \
  } else {                                                              \
    QL_GEMV4(DQV, TPV, false)                                           \
  }
#define QL_GEMV(TPV)                                                    \
  if (in[0].sc.dq) {                                                    \
    QL_GEMV3(true, TPV)                                                 \
  } else {                                                              \
    QL_GEMV3(false, TPV)                                                \
  }
    if (tp == 1) { QL_GEMV(1) } else if (tp == 2) { QL_GEMV(2) } else if (tp == 3) { QL_GEMV(3) } else { QL_GEMV(4) }
#undef QL_GEMV
#undef QL_GEMV3
#undef QL_GEMV4
#undef QL_GEMV5
  }
  {
    e.nw = nw;
    e.part = part;
    e.S = (int)S;
    e.M = M;
    e.dtot = dtot;
    e.nhp = (int)(S * GW);
    e.rp = rp;
    e.r = r;
    e.s = s;
    QlProf prof(QLORA_K_GEMV_EPILOGUE, st);
    dim3 eg((unsigned)eblocks, (unsigned)M);
    gemv_epilogue_kernel<<<eg, 256, 0, st>>>(e);
  }
  QL_LAUNCH_CHECK();
  return QLORA_OK;
}
