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
// row (forward) or per 8-row column strip (dX); one workgroup per CU for the
// 4096 x 2048 problem. Eight waves with two roles:
//   * 4 consumer waves (2 x 2 grid, 64 x 128 each) only read LDS and issue
//     v_mfma_f32_32x32x16_bf16 (8 accumulator tiles per wave);
//   * 4 producer waves fetch everything by LDS DMA (global_load_lds): the In
//     tile (three-stage ring, two steps ahead) and the packed codes with their
//     scale words (three-stage ring, three steps ahead); they decode the codes
//     into the bf16 W' tile (two-stage ring, one step ahead).
// Two waves share each SIMD, so decode and loads overlap the matrix cores.
// One barrier per K-step. LDS rows of 128 bytes are stored with the 16-byte
// chunks permuted by f(row) = (row ^ row>>2) & 7, which makes the MFMA operand
// reads, the decoded-tile writes of both forms and the raw-code reads of the
// dX form bank-conflict free.
// Workgroups are mapped XCD-aware: consecutive tiles of one token block land
// on the same XCD (its L2 then holds that X/dY block).
#include "kernels.h"
#include "nf4_tables.h"

namespace {

constexpr int BN = 128, BM = 256, BK = 64, NT = 512;
constexpr int NXB = 3;   // In-tile stages (fetched two steps ahead)
constexpr int NCB = 3;   // code/scale stages (fetched three steps ahead)
constexpr int NWB = 2;   // decoded W' stages (decoded one step ahead)
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

// LDS. Everything the producers fetch from global memory arrives by LDS DMA
// (global_load_lds), so loaded data never occupies registers across steps
// and every step issues the same loads.
__shared__ uint4 s_X[NXB][BM * 8];   // In tiles, 256 rows x 128 bytes
__shared__ uint4 s_C[NCB][256];      // 16 bytes of codes per producer lane
__shared__ uint32_t s_Q[NCB][256];   // dword holding the lane's int8 absmax code (or absmax)
__shared__ float s_S[NCB][256];      // s2 of the lane's block (double quant)
__shared__ uint4 s_W[NWB][BN * 8];   // decoded W' tiles, 128 rows x 128 bytes
__shared__ float s_lv[16];

QL_DEV int swz(int row, int chunk) { return row * 8 + (chunk ^ ((row ^ (row >> 2)) & 7)); }

typedef __attribute__((address_space(3))) void lds_void;
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

QL_DEV uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

// Workgroup barrier without memory fences; the asm statements keep the
// compiler from moving memory accesses across it.
QL_DEV void block_sync() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

QL_DEV void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// s_waitcnt with vmcnt <= n (n < 64), expcnt and lgkmcnt left unconstrained.
template <int N>
QL_DEV void wait_vm_le() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Loads per producer step: 8 In-tile rows groups, the code word, the scale
// dword and (double quant) the s2 scale.
template <bool DQ>
constexpr int kLoadsPerStep() { return DQ ? 11 : 10; }

// ---- producer fetch plan ----------------------------------------------------
// In tile: lane l of producer wave pw fetches, for each of 8 groups of 8 rows,
// the chunk that the LDS permutation places at position l of the group.
// Codes: forward form, lane p fetches 32 codes of W' row n0 + p/2 (half p%2);
// dX form, lane p fetches 32 codes of W' row kk + p/4, columns
// n0 + 32(p%4) .. +31. Each lane also fetches its block's scale.
struct Plan {
  uint32_t xoff[8];   // byte offsets of the In rows (from In + kk)
  int64_t row;        // forward: weight row; dX: row offset inside the step
  int64_t col;        // first code column of the lane's 32
};

QL_DEV Plan make_plan(const GemmArgs &g, int mode, int64_t m0, int64_t n0, int pw, int lane,
                      int p) {
  Plan pl;
  const int rl = lane >> 3, phys = lane & 7;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = 64 * pw + 8 * i + rl;
    const int chunk = phys ^ ((row ^ (row >> 2)) & 7);
    int64_t m = m0 + row;
    m = m < g.M ? m : g.M - 1;  // rows past M: duplicate data, outputs discarded
    pl.xoff[i] = (uint32_t)((m * g.Ktot + 8 * chunk) * 2);
  }
  if (mode == 0) {
    int64_t row = n0 + (p >> 1);
    pl.row = row < g.d ? row : g.d - 1;   // rows past d feed only discarded outputs
    pl.col = 32 * (p & 1);
  } else {
    pl.row = p >> 2;
    const int64_t col = n0 + 32 * (p & 3);
    pl.col = col < g.k ? col : g.k - 32;  // columns past k feed discarded outputs
  }
  return pl;
}

// Weight element index of the lane's first code at step kk.
QL_DEV int64_t code_elem(const GemmArgs &g, int mode, const Plan &pl, int64_t kk) {
  if (mode == 0) return pl.row * g.k + kk + pl.col;
  int64_t j = kk + pl.row;
  j = j < g.d ? j : g.d - 1;
  return j * g.k + pl.col;
}

// Issue the loads of step kk: the In tile (do_x) and/or the codes (do_c).
// ALWAYS_FULL: the caller knows the In tile lies inside Ktot.
template <int MODE, bool DQ, bool ALWAYS_FULL = false>
QL_DEV void issue_step(const GemmArgs &g, int64_t kk, bool do_x, bool do_c, int pw, int lane,
                       int p, const Plan &pl) {
  if (do_x) {
    const int xb = (int)((kk / BK) % NXB);
    const bool full = ALWAYS_FULL || kk + BK <= g.Ktot;
    const char *base = (const char *)(g.In + kk);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t off = pl.xoff[i];
      if (!full) {  // chunks past Ktot: last valid chunk (finite data times a zero W')
        const int row = 64 * pw + 8 * i + (lane >> 3);
        const int chunk = (lane & 7) ^ ((row ^ (row >> 2)) & 7);
        if (kk + 8 * chunk >= g.Ktot) off -= (uint32_t)((kk + 8 * chunk - (g.Ktot - 8)) * 2);
      }
      __builtin_amdgcn_global_load_lds((const void *)(base + off),
                                       (lds_void *)&s_X[xb][(64 * pw + 8 * i) * 8], 16, 0, 0);
    }
  }
  if (do_c) {
    const int cb = (int)((kk / BK) % NCB);
    const int64_t e0 = code_elem(g, MODE, pl, kk);
    const int64_t blk = e0 >> 6;
    __builtin_amdgcn_global_load_lds((const void *)(g.codes + (e0 >> 1)),
                                     (lds_void *)&s_C[cb][64 * pw], 16, 0, 0);
    if (DQ) {
      // nb is a multiple of 8 (d % 8 == 0), so the aligned dword is in bounds
      __builtin_amdgcn_global_load_lds((const void *)(g.sc.q + (blk & ~(int64_t)3)),
                                       (lds_void *)&s_Q[cb][64 * pw], 4, 0, 0);
      __builtin_amdgcn_global_load_lds((const void *)(g.sc.s2 + (blk >> 8)),
                                       (lds_void *)&s_S[cb][64 * pw], 4, 0, 0);
    } else {
      __builtin_amdgcn_global_load_lds((const void *)(g.sc.absmax + blk),
                                       (lds_void *)&s_Q[cb][64 * pw], 4, 0, 0);
    }
  }
}

// a' from a fetched scale dword: int8 code byte (blk % 4) times s2 plus mu,
// rounded separately (no fused multiply-add); or the absmax itself.
template <bool DQ>
QL_DEV float scale_of(uint32_t qd, float s2, int64_t blk, float mu) {
  if (!DQ) return __uint_as_float(qd);
  const int q = (int)(int8_t)(qd >> (8 * (blk & 3)));
  const float prod = (float)q * s2;
  return prod + mu;
}

// Forward form decode of stage t into W'[wb]: lane p owns 32 codes of one row.
template <bool DQ>
QL_DEV void decode_fwd(const GemmArgs &g, const Plan &pl, int64_t kk, int wb, int p, float mu) {
  const int cb = (int)((kk / BK) % NCB);
  u32x4 c;
  uint32_t qd;
  float s2;
  // own DMA data; the loads wait in the same asm block
  asm volatile(
      "ds_read_b128 %0, %3\n\t"
      "ds_read_b32 %1, %4\n\t"
      "ds_read_b32 %2, %5\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(c), "=&v"(qd), "=&v"(s2)
      : "v"(lds_addr(&s_C[cb][p])), "v"(lds_addr(&s_Q[cb][p])), "v"(lds_addr(&s_S[cb][p])));
  const int64_t blk = (pl.row * g.k + kk) >> 6;
  const float a = scale_of<DQ>(qd, s2, blk, mu);
  const char *lvb = (const char *)s_lv;
  const int n = p >> 1, half = p & 1;
  // byte b of a code word holds elements 2b (high nibble) and 2b+1 (low
  // nibble); spread them into byte lanes pre-multiplied by 4 (LDS address)
  float f[32];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t ev4 = (c[i] >> 2) & 0x3C3C3C3Cu;
    const uint32_t od4 = (c[i] << 2) & 0x3C3C3C3Cu;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      f[8 * i + 2 * b] = *(const float *)(lvb + __builtin_amdgcn_ubfe(ev4, 8 * b, 8));
      f[8 * i + 2 * b + 1] = *(const float *)(lvb + __builtin_amdgcn_ubfe(od4, 8 * b, 8));
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint4 o;
    o.x = ql::pack_bf16x2(f[8 * i + 0] * a, f[8 * i + 1] * a);
    o.y = ql::pack_bf16x2(f[8 * i + 2] * a, f[8 * i + 3] * a);
    o.z = ql::pack_bf16x2(f[8 * i + 4] * a, f[8 * i + 5] * a);
    o.w = ql::pack_bf16x2(f[8 * i + 6] * a, f[8 * i + 7] * a);
    s_W[wb][swz(n, 4 * half + i)] = o;
  }
}

// dX form decode of stage t into W'[wb]: lane p (jg = p/32, kg = p%32) turns
// rows 8jg..8jg+7, columns 4kg..4kg+3 of the stage's codes (row r occupies
// lanes 4r..4r+3, 64 bytes) into 4 column fragments of 8 consecutive rows.
template <bool DQ>
QL_DEV void decode_dx(const GemmArgs &g, int64_t n0, int64_t kk, int wb, int p, float mu) {
  const int cb = (int)((kk / BK) % NCB);
  const int jg = p >> 5, kg = p & 31, bsel = kg >> 4;
  uint32_t raw[8], qd[8];
  float s2[8];
  const uint32_t ra = lds_addr(&s_C[cb][0]) + 8 * jg * 64 + 2 * kg;
  const uint32_t qa = lds_addr(&s_Q[cb][32 * jg + 2 * bsel]);
  const uint32_t sa = lds_addr(&s_S[cb][32 * jg + 2 * bsel]);
  asm volatile(
      "ds_read_u16 %0, %24\n\t"
      "ds_read_u16 %1, %24 offset:64\n\t"
      "ds_read_u16 %2, %24 offset:128\n\t"
      "ds_read_u16 %3, %24 offset:192\n\t"
      "ds_read_u16 %4, %24 offset:256\n\t"
      "ds_read_u16 %5, %24 offset:320\n\t"
      "ds_read_u16 %6, %24 offset:384\n\t"
      "ds_read_u16 %7, %24 offset:448\n\t"
      "ds_read_b32 %8, %25\n\t"
      "ds_read_b32 %9, %25 offset:16\n\t"
      "ds_read_b32 %10, %25 offset:32\n\t"
      "ds_read_b32 %11, %25 offset:48\n\t"
      "ds_read_b32 %12, %25 offset:64\n\t"
      "ds_read_b32 %13, %25 offset:80\n\t"
      "ds_read_b32 %14, %25 offset:96\n\t"
      "ds_read_b32 %15, %25 offset:112\n\t"
      "ds_read_b32 %16, %26\n\t"
      "ds_read_b32 %17, %26 offset:16\n\t"
      "ds_read_b32 %18, %26 offset:32\n\t"
      "ds_read_b32 %19, %26 offset:48\n\t"
      "ds_read_b32 %20, %26 offset:64\n\t"
      "ds_read_b32 %21, %26 offset:80\n\t"
      "ds_read_b32 %22, %26 offset:96\n\t"
      "ds_read_b32 %23, %26 offset:112\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(raw[0]), "=&v"(raw[1]), "=&v"(raw[2]), "=&v"(raw[3]), "=&v"(raw[4]),
        "=&v"(raw[5]), "=&v"(raw[6]), "=&v"(raw[7]), "=&v"(qd[0]), "=&v"(qd[1]),
        "=&v"(qd[2]), "=&v"(qd[3]), "=&v"(qd[4]), "=&v"(qd[5]), "=&v"(qd[6]), "=&v"(qd[7]),
        "=&v"(s2[0]), "=&v"(s2[1]), "=&v"(s2[2]), "=&v"(s2[3]), "=&v"(s2[4]), "=&v"(s2[5]),
        "=&v"(s2[6]), "=&v"(s2[7])
      : "v"(ra), "v"(qa), "v"(sa));
  int64_t col = n0 + 64 * bsel;
  col = col < g.k ? col : g.k - 32;
  float a[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t j = kk + 8 * jg + i;
    const int64_t jc = j < g.d ? j : g.d - 1;
    const int64_t blk = (jc * g.k + col) >> 6;
    a[i] = j < g.d ? scale_of<DQ>(qd[i], s2[i], blk, mu) : 0.0f;  // rows past d: zero
  }
  const float *lv = s_lv;
  uint32_t o[4][4];  // [column cc][row pair]
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t c0 = raw[2 * q], c1 = raw[2 * q + 1];
    const float a0 = a[2 * q], a1 = a[2 * q + 1];
    o[0][q] = ql::pack_bf16x2(lv[(c0 >> 4) & 15] * a0, lv[(c1 >> 4) & 15] * a1);
    o[1][q] = ql::pack_bf16x2(lv[c0 & 15] * a0, lv[c1 & 15] * a1);
    o[2][q] = ql::pack_bf16x2(lv[(c0 >> 12) & 15] * a0, lv[(c1 >> 12) & 15] * a1);
    o[3][q] = ql::pack_bf16x2(lv[(c0 >> 8) & 15] * a0, lv[(c1 >> 8) & 15] * a1);
  }
#pragma unroll
  for (int cc = 0; cc < 4; ++cc)
    s_W[wb][swz(4 * kg + cc, jg)] = make_uint4(o[cc][0], o[cc][1], o[cc][2], o[cc][3]);
}

template <int MODE, bool DQ>
__global__ __launch_bounds__(NT, 1) void nf4_gemm_kernel(GemmArgs g) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const bool producer = wave >= 4;
  const int p = tid - 256;      // producer thread index 0..255
  const int pw = wave - 4;      // producer wave 0..3
  if (tid < 16) s_lv[tid] = __uint_as_float(c_levels_g[tid]);

  // XCD-aware tile order
  const int64_t ntn = ql_cdiv(g.Ntot, BN), ntm = ql_cdiv(g.M, BM);
  const int64_t total = ntn * ntm;
  int64_t tile = blockIdx.x;
  if ((total & 7) == 0) tile = (int64_t)(blockIdx.x & 7) * (total >> 3) + (blockIdx.x >> 3);
  const int64_t tm = tile / ntn, tn = tile % ntn;
  const int64_t m0 = tm * BM, n0 = tn * BN;
  const float mu = DQ ? g.sc.mu[0] : 0.0f;
  const int64_t nk = ql_cdiv(g.Ktot, BK);
  __syncthreads();  // level table

  // ---- producers -------------------------------------------------------------
  // Step s issues the In tile of step s+2 and the codes of step s+3, then
  // decodes the codes of step s+1 into W'[(s+1) % 2]. Barriers are bare
  // s_barrier; before each one the producers wait (vmcnt) exactly for the
  // loads that the next step needs: vector-memory loads retire in issue order.
  if (producer) {
    const Plan pl = make_plan(g, MODE, m0, n0, pw, lane, p);
    constexpr int L = kLoadsPerStep<DQ>(), LC = L - 8;
    auto decode = [&](int64_t t) {
      if (MODE == 0)
        decode_fwd<DQ>(g, pl, t * BK, (int)(t & 1), p, mu);
      else
        decode_dx<DQ>(g, n0, t * BK, (int)(t & 1), p, mu);
    };
    // prologue: In tiles 0, 1 and codes 0, 1, 2; decode codes 0
    issue_step<MODE, DQ>(g, 0, true, true, pw, lane, p, pl);
    issue_step<MODE, DQ>(g, BK, nk > 1, nk > 1, pw, lane, p, pl);
    issue_step<MODE, DQ>(g, 2 * BK, false, nk > 2, pw, lane, p, pl);
    __builtin_amdgcn_s_waitcnt(0);
    if (MODE == 1) block_sync();  // every lane's codes of stage 0 visible
    decode(0);
    wait_lgkm0();
    block_sync();
    int64_t s = 0;
    for (; s + 3 < nk; ++s) {
      // the In tile of step s+2 < nk-1 is never the partial last one
      issue_step<MODE, DQ, true>(g, (s + 2) * BK, true, false, pw, lane, p, pl);
      issue_step<MODE, DQ>(g, (s + 3) * BK, false, true, pw, lane, p, pl);
      asm volatile("" ::: "memory");
      if (MODE == 0) {
        // own codes of step s+1 (issued two steps ago) landed
        wait_vm_le<8 + LC + 8 + LC>();
        decode(s + 1);
        // In tile of step s+1 (issued last step, before the codes of s+2) landed
        wait_vm_le<LC + 8 + LC>();
      } else {
        // codes of step s+1 landed before the last barrier
        decode(s + 1);
        // In tile of s+1 and codes of s+2 (issued last step) landed
        wait_vm_le<8 + LC>();
      }
      wait_lgkm0();
      block_sync();
    }
    for (; s < nk; ++s) {   // tail: synchronous
      __builtin_amdgcn_s_waitcnt(0);
      issue_step<MODE, DQ>(g, (s + 2) * BK, s + 2 < nk, false, pw, lane, p, pl);
      if (s + 1 < nk) decode(s + 1);
      __builtin_amdgcn_s_waitcnt(0);
      block_sync();
    }
    return;
  }

  // ---- consumers --------------------------------------------------------------
  block_sync();
  if (MODE == 1) block_sync();

  f32x16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  const int wn = wave & 1, wm = (wave >> 1) & 1;
  const int r32 = lane & 31, hk = lane >> 5;

  for (int64_t s = 0; s < nk; ++s) {
    const uint4 *W = s_W[s & 1];
    const uint4 *Xs = s_X[s % NXB];
    // all operand fragments of the step are read up front (one LDS latency
    // per step instead of one per 16-wide K slice), then 32 MFMAs back to back
    uint4 a[4][2], b[4][4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int chunk = 2 * ks + hk;
#pragma unroll
      for (int i = 0; i < 2; ++i) a[ks][i] = W[swz(wn * 64 + 32 * i + r32, chunk)];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[ks][j] = Xs[swz(wm * 128 + 32 * j + r32, chunk)];
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = ql::mfma32(a[ks][i], b[ks][j], acc[i][j]);
    __builtin_amdgcn_sched_group_barrier(0x100, 24, 0);  // the 24 LDS reads first
    __builtin_amdgcn_sched_group_barrier(0x008, 32, 0);  // then the 32 MFMAs
    block_sync();
  }

  // ---- LoRA rank-r term: two extra K-chunks per 16 of rp (hi and lo of S) ----
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

  // ---- store: lane holds D[8(e/4) + 4(l/32) + e%4][l%32] = Out[m][n] ---------
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
  const unsigned grid = (unsigned)tiles;
  if (mode == 0) {
    if (g.sc.dq)
      nf4_gemm_kernel<0, true><<<grid, NT, 0, st>>>(g);
    else
      nf4_gemm_kernel<0, false><<<grid, NT, 0, st>>>(g);
  } else {
    if (g.sc.dq)
      nf4_gemm_kernel<1, true><<<grid, NT, 0, st>>>(g);
    else
      nf4_gemm_kernel<1, false><<<grid, NT, 0, st>>>(g);
  }
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
