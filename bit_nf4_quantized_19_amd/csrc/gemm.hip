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
// row (forward) or per 8-row column strip (dX); one workgroup of eight waves
// per CU, two waves per SIMD (so one wave's LDS waits are covered by the
// other's matrix work), every wave doing all of:
//   * fetching its eighth of the step's In tile (256 rows x 128 bytes) by
//     LDS DMA (global_load_lds, 16 bytes per lane), three stages, two steps
//     ahead. On this part LDS DMA moves about three times the bytes per clock
//     that loads into registers do, and the In tile is the bulk of the bytes
//     a CU reads;
//   * fetching codes (waves 0-3) or block-scale words (waves 4-7) three
//     steps ahead, also by LDS DMA;
//   * decoding its share of the next step's W' tile (16 weights per lane)
//     into LDS, three stages (forward: levels from a 16-entry LDS table
//     times the row's a'; dX: each lane first writes four entries of a
//     per-row table of the 16 products bf16(level * a') over its wave's
//     codes in the code stage, then reads each weight's product with one
//     2-byte load, which needs no multiply or rounding per weight);
//   * 16 v_mfma_f32_32x32x16_bf16 per step on its 64 (n) x 64 (m) eighth of
//     the tile (2 x 4 waves), operands read from LDS.
// Timeline probes of the four-wave form (one wave per SIMD, 64 x 128 per
// wave) showed each wave's step dominated by its own LDS waits; with two
// waves per SIMD the operand reads grow by a third but the waits overlap.
// K order inside a step: MFMA K-slice c, lane half h covers K = 16c + 8h ..
// +7 for both operands. LDS rows of 128 bytes are stored with the 16-byte
// chunks permuted by f(row) = (row ^ row>>2) & 7 (conflict-free operand reads,
// DMA row groups and decoded-tile writes). Every LDS stage is a separate
// object and the main loop is unrolled by three, so each access names its
// stage at compile time. The DMAs are issued from inline asm: the main loop
// has no vector-memory instruction the compiler knows of, so it inserts no
// vmcnt waits of its own; one barrier per K-step, before which each wave
// waits (vmcnt, in-order retirement) exactly for its own DMAs of the next
// step, orders everything.
// Workgroups are mapped XCD-aware: the 32 column tiles of one token block
// land on the same XCD, whose L2 then holds that In block.
#include "kernels.h"
#include "nf4_tables.h"

namespace {

constexpr int BN = 128, BM = 256, BK = 64, NT = 512;
__constant__ uint32_t c_levels_g[16] = NF4_LEVEL_BITS;

struct GemmArgs {
  const uint8_t *codes;
  ql::ScaleSrc sc;
  int64_t d, k;          // weight shape
  const uint16_t *In;    // M x Ktot
  int64_t M;
  int64_t Ntot, Ktot;    // output columns, contraction length
  const uint16_t *L;     // L[n][t] = L[n * r + t] (forward: B) or L[t * Ntot + n] (dX: A)
  const uint16_t *Shi, *Slo;  // M x rp
  int r, rp;
  uint16_t *Out;         // M x Ntot
  const uint8_t *keep;   // dX with adapter-input dropout: keep nibbles (M x Ntot/4), else NULL
  float inv_keep;        // 1/(1-p)
};

// LDS, one object per stage. The level table is the most aligned object, so
// it is placed at LDS address 0 and the forward decode's table addresses need
// no base added (an instruction offset cannot reach the top of 160 KB).
__shared__ __align__(1024) float s_lv[16];
__shared__ uint4 s_X0[BM * 8], s_X1[BM * 8], s_X2[BM * 8];  // In tiles, 256 rows x 128 B
__shared__ uint4 s_W0[BN * 8], s_W1[BN * 8], s_W2[BN * 8];  // W' tiles, 128 rows x 128 B
// codes, 16 B per lane (256-byte aligned: the dX decode's product tables
// overwrite them in place, addressed by byte permutes within 256-byte windows)
__shared__ __align__(256) uint4 s_C0[256], s_C1[256], s_C2[256];
__shared__ uint32_t s_Q0[128], s_Q1[128], s_Q2[128];        // scale dword per entry
__shared__ float s_S0[128], s_S1[128], s_S2[128];           // s2 per entry

template <int S> QL_DEV uint4 *sX() { return S == 0 ? s_X0 : S == 1 ? s_X1 : s_X2; }
template <int S> QL_DEV uint4 *sW() { return S == 0 ? s_W0 : S == 1 ? s_W1 : s_W2; }
template <int S> QL_DEV uint4 *sC() { return S == 0 ? s_C0 : S == 1 ? s_C1 : s_C2; }
template <int S> QL_DEV uint32_t *sQ() { return S == 0 ? s_Q0 : S == 1 ? s_Q1 : s_Q2; }
template <int S> QL_DEV float *sS() { return S == 0 ? s_S0 : S == 1 ? s_S1 : s_S2; }

QL_DEV int swz(int row, int chunk) { return row * 8 + (chunk ^ ((row ^ (row >> 2)) & 7)); }

QL_DEV uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

// LDS DMA: each lane's 16 (or 4) bytes at gptr land at LDS address
// lds + 16 * lane (4 * lane); lds must be wave-uniform. M0 carries the LDS
// base; nothing else in these kernels uses M0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
QL_DEV void dma16(const void *gptr, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(gptr), "s"(lds) : "memory", "m0");
}
QL_DEV void dma4(const void *gptr, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :: "v"(gptr), "s"(lds) : "memory", "m0");
}
#pragma clang diagnostic pop

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

// a' from a scale dword: int8 code byte (blk % 4) times s2 plus mu, rounded
// separately (no fused multiply-add); or the absmax itself.
template <bool DQ>
QL_DEV float scale_of(uint32_t qd, float s2, int64_t blk, float mu) {
  if (!DQ) return __uint_as_float(qd);
  const int q = (int)(int8_t)(qd >> (8 * (blk & 3)));
  const float prod = (float)q * s2;
  return prod + mu;
}

// DMAs each wave issues per step: 4 for its eighth of the In tile and 1 for
// codes (waves 0-3) or scale words (waves 4-7).
constexpr int kLoadsPerStep = 5;

template <int MODE, bool DQ>
struct Tile {
  GemmArgs g;
  int tid, lane, wave, r32, h, wn, wm;
  int64_t m0, n0, nk;
  float mu;
  int64_t xoff[4];    // byte offsets of this lane's 4 In DMA chunks (from In + kk)
  // code DMA (waves 0-3): forward weight row (clamped) and half block; dX code
  // row inside the step and first column. Scale DMA (waves 4-7): forward
  // weight row; dX entry row and block column. Decode: forward weight row;
  // dX block column.
  int64_t crow64, srow64, drow64;
  int chalf, crow_off, ccol, srow, sblk, dcol;
  // dX decode (patch rows 4jg..4jg+3, columns 4kg..4kg+3 of the step): the
  // product-table entries this thread builds, levels 4 tm .. 4 tm + 3 of
  // table row tr (and the bit offset of that row's int8 scale code in its
  // dword: row j of step kk is kk + 4 jg + tr with kk a multiple of 64, so
  // j % 4 == tr and the block index j (k / 64) + dcol / 64 has the same value
  // mod 4 in every step); the byte offset of that entry pair in the stage;
  // the tables' 256-byte window (jg) and the rows' offsets in it.
  int tr, tqsh, toff, twin;
  float tlv[4];
  uint32_t roff[2];

  f32x16 acc[2][2];
  // the rank-r epilogue's operands of rank chunk 0 (L rows of the forward's
  // whole-piece path, and the S hi/lo parts), loaded before the last K-steps
  uint4 pre_a[2], pre_b[2][2];

  // tile (tm, tn): token rows tm*BM.., output columns tn*BN..
  QL_DEV void init(const GemmArgs &ga, int64_t tm, int64_t tn) {
    g = ga;
    tid = threadIdx.x;
    lane = tid & 63;
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    r32 = lane & 31;
    h = lane >> 5;
    wn = wave & 1;
    wm = wave >> 1;
    m0 = tm * BM;
    n0 = tn * BN;
    nk = ql_cdiv(g.Ktot, BK);
    mu = DQ ? g.sc.mu[0] : 0.0f;
    // In DMA: wave w fetches rows 32w .. 32w+31 in 4 groups of 8 rows; lane l
    // of a group fetches the chunk that the LDS permutation puts at slot l%8
    // of row l/8 (the DMA writes lane l's 16 bytes at group base + 16 l).
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 32 * wave + 8 * i + (lane >> 3);
      const int chunk = (lane & 7) ^ ((row ^ (row >> 2)) & 7);
      int64_t m = m0 + row;
      m = m < g.M ? m : g.M - 1;  // rows past M: duplicate data, outputs discarded
      xoff[i] = (m * g.Ktot + 8 * chunk) * 2;
    }
    const int p = 64 * (wave & 3) + lane;   // code DMA lane (waves 0-3)
    const int e = 64 * (wave & 1) + lane;   // scale DMA entry (waves 4-7)
    if (MODE == 0) {
      const int64_t cr = n0 + (p >> 1);
      crow64 = cr < g.d ? cr : g.d - 1;   // rows past d feed only discarded outputs
      chalf = p & 1;
      const int64_t sr = n0 + e;          // scale entry = tile row
      srow64 = sr < g.d ? sr : g.d - 1;
      const int64_t dr = n0 + (tid >> 2);
      drow64 = dr < g.d ? dr : g.d - 1;
    } else {
      crow_off = p >> 2;                  // code row inside the step
      const int64_t col = n0 + 32 * (p & 3);
      ccol = (int)(col < g.k ? col : g.k - 32);  // columns past k: discarded outputs
      srow = e >> 1;                      // scale entry 2r + b
      const int64_t c0 = n0 + 64 * (e & 1);
      sblk = (int)(c0 < g.k ? c0 : g.k - 64);
      const int64_t dc = n0 + 64 * (((tid >> 1) & 31) >> 4);
      dcol = (int)(dc < g.k ? dc : g.k - 64);
      const int jg = 2 * (tid >> 6) + (tid & 1), kg = (tid >> 1) & 31, bsel = kg >> 4;
      tr = (kg & 15) >> 2;
      const int tm = kg & 3;
      tqsh = 8 * (int)(((uint32_t)tr * (uint32_t)(g.k >> 6) + (uint32_t)(dcol >> 6)) & 3u);
      // table (patch row i, block b) holds bf16(level[c] * a') at byte 2c of
      // 32-byte slot (2i + b + 2 (jg % 2)) % 8 of the 256-byte window of rows
      // 4jg..4jg+3, i.e. over codes of those rows, which the same wave reads
      // before it overwrites them; the rotation by jg puts the four tables
      // one lookup instruction of a wave reads (two windows, two blocks) on
      // four different groups of 8 LDS banks
      const int rot = 2 * (jg & 1);
      toff = 256 * jg + ((2 * tr + bsel + rot) & 7) * 32 + 8 * tm;
      twin = 256 * jg;
#pragma unroll
      for (int x = 0; x < 4; ++x) tlv[x] = __uint_as_float(c_levels_g[4 * tm + x]);
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const uint32_t ra = (uint32_t)((4 * h2 + bsel + rot) & 7) * 32u;
        const uint32_t rb = (uint32_t)((4 * h2 + 2 + bsel + rot) & 7) * 32u;
        roff[h2] = ra | (ra << 8) | (rb << 16) | (rb << 24);
      }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;
  }

  // Row group i (8 rows, 1 KB) of this wave's eighth of the In tile of step
  // kk into stage ST by LDS DMA (chunks past Ktot fetch the last valid chunk:
  // finite data times a zero W').
  template <int ST, bool FULL>
  QL_DEV void issue_x(int64_t kk, int i) {
    int64_t off = xoff[i];   // signed: the clamp below may step back past In + kk
    if (!FULL) {
      const int row = 32 * wave + 8 * i + (lane >> 3);
      const int chunk = (lane & 7) ^ ((row ^ (row >> 2)) & 7);
      if (kk + 8 * chunk >= g.Ktot) off -= (kk + 8 * chunk - (g.Ktot - 8)) * 2;
    }
    dma16((const char *)(g.In + kk) + off, lds_addr(&sX<ST>()[(32 * wave + 8 * i) * 8]));
  }
  template <int ST, bool FULL>
  QL_DEV void issue_x_all(int64_t kk) {
#pragma unroll
    for (int i = 0; i < 4; ++i) issue_x<ST, FULL>(kk, i);
  }

  // Codes (waves 0-3) or scale words (waves 4-7) of step kk into code stage
  // ST (LDS DMA). Forward: lane p fetches 32 codes of tile row p/2; scale
  // entry e (waves 4-5: int8-code dword or absmax, waves 6-7: s2 or absmax
  // again) is tile row e. dX: lane p fetches columns 32(p%4).. of code row
  // p/4; entry e = 2r + b is row r, block column b.
  template <int ST>
  QL_DEV void issue_c(int64_t kk) {
    if (kk >= g.Ktot) kk = (nk - 1) * BK;   // prologue past the end: any valid step
    if (wave < 4) {
      const void *src;
      if (MODE == 0) {
        src = g.codes + ((crow64 * g.k + kk + 32 * chalf) >> 1);
      } else {
        int64_t j = kk + crow_off;
        j = j < g.d ? j : g.d - 1;
        src = g.codes + ((j * g.k + ccol) >> 1);
      }
      dma16(src, lds_addr(&sC<ST>()[64 * wave]));
    } else {
      int64_t blk;
      if (MODE == 0) {
        blk = (srow64 * g.k + kk) >> 6;
      } else {
        int64_t js = kk + srow;
        js = js < g.d ? js : g.d - 1;
        blk = (js * g.k + sblk) >> 6;
      }
      // int8 codes: the aligned dword (nb is a multiple of 8, so in bounds)
      const bool qw = wave < 6;
      const void *src;
      if (DQ)
        src = qw ? (const void *)(g.sc.q + (blk & ~(int64_t)3))
                 : (const void *)(g.sc.s2 + (blk >> 8));
      else
        src = (const void *)(g.sc.absmax + blk);
      dma4(src, qw ? lds_addr(&sQ<ST>()[64 * (wave - 4)]) : lds_addr(&sS<ST>()[64 * (wave - 6)]));
    }
  }

  // ---- decode: the codes of one step into a W' tile ----------------------
  // Forward (two parts): thread t owns code words 2(t%2), +1 of code entry
  // t/2, i.e. 16 weights of tile row t/4; part i turns one word (8 weights)
  // into one 16-byte fragment. dX (four parts): thread t (jg = 2(t/64) +
  // t%2, kg = (t/2)%32) owns rows 4jg..4jg+3, columns 4kg..4kg+3 of the
  // stage's codes (row r at bytes 64r..64r+63); part i writes column 4kg+i,
  // 4 rows (8 bytes). Neighbouring lanes take the two halves of one 16-byte
  // fragment slot, so the 8-byte writes of 16 lanes fall on 16 distinct
  // slots (the row permutation alone gives 8).
  static constexpr int kParts = MODE == 0 ? 2 : 4;
  struct DecIn {
    uint32_t c[4];   // forward: 2 code words; dX: the table-address bytes ev[0..1], od[0..1]
    float a[4];      // forward: a[0] = the row's a'
  };

  template <int CS>
  QL_DEV DecIn dec_load(int64_t kk) {
    DecIn di;
    if (MODE == 0) {
      const uint2 c = ((const uint2 *)sC<CS>())[tid];
      di.c[0] = c.x; di.c[1] = c.y;
      const int64_t blk = (drow64 * g.k + kk) >> 6;
      di.a[0] = scale_of<DQ>(sQ<CS>()[tid >> 2], sS<CS>()[tid >> 2], blk, mu);
    } else {
      // dX: the patch's four rows' code pairs, and the a' of the table row
      // this thread fills
      const int jg = 2 * (tid >> 6) + (tid & 1), kg = (tid >> 1) & 31, bsel = kg >> 4;
      const uint16_t *raw = (const uint16_t *)sC<CS>();
      uint32_t c[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) c[i] = raw[(4 * jg + i) * 32 + kg];
      const uint32_t qd = sQ<CS>()[8 * jg + 2 * tr + bsel];
      const float s2 = sS<CS>()[8 * jg + 2 * tr + bsel];
      float a;
      if (DQ) {
        const int qv = (int)(int8_t)(qd >> tqsh);
        const float prod = (float)qv * s2;
        a = prod + mu;
      } else {
        a = __uint_as_float(qd);
      }
      if (kk + 4 * jg + tr >= g.d) a = 0.0f;   // the last step of a ragged K: rows past d are zero
      // the code reads above and the table write below touch the same bytes;
      // LDS accesses of a wave execute in order, and the asm statements keep
      // the compiler from reordering them
      asm volatile("" ::: "memory");
      *(uint2 *)((char *)sC<CS>() + toff) =
          make_uint2(ql::pack_bf16x2(tlv[0] * a, tlv[1] * a), ql::pack_bf16x2(tlv[2] * a, tlv[3] * a));
      asm volatile("" ::: "memory");
      // table-address bytes, two rows per word: each nibble times 2 plus the
      // row's table offset in the window (ev: high nibbles = columns 4kg and
      // 4kg+2, od: low nibbles = columns 4kg+1 and 4kg+3; row 2 h2 in bytes
      // 0-1, row 2 h2 + 1 in bytes 2-3)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const uint32_t w = c[2 * h2] | (c[2 * h2 + 1] << 16);
        di.c[h2] = ((w >> 3) & 0x1E1E1E1Eu) | roff[h2];
        di.c[2 + h2] = ((w << 1) & 0x1E1E1E1Eu) | roff[h2];
      }
    }
    return di;
  }

  template <int WS>
  QL_DEV void dec_part(const DecIn &di, int i) {
    if (MODE == 0) {
      // byte b of a code word holds elements 2b (high nibble) and 2b+1 (low
      // nibble); spread them into byte lanes pre-multiplied by 4 (LDS address)
      const char *lvb = (const char *)s_lv;
      const uint32_t ev4 = (di.c[i] >> 2) & 0x3C3C3C3Cu;
      const uint32_t od4 = (di.c[i] << 2) & 0x3C3C3C3Cu;
      float f[8];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        // byte b of ev4 / od4 zero-extended by one byte permute (the level
        // table is at LDS address 0, so this is the whole address)
        f[2 * b] = *(const float *)(lvb + __builtin_amdgcn_perm(0u, ev4, 0x0C0C0C00u | (uint32_t)b));
        f[2 * b + 1] = *(const float *)(lvb + __builtin_amdgcn_perm(0u, od4, 0x0C0C0C00u | (uint32_t)b));
      }
      const float a = di.a[0];
      uint4 o;
      o.x = ql::pack_bf16x2(f[0] * a, f[1] * a);
      o.y = ql::pack_bf16x2(f[2] * a, f[3] * a);
      o.z = ql::pack_bf16x2(f[4] * a, f[5] * a);
      o.w = ql::pack_bf16x2(f[6] * a, f[7] * a);
      sW<WS>()[swz(tid >> 2, 4 * ((tid >> 1) & 1) + 2 * (tid & 1) + i)] = o;
    } else {
      // column 4kg+i of the patch: row r's bf16 W' from its table by a
      // 2-byte read, the address = the window's upper bytes with the row's
      // address byte (ev for even columns, od for odd; byte 2 (r%2) + i/2 of
      // word r/2)
      const int jg = 2 * (tid >> 6) + (tid & 1), kg = (tid >> 1) & 31;
      const uint32_t hb = lds_addr(sC<WS>()) + (uint32_t)twin;
      uint32_t v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t x = di.c[(i & 1) * 2 + (r >> 1)];
        const uint32_t sel = 0x07060500u | (uint32_t)(2 * (r & 1) + (i >> 1));
        const uint32_t addr = __builtin_amdgcn_perm(hb, x, sel);
        v[r] = *(const __attribute__((address_space(3))) uint16_t *)(uintptr_t)addr;
      }
      uint2 o;
      o.x = v[0] | (v[1] << 16);
      o.y = v[2] | (v[3] << 16);
      ((uint2 *)sW<WS>())[2 * swz(4 * kg + i, jg >> 1) + (jg & 1)] = o;
    }
  }

  template <int CS, int WS>
  QL_DEV void decode(int64_t t) {
    const DecIn di = dec_load<CS>(t * BK);
#pragma unroll
    for (int i = 0; i < kParts; ++i) dec_part<WS>(di, i);
  }

  // MFMA operands of K-slice c of stage ST: W' rows wn*64.., In rows wm*64..
  template <int ST>
  QL_DEV void load_slice(int c, uint4 (&a)[2], uint4 (&b)[2]) {
#pragma unroll
    for (int i = 0; i < 2; ++i) a[i] = sW<ST>()[swz(wn * 64 + 32 * i + r32, 2 * c + h)];
#pragma unroll
    for (int j = 0; j < 2; ++j) b[j] = sX<ST>()[swz(wm * 64 + 32 * j + r32, 2 * c + h)];
  }

  // One K-step s (ST = s % 3). Main steps (TAIL = false) have s + 3 < nk.
  // Stages: In tile, W' tile and codes of step t live in stage t % 3. The
  // step is cut into its four K-slices; each slice issues the next slice's
  // operand reads, one of this wave's In DMAs of step s+2 (the last one also
  // its code or scale DMA of step s+3), its 4 MFMAs and a share of the decode
  // of step s+1 (forward: slices 1 and 3; dX: every slice), so the decode and
  // the DMA issue overlap the matrix cores of both waves on the SIMD.
  template <int ST, bool TAIL>
  QL_DEV void step(int64_t s) {
    constexpr int S1 = (ST + 1) % 3, S2 = (ST + 2) % 3;
    const bool do_x = !TAIL || s + 2 < nk, do_c = !TAIL || s + 3 < nk;
    const bool do_d = !TAIL || s + 1 < nk;
    DecIn di;
    if (do_d) di = dec_load<S1>((s + 1) * BK);
    uint4 a[2][2], b[2][2];
    load_slice<ST>(0, a[0], b[0]);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if (c < 3) load_slice<ST>(c + 1, a[(c + 1) & 1], b[(c + 1) & 1]);
      if (do_x) issue_x<S2, !TAIL>((s + 2) * BK, c);
      if (c == 3 && do_c) issue_c<ST>((s + 3) * BK);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = ql::mfma32(a[c & 1][i], b[c & 1][j], acc[i][j]);
      if (do_d) {
        if (MODE == 0) {
          if (c & 1) dec_part<S1>(di, c >> 1);
        } else {
          dec_part<S1>(di, c);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // the In tile of step s+1 and the codes of step s+2 (issued last step)
    // have landed: allowed in flight are this step's loads
    if (TAIL)
      __builtin_amdgcn_s_waitcnt(0);
    else
      wait_vm_le<kLoadsPerStep>();
    wait_lgkm0();
    block_sync();
  }

  QL_DEV void run() {
    // prologue (unconditional, with clamped addresses, so the loop is entered
    // with the same loads in flight as it carries around its back edge):
    // codes 0, then In 0 + codes 1, In 1 + codes 2; decode codes 0
    issue_c<0>(0);
    issue_x_all<0, false>(0);
    issue_c<1>(BK);
    issue_x_all<1, false>(BK);
    issue_c<2>(2 * BK);
    wait_vm_le<2 * kLoadsPerStep>();   // codes 0 landed
    block_sync();
    decode<0, 0>(0);
    wait_vm_le<kLoadsPerStep>();       // In 0 and codes 1 landed
    wait_lgkm0();
    block_sync();
    int64_t s = 0;
    for (; s + 5 < nk; s += 3) {
      step<0, false>(s);
      step<1, false>(s + 1);
      step<2, false>(s + 2);
    }
    lora_prefetch();
    for (; s < nk; s += 3) {
      step<0, true>(s);
      if (s + 1 < nk) step<1, true>(s + 1);
      if (s + 2 < nk) step<2, true>(s + 2);
    }
  }

  // LoRA rank-r term: two extra K-chunks per 16 of rp (hi and lo of S), then
  // the bf16 stores. Lane holds D[8(e/4) + 4(l/32) + e%4][l%32] = Out[m][n].
  // With adapter-input dropout (dX only) the rank-r term of each 32 x 32
  // block goes to an accumulator of its own and is added where the input
  // element was kept, times 1/(1-p): dX = dY W' + s (G A) * keep / (1 - p).
  QL_DEV void epilogue() {
    if (MODE == 1 && g.keep) {
      // keep bits of the lane's two token rows: byte (n - bc) / 4 of the
      // wave's 64-column block bc (bit n % 4), one 16-byte load per row,
      // issued before the rank-r products (Ntot % 64 == 0, so a block is
      // either inside the row or wholly past it)
      int64_t bc = n0 + wn * 64;
      bc = bc + 64 <= g.Ntot ? bc : g.Ntot - 64;   // blocks past Ntot: not stored
      uint4 kw[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        int64_t m = m0 + wm * 64 + 32 * j + r32;
        m = m < g.M ? m : g.M - 1;   // rows past M: not stored
        kw[j] = *(const uint4 *)(g.keep + m * (g.Ntot >> 2) + (bc >> 2));
      }
      keep_block<0, 0>(kw);
      keep_block<0, 1>(kw);
      keep_block<1, 0>(kw);
      keep_block<1, 1>(kw);
    } else {
      lora_term<0, 2, 0, 2>(acc);
    }
    store();
  }

  // One 32 x 32 block of the dropout epilogue (one block at a time keeps the
  // extra accumulator at 16 registers).
  template <int I, int J>
  QL_DEV void keep_block(const uint4 (&kw)[2]) {
    f32x16 lacc[1][1];
#pragma unroll
    for (int q = 0; q < 16; ++q) lacc[0][0][q] = 0.0f;
    lora_term<I, 1, J, 1>(lacc);
    const uint32_t w4[4] = {kw[J].x, kw[J].y, kw[J].z, kw[J].w};
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      // columns 32 I + 8 q4 + 4 h of the block: byte 8 I + 2 q4 + h
      const uint32_t kb = w4[2 * I + (q4 >> 1)] >> (8 * (2 * (q4 & 1) + h));
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if ((kb >> e) & 1u) acc[I][J][4 * q4 + e] += lacc[0][0][4 * q4 + e] * g.inv_keep;
    }
  }

  // Unconditional loads from clamped addresses (their latency then runs
  // under the last K-steps); out-of-range lanes are zeroed where used.
  QL_DEV void lora_prefetch() {
    if (MODE == 0 && g.r % 8 == 0) {
      const int tq = 8 * h < g.r ? 8 * h : g.r - 8;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int64_t n = n0 + wn * 64 + 32 * i + r32;
        const int64_t nc = n < g.Ntot ? n : g.Ntot - 1;
        pre_a[i] = *(const uint4 *)(g.L + nc * g.r + tq);
      }
    }
#pragma unroll
    for (int part = 0; part < 2; ++part) {
      const uint16_t *S = part ? g.Slo : g.Shi;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int64_t m = m0 + wm * 64 + 32 * j + r32;
        const int64_t mc = m < g.M ? m : g.M - 1;
        pre_b[part][j] = *(const uint4 *)(S + mc * g.rp + 8 * h);
      }
    }
  }

  // the rank-r term of the 32 x 32 blocks (I0 .., J0 ..), NI x NJ of them
  template <int I0, int NI, int J0, int NJ>
  QL_DEV void lora_term(f32x16 (&dst)[NI][NJ]) {
    for (int t0 = 0; t0 < g.rp; t0 += 16) {
      // L[n][t0 + 8h .. +7] read in place (ranks past r and n past Ntot: 0);
      // loads from clamped addresses, the zeroing applied afterwards
      uint4 a[NI];
      if (MODE == 0 && g.r % 8 == 0) {
        // forward, B rows of whole 16-byte pieces: one load per operand
        const int tq = t0 + 8 * h;
#pragma unroll
        for (int ii = 0; ii < NI; ++ii) {
          const int64_t n = n0 + wn * 64 + 32 * (I0 + ii) + r32;
          const int64_t nc = n < g.Ntot ? n : g.Ntot - 1;
          const uint4 v = t0 == 0 ? pre_a[I0 + ii]
                                  : *(const uint4 *)(g.L + nc * g.r + (tq < g.r ? tq : g.r - 8));
          a[ii] = (n < g.Ntot && tq < g.r) ? v : ql::zero4();
        }
      } else {
        // gather: all loads issued before any use
        uint32_t e[NI][8];
#pragma unroll
        for (int ii = 0; ii < NI; ++ii) {
          const int64_t n = n0 + wn * 64 + 32 * (I0 + ii) + r32;
          const int64_t nc = n < g.Ntot ? n : g.Ntot - 1;
#pragma unroll
          for (int x = 0; x < 8; ++x) {
            const int t = t0 + 8 * h + x, tc = t < g.r ? t : g.r - 1;
            e[ii][x] = g.L[MODE == 0 ? nc * g.r + tc : (int64_t)tc * g.Ntot + nc];
          }
        }
#pragma unroll
        for (int ii = 0; ii < NI; ++ii) {
          const bool n_ok = n0 + wn * 64 + 32 * (I0 + ii) + r32 < g.Ntot;
          uint32_t w[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int t = t0 + 8 * h + 2 * q;
            const uint32_t lo = (n_ok && t < g.r) ? e[ii][2 * q] : 0u;
            const uint32_t hi = (n_ok && t + 1 < g.r) ? e[ii][2 * q + 1] : 0u;
            w[q] = lo | (hi << 16);
          }
          a[ii] = make_uint4(w[0], w[1], w[2], w[3]);
        }
      }
#pragma unroll
      for (int part = 0; part < 2; ++part) {
        const uint16_t *S = part ? g.Slo : g.Shi;
        uint4 b[NJ];
#pragma unroll
        for (int jj = 0; jj < NJ; ++jj) {
          const int64_t m = m0 + wm * 64 + 32 * (J0 + jj) + r32;
          if (t0 == 0)
            b[jj] = m < g.M ? pre_b[part][J0 + jj] : ql::zero4();
          else
            b[jj] = (m < g.M) ? *(const uint4 *)(S + m * g.rp + t0 + 8 * h) : ql::zero4();
        }
#pragma unroll
        for (int ii = 0; ii < NI; ++ii)
#pragma unroll
          for (int jj = 0; jj < NJ; ++jj) dst[ii][jj] = ql::mfma32(a[ii], b[jj], dst[ii][jj]);
      }
    }
  }

  QL_DEV void store() {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int64_t m = m0 + wm * 64 + 32 * j + r32;
        if (m >= g.M) continue;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int64_t n = n0 + wn * 64 + 32 * i + 8 * q4 + 4 * h;
          if (n >= g.Ntot) continue;
          uint2 o;
          o.x = ql::pack_bf16x2(acc[i][j][4 * q4 + 0], acc[i][j][4 * q4 + 1]);
          o.y = ql::pack_bf16x2(acc[i][j][4 * q4 + 2], acc[i][j][4 * q4 + 3]);
          *(uint2 *)(g.Out + m * g.Ntot + n) = o;
        }
      }
  }
};

// Workgroup -> tile, XCD-aware: with 8 XCDs taking workgroups round-robin,
// consecutive tiles (the column tiles of one token block) land on one XCD,
// whose L2 then holds that token block.
QL_DEV void tile_of(int64_t ntn, int64_t ntm, int64_t &tm, int64_t &tn) {
  const int64_t total = ntn * ntm;
  int64_t tile = blockIdx.x;
  if ((total & 7) == 0) tile = (int64_t)(blockIdx.x & 7) * (total >> 3) + (blockIdx.x >> 3);
  tm = tile / ntn;
  tn = tile % ntn;
}

template <int MODE, bool DQ>
__global__ __launch_bounds__(NT, 1) void nf4_gemm_kernel(GemmArgs g) {
  if (threadIdx.x < 16) s_lv[threadIdx.x] = __uint_as_float(c_levels_g[threadIdx.x]);
  int64_t tm, tn;
  tile_of(ql_cdiv(g.Ntot, BN), ql_cdiv(g.M, BM), tm, tn);
  Tile<MODE, DQ> t;
  t.init(g, tm, tn);
  __syncthreads();  // level table
  t.run();
  t.epilogue();
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
                             const uint16_t *X, int64_t M, const uint16_t *B, int r,
                             const uint16_t *Hs_hi, const uint16_t *Hs_lo, int rp,
                             uint16_t *Y, hipStream_t st) {
  GemmArgs g{codes, sc, d, k, X, M, d, k, B, Hs_hi, Hs_lo, r, rp, Y};
  return launch_gemm(0, g, st);
}

qlora_status launch_gemm_dx(const uint8_t *codes, ql::ScaleSrc sc, int64_t d, int64_t k,
                            const uint16_t *dY, int64_t M, const uint16_t *A, int r,
                            const uint16_t *Gs_hi, const uint16_t *Gs_lo, int rp,
                            uint16_t *dX, const uint8_t *keep, float inv_keep, hipStream_t st) {
  GemmArgs g{codes, sc, d, k, dY, M, k, d, A, Gs_hi, Gs_lo, r, rp, dX, keep, inv_keep};
  return launch_gemm(1, g, st);
}
