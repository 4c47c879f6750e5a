// Host launchers of the gfx950 kernels (internal; the C ABI in capi.hip
// validates arguments and calls these).
#pragma once

#include "common.h"
#include "philox.h"

// quantize.hip
qlora_status launch_quantize(const uint16_t *W0, int64_t n, uint8_t *codes,
                             float *absmax_out, int dq, int8_t *q, float *s2,
                             float *mu, void *ws, hipStream_t st);
size_t quantize_ws_bytes(int64_t n, int dq);

// Output buffers of one quantisation (the fields of qlora_nf4_weight) and
// the same record read back as a scale source.
struct QuantOut {
  uint8_t *codes;
  float *absmax;
  int8_t *q;
  float *s2;
  float *mu;
  ql::ScaleSrc sc;
};

// loftq.hip
size_t loftq_ws_bytes(int64_t d, int64_t k, int r, int dq);
size_t residual_quantize_ws_bytes(int64_t d, int64_t k, int dq);
// NF4 (+DQ) of bf16(W - s B A) into qo; Wt (d x k bf16) and qws are scratch.
qlora_status launch_residual_quantize(const uint16_t *W, const uint16_t *A, const uint16_t *B,
                                      int64_t d, int64_t k, int r, float s, const QuantOut &qo,
                                      uint16_t *Wt, void *qws, hipStream_t st);
qlora_status launch_residual_quantize_ws(const uint16_t *W, const uint16_t *A, const uint16_t *B,
                                         int64_t d, int64_t k, int r, float s, const QuantOut &qo,
                                         void *ws, hipStream_t st);
qlora_status launch_loftq(const uint16_t *W, const float *omega, int64_t d, int64_t k, int r,
                          float s, int iters, int power_iters, const QuantOut &qo, uint16_t *A,
                          uint16_t *B, float *sigma, void *ws, hipStream_t st);

// dequant.hip
qlora_status launch_dequantize(const uint8_t *codes, ql::ScaleSrc sc, int64_t n,
                               uint16_t *out, hipStream_t st);

// lora_small.hip : small LoRA contractions and layout helpers
// Up to four zero-padded / transposed bf16 copies in one launch:
// dst (drows x dcols) [i][j] = src[i][j] (or src[j][i] when transpose), zero
// outside src (rows x cols). Requests with dst == NULL are skipped.
struct LayoutReq {
  const uint16_t *src;
  int64_t rows, cols;
  uint16_t *dst;
  int64_t drows, dcols;
  int transpose;
};
qlora_status launch_layout(const LayoutReq *req, int nreq, hipStream_t st);
// out[m][t] (fp32, M x rp) = sum_c In[m][c] * P[t][c] for t < r (zero for
// r <= t < rp), one launch. P[t][c] = P[t * C + c] (p_col false: r x C) or
// P[c * r + t] (p_col true: C x r, requires r % 16 == 0). out2 (optional)
// receives the first out2_ld columns with leading dim out2_ld. Also writes
// s*out split into bf16 hi/lo (M x rp each) when hi != NULL.
// zero (optional): nzero ints cleared by the launch, for a later launch of
// the same call (the colacc counters).
qlora_status launch_skinny(const uint16_t *In, int64_t M, int64_t C, const uint16_t *P,
                           bool p_col, int r, int rp, float *out, float *out2, int out2_ld,
                           float s, uint16_t *hi, uint16_t *lo, hipStream_t st,
                           int *zero = nullptr, int64_t nzero = 0);
// The same for nw (1..4) contractions of one In (sibling projections) in one
// launch: o[i] = {P, out, out2, hi, lo} of contraction i.
struct SkinnyOut {
  const uint16_t *P;
  float *out, *out2;
  uint16_t *hi, *lo;
  DropParams dp;   // dropout on In (row form only; dp.on == 0: none)
};
qlora_status launch_skinny(const uint16_t *In, int64_t M, int64_t C, int nw, const SkinnyOut *o,
                           bool p_col, int r, int rp, int out2_ld, float s, hipStream_t st,
                           int *zero = nullptr, int64_t nzero = 0);
// Two problems out = s * sum_m In[m][c] * Q[m][t] rounded to bf16 (In M x C,
// Q M x rp fp32) in one launch, including the reduction of its token splits.
// transpose_out == 0: out is C x r (ld r); == 1: out is r x C (ld C).
struct ColaccReq {
  const uint16_t *In;
  int64_t C;
  const float *Q;
  uint16_t *out;
  int transpose_out;
  DropParams dp;     // dropout of In (dp.on == 0: none); the result is scaled by 1/(1-p)
  uint8_t *keep;     // with dropout: M x C/4 keep nibbles written here (may be NULL)
};
// part: colacc_part_bytes(M, a.C, b.C, rp) bytes of workspace, holding the
// split partial sums and colacc_counter_count(a.C, b.C) counters at
// colacc_counters(part, ...), which must be zero when the launch starts (the
// G launch of the same call clears them) and are zero when it ends.
qlora_status launch_colacc2(const ColaccReq &a, const ColaccReq &b, int64_t M, int rp,
                            int r, float s, float *part, hipStream_t st);
size_t colacc_part_bytes(int64_t M, int64_t C0, int64_t C1, int rp);
int64_t colacc_counter_count(int64_t C0, int64_t C1);
int *colacc_counters(float *part, int64_t M, int64_t C0, int64_t C1, int rp);

// gemm.hip : fused dequant-GEMM, forward (Y) and input-gradient (dX) forms.
// The rank-r epilogue reads B (d x r) resp. A (r x k) in place.
qlora_status launch_gemm_fwd(const uint8_t *codes, ql::ScaleSrc sc, int64_t d,
                             int64_t k, const uint16_t *X, int64_t M,
                             const uint16_t *B, int r, const uint16_t *Hs_hi,
                             const uint16_t *Hs_lo, int rp, uint16_t *Y,
                             hipStream_t st);
// keep (M x k/4 keep nibbles, or NULL): adapter-input dropout of the forward;
// the rank-r term of dX is then kept per element and scaled by inv_keep.
qlora_status launch_gemm_dx(const uint8_t *codes, ql::ScaleSrc sc, int64_t d,
                            int64_t k, const uint16_t *dY, int64_t M,
                            const uint16_t *A, int r, const uint16_t *Gs_hi,
                            const uint16_t *Gs_lo, int rp, uint16_t *dX,
                            const uint8_t *keep, float inv_keep, hipStream_t st);

// gemv.hip : memory-bound forward for M <= 16, including the LoRA down
// projection, for nw (1..4) weights that read the same X (sibling
// projections) in one launch plus one epilogue launch. Per weight: codes and
// scales, d, Ap (rp x k) and Bp (d x rp) zero-padded to rp ranks, H_save
// (M x r, may be NULL) and Y (M x d). All weights share k and the
// double-quantisation mode.
struct GemvIn {
  const uint8_t *codes;
  ql::ScaleSrc sc;
  int64_t d;
  const uint16_t *Ap, *Bp;
  float *H_save;
  uint16_t *Y;
  DropParams dp;   // adapter-input dropout (dp.on == 0: none)
};
qlora_status launch_gemv_fwd(int nw, const GemvIn *in, int64_t k, const uint16_t *X, int64_t M,
                             int r, int rp, float s, float *part, hipStream_t st);
size_t gemv_part_bytes(int64_t dtot, int64_t k, int64_t M, int rp, int nw);

// merge.hip
qlora_status launch_merge(const uint8_t *codes, ql::ScaleSrc sc, int64_t d,
                          int64_t k, const uint16_t *A, const uint16_t *B,
                          int r, float s, uint16_t *Wm, hipStream_t st);

// adamw.hip : one AdamW step over n elements (scalars prepared on the host)
struct AdamScalars {
  float b1, b2, c1, c2, bc1, bc2, lr, eps, wd;
};
qlora_status launch_adamw(float *p, float *m, float *v, const uint16_t *g, uint16_t *out,
                          int64_t n, const AdamScalars &s, hipStream_t st);

// compute units of the current device (capi.hip; queried on every call, 256
// if the query fails)
int ql_num_cus();

// tables (quantize.hip)
void host_codebook(float levels[16], float thresholds[15]);

// Kernel timing. The product library compiles QlProf to nothing; the timing
// build (QLORA_KERNEL_TIMING, libqlora_nf4_timing.so) brackets each launch
// with HIP events (timing/hooks.hip, API in include/qlora_nf4_timing.h).
#include "../../include/qlora_nf4_timing.h"
#ifdef QLORA_KERNEL_TIMING
int ql_prof_begin(int kernel_id, hipStream_t st);
void ql_prof_end(int slot, hipStream_t st);
struct QlProf {
  int slot;
  hipStream_t st;
  QlProf(int kid, hipStream_t s) : slot(ql_prof_begin(kid, s)), st(s) {}
  ~QlProf() { ql_prof_end(slot, st); }
};
#else
struct QlProf {
  QlProf(int, hipStream_t) {}
};
#endif
