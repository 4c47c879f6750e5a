// C ABI of libqlora_nf4: argument checks, workspace layout and dispatch to
// the gfx950 kernels. Every check runs on the host before anything is
// enqueued; no HIP call is made for an invalid argument.
#include <math.h>
#include <string.h>

#include <algorithm>

#include "kernels.h"

namespace {

constexpr int64_t kAlign = 256;

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Shape checks shared by all entry points.
qlora_status check_weight_shape(int64_t d, int64_t k) {
  if (d < 1 || k < 1) return QLORA_ERR_INVALID_ARG;
  if (k % 64 != 0 || d % 8 != 0) return QLORA_ERR_UNSUPPORTED;
  if (d > (int64_t(1) << 31) || k > (int64_t(1) << 31)) return QLORA_ERR_UNSUPPORTED;
  const int64_t n = d * k;
  if (n / 64 >= (int64_t(1) << 32)) return QLORA_ERR_UNSUPPORTED;
  return QLORA_OK;
}

qlora_status check_weight(const qlora_nf4_weight *w, bool need_outputs_only) {
  (void)need_outputs_only;
  if (!w) return QLORA_ERR_INVALID_ARG;
  qlora_status s = check_weight_shape(w->d, w->k);
  if (s != QLORA_OK) return s;
  if (w->blocksize != 64) return QLORA_ERR_UNSUPPORTED;
  if (w->double_quant != 0 && w->double_quant != 1) return QLORA_ERR_INVALID_ARG;
  if (w->double_quant && w->dq_blocksize != 256) return QLORA_ERR_UNSUPPORTED;
  if (!w->codes || !aligned16(w->codes)) return QLORA_ERR_INVALID_ARG;
  if (w->double_quant) {
    if (!w->absmax_q || !w->absmax_scale || !w->absmax_offset) return QLORA_ERR_INVALID_ARG;
    if (!aligned16(w->absmax_q)) return QLORA_ERR_INVALID_ARG;  // read as dwords
    if (((uintptr_t)w->absmax_scale & 3u) || ((uintptr_t)w->absmax_offset & 3u))
      return QLORA_ERR_INVALID_ARG;
  } else {
    if (!w->absmax || ((uintptr_t)w->absmax & 3u)) return QLORA_ERR_INVALID_ARG;
  }
  return QLORA_OK;
}

ql::ScaleSrc scale_src(const qlora_nf4_weight *w) {
  return ql::ScaleSrc{w->absmax, w->absmax_q, w->absmax_scale, w->absmax_offset,
                      w->double_quant};
}

// Bump allocator over the caller's workspace (also used to size it).
struct Carve {
  char *base;
  int64_t off = 0;
  template <class T>
  T *take(int64_t bytes) {
    T *p = base ? (T *)(base + off) : nullptr;
    off += ql_rup(bytes > 0 ? bytes : 0, kAlign);
    return p;
  }
};

constexpr int kMaxGroup = 4;   // weights per qlora_linear_fwd_multi call

struct FwdWs {
  uint16_t *Ap[kMaxGroup], *Bp[kMaxGroup], *Hs_hi[kMaxGroup], *Hs_lo[kMaxGroup];
  float *H[kMaxGroup], *gpart;
  int64_t bytes;
};

// nw weights of d[i] rows each that read the same X (M x k)
FwdWs fwd_layout(char *base, const int64_t *d, int nw, int64_t k, int64_t M, int r) {
  const int rp = (int)ql_rup(r, 16);
  Carve c{base};
  FwdWs L{};
  int64_t dtot = 0;
  for (int i = 0; i < nw; ++i) dtot += d[i];
  if (M > 16) {
    for (int i = 0; i < nw; ++i) {
      L.H[i] = c.take<float>(M * rp * 4);
      L.Hs_hi[i] = c.take<uint16_t>(M * rp * 2);
      L.Hs_lo[i] = c.take<uint16_t>(M * rp * 2);
    }
    L.gpart = nullptr;
  } else {  // the GEMV computes H itself from zero-padded A and B
    for (int i = 0; i < nw; ++i) {
      L.Ap[i] = (r % 16) ? c.take<uint16_t>((int64_t)rp * k * 2) : nullptr;
      L.Bp[i] = (r % 16) ? c.take<uint16_t>(d[i] * rp * 2) : nullptr;
    }
    L.gpart = c.take<float>((int64_t)gemv_part_bytes(dtot, k, M, rp, nw));
  }
  L.bytes = c.off;
  return L;
}

// Bound for any split of dtot rows over up to kMaxGroup weights: the pieces
// that scale with d sum to the same bytes up to one alignment each.
int64_t fwd_multi_bytes(int64_t dtot, int64_t k, int64_t M, int r) {
  const int64_t d[kMaxGroup] = {dtot, 0, 0, 0};
  return fwd_layout(nullptr, d, kMaxGroup, k, M, r).bytes + kMaxGroup * kAlign;
}

struct BwdWs {
  uint16_t *Bt, *Gs_hi, *Gs_lo;
  float *H, *G, *cpart;
  uint8_t *keep;
  int64_t bytes;
};

// Kernel-side dropout parameters of weight `i` of a call (seed + i, so the
// sibling projections of one call draw independent masks).
DropParams drop_params(const qlora_lora_dropout *dr, int i) {
  DropParams dp{0u, 0u, 0u, 1.0f, 0};
  if (dr && dr->p > 0.0f) {
    const uint64_t seed = dr->seed + (uint64_t)i;
    dp.k0 = (uint32_t)seed;
    dp.k1 = (uint32_t)(seed >> 32);
    dp.thr = (uint32_t)floor((double)dr->p * 4294967296.0);
    dp.inv_keep = (float)(1.0 / (1.0 - (double)dr->p));
    dp.on = 1;
    dp.mask = i == 0 ? dr->mask : nullptr;
  }
  return dp;
}
bool drop_ok(const qlora_lora_dropout *dr) {
  return !dr || (isfinite(dr->p) && dr->p >= 0.0f && dr->p < 1.0f &&
                 ((uintptr_t)dr->mask & 15u) == 0);
}

BwdWs bwd_layout(char *base, int64_t d, int64_t k, int64_t M, int r, bool need_h, bool need_dx) {
  const int rp = (int)ql_rup(r, 16);
  Carve c{base};
  BwdWs L{};
  L.H = need_h ? c.take<float>(M * rp * 4) : nullptr;
  // B is read in place for G when r % 16 == 0; otherwise a zero-padded B^T
  L.Bt = (r % 16) ? c.take<uint16_t>((int64_t)rp * d * 2) : nullptr;
  L.G = c.take<float>(M * rp * 4);
  L.Gs_hi = need_dx ? c.take<uint16_t>(M * rp * 2) : nullptr;
  L.Gs_lo = need_dx ? c.take<uint16_t>(M * rp * 2) : nullptr;
  L.cpart = c.take<float>((int64_t)colacc_part_bytes(M, d, k, rp));
  L.keep = c.take<uint8_t>(M * (k >> 2));   // adapter-input dropout: keep nibbles of X
  L.bytes = c.off;
  return L;
}

bool ws_ok(const void *ws, size_t ws_bytes, int64_t need) {
  if (need == 0) return true;
  return ws && (((uintptr_t)ws & (kAlign - 1)) == 0) && (int64_t)ws_bytes >= need;
}

}  // namespace

extern "C" {

const char *qlora_status_string(int status) {
  switch (status) {
    case QLORA_OK: return "ok";
    case QLORA_ERR_INVALID_ARG: return "invalid argument";
    case QLORA_ERR_UNSUPPORTED: return "unsupported shape or format";
    case QLORA_ERR_WORKSPACE: return "workspace too small or misaligned";
    case QLORA_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

size_t qlora_nf4_storage_bytes(int64_t d, int64_t k, int32_t double_quant) {
  if (check_weight_shape(d, k) != QLORA_OK) return 0;
  const int64_t n = d * k, nb = n / 64;
  if (!double_quant) return (size_t)(n / 2 + 4 * nb);
  return (size_t)(n / 2 + nb + 4 * ql_cdiv(nb, 256) + 4);
}

size_t qlora_workspace_bytes(int32_t op, int64_t d, int64_t k, int64_t M, int32_t r,
                             int32_t double_quant) {
  if (check_weight_shape(d, k) != QLORA_OK) return (size_t)-1;
  if (op == QLORA_OP_QUANTIZE) return quantize_ws_bytes(d * k, double_quant);
  if (op == QLORA_OP_QUANTIZE_RESIDUAL || op == QLORA_OP_LOFTQ) {
    if (r < 1 || r > 64) return (size_t)-1;
    return op == QLORA_OP_LOFTQ ? loftq_ws_bytes(d, k, r, double_quant)
                                : residual_quantize_ws_bytes(d, k, double_quant);
  }
  if (M < 1 || r < 1 || r > 128) return (size_t)-1;
  if (op == QLORA_OP_FWD) return (size_t)fwd_layout(nullptr, &d, 1, k, M, r).bytes;
  if (op == QLORA_OP_FWD_MULTI) return (size_t)fwd_multi_bytes(d, k, M, r);
  // backward: sized for the largest case (H recomputed, dX requested)
  if (op == QLORA_OP_BWD) return (size_t)bwd_layout(nullptr, d, k, M, r, true, true).bytes;
  return (size_t)-1;
}

qlora_status qlora_nf4_codebook(float levels[16], float thresholds[15]) {
  if (!levels || !thresholds) return QLORA_ERR_INVALID_ARG;
  host_codebook(levels, thresholds);
  return QLORA_OK;
}

qlora_status qlora_nf4_quantize(const uint16_t *W0, const qlora_nf4_weight *w, void *ws,
                                size_t ws_bytes, void *stream) {
  qlora_status s = check_weight(w, true);
  if (s != QLORA_OK) return s;
  if (!W0 || !aligned16(W0)) return QLORA_ERR_INVALID_ARG;
  const int64_t n = w->d * w->k;
  const int64_t need = (int64_t)quantize_ws_bytes(n, w->double_quant);
  if (!ws_ok(ws, ws_bytes, need)) return QLORA_ERR_WORKSPACE;
  return launch_quantize(W0, n, w->codes, w->absmax, w->double_quant, w->absmax_q,
                         w->absmax_scale, w->absmax_offset, ws, (hipStream_t)stream);
}

static QuantOut quant_out(const qlora_nf4_weight *w) {
  return QuantOut{w->codes, w->absmax, w->absmax_q, w->absmax_scale, w->absmax_offset,
                  scale_src(w)};
}

// shared checks of the two LoftQ entry points
static qlora_status check_loftq_common(const uint16_t *W, const qlora_nf4_weight *out, int32_t r,
                                       float lora_alpha) {
  qlora_status s = check_weight(out, true);
  if (s != QLORA_OK) return s;
  if (!W || !aligned16(W)) return QLORA_ERR_INVALID_ARG;
  if (r < 1) return QLORA_ERR_INVALID_ARG;
  if (r > 64) return QLORA_ERR_UNSUPPORTED;
  if (!isfinite(lora_alpha)) return QLORA_ERR_INVALID_ARG;
  return QLORA_OK;
}

qlora_status qlora_nf4_quantize_residual(const uint16_t *W, const uint16_t *A, const uint16_t *B,
                                         int32_t r, float lora_alpha, const qlora_nf4_weight *out,
                                         void *ws, size_t ws_bytes, void *stream) {
  qlora_status s = check_loftq_common(W, out, r, lora_alpha);
  if (s != QLORA_OK) return s;
  if (!A || !B || !aligned16(A) || !aligned16(B)) return QLORA_ERR_INVALID_ARG;
  const int64_t need = (int64_t)residual_quantize_ws_bytes(out->d, out->k, out->double_quant);
  if (!ws_ok(ws, ws_bytes, need)) return QLORA_ERR_WORKSPACE;
  const float sc = lora_alpha / (float)r;
  return launch_residual_quantize_ws(W, A, B, out->d, out->k, r, sc, quant_out(out), ws,
                                     (hipStream_t)stream);
}

qlora_status qlora_loftq_init(const uint16_t *W, const float *omega, int32_t r, float lora_alpha,
                              int32_t iters, int32_t power_iters, const qlora_nf4_weight *out,
                              uint16_t *A, uint16_t *B, float *sigma, void *ws, size_t ws_bytes,
                              void *stream) {
  qlora_status s = check_loftq_common(W, out, r, lora_alpha);
  if (s != QLORA_OK) return s;
  if (!omega || ((uintptr_t)omega & 3u)) return QLORA_ERR_INVALID_ARG;
  if (!A || !B || !aligned16(A) || !aligned16(B)) return QLORA_ERR_INVALID_ARG;
  if (sigma && ((uintptr_t)sigma & 3u)) return QLORA_ERR_INVALID_ARG;
  if (iters < 1 || iters > 64 || power_iters < 0 || power_iters > 64)
    return QLORA_ERR_INVALID_ARG;
  if (lora_alpha == 0.0f) return QLORA_ERR_INVALID_ARG;   // B = U sqrt(S) / s
  const int64_t need = (int64_t)loftq_ws_bytes(out->d, out->k, r, out->double_quant);
  if (!ws_ok(ws, ws_bytes, need)) return QLORA_ERR_WORKSPACE;
  const float sc = lora_alpha / (float)r;
  return launch_loftq(W, omega, out->d, out->k, r, sc, iters, power_iters, quant_out(out), A, B,
                      sigma, ws, (hipStream_t)stream);
}

qlora_status qlora_nf4_dequantize(const qlora_nf4_weight *w, uint16_t *W_out, void *stream) {
  qlora_status s = check_weight(w, false);
  if (s != QLORA_OK) return s;
  if (!W_out || !aligned16(W_out)) return QLORA_ERR_INVALID_ARG;
  return launch_dequantize(w->codes, scale_src(w), w->d * w->k, W_out, (hipStream_t)stream);
}

static qlora_status check_lora(const uint16_t *A, const uint16_t *B, int32_t r, float alpha) {
  if (!A || !B || !aligned16(A) || !aligned16(B)) return QLORA_ERR_INVALID_ARG;
  if (r < 1) return QLORA_ERR_INVALID_ARG;
  if (r > 128) return QLORA_ERR_UNSUPPORTED;
  if (!isfinite(alpha)) return QLORA_ERR_INVALID_ARG;
  return QLORA_OK;
}

// Forward of nw weights that read the same X (nw == 1: qlora_linear_fwd).
static qlora_status linear_fwd_group(const qlora_nf4_weight *const *w, int nw, const uint16_t *X,
                                     int64_t M, const uint16_t *const *A,
                                     const uint16_t *const *B, int32_t r, float lora_alpha,
                                     const qlora_lora_dropout *drop, uint16_t *const *Y,
                                     float *const *H_save, void *ws, size_t ws_bytes,
                                     void *stream, int64_t ws_need) {
  if (nw < 1 || nw > kMaxGroup || !w || !A || !B || !Y) return QLORA_ERR_INVALID_ARG;
  if (!drop_ok(drop)) return QLORA_ERR_INVALID_ARG;
  qlora_status s;
  int64_t d[kMaxGroup];
  for (int i = 0; i < nw; ++i) {
    if ((s = check_weight(w[i], false)) != QLORA_OK) return s;
    if ((s = check_lora(A[i], B[i], r, lora_alpha)) != QLORA_OK) return s;
    if (!Y[i] || !aligned16(Y[i])) return QLORA_ERR_INVALID_ARG;
    if (H_save && H_save[i] && ((uintptr_t)H_save[i] & 3u)) return QLORA_ERR_INVALID_ARG;
    if (w[i]->k != w[0]->k || w[i]->double_quant != w[0]->double_quant)
      return QLORA_ERR_INVALID_ARG;
    d[i] = w[i]->d;
  }
  if (!X || !aligned16(X) || M < 1) return QLORA_ERR_INVALID_ARG;
  const int64_t k = w[0]->k;
  const FwdWs L = fwd_layout((char *)ws, d, nw, k, M, r);
  if (ws_need < L.bytes) ws_need = L.bytes;
  if (!ws_ok(ws, ws_bytes, ws_need)) return QLORA_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  const int rp = (int)ql_rup(r, 16);
  const float sc = lora_alpha / (float)r;

  if (M <= 16) {  // H = X A^T inside the GEMV; H_save gets the M x r copy
    GemvIn in[kMaxGroup];
    for (int i = 0; i < nw; ++i) {
      const uint16_t *Ap = A[i], *Bp = B[i];
      if (r % 16) {
        const LayoutReq req[2] = {{A[i], r, k, L.Ap[i], rp, k, 0}, {B[i], d[i], r, L.Bp[i], d[i], rp, 0}};
        if ((s = launch_layout(req, 2, st)) != QLORA_OK) return s;
        Ap = L.Ap[i];
        Bp = L.Bp[i];
      }
      in[i] = GemvIn{w[i]->codes, scale_src(w[i]), d[i], Ap, Bp, H_save ? H_save[i] : nullptr, Y[i],
                     drop_params(drop, i)};
    }
    return launch_gemv_fwd(nw, in, k, X, M, r, rp, sc, L.gpart, st);
  }
  // H_i = X A_i^T (float32, M x rp) and s*H_i as bf16 hi/lo for every weight
  // in one launch; H_save gets the M x r copies
  SkinnyOut so[kMaxGroup];
  for (int i = 0; i < nw; ++i) {
    so[i] = SkinnyOut{A[i], L.H[i], H_save ? H_save[i] : nullptr, L.Hs_hi[i], L.Hs_lo[i],
                      drop_params(drop, i)};
    so[i].dp.mask_write = 1;   // the drawn bits go to the caller's mask, if any
  }
  if ((s = launch_skinny(X, M, k, nw, so, false, r, rp, r, sc, st)) != QLORA_OK) return s;
  // one fused dequant-GEMM launch per weight: a 4096-row weight at this size
  // already fills the chip, and X is shared through L2 either way (one
  // grouped launch over all weights' column tiles measured no faster)
  for (int i = 0; i < nw; ++i)
    if ((s = launch_gemm_fwd(w[i]->codes, scale_src(w[i]), d[i], k, X, M, B[i], r, L.Hs_hi[i],
                             L.Hs_lo[i], rp, Y[i], st)) != QLORA_OK)
      return s;
  return QLORA_OK;
}

qlora_status qlora_linear_fwd(const qlora_nf4_weight *w, const uint16_t *X, int64_t M,
                              const uint16_t *A, const uint16_t *B, int32_t r, float lora_alpha,
                              uint16_t *Y, float *H_save, void *ws, size_t ws_bytes,
                              void *stream) {
  if (!w) return QLORA_ERR_INVALID_ARG;
  const qlora_nf4_weight *const wl[1] = {w};
  const uint16_t *const Al[1] = {A}, *const Bl[1] = {B};
  uint16_t *const Yl[1] = {Y};
  float *const Hl[1] = {H_save};
  return linear_fwd_group(wl, 1, X, M, Al, Bl, r, lora_alpha, nullptr, Yl, Hl, ws, ws_bytes,
                          stream, 0);
}

qlora_status qlora_linear_fwd_ex(const qlora_nf4_weight *w, const uint16_t *X, int64_t M,
                                 const uint16_t *A, const uint16_t *B, int32_t r,
                                 float lora_alpha, const qlora_lora_dropout *dropout,
                                 uint16_t *Y, float *H_save, void *ws, size_t ws_bytes,
                                 void *stream) {
  if (!w) return QLORA_ERR_INVALID_ARG;
  const qlora_nf4_weight *const wl[1] = {w};
  const uint16_t *const Al[1] = {A}, *const Bl[1] = {B};
  uint16_t *const Yl[1] = {Y};
  float *const Hl[1] = {H_save};
  return linear_fwd_group(wl, 1, X, M, Al, Bl, r, lora_alpha, dropout, Yl, Hl, ws, ws_bytes,
                          stream, 0);
}

qlora_status qlora_linear_fwd_multi(const qlora_nf4_weight *const *w, int32_t nw,
                                    const uint16_t *X, int64_t M, const uint16_t *const *A,
                                    const uint16_t *const *B, int32_t r, float lora_alpha,
                                    uint16_t *const *Y, float *const *H_save, void *ws,
                                    size_t ws_bytes, void *stream) {
  if (nw < 1 || nw > kMaxGroup || !w) return QLORA_ERR_INVALID_ARG;
  int64_t dtot = 0;
  for (int i = 0; i < nw; ++i) {
    if (!w[i]) return QLORA_ERR_INVALID_ARG;
    dtot += w[i]->d;
  }
  if (check_weight_shape(dtot, w[0]->k) != QLORA_OK) return QLORA_ERR_UNSUPPORTED;
  // the documented size (qlora_workspace_bytes(QLORA_OP_FWD_MULTI, sum of d, ...))
  const int64_t need = (r >= 1 && r <= 128 && M >= 1) ? fwd_multi_bytes(dtot, w[0]->k, M, r) : 0;
  return linear_fwd_group(w, nw, X, M, A, B, r, lora_alpha, nullptr, Y, H_save, ws, ws_bytes,
                          stream, need);
}

qlora_status qlora_linear_bwd(const qlora_nf4_weight *w, const uint16_t *X, int64_t M,
                              const uint16_t *A, const uint16_t *B, int32_t r, float lora_alpha,
                              const uint16_t *dY, const float *H, uint16_t *dX, uint16_t *dA,
                              uint16_t *dB, void *ws, size_t ws_bytes, void *stream) {
  return qlora_linear_bwd_ex(w, X, M, A, B, r, lora_alpha, nullptr, dY, H, dX, dA, dB, ws,
                             ws_bytes, stream);
}

qlora_status qlora_linear_bwd_ex(const qlora_nf4_weight *w, const uint16_t *X, int64_t M,
                                 const uint16_t *A, const uint16_t *B, int32_t r,
                                 float lora_alpha, const qlora_lora_dropout *dropout,
                                 const uint16_t *dY, const float *H, uint16_t *dX, uint16_t *dA,
                                 uint16_t *dB, void *ws, size_t ws_bytes, void *stream) {
  if (!drop_ok(dropout)) return QLORA_ERR_INVALID_ARG;
  const DropParams dp = drop_params(dropout, 0);
  qlora_status s = check_weight(w, false);
  if (s != QLORA_OK) return s;
  if ((s = check_lora(A, B, r, lora_alpha)) != QLORA_OK) return s;
  if (!X || !dY || !dA || !dB || M < 1) return QLORA_ERR_INVALID_ARG;
  if (!aligned16(X) || !aligned16(dY) || !aligned16(dA) || !aligned16(dB))
    return QLORA_ERR_INVALID_ARG;
  if (dX && !aligned16(dX)) return QLORA_ERR_INVALID_ARG;
  if (H && ((uintptr_t)H & 3u)) return QLORA_ERR_INVALID_ARG;
  const int64_t d = w->d, k = w->k;
  const bool need_h = (H == nullptr) || (r % 16 != 0);
  const bool need_dx = dX != nullptr;
  const BwdWs need = bwd_layout(nullptr, d, k, M, r, need_h, need_dx);
  if (!ws_ok(ws, ws_bytes, need.bytes)) return QLORA_ERR_WORKSPACE;
  const BwdWs L = bwd_layout((char *)ws, d, k, M, r, need_h, need_dx);
  hipStream_t st = (hipStream_t)stream;
  const int rp = (int)ql_rup(r, 16);
  const float sc = lora_alpha / (float)r;

  const float *Hq = H;  // M x rp
  if (need_h) {
    const SkinnyOut so{A, L.H, nullptr, nullptr, nullptr, dp};
    if ((s = launch_skinny(X, M, k, 1, &so, false, r, rp, 0, sc, st)) != QLORA_OK) return s;
    Hq = L.H;
  }
  // G = dY B (float32, M x rp) and s*G as bf16 hi/lo for the dX epilogue; B
  // is read in place unless r % 16 != 0 (then from a zero-padded B^T)
  // the G launch also clears the counters the dA/dB launch below uses
  int *cnt = colacc_counters(L.cpart, M, d, k, rp);
  const int64_t ncnt = colacc_counter_count(d, k);
  if (r % 16) {
    const LayoutReq req[1] = {{B, d, r, L.Bt, rp, d, 1}};
    if ((s = launch_layout(req, 1, st)) != QLORA_OK) return s;
    s = launch_skinny(dY, M, d, L.Bt, false, rp, rp, L.G, nullptr, 0, sc, L.Gs_hi, L.Gs_lo, st,
                      cnt, ncnt);
  } else {
    s = launch_skinny(dY, M, d, B, true, r, rp, L.G, nullptr, 0, sc, L.Gs_hi, L.Gs_lo, st, cnt,
                      ncnt);
  }
  if (s != QLORA_OK) return s;
  // dB = s dY^T H (d x r) and dA = s G^T X (r x k), one launch
  const DropParams none{0u, 0u, 0u, 1.0f, 0};
  // with a mask stored by the forward (M > 16) colacc reads the bits from it
  // and the dX epilogue uses it directly; otherwise colacc draws them and
  // keeps a copy in the workspace for the dX epilogue
  DropParams dpa = dp;
  dpa.mask_write = 0;
  if (M <= 16) dpa.mask = nullptr;
  uint8_t *keep = dp.on ? (dpa.mask ? dpa.mask : L.keep) : nullptr;
  if ((s = launch_colacc2(ColaccReq{dY, d, Hq, dB, 0, none, nullptr},
                          ColaccReq{X, k, L.G, dA, 1, dpa,
                                    (dp.on && need_dx && !dpa.mask) ? L.keep : nullptr},
                          M, rp, r, sc,
                          L.cpart, st)) != QLORA_OK)
    return s;
  if (need_dx) {
    if ((s = launch_gemm_dx(w->codes, scale_src(w), d, k, dY, M, A, r, L.Gs_hi, L.Gs_lo, rp, dX,
                            keep, dp.inv_keep, st)) != QLORA_OK)
      return s;
  }
  return QLORA_OK;
}

qlora_status qlora_merge(const qlora_nf4_weight *w, const uint16_t *A, const uint16_t *B,
                         int32_t r, float lora_alpha, uint16_t *W_merged, void *stream) {
  qlora_status s = check_weight(w, false);
  if (s != QLORA_OK) return s;
  if ((s = check_lora(A, B, r, lora_alpha)) != QLORA_OK) return s;
  if (!W_merged || !aligned16(W_merged)) return QLORA_ERR_INVALID_ARG;
  const float sc = lora_alpha / (float)r;
  return launch_merge(w->codes, scale_src(w), w->d, w->k, A, B, r, sc, W_merged,
                      (hipStream_t)stream);
}

// Device address of a buffer the AdamW step may touch: device memory as is,
// page-locked host memory through its device mapping. Anything else
// (pageable host memory, unknown pointers) is refused, so the kernel never
// dereferences an address the device cannot reach.
static bool device_view(const void *p, void **dp) {
  hipPointerAttribute_t a;
  if (hipPointerGetAttributes(&a, p) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  if (a.type == hipMemoryTypeDevice) {
    *dp = const_cast<void *>(p);
    return true;
  }
  if (a.type == hipMemoryTypeHost && a.devicePointer) {
    // the offset of p inside its allocation carries over to the mapping
    *dp = (char *)a.devicePointer + ((const char *)p - (const char *)a.hostPointer);
    return true;
  }
  return false;
}

qlora_status qlora_adamw_step(float *param, float *exp_avg, float *exp_avg_sq,
                              const uint16_t *grad, uint16_t *param_bf16, int64_t n,
                              const qlora_adamw_hparams *hp, int64_t step, void *stream) {
  if (!param || !exp_avg || !exp_avg_sq || !grad || !param_bf16 || !hp || n < 1 || step < 1)
    return QLORA_ERR_INVALID_ARG;
  if (!aligned16(param) || !aligned16(exp_avg) || !aligned16(exp_avg_sq) ||
      ((uintptr_t)grad & 7u) || ((uintptr_t)param_bf16 & 7u))
    return QLORA_ERR_INVALID_ARG;
  const double b1 = hp->beta1, b2 = hp->beta2;
  if (!(b1 >= 0.0 && b1 < 1.0) || !(b2 >= 0.0 && b2 < 1.0)) return QLORA_ERR_INVALID_ARG;
  if (!(isfinite(hp->lr) && hp->lr >= 0.0) || !(isfinite(hp->eps) && hp->eps >= 0.0) ||
      !(isfinite(hp->weight_decay) && hp->weight_decay >= 0.0))
    return QLORA_ERR_INVALID_ARG;
  void *dv[5];
  const void *hv[5] = {param, exp_avg, exp_avg_sq, grad, param_bf16};
  for (int i = 0; i < 5; ++i)
    if (!device_view(hv[i], &dv[i])) return QLORA_ERR_INVALID_ARG;
  AdamScalars s;
  s.b1 = (float)b1;
  s.b2 = (float)b2;
  s.c1 = (float)(1.0 - b1);
  s.c2 = (float)(1.0 - b2);
  s.bc1 = (float)(1.0 - pow(b1, (double)step));
  s.bc2 = (float)(1.0 - pow(b2, (double)step));
  s.lr = (float)hp->lr;
  s.eps = (float)hp->eps;
  s.wd = (float)hp->weight_decay;
  return launch_adamw((float *)dv[0], (float *)dv[1], (float *)dv[2], (const uint16_t *)dv[3],
                      (uint16_t *)dv[4], n, s, (hipStream_t)stream);
}

// Memory kind of p: device memory, page-locked host memory, or neither.
enum class MemKind { Other, Device, PinnedHost };
static MemKind mem_kind(const void *p) {
  hipPointerAttribute_t a;
  if (hipPointerGetAttributes(&a, p) != hipSuccess) {
    (void)hipGetLastError();
    return MemKind::Other;
  }
  if (a.type == hipMemoryTypeDevice) return MemKind::Device;
  if (a.type == hipMemoryTypeHost) return MemKind::PinnedHost;
  return MemKind::Other;
}

// nbuf copies of n float32 between device memory and page-locked host
// memory, enqueued on the stream after every pointer has been checked.
static qlora_status adamw_page(float *const *dst, const float *const *src, int32_t nbuf,
                               int64_t n, bool to_host, void *stream) {
  if (!dst || !src || nbuf < 1 || nbuf > 3 || n < 1 || n > (INT64_MAX >> 2))
    return QLORA_ERR_INVALID_ARG;
  const MemKind want_dst = to_host ? MemKind::PinnedHost : MemKind::Device;
  const MemKind want_src = to_host ? MemKind::Device : MemKind::PinnedHost;
  for (int i = 0; i < nbuf; ++i) {
    if (!dst[i] || !src[i] || !aligned16(dst[i]) || !aligned16(src[i]))
      return QLORA_ERR_INVALID_ARG;
    if (mem_kind(dst[i]) != want_dst || mem_kind(src[i]) != want_src)
      return QLORA_ERR_INVALID_ARG;
  }
  const hipMemcpyKind kind = to_host ? hipMemcpyDeviceToHost : hipMemcpyHostToDevice;
  for (int i = 0; i < nbuf; ++i) {
    if (hipMemcpyAsync(dst[i], src[i], (size_t)n * sizeof(float), kind,
                       (hipStream_t)stream) != hipSuccess) {
      (void)hipGetLastError();
      return QLORA_ERR_HIP;
    }
  }
  return QLORA_OK;
}

qlora_status qlora_adamw_page_out(float *const *host, const float *const *dev, int32_t nbuf,
                                  int64_t n, void *stream) {
  return adamw_page(host, dev, nbuf, n, true, stream);
}

qlora_status qlora_adamw_page_in(float *const *dev, const float *const *host, int32_t nbuf,
                                 int64_t n, void *stream) {
  return adamw_page(dev, host, nbuf, n, false, stream);
}

}  // extern "C"

int ql_num_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      n < 1) {
    (void)hipGetLastError();   // not a launch failure: fall back to the MI355X count
    n = 256;
  }
  return n;
}
