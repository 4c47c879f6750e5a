/*
 * qlora_nf4.h -- C ABI of the MI355X (gfx950) QLoRA frozen-base NF4 linear.
 *
 * The layer (QLoRA glossary, Ultralytics, "QLoRA 的工作原理"; Day-25 LoRA/QLoRA
 * notes, sections 2.1 and 6.2): a frozen base weight W0 (d x k, row-major,
 * out_features x in_features) is stored as 4-bit NormalFloat codes in blocks
 * of 64 consecutive weights with one absmax per block; the absmax values may
 * be double-quantised to 8 bits with one float32 scale per 256 blocks. The
 * forward pass dequantises W0 to bfloat16 and computes, for M token rows X
 * (M x k),
 *
 *     Y = X W'^T + s (X A^T) B^T,       s = fl32(lora_alpha / r),
 *
 * with LoRA matrices A (r x k) and B (d x r). The backward pass produces dX
 * through the same dequantised W' and gradients for A and B only.
 *
 * Conventions shared by every entry point
 *   - bf16 tensors are passed as uint16_t bit patterns, row-major, dense.
 *   - Every tensor pointer is a device pointer owned by the caller, 16-byte
 *     aligned; the weight descriptor itself is host memory. The library never
 *     allocates, frees or keeps a pointer after a call returns.
 *   - `stream` is a hipStream_t (NULL = the legacy default stream). Calls only
 *     enqueue work on it and never synchronise; results are valid once the
 *     stream has reached them. Calls on different streams that write the
 *     same buffers race.
 *   - Arguments are checked on the host before anything is enqueued; on any
 *     error nothing is launched. A launch failure returns QLORA_ERR_HIP.
 *     Device faults surface at the caller's next synchronisation.
 *   - Outputs must not alias inputs. Results are deterministic: the same
 *     inputs give bit-identical outputs on every call.
 */
#ifndef QLORA_NF4_H
#define QLORA_NF4_H

#include <stddef.h>
#include <stdint.h>

/* Symbols of the C ABI; everything else in the library is hidden. */
#if defined(__GNUC__) || defined(__clang__)
#define QLORA_API __attribute__((visibility("default")))
#else
#define QLORA_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QLORA_OK = 0,
  QLORA_ERR_INVALID_ARG = -1, /* NULL/misaligned pointer, size < 1, non-finite alpha */
  QLORA_ERR_UNSUPPORTED = -2, /* blocksize != 64, dq_blocksize != 256, k % 64 != 0,
                                 d % 8 != 0, d*k/64 >= 2^32, r > 128 */
  QLORA_ERR_WORKSPACE = -3,   /* workspace smaller than qlora_workspace_bytes() */
  QLORA_ERR_HIP = -4          /* a kernel launch failed */
} qlora_status;

/*
 * Quantised weight (QLoRA glossary, "QLoRA 的工作原理", NF4 and
 * double-quantisation bullets; LLM tutorial ch. 3, "双重量化").
 *
 *   codes         [d*k/2] bytes; element 2j of the row-major weight is the
 *                 high nibble of byte j, element 2j+1 the low nibble. A code
 *                 indexes the 16 ascending NF4 levels (code 7 is exactly 0).
 *   absmax        [d*k/64] float32, one per block       (double_quant == 0)
 *   absmax_q      [d*k/64] int8 codes of (absmax - mu)  (double_quant == 1)
 *   absmax_scale  [ceil(d*k/64/256)] float32 scales s2  (double_quant == 1)
 *   absmax_offset [1] float32 mean mu                   (double_quant == 1)
 * The dequantised block scale is a' = fl(fl(q * s2) + mu) (or absmax) and a
 * weight dequantises to w' = bf16_rne(fl(level[code] * a')).
 * Pointers unused by the chosen mode may be NULL.
 */
typedef struct qlora_nf4_weight {
  int64_t d;             /* rows (out_features), multiple of 8 */
  int64_t k;             /* columns (in_features), multiple of 64 */
  int32_t blocksize;     /* must be 64 */
  int32_t double_quant;  /* 0 or 1 */
  int32_t dq_blocksize;  /* must be 256 when double_quant == 1 */
  int32_t reserved;      /* set to 0 */
  uint8_t *codes;
  float *absmax;
  int8_t *absmax_q;
  float *absmax_scale;
  float *absmax_offset;
} qlora_nf4_weight;

/* Operation ids for qlora_workspace_bytes. For QLORA_OP_FWD_MULTI pass the
 * sum of the weights' d as `d`; QLORA_OP_QUANTIZE_RESIDUAL and QLORA_OP_LOFTQ
 * take r and ignore M. */
enum { QLORA_OP_QUANTIZE = 0, QLORA_OP_FWD = 1, QLORA_OP_BWD = 2, QLORA_OP_FWD_MULTI = 3,
       QLORA_OP_QUANTIZE_RESIDUAL = 4, QLORA_OP_LOFTQ = 5 };

/*
 * Quantise a bf16 weight W0 (d x k) into `w` (all of w's pointers are
 * outputs; d, k, blocksize, double_quant, dq_blocksize are inputs).
 * Per block of 64: a = max|w|; each weight gets the code of the level nearest
 * to fl32(w / a) (float32 distance, lower code on equal distances); an
 * all-zero block gets code 7 and absmax 0 (QLoRA glossary, "QLoRA 的工作原理",
 * snippet). With double quantisation (same page, double-quantisation bullet;
 * Day-25 notes 3.3: constants are quantised after the weights):
 * mu = exact mean of all absmax values rounded once to float32; per group of
 * 256 blocks s2 = fl(max|fl(a - mu)| / 127) and
 * q = clamp(rne(fl(fl(a - mu) / s2)), -127, 127) (q = 0 when s2 == 0).
 * Workspace: qlora_workspace_bytes(QLORA_OP_QUANTIZE, d, k, 0, 0, dq) bytes
 * of device memory (0 without double quantisation; ws may then be NULL).
 * Non-finite weights are outside the method's domain; their codes are
 * unspecified.
 */
QLORA_API qlora_status qlora_nf4_quantize(const uint16_t *W0, const qlora_nf4_weight *w,
                                void *ws, size_t ws_bytes, void *stream);

/*
 * Dequantise `w` to bf16 W_out (d x k): w' = bf16(fl(level[code] * a'))
 * (QLoRA glossary, "QLoRA 的工作原理": weights are dequantised to bfloat16
 * before the matrix product; LLM tutorial ch. 3, 3.8: dequantise to bf16
 * before merging). Bit-exact.
 */
QLORA_API qlora_status qlora_nf4_dequantize(const qlora_nf4_weight *w, uint16_t *W_out,
                                  void *stream);

/*
 * Forward: Y (M x d, bf16) = bf16(X W'^T + s H B^T), H = X A^T (Day-25 notes
 * 2.1 and 6.2; QLoRA glossary forward paragraph). X is M x k, A is r x k,
 * B is d x r, all bf16; accumulation is float32. If H_save is non-NULL the
 * float32 H (M x r) is written there for the backward pass. M <= 16 uses the
 * memory-bound GEMV kernel, larger M the fused dequant-GEMM.
 * Workspace: qlora_workspace_bytes(QLORA_OP_FWD, d, k, M, r, dq) bytes.
 */
QLORA_API qlora_status qlora_linear_fwd(const qlora_nf4_weight *w, const uint16_t *X,
                              int64_t M, const uint16_t *A, const uint16_t *B,
                              int32_t r, float lora_alpha, uint16_t *Y,
                              float *H_save, void *ws, size_t ws_bytes,
                              void *stream);

/*
 * LoRA dropout on the adapter input (LLM tutorial ch. 3, 3.3 and Day-25
 * notes 4.3: LoraConfig(lora_dropout=0.05); notes 7.x: 0.1 against
 * overfitting). The pages give only the rate; reading taken: inverted
 * dropout of X before A on the LoRA branch only, so with keep mask K
 *   H  = ((X * K) A^T) / (1 - p),       Y  = X W'^T + s H B^T,
 *   dA = s G^T (X * K) / (1 - p),       dB = s dY^T H,
 *   dX = dY W' + s (G A) * K / (1 - p).
 * K[m][c] is drawn from Philox4x32-10 (Salmon et al., SC'11): element
 * e = m*k + c keeps when word e%4 of philox(counter (e/4 low, e/4 high, 0,
 * 0), key (seed low, seed high)) >= floor(p * 2^32). The forward and the
 * backward of one step must get the same p and seed. p == 0 (or a NULL
 * pointer) is no dropout. 0 <= p < 1, else QLORA_ERR_INVALID_ARG.
 */
typedef struct qlora_lora_dropout {
  float p;
  uint32_t reserved;   /* set to 0 */
  uint64_t seed;
  /* Optional (NULL: none), M > 16 only: M*k/4 bytes of device memory,
   * 16-byte aligned, owned by the caller. The forward stores the keep bits it
   * draws there (byte (m*k + c)/4, bit c%4) and the backward of the same step
   * reads them instead of drawing them again; pass the same pointer to both
   * and keep its contents between them. Ignored for M <= 16 (the backward
   * then draws the bits itself). A pointer not 16-byte aligned:
   * QLORA_ERR_INVALID_ARG. */
  uint8_t *mask;
} qlora_lora_dropout;

/* qlora_linear_fwd with adapter-input dropout (workspace as for QLORA_OP_FWD). */
QLORA_API qlora_status qlora_linear_fwd_ex(const qlora_nf4_weight *w, const uint16_t *X,
                                 int64_t M, const uint16_t *A, const uint16_t *B,
                                 int32_t r, float lora_alpha,
                                 const qlora_lora_dropout *dropout, uint16_t *Y,
                                 float *H_save, void *ws, size_t ws_bytes,
                                 void *stream);

/*
 * Sibling projections: the forward above for nw (1..4) weights that read the
 * same activations X -- q, k, v of an attention block, or gate and up of the
 * MLP (LLM tutorial ch. 3, 3.3 and Day-25 notes 4.3: the adapters target
 * every such linear; QLoRA glossary, "QLoRA 的工作原理": adapters on every
 * linear layer of the block). Weight i has its own d_i, A[i] (r x k),
 * B[i] (d_i x r) and output Y[i] (M x d_i); H_save may be NULL or hold a
 * NULL / an M x r float32 buffer per weight. All weights share k, r,
 * lora_alpha and the double-quantisation mode. For M <= 16 the weights run
 * as one GEMV launch (row groups of all weights in one grid; X and the LoRA
 * down projections read once) plus one epilogue launch; for larger M as one
 * launch computing every H_i = X A_i^T (X read once) plus one fused
 * dequant-GEMM launch per weight. Results are bit-identical to nw
 * separate qlora_linear_fwd calls.
 * Workspace: qlora_workspace_bytes(QLORA_OP_FWD_MULTI, sum of d_i, k, M, r, dq).
 */
QLORA_API qlora_status qlora_linear_fwd_multi(const qlora_nf4_weight *const *w, int32_t nw,
                                    const uint16_t *X, int64_t M,
                                    const uint16_t *const *A, const uint16_t *const *B,
                                    int32_t r, float lora_alpha, uint16_t *const *Y,
                                    float *const *H_save, void *ws, size_t ws_bytes,
                                    void *stream);

/*
 * qlora_linear_fwd for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same computation, arguments and results as qlora_linear_fwd (bit-identical
 * outputs), but without a workspace argument: the scratch comes from a
 * device array of QLORA_NOALLOC_SCRATCH_BYTES (16 MiB) inside the library,
 * one per device, allocated when the library is loaded and held until the
 * process ends. The call allocates nothing (no hipMalloc, no library
 * allocation). It uses the array of the current device (hipGetDevice); the
 * stream must belong to that device. Every call on a device shares its
 * array, so calls on one device that overlap in time (different streams,
 * threads, or graphs replayed concurrently) race and give undefined results;
 * calls ordered on one stream do not. Each call writes every scratch word it
 * reads; nothing carries over between calls.
 * Returns QLORA_ERR_WORKSPACE, before any launch, when the forward's
 * workspace for this shape (qlora_workspace_bytes(QLORA_OP_FWD, ...)) exceeds
 * 16 MiB -- every decode shape (M <= 16) up to 22016 x 8192 at r = 128 and
 * the GEMM path up to M * ceil(r/16)*16 <= 2^21 fit; QLORA_ERR_HIP if the
 * device or the array's address cannot be queried.
 */
#define QLORA_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
QLORA_API qlora_status qlora_linear_fwd_noalloc(const qlora_nf4_weight *w, const uint16_t *X,
                                                int64_t M, const uint16_t *A, const uint16_t *B,
                                                int32_t r, float lora_alpha, uint16_t *Y,
                                                float *H_save, void *stream);

/*
 * Backward of the forward above for upstream gradient dY (M x d, bf16)
 * (chain rule; QLoRA glossary forward paragraph: gradients pass through the
 * dequantised weight, only A and B are updated):
 *   G  = dY B                    (float32, M x r, workspace)
 *   dX = bf16(dY W' + s G A)     (M x k; skipped when dX == NULL)
 *   dA = bf16(s G^T X)           (r x k)
 *   dB = bf16(s dY^T H)          (d x r)
 * H is the float32 X A^T saved by the forward, or NULL to recompute it.
 * Workspace: qlora_workspace_bytes(QLORA_OP_BWD, d, k, M, r, dq) bytes.
 */
QLORA_API qlora_status qlora_linear_bwd(const qlora_nf4_weight *w, const uint16_t *X,
                              int64_t M, const uint16_t *A, const uint16_t *B,
                              int32_t r, float lora_alpha, const uint16_t *dY,
                              const float *H, uint16_t *dX, uint16_t *dA,
                              uint16_t *dB, void *ws, size_t ws_bytes,
                              void *stream);

/* qlora_linear_bwd for a forward run with adapter-input dropout (same p and
 * seed); H, if passed, is the H_save of that forward. Workspace as for
 * QLORA_OP_BWD. */
QLORA_API qlora_status qlora_linear_bwd_ex(const qlora_nf4_weight *w, const uint16_t *X,
                                 int64_t M, const uint16_t *A, const uint16_t *B,
                                 int32_t r, float lora_alpha,
                                 const qlora_lora_dropout *dropout, const uint16_t *dY,
                                 const float *H, uint16_t *dX, uint16_t *dA,
                                 uint16_t *dB, void *ws, size_t ws_bytes,
                                 void *stream);

/*
 * Merge: W_merged (d x k, bf16) = bf16(float(w') + s (B A)) with B A summed
 * in float32 (Day-25 notes 2.6 and 6.2; LLM tutorial ch. 3, 3.8: a 4-bit base
 * is dequantised to bf16 and then merged).
 */
QLORA_API qlora_status qlora_merge(const qlora_nf4_weight *w, const uint16_t *A,
                         const uint16_t *B, int32_t r, float lora_alpha,
                         uint16_t *W_merged, void *stream);

/*
 * One 32-bit AdamW step over the n elements of a LoRA matrix (A or B): the
 * update of the paged optimiser (Day-25 notes 3.4: Adam's two moments kept in
 * float32 and paged out to CPU RAM when device memory runs short; QLoRA
 * glossary, "QLoRA 的工作原理", paged-optimiser bullet;
 * "如何利用QLoRA在消费级GPU上实现大模型的高效微调", sections 3 and 4:
 * paged_adamw_32bit). The pages print no update rule; this is AdamW as
 * published (bias-corrected moments, decoupled weight decay).
 *   param      [n] float32 master copy of A or B              (in/out)
 *   exp_avg    [n] float32 first moment m                      (in/out)
 *   exp_avg_sq [n] float32 second moment v                     (in/out)
 *   grad       [n] bf16 gradient (dA or dB of qlora_linear_bwd) (in)
 *   param_bf16 [n] bf16 copy of the updated param: the A or B the next
 *              forward and backward read                      (out)
 * `step` is the 1-based step count t. Per element, every float32 operation
 * rounded once (IEEE division and square root), in this order:
 *   m = b1*m + c1*g;  v = b2*v + c2*(g*g);
 *   u = (m / bc1) / (sqrt(v / bc2) + eps);
 *   param = param - lr * (u + weight_decay * param);  param_bf16 = bf16_rne(param)
 * with b1, b2, lr, eps, weight_decay the float32 roundings of the
 * hyperparameters and c1 = 1 - beta1, c2 = 1 - beta2, bc1 = 1 - beta1^t,
 * bc2 = 1 - beta2^t evaluated in double and rounded once to float32.
 * Paging: param, exp_avg and exp_avg_sq may be device memory or page-locked
 * host memory mapped into the device address space (hipHostMalloc); the
 * caller moves the state out to host memory when device memory is short and
 * back when it is not, and the step updates it in place either way (over the
 * host link when it is paged out). param, exp_avg, exp_avg_sq: 16-byte
 * aligned; grad, param_bf16: 8-byte aligned; n >= 1; step >= 1;
 * 0 <= beta1, beta2 < 1; lr, eps, weight_decay finite and >= 0; otherwise
 * QLORA_ERR_INVALID_ARG and nothing is launched.
 */
typedef struct qlora_adamw_hparams {
  double lr, beta1, beta2, eps, weight_decay;
} qlora_adamw_hparams;
QLORA_API qlora_status qlora_adamw_step(float *param, float *exp_avg, float *exp_avg_sq,
                              const uint16_t *grad, uint16_t *param_bf16, int64_t n,
                              const qlora_adamw_hparams *hp, int64_t step, void *stream);

/*
 * Paging of the AdamW state (Day-25 notes 3.4: the optimiser state moves to
 * CPU RAM when device memory runs short and back when it is needed; QLoRA
 * glossary, "QLoRA 的工作原理", paged-optimiser bullet).
 *
 * qlora_adamw_page_out: for i = 0..nbuf-1, copy n float32 elements from the
 * device buffer dev[i] to the page-locked host buffer host[i].
 * qlora_adamw_page_in: the same copies from host[i] back to dev[i].
 * The buffers are typically param, exp_avg and exp_avg_sq of one LoRA
 * matrix (1 <= nbuf <= 3). The copies are enqueued on `stream` without
 * synchronising; a qlora_adamw_step enqueued later on the same stream sees
 * the moved state, and after page_out the caller may reuse or free dev[i]
 * once the stream has passed the copy. Between page_out and page_in the
 * step can also run on the host buffers directly (qlora_adamw_step accepts
 * page-locked state). Values are copied bit for bit.
 * dev[i]: device memory; host[i]: page-locked host memory (hipHostMalloc,
 * torch pin_memory); every pointer 16-byte aligned and holding n floats;
 * n >= 1. A pointer of the wrong kind (pageable host memory, a device
 * pointer where a host one is expected), a NULL or a misaligned pointer
 * returns QLORA_ERR_INVALID_ARG with nothing enqueued; a failed copy
 * enqueue returns QLORA_ERR_HIP (copies of earlier buffers may already be
 * enqueued).
 */
QLORA_API qlora_status qlora_adamw_page_out(float *const *host, const float *const *dev,
                                            int32_t nbuf, int64_t n, void *stream);
QLORA_API qlora_status qlora_adamw_page_in(float *const *dev, const float *const *host,
                                           int32_t nbuf, int64_t n, void *stream);

/*
 * LoftQ initialisation (LLM-train tutorial ch. 3, jwzheng96.github.io,
 * section 3.10: factor the gap between the 16-bit weight and its 4-bit base
 * into the LoRA branch, alternating an SVD with the quantisation).
 *
 * qlora_nf4_quantize_residual: quantise bf16(W - s B A) into `out` exactly as
 * qlora_nf4_quantize would quantise that bf16 matrix (the base of one LoftQ
 * step). Per element, in float32: acc = 0; acc = fma(B[i][j], A[j][c], acc)
 * for j = 0..r-1 in order (each product is exact); t = fl(s * acc);
 * W~ = bf16_rne(fl(W - t)); s = fl32(lora_alpha / r).
 * W: d x k bf16, A: r x k bf16, B: d x r bf16 (row-major, 16-byte aligned),
 * 1 <= r <= 64. `out` as for qlora_nf4_quantize (its pointers are outputs).
 * Workspace: qlora_workspace_bytes(QLORA_OP_QUANTIZE_RESIDUAL, d, k, 0, r, dq).
 *
 * qlora_loftq_init: `iters` (>= 1) alternations, t = 1..iters:
 *   R = fl32(W - W'_{t-1}) with W'_0 = 0 (the first SVD is of W itself);
 *   a rank-r SVD R ~ U S V^T by randomized subspace iteration (Halko,
 *   Martinsson, Tropp 2011): Y = R Omega, Q = orth(Y), then `power_iters`
 *   times Z = orth(R^T Q), Q = orth(R Z); finally the SVD of Q^T R; every
 *   orth is CholeskyQR twice (float64 Gram), the products accumulate in
 *   float32, the small SVD is a float64 Jacobi eigen-decomposition;
 *   A = bf16(sqrt(S) V^T), B = bf16(U sqrt(S) / s), so s B A ~ U S V^T;
 *   out = NF4 of bf16(W - s B A) (as qlora_nf4_quantize_residual), W'_t its
 *   dequantised weight.
 * omega: k x r float32 test matrix (row-major; the caller draws it, e.g.
 * standard normal), read-only. A (r x k), B (d x r): bf16 outputs; sigma:
 * r float32 singular values of the last SVD (descending), may be NULL.
 * Directions with sigma below 1e-12 sigma_0 (a rank-deficient R) give zero
 * rows of A and zero columns of B. 1 <= r <= 64, 0 <= power_iters <= 64,
 * 1 <= iters <= 64. Workspace: qlora_workspace_bytes(QLORA_OP_LOFTQ, d, k,
 * 0, r, dq) bytes (about 6 d k bytes plus split partial products of a few
 * MB). All outputs are written
 * on `stream`; results are deterministic.
 */
QLORA_API qlora_status qlora_nf4_quantize_residual(const uint16_t *W, const uint16_t *A,
                                         const uint16_t *B, int32_t r, float lora_alpha,
                                         const qlora_nf4_weight *out, void *ws,
                                         size_t ws_bytes, void *stream);
QLORA_API qlora_status qlora_loftq_init(const uint16_t *W, const float *omega, int32_t r,
                              float lora_alpha, int32_t iters, int32_t power_iters,
                              const qlora_nf4_weight *out, uint16_t *A, uint16_t *B,
                              float *sigma, void *ws, size_t ws_bytes, void *stream);

/* Bytes of the quantised record for d x k: d*k/2 + 4*nb (no double quant)
 * or d*k/2 + nb + 4*ceil(nb/256) + 4 (double quant), nb = d*k/64.
 * Returns 0 for an unsupported shape. */
QLORA_API size_t qlora_nf4_storage_bytes(int64_t d, int64_t k, int32_t double_quant);

/* Device workspace in bytes for `op` (QLORA_OP_*); 0 means none needed.
 * Returns (size_t)-1 for an unsupported shape. */
QLORA_API size_t qlora_workspace_bytes(int32_t op, int64_t d, int64_t k, int64_t M,
                             int32_t r, int32_t double_quant);

/* Host copy of the constant tables compiled into the kernels: the 16 NF4
 * levels (ascending) and the 15 code thresholds T_i (code = #{i: x > T_i}).
 * Touches no device; for inspection and tests. Returns QLORA_OK. */
QLORA_API qlora_status qlora_nf4_codebook(float levels[16], float thresholds[15]);

/* Static text for a status code. */
QLORA_API const char *qlora_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* QLORA_NF4_H */
