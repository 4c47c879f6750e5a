"""LoftQ initialisation of the LoRA factors of a quantised base weight.

CPU oracle -- test infrastructure only (see ``oracle/__init__.py``).

Pages followed
--------------
* LLM-train tutorial ch. 3 (jwzheng96.github.io), section 3.10 (LoftQ): a
  plain 4-bit base with B = 0 starts from the quantised weight, already off
  the 16-bit one; LoftQ factors the gap between the two into the LoRA branch
  so that base + LoRA approximates the 16-bit weight. Its listed steps, in
  order: an SVD of the 16-bit weight; the top r singular triplets become the
  branch, A = sqrt(S_r) V_r^T and B = U_r sqrt(S_r); what remains is the base,
  quantised to 4 bits; repeat a number of times so the residual settles.

Readings taken (the pages leave these open)
-------------------------------------------
* Iteration t = 1..T: R_t = W - W'_{t-1} with W'_0 = 0 (so the first SVD is
  of W itself, the pages' step 1); (A_t, B_t) from the rank-r factorisation
  of R_t; the base Q_t = NF4(bf16(W - s B_t A_t)) and W'_t its dequantised
  weight. Output: Q_T, A_T, B_T. The layer computes W' + s B A, so B carries
  the 1/s that makes s B A equal the truncated SVD (s = alpha / r).
* The rank-r SVD is computed by randomized subspace iteration (Halko,
  Martinsson and Tropp, "Finding structure with randomness", SIAM Review
  2011, the range finder with q power iterations and an orthonormalisation
  after every product), with p = r columns and a Gaussian test matrix Omega
  (k x r) that the caller draws and passes in. The small SVD of Q^T R and
  every orthonormalisation are library routines here (numpy QR with a
  positive diagonal, numpy SVD).
* The LoRA factors are stored in bf16 (rounded from float32), as the layer
  reads them.
* bf16(W - s B A) is evaluated per element as: acc = 0; for j = 0..r-1
  acc = fl32(acc + b_ij a_jc) (each product of two bf16 values is exact in
  float32); t = fl32(s * acc); bf16_rne(fl32(w - t)).
"""

from __future__ import annotations

import numpy as np

from . import nf4 as onf4


def orth(Y: np.ndarray) -> np.ndarray:
    """Orthonormal basis of the columns of Y: the Q of Y = QR with diag(R) >= 0
    (unique for full column rank)."""
    Q, Rf = np.linalg.qr(np.asarray(Y, dtype=np.float64))
    sgn = np.where(np.diag(Rf) < 0, -1.0, 1.0)
    return Q * sgn


def lowrank_svd(R: np.ndarray, omega: np.ndarray, power_iters: int):
    """Rank-p SVD of R (n x m) from the test matrix omega (m x p), p = its
    column count: range finder with ``power_iters`` subspace iterations, then
    the SVD of the p x m matrix Q^T R. Returns (U n x p, sigma p, Vt p x m)
    with sigma in descending order."""
    R = np.asarray(R, dtype=np.float64)
    Q = orth(R @ np.asarray(omega, dtype=np.float64))
    for _ in range(power_iters):
        Z = orth(R.T @ Q)
        Q = orth(R @ Z)
    C = Q.T @ R
    Uc, sigma, Vt = np.linalg.svd(C, full_matrices=False)
    return Q @ Uc, sigma, Vt


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float64 -> float32 (nearest) -> bf16 (nearest even) bits."""
    return onf4.f32_to_bf16_bits(np.asarray(x, dtype=np.float64).astype(np.float32))


def lora_factors(U, sigma, Vt, s):
    """A = sqrt(S) V^T (r x k) and B = U sqrt(S) / s (d x r), as bf16 bits,
    so that s B A is the truncated SVD (tutorial ch. 3, section 3.10, step 2)."""
    rs = np.sqrt(np.maximum(np.asarray(sigma, dtype=np.float64), 0.0))
    A = rs[:, None] * np.asarray(Vt, dtype=np.float64)
    B = np.asarray(U, dtype=np.float64) * rs[None, :] / float(s)
    return to_bf16_bits(A), to_bf16_bits(B)


def residual_bf16(W_bits: np.ndarray, B_bits: np.ndarray, A_bits: np.ndarray, s) -> np.ndarray:
    """bf16 bits of W - s B A in the float32 order stated in the header
    (the base that step 3 of section 3.10 quantises)."""
    W = onf4.bf16_bits_to_f32(W_bits)
    B = onf4.bf16_bits_to_f32(B_bits)
    A = onf4.bf16_bits_to_f32(A_bits)
    acc = np.zeros(W.shape, dtype=np.float32)
    for j in range(A.shape[0]):
        acc = (acc + B[:, j:j + 1] * A[j:j + 1, :]).astype(np.float32)
    t = (np.float32(s) * acc).astype(np.float32)
    return onf4.f32_to_bf16_bits((W - t).astype(np.float32))


def residual_f32(W_bits: np.ndarray, Wq_bits: np.ndarray | None) -> np.ndarray:
    """R = fl32(W - W') (W' = 0 before the first quantisation)."""
    W = onf4.bf16_bits_to_f32(W_bits)
    if Wq_bits is None:
        return W.astype(np.float32)
    return (W - onf4.bf16_bits_to_f32(Wq_bits)).astype(np.float32)


def loftq(W_bits: np.ndarray, r: int, s, iters: int, power_iters: int,
          omega: np.ndarray, double_quant: bool = True) -> dict:
    """T = ``iters`` alternations of section 3.10's steps on W (d x k bf16
    bits). Returns the last quantised weight ``qw`` (as ``oracle.nf4``'s
    quantize_weight), its dequantised bf16 bits ``Wq``, the factors ``A``
    (r x k) and ``B`` (d x r) as bf16 bits, the last ``sigma`` and the
    Frobenius error of W'_t + s B_t A_t against W after every iteration."""
    if iters < 1:
        raise ValueError("at least one iteration")
    W_bits = np.asarray(W_bits, dtype=np.uint16)
    d, k = W_bits.shape
    Wf = onf4.bf16_bits_to_f32(W_bits).astype(np.float64)
    Wq = None
    errs = []
    for _ in range(iters):
        R = residual_f32(W_bits, Wq)
        U, sigma, Vt = lowrank_svd(R, omega[:, :r], power_iters)
        A, B = lora_factors(U, sigma, Vt, s)
        Wt = residual_bf16(W_bits, B, A, s)
        qw = onf4.quantize_weight(Wt, double_quant)
        Wq = onf4.dequantize_weight(qw).reshape(d, k)
        approx = (onf4.bf16_bits_to_f32(Wq).astype(np.float64)
                  + float(s) * (onf4.bf16_bits_to_f32(B).astype(np.float64)
                                @ onf4.bf16_bits_to_f32(A).astype(np.float64)))
        errs.append(float(np.linalg.norm(Wf - approx)))
    return {"qw": qw, "Wq": Wq, "A": A, "B": B, "sigma": sigma, "errors": errs}
