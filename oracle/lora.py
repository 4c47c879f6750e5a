"""LoRA linear on a frozen dequantised base: forward, backward, merge.

CPU oracle -- test infrastructure only (see ``oracle/__init__.py``).

Pages followed
--------------
* Day-25 LoRA/QLoRA notes (itingyu.github.io), section 2.1 "核心思想":
  ``W = W0 + B A`` with ``W0`` d x k frozen, ``B`` d x r, ``A`` r x k; the
  output is ``W0 x + B A x``.
* Same notes, section 6.2 "alpha 选择": the LoRA branch is scaled by
  ``alpha / r``.
* Same notes, section 2.5: ``B = 0`` at start, so the output equals the base.
* Same notes, section 2.6 / LLM tutorial ch. 3 section 3.8: merging adds
  ``B A`` to the base; a 4-bit base must first be dequantised to bf16.
* QLoRA glossary (Ultralytics), "QLoRA 的工作原理", forward paragraph: the
  frozen weight is dequantised to bfloat16 before the matmul and the LoRA
  output is added; backpropagation goes through the dequantised weight but
  only the two low-rank matrices receive updates.

Conventions: activations are row vectors, ``X`` is M x k (M tokens), so the
layer computes ``Y = X W'^T + s (X A^T) B^T`` with ``s = fl32(alpha / r)``.
Every input is a bf16-exact value widened to float64; all arithmetic is
float64 (the pages fix no accumulation precision); outputs are rounded once
to bf16 by the ``*_bf16`` wrappers. The backward pass is the chain rule of
the forward with upstream gradient ``dY`` (M x d).
"""

from __future__ import annotations

import numpy as np

from .nf4 import f32_to_bf16_bits


def lora_scale(alpha: float, r: int) -> np.float32:
    """``s = alpha / r`` computed in float32 (Day-25 notes, 6.2)."""
    return np.float32(np.float32(alpha) / np.float32(r))


def forward(Wd, X, A, B, s):
    """Float64 forward. Returns ``(Y, H)`` with ``H = X A^T`` (M x r)."""
    Wd, X, A, B = (np.asarray(t, dtype=np.float64) for t in (Wd, X, A, B))
    H = X @ A.T
    Y = X @ Wd.T + float(s) * (H @ B.T)
    return Y, H


def backward(Wd, X, A, B, s, dY):
    """Float64 gradients of ``<dY, Y>`` w.r.t. X, A and B.

    ``G = dY B`` (M x r); ``dX = dY W' + s G A``; ``dA = s G^T X``;
    ``dB = s dY^T H`` with ``H = X A^T``. The frozen base gets no gradient.
    Returns ``(dX, dA, dB, G)``.
    """
    Wd, X, A, B, dY = (np.asarray(t, dtype=np.float64) for t in (Wd, X, A, B, dY))
    s = float(s)
    H = X @ A.T
    G = dY @ B
    dX = dY @ Wd + s * (G @ A)
    dA = s * (G.T @ X)
    dB = s * (dY.T @ H)
    return dX, dA, dB, G


def merge(Wd, A, B, s):
    """Float64 merged weight ``W' + s B A`` (d x k)."""
    Wd, A, B = (np.asarray(t, dtype=np.float64) for t in (Wd, A, B))
    return Wd + float(s) * (B @ A)


def to_bf16(x) -> np.ndarray:
    """Round float64 results once to bf16 bits (via the exact float64 value:
    float64 -> float32 -> bf16 can double-round, so round from float64)."""
    x = np.asarray(x, dtype=np.float64)
    # Round float64 to bf16 directly: keep 8 significant bits, ties to even.
    m, e = np.frexp(x)                       # x = m * 2**e, 0.5 <= |m| < 1
    e = np.maximum(e, -125)                  # bf16 subnormal spacing 2**-133
    scaled = np.ldexp(x, 8 - e)              # |scaled| < 256, exact
    r = np.rint(scaled)                      # ties to even
    y = np.ldexp(r, e - 8).astype(np.float32)  # exact: <= 8 significant bits
    return f32_to_bf16_bits(y)


def forward_bf16(Wd, X, A, B, s):
    Y, H = forward(Wd, X, A, B, s)
    return to_bf16(Y), H


def backward_bf16(Wd, X, A, B, s, dY):
    dX, dA, dB, G = backward(Wd, X, A, B, s, dY)
    return to_bf16(dX), to_bf16(dA), to_bf16(dB), G


def merge_bf16(Wd, A, B, s):
    return to_bf16(merge(Wd, A, B, s))
