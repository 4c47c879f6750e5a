"""LoRA dropout on the adapter input, with its counter-based random mask.

CPU oracle -- test infrastructure only (see ``oracle/__init__.py``).

Pages followed
--------------
* LLM-train tutorial ch. 3 (jwzheng96.github.io), section 3.3 code, and
  Day-25 notes 4.3 code: ``LoraConfig(..., lora_dropout=0.05)``; Day-25
  notes 7.x (overfitting remedies): raise lora_dropout to 0.1.
* The pages give the rate only. Reading taken (the plainest one, and the
  meaning of the name in the configuration the pages use): inverted dropout
  on the input of the adapter branch only, ``x~ = x * keep / (1 - p)``; the
  frozen base path sees the undropped ``x``. With dropout the layer is
  ``Y = X W'^T + s (X~ A^T) B^T``; its gradients are
  ``dA = s G^T X~``, ``dB = s dY^T H`` (H = X~ A^T) and
  ``dX = dY W' + s (G A) * keep / (1 - p)``.

The keep decision of element (m, c) of X (M x k) is drawn from the
counter-based generator Philox4x32-10 (Salmon, Moraes, Dror and Shaw,
"Parallel Random Numbers: As Easy as 1, 2, 3", SC'11): with flat index
``e = m * k + c``, counter ``(e // 4 mod 2^32, e // 4 div 2^32, 0, 0)`` and
key ``(seed mod 2^32, seed div 2^32)``, the element keeps when word
``e % 4`` of the output is >= ``floor(p * 2^32)`` (so it drops with
probability p up to 2^-32). The GPU library implements the same generator
from the same published definition.

The rate is a float32 value: the library's interface takes it as a C
``float``, so every function here first rounds the given p to float32
(``rate32``) and uses that value for the threshold and for 1/(1 - p). The
keep decision is an integer comparison, so both sides must start from the
same rate; a float64 0.1 and its float32 rounding give thresholds 7 apart.
"""

from __future__ import annotations

import numpy as np

from . import lora as olora

_M0, _M1 = np.uint64(0xD2511F53), np.uint64(0xCD9E8D57)
_W0, _W1 = 0x9E3779B9, 0xBB67AE85
_MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(ctr, key):
    """Philox4x32 with 10 rounds, vectorised over counters.

    ``ctr``: uint32 array of shape (..., 4); ``key``: two uint32 values.
    Returns the uint32 output block of shape (..., 4). Each round multiplies
    words 0 and 2 by the two round constants (full 64-bit products), mixes
    the high halves with words 1 and 3 and the key, and the key is bumped by
    the two Weyl constants between rounds.
    """
    c = np.asarray(ctr, dtype=np.uint32).astype(np.uint64)
    c0, c1, c2, c3 = c[..., 0], c[..., 1], c[..., 2], c[..., 3]
    k0, k1 = int(key[0]) & 0xFFFFFFFF, int(key[1]) & 0xFFFFFFFF
    for rnd in range(10):
        if rnd:
            k0 = (k0 + _W0) & 0xFFFFFFFF
            k1 = (k1 + _W1) & 0xFFFFFFFF
        p0 = _M0 * c0
        p1 = _M1 * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK32
        c0, c1, c2, c3 = (hi1 ^ c1 ^ np.uint64(k0), lo1, hi0 ^ c3 ^ np.uint64(k1), lo0)
    return np.stack([c0, c1, c2, c3], axis=-1).astype(np.uint32)


def rate32(p: float) -> float:
    """The dropout rate as the library receives it: p rounded to float32."""
    return float(np.float32(p))


def drop_threshold(p: float) -> int:
    """floor(p32 * 2^32) for the float32 rate p32: a random word below it
    drops the element (p32 * 2^32 is exact in float64, so is the floor)."""
    p = rate32(p)
    if not (0.0 <= p < 1.0):
        raise ValueError("dropout rate must be in [0, 1)")
    return int(np.floor(p * 4294967296.0))


def philox_words(seed: int, first: int, count: int) -> np.ndarray:
    """The generator's words for flat element indices first .. first+count-1
    (word e % 4 of the block with counter e // 4)."""
    b0, b1 = first // 4, (first + count - 1) // 4 + 1
    idx = np.arange(b0, b1, dtype=np.uint64)
    ctr = np.zeros((b1 - b0, 4), dtype=np.uint32)
    ctr[:, 0] = (idx & _MASK32).astype(np.uint32)
    ctr[:, 1] = (idx >> np.uint64(32)).astype(np.uint32)
    out = philox4x32_10(ctr, (seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)).reshape(-1)
    return out[first - 4 * b0:first - 4 * b0 + count]


def keep_mask(seed: int, M: int, k: int, p: float) -> np.ndarray:
    """Boolean keep mask of X (M x k) for rate p and a 64-bit seed."""
    out = philox_words(seed, 0, M * k)
    return (out >= np.uint32(drop_threshold(p))).reshape(M, k)


def forward(Wd, X, A, B, s, keep, p):
    """Float64 forward with dropout on the adapter input (rate p taken as
    float32, like the keep mask). Returns (Y, H)."""
    p = rate32(p)
    Wd, X, A, B = (np.asarray(t, dtype=np.float64) for t in (Wd, X, A, B))
    Xd = X * keep / (1.0 - p)
    H = Xd @ A.T
    Y = X @ Wd.T + float(s) * (H @ B.T)
    return Y, H


def backward(Wd, X, A, B, s, dY, keep, p):
    """Float64 gradients of <dY, Y> for the forward above: (dX, dA, dB, G)."""
    p = rate32(p)
    Wd, X, A, B, dY = (np.asarray(t, dtype=np.float64) for t in (Wd, X, A, B, dY))
    s = float(s)
    Xd = X * keep / (1.0 - p)
    H = Xd @ A.T
    G = dY @ B
    dX = dY @ Wd + s * (G @ A) * keep / (1.0 - p)
    dA = s * (G.T @ Xd)
    dB = s * (dY.T @ H)
    return dX, dA, dB, G


def reduces_to_plain_lora(Wd, X, A, B, s, dY):
    """p = 0 keeps every element: the plain LoRA forward and backward."""
    return olora.forward(Wd, X, A, B, s), olora.backward(Wd, X, A, B, s, dY)
