"""Seeded synthetic inputs for the QLoRA NF4 linear.

This module generates inputs only; it holds none of the method's arithmetic
and imports nothing else from this package, so the CPU oracle's tests and the
HIP path's tests can draw identical inputs from it.

Every tensor is drawn in float32 from ``numpy.random.default_rng(seed)``
(normal, given standard deviation) and rounded to bfloat16 (nearest, ties to
even); arrays are returned as uint16 bf16 bit patterns. The distributions are
those of the workloads the pages describe: pretrained weights roughly normal
with std 0.02 (QLoRA glossary, "QLoRA 的工作原理" snippet), activations and
upstream gradients N(0, 1), LoRA A ~ N(0, 0.01) and B = 0 at start then
N(0, 0.01) (Day-25 notes, section 2.5).
"""

from __future__ import annotations

import numpy as np

# Seed bases per tensor role; a layer/linear index is added on top.
SEED_W0, SEED_X, SEED_A, SEED_B, SEED_DY = 1000, 2000, 3000, 4000, 5000


def _round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def normal_bf16(shape, std: float, seed: int) -> np.ndarray:
    """bf16 bits of ``std * N(0, 1)`` drawn in float32 with ``seed``."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(size=shape, dtype=np.float32) * np.float32(std)
    return _round_to_bf16_bits(x).reshape(shape)


def normal_f32(shape, seed: int) -> np.ndarray:
    """float32 ``N(0, 1)`` drawn with ``seed`` (a Gaussian test matrix for the
    randomized range finder of the LoftQ factorisation)."""
    rng = np.random.default_rng(seed)
    return rng.standard_normal(size=shape, dtype=np.float32)


def lowrank_bf16(d: int, k: int, rank: int, scale: float, noise: float, seed: int) -> np.ndarray:
    """bf16 bits of a d x k matrix with ``rank`` dominant directions plus noise:
    ``sum_j scale * (1 - j / (2 rank)) u_j v_j^T + noise * N(0, 1)`` with
    u_j, v_j unit vectors drawn from ``seed`` (a weight with a decaying
    spectrum, as pretrained weights have, unlike i.i.d. normal ones)."""
    rng = np.random.default_rng(seed)
    U = rng.standard_normal((d, rank))
    V = rng.standard_normal((k, rank))
    U /= np.linalg.norm(U, axis=0)
    V /= np.linalg.norm(V, axis=0)
    sv = scale * (1.0 - np.arange(rank) / (2.0 * rank))
    x = (U * sv) @ V.T + noise * rng.standard_normal((d, k))
    return _round_to_bf16_bits(x.astype(np.float32)).reshape(d, k)


def zeros_bf16(shape) -> np.ndarray:
    return np.zeros(shape, dtype=np.uint16)


def bf16_to_float(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bits to float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def linear_inputs(d: int, k: int, M: int, r: int, idx: int = 0,
                  w_std: float = 0.02, ab_std: float = 0.01,
                  b_zero: bool = False, with_dy: bool = True) -> dict:
    """All inputs of one linear: W0 (d x k), X (M x k), A (r x k), B (d x r),
    dY (M x d). ``idx`` selects the seeds (layer * 16 + linear index)."""
    out = {
        "W0": normal_bf16((d, k), w_std, SEED_W0 + idx),
        "X": normal_bf16((M, k), 1.0, SEED_X + idx),
        "A": normal_bf16((r, k), ab_std, SEED_A + idx),
        "B": zeros_bf16((d, r)) if b_zero else normal_bf16((d, r), ab_std, SEED_B + idx),
    }
    if with_dy:
        out["dY"] = normal_bf16((M, d), 1.0, SEED_DY + idx)
    return out


def to_device_bf16(bits: np.ndarray, device="cuda"):
    """Copy bf16 bits (uint16 array) to a torch.bfloat16 device tensor."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).to(device)


def normal_bf16_device(shape, std: float, seed: int, device="cuda"):
    """Device-side variant for shapes too large to draw on the host: a seeded
    torch generator on ``device``, float32 normal times ``std``, rounded to
    bf16 by torch (nearest even). Returns a torch.bfloat16 tensor."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    return (x * std).to(torch.bfloat16)
