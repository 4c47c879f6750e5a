"""Shared test utilities: device transfer of bf16 bit arrays, comparisons, and
oracle pipelines over the seeded synthetic inputs. Not a test module."""

from __future__ import annotations

import numpy as np

from oracle import lora as olora
from oracle import nf4 as onf4


def rel_frob(got, want) -> float:
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    den = np.linalg.norm(want)
    num = np.linalg.norm(got - want)
    return float(num / den) if den > 0 else float(num)


def bf16_f64(bits) -> np.ndarray:
    return onf4.bf16_bits_to_f32(np.asarray(bits, dtype=np.uint16)).astype(np.float64)


def to_dev(bits: np.ndarray):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).cuda()


def to_host_bits(t) -> np.ndarray:
    import torch
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def oracle_quant(W0_bits: np.ndarray, dq: bool) -> dict:
    return onf4.quantize_weight(W0_bits, dq)


def oracle_wdeq(qw: dict, d: int, k: int) -> np.ndarray:
    """Oracle dequantised weight as float64 (d x k), from its bf16 bits."""
    return bf16_f64(onf4.dequantize_weight(qw)).reshape(d, k)


def oracle_linear(Wd, X_bits, A_bits, B_bits, alpha, r, dY_bits=None):
    s = olora.lora_scale(alpha, r)
    X, A, B = bf16_f64(X_bits), bf16_f64(A_bits), bf16_f64(B_bits)
    Y, H = olora.forward(Wd, X, A, B, s)
    out = {"Y": Y, "H": H}
    if dY_bits is not None:
        dY = bf16_f64(dY_bits)
        dX, dA, dB, G = olora.backward(Wd, X, A, B, s, dY)
        out.update(dX=dX, dA=dA, dB=dB, G=G)
    return out


def bf16_ulp_diff(a_bits, b_bits) -> np.ndarray:
    """Distance in bf16 ulps on the ordered integer line."""
    def key(b):
        u = np.asarray(b, dtype=np.uint16).astype(np.int32)
        return np.where(u & 0x8000, -(u & 0x7FFF), u)
    return np.abs(key(a_bits) - key(b_bits))


def oracle_deq_blocks(W0_bits: np.ndarray, dq: bool, block_ids: np.ndarray):
    """Oracle dequantised values of selected 64-blocks (float64 [nsel, 64]).

    The double-quant record needs every block's absmax (the mean and the
    group scales), which is cheap; the codes are computed only for the
    selected blocks (each block is quantised on its own)."""
    wf = onf4.bf16_bits_to_f32(np.asarray(W0_bits).reshape(-1))
    a = onf4.block_absmax(wf)
    if dq:
        q, s2, mu = onf4.double_quantize(a)
        a_deq = onf4.dequantize_absmax(q, s2, mu)
    else:
        a_deq = a
    blocks = wf.reshape(-1, 64)[block_ids]
    codes, _ = onf4.quantize_blocks(blocks.reshape(-1))
    vals = onf4.dequantize_bf16(codes, a_deq[block_ids])
    return bf16_f64(vals).reshape(-1, 64)
