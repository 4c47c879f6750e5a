"""NF4 levels, blockwise quantisation, double quantisation, dequantisation.

CPU oracle -- test infrastructure only (see ``oracle/__init__.py``).

Pages followed
--------------
* QLoRA glossary (Ultralytics, zh), section "QLoRA 的工作原理":
  - NF4 bullet: each weight is a 4-bit code indexing one of 16 levels placed
    at normal quantiles; every 64 weights form a block with one absmax scale.
  - double-quantisation bullet: the per-block scales are themselves quantised
    to 8 bits in blocks of 256 scales (0.5 -> about 0.127 bit per parameter).
  - the worked example after the bullets: the levels are standard-normal
    quantiles at probabilities spaced evenly between 1/2 and a top
    probability the example gives (0.9677083), eight steps on the positive
    side and seven, mirrored, on the negative side, plus an exact zero, all
    divided by the positive end so they span [-1, 1]; a weight is coded as
    the level nearest to it after division by its block's absmax, and
    restored as that level times the absmax.
  - forward paragraph: frozen weights are dequantised to bfloat16 before the
    matrix product.
* Day-25 LoRA/QLoRA notes (itingyu.github.io), section 3.3 "双重量化":
  first the weights are quantised (giving float32 constants), then those
  constants are quantised to 8 bits.
* LLM-train tutorial ch. 3 (jwzheng96.github.io), section "双重量化": one
  float32 absmax per 64-element block costs 32/64 = 0.5 bit per parameter.

Readings where the pages are silent
----------------------------------
* Levels: each probability 1/2 + (j/n)(p_top - 1/2) is formed exactly and
  rounded once to float64 (p_top the float64 nearest the printed decimal),
  the quantile is evaluated in float64, and the normalised level is rounded
  once to float32.
* Tie-break of the nearest-level search: lowest index.
* All-zero block (absmax 0, ``0/0`` undefined): every code is the zero level.
* Code packing: element ``2j`` in the high nibble of byte ``j``.
* 8-bit absmax format: one global float32 mean ``mu`` (the exact mean of all
  block absmax values, rounded once to float32), then per group of 256
  blocks a float32 scale ``s2 = fl(max|a - mu| / 127)`` and int8 codes
  ``q = clamp(rne(fl((a - mu) / s2)), -127, 127)``; ``s2 == 0`` gives q = 0.
* Dequantised absmax ``a' = fl(fl(q * s2) + mu)`` (no fused multiply-add);
  without double quantisation ``a' = a``.
* Dequantised weight ``w' = bf16_rne(fl(level[code] * a'))``.
"""

from __future__ import annotations

from fractions import Fraction
from statistics import NormalDist

import numpy as np

#: Top probability of the quantile grid, as printed in the glossary's worked
#: example (QLoRA glossary, "QLoRA 的工作原理").
P_TOP = 0.9677083
BLOCKSIZE = 64
DQ_GROUP = 256
ZERO_CODE = 7  # index of the exact-zero level in the ascending table


# --------------------------------------------------------------------------
# Levels
# --------------------------------------------------------------------------
def _grid_probability(j: int, n: int) -> float:
    """1/2 + (j/n)(P_TOP - 1/2), formed exactly and rounded once; j = n gives
    P_TOP itself."""
    return float(Fraction(1, 2) + Fraction(j, n) * (Fraction(P_TOP) - Fraction(1, 2)))


def nf4_levels_f64() -> np.ndarray:
    """The 16 NF4 levels in float64, ascending.

    QLoRA glossary (Ultralytics), "QLoRA 的工作原理" (NF4 bullet and the worked
    example): with z the standard-normal quantile function, the positive
    levels are z(p_j) for p_j = 1/2 + (j/8)(P_TOP - 1/2), j = 1..8; the
    negative levels are -z(p) at p = 1/2 + (j/7)(P_TOP - 1/2), j = 1..7; level
    zero is exact; every level is divided by the positive end z(P_TOP), so the
    table runs from -1 to 1.
    """
    z = NormalDist(0.0, 1.0).inv_cdf
    top = z(P_TOP)
    negative = [-z(_grid_probability(j, 7)) / top for j in range(7, 0, -1)]
    positive = [z(_grid_probability(j, 8)) / top for j in range(1, 9)]
    return np.array(negative + [0.0] + positive, dtype=np.float64)


def nf4_levels() -> np.ndarray:
    """The float32 level table (float64 construction rounded once)."""
    return nf4_levels_f64().astype(np.float32)


def int4_levels() -> np.ndarray:
    """16 evenly spaced levels from -1 to 1 (step 2/15), the grid the
    glossary's worked example compares NF4 against (QLoRA glossary, "QLoRA
    的工作原理")."""
    return np.linspace(-1.0, 1.0, 16).astype(np.float32)


# --------------------------------------------------------------------------
# Blockwise quantisation
# --------------------------------------------------------------------------
def nearest_level(x: np.ndarray, levels: np.ndarray) -> np.ndarray:
    """Index of the level nearest to each float32 ``x``.

    Nearest by absolute difference, the difference taken as one float32
    subtraction; among equal distances the lowest index wins.
    """
    x = np.asarray(x, dtype=np.float32)
    lv = np.asarray(levels, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint8)
    flat_x, flat_o = x.reshape(-1), out.reshape(-1)
    step = 1 << 20  # elementwise; chunked only to bound memory
    for s in range(0, flat_x.size, step):
        dist = np.abs(flat_x[s:s + step, None] - lv[None, :])
        flat_o[s:s + step] = dist.argmin(axis=1)
    return out


def block_absmax(w: np.ndarray, blocksize: int = BLOCKSIZE) -> np.ndarray:
    """``a = max |w|`` over each block of ``blocksize`` consecutive weights
    (QLoRA glossary, "QLoRA 的工作原理": one absmax scale per 64 weights)."""
    w = np.asarray(w, dtype=np.float32).reshape(-1)
    if w.size % blocksize:
        raise ValueError("length must be a multiple of the blocksize")
    return np.abs(w.reshape(-1, blocksize)).max(axis=1)


def quantize_blocks(w: np.ndarray, levels: np.ndarray | None = None,
                    blocksize: int = BLOCKSIZE):
    """Blockwise absmax quantisation of a flat float32 array.

    QLoRA glossary, "QLoRA 的工作原理" (NF4 bullet and worked example): per block of
    ``blocksize`` consecutive weights, ``a = max |w|``, ``x = fl(w / a)``,
    code = nearest level. Returns ``(codes uint8 [n], absmax float32 [nb])``.
    An all-zero block gets the zero level's code.
    """
    lv = nf4_levels() if levels is None else np.asarray(levels, np.float32)
    w = np.asarray(w, dtype=np.float32).reshape(-1)
    absmax = block_absmax(w, blocksize)
    wb = w.reshape(-1, blocksize)
    with np.errstate(invalid="ignore", divide="ignore"):
        x = wb / absmax[:, None]  # IEEE float32 division, correctly rounded
    codes = nearest_level(x, lv)
    zero_code = int(np.flatnonzero(lv == 0.0)[0]) if (lv == 0).any() else 0
    codes[absmax == 0] = zero_code
    return codes.reshape(-1), absmax


def pack_codes(codes: np.ndarray) -> np.ndarray:
    """Two codes per byte: element ``2j`` -> high nibble of byte ``j``."""
    c = np.asarray(codes, dtype=np.uint8).reshape(-1)
    return ((c[0::2] << 4) | c[1::2]).astype(np.uint8)


def unpack_codes(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8).reshape(-1)
    out = np.empty(p.size * 2, dtype=np.uint8)
    out[0::2] = p >> 4
    out[1::2] = p & 0x0F
    return out


# --------------------------------------------------------------------------
# Double quantisation of the absmax values
# --------------------------------------------------------------------------
def fraction_to_f32(q: Fraction) -> np.float32:
    """Round an exact rational to the nearest float32, ties to even."""
    if q == 0:
        return np.float32(0.0)
    sign = -1 if q < 0 else 1
    q = abs(q)
    # exponent e with 2**e <= q < 2**(e+1)
    e = q.numerator.bit_length() - q.denominator.bit_length()
    if Fraction(2) ** e > q:
        e -= 1
    e = max(e, -126)                     # below this the spacing is 2**-149
    quantum = Fraction(2) ** (e - 23)
    n = round(q / quantum)               # Fraction.__round__: half to even
    value = float(n) * 2.0 ** (e - 23)   # exact in float64
    if value > float(np.finfo(np.float32).max):
        return np.float32(sign * np.inf)
    return np.float32(sign * value)


def exact_mean_f32(a: np.ndarray) -> np.float32:
    """Mean of float32 values: exact rational mean, rounded once to float32.

    Every float32 is an integer multiple of 2**-149, so the sum is an exact
    Python integer in those units.
    """
    a = np.asarray(a, dtype=np.float32).reshape(-1)
    units = (a.astype(np.float64) * 2.0 ** 149).tolist()  # exact scaling
    total = sum(int(u) for u in units)
    return fraction_to_f32(Fraction(total, a.size) / Fraction(2) ** 149)


def double_quantize(absmax: np.ndarray, group: int = DQ_GROUP):
    """8-bit quantisation of the block absmax values, 256 per group.

    QLoRA glossary, "QLoRA 的工作原理", double-quantisation bullet; Day-25
    notes section 3.3 (first quantise the weights, then their constants).
    Mean subtraction and the int8 format are the reading described in the
    module docstring. Returns ``(q int8 [nb], s2 float32 [ng], mu float32)``.
    """
    a = np.asarray(absmax, dtype=np.float32).reshape(-1)
    nb = a.size
    ng = -(-nb // group)
    mu = exact_mean_f32(a)
    d = (a - mu).astype(np.float32)            # float32 subtraction
    q = np.zeros(nb, dtype=np.int8)
    s2 = np.zeros(ng, dtype=np.float32)
    for g in range(ng):
        dg = d[g * group:(g + 1) * group]
        gmax = np.abs(dg).max()
        scale = np.float32(gmax / np.float32(127.0))   # float32 division
        s2[g] = scale
        if scale == 0:
            continue
        r = np.rint(dg / scale)              # float32 division, then RNE
        q[g * group:(g + 1) * group] = np.clip(r, -127, 127).astype(np.int8)
    return q, s2, mu


def dequantize_absmax(q: np.ndarray, s2: np.ndarray, mu, group: int = DQ_GROUP):
    """``a' = fl(fl(q * s2) + mu)`` per block, float32, no fused multiply-add."""
    q = np.asarray(q, dtype=np.int8).reshape(-1)
    s2 = np.asarray(s2, dtype=np.float32).reshape(-1)
    scale = np.repeat(s2, group)[: q.size]
    prod = (q.astype(np.float32) * scale).astype(np.float32)
    return (prod + np.float32(mu)).astype(np.float32)


# --------------------------------------------------------------------------
# Dequantisation
# --------------------------------------------------------------------------
def restore_f32(codes: np.ndarray, absmax_deq: np.ndarray,
                levels: np.ndarray | None = None,
                blocksize: int = BLOCKSIZE) -> np.ndarray:
    """``levels[code] * a'`` in float32: a weight is restored as its level
    times its block's scale (QLoRA glossary, "QLoRA 的工作原理")."""
    lv = nf4_levels() if levels is None else np.asarray(levels, np.float32)
    c = np.asarray(codes, dtype=np.uint8).reshape(-1, blocksize)
    a = np.asarray(absmax_deq, dtype=np.float32).reshape(-1, 1)
    return (lv[c] * a).astype(np.float32).reshape(-1)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bits."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    r[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def dequantize_bf16(codes, absmax_deq, levels=None) -> np.ndarray:
    """``w' = bf16(fl(level[code] * a'))`` (forward paragraph of the glossary
    page: weights are dequantised to bfloat16 before the matmul)."""
    return f32_to_bf16_bits(restore_f32(codes, absmax_deq, levels))


# --------------------------------------------------------------------------
# Whole-tensor convenience and storage
# --------------------------------------------------------------------------
def quantize_weight(w_bf16_bits: np.ndarray, double_quant: bool):
    """Quantise a bf16 weight (uint16 bits, any shape, row-major).

    Returns a dict with ``codes`` (packed uint8), and either ``absmax``
    (float32) or ``q``, ``s2``, ``mu``.
    """
    w = bf16_bits_to_f32(np.asarray(w_bf16_bits).reshape(-1))
    codes, absmax = quantize_blocks(w)
    out = {"codes": pack_codes(codes), "codes_unpacked": codes}
    if double_quant:
        q, s2, mu = double_quantize(absmax)
        out.update(q=q, s2=s2, mu=mu, absmax_exact=absmax)
    else:
        out.update(absmax=absmax)
    return out


def dequantize_weight(qw: dict) -> np.ndarray:
    """bf16 bits of the dequantised weight, flat."""
    codes = qw.get("codes_unpacked")
    if codes is None:
        codes = unpack_codes(qw["codes"])
    if "q" in qw:
        a = dequantize_absmax(qw["q"], qw["s2"], qw["mu"])
    else:
        a = qw["absmax"]
    return dequantize_bf16(codes, a)


def storage_bytes(d: int, k: int, double_quant: bool) -> int:
    """Bytes of one quantised d x k weight: packed codes plus scales.

    Without double quantisation one float32 per block (0.5 bit/param, LLM
    tutorial ch. 3 "双重量化"); with it one byte per block, one float32 per
    256 blocks and one float32 mean.
    """
    n = d * k
    nb = n // BLOCKSIZE
    if not double_quant:
        return n // 2 + 4 * nb
    ng = -(-nb // DQ_GROUP)
    return n // 2 + nb + 4 * ng + 4
