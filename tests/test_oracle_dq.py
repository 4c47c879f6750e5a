"""Pins for the oracle's double quantisation and storage accounting
(QLoRA glossary, Ultralytics, "QLoRA 的工作原理" and "权衡"; LLM tutorial
ch. 3 "双重量化"; Day-25 notes 3.3)."""

import json
import os
from fractions import Fraction

import numpy as np

from oracle import nf4

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _gold():
    with open(os.path.join(GOLDEN, "storage_figures.json")) as f:
        return json.load(f)


def _model_65b_linears(g):
    h, i = g["model_65b_shape"]["hidden"], g["model_65b_shape"]["intermediate"]
    per_layer = [(h, h)] * 4 + [(i, h), (i, h), (h, i)]
    return per_layer * g["model_65b_shape"]["layers"]


def test_bits_per_param_closed_forms():
    g = _gold()
    d = k = 4096
    n = d * k
    no_dq = (nf4.storage_bytes(d, k, False) - n // 2) * 8 / n
    dq = (nf4.storage_bytes(d, k, True) - n // 2) * 8 / n
    assert no_dq == g["absmax_bits_per_param"]["value"]
    assert round(dq, g["dq_bits_per_param"]["printed_digits"]) == g["dq_bits_per_param"]["value"]
    # one int8 per block, one float32 per 256 blocks, one float32 mean
    assert abs(dq - (8 / 64 + 32 / (64 * 256) + 32 / n)) < 1e-12


def test_65b_storage_figures():
    g = _gold()
    lin = _model_65b_linears(g)
    params = sum(d * k for d, k in lin)
    dq = sum(nf4.storage_bytes(d, k, True) for d, k in lin) / 1e9
    no_dq = sum(nf4.storage_bytes(d, k, False) for d, k in lin) / 1e9
    bf16 = 2 * params / 1e9

    def close(x, key):
        return abs(x - g[key]["value"]) <= g[key]["rel_tol"] * g[key]["value"]
    assert close(dq, "nf4_dq_65b_gb")
    assert close(no_dq - dq, "dq_saving_65b_gb")
    assert close(bf16, "bf16_65b_gb")
    assert 0.24 < dq / bf16 < 0.27     # "about a quarter"


def test_fraction_to_f32_is_correct_rounding():
    rng = np.random.default_rng(0)
    xs = np.concatenate([rng.standard_normal(2000) * 10.0 ** rng.integers(-40, 38, 2000),
                         rng.standard_normal(200) * 1e-42,     # float32 subnormal range
                         [1 + 2 ** -24, 1 + 3 * 2 ** -24, 2 ** -149 * 1.5, 2 ** -149 * 2.5]])
    for x in xs:
        # float64 -> float32 by numpy is a single correct rounding of x
        assert nf4.fraction_to_f32(Fraction(float(x))) == np.float32(x)


def test_exact_mean():
    assert nf4.exact_mean_f32(np.array([1, 2], np.float32)) == np.float32(1.5)
    v = np.full(1000, 0.0371, np.float32)
    assert nf4.exact_mean_f32(v) == v[0]
    a = np.array([1.0, 1.0, 2.0 ** -30], np.float32)
    want = np.float32(Fraction(2) / 3 + Fraction(1, 3 * 2 ** 30))
    assert nf4.exact_mean_f32(a) == nf4.fraction_to_f32(Fraction(2, 3) + Fraction(1, 3 * 2 ** 30))
    assert abs(float(nf4.exact_mean_f32(a)) - float(want)) <= 2 ** -24
    rng = np.random.default_rng(1)
    a = np.abs(rng.standard_normal(5000)).astype(np.float32)
    ex = sum(Fraction(float(t)) for t in a) / a.size
    assert nf4.exact_mean_f32(a) == nf4.fraction_to_f32(ex)


def _absmax_of_normal_weight(d, k, seed):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal(d * k).astype(np.float32) * np.float32(0.02))
    _, a = nf4.quantize_blocks(w)
    return a


def test_double_quant_error_bound():
    a = _absmax_of_normal_weight(1024, 4096, 2)
    q, s2, mu = nf4.double_quantize(a)
    ad = nf4.dequantize_absmax(q, s2, mu)
    s2_per_block = np.repeat(s2, 256)[: a.size].astype(np.float64)
    ulp = np.spacing(np.float32(a.max()))
    err = np.abs(ad.astype(np.float64) - a.astype(np.float64))
    assert np.all(err <= 0.5 * s2_per_block * (1 + 2 ** -16) + 2 * ulp)
    # the quantised absmax stays within about 1% of the exact one
    assert np.max(err / a) < 1e-2
    assert q.min() >= -127 and q.max() <= 127
    assert np.any(np.abs(q) == 127)


def test_equal_absmax_group_is_exact():
    a = np.full(512, 0.0431, np.float32)
    q, s2, mu = nf4.double_quantize(a)
    assert mu == a[0] and np.all(s2 == 0) and np.all(q == 0)
    assert np.array_equal(nf4.dequantize_absmax(q, s2, mu), a)


def test_int8_codes_round_half_even_and_clamp():
    # a = [1, 3] -> mu = 2, d = [-1, 1], s2 = fl(1/127): q = -127, 127.
    q, s2, mu = nf4.double_quantize(np.array([1.0, 3.0], np.float32))
    assert mu == 2.0 and s2[0] == np.float32(np.float32(1) / np.float32(127))
    assert list(q) == [-127, 127]
    # Symmetric values around 4 give mu = 4 exactly and g = 127 -> s2 = 1, so
    # d / s2 hits exact halves: 2.5 -> 2 and -2.5 -> -2 (half to even),
    # 3.5 -> 4, 0.5 -> 0.
    a = np.array([4.0, 6.5, 1.5, 131.0, -123.0, 7.5, 0.5, 4.5, 3.5], np.float32)
    q, s2, mu = nf4.double_quantize(a)
    assert mu == np.float32(4.0) and s2[0] == np.float32(1.0)
    assert list(q) == [0, 2, -2, 127, -127, 4, -4, 0, 0]


def test_partial_last_group():
    a = _absmax_of_normal_weight(3, 64 * 300, 4)     # 900 blocks -> 4 groups
    q, s2, mu = nf4.double_quantize(a)
    assert s2.size == 4 and q.size == 900
    ad = nf4.dequantize_absmax(q, s2, mu)
    assert np.max(np.abs(ad - a) / a) < 1e-2
