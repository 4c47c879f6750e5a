"""Pins for the oracle's NF4 level table (QLoRA glossary, Ultralytics,
"QLoRA 的工作原理": NF4 bullet and the worked example after the bullets).

The table is pinned by its closed-form properties, by mapping every level
back through the normal CDF (a different routine from the quantile function
that builds it), and by the mean squared errors the page prints for its
worked example (tests/golden/p4_snippet_mse.json): the float32 table
reproduces both printed figures, and plausible misreadings of the
construction do not."""

import json
import math
import os
from statistics import NormalDist

import numpy as np
import pytest

from oracle import nf4

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_sixteen_levels_exact_zero_and_unit_ends():
    L = nf4.nf4_levels()
    assert L.shape == (16,) and L.dtype == np.float32
    assert np.all(np.diff(L) > 0), "levels must be strictly increasing"
    assert L.view(np.uint32)[7] == 0, "level 7 must be +0.0 exactly"
    assert L[0] == np.float32(-1.0) and L[15] == np.float32(1.0)
    assert int((L > 0).sum()) == 8 and int((L < 0).sum()) == 7


def _phi(x):
    return 0.5 * math.erfc(-x / math.sqrt(2.0))


def test_levels_are_the_stated_normal_quantiles():
    # Map each normalised level back through the normal CDF (erfc) and recover
    # the evenly spaced probabilities: 8 steps from 1/2 to the top on the
    # positive side, 7 on the negative side.
    Lf = nf4.nf4_levels_f64()
    zmax = NormalDist().inv_cdf(nf4.P_TOP)
    assert abs(_phi(zmax) - nf4.P_TOP) < 1e-15
    span = nf4.P_TOP - 0.5
    want_pos = [0.5 + j * span / 8 for j in range(1, 9)]
    want_neg = [0.5 + j * span / 7 for j in range(1, 8)]
    got_pos = sorted(_phi(z * zmax) for z in Lf[8:])
    got_neg = sorted(1.0 - _phi(z * zmax) for z in Lf[:7])
    np.testing.assert_allclose(got_pos, want_pos, rtol=0, atol=2e-15)
    np.testing.assert_allclose(got_neg, want_neg, rtol=0, atol=2e-15)


def test_inverse_cdf_agrees_with_scipy():
    sp = pytest.importorskip("scipy.special")
    icdf = NormalDist().inv_cdf
    ps = np.concatenate([[0.5 + j * (nf4.P_TOP - 0.5) / 8 for j in range(9)],
                         np.linspace(0.01, 0.99, 99)])
    for p in ps:
        a, b = icdf(p), float(sp.ndtri(p))
        assert abs(a - b) <= 1e-15 * max(1.0, abs(b)) + 1e-16


def _page_example_mse(levels):
    """Mean squared error of the page's worked example with `levels`: the
    example's seeded weights (4096 blocks of 64 normal values times 0.02),
    coded to the nearest level after dividing by each block's absmax and
    restored as level times absmax."""
    torch = pytest.importorskip("torch")
    torch.manual_seed(0)
    w = (torch.randn(4096, 64) * 0.02).numpy().astype(np.float32)
    codes, absmax = nf4.quantize_blocks(w, levels)
    restored = nf4.restore_f32(codes, absmax, levels)
    diff = restored.astype(np.float64) - w.reshape(-1).astype(np.float64)
    return f"{float(np.mean(diff * diff)):.3e}"


def _golden():
    with open(os.path.join(GOLDEN, "p4_snippet_mse.json")) as f:
        return json.load(f)


def test_float32_table_reproduces_the_printed_errors():
    g = _golden()
    assert _page_example_mse(nf4.nf4_levels()) == g["nf4_mse"]
    assert _page_example_mse(nf4.int4_levels()) == g["int4_mse"]


def _normalised(v):
    v = np.sort(np.asarray(v, np.float64))
    return (v / v.max()).astype(np.float32)


@pytest.mark.parametrize("reading", ["midpoint_quantiles", "split_7_positive_8_negative",
                                     "no_zero_level", "top_probability_one_step_lower"])
def test_misreadings_miss_the_printed_error(reading):
    # Each is a plausible wrong construction; the page's printed NF4 figure
    # must reject it (so the golden value pins the table, not just its shape).
    z = NormalDist().inv_cdf
    span = nf4.P_TOP - 0.5
    if reading == "midpoint_quantiles":       # q_i = z((i + 1/2) / 16)
        L = _normalised([z((i + 0.5) / 16) for i in range(16)])
    elif reading == "split_7_positive_8_negative":
        L = _normalised([z(0.5 + j * span / 7) for j in range(1, 8)] + [0.0] +
                        [-z(0.5 + j * span / 8) for j in range(1, 9)])
    elif reading == "no_zero_level":          # 8 + 8 quantiles, no exact zero
        L = _normalised([z(0.5 + j * span / 8) for j in range(1, 9)] +
                        [-z(0.5 + j * span / 8) for j in range(1, 9)])
    else:                                     # grid top at 1/2 + 7/8 of the span
        top = 0.5 + 7 * span / 8
        s2 = top - 0.5
        L = _normalised([z(0.5 + j * s2 / 8) for j in range(1, 9)] + [0.0] +
                        [-z(0.5 + j * s2 / 7) for j in range(1, 8)])
    assert L.shape == (16,)
    assert _page_example_mse(L) != _golden()["nf4_mse"], reading


def test_int4_levels_evenly_spaced():
    I = nf4.int4_levels()
    assert I.shape == (16,) and I[0] == -1 and I[-1] == 1
    np.testing.assert_allclose(np.diff(I.astype(np.float64)), 2.0 / 15, rtol=1e-6)
