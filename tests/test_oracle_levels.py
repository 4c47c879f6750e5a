"""Pins for the oracle's NF4 level table (QLoRA glossary, Ultralytics,
"QLoRA 的工作原理": NF4 bullet and snippet)."""

import math

import numpy as np
import pytest

from oracle import nf4


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
    # Map each normalised level back through the normal CDF (erfc: a different
    # routine from the inverse CDF used to build them) and recover the grid.
    Lf = nf4.nf4_levels_f64()
    zmax = abs(np.float64(0)) + 0.0
    # the positive end is the quantile of the top probability
    from statistics import NormalDist
    zmax = NormalDist().inv_cdf(nf4.P_TOP)
    assert abs(_phi(zmax) - nf4.P_TOP) < 1e-15
    pos_p = np.linspace(nf4.P_TOP, 0.5, 9)[:-1]
    neg_p = np.linspace(nf4.P_TOP, 0.5, 8)[:-1]
    got_pos = sorted(_phi(z * zmax) for z in Lf[8:])
    got_neg = sorted(1.0 - _phi(z * zmax) for z in Lf[:7])
    np.testing.assert_allclose(got_pos, sorted(pos_p), rtol=0, atol=2e-15)
    np.testing.assert_allclose(got_neg, sorted(neg_p), rtol=0, atol=2e-15)


def test_inverse_cdf_agrees_with_scipy():
    sp = pytest.importorskip("scipy.special")
    from statistics import NormalDist
    icdf = NormalDist().inv_cdf
    ps = np.concatenate([np.linspace(nf4.P_TOP, 0.5, 9), np.linspace(0.01, 0.99, 99)])
    for p in ps:
        a, b = icdf(p), float(sp.ndtri(p))
        assert abs(a - b) <= 1e-15 * max(1.0, abs(b)) + 1e-16


def test_snippet_float32_construction_is_within_8_ulp():
    # The page builds the table with torch in float32; the oracle's table is
    # the float64 construction rounded once. They differ by a few ulp (the
    # float32 probability grid and float32 inverse CDF), never by more than 8.
    torch = pytest.importorskip("torch")
    normal = torch.distributions.Normal(0.0, 1.0)
    positive = normal.icdf(torch.linspace(0.9677083, 0.5, 9)[:-1])
    negative = -normal.icdf(torch.linspace(0.9677083, 0.5, 8)[:-1])
    t = torch.cat([negative, torch.zeros(1), positive]).sort().values
    t = (t / t.max()).numpy().astype(np.float32)
    L = nf4.nf4_levels()
    # ulp distance on the ordered integer line of float32
    def key(a):
        u = a.view(np.int32).astype(np.int64)
        return np.where(u < 0, -(u & 0x7FFFFFFF), u)
    assert np.max(np.abs(key(t) - key(L))) <= 8
    np.testing.assert_allclose(t, L, rtol=1e-6, atol=0)


def test_int4_levels_evenly_spaced():
    I = nf4.int4_levels()
    assert I.shape == (16,) and I[0] == -1 and I[-1] == 1
    np.testing.assert_allclose(np.diff(I.astype(np.float64)), 2.0 / 15, rtol=1e-6)
