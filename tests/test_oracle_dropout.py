"""Pins of the LoRA-dropout oracle (CPU only): Philox4x32-10 against the
known-answer values its authors publish with the generator, the keep rate
and independence of the mask, gradients by finite differences, and the
p = 0 case against plain LoRA."""

import json
import os

import numpy as np
import pytest

from oracle import dropout as od
from oracle import lora as olora


# Known-answer vectors of Philox4x32-10 as distributed with the generator's
# reference implementation (Random123, kat_vectors): counter, key, output.
KAT = [
    ((0x00000000, 0x00000000, 0x00000000, 0x00000000), (0x00000000, 0x00000000),
     (0x6627e8d5, 0xe169c58d, 0xbc57ac4c, 0x9b00dbd8)),
    ((0xffffffff, 0xffffffff, 0xffffffff, 0xffffffff), (0xffffffff, 0xffffffff),
     (0x408f276d, 0x41c83b0e, 0xa20bc7c6, 0x6d5451fd)),
    ((0x243f6a88, 0x85a308d3, 0x13198a2e, 0x03707344), (0xa4093822, 0x299f31d0),
     (0xd16cfe09, 0x94fdcceb, 0x5001e420, 0x24126ea1)),
]


@pytest.mark.parametrize("ctr,key,want", KAT)
def test_philox_known_answers(ctr, key, want):
    got = od.philox4x32_10(np.array([ctr], dtype=np.uint32), key)[0]
    assert [int(x) for x in got] == list(want)


def test_keep_rate_and_seed_independence():
    M, k, p = 64, 4096, 0.05
    a = od.keep_mask(1234, M, k, p)
    b = od.keep_mask(1235, M, k, p)
    n = a.size
    # binomial: the kept fraction within 6 standard deviations of 1 - p
    sd = np.sqrt(p * (1 - p) / n)
    assert abs(a.mean() - (1 - p)) < 6 * sd
    # two seeds agree on a fraction (1-p)^2 + p^2 of elements
    agree = (a == b).mean()
    q = (1 - p) ** 2 + p ** 2
    assert abs(agree - q) < 6 * np.sqrt(q * (1 - q) / n)
    # the mask of a sub-block equals the corresponding block of a larger mask
    # only through the flat index: rows are independent streams of the index
    assert not np.array_equal(a[0], a[1])


def test_threshold_and_p_zero():
    # the rate is the float32 the library receives: fl32(0.05) = 13421773 *
    # 2^-28, so its threshold is 13421773 * 2^4 (not floor(0.05 * 2^32) =
    # 214748364); fl32(0.1) = 13421773 * 2^-27, fl32(0.3) = 10066330 * 2^-25
    assert od.drop_threshold(0.0) == 0
    assert od.drop_threshold(0.05) == 13421773 * 16 == 214748368
    assert od.drop_threshold(0.1) == 13421773 * 32 == 429496736
    assert od.drop_threshold(0.3) == 10066330 * 128 == 1288490240
    assert od.drop_threshold(0.5) == 2147483648
    assert od.drop_threshold(np.float32(0.1)) == od.drop_threshold(0.1)
    assert od.keep_mask(7, 3, 64, 0.0).all()
    with pytest.raises(ValueError):
        od.drop_threshold(1.0)


def _gap_cases():
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                        "dropout_gap.json")
    with open(path) as f:
        return json.load(f)


@pytest.mark.parametrize("case", _gap_cases(), ids=lambda c: f"p{c['p']}")
def test_gap_element_is_dropped(case):
    # an element whose word lies between the float64 and float32 thresholds
    # (found by tests/golden/dropout_gap.py): dropped at the float32 rate
    p, seed, e = case["p"], case["seed"], case["index"]
    w = int(od.philox_words(seed, e, 1)[0])
    assert w == case["word"]
    assert int(np.floor(p * 4294967296.0)) <= w < od.drop_threshold(p)
    keep = od.keep_mask(seed, case["M"], case["k"], p).reshape(-1)
    assert not keep[e]
    assert keep.mean() > 1 - p - 0.01


def test_gradients_by_finite_differences():
    rng = np.random.default_rng(3)
    d, k, M, r, p = 6, 8, 5, 3, 0.3
    Wd, X = rng.standard_normal((d, k)), rng.standard_normal((M, k))
    A, B = rng.standard_normal((r, k)), rng.standard_normal((d, r))
    dY, s = rng.standard_normal((M, d)), 0.7
    keep = od.keep_mask(99, M, k, p)
    dX, dA, dB, _ = od.backward(Wd, X, A, B, s, dY, keep, p)
    f = lambda X_, A_, B_: float(np.sum(dY * od.forward(Wd, X_, A_, B_, s, keep, p)[0]))
    eps = 1e-6
    for name, T, grad in (("X", X, dX), ("A", A, dA), ("B", B, dB)):
        for idx in [(0, 0), (1, 2), (T.shape[0] - 1, T.shape[1] - 1)]:
            Tp, Tm = T.copy(), T.copy()
            Tp[idx] += eps
            Tm[idx] -= eps
            args_p = {"X": (Tp, A, B), "A": (X, Tp, B), "B": (X, A, Tp)}[name]
            args_m = {"X": (Tm, A, B), "A": (X, Tm, B), "B": (X, A, Tm)}[name]
            num = (f(*args_p) - f(*args_m)) / (2 * eps)
            assert abs(num - grad[idx]) < 1e-6 * max(1.0, abs(num)), (name, idx)


def test_p_zero_is_plain_lora():
    rng = np.random.default_rng(4)
    d, k, M, r = 5, 7, 4, 2
    Wd, X = rng.standard_normal((d, k)), rng.standard_normal((M, k))
    A, B, dY = rng.standard_normal((r, k)), rng.standard_normal((d, r)), rng.standard_normal((M, d))
    keep = od.keep_mask(1, M, k, 0.0)
    Y, H = od.forward(Wd, X, A, B, 0.5, keep, 0.0)
    (Y0, H0), (dX0, dA0, dB0, G0) = od.reduces_to_plain_lora(Wd, X, A, B, 0.5, dY)
    assert np.allclose(Y, Y0) and np.allclose(H, H0)
    dX, dA, dB, G = od.backward(Wd, X, A, B, 0.5, dY, keep, 0.0)
    assert np.allclose(dX, dX0) and np.allclose(dA, dA0) and np.allclose(dB, dB0)
