"""Pins for the oracle's blockwise NF4 quantiser and dequantiser
(QLoRA glossary, Ultralytics, "QLoRA 的工作原理")."""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import nf4

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _mse(w, levels):
    codes, absmax = nf4.quantize_blocks(w, levels)
    restored = nf4.restore_f32(codes, absmax, levels)
    diff = restored.astype(np.float64) - w.reshape(-1).astype(np.float64)
    return float(np.mean(diff * diff))


def test_page_example_mse_values():
    torch = pytest.importorskip("torch")
    with open(os.path.join(GOLDEN, "p4_snippet_mse.json")) as f:
        gold = json.load(f)
    torch.manual_seed(0)
    w = (torch.randn(4096, 64) * 0.02).numpy().astype(np.float32)
    nf4_mse = _mse(w, nf4.nf4_levels())
    int4_mse = _mse(w, nf4.int4_levels())
    assert f"{nf4_mse:.3e}" == gold["nf4_mse"]
    assert f"{int4_mse:.3e}" == gold["int4_mse"]


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_nf4_error_below_int4_on_normal_blocks(seed):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((2048, 64)).astype(np.float32) * np.float32(0.02))
    ratio = _mse(w, nf4.nf4_levels()) / _mse(w, nf4.int4_levels())
    # the page reports about 16% lower error (3.395e-6 / 4.053e-6 = 0.838)
    assert 0.78 < ratio < 0.90


def test_level_times_absmax_round_trips():
    rng = np.random.default_rng(7)
    L = nf4.nf4_levels()
    nblk = 4000
    a = (np.exp(rng.uniform(-12, 4, nblk)).astype(np.float32))
    idx = np.stack([rng.permutation(np.tile(np.arange(16), 4)) for _ in range(nblk)])
    w = (L[idx] * a[:, None]).astype(np.float32)       # contains -a and +a
    codes, absmax = nf4.quantize_blocks(w.reshape(-1))
    assert np.array_equal(absmax, a)
    assert np.array_equal(codes.reshape(nblk, 64), idx.astype(np.uint8))


def _f32(x):
    return np.float32(x)


def test_ties_go_to_the_lower_level():
    # Search float32 x near each midpoint for exact float32 distance ties and
    # check the lower index wins (argmin returns the first minimum).
    L = nf4.nf4_levels()
    found = 0
    for i in range(15):
        mid = (np.float64(L[i]) + np.float64(L[i + 1])) / 2
        x0 = np.float32(mid)
        cand = [np.nextafter(x0, np.float32(-2), dtype=np.float32)]
        x = x0
        for _ in range(6):
            cand.append(x)
            x = np.nextafter(x, np.float32(2), dtype=np.float32)
        for x in cand:
            dl = abs(np.float32(x - L[i]))
            dh = abs(np.float32(x - L[i + 1]))
            if dl == dh:
                found += 1
                w = np.full(64, x, dtype=np.float32)
                w[0] = 1.0   # absmax 1 -> x = w exactly
                codes, _ = nf4.quantize_blocks(w)
                assert codes[1] == i
    assert found >= 3, "expected exact float32 ties on several level pairs"


def test_codes_are_monotone_in_x():
    # Threshold form == nearest-level form: the code never decreases as x
    # grows. Dense sample of float32 in [-1, 1].
    rng = np.random.default_rng(11)
    x = np.sort(np.concatenate([
        rng.uniform(-1, 1, 1 << 20).astype(np.float32),
        np.linspace(-1, 1, 1 << 18, dtype=np.float32)]))
    c = nf4.nearest_level(x, nf4.nf4_levels()).astype(np.int16)
    assert np.all(np.diff(c) >= 0)
    assert c[0] == 0 and c[-1] == 15


def test_brute_force_exact_distances_on_tiny_blocks():
    rng = np.random.default_rng(5)
    L = nf4.nf4_levels()
    Lq = [Fraction(float(v)) for v in L]
    w = (rng.standard_normal(64 * 40).astype(np.float32) * np.float32(0.02))
    codes, absmax = nf4.quantize_blocks(w)
    for b in range(40):
        a = absmax[b]
        for j in range(64):
            x = np.float32(w[64 * b + j] / a)
            ex = Fraction(float(x))
            dist = [abs(ex - l) for l in Lq]
            best = min(dist)
            c = int(codes[64 * b + j])
            # exact nearest level unless two distances agree within 1 ulp
            assert dist[c] - best <= Fraction(1, 1 << 24)
            if dist[c] != best:
                assert sorted(dist)[1] - best <= Fraction(1, 1 << 24)


def test_zero_block_uses_the_zero_level():
    w = np.zeros(128, dtype=np.float32)
    w[64:] = np.float32(0.5)
    w[64] = np.float32(-0.0)
    codes, absmax = nf4.quantize_blocks(w)
    assert absmax[0] == 0 and np.all(codes[:64] == nf4.ZERO_CODE)
    deq = nf4.dequantize_bf16(codes, absmax)
    assert np.all(deq[:64] == 0)


def test_nibble_order_high_nibble_first():
    a = np.float32(0.25)
    w = np.zeros(64, dtype=np.float32)
    w[0], w[1], w[2], w[3] = -a, a, 0, a
    codes, _ = nf4.quantize_blocks(w)
    packed = nf4.pack_codes(codes)
    assert packed[0] == 0x0F and packed[1] == 0x7F and packed[2] == 0x77
    assert np.array_equal(nf4.unpack_codes(packed), codes)


def test_subnormal_weights_quantise_like_normal_ones():
    # Scaling a block by a power of two leaves every code unchanged.
    rng = np.random.default_rng(3)
    w = rng.standard_normal(64 * 16).astype(np.float32)
    w = nf4.bf16_bits_to_f32(nf4.f32_to_bf16_bits(w))        # 8 significant bits
    c_ref, _ = nf4.quantize_blocks(w)
    tiny = (w * np.float32(2.0 ** -130)).astype(np.float32)  # float32 subnormals
    back = (tiny * np.float32(2.0 ** 65) * np.float32(2.0 ** 65)).astype(np.float32)
    exact = back == w
    c_tiny, a_tiny = nf4.quantize_blocks(tiny)
    blocks_exact = exact.reshape(-1, 64).all(axis=1)
    assert blocks_exact.sum() >= 8
    assert np.all(np.abs(tiny) < np.finfo(np.float32).tiny)
    cr = c_ref.reshape(-1, 64)[blocks_exact]
    ct = c_tiny.reshape(-1, 64)[blocks_exact]
    assert np.array_equal(cr, ct)
    assert np.all(a_tiny > 0)


def test_dequantised_values_round_to_bf16_nearest_even():
    # 1 + 2**-8 is a bf16 tie -> rounds to even (1.0); 1 + 3*2**-8 -> up.
    v = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8)], dtype=np.float32)
    bits = nf4.f32_to_bf16_bits(v)
    assert bits[0] == 0x3F80 and bits[1] == 0x3F82 and bits[2] == 0xBF80
    # dequant of a block: level * absmax in float32 then bf16
    codes = np.arange(64, dtype=np.uint8) % 16
    a = np.array([0.0371], dtype=np.float32)
    got = nf4.bf16_bits_to_f32(nf4.dequantize_bf16(codes, a))
    want = nf4.bf16_bits_to_f32(nf4.f32_to_bf16_bits(
        (nf4.nf4_levels()[codes] * a[0]).astype(np.float32)))
    assert np.array_equal(got, want)
    assert np.max(np.abs(got - nf4.nf4_levels()[codes] * a[0])) <= 2 ** -9 * 0.0371
