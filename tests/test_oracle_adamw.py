"""Pins of the AdamW oracle (CPU only): a library implementation of the same
optimiser, closed forms of its first steps, pure decay and the bias
corrections."""

import numpy as np
import pytest
import torch

from oracle import adamw
from oracle.nf4 import f32_to_bf16_bits, bf16_bits_to_f32

HP = dict(lr=2e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


def _grads(n, steps, seed):
    rng = np.random.default_rng(seed)
    return [f32_to_bf16_bits(rng.standard_normal(n).astype(np.float32) * 0.01) for _ in range(steps)]


def test_matches_torch_adamw_over_several_steps():
    # torch.optim.AdamW (CPU, float32, its own operation order) is an
    # independent implementation of the same update: agreement to a few ulp
    # of the parameter change per step.
    n, steps = 4096, 6
    rng = np.random.default_rng(7)
    p0 = (rng.standard_normal(n) * 0.01).astype(np.float32)
    gs = _grads(n, steps, 8)
    t = torch.nn.Parameter(torch.from_numpy(p0.copy()))
    opt = torch.optim.AdamW([t], lr=HP["lr"], betas=(HP["beta1"], HP["beta2"]), eps=HP["eps"],
                            weight_decay=HP["weight_decay"], foreach=False)
    p, m, v = p0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    for s, g in enumerate(gs, start=1):
        t.grad = torch.from_numpy(bf16_bits_to_f32(g).copy())
        opt.step()
        p, m, v, _ = adamw.adamw_step(p, m, v, g, step=s, **HP)
        ref = t.detach().numpy()
        # parameter change per step is ~lr; allow 1e-4 of it per element
        assert np.max(np.abs(p - ref)) <= 1e-4 * HP["lr"] * s + 1e-9, s
    st = opt.state[t]
    # torch forms m' as a lerp, m + (1 - b1)(g - m): the same value up to a
    # few float32 roundings of the larger terms
    tm, tv = st["exp_avg"].numpy(), st["exp_avg_sq"].numpy()
    assert np.max(np.abs(m - tm)) <= 4e-7 * np.max(np.abs(tm))
    assert np.max(np.abs(v - tv)) <= 4e-7 * np.max(np.abs(tv))


def test_first_step_from_zero_state_is_a_normalised_sign_step():
    # t = 1, m = v = 0: mh = g and vh = g*g up to rounding, so without decay
    # the change is lr * g / (|g| + eps), i.e. ~lr * sign(g) for |g| >> eps.
    n = 1000
    g = _grads(n, 1, 3)[0]
    gf = bf16_bits_to_f32(g).astype(np.float64)
    p0 = np.zeros(n, np.float32) + np.float32(0.5)
    p, m, v, _ = adamw.adamw_step(p0, np.zeros(n), np.zeros(n), g, lr=1e-3, beta1=0.9,
                                  beta2=0.999, eps=1e-8, weight_decay=0.0, step=1)
    expect = 0.5 - 1e-3 * gf / (np.abs(gf) + 1e-8)
    assert np.allclose(p, expect, rtol=0, atol=2e-7)
    assert np.allclose(m, 0.1 * gf, rtol=1e-6)
    assert np.allclose(v, 0.001 * gf * gf, rtol=1e-6)


def test_zero_gradient_is_pure_decoupled_decay():
    n = 257
    p0 = np.linspace(-1, 1, n).astype(np.float32)
    z = np.zeros(n, np.uint16)   # +0.0 in bf16
    p, m, v, _ = adamw.adamw_step(p0, np.zeros(n), np.zeros(n), z, lr=0.1, beta1=0.9,
                                  beta2=0.999, eps=1e-8, weight_decay=0.5, step=3)
    assert np.array_equal(m, np.zeros(n, np.float32)) and np.array_equal(v, np.zeros(n, np.float32))
    # p' = p - lr * (0 + wd * p) = p * (1 - 0.05), rounded twice in float32
    wdp = (np.float32(0.5) * p0).astype(np.float32)
    assert np.array_equal(p, (p0 - (np.float32(0.1) * wdp).astype(np.float32)).astype(np.float32))
    assert np.allclose(p, 0.95 * p0, rtol=1e-6, atol=0)


def test_constant_gradient_keeps_a_constant_step():
    # with a constant gradient from zero state, mh = g and vh = g*g for every
    # t (the bias corrections undo the geometric sums), so each step moves p
    # by the same lr * g / (|g| + eps)
    n, T = 64, 25
    g = np.full(n, f32_to_bf16_bits(np.array([0.0123], np.float32))[0], np.uint16)
    gf = float(bf16_bits_to_f32(g[:1])[0])
    p, m, v = np.zeros(n, np.float32), np.zeros(n, np.float32), np.zeros(n, np.float32)
    for s in range(1, T + 1):
        p, m, v, _ = adamw.adamw_step(p, m, v, g, lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8,
                                      weight_decay=0.0, step=s)
    assert np.allclose(p, -T * 1e-3 * gf / (abs(gf) + 1e-8), rtol=1e-5)
    assert np.allclose(m, gf * (1 - 0.9 ** T), rtol=1e-5)
    assert np.allclose(v, gf * gf * (1 - 0.999 ** T), rtol=1e-4)


def test_bias_corrections_and_bf16_copy():
    bc1, bc2 = adamw.bias_corrections(0.9, 0.999, 1)
    assert bc1 == np.float32(0.1) and bc2 == np.float32(0.001)
    bc1, bc2 = adamw.bias_corrections(0.9, 0.999, 10)
    assert bc1 == np.float32(1 - 0.9 ** 10) and bc2 == np.float32(1 - 0.999 ** 10)
    with pytest.raises(ValueError):
        adamw.bias_corrections(0.9, 0.999, 0)
    n = 100
    g = _grads(n, 1, 5)[0]
    p, _, _, out = adamw.adamw_step(np.ones(n, np.float32), np.zeros(n), np.zeros(n), g, step=1, **HP)
    assert np.array_equal(out, f32_to_bf16_bits(p))
