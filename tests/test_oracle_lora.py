"""Pins for the oracle's LoRA linear (Day-25 notes 2.1, 2.5, 2.6, 6.2;
QLoRA glossary "QLoRA 的工作原理" forward/backward paragraph)."""

import numpy as np

from oracle import lora, nf4


def _tiny(seed, d=64, k=64, M=3, r=2):
    rng = np.random.default_rng(seed)
    W = rng.standard_normal((d, k)) * 0.02
    X = rng.standard_normal((M, k))
    A = rng.standard_normal((r, k)) * 0.1
    B = rng.standard_normal((d, r)) * 0.1
    dY = rng.standard_normal((M, d))
    return W, X, A, B, dY


def test_scale_is_alpha_over_r():
    assert lora.lora_scale(32, 16) == np.float32(2.0)
    assert lora.lora_scale(16, 64) == np.float32(0.25)
    assert lora.lora_scale(16, 8) == np.float32(2.0)


def test_forward_matches_brute_force_loops():
    W, X, A, B, _ = _tiny(0, d=5, k=7, M=3, r=2)
    s = 0.75
    Y, H = lora.forward(W, X, A, B, s)
    for m in range(3):
        for j in range(5):
            base = sum(W[j, c] * X[m, c] for c in range(7))
            ax = [sum(A[t, c] * X[m, c] for c in range(7)) for t in range(2)]
            bax = sum(B[j, t] * ax[t] for t in range(2))
            assert abs(Y[m, j] - (base + s * bax)) < 1e-12
    for m in range(3):
        for t in range(2):
            assert abs(H[m, t] - sum(A[t, c] * X[m, c] for c in range(7))) < 1e-12


def test_gradients_match_central_differences():
    W, X, A, B, R = _tiny(1)
    s = 2.0
    dX, dA, dB, G = lora.backward(W, X, A, B, s, R)
    rng = np.random.default_rng(9)

    def L(X_, A_, B_):
        return float(np.sum(R * lora.forward(W, X_, A_, B_, s)[0]))
    h = 1e-3
    for name, base, grad in (("X", X, dX), ("A", A, dA), ("B", B, dB)):
        V = rng.standard_normal(base.shape)
        args_p = {"X": X, "A": A, "B": B}
        args_m = dict(args_p)
        args_p[name] = base + h * V
        args_m[name] = base - h * V
        fd = (L(**{k + "_": v for k, v in args_p.items()}) -
              L(**{k + "_": v for k, v in args_m.items()})) / (2 * h)
        an = float(np.sum(grad * V))
        assert abs(fd - an) <= 1e-8 * max(1.0, abs(an)), name
    np.testing.assert_allclose(G, R @ B, rtol=1e-13)


def test_zero_B_gives_base_output_and_zero_dA():
    W, X, A, B, dY = _tiny(2)
    B0 = np.zeros_like(B)
    Y, _ = lora.forward(W, X, A, B0, 2.0)
    assert np.array_equal(Y, X @ W.T)
    dX, dA, dB, _ = lora.backward(W, X, A, B0, 2.0, dY)
    assert np.all(dA == 0)
    assert np.any(dB != 0)


def test_merged_weight_equals_unmerged_path():
    W, X, A, B, _ = _tiny(3, d=96, k=128, M=5, r=4)
    s = 0.25
    Y, _ = lora.forward(W, X, A, B, s)
    Wm = lora.merge(W, A, B, s)
    np.testing.assert_allclose(X @ Wm.T, Y, rtol=1e-12, atol=1e-12)


def test_bf16_rounding_from_float64_avoids_double_rounding():
    x = np.array([1 + 2 ** -8 + 2 ** -30, 1 + 2 ** -8, -3.0, 0.0, 2.0 ** -130 * 1.25])
    b = lora.to_bf16(x)
    assert b[0] == 0x3F81          # just above the tie -> up
    assert b[1] == 0x3F80          # exact tie -> even
    assert b[2] == 0xC040 and b[3] == 0
    f = nf4.bf16_bits_to_f32(b)
    assert abs(float(f[4]) - 2.0 ** -130 * 1.25) <= 2.0 ** -134
    rng = np.random.default_rng(4)
    v = rng.standard_normal(10000).astype(np.float32)
    assert np.array_equal(lora.to_bf16(v.astype(np.float64)), nf4.f32_to_bf16_bits(v))
