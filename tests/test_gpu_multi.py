"""GPU checks of the sibling-projection forward (qlora_linear_fwd_multi):
weights that read the same X (q/k/v, gate/up) in one call give bit-identical
Y and H to separate qlora_linear_fwd calls, on the GEMV path (one grouped
launch) and the GEMM path (one launch for all H, one grouped GEMM), and
agree with the float64 oracle."""

import numpy as np
import pytest

from _helpers import oracle_linear, oracle_quant, oracle_wdeq, rel_frob, bf16_f64, to_dev, to_host_bits
from bit_nf4_quantized_19_amd import synth

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from bit_nf4_quantized_19_amd import ops as o
    o.lib()
    return o


CASES = [
    # (d list, k, M, r, dq)
    ([704, 704], 1088, 1, 16, True),          # gate/up shaped, ragged slice
    ([192, 320, 64], 2112, 2, 16, False),     # two tokens (VALU path), three sizes
    ([256, 512], 4096, 1, 16, True),           # one token, aligned int8 codes (dword loads)
    ([512, 256, 768], 2112, 4, 16, True),      # q/k/v-like, three sizes
    ([1024, 1024, 1024, 1024], 1024, 16, 16, False),  # four weights, absmax path
    ([200, 320], 576, 7, 5, True),             # padded ranks, ragged row groups
    ([256, 512], 512, 40, 16, True),           # GEMM path
    ([136, 264, 64], 192, 300, 8, False),      # GEMM path, ragged tiles, padded ranks
    ([128, 64, 192, 256], 320, 100, 16, True), # GEMM path, four weights in one launch
    ([4096, 4096, 4096], 4096, 512, 16, True), # q/k/v-shaped
]


@pytest.mark.parametrize("ds,k,M,r,dq", CASES)
def test_multi_equals_separate_calls(ops, ds, k, M, r, dq):
    print(f"[multi] d={ds} k={k} M={M} r={r} dq={dq}", flush=True)
    dev = torch.device("cuda")
    alpha = 2.0 * r
    X = synth.normal_bf16_device((M, k), 1.0, 7100 + M, device=dev)
    ws_, As, Bs = [], [], []
    for i, d in enumerate(ds):
        ws_.append(ops.quantize(synth.normal_bf16_device((d, k), 0.02, 7200 + i, device=dev), dq))
        As.append(synth.normal_bf16_device((r, k), 0.01, 7300 + i, device=dev))
        Bs.append(synth.normal_bf16_device((d, r), 0.01, 7400 + i, device=dev))
    Ys, Hs = ops.linear_fwd_multi(ws_, X, As, Bs, alpha)
    for i in range(len(ds)):
        Y1, H1 = ops.linear_fwd(ws_[i], X, As[i], Bs[i], alpha)
        torch.cuda.synchronize()
        assert np.array_equal(to_host_bits(Ys[i]), to_host_bits(Y1)), i
        assert np.array_equal(Hs[i].cpu().numpy().view(np.uint32), H1.cpu().numpy().view(np.uint32)), i


def test_multi_matches_oracle(ops):
    # gate/up-shaped pair against the float64 oracle (tolerance of the layer)
    ds, k, M, r = [320, 448], 1024, 4, 16
    dev = torch.device("cuda")
    Xb = synth.normal_bf16((M, k), 1.0, 7500)
    X = to_dev(Xb)
    ws_, As, Bs, inps = [], [], [], []
    for i, d in enumerate(ds):
        inp = {"W0": synth.normal_bf16((d, k), 0.02, 7600 + i), "X": Xb,
               "A": synth.normal_bf16((r, k), 0.01, 7700 + i),
               "B": synth.normal_bf16((d, r), 0.01, 7800 + i)}
        inps.append(inp)
        ws_.append(ops.quantize(to_dev(inp["W0"]), True))
        As.append(to_dev(inp["A"]))
        Bs.append(to_dev(inp["B"]))
    Ys, Hs = ops.linear_fwd_multi(ws_, X, As, Bs, 32.0)
    torch.cuda.synchronize()
    for i, (d, inp) in enumerate(zip(ds, inps)):
        qw = oracle_quant(inp["W0"], True)
        o = oracle_linear(oracle_wdeq(qw, d, k), inp["X"], inp["A"], inp["B"], 32.0, r, None)
        assert rel_frob(bf16_f64(to_host_bits(Ys[i])), o["Y"]) <= 2e-2
        assert rel_frob(Hs[i].cpu().numpy().astype(np.float64), o["H"]) < 1e-5


def test_multi_rejects_mismatched_weights(ops):
    dev = torch.device("cuda")
    X = synth.normal_bf16_device((4, 512), 1.0, 1, device=dev)
    w1 = ops.quantize(synth.normal_bf16_device((64, 512), 0.02, 2, device=dev), True)
    w2 = ops.quantize(synth.normal_bf16_device((64, 256), 0.02, 3, device=dev), True)  # other k
    A = synth.normal_bf16_device((16, 512), 0.01, 4, device=dev)
    B = synth.normal_bf16_device((64, 16), 0.01, 5, device=dev)
    with pytest.raises(ops.QLoRAError):
        ops.linear_fwd_multi([w1, w2], X, [A, A], [B, B], 32.0)


def test_qkv_multi_matches_oracle(ops):
    # q, k, v of a Llama-7B-shaped block (3 x 4096 x 4096, NF4 + DQ) reading
    # the same 2048 tokens, r = 16, alpha = 32, in one call: each Y_i and H_i
    # against the float64 oracle, and each rank-r term through the delta of a
    # second call with every B_i = 0 (the term is ~4% of |Y_i|; the rounded
    # deltas are compared as in test_gpu_lora_delta)
    from oracle import lora as olora
    d = k = 4096
    M, r, alpha = 2048, 16, 32.0
    print(f"[multi-oracle] 3 x {d}x{k} M={M} r={r}", flush=True)
    Xb = synth.normal_bf16((M, k), 1.0, 7900)
    X = to_dev(Xb)
    inps = [{"W0": synth.normal_bf16((d, k), 0.02, 7910 + i),
             "A": synth.normal_bf16((r, k), 0.01, 7920 + i),
             "B": synth.normal_bf16((d, r), 0.01, 7930 + i)} for i in range(3)]
    ws_ = [ops.quantize(to_dev(p["W0"]), True) for p in inps]
    As = [to_dev(p["A"]) for p in inps]
    Bs = [to_dev(p["B"]) for p in inps]
    Ys, Hs = ops.linear_fwd_multi(ws_, X, As, Bs, alpha)
    Y0s, _ = ops.linear_fwd_multi(ws_, X, As, [torch.zeros_like(b) for b in Bs], alpha)
    torch.cuda.synchronize()
    s = float(olora.lora_scale(alpha, r))
    Xf = bf16_f64(Xb)
    rb = lambda a: bf16_f64(olora.to_bf16(a))
    for i, p in enumerate(inps):
        Wd = oracle_wdeq(oracle_quant(p["W0"], True), d, k)
        H = Xf @ bf16_f64(p["A"]).T
        base = Xf @ Wd.T
        full = base + s * (H @ bf16_f64(p["B"]).T)
        Yg, Y0g = bf16_f64(to_host_bits(Ys[i])), bf16_f64(to_host_bits(Y0s[i]))
        errs = (rel_frob(Yg, full), rel_frob(Hs[i].cpu().numpy().astype(np.float64), H),
                rel_frob(Yg - Y0g, rb(full) - rb(base)))
        print(f"   weight {i}: Y {errs[0]:.2e} H {errs[1]:.2e} delta {errs[2]:.2e}", flush=True)
        assert errs[0] <= 2e-2 and errs[1] < 1e-5 and errs[2] <= 2e-2, (i, errs)
