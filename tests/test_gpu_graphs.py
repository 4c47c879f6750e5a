"""The C ABI only enqueues work on the caller's stream (no allocation, no
synchronisation, no memset): a HIP graph captured from a quantise + forward +
backward sequence replays bit-identically to the eager calls, replay after
replay with other eager work in between, and calls on a non-default stream
give the same bits as on the default one."""

import numpy as np
import pytest

from _helpers import to_dev, to_host_bits
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


def _ws(ops, op, d, k, M, r, dev):
    n = ops.workspace_bytes(op, d, k, M, r, True)
    t = torch.empty(n + 256, dtype=torch.uint8, device=dev)
    off = (-t.data_ptr()) % 256
    return t[off:off + n]


def _bufs(ops, d, k, M, r, dev):
    return {"w": ops.NF4Weight.empty(d, k, True, dev),
            "Y": torch.empty(M, d, dtype=torch.bfloat16, device=dev),
            "H": torch.empty(M, r, dtype=torch.float32, device=dev),
            "dX": torch.empty(M, k, dtype=torch.bfloat16, device=dev),
            "dA": torch.empty(r, k, dtype=torch.bfloat16, device=dev),
            "dB": torch.empty(d, r, dtype=torch.bfloat16, device=dev),
            "wsq": _ws(ops, ops.OP_QUANTIZE, d, k, M, r, dev),
            "wsf": _ws(ops, ops.OP_FWD, d, k, M, r, dev),
            "wsb": _ws(ops, ops.OP_BWD, d, k, M, r, dev)}


def _sequence(ops, t, b, alpha, dropout, stream=None):
    mask = b.get("mask")
    ops.quantize(t["W0"], True, out=b["w"], ws=b["wsq"], stream=stream)
    ops.linear_fwd(b["w"], t["X"], t["A"], t["B"], alpha, Y=b["Y"], H=b["H"], ws=b["wsf"],
                   stream=stream, dropout=dropout, seed=99, mask=mask)
    ops.linear_bwd(b["w"], t["X"], t["A"], t["B"], alpha, t["dY"], H=b["H"], dX=b["dX"],
                   dA=b["dA"], dB=b["dB"], ws=b["wsb"], stream=stream, dropout=dropout, seed=99,
                   mask=mask)


def _snapshot(b):
    return {"codes": b["w"].codes.cpu().numpy(), "q": b["w"].absmax_q.cpu().numpy(),
            "Y": to_host_bits(b["Y"]), "H": b["H"].cpu().numpy().view(np.uint32),
            "dX": to_host_bits(b["dX"]), "dA": to_host_bits(b["dA"]), "dB": to_host_bits(b["dB"])}


@pytest.mark.parametrize("d,k,M,r,dropout,mask", [
    (512, 768, 96, 16, 0.0, False),    # GEMM path
    (1024, 1088, 4, 16, 0.0, False),   # GEMV path
    (1024, 2112, 1, 16, 0.0, False),   # GEMV path for one token (VALU)
    (512, 768, 96, 16, 0.1, False),    # with dropout (bits redrawn in the backward)
    (512, 768, 96, 16, 0.1, True)])    # with dropout, bits stored by the forward
def test_graph_replays_match_eager(ops, d, k, M, r, dropout, mask):
    print(f"[graph] d={d} k={k} M={M} r={r} p={dropout} mask={mask}", flush=True)
    dev = torch.device("cuda")
    inp = synth.linear_inputs(d, k, M, r, idx=21)
    t = {n: to_dev(inp[n]) for n in ("W0", "X", "A", "B", "dY")}
    eager = _bufs(ops, d, k, M, r, dev)
    if mask:
        eager["mask"] = ops.dropout_mask(M, k, dev)
    _sequence(ops, t, eager, 32.0, dropout)
    torch.cuda.synchronize()
    want = _snapshot(eager)
    if mask:
        want["mask"] = eager["mask"].cpu().numpy()

    b = _bufs(ops, d, k, M, r, dev)
    if mask:
        b["mask"] = ops.dropout_mask(M, k, dev)
    _sequence(ops, t, b, 32.0, dropout)   # warm-up outside the capture
    torch.cuda.synchronize()
    for key in ("Y", "dX", "dA", "dB"):
        b[key].zero_()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            _sequence(ops, t, b, 32.0, dropout)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    other = _bufs(ops, d, k, M, r, dev)
    for rep in range(3):
        for key in ("Y", "dX", "dA", "dB", "H"):
            b[key].fill_(7.0)
        b["w"].codes.fill_(0)
        if mask:
            b["mask"].fill_(0)
        g.replay()
        torch.cuda.synchronize()
        got = _snapshot(b)
        if mask:
            got["mask"] = b["mask"].cpu().numpy()
        for key in want:
            assert np.array_equal(got[key], want[key]), (rep, key)
        if mask:
            other["mask"] = ops.dropout_mask(M, k, dev)
        _sequence(ops, t, other, 32.0, dropout)   # eager work between replays
        torch.cuda.synchronize()


def test_non_default_stream_gives_the_same_bits(ops):
    d, k, M, r = 512, 768, 96, 16
    dev = torch.device("cuda")
    inp = synth.linear_inputs(d, k, M, r, idx=22)
    t = {n: to_dev(inp[n]) for n in ("W0", "X", "A", "B", "dY")}
    a = _bufs(ops, d, k, M, r, dev)
    _sequence(ops, t, a, 32.0, 0.0)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    b = _bufs(ops, d, k, M, r, dev)
    with torch.cuda.stream(s):
        _sequence(ops, t, b, 32.0, 0.0, stream=s)
    s.synchronize()
    wa, wb = _snapshot(a), _snapshot(b)
    for key in wa:
        assert np.array_equal(wa[key], wb[key]), key
