"""GPU parity of the 32-bit AdamW step (the paged optimiser's update) against
the CPU oracle: bit-exact float32 master parameters, moments and bf16
copies, with the optimiser state in device memory, paged out to page-locked
host memory, and moved between the two from step to step."""

import numpy as np
import pytest

from _helpers import to_dev, to_host_bits
from oracle import adamw as oadam
from oracle.nf4 import f32_to_bf16_bits

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

HP = dict(lr=2e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from bit_nf4_quantized_19_amd import ops as o
    o.lib()
    return o


def _state(n, seed):
    rng = np.random.default_rng(seed)
    p = (rng.standard_normal(n) * 0.02).astype(np.float32)
    return p, np.zeros(n, np.float32), np.zeros(n, np.float32)


def _grad(n, seed, scale=0.01):
    rng = np.random.default_rng(seed)
    return f32_to_bf16_bits((rng.standard_normal(n) * scale).astype(np.float32))


def _f32(a, where):
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    if where == "device":
        return t.cuda()
    return t.pin_memory()


def _bits_equal(got, want):
    return np.array_equal(np.asarray(got, np.float32).view(np.uint32),
                          np.asarray(want, np.float32).view(np.uint32))


@pytest.mark.parametrize("n", [1, 3, 4, 1000, 4096 * 37 + 3])
@pytest.mark.parametrize("where", ["device", "host"])
def test_steps_match_oracle_bit_exact(ops, n, where):
    print(f"[adamw] n={n} state={where}", flush=True)
    p, m, v = _state(n, 10 + n)
    tp, tm, tv = _f32(p, where), _f32(m, where), _f32(v, where)
    out = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    for step in range(1, 5):
        g = _grad(n, 100 * n + step, scale=10.0 ** (-step))   # magnitudes over 4 decades
        ops.adamw_step(tp, tm, tv, to_dev(g), out, step, **HP)
        p, m, v, ob = oadam.adamw_step(p, m, v, g, step=step, **HP)
        torch.cuda.synchronize()
        assert _bits_equal(tp.cpu().numpy(), p), step
        assert _bits_equal(tm.cpu().numpy(), m), step
        assert _bits_equal(tv.cpu().numpy(), v), step
        assert np.array_equal(to_host_bits(out), ob), step


def test_paging_the_state_out_and_back_changes_nothing(ops):
    # step 1 with the state on the device, step 2 paged out to host memory,
    # step 3 paged back: identical bits to three steps on the device
    n = 65536 + 8
    p, m, v = _state(n, 5)
    grads = [to_dev(_grad(n, 50 + s)) for s in range(3)]
    out = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    dev = [_f32(x, "device") for x in (p, m, v)]
    for s in range(3):
        ops.adamw_step(*dev, grads[s], out, s + 1, **HP)
    ref = [x.cpu().numpy() for x in dev]
    st = [_f32(x, "device") for x in (p, m, v)]
    ops.adamw_step(*st, grads[0], out, 1, **HP)
    host = [torch.empty(n, dtype=torch.float32).pin_memory() for _ in range(3)]
    for h, d in zip(host, st):
        h.copy_(d)                      # page out
    torch.cuda.synchronize()
    del st
    ops.adamw_step(*host, grads[1], out, 2, **HP)
    back = [h.cuda() for h in host]    # page in
    ops.adamw_step(*back, grads[2], out, 3, **HP)
    torch.cuda.synchronize()
    for got, want in zip(back, ref):
        assert _bits_equal(got.cpu().numpy(), want)


def test_step_after_backward_on_the_lora_matrices(ops):
    # the optimiser's real inputs: dA and dB of a backward pass, r = 16
    from bit_nf4_quantized_19_amd import synth
    d, k, M, r = 512, 768, 96, 16
    inp = synth.linear_inputs(d, k, M, r, idx=3)
    dev = {n: synth.to_device_bf16(inp[n], torch.device("cuda")) for n in ("W0", "X", "A", "B", "dY")}
    w = ops.quantize(dev["W0"], True)
    Y, H = ops.linear_fwd(w, dev["X"], dev["A"], dev["B"], 32.0)
    dX, dA, dB = ops.linear_bwd(w, dev["X"], dev["A"], dev["B"], 32.0, dev["dY"], H=H)
    for name, P, G in (("A", dev["A"], dA), ("B", dev["B"], dB)):
        n = P.numel()
        p = to_host_bits(P).reshape(-1)
        p32 = (p.astype(np.uint32) << 16).view(np.float32)
        tp, tm, tv = _f32(p32, "device"), _f32(np.zeros(n), "device"), _f32(np.zeros(n), "device")
        out = torch.empty(n, dtype=torch.bfloat16, device="cuda")
        ops.adamw_step(tp, tm, tv, G.reshape(-1), out, 1, **HP)
        g = to_host_bits(G).reshape(-1)
        q, mm, vv, ob = oadam.adamw_step(p32, np.zeros(n), np.zeros(n), g, step=1, **HP)
        torch.cuda.synchronize()
        assert _bits_equal(tp.cpu().numpy(), q), name
        assert np.array_equal(to_host_bits(out), ob), name
        # one step moves every element with a nonzero gradient by ~lr
        moved = np.abs(tp.cpu().numpy() - p32)
        nz = g != 0
        assert np.all(moved[nz] > 0.5 * HP["lr"]) and np.all(moved[nz] < 1.5 * HP["lr"] + 1e-3 * np.abs(p32[nz]))


def test_library_paging_out_and_back_is_bit_exact(ops):
    # steps 1-2 on the device; the library pages the state out to page-locked
    # host memory, the device copies are overwritten, step 3 runs on the
    # host copies, the library pages them back in, step 4 runs on the
    # device: every bit equals four steps of the oracle
    n = 4096 * 5 + 12
    print(f"[adamw] library paging n={n}", flush=True)
    p, m, v = _state(n, 21)
    dev = [_f32(x, "device") for x in (p, m, v)]
    host = [torch.empty(n, dtype=torch.float32).pin_memory() for _ in range(3)]
    out = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    grads = [_grad(n, 70 + s) for s in range(4)]
    want = (p, m, v)
    for s in range(4):
        if s == 2:
            ops.adamw_page_out(host, dev)
            for t in dev:
                t.fill_(float("nan"))   # stream-ordered after the copies
            ops.adamw_step(*host, to_dev(grads[s]), out, s + 1, **HP)
            ops.adamw_page_in(dev, host)
        else:
            ops.adamw_step(*dev, to_dev(grads[s]), out, s + 1, **HP)
        *want, ob = oadam.adamw_step(*want, grads[s], step=s + 1, **HP)
    torch.cuda.synchronize()
    for got, w in zip(dev, want):
        assert _bits_equal(got.cpu().numpy(), w)
    assert np.array_equal(to_host_bits(out), ob)


def test_library_paging_refuses_the_wrong_memory_kind(ops):
    n = 1024
    dev = [torch.zeros(n, dtype=torch.float32, device="cuda") for _ in range(2)]
    pinned = [torch.zeros(n, dtype=torch.float32).pin_memory() for _ in range(2)]
    pageable = [torch.zeros(n, dtype=torch.float32) for _ in range(2)]
    with pytest.raises(ops.QLoRAError):
        ops.adamw_page_out(pageable, dev)        # pageable host destination
    with pytest.raises(ops.QLoRAError):
        ops.adamw_page_out(dev, dev)             # device memory as the host side
    with pytest.raises(ops.QLoRAError):
        ops.adamw_page_in(pinned, pinned)        # host memory as the device side
    ops.adamw_page_out(pinned, dev)
    torch.cuda.synchronize()
