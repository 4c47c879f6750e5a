#!/usr/bin/env python3
"""Benchmark of the QLoRA NF4 linear on one MI355X.

A step is one training step of the frozen-base linear on the Llama-7B-shaped
q_proj workload: W0 4096 x 4096 stored as NF4 (blocks of 64) with
double-quantised absmax (8-bit, groups of 256), 2048 tokens (batch 4 x
sequence 512), LoRA r = 16, alpha = 32: the forward pass (LoRA down
projection H = X A^T, fused dequant-GEMM with the LoRA epilogue) and the
backward pass (G and dB from one pass over dY, dA, fused dequant-GEMM for
dX). Inputs are seeded synthetic tensors already resident in HBM. The weight
is quantised once before timing (a frozen base is quantised at load time).

Printed: one JSON line with the step throughput in TFLOP/s (algorithmic
flops 4Mdk + 6Mr(d+k) per step), the roofline of the dominant kernel timed
with HIP events inside the timed region, the CPU oracle timed on the host,
and per-row measurements of every other kernel of the path (quantise,
dequantise, decode-shaped GEMV, merge) on inputs rotated through more than
the 256 MB last-level cache.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "QLoRA linear fwd+bwd TFLOP/s & dequant/GEMV HBM GB/s (% roofline), 1×MI355X"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
D = K = 4096
M = 2048
R = 16
ALPHA = 32.0


def step_flops(M, d, k, r):
    return 4 * M * d * k + 6 * M * r * (d + k)


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def source_digest(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "bit_nf4_quantized_19_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_for(kernel, digest):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when the kernel source changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic_counters.json")
    try:
        with open(path) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    e = data.get("kernels", {}).get(kernel)
    if not e or e.get("source_digest") != digest:
        return None
    return e.get("bytes_per_launch")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--spinup", type=float, default=0.25, metavar="SECONDS",
                    help="untimed steps for this long before the warm-up steps, so the timed "
                         "steps run at the settled clock (0 = none)")
    ap.add_argument("--cpu-baseline", choices=["on", "off"], default="on")
    ap.add_argument("--rows", choices=["on", "off"], default="on")
    ap.add_argument("--configs", choices=["on", "off"], default="on",
                    help="the seven-linear Llama-7B block and the 80-layer 65B-shaped stack")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only copy a MIB-sized bf16 buffer 4 times (a plain copy kernel of "
                         "known size, to scale HBM byte counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this path runs on a single MI355X "
              "(the multi-GPU sharding is a design note, not a measured mode).")
        sys.exit(2)

    import numpy as np
    import torch
    from bit_nf4_quantized_19_amd import ops, synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        nbytes = args.copy_calibration << 20
        src = torch.ones(nbytes // 2, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": nbytes, "bytes_written": nbytes,
                          "launches": 4}), flush=True)
        return
    ops.lib()
    log(f"[bench] device {torch.cuda.get_device_name(0)}")

    inp = synth.linear_inputs(D, K, M, R, idx=0)
    W0 = synth.to_device_bf16(inp["W0"], dev)
    X, A, B, dY = (synth.to_device_bf16(inp[n], dev) for n in ("X", "A", "B", "dY"))
    w = ops.quantize(W0, double_quant=True)
    Y = torch.empty(M, D, dtype=torch.bfloat16, device=dev)
    H = torch.empty(M, R, dtype=torch.float32, device=dev)
    dX = torch.empty(M, K, dtype=torch.bfloat16, device=dev)
    dA = torch.empty(R, K, dtype=torch.bfloat16, device=dev)
    dB = torch.empty(D, R, dtype=torch.bfloat16, device=dev)

    def ws(op):
        n = ops.workspace_bytes(op, D, K, M, R, True)
        t = torch.empty(n + 256, dtype=torch.uint8, device=dev)
        off = (-t.data_ptr()) % 256
        return t[off:off + n]
    ws_f, ws_b = ws(ops.OP_FWD), ws(ops.OP_BWD)

    def step():
        ops.linear_fwd(w, X, A, B, ALPHA, save_h=True, Y=Y, H=H, ws=ws_f)
        ops.linear_bwd(w, X, A, B, ALPHA, dY, H=H, dX=dX, dA=dA, dB=dB, ws=ws_b)

    # the clock ramps up over the first ~0.05 s of sustained load: spin up
    # untimed first, then the W warm-up steps
    t_spin = time.perf_counter()
    while args.spinup > 0 and time.perf_counter() - t_spin < args.spinup:
        for _ in range(25):
            step()
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] warmup {args.warmup} done; timing {args.steps} steps")
    # timed region: the product library, nothing but the K steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    flops = step_flops(M, D, K, R)
    tflops = flops / (ms_step * 1e-3) / 1e12
    log(f"[bench] {ms_step:.3f} ms/step, {tflops:.1f} TFLOP/s")

    # kernel durations: the same K steps again through the timing build of
    # the same sources (identical kernels; HIP events recorded on the launch
    # stream around the two fused GEMMs, the candidates for the dominant
    # kernel), then one more pass with events around every kernel
    kern = {}
    with ops.timing_build():
        for _ in range(25):
            step()
        torch.cuda.synchronize()
        ops.profile_begin(8 * max(1, args.steps), kernels=("gemm_fwd", "gemm_dx"))
        t2 = time.perf_counter()
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        t3 = time.perf_counter()
        ops.profile_end()
        ms_step_timed = (t3 - t2) * 1e3 / args.steps
        for name in ("gemm_fwd", "gemm_dx"):
            cnt, tot = ops.profile_query(name)
            if cnt:
                kern[name] = {"launches": cnt, "avg_us": 1e3 * tot / cnt}
        ops.profile_begin(64 * max(1, args.steps))
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        ops.profile_end()
        for name in ops.KERNELS:
            if name in kern:
                continue
            cnt, tot = ops.profile_query(name)
            if cnt:
                kern[name] = {"launches": cnt, "avg_us": 1e3 * tot / cnt}
    fwd_gemm_flops = 2 * M * D * K + 2 * M * R * D
    dx_gemm_flops = 2 * M * D * K + 2 * M * R * K
    cand = [("gemm_fwd", fwd_gemm_flops, "gemm.hip"), ("gemm_dx", dx_gemm_flops, "gemm.hip")]
    dom = max(cand, key=lambda c: kern.get(c[0], {"avg_us": 0})["avg_us"])
    avg_s = kern[dom[0]]["avg_us"] * 1e-6
    achieved = dom[1] / avg_s / 1e12
    digest = source_digest(dom[2], "common.h")
    roofline = {"kernel": dom[0], "bound": "mfma", "achieved": round(achieved, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": traffic_for(dom[0], digest),
                "algorithmic_flops_per_launch": dom[1], "avg_launch_us": round(avg_s * 1e6, 2),
                "events_pass_ms_per_step": round(ms_step_timed, 4)}

    rows = measure_rows(ops, synth, torch, dev) if args.rows == "on" else None
    if rows is not None:
        # the same step with dropout 0.05 on the adapter input (mask drawn in
        # the kernels from a per-step seed) against the step without
        dmask = ops.dropout_mask(M, K, dev)

        def step_drop(i):   # the forward stores the keep bits, the backward reads them
            ops.linear_fwd(w, X, A, B, ALPHA, save_h=True, Y=Y, H=H, ws=ws_f,
                           dropout=0.05, seed=1000 + i, mask=dmask)
            ops.linear_bwd(w, X, A, B, ALPHA, dY, H=H, dX=dX, dA=dA, dB=dB, ws=ws_b,
                           dropout=0.05, seed=1000 + i, mask=dmask)
        ms_plain = _rotated(lambda i: step(), 1, 20)
        ms_drop = _rotated(step_drop, 4, 20)
        rows["lora_dropout_step"] = {
            "p": 0.05, "shape": [D, K], "tokens": M, "r": R,
            "step_ms_plain": round(ms_plain, 4), "step_ms_dropout": round(ms_drop, 4),
            "overhead_frac": round(ms_drop / ms_plain - 1.0, 4),
            "gemm_dx_us_dropout": round(_kernel_us(ops, "gemm_dx", step_drop, 4, 8), 2),
            "lora_colacc_us_dropout": round(_kernel_us(ops, "lora_colacc", step_drop, 4, 8), 2),
            "lora_down_us_dropout": round(_kernel_us(ops, "lora_down", step_drop, 4, 8), 2)}
        log(f"[bench] dropout row: {json.dumps(rows['lora_dropout_step'])}")
    configs = None
    if args.configs == "on":
        configs = {"llama7b_block": measure_block7b(ops, torch, dev, args.cpu_baseline == "on"),
                   "stack65b": measure_stack65b(ops, torch, dev, args.cpu_baseline == "on")}
    probes = measure_probes(torch, dev) if args.rows == "on" else None
    if probes:
        roofline["frac_of_measured_gemm_probe"] = round(achieved / probes["bf16_gemm_8192_TFLOP_s"], 4)
        probes["nf4_step_over_bf16_lora_step"] = round(ms_step / probes["bf16_lora_step_ms"], 4)
    cpu = cpu_baseline(inp, flops) if args.cpu_baseline == "on" else None

    line = {
        "metric": METRIC, "value": round(tflops, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "spinup_s": args.spinup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded normal: W0 ~ N(0,0.02), X, dY ~ N(0,1), A, B ~ N(0,0.01))",
        "config": {"workload": "llama7b_q_proj_nf4_dq_4096x4096_tokens2048_r16_fwd_bwd",
                   "d": D, "k": K, "tokens": M, "r": R, "lora_alpha": ALPHA,
                   "blocksize": 64, "double_quant": True, "dq_blocksize": 256,
                   "parallelism": "single_gpu"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "kernels_us": {k: round(v["avg_us"], 2) for k, v in kern.items()},
        "rows": rows,
        "probes": probes,
        "configs": configs,
    }
    print(json.dumps(line), flush=True)


def _rotated(fn, n_sets, iters):
    """Average milliseconds of fn(i % n_sets) over iters calls, events on the
    current stream."""
    import torch
    for i in range(n_sets):
        fn(i)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for i in range(iters):
        fn(i % n_sets)
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / iters


def _graphed(fn, n_sets, iters):
    """Average milliseconds per call of fn(i) when the n_sets calls are
    captured once in a HIP graph and replayed (launch overhead of the Python
    binding excluded); None if the capture fails."""
    import torch
    try:
        for i in range(n_sets):
            fn(i)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                for i in range(n_sets):
                    fn(i)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        reps = max(1, iters // n_sets)
        g.replay()
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(reps):
            g.replay()
        e.record()
        torch.cuda.synchronize()
        return s.elapsed_time(e) / (reps * n_sets)
    except Exception as ex:  # noqa: BLE001 - report and fall back to eager timing
        log(f"[bench] graph capture failed ({ex}); eager timing")
        return None


def _call_ms(fn, n_sets, iters):
    ms = _graphed(fn, n_sets, iters)
    return ms if ms is not None else _rotated(fn, n_sets, iters)


def _row(nbytes, call_ms, kernel_us):
    """Row record: whole-call time (all kernels of the call, replayed from a
    HIP graph, no per-kernel events) and the main kernel's event-bracketed
    time, each as HBM GB/s."""
    call_us = 1e3 * call_ms
    out = {"call_us": round(call_us, 2), "kernel_us": round(kernel_us, 2),
           "algorithmic_bytes": nbytes,
           "GB_s_call": round(nbytes / (call_us * 1e-6) / 1e9, 1),
           "GB_s_kernel": round(nbytes / (kernel_us * 1e-6) / 1e9, 1)}
    out["frac_hbm_call"] = round(out["GB_s_call"] / PEAK_HBM_GBS, 4)
    out["frac_hbm_kernel"] = round(out["GB_s_kernel"] / PEAK_HBM_GBS, 4)
    return out


def _kernel_us(ops, name, fn, n_sets, iters):
    """Average event-bracketed duration of library kernel `name` over iters
    calls of fn (a separate pass from the call timing, through the timing
    build of the library)."""
    with ops.timing_build():
        _rotated(fn, n_sets, 2)
        ops.profile_begin(64 * iters, kernels=(name,))
        _rotated(fn, n_sets, iters)
        ops.profile_end()
    c, t = ops.profile_query(name)
    return 1e3 * t / c if c else float("nan")


def measure_rows(ops, synth, torch, dev):
    """Per-row measurements (quantise, dequantise, GEMV, merge): call time of
    back-to-back calls on inputs rotated through more than the last-level
    cache, and the main kernel's event-bracketed time from a separate pass."""
    import numpy as np
    out = {}
    # quantise / dequantise: 12 distinct 4096x4096 weights (403 MB bf16)
    nset = 12
    Ws = [synth.normal_bf16_device((D, K), 0.02, 9000 + i, device=dev) for i in range(nset)]
    qs = [ops.NF4Weight.empty(D, K, True, dev) for _ in range(nset)]
    wsq = torch.empty(ops.workspace_bytes(ops.OP_QUANTIZE, D, K, 0, 0, True) + 256,
                      dtype=torch.uint8, device=dev)
    off = (-wsq.data_ptr()) % 256
    wsq = wsq[off:off + ops.workspace_bytes(ops.OP_QUANTIZE, D, K, 0, 0, True)]
    n = D * K
    fq = lambda i: ops.quantize(Ws[i], True, out=qs[i], ws=wsq)
    ms_q = _call_ms(fq, nset, 48)
    qbytes = 2 * n + ops.storage_bytes(D, K, True)
    out["quantize"] = {"shape": [D, K], "double_quant": True,
                       **_row(qbytes, ms_q, _kernel_us(ops, "quantize", fq, nset, 48)),
                       "double_quant_kernel_us": round(_kernel_us(ops, "double_quant", fq, nset, 48), 2)}
    outs = [torch.empty(D, K, dtype=torch.bfloat16, device=dev) for _ in range(nset)]
    fd = lambda i: ops.dequantize(qs[i], out=outs[i])
    ms_d = _call_ms(fd, nset, 48)
    dbytes = ops.storage_bytes(D, K, True) + 2 * n
    out["dequantize"] = {"shape": [D, K], **_row(dbytes, ms_d, _kernel_us(ops, "dequantize", fd, nset, 48))}
    # merge (r = 16)
    Ad = synth.normal_bf16_device((R, K), 0.01, 31, device=dev)
    Bd = synth.normal_bf16_device((D, R), 0.01, 32, device=dev)
    fm = lambda i: ops.merge(qs[i], Ad, Bd, ALPHA, out=outs[i])
    ms_m = _call_ms(fm, nset, 48)
    mbytes = ops.storage_bytes(D, K, True) + 2 * n + 2 * R * (D + K)
    out["merge"] = {"shape": [D, K], "r": R, **_row(mbytes, ms_m, _kernel_us(ops, "merge", fm, nset, 48))}
    del Ws, outs, qs
    torch.cuda.empty_cache()
    # decode-shaped GEMV: gate/up 4096 -> 11008 and down 11008 -> 4096, 16
    # distinct weights each (372 MB of NF4 per shape); the call also runs the
    # LoRA down projection and the split/LoRA epilogue
    out["gemv"] = {}
    for (d, k) in ((11008, 4096), (4096, 11008)):
        nset = 16
        gq = []
        for i in range(nset):
            Wt = synth.normal_bf16_device((d, k), 0.02, 9100 + i, device=dev)
            gq.append(ops.quantize(Wt, True))
            del Wt
        Ag = synth.normal_bf16_device((R, k), 0.01, 41, device=dev)
        Bg = synth.normal_bf16_device((d, R), 0.01, 42, device=dev)
        for Mt in (1, 4, 16):
            Xg = synth.normal_bf16_device((Mt, k), 1.0, 43, device=dev)
            Yg = torch.empty(Mt, d, dtype=torch.bfloat16, device=dev)
            wsn = ops.workspace_bytes(ops.OP_FWD, d, k, Mt, R, True)
            wst = torch.empty(wsn + 256, dtype=torch.uint8, device=dev)
            o2 = (-wst.data_ptr()) % 256
            wst = wst[o2:o2 + wsn]
            fg = lambda i: ops.linear_fwd(gq[i], Xg, Ag, Bg, ALPHA, save_h=False, Y=Yg, ws=wst)
            ms_call = _call_ms(fg, nset, 96)
            gbytes = (ops.storage_bytes(d, k, True) + 2 * R * (d + k) + 2 * Mt * k + 2 * Mt * d)
            out["gemv"][f"{d}x{k}_M{Mt}"] = _row(gbytes, ms_call, _kernel_us(ops, "gemv", fg, nset, 96))
            if d == 11008:
                # sibling projections: gate and up (both 4096 -> 11008) read the
                # same X in one call (8 distinct pairs)
                Y2 = [torch.empty(Mt, d, dtype=torch.bfloat16, device=dev) for _ in range(2)]
                wsm = ops.workspace_bytes(ops.OP_FWD_MULTI, 2 * d, k, Mt, R, True)
                wsmt = torch.empty(wsm + 256, dtype=torch.uint8, device=dev)
                o3 = (-wsmt.data_ptr()) % 256
                wsmt = wsmt[o3:o3 + wsm]
                fp = lambda i: ops.linear_fwd_multi([gq[2 * i], gq[2 * i + 1]], Xg, [Ag, Ag],
                                                    [Bg, Bg], ALPHA, save_h=False, Ys=Y2, ws=wsmt)
                ms_pair = _call_ms(fp, nset // 2, 48)
                pbytes = 2 * gbytes - 2 * Mt * k   # X read once
                out["gemv"][f"gate_up_2x{d}x{k}_M{Mt}"] = _row(
                    pbytes, ms_pair, _kernel_us(ops, "gemv", fp, nset // 2, 48))
        del gq
        torch.cuda.empty_cache()
    # sibling projections on the GEMM path: q, k, v (3 x 4096x4096) of one
    # block reading the same 2048 tokens, one multi call against three calls
    Xq = synth.normal_bf16_device((M, K), 1.0, 61, device=dev)
    wq = [ops.quantize(synth.normal_bf16_device((D, K), 0.02, 62 + i, device=dev), True)
          for i in range(3)]
    Aq = [synth.normal_bf16_device((R, K), 0.01, 65 + i, device=dev) for i in range(3)]
    Bq = [synth.normal_bf16_device((D, R), 0.01, 68 + i, device=dev) for i in range(3)]
    Yq = [torch.empty(M, D, dtype=torch.bfloat16, device=dev) for _ in range(3)]
    wsq3 = torch.empty(ops.workspace_bytes(ops.OP_FWD_MULTI, 3 * D, K, M, R, True) + 256,
                       dtype=torch.uint8, device=dev)
    wsq3 = wsq3[(-wsq3.data_ptr()) % 256:]
    fq3 = lambda i: ops.linear_fwd_multi(wq, Xq, Aq, Bq, ALPHA, save_h=False, Ys=Yq, ws=wsq3)
    f3 = lambda i: [ops.linear_fwd(wq[j], Xq, Aq[j], Bq[j], ALPHA, save_h=False, Y=Yq[j])
                    for j in range(3)]
    # alternate the two forms so neither gets a clock or cache state of its own
    tm, t3 = [], []
    for _ in range(5):
        t3.append(_call_ms(f3, 1, 20))
        tm.append(_call_ms(fq3, 1, 20))
    ms_multi, ms_three = float(np.median(tm)), float(np.median(t3))
    qflops = 3 * (2 * M * D * K + 4 * M * R * D)
    out["qkv_fwd_multi"] = {"shape": [3, D, K], "tokens": M, "r": R,
                            "multi_call_us": round(1e3 * ms_multi, 2),
                            "three_calls_us": round(1e3 * ms_three, 2),
                            "multi_TFLOP_s": round(qflops / (ms_multi * 1e-3) / 1e12, 1)}
    del wq, Xq, Yq
    torch.cuda.empty_cache()
    # paged 32-bit AdamW step over the LoRA parameters of a Llama-7B-shaped
    # all-linear adapter set (32 layers x q,k,v,o 4096^2, gate/up 4096->11008,
    # down 11008->4096; r = 16: 39,976,960 parameters) as one flat buffer,
    # state in device memory; then a 4M-parameter slice of it with the state
    # paged out to page-locked host memory (updated over the host link)
    npar = 32 * (4 * 2 * R * 4096 + 3 * R * (4096 + 11008))
    st = [torch.zeros(npar, dtype=torch.float32, device=dev) for _ in range(3)]
    ga = synth.normal_bf16_device((npar,), 0.01, 51, device=dev)
    oa = torch.empty(npar, dtype=torch.bfloat16, device=dev)
    fa = lambda i: ops.adamw_step(st[0], st[1], st[2], ga, oa, 1)
    abytes = 28 * npar
    out["adamw"] = {"params": npar, "state": "device",
                    **_row(abytes, _call_ms(fa, 1, 20), _kernel_us(ops, "adamw", fa, 1, 20))}
    nh = 4 * 1024 * 1024
    sth = [torch.zeros(nh, dtype=torch.float32).pin_memory() for _ in range(3)]
    fh = lambda i: ops.adamw_step(sth[0], sth[1], sth[2], ga[:nh], oa[:nh], 1)
    hbytes = 28 * nh
    out["adamw_paged_out"] = {"params": nh, "state": "page-locked host",
                              **_row(hbytes, _rotated(fh, 1, 10), _kernel_us(ops, "adamw", fh, 1, 10))}
    del st, sth, ga, oa
    torch.cuda.empty_cache()
    # LoftQ initialisation of one 4096x4096 weight, r = 16, four power
    # iterations per SVD: one alternation and five; the products with the
    # float32 residual (read 4dk bytes per launch) dominate
    Wl = synth.normal_bf16_device((D, K), 0.02, 71, device=dev)
    oml = torch.from_numpy(synth.normal_f32((K, R), 72)).to(dev)
    wsl = torch.empty(ops.workspace_bytes(ops.OP_LOFTQ, D, K, 0, R, True) + 256,
                      dtype=torch.uint8, device=dev)
    wsl = wsl[(-wsl.data_ptr()) % 256:]
    f1 = lambda i: ops.loftq_init(Wl, oml, ALPHA, 1, 4, True, ws=wsl)
    f5 = lambda i: ops.loftq_init(Wl, oml, ALPHA, 5, 4, True, ws=wsl)
    ms1, ms5 = _rotated(f1, 1, 5), _rotated(f5, 1, 2)
    prod_us = _kernel_us(ops, "loftq_product", f1, 1, 2)
    rbytes = 4 * D * K
    out["loftq_init"] = {"shape": [D, K], "r": R, "power_iters": 4,
                         "ms_1_alternation": round(ms1, 3), "ms_5_alternations": round(ms5, 3),
                         "product_kernel_us": round(prod_us, 2),
                         "product_GB_s": round(rbytes / (prod_us * 1e-6) / 1e9, 1),
                         "product_frac_hbm": round(rbytes / (prod_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                         "residual_kernel_us": round(_kernel_us(ops, "residual", f1, 1, 2), 2),
                         "small_kernels_us": round(_kernel_us(ops, "loftq_small", f1, 1, 2), 2)}
    del Wl, wsl
    torch.cuda.empty_cache()
    log(f"[bench] rows: {json.dumps(out)}")
    return out


def _aligned(torch, dev, nbytes):
    if nbytes == 0:
        return None
    t = torch.empty(nbytes + 256, dtype=torch.uint8, device=dev)
    return t[(-t.data_ptr()) % 256:][:nbytes]


class LayerRun:
    """The seven linears of one decoder layer at M tokens: forward with the
    sibling projections grouped (q/k/v on the attention input, gate/up on the
    MLP input), then the backward of each linear. Activations (one X per
    sibling group, one dY per linear) are synthetic and shared by all layers;
    A and B are drawn per layer; H of every linear of every layer is kept from
    the forward for the backward."""

    def __init__(self, ops, torch, dev, shapes, M, r, alpha, layers):
        from bit_nf4_quantized_19_amd import synth, workloads
        self.ops, self.shapes, self.M, self.r, self.alpha = ops, shapes, M, r, alpha
        names = [n for n, _, _ in shapes]
        self.groups = [[names.index(n) for n in g] for g in workloads.SIBLINGS]
        self.X = {}
        for gi, g in enumerate(self.groups):
            k = shapes[g[0]][2]
            self.X[gi] = synth.normal_bf16_device((M, k), 1.0, synth.SEED_X + gi, device=dev)
        self.dY = [synth.normal_bf16_device((M, d), 1.0, synth.SEED_DY + i, device=dev)
                   for i, (_, d, _) in enumerate(shapes)]
        self.A = [[synth.normal_bf16_device((r, k), 0.01, synth.SEED_A + 16 * L + i, device=dev)
                   for i, (_, _, k) in enumerate(shapes)] for L in range(layers)]
        self.B = [[synth.normal_bf16_device((d, r), 0.01, synth.SEED_B + 16 * L + i, device=dev)
                   for i, (_, d, _) in enumerate(shapes)] for L in range(layers)]
        self.H = [[torch.empty(M, r, dtype=torch.float32, device=dev) for _ in shapes]
                  for _ in range(layers)]
        self.Y = [torch.empty(M, d, dtype=torch.bfloat16, device=dev) for _, d, _ in shapes]
        self.dX = [torch.empty(M, k, dtype=torch.bfloat16, device=dev) for _, _, k in shapes]
        self.dA = [torch.empty(r, k, dtype=torch.bfloat16, device=dev) for _, _, k in shapes]
        self.dB = [torch.empty(d, r, dtype=torch.bfloat16, device=dev) for _, d, _ in shapes]
        fw = max(ops.workspace_bytes(ops.OP_FWD_MULTI, sum(shapes[i][1] for i in g),
                                     shapes[g[0]][2], M, r, True) for g in self.groups)
        bw = max(ops.workspace_bytes(ops.OP_BWD, d, k, M, r, True) for _, d, k in shapes)
        self.wsf, self.wsb = _aligned(torch, dev, fw), _aligned(torch, dev, bw)

    def forward(self, L, weights):
        ops = self.ops
        for gi, g in enumerate(self.groups):
            ops.linear_fwd_multi([weights[i] for i in g], self.X[gi], [self.A[L][i] for i in g],
                                 [self.B[L][i] for i in g], self.alpha, save_h=True,
                                 Ys=[self.Y[i] for i in g], Hs=[self.H[L][i] for i in g],
                                 ws=self.wsf)

    def backward(self, L, weights):
        ops = self.ops
        for gi, g in enumerate(self.groups):
            for i in g:
                ops.linear_bwd(weights[i], self.X[gi], self.A[L][i], self.B[L][i], self.alpha,
                               self.dY[i], H=self.H[L][i], dX=self.dX[i], dA=self.dA[i],
                               dB=self.dB[i], ws=self.wsb)


def _oracle_linear_seconds(d, k, M, r, alpha, rows=None):
    """One oracle step of a d x k linear at M tokens (dequantise + float64
    forward and backward), on the first `rows` output rows if given; the
    quantised record is prepared untimed. Returns (seconds, flops timed)."""
    import numpy as np
    from bit_nf4_quantized_19_amd import synth
    from oracle import lora as olora
    from oracle import nf4 as onf4
    dd = d if rows is None else rows
    inp = synth.linear_inputs(dd, k, M, r, idx=90)
    qw = onf4.quantize_weight(inp["W0"], True)
    s = olora.lora_scale(alpha, r)
    widen = lambda b: onf4.bf16_bits_to_f32(b).astype(np.float64)
    X, A, B, dY = (widen(inp[n]) for n in ("X", "A", "B", "dY"))
    t0 = time.perf_counter()
    Wd = widen(onf4.dequantize_weight(qw)).reshape(dd, k)
    olora.forward(Wd, X, A, B, s)
    olora.backward(Wd, X, A, B, s, dY)
    return time.perf_counter() - t0, 4 * M * dd * k + 6 * M * r * (dd + k)


def measure_block7b(ops, torch, dev, with_cpu):
    """The seven linears of a Llama-7B-shaped block (q,k,v,o 4096^2; gate, up
    4096 -> 11008; down 11008 -> 4096), NF4 + double quant, r = 16,
    alpha = 32, 2048 tokens: forward (q/k/v and gate/up as sibling calls) and
    backward of all seven per block step."""
    from bit_nf4_quantized_19_amd import workloads
    shapes, M, r, alpha = workloads.LLAMA7B, 2048, 16, 32.0
    layer = [ops.quantize(_w0(torch, dev, d, k, workloads.w0_seed(0, i)), True)
             for i, (_, d, k) in enumerate(shapes)]
    run = LayerRun(ops, torch, dev, shapes, M, r, alpha, 1)

    def block():
        run.forward(0, layer)
        run.backward(0, layer)
    for _ in range(10):
        block()
    torch.cuda.synchronize()
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s0.record()
    for _ in range(20):
        block()
    s1.record()
    torch.cuda.synchronize()
    ms = s0.elapsed_time(s1) / 20
    fl = workloads.layer_flops(shapes, M, r)
    out = {"workload": "llama7b_block_7_linears_nf4_dq_tokens2048_r16_fwd_bwd",
           "gflop_per_block": round(fl / 1e9, 1), "ms_per_block": round(ms, 4),
           "TFLOP_s": round(fl / (ms * 1e-3) / 1e12, 1),
           "frac_bf16_peak": round(fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
           "nf4_dq_bytes": sum(ops.storage_bytes(d, k, True) for _, d, k in shapes)}
    if with_cpu:
        # oracle: one linear per distinct shape, summed with multiplicity
        cores = _oracle_cores()
        tot = 0.0
        with _oracle_threads(cores):
            for (d, k), mult in (((4096, 4096), 4), ((11008, 4096), 2), ((4096, 11008), 1)):
                sec, _ = _oracle_linear_seconds(d, k, M, r, alpha)
                tot += mult * sec
        out["cpu_oracle"] = {"seconds_per_block": round(tot, 2),
                             "TFLOP_s": round(fl / tot / 1e12, 4), "cores": cores,
                             "sample": "one linear per distinct shape (4096^2, 11008x4096, "
                                       "4096x11008), dequantise + float64 fwd + bwd at 2048 "
                                       "tokens, summed with multiplicity 4, 2, 1"}
    del layer, run
    torch.cuda.empty_cache()
    log(f"[bench] llama7b block: {json.dumps(out)}")
    return out


def _w0(torch, dev, d, k, seed):
    from bit_nf4_quantized_19_amd import synth
    return synth.normal_bf16_device((d, k), 0.02, seed, device=dev)


def measure_stack65b(ops, torch, dev, with_cpu):
    """The 65B-shaped stack: 80 layers of q,k,v,o 8192^2, gate, up 8192 ->
    22016, down 22016 -> 8192. Every base weight is drawn on the device,
    quantised (NF4 + double quant) and its bf16 copy freed, so the whole NF4
    stack is resident at once; then one training pass over all 80 layers at
    2048 tokens, r = 64, alpha = 16 (forward of every layer, then backward in
    reverse layer order), and the quantiser's rate at the two weight shapes."""
    from bit_nf4_quantized_19_amd import workloads
    shapes, M, r, alpha, nl = workloads.L65B, 2048, 64, 16.0, workloads.L65B_LAYERS
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    stack = workloads.build_quantized_stack(ops, shapes, nl, dev, True)
    torch.cuda.synchronize()
    build_s = time.perf_counter() - t0
    resident = stack.resident_bytes()
    params = nl * sum(d * k for _, d, k in shapes)
    run = LayerRun(ops, torch, dev, shapes, M, r, alpha, nl)

    def train_pass(layers):
        for L in range(layers):
            run.forward(L, stack.weights[L])
        for L in reversed(range(layers)):
            run.backward(L, stack.weights[L])
    train_pass(2)
    torch.cuda.synchronize()
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s0.record()
    train_pass(nl)
    s1.record()
    torch.cuda.synchronize()
    ms = s0.elapsed_time(s1)
    fl = nl * workloads.layer_flops(shapes, M, r)
    out = {"workload": "stack65b_80_layers_nf4_dq_tokens2048_r64_fwd_bwd",
           "layers": nl, "params": params, "resident_nf4_dq_bytes": resident,
           "resident_GB": round(resident / 1e9, 3),
           "bits_per_param": round(8 * resident / params, 5),
           "draw_and_quantize_all_s": round(build_s, 3),
           "tflop_per_pass": round(fl / 1e12, 2), "ms_per_pass": round(ms, 2),
           "TFLOP_s": round(fl / (ms * 1e-3) / 1e12, 1),
           "frac_bf16_peak": round(fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
    del run
    torch.cuda.empty_cache()
    # the quantiser alone at the two weight shapes, 12 distinct weights each
    out["quantize"] = {}
    for (d, k) in ((8192, 8192), (22016, 8192)):
        Ws = [_w0(torch, dev, d, k, 9500 + i) for i in range(12)]
        qs = [ops.NF4Weight.empty(d, k, True, dev) for _ in range(12)]
        wsq = _aligned(torch, dev, ops.workspace_bytes(ops.OP_QUANTIZE, d, k, 0, 0, True))
        fq = lambda i: ops.quantize(Ws[i], True, out=qs[i], ws=wsq)
        qbytes = 2 * d * k + ops.storage_bytes(d, k, True)
        out["quantize"][f"{d}x{k}"] = _row(qbytes, _call_ms(fq, 12, 48),
                                           _kernel_us(ops, "quantize", fq, 12, 48))
        del Ws, qs
        torch.cuda.empty_cache()
    if with_cpu:
        # oracle: one linear per distinct shape on its first 2048 output rows
        # (a bounded sample), its rate applied to the whole stack's flops
        cores = _oracle_cores()
        sec = fls = 0.0
        with _oracle_threads(cores):
            for (d, k), mult in (((8192, 8192), 4), ((22016, 8192), 2), ((8192, 22016), 1)):
                t, f = _oracle_linear_seconds(d, k, M, r, alpha, rows=2048)
                sec += mult * t
                fls += mult * f
        rate = fls / sec
        out["cpu_oracle"] = {"TFLOP_s": round(rate / 1e12, 4), "cores": cores,
                             "seconds_per_pass_extrapolated": round(fl / rate, 1),
                             "sample": "one linear per distinct shape (8192^2, 22016x8192, "
                                       "8192x22016) on its first 2048 output rows, dequantise "
                                       "+ float64 fwd + bwd at 2048 tokens, weighted 4, 2, 1; "
                                       "the rate is extrapolated to 80 layers"}
    del stack
    torch.cuda.empty_cache()
    log(f"[bench] 65B stack: {json.dumps(out)}")
    return out


def measure_probes(torch, dev):
    """Measured ceilings beside the published peaks: a device-to-device copy
    streaming 2 GiB (and one of the 32 MiB a 4096x4096 bf16 weight occupies,
    the size of the quantise / dequantise rows), and a large bf16 GEMM
    (8192^3, the vendor library) for the matrix cores."""
    def copy_rate(nbytes, iters):
        src = torch.empty(nbytes // 2, dtype=torch.bfloat16, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        srcs = [src] if nbytes > (1 << 30) else \
            [torch.empty_like(src).fill_(1.0) for _ in range(16)]   # past the 256 MB cache
        dsts = [dst] if nbytes > (1 << 30) else [torch.empty_like(src) for _ in range(16)]
        for i in range(3):
            dsts[i % len(dsts)].copy_(srcs[i % len(srcs)])
        torch.cuda.synchronize()
        s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s0.record()
        for i in range(iters):
            dsts[i % len(dsts)].copy_(srcs[i % len(srcs)])
        s1.record()
        torch.cuda.synchronize()
        us = 1e3 * s0.elapsed_time(s1) / iters
        return round(2 * nbytes / (us * 1e-6) / 1e9, 1)
    out = {"hbm_copy_2GiB_GB_s": copy_rate(2 << 30, 10),
           "hbm_copy_32MiB_GB_s": copy_rate(32 << 20, 64)}
    a = torch.randn(8192, 8192, device=dev, dtype=torch.bfloat16)
    b = torch.randn(8192, 8192, device=dev, dtype=torch.bfloat16)
    for _ in range(3):
        torch.matmul(a, b)
    torch.cuda.synchronize()
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s0.record()
    for _ in range(10):
        torch.matmul(a, b)
    s1.record()
    torch.cuda.synchronize()
    ms = s0.elapsed_time(s1) / 10
    out["bf16_gemm_8192_TFLOP_s"] = round(2 * 8192 ** 3 / (ms * 1e-3) / 1e12, 1)
    del a, b
    # the same layer step with a 16-bit base (plain bf16 W, vendor matmuls,
    # 2-D products with contiguous right operands): the pages put QLoRA's
    # training slowdown against 16-bit LoRA at 15-30%
    g = torch.Generator(device=dev)
    g.manual_seed(81)
    rn = lambda *sh: torch.randn(*sh, generator=g, device=dev, dtype=torch.float32)
    Wb = (rn(D, K) * 0.02).bfloat16()
    WbT = Wb.t().contiguous()
    Xb, dYb = rn(M, K).bfloat16(), rn(M, D).bfloat16()
    Ab, Bb = (rn(R, K) * 0.01).bfloat16(), (rn(D, R) * 0.01).bfloat16()
    AbT, BbT = Ab.t().contiguous(), Bb.t().contiguous()
    sc = ALPHA / R

    def lora16_step():
        Hb = Xb @ AbT
        Yb = torch.addmm(Xb @ WbT, Hb, BbT, alpha=sc)
        Gb = dYb @ Bb
        dXb = torch.addmm(dYb @ Wb, Gb, Ab, alpha=sc)
        dAb = (Gb.t() @ Xb) * sc
        dBb = (dYb.t() @ Hb) * sc
        return Yb, dXb, dAb, dBb
    for _ in range(20):
        lora16_step()
    torch.cuda.synchronize()
    s0.record()
    for _ in range(100):
        lora16_step()
    s1.record()
    torch.cuda.synchronize()
    out["bf16_lora_step_ms"] = round(s0.elapsed_time(s1) / 100, 4)
    del Wb, WbT, Xb, dYb
    torch.cuda.empty_cache()
    torch.cuda.empty_cache()
    log(f"[bench] probes: {json.dumps(out)}")
    return out


def _oracle_cores():
    """Threads for the oracle: the CPUs this process may run on, capped at the
    share a launcher grants through OMP_NUM_THREADS."""
    affinity = len(os.sched_getaffinity(0))
    share = int(os.environ.get("OMP_NUM_THREADS", "0") or 0)
    return min(affinity, share) if share > 0 else affinity


def _oracle_threads(n):
    """Context in which the oracle's BLAS/OpenMP pools use n threads."""
    from threadpoolctl import threadpool_limits
    return threadpool_limits(limits=n)


def _cpu_model():
    """The host CPU's model name as lscpu reports it."""
    import subprocess
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
    except (OSError, subprocess.SubprocessError):
        return None
    for ln in out.splitlines():
        if ln.strip().startswith("Model name:"):
            return ln.split(":", 1)[1].strip()
    return None


def cpu_baseline(inp, flops):
    """The CPU oracle (as it stands) on the host cores: one full step of the
    workload (oracle dequantisation of W0 plus float64 forward and backward on
    all 2048 tokens), median of 3 runs; the quantised record is prepared once,
    untimed."""
    import numpy as np
    from oracle import lora as olora
    from oracle import nf4 as onf4
    affinity = len(os.sched_getaffinity(0))
    cores = _oracle_cores()
    log(f"[bench] cpu oracle baseline on {cores} threads ({affinity} CPUs in the affinity set)")
    qw = onf4.quantize_weight(inp["W0"], True)
    s = olora.lora_scale(ALPHA, R)
    widen = lambda b: onf4.bf16_bits_to_f32(b).astype(np.float64)
    X, A, B, dY = (widen(inp[n]) for n in ("X", "A", "B", "dY"))
    times = []
    with _oracle_threads(cores):
        for _ in range(3):
            t0 = time.perf_counter()
            Wd = widen(onf4.dequantize_weight(qw)).reshape(D, K)
            Yo, Ho = olora.forward(Wd, X, A, B, s)
            olora.backward(Wd, X, A, B, s, dY)
            times.append(time.perf_counter() - t0)
    t = statistics.median(times)
    model = _cpu_model()
    return {"value": round(flops / t / 1e12, 4), "unit": "TFLOP/s", "cores": int(cores),
            "affinity_cpus": affinity, "kind": "oracle", "cpu_model": model,
            "sample": "one full step of the workload (oracle dequantise + float64 forward "
                      f"and backward, 2048 tokens), median of 3 runs: {t:.2f} s"}


if __name__ == "__main__":
    main()
