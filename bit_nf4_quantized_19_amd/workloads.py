"""Workload shapes and device-resident builders for the block- and
stack-level runs (the seven linears of a Llama-7B-shaped block and the
80-layer 65B-shaped stack).

Shapes: the adapters target every linear of a decoder layer -- q, k, v, o of
attention and gate, up, down of the MLP (LLM-train tutorial ch. 3, 3.3,
``target_modules``; QLoRA glossary, "QLoRA 的工作原理": adapters on every
linear layer). Llama-7B: hidden 4096, intermediate 11008 (Day-25 notes 2.1:
d = k = 4096 for the attention projections). 65B-shaped stack: hidden 8192,
intermediate 22016, 80 layers (the pages give only "65B"; the glossary's
"权衡" section puts its 4-bit weights plus double-quantised scales at about
34 GB, which this shape reproduces: 33.41 GB).

Nothing here computes any part of the method: weights are drawn by
``synth`` and quantised through the C ABI (``ops.quantize``).
"""

from __future__ import annotations

from dataclasses import dataclass

from . import synth

#: (name, d = out_features, k = in_features) of the seven linears of a layer
LLAMA7B = (("q", 4096, 4096), ("k", 4096, 4096), ("v", 4096, 4096), ("o", 4096, 4096),
           ("gate", 11008, 4096), ("up", 11008, 4096), ("down", 4096, 11008))
L65B = (("q", 8192, 8192), ("k", 8192, 8192), ("v", 8192, 8192), ("o", 8192, 8192),
        ("gate", 22016, 8192), ("up", 22016, 8192), ("down", 8192, 22016))
L65B_LAYERS = 80

#: linears that read the same activations in one forward call (sibling
#: projections): q/k/v read the attention input, gate/up the MLP input
SIBLINGS = (("q", "k", "v"), ("o",), ("gate", "up"), ("down",))


def flops_fwd_bwd(M: int, d: int, k: int, r: int) -> int:
    """Algorithmic flops of one linear's forward + backward: 4Mdk + 6Mr(d+k)
    (two base products and six rank-r products of M tokens)."""
    return 4 * M * d * k + 6 * M * r * (d + k)


def layer_flops(shapes, M: int, r: int) -> int:
    return sum(flops_fwd_bwd(M, d, k, r) for _, d, k in shapes)


def w0_seed(layer: int, linear: int) -> int:
    """Seed of the base weight of linear `linear` of layer `layer`."""
    return synth.SEED_W0 + 16 * layer + linear


@dataclass
class QuantStack:
    """Quantised base weights of a stack: weights[layer][linear]."""
    weights: list
    shapes: tuple

    def resident_bytes(self) -> int:
        """Bytes of the NF4 records (codes, int8 absmax codes, scales, mean)
        as allocated on the device."""
        tot = 0
        for layer in self.weights:
            for w in layer:
                for t in (w.codes, w.absmax, w.absmax_q, w.absmax_scale, w.absmax_offset):
                    if t is not None:
                        tot += t.numel() * t.element_size()
        return tot


def build_quantized_stack(ops, shapes, layers: int, device, double_quant: bool = True,
                          std: float = 0.02, progress=None) -> QuantStack:
    """Draw each layer's base weights on the device (seeded per layer and
    linear), quantise them, and free the bf16 weight before the next one: at
    most one bf16 weight is resident at a time."""
    import torch
    big = max(shapes, key=lambda s: s[1] * s[2])
    nws = ops.workspace_bytes(ops.OP_QUANTIZE, big[1], big[2], 0, 0, double_quant)
    ws = None
    if nws:
        raw = torch.empty(nws + 256, dtype=torch.uint8, device=device)
        ws = raw[(-raw.data_ptr()) % 256:][:nws]
    out = []
    for L in range(layers):
        layer = []
        for i, (_, d, k) in enumerate(shapes):
            W = synth.normal_bf16_device((d, k), std, w0_seed(L, i), device=device)
            layer.append(ops.quantize(W, double_quant, ws=ws))
            del W
        out.append(layer)
        if progress is not None:
            progress(L)
    return QuantStack(out, tuple(shapes))
