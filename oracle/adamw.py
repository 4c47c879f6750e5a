"""32-bit AdamW step of the LoRA matrices (the paged optimiser's update).

CPU oracle -- test infrastructure only (see ``oracle/__init__.py``).

Pages followed
--------------
* Day-25 LoRA/QLoRA notes (itingyu.github.io), section 3.4 "分页优化器":
  Adam keeps two moment terms per parameter (momentum and variance) in
  float32; under GPU memory pressure that state is paged out to CPU RAM and
  paged back when needed.
* QLoRA glossary (Ultralytics), "QLoRA 的工作原理", paged-optimiser bullet:
  the optimiser state lives in unified memory and moves to CPU RAM during
  memory peaks.
* "如何利用QLoRA在消费级GPU上实现大模型的高效微调" (tbr8.org), section 3
  (training arguments) and section 4: the optimiser is ``paged_adamw_32bit``
  with learning rate 2e-4; it swaps state that is not in use to host memory.
* Same page, section 1, and the QLoRA glossary: only the LoRA matrices A and
  B are trained, so the step runs over their elements only.

The pages name the optimiser but print no update rule. Reading taken: AdamW
as published (Adam's bias-corrected first and second moments, Kingma & Ba;
weight decay decoupled from the gradient, Loshchilov & Hutter), with the
parameters kept as a float32 master copy and the bf16 copy that the forward
and backward read produced from it each step. Per element, every operation
in float32, rounded once, in this order (t = step number, from 1)::

    g   = float32(grad_bf16)
    m'  = fl(fl(b1 * m) + fl(c1 * g))            c1 = fl32(1 - beta1)
    v'  = fl(fl(b2 * v) + fl(c2 * fl(g * g)))    c2 = fl32(1 - beta2)
    mh  = fl(m' / bc1)                           bc1 = fl32(1 - beta1**t)
    vh  = fl(v' / bc2)                           bc2 = fl32(1 - beta2**t)
    u   = fl(mh / fl(fl(sqrt(vh)) + eps))
    p'  = fl(p - fl(lr * fl(u + fl(wd * p))))
    out = bf16_rne(p')

with b1 = fl32(beta1), b2 = fl32(beta2), and 1 - beta1, 1 - beta2,
1 - beta1**t, 1 - beta2**t evaluated in float64 from the given
hyperparameters and rounded once to float32 (division and square root
correctly rounded, as IEEE float32 defines them).
"""

from __future__ import annotations

import numpy as np

from .nf4 import f32_to_bf16_bits

F32 = np.float32


def bias_corrections(beta1: float, beta2: float, step: int):
    """``(bc1, bc2) = (1 - beta1**t, 1 - beta2**t)`` in float64, rounded once
    to float32."""
    if step < 1:
        raise ValueError("step counts from 1")
    return F32(1.0 - float(beta1) ** step), F32(1.0 - float(beta2) ** step)


def adamw_step(p, m, v, g_bf16_bits, *, lr, beta1, beta2, eps, weight_decay, step):
    """One AdamW step over flat float32 arrays ``p`` (master parameters),
    ``m``, ``v`` (moments) and uint16 ``g_bf16_bits`` (the gradient as bf16
    bit patterns). Returns ``(p', m', v', out_bf16_bits)``; the inputs are
    not modified."""
    p = np.asarray(p, dtype=F32)
    m = np.asarray(m, dtype=F32)
    v = np.asarray(v, dtype=F32)
    g = (np.asarray(g_bf16_bits, dtype=np.uint16).astype(np.uint32) << 16).view(F32)
    b1, b2 = F32(beta1), F32(beta2)
    c1, c2 = F32(1.0 - float(beta1)), F32(1.0 - float(beta2))
    bc1, bc2 = bias_corrections(beta1, beta2, step)
    lr32, eps32, wd32 = F32(lr), F32(eps), F32(weight_decay)
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        m1 = (b1 * m).astype(F32) + (c1 * g).astype(F32)
        v1 = (b2 * v).astype(F32) + (c2 * (g * g).astype(F32)).astype(F32)
        m1, v1 = m1.astype(F32), v1.astype(F32)
        mh = (m1 / bc1).astype(F32)
        vh = (v1 / bc2).astype(F32)
        den = (np.sqrt(vh).astype(F32) + eps32).astype(F32)
        u = (mh / den).astype(F32)
        step_dir = (u + (wd32 * p).astype(F32)).astype(F32)
        p1 = (p - (lr32 * step_dir).astype(F32)).astype(F32)
    return p1, m1, v1, f32_to_bf16_bits(p1)
