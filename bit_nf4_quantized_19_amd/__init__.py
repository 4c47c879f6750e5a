"""QLoRA frozen-base NF4 linear layer on MI355X (gfx950).

The compute path is the HIP library ``libqlora_nf4.so`` built from ``csrc/``
and reached through the C ABI declared in ``include/qlora_nf4.h``; the Python
binding in ``ops.py`` only marshals torch device tensors and streams into that
ABI. Importing this package loads nothing; ``ops`` loads the library on first
use and raises if it is missing.
"""

__all__ = ["ops", "synth"]
