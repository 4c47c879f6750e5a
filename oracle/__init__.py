"""Plain CPU oracle for the QLoRA frozen-base NF4 linear layer.

TEST INFRASTRUCTURE ONLY. Nothing in the product path imports, calls, links or
executes anything in this package. Only the test suite, the smoke check in
``__graft_entry__.smoke`` and the ``cpu_baseline`` leg of ``bench.py`` may use
it. The oracle shares no code, table or constant generator with the HIP
library: it rebuilds every constant from the pages' definitions.

Modules
-------
``oracle.nf4``   NF4 level construction, blockwise absmax quantisation,
                 double quantisation of the absmax values, dequantisation,
                 storage sizes. Floating point is IEEE float32 where the pages
                 compute in float32 (the level search and the restore), exact
                 rational arithmetic for the mean, float64 for the levels.
``oracle.lora``  The LoRA linear: forward, backward (chain rule) and merge,
                 all in float64 on bf16-exact inputs, rounded once to bf16.
``oracle.adamw`` The 32-bit AdamW step of the LoRA matrices (the paged
                 optimiser's update), elementwise float32 in a stated order.
``oracle.dropout`` LoRA dropout on the adapter input: Philox4x32-10 keep
                 mask and the float64 forward/backward with the mask.
``oracle.loftq`` LoftQ initialisation: randomized rank-r SVD (float64,
                 numpy QR/SVD as steps), LoRA factors, the float32 residual
                 W - s B A rounded to bf16, and the alternation with NF4.

Every function cites the page passage it follows. A page is cited by its
title and section, e.g. "QLoRA glossary (Ultralytics), 'QLoRA 的工作原理'".

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
against values the pages print, closed forms, invariants or brute force,
except the 8-bit format of the double-quantised absmax (symmetric int8 with
one float32 scale per 256 blocks and one global mean), which the pages do not
define; that format is the plainest reading of "8-bit" and its code
format is "parity unpinned" beyond the invariants tested (error bound,
equal-value special case, exact mean).
"""
