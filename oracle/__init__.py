"""CPU oracle for the MXFP4 MoE expert block -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or call anything in this package.  The product path
(the HIP library and its Python binding) never does, and this package never
imports the product: the two share nothing but the seeded input generators in
``moe_synth``.

The oracle is plain numpy in float64: slow and meant to be read against the
pages.  Sources, cited by title and section:

[P1] "Add MXFP4 training support via a dequantize-on-the-fly fallback"
     (huggingface/transformers pull request 47464): sections "What this
     does", "Why (the silent-gradient trap)", "Relation to the backward
     triton kernels" and "Tests".  The eager path -- top-k router, then a
     per-expert loop over weights dequantized on the fly -- is named there as
     the numerical reference implementation; this oracle follows it.
[P3] "Integrate finegrained kernels: SOTA performance and per-module
     quantization" (pull request 49658): the commit notes on the gate|up row
     interleave and stride-2 split, on the per-expert ``bias=`` operand and the
     routing-weighted reduce, on the row-wise MXFP4 quantizers with UE8M0
     scales, and on the bit-equal ``dequantize=True`` converter.
[OCP] OCP Microscaling Formats (MX) Specification v1.0: the E2M1 element
     and E8M0 scale encodings.  The pages name MXFP4 and UE8M0 scales but do
     not print the encodings.

Readings where the pages are silent (each marked "reading" in the code):
the E2M1 round-half-to-even rule, the nibble order, the scale rule
e = ceil(log2(amax / 6)) and its clamp, the clamped-SwiGLU form, the
router's top-k tie order, the stable permutation order, the per-expert LoRA
placement on the down projection, and that dX includes the router path.

Parity pins: every function here is checked in ``tests/test_oracle_*.py``
against something other than itself (closed forms, brute force, finite
differences, library routines, invariants).  No function is parity-unpinned.
"""
from . import mxfp4, moe  # noqa: F401
