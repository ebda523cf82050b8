"""CPU oracle for the MXFP4 producers and the block-scaled E2M1 GEMM.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links
this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it.  It shares no code, tables or
constant generators with the HIP library; the only module both sides use is
``synthetic`` (seeded inputs, none of the method's arithmetic).

The oracle is plain and slow on purpose: numpy, fp64 wherever the method is an
exact definition (scale choice, rounding decision, decode, contraction), fp32
exactly where the contract fixes fp32 arithmetic (the H32 butterfly, the SwiGLU
chain).  Each function cites the passage of "Format-Aware Fusion for Fast FP4
Pretraining" (arXiv 2610.00053, HTML text and its section summary) it follows.

Modules
-------
formats   E2M1 grid, upward E8M0 exponent, RTN and adjacent-bin SR decisions,
          nibble packing, decode.
philox    Philox4x32-10 counter generator and the fixed sign mask; pinned
          against rocRAND's independent Philox4x32-10 engine (host build of
          its open-source header), since no published known-answer vectors
          are available offline, and by structure and statistics.
hadamard  Fixed-sign H32 transform (signs, Sylvester butterfly, 2^-2.5).
quant     Row-facing, column-facing (optionally H32) and 2D32 producers.
gemm      Decode-then-contract reference and the per-element error bound.
swiglu    The exp used by both sides, SwiGLU forward/backward in fp32.
nvfp4     CTA-local NVFP4: E4M3 16-value block scales with per-panel fp32
          outer factors, the 2D16 weight producer, and its contraction.
"""

from . import formats, philox, hadamard, quant, gemm, swiglu, nvfp4  # noqa: F401
