"""CPU oracle for the MXFP4-weight / MXFP8-activation sparse MoE layer.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: only the test suite, the smoke check and the CPU-baseline
leg of the benchmark use it.  It shares no code with the HIP library (no
kernels, tables, constants or helpers); the only thing both sides consume is the
seeded input generator, which holds none of the layer's arithmetic.

What it computes is the plain definition of the layer, step by step, in numpy
float64, with every MX element and scale decoded exactly:

* ``mx``  -- the E2M1 / E4M3 / E8M0 encodings and the MX block quantiser.
* ``moe`` -- router (logits, top-k, sigmoid renormalisation), token permutation,
  expert SwiGLU MLPs with MXFP8 re-quantisation, weighted combine.

Sources: the Kimi K3 pages describe the layer only structurally
("Kimi K3 Tech Intro", section 4.3 "MXFP4 MoE + SiTU": router with top-16,
routed experts plus shared expert; section 1 architecture table: 16 of 896
experts, MXFP4 weights; "Kimi K3 ... MoE推理系统工程分析": MXFP4 weights with
MXFP8 activations).  The bit formats follow the public OCP Microscaling (MX)
v1.0 definitions.  Every point the pages leave open is a stated reading,
listed in the design notes of the repository.

Parity status: every function here is pinned by tests that do not re-type its
formula (exhaustive decode tables cross-checked against torch's float8 dtypes,
brute-force nearest-code search, brute-force top-k subset search, a library
stable sort, and a dense all-experts computation); none is "parity unpinned".
"""

from . import mx, moe  # noqa: F401

__all__ = ["mx", "moe"]
