"""CPU oracle for the MoE expert-dispatch hot path.

TEST INFRASTRUCTURE.  Only the tests, the package's smoke check and the
benchmark's CPU-baseline leg may import or run anything in this package.  The
HIP path never calls it, shares no code with it, and this package imports
nothing from the HIP path.

Each function is the plain definition of one step, written from the pages:

* ``layout.route_layout`` - the stable counting sort of routed (token, expert)
  assignments into expert-major rows with a rowmap ("poc(cco): MegaMoE stage1
  dispatch over SDMA", commit "recv_layout": the receiver counts the routes per
  expert and writes rowmap / srcmap tables; "EPDispatchKernel":
  wait_for_arrivals_and_compute_offsets computes per-local-expert offsets).
* ``quant.quant_dispatch`` - per-landed-token fp8 quantisation, each token read
  and quantised once (MegaMoE PR, commit 2 "each token read and quantised
  once").
* ``gemm1.grouped_gemm1`` - per-local-expert GEMM1 reading its A rows through
  the rowmap (MegaMoE PR, "What" and "How it works now").
* ``combine.combine`` - the top-k weighted combine back to token order
  (TilePipe "Communication Kernels": push combine; MegaMoE PR "What": stage2 +
  combine).
* ``mx.quant_dispatch`` / ``mx.grouped_gemm1`` - the same quant and GEMM1 with
  the pages' own scale format: power-of-two (e8m0) scales per group of 32 K
  elements, packed four per dword (MegaMoE PR, "Where we stand" and commit
  "ready-first / quant-lds-store").
* ``stage2.act_quant`` / ``stage2.grouped_gemm2`` / ``stage2.combine_rows`` -
  stage2 after GEMM1: silu(gate) * up, its fp8 quantisation, the grouped
  down-projection with each row's routing weight, and the combine of the
  weighted rows (MegaMoE PR, "What": stage1 feeds stage2 + combine; commit
  "recv_layout": the layout's per-row routing weights serve stage2).
* ``fp8`` / ``bf16`` - the OCP FP8 E4M3 encoding and bf16 rounding the steps
  rely on.

Parity pins (see tests/test_oracle_*.py): brute-force loops on tiny inputs,
invariants (bijection, contiguity, stability, half-ulp round trip, identity
experts), torch's independent fp8/bf16 casts, and exact special cases.
Every function here has at least one such pin; none is "parity unpinned".
"""
from . import bf16, fp8, layout, quant, gemm1, combine, mx, stage2  # noqa: F401
