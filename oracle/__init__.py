"""CPU oracle for the fused MoE-FFN expert computation (test infrastructure only).

This package is the reference that the HIP path is checked against.  It is
plain, slow numpy code in float64, written from the definition of the method
on the pages "HyperParallel Multicore HyperMegaMoE fused forward/backward
operator" (RFC, sections 2.1, 2.2, 3.1 and 4.1) and "MoE multicore parallel
usage guide" (section "inputs and weights"), plus the per-token dynamic
quantisation of "MoeDistributeDispatchV2" (function description, case 3).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import anything from here.  The product path never does: it
shares no code, header, table or helper with this package.

Modules
-------
numerics  rounding to bfloat16 and to FP8 E4M3 (round to nearest even), SiLU.
routing   top-k expand, per-expert histogram, prefix offsets, stable permutation.
moe_ffn   forward and backward as a per-token loop over the K chosen experts,
          in a PURE mode (no intermediate rounding) and a FAITHFUL mode
          (bfloat16 rounding at the stored intermediates), plus samplers that
          evaluate selected outputs of large problems one by one.
quant     per-token and per-column dynamic FP8 E4M3 quantisation.

Every function here is pinned by ``tests/test_oracle_*.py`` to something other
than itself (library routines, closed forms, brute force, finite differences,
invariants); none is "parity unpinned".
"""

from . import numerics, routing, quant, moe_ffn  # noqa: F401
