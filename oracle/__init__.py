"""CPU oracle for the batched lossless verify-and-resample step (fp64, numpy).

TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check in __graft_entry__.py
and the cpu_baseline leg of bench.py may import anything from this package.
The GPU library never imports, links or calls it, and the two share no code:
both implement the same written specification independently.

Modules:
  philox -- Philox4x32-10 (Salmon et al., SC'11), the stream layout, uniforms
            and Gumbel draws.
  ssd    -- decode, softmax_t, topf, sigma (Saguaro sampling), the two-level
            Gumbel-max sampler, draft sampling, verification (acceptance and
            bonus), fan-out and the speculation cache.

Parity pins: every function here is checked by tests marked "not gpu" against
facts that do not come from this package (published known-answer vectors,
library routines, closed forms, exact enumeration, brute force, chi-square
tests of the sampling distributions).  No function is "parity unpinned".
"""
from . import philox, ssd  # noqa: F401
