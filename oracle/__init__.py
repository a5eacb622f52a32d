"""CPU oracle for the GIFT FP8 gradient round trip -- TEST INFRASTRUCTURE ONLY.

Plain, slow, fp64 numpy restatement of what the method computes, written
from the pages and from the published definitions the pages point to.  It
exists to check the HIP path, never to serve it: only the test-suite, the
package smoke check and the CPU-baseline leg of the benchmark may import it.
The HIP library neither imports nor links anything here, and nothing here
imports the HIP library or its Python binding.

Sources, cited by title and section throughout:

* "GIFT review" -- the pith.science review page of arXiv 2607.07494,
  "GIFT: Geometry-Informed Low-precision Gradient Communication for LLM
  Pretraining" (Wang, Fan, Zheng, Zhang).  Sections used: "The pith",
  "Core claim", "What carries the argument", "Load-bearing premise",
  "What would settle it", the referee report (major comment 2, on the
  paper's Algorithm 1), the axiom and free-parameter ledger, and the
  abstract.
* "FP8 formats" -- reference [28] of that page, Micikevicius et al.,
  "FP8 Formats for Deep Learning" (arXiv 2209.05433): the E4M3 encoding.
* Philox4x32-10 -- Salmon, Moraes, Dror and Shaw, "Parallel random numbers:
  as easy as 1, 2, 3" (SC'11); Box-Muller -- Box and Muller (1958).

Modules:

* ``e4m3``    -- the 256-code E4M3 table, RNE encode with saturation, decode.
* ``philox``  -- Philox4x32-10 and the Box-Muller sketch.
* ``gift``    -- covariance, damping, subspace iteration, Rayleigh-Ritz,
                 whitening coefficients, whiten / quantize / dequantize /
                 un-whiten, the Euclidean baseline, 1x128 block scaling and the
                 error metrics.

Parity pins: every function here is pinned by a CPU test against a closed
form, an invariant, an independent library routine or brute force
(tests/test_oracle_*.py).  The one exception is the pages' own aggregate
number (about 67% lower round-trip error on their Llama-600M gradients):
their gradients are not available, so that figure is parity unpinned.
"""

from . import e4m3, philox, gift  # noqa: F401
