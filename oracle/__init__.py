"""CPU fp64 oracle for Newton-Schulz orthogonalisation (test infrastructure).

This package is test infrastructure only. Only the test suite, the smoke check
in ``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import
it. The GPU library never calls into it, and it shares no code, tables or
helpers with the GPU library.

Sources followed (DMuon documentation, "Newton-Schulz 变体" page, and the
"Core Concepts" page):

* ``ns_oracle``   -- the method itself in fp64: precision pipeline step 1
  (normalisation), the direct iteration, the Gram-space iteration with
  restarts, and the singular-value closed form used to pin both.
* ``fp16_model``  -- a labelled diagnostic: the same method with every stored
  matrix rounded to fp16 and products accumulated in fp32, used to estimate
  the rounding floor of an fp16 implementation. It is not a parity oracle.
"""

from .ns_oracle import (  # noqa: F401
    POLAR_EXPRESS_COEFFICIENTS,
    YOU_COEFFICIENTS,
    COEFFICIENT_SETS,
    normalize,
    direct_newton_schulz,
    gram_newton_schulz,
    gram_newton_schulz_sharded,
    shard_bounds,
    muon_step,
    closed_form,
    scalar_map,
    step_maps,
)
