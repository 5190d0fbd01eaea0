"""CPU oracle for the fused LoRA linear path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. The product path
(``rank_gemm_lora_amd``) never imports, calls or links it, and shares no code
with it: the two meet only through the seeded inputs of ``lora_workloads``.

Two parts:

* ``lora_oracle``: the plain definitions in float64 (numpy), i.e. what the
  method computes in exact arithmetic up to fp64 rounding:
  y = x.W^T + b + s.(x.A^T).B^T with s = (alpha/rank).strength.request_scale,
  its stacked-group and 4-bit-codebook forms, and the dense patch payloads.
* ``exact_chain``: the separate-pass chain whose rounding points define the
  exact tier, emulated element by element with explicit IEEE roundings.

Pins: every function here is checked by ``tests/test_oracle_*.py`` against
something other than itself (brute force in ``fractions.Fraction``, algebraic
identities, special cases that reduce to a library routine, rounding tables).
"""
from . import lora_oracle, exact_chain  # noqa: F401
