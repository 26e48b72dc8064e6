"""CPU oracle for the rotated K4/V3 quantized KV cache (TEST INFRASTRUCTURE ONLY).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or run anything in this package.  The product path
(``rotated_bit_quantized_amd``) never imports it, and this package imports
nothing from the product path: the two share no code.  The only module both
sides use is ``workloads`` (seeded random inputs, no method arithmetic).

Modules:
  ``rbq_oracle`` - vectorised numpy oracle (rotation, quantizer, packer,
                   cache bookkeeping, attention), fp64 wherever the method
                   works in floating point, except where the quantizer's
                   decisions are defined in fp32.
  ``brute``      - pure-Python loop twin of the quantizer, the packer and the
                   attention, for tiny inputs only.

Every function in ``rbq_oracle`` is pinned by ``tests/test_oracle_pins.py``
against closed forms, special cases, invariants, brute force or independent
library routines; none is "parity unpinned".
"""
