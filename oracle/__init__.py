"""CPU fp64 oracle of the Range-Doppler focusing chain -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline leg may import
this package.  The HIP library (``range_doppler_focusing_amd``) never imports it, and the two
share no code: only the seeded scene generator (``rdscene``) feeds both.

Parity pinning: every function here is pinned by ``tests/test_oracle_pins.py`` to closed
forms, brute-force definitions on tiny inputs, textbook point-response values and invariants;
the exact image values of a full noisy scene have no printed worked example in the pages and
are pinned only through those special cases.
"""
from . import metrics, rd_oracle  # noqa: F401
