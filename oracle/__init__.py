"""Oracles for the angle-quantised KV-cache codec and the triplet (octahedral) codec
(float64 NumPy references).

TEST INFRASTRUCTURE: only the tests, the smoke check and the benchmark's CPU-baseline
leg may import this package. It shares no code with the HIP library.

Parity pins: every function here is checked by tests/test_oracle.py,
tests/test_layout.py and tests/test_oracle_triplet.py against closed forms, brute force,
published values and library routines; none is "parity unpinned" except the quality
figures the pages report for trained models (not computed here at all).
"""

from . import codec, layout, triplet  # noqa: F401
