"""Oracle for the angle-quantised KV-cache codec (float64 NumPy reference).

TEST INFRASTRUCTURE: only the tests, the smoke check and the benchmark's CPU-baseline
leg may import this package. It shares no code with the HIP library.

Parity pins: every function here is checked by tests/test_oracle.py and
tests/test_layout.py against closed forms, brute force, published check values and a
library routine; none is "parity unpinned" except the quality figures the TurboAngle
abstract reports for trained models (not computed here at all).
"""

from . import codec, layout  # noqa: F401
