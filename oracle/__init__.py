"""Float64 CPU oracle for the WKV operator.

TEST INFRASTRUCTURE: only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package. It shares no code with the HIP
library (wkv_recurrence_scan_amd) and never imports it.

parity pins: every function here is pinned by tests/test_oracle.py against the
mpmath brute force, closed forms of the defining equation, invariants and
special cases that reduce to a softmax; none is "parity unpinned".
"""

from .wkv_oracle import (  # noqa: F401
    EMPTY_MAX_EXP,
    canonical,
    empty_state,
    normalised_error,
    wkv_combine,
    wkv_direct,
    wkv_recurrent,
    wkv_segment_summary,
    wkv_step_ref,
)
