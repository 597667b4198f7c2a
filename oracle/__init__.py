"""Float64 CPU oracle for the WKV operator.

TEST INFRASTRUCTURE: only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package. It shares no code with the HIP
library (wkv_recurrence_scan_amd) and never imports it.

parity pins: every forward function here is pinned by tests/test_oracle.py
against the mpmath brute force, closed forms of the defining equation,
invariants and special cases that reduce to a softmax; the gradients
(wkv_grad) by tests/test_oracle_grad.py against central finite differences
of the pinned forward and by invariants of the operator; the per-token-decay
operator (wkv_decay) by tests/test_oracle_decay.py against its own mpmath
recurrence, the constant-decay operator, a hand-worked case and invariants;
the matrix-valued-state recurrence (wkv_matrix) by tests/test_oracle_matrix.py
against its own mpmath attention form, causal linear attention by matmul,
closed forms and invariants; the token shift (wkv_shift) by
tests/test_oracle_shift.py against the mixing fraction's end points and
midpoint, affinity, split/resume, one-token steps, constant sequences, a
hand-worked case and planted mistakes. None is "parity unpinned".
"""

from .wkv_decay import wkv_dd_direct, wkv_dd_recurrent, wkv_dd_step_ref  # noqa: F401
from .wkv_grad import (  # noqa: F401
    wkv_backward_direct, wkv_dd_backward_direct, wkv_gated_backward_direct)
from .wkv_matrix import wkv6_direct, wkv6_recurrent, wkv6_step_ref  # noqa: F401
from .wkv_shift import token_shift  # noqa: F401
from .wkv_oracle import (  # noqa: F401
    EMPTY_MAX_EXP,
    canonical,
    empty_state,
    normalised_error,
    wkv_combine,
    sigmoid,
    wkv_direct,
    wkv_gated,
    wkv_recurrent,
    wkv_segment_summary,
    wkv_step_ref,
)
