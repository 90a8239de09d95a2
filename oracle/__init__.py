"""CPU oracle for the long-sequence attention hot path (test infrastructure).

Plain, slow, float64 numpy definitions of what the HIP library computes:
attention with log-sum-exp, the log-sum-exp merge of partial results, and the
Ulysses seq-major to head-major relayout.  Only the test suite, the smoke check
in ``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import this
package.  It shares no code with the HIP path and never imports it.
"""

from .ref import (  # noqa: F401
    bf16_bits_to_f64,
    attention,
    attention_rows,
    merge,
    merge_two_logsigmoid,
    relayout_seq_to_head,
    relayout_head_to_seq,
)
