"""fp64 CPU oracle for exact attention.

TEST INFRASTRUCTURE ONLY: imported by tests/, by __graft_entry__.smoke() and by
bench.py's CPU-baseline leg.  The library never imports it, and it imports
nothing from the library.

Functions and the passages they follow are documented in oracle/attention.py
(attention), oracle/dropout.py (dropout on the attention probabilities, with
its counter-based generator) and oracle/decode.py (few queries against a long
key/value cache).
Every function here is pinned by tests/test_oracle_pins.py,
tests/test_oracle_dropout_pins.py and tests/test_oracle_decode_pins.py against closed
forms, brute force, finite differences and an independent library
implementation; none is "parity unpinned".
"""
from .attention import (  # noqa: F401
    MASK_BLOCK,
    allowed,
    attention_bwd,
    attention_dkdv_rows,
    attention_dq_rows,
    attention_fwd,
    attention_fwd_rows,
)
from .dropout import (  # noqa: F401
    attention_bwd_dropout,
    attention_fwd_dropout,
    drop_threshold,
    keep_mask,
    philox4x32_10,
)
from .decode import attention_fwd_decode  # noqa: F401
