"""fp64 CPU oracle (test infrastructure only; see oracle/oracle.py)."""
from .oracle import (  # noqa: F401
    HEAD_MAJOR, TOKEN_MAJOR, attention, attention_probs_head, bf16_to_f64,
    fm_euler_state, fm_euler_step, fm_euler_unit, kv_append, streaming_keys, visible)
