"""CPU oracle (test infrastructure only; see ttt_oracle's header)."""
from .ttt_oracle import (  # noqa: F401
    chunk_ranges,
    clip_update,
    conv_targets,
    final_state_columns,
    gated_activation,
    ntp_targets,
    silu,
    ttt_forward,
    ttt_forward_docs,
    ttt_forward_one,
    window_outputs,
)
