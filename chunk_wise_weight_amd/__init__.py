"""MI355X (gfx950) chunk-wise fast-weight update of In-Place Test-Time Training.

The computation lives in libttt.so (hand-written HIP kernels behind a C ABI,
declared in include/ttt.h); this package only binds it.
"""
from .binding import (  # noqa: F401
    EXPORTS,
    LIB_PATH,
    PHASES,
    Handle,
    TTTError,
    lib,
    ttt_destroy,
    ttt_forward_chunked,
    ttt_forward_chunked_noalloc,
    ttt_forward_docs,
    ttt_init,
    ttt_last_error,
    ttt_phase_times,
    ttt_plan,
    ttt_reset,
    ttt_set_clip,
    ttt_set_target_conv,
    ttt_set_group_chunks,
    ttt_set_output_f32,
    ttt_set_profiling,
    ttt_state_delta,
    ttt_workspace_bytes,
)
