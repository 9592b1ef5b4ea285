"""MI355X-native Ladder Residual Transformer forward step (decode and prefill).

The computation lives in ``libladder.so`` (hand-written HIP kernels for gfx950 behind
the C ABI of ``include/ladder.h``); ``abi`` is its ctypes binding with the same
function names and ``model`` a small handle that lets torch own device memory and
streams.  There is no other execution path: without the built library, loading
raises.
"""
from .abi import (  # noqa: F401
    LADDER_BF16, LADDER_F32, LADDER_SCHED_DUAL, LADDER_SCHED_FUSED, LADDER_SCHED_FUSED_LATE_ATTN, LADDER_SCHED_PERSISTENT, LADDER_SCHED_SERIAL, LADDER_SCHED_SIDE, LadderError, load,
    ladder_decode_step, ladder_decode_step_static, ladder_filled, ladder_free, ladder_init, ladder_prefill, ladder_sample, ladder_set_sampling,
    ladder_set_schedule,
    ladder_sync, ladder_time_kernels, ladder_workspace_bytes, status_string,
)


def __getattr__(name):
    # torch-dependent helpers are imported on first use
    if name in ("LadderModel", "DeviceWeights"):
        from . import model
        return getattr(model, name)
    raise AttributeError(name)
