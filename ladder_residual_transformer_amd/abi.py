"""ctypes binding of libladder (include/ladder.h): argument marshalling only.

Every step of the forward pass runs in the HIP kernels of libladder.so; this module
only builds the C structs, passes device pointers and streams through, and turns
status codes into exceptions.  PyTorch provides device memory and streams.
The library must have been built (``ladder_residual_transformer_amd.build``);
importing the product without it raises instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_double, c_float, c_int32, c_size_t, c_uint8, c_void_p

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libladder.so")

LADDER_OK = 0
LADDER_STATIC_SCRATCH_BYTES = 64 << 20   # device bytes of the library's static scratch, per GPU
LADDER_ERR_ARG = -1
LADDER_ERR_SHAPE = -2
LADDER_ERR_CAPACITY = -3
LADDER_ERR_STATE = -4
LADDER_ERR_HIP = -5
LADDER_ERR_OOM = -6

LADDER_F32 = 0
LADDER_BF16 = 1

LADDER_SCHED_SERIAL = 0
LADDER_SCHED_SIDE = 1
LADDER_SCHED_DUAL = 2
LADDER_SCHED_FUSED = 3
LADDER_SCHED_PERSISTENT = 4
LADDER_SCHED_FUSED_LATE_ATTN = 5

EXPORTED = ("ladder_init", "ladder_prefill", "ladder_decode_step", "ladder_decode_step_static", "ladder_set_schedule", "ladder_set_sampling",
            "ladder_filled",
            "ladder_workspace_bytes", "ladder_sync", "ladder_free", "ladder_status_string", "ladder_last_error",
            "ladder_time_kernels", "ladder_trace_kernel", "ladder_trace_result", "ladder_read_probe", "ladder_sample")

LADDER_KERNEL_LAYER_STACK = 9
LADDER_KERNEL_QKV_ATTN_GATEUP = 10
LADDER_KERNEL_DOWN_OPROJ = 11
LADDER_KERNEL_SAMPLE = 12
LADDER_N_KERNELS = 13
KERNEL_KINDS = ("qkv", "attn", "oproj", "gateup", "down", "lmhead", "qkv_gateup", "attn_down", "oproj_add2", "layer_stack",
                "qkv_attn_gateup", "down_oproj", "sample")


class ladder_config(ctypes.Structure):
    _fields_ = [("n_layers", c_int32), ("hidden", c_int32), ("n_q_heads", c_int32), ("n_kv_heads", c_int32),
                ("head_dim", c_int32), ("ffn", c_int32), ("vocab", c_int32), ("rope_theta", c_double),
                ("norm_eps", c_float), ("dtype", c_int32), ("max_batch", c_int32), ("max_seq", c_int32),
                ("max_prefill_tokens", c_int32), ("kv_filled", c_int32), ("ladder_mask", POINTER(c_uint8)),
                ("rope_scale_factor", c_double), ("rope_low_freq_factor", c_double),
                ("rope_high_freq_factor", c_double), ("rope_orig_max_pos", c_int32)]


class ladder_layer_weights(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate", "w_up",
                                        "w_down")]


class ladder_weights(ctypes.Structure):
    _fields_ = [("tok_embed", c_void_p), ("final_norm", c_void_p), ("lm_head", c_void_p),
                ("layers", POINTER(ladder_layer_weights))]


class ladder_kv(ctypes.Structure):
    _fields_ = [("k", c_void_p), ("v", c_void_p)]


class LadderError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str = ""):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({status}){': ' + detail if detail else ''}")


_lib = None


def load(path: str = LIB_PATH):
    """Load libladder.so (after torch, so both share torch's HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    import torch  # noqa: F401  -- loads libamdhip64 first; libladder links the same soname
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with ladder_residual_transformer_amd.build.build()")
    lib = ctypes.CDLL(path)
    lib.ladder_init.argtypes = [POINTER(ladder_config), POINTER(ladder_weights), POINTER(ladder_kv), c_void_p,
                                POINTER(c_void_p)]
    lib.ladder_prefill.argtypes = [c_void_p, c_void_p, c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p]
    lib.ladder_decode_step.argtypes = [c_void_p, c_void_p, c_int32, c_int32, c_void_p, c_void_p, c_void_p]
    lib.ladder_decode_step_static.argtypes = [c_void_p, c_void_p, c_int32, c_int32, c_void_p, c_void_p, c_void_p]
    lib.ladder_set_schedule.argtypes = [c_void_p, c_int32, c_int32]
    lib.ladder_set_sampling.argtypes = [c_void_p, c_float, c_int32, ctypes.c_uint64]
    lib.ladder_sample.argtypes = [c_void_p, c_int32, c_int32, c_int32, c_float, c_int32, ctypes.c_uint64, c_int32,
                                  c_void_p, c_void_p]
    lib.ladder_filled.argtypes = [c_void_p, POINTER(c_int32)]
    lib.ladder_workspace_bytes.argtypes = [c_void_p, POINTER(c_size_t)]
    lib.ladder_sync.argtypes = [c_void_p]
    lib.ladder_time_kernels.argtypes = [c_void_p, c_int32, c_int32, POINTER(c_float)]
    lib.ladder_trace_kernel.argtypes = [c_void_p, c_int32]
    lib.ladder_trace_result.argtypes = [c_void_p, POINTER(c_float), POINTER(c_int32)]
    lib.ladder_free.argtypes = [c_void_p]
    lib.ladder_read_probe.argtypes = [c_void_p, c_size_t, c_int32, POINTER(c_float)]
    lib.ladder_free.restype = None
    lib.ladder_status_string.argtypes = [c_int32]
    lib.ladder_status_string.restype = ctypes.c_char_p
    lib.ladder_last_error.argtypes = [c_void_p]
    lib.ladder_last_error.restype = ctypes.c_char_p
    for name in ("ladder_init", "ladder_prefill", "ladder_decode_step", "ladder_decode_step_static", "ladder_set_schedule", "ladder_set_sampling",
                 "ladder_filled",
                 "ladder_workspace_bytes", "ladder_sync", "ladder_time_kernels", "ladder_trace_kernel",
                 "ladder_trace_result", "ladder_read_probe", "ladder_sample"):
        getattr(lib, name).restype = c_int32
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().ladder_status_string(int(status)).decode()


# --- same-named wrappers (raw pointers as Python ints) -----------------------

def ladder_init(cfg: ladder_config, weights: ladder_weights, kv: ladder_kv, stream: int = 0) -> int:
    out = c_void_p()
    st = load().ladder_init(ctypes.byref(cfg), ctypes.byref(weights), ctypes.byref(kv), c_void_p(stream or None),
                            ctypes.byref(out))
    if st != LADDER_OK:
        raise LadderError(st, "ladder_init")
    return out.value


def _check(ctx: int, st: int, where: str):
    if st != LADDER_OK:
        raise LadderError(st, where, load().ladder_last_error(c_void_p(ctx)).decode())


def ladder_prefill(ctx: int, d_ids: int, B: int, T: int, start_pos: int, d_logits: int = 0, d_next: int = 0,
                   d_hidden: int = 0) -> None:
    _check(ctx, load().ladder_prefill(c_void_p(ctx), c_void_p(d_ids), B, T, start_pos, c_void_p(d_logits or None),
                                      c_void_p(d_next or None), c_void_p(d_hidden or None)), "ladder_prefill")


def ladder_decode_step(ctx: int, d_ids: int, B: int, pos: int, d_logits: int = 0, d_next: int = 0,
                       d_hidden: int = 0) -> None:
    _check(ctx, load().ladder_decode_step(c_void_p(ctx), c_void_p(d_ids), B, pos, c_void_p(d_logits or None),
                                          c_void_p(d_next or None), c_void_p(d_hidden or None)),
           "ladder_decode_step")


def ladder_decode_step_static(ctx: int, d_ids: int, B: int, pos: int, d_logits: int = 0, d_next: int = 0,
                              d_hidden: int = 0) -> None:
    _check(ctx, load().ladder_decode_step_static(c_void_p(ctx), c_void_p(d_ids), B, pos, c_void_p(d_logits or None),
                                                 c_void_p(d_next or None), c_void_p(d_hidden or None)),
           "ladder_decode_step_static")


def ladder_set_schedule(ctx: int, schedule: int, use_graph: bool = True) -> None:
    _check(ctx, load().ladder_set_schedule(c_void_p(ctx), schedule, 1 if use_graph else 0), "ladder_set_schedule")


def ladder_set_sampling(ctx: int, temperature: float, top_k: int = 0, seed: int = 0) -> None:
    _check(ctx, load().ladder_set_sampling(c_void_p(ctx), temperature, top_k, seed), "ladder_set_sampling")


def ladder_sample(d_logits: int, B: int, V: int, ld: int, temperature: float, top_k: int, seed: int, pos: int,
                  d_next: int, stream: int = 0) -> None:
    _check(0, load().ladder_sample(c_void_p(d_logits), B, V, ld, temperature, top_k, seed, pos, c_void_p(d_next),
                                   c_void_p(stream or None)), "ladder_sample")


def ladder_filled(ctx: int) -> int:
    v = c_int32()
    _check(ctx, load().ladder_filled(c_void_p(ctx), ctypes.byref(v)), "ladder_filled")
    return v.value


def ladder_workspace_bytes(ctx: int) -> int:
    v = c_size_t()
    _check(ctx, load().ladder_workspace_bytes(c_void_p(ctx), ctypes.byref(v)), "ladder_workspace_bytes")
    return v.value


def ladder_sync(ctx: int) -> None:
    _check(ctx, load().ladder_sync(c_void_p(ctx)), "ladder_sync")


def ladder_time_kernels(ctx: int, B: int, reps: int = 3) -> dict:
    """Mean launch duration (microseconds) of each decode kernel kind at batch B."""
    out = (c_float * len(KERNEL_KINDS))()
    _check(ctx, load().ladder_time_kernels(c_void_p(ctx), B, reps, out), "ladder_time_kernels")
    return {k: float(v) for k, v in zip(KERNEL_KINDS, out)}


def ladder_trace_kernel(ctx: int, kind: int) -> None:
    """Bracket every decode launch of kernel kind ``kind`` (-1: none) with HIP events."""
    _check(ctx, load().ladder_trace_kernel(c_void_p(ctx), kind), "ladder_trace_kernel")


def ladder_trace_result(ctx: int):
    """(mean microseconds, launches) of the traced kind in the most recent decode step."""
    us, n = c_float(), c_int32()
    _check(ctx, load().ladder_trace_result(c_void_p(ctx), ctypes.byref(us), ctypes.byref(n)), "ladder_trace_result")
    return float(us.value), int(n.value)


def ladder_read_probe(stream: int, nbytes: int, reps: int) -> float:
    """Streaming-read ceiling of the current device in GB/s (allocates nbytes of device memory)."""
    g = c_float()
    _check(0, load().ladder_read_probe(c_void_p(stream or None), nbytes, reps, ctypes.byref(g)), "ladder_read_probe")
    return float(g.value)


def ladder_free(ctx: int) -> None:
    load().ladder_free(c_void_p(ctx or None))
