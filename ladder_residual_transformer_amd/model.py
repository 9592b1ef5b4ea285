"""Device-side model handle: torch owns the memory, libladder does the computing."""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence

import numpy as np
import torch

from . import abi

LAYER_FIELDS = ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate", "w_up", "w_down")


def _to_device(a: np.ndarray, device) -> torch.Tensor:
    """Host array -> device tensor with identical bytes (bf16 bit patterns stay bit patterns)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    if a.dtype == np.float32:
        return torch.from_numpy(a).to(device)
    raise TypeError(f"unsupported weight dtype {a.dtype}")


class DeviceWeights:
    """Weights of one model on one GPU.  ``host`` has attributes tok_embed, final_norm,
    lm_head and layers[i].<LAYER_FIELDS> holding numpy arrays (bf16 as uint16 bits)."""

    def __init__(self, host, device="cuda"):
        self.dtype = "bf16" if host.tok_embed.dtype == np.uint16 else "f32"
        self.tok_embed = _to_device(host.tok_embed, device)
        self.final_norm = _to_device(host.final_norm, device)
        self.lm_head = _to_device(host.lm_head, device)
        self.layers = []
        for lw in host.layers:
            self.layers.append({f: _to_device(getattr(lw, f), device) for f in LAYER_FIELDS})

    def nbytes(self) -> int:
        t = self.tok_embed.nbytes + self.final_norm.nbytes + self.lm_head.nbytes
        return t + sum(x.nbytes for l in self.layers for x in l.values())


class LadderModel:
    """A libladder context over ``DeviceWeights``.

    ``cfg`` needs n_layers, hidden, n_q_heads, n_kv_heads, head_dim, ffn, vocab,
    rope_theta, norm_eps, dtype ("f32"/"bf16") and ladder_mask (and may carry rope_scaling,
    (factor, low_freq_factor, high_freq_factor, original context)).  The KV cache
    [n_layers][max_batch][n_kv][max_seq][head_dim] is allocated here unless given.
    """

    def __init__(self, cfg, weights: DeviceWeights, max_batch: int, max_seq: int, *,
                 kv: Optional[Sequence[torch.Tensor]] = None, kv_filled: int = 0, max_prefill_tokens: int = 0,
                 ladder_mask: Optional[Sequence[int]] = None, device="cuda"):
        self.cfg = cfg
        self.w = weights
        self.device = torch.device(device)
        self.max_batch, self.max_seq = max_batch, max_seq
        tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
        shape = (cfg.n_layers, max_batch, cfg.n_kv_heads, max_seq, cfg.head_dim)
        if kv is None:
            kv = (torch.zeros(shape, dtype=tdt, device=self.device), torch.zeros(shape, dtype=tdt, device=self.device))
        self.k_cache, self.v_cache = kv
        mask = list(cfg.ladder_mask if ladder_mask is None else ladder_mask)
        self._mask = (ctypes.c_uint8 * len(mask))(*[int(m) for m in mask])
        c = abi.ladder_config()
        c.n_layers, c.hidden, c.n_q_heads, c.n_kv_heads = cfg.n_layers, cfg.hidden, cfg.n_q_heads, cfg.n_kv_heads
        c.head_dim, c.ffn, c.vocab = cfg.head_dim, cfg.ffn, cfg.vocab
        c.rope_theta, c.norm_eps = float(cfg.rope_theta), float(cfg.norm_eps)
        c.dtype = abi.LADDER_BF16 if cfg.dtype == "bf16" else abi.LADDER_F32
        c.max_batch, c.max_seq, c.max_prefill_tokens, c.kv_filled = max_batch, max_seq, max_prefill_tokens, kv_filled
        c.ladder_mask = ctypes.cast(self._mask, ctypes.POINTER(ctypes.c_uint8))
        scaling = getattr(cfg, "rope_scaling", None)
        if scaling is not None:
            (c.rope_scale_factor, c.rope_low_freq_factor, c.rope_high_freq_factor,
             c.rope_orig_max_pos) = float(scaling[0]), float(scaling[1]), float(scaling[2]), int(scaling[3])
        self._cfg = c
        self._layers = (abi.ladder_layer_weights * cfg.n_layers)()
        for i, lw in enumerate(weights.layers):
            for f in LAYER_FIELDS:
                setattr(self._layers[i], f, lw[f].data_ptr())
        self._w = abi.ladder_weights(weights.tok_embed.data_ptr(), weights.final_norm.data_ptr(),
                                     weights.lm_head.data_ptr(), self._layers)
        self._kv = abi.ladder_kv(self.k_cache.data_ptr(), self.v_cache.data_ptr())
        self.stream = torch.cuda.current_stream(self.device)
        self.ctx = abi.ladder_init(self._cfg, self._w, self._kv, self.stream.cuda_stream)

    # -- calls -------------------------------------------------------------
    def set_schedule(self, schedule: int, use_graph: bool = True):
        abi.ladder_set_schedule(self.ctx, schedule, use_graph)

    def set_sampling(self, temperature: float, top_k: int = 0, seed: int = 0):
        """temperature <= 0: greedy next tokens; else a seeded draw (see ladder_set_sampling)."""
        abi.ladder_set_sampling(self.ctx, temperature, top_k, seed)

    def _outs(self, B, logits, hidden):
        lg = torch.empty((B, self.cfg.vocab), dtype=torch.float32, device=self.device) if logits else None
        nx = torch.empty((B,), dtype=torch.int32, device=self.device)
        hd = torch.empty((B, self.cfg.hidden), dtype=torch.float32, device=self.device) if hidden else None
        return lg, nx, hd

    @staticmethod
    def _ptr(t):
        return t.data_ptr() if t is not None else 0

    def prefill(self, ids: torch.Tensor, start_pos: int = 0, logits: bool = True, hidden: bool = True):
        """ids: int32 [B, T] on the device.  Returns (logits, next, hidden) of the last position."""
        assert ids.dtype == torch.int32 and ids.is_contiguous() and ids.dim() == 2
        B, T = ids.shape
        lg, nx, hd = self._outs(B, logits, hidden)
        abi.ladder_prefill(self.ctx, ids.data_ptr(), B, T, start_pos, self._ptr(lg), nx.data_ptr(), self._ptr(hd))
        return lg, nx, hd

    def decode_step(self, ids: torch.Tensor, pos: int, logits: bool = True, hidden: bool = True, out=None):
        """ids: int32 [B] on the device (may be the previous step's ``next``)."""
        assert ids.dtype == torch.int32 and ids.is_contiguous() and ids.dim() == 1
        B = ids.shape[0]
        lg, nx, hd = out if out is not None else self._outs(B, logits, hidden)
        abi.ladder_decode_step(self.ctx, ids.data_ptr(), B, pos, self._ptr(lg), self._ptr(nx), self._ptr(hd))
        return lg, nx, hd

    def decode_step_static(self, ids: torch.Tensor, pos: int, out):
        """decode_step through ladder_decode_step_static: out = (logits, next, hidden)
        tensors allocated beforehand (entries may be None), since the call allocates
        nothing."""
        assert ids.dtype == torch.int32 and ids.is_contiguous() and ids.dim() == 1
        lg, nx, hd = out
        abi.ladder_decode_step_static(self.ctx, ids.data_ptr(), ids.shape[0], pos, self._ptr(lg), self._ptr(nx),
                                      self._ptr(hd))
        return lg, nx, hd

    def time_kernels(self, B: int, reps: int = 3) -> dict:
        return abi.ladder_time_kernels(self.ctx, B, reps)

    def trace_kernel(self, kind) -> None:
        """Time every decode launch of one kernel kind (a name of abi.KERNEL_KINDS, or None)."""
        abi.ladder_trace_kernel(self.ctx, -1 if kind is None else abi.KERNEL_KINDS.index(kind))

    def trace_result(self):
        return abi.ladder_trace_result(self.ctx)

    def filled(self) -> int:
        return abi.ladder_filled(self.ctx)

    def sync(self) -> None:
        """Wait for the context's work; raises if a kernel's bounded wait gave up."""
        abi.ladder_sync(self.ctx)

    def workspace_bytes(self) -> int:
        return abi.ladder_workspace_bytes(self.ctx)

    def free(self):
        if getattr(self, "ctx", None):
            abi.ladder_free(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass
