"""Seeded synthetic workloads for the Ladder Residual Transformer forward step.

This module only describes model shapes and draws random numbers: it holds
none of the model's arithmetic. Both sides of every comparison (the CPU
oracle and the GPU library) consume the exact arrays produced here, so a
difference between them can never come from the inputs.

Recipe (the same for every workload):
  * every weight matrix is drawn from N(0, 0.02) in float32 and stored either
    as float32 (``dtype == "f32"``) or rounded to bfloat16 with
    round-to-nearest-even and stored as its 16-bit pattern (``"bf16"``);
  * norm gains are exactly 1 (N(0, 0.02) applies to matrices only);
  * token ids are uniform over ``[0, vocab)``;
  * each tensor has its own seed ``(seed, tensor_index, chunk_index)`` so the
    result does not depend on how many threads generate it.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import List, Optional, Sequence

import numpy as np

__all__ = [
    "ModelConfig", "Workload", "CONFIGS", "LLAMA31_ROPE_SCALING", "WORKLOADS", "LayerWeights", "ModelWeights",
    "gen_weights", "gen_ids", "f32_to_bf16_bits", "scaled_config",
]

INIT_STD = 0.02
_CHUNK = 1 << 22          # elements per independently seeded chunk
_BF16_ONE = np.uint16(0x3F80)


@dataclasses.dataclass(frozen=True)
class ModelConfig:
    """Shape of one model (or one tensor-parallel rank's shard of it)."""
    name: str
    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    rope_theta: float
    dtype: str                      # "f32" or "bf16": weights and KV cache
    ladder_mask: tuple              # one entry per layer: 0 = standard, 1 = ladder, 2 = parallel
    norm_eps: float = 1e-5
    # rotary frequency scaling (factor, low_freq_factor, high_freq_factor, original context
    # length) of Llama-3.1 checkpoints, or None
    rope_scaling: Optional[tuple] = None

    def __post_init__(self):
        if len(self.ladder_mask) != self.n_layers:
            raise ValueError("ladder_mask needs one entry per layer")
        if any(int(m) not in (0, 1, 2) for m in self.ladder_mask):
            raise ValueError("ladder_mask entries are 0, 1 or 2")
        if self.dtype not in ("f32", "bf16"):
            raise ValueError("dtype must be 'f32' or 'bf16'")

    @property
    def n_modules(self) -> int:
        return 2 * self.n_layers

    def with_mask(self, mask: Sequence[int], name: Optional[str] = None) -> "ModelConfig":
        return dataclasses.replace(self, ladder_mask=tuple(int(m) for m in mask),
                                   name=name or self.name)

    def weight_bytes(self) -> int:
        """Bytes of every weight tensor as stored, the whole token-embedding table included."""
        e = 4 if self.dtype == "f32" else 2
        H, F, hd = self.hidden, self.ffn, self.head_dim
        per_layer = (H * (self.n_q_heads + 2 * self.n_kv_heads) * hd
                     + self.n_q_heads * hd * H + 3 * H * F + 2 * H)
        return e * (self.n_layers * per_layer + 2 * self.vocab * H + H)

    def decode_weight_bytes(self, batch: int) -> int:
        """Weight bytes one decode step of `batch` sequences reads: every layer's matrices
        and norm gains, the final norm and the LM head once, and one embedding row per
        sequence (not the whole table)."""
        e = 4 if self.dtype == "f32" else 2
        return self.weight_bytes() - e * (self.vocab - batch) * self.hidden


@dataclasses.dataclass(frozen=True)
class Workload:
    """A model plus the batch sizes and lengths it is exercised with."""
    name: str
    model: ModelConfig
    batches: tuple
    prompt_len: int
    decode_len: int

    @property
    def max_seq(self) -> int:
        return self.prompt_len + self.decode_len


def _all_ladder(n):
    return tuple([1] * n)


# Llama-3.1's published rotary scaling constants (its checkpoints' "llama3" rope_scaling).
LLAMA31_ROPE_SCALING = (8.0, 1.0, 4.0, 8192)

# The five workloads.  The 70B and 405B rows are one tensor-parallel rank's
# shard: per-rank heads and ffn slice, vocabulary split over the ranks
# (128256 / 8 = 16032 and 128256 / 16 = 8016 rows of embedding and LM head).
CONFIGS = {
    "tiny": ModelConfig("tiny", 2, 256, 4, 2, 64, 688, 1024, 1e4, "f32", _all_ladder(2)),
    "1b": ModelConfig("1b", 16, 2048, 32, 8, 64, 8192, 32000, 1e4, "bf16", _all_ladder(16)),
    "8b_hybrid": ModelConfig("8b_hybrid", 32, 4096, 32, 8, 128, 14336, 128256, 5e5, "bf16",
                             tuple([0] * 16 + [1] * 16), rope_scaling=LLAMA31_ROPE_SCALING),
    # the hybrid with 20 converted layers: the upper 20 of 32 layers ladder
    "8b_hybrid20": ModelConfig("8b_hybrid20", 32, 4096, 32, 8, 128, 14336, 128256, 5e5, "bf16",
                               tuple([0] * 12 + [1] * 20), rope_scaling=LLAMA31_ROPE_SCALING),
    "70b_tp8_shard": ModelConfig("70b_tp8_shard", 80, 8192, 8, 1, 128, 3584, 16032, 5e5,
                                 "bf16", _all_ladder(80), rope_scaling=LLAMA31_ROPE_SCALING),
    "405b_tp16_shard": ModelConfig("405b_tp16_shard", 126, 16384, 8, 1, 128, 3328, 8016, 5e5,
                                   "bf16", _all_ladder(126), rope_scaling=LLAMA31_ROPE_SCALING),
}

WORKLOADS = {
    "tiny": Workload("tiny", CONFIGS["tiny"], (1,), 16, 16),
    "1b": Workload("1b", CONFIGS["1b"], (1, 8), 512, 128),
    "8b_hybrid": Workload("8b_hybrid", CONFIGS["8b_hybrid"], (1, 16), 1024, 256),
    "70b_tp8_shard": Workload("70b_tp8_shard", CONFIGS["70b_tp8_shard"], (1, 4, 16), 1024, 512),
    "405b_tp16_shard": Workload("405b_tp16_shard", CONFIGS["405b_tp16_shard"], (1, 16, 64),
                                2048, 256),
}


def scaled_config(base: ModelConfig, n_layers: int, name: Optional[str] = None) -> ModelConfig:
    """The same widths with fewer layers (mask truncated / extended with its last entry)."""
    mask = list(base.ladder_mask[:n_layers])
    while len(mask) < n_layers:
        mask.append(base.ladder_mask[-1])
    return dataclasses.replace(base, n_layers=n_layers, ladder_mask=tuple(mask),
                               name=name or f"{base.name}_{n_layers}L")


@dataclasses.dataclass
class LayerWeights:
    attn_norm: np.ndarray   # [H]
    wq: np.ndarray          # [nq*hd, H]   (row-major [out][in])
    wk: np.ndarray          # [nkv*hd, H]
    wv: np.ndarray          # [nkv*hd, H]
    wo: np.ndarray          # [H, nq*hd]
    mlp_norm: np.ndarray    # [H]
    w_gate: np.ndarray      # [F, H]
    w_up: np.ndarray        # [F, H]
    w_down: np.ndarray      # [H, F]

    FIELDS = ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate", "w_up", "w_down")


@dataclasses.dataclass
class ModelWeights:
    """Stored weights. bf16 tensors are uint16 bit patterns, f32 tensors float32."""
    dtype: str
    tok_embed: np.ndarray   # [V, H]
    final_norm: np.ndarray  # [H]
    lm_head: np.ndarray     # [V, H]
    layers: List[LayerWeights]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round-to-nearest-even) and return the 16-bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def _fill_normal(out: np.ndarray, seed: int, tensor_index: int, dtype: str, lo: int, hi: int):
    flat = out.reshape(-1)
    chunk = lo // _CHUNK
    rng = np.random.Generator(np.random.PCG64DXSM(np.random.SeedSequence([seed, tensor_index, chunk])))
    z = rng.standard_normal(hi - lo, dtype=np.float32)
    z *= np.float32(INIT_STD)
    flat[lo:hi] = f32_to_bf16_bits(z) if dtype == "bf16" else z


def _shapes(cfg: ModelConfig):
    H, F = cfg.hidden, cfg.ffn
    q, kv = cfg.n_q_heads * cfg.head_dim, cfg.n_kv_heads * cfg.head_dim
    layer = {"attn_norm": (H,), "wq": (q, H), "wk": (kv, H), "wv": (kv, H), "wo": (H, q),
             "mlp_norm": (H,), "w_gate": (F, H), "w_up": (F, H), "w_down": (H, F)}
    return layer


def gen_weights(cfg: ModelConfig, seed: int = 0, threads: Optional[int] = None,
                layers: Optional[Sequence[int]] = None) -> ModelWeights:
    """Draw the weights of ``cfg``.

    ``layers`` restricts generation to a subset of layer indices (the others
    are left as ``None``); the values of a generated layer do not depend on
    which other layers were generated.
    """
    st = np.uint16 if cfg.dtype == "bf16" else np.float32
    one = _BF16_ONE if cfg.dtype == "bf16" else np.float32(1.0)
    H, V = cfg.hidden, cfg.vocab
    jobs = []

    def matrix(shape, tensor_index):
        a = np.empty(shape, dtype=st)
        n = a.size
        for lo in range(0, n, _CHUNK):
            jobs.append((a, tensor_index, lo, min(n, lo + _CHUNK)))
        return a

    def gain():
        return np.full((H,), one, dtype=st)

    tok_embed = matrix((V, H), 0)
    shapes = _shapes(cfg)
    wanted = set(range(cfg.n_layers)) if layers is None else set(int(i) for i in layers)
    lw: List[Optional[LayerWeights]] = []
    for li in range(cfg.n_layers):
        if li not in wanted:
            lw.append(None)
            continue
        base = 1 + 9 * li
        fields = {}
        for j, name in enumerate(LayerWeights.FIELDS):
            fields[name] = gain() if name.endswith("norm") else matrix(shapes[name], base + j)
        lw.append(LayerWeights(**fields))
    final_norm = gain()
    lm_head = matrix((V, H), 2 + 9 * cfg.n_layers)

    nthreads = threads or min(16, len(os.sched_getaffinity(0)))
    with ThreadPoolExecutor(max_workers=max(1, nthreads)) as ex:
        list(ex.map(lambda j: _fill_normal(j[0], seed, j[1], cfg.dtype, j[2], j[3]), jobs))
    return ModelWeights(cfg.dtype, tok_embed, final_norm, lm_head, lw)


def gen_ids(batch: int, length: int, vocab: int, seed: int = 1, stream: int = 0) -> np.ndarray:
    """Uniform token ids in ``[0, vocab)``, shape ``[batch, length]``, int32.

    ``stream`` selects an independent sequence for the same seed (0 = prompt,
    1 = teacher-forced continuation ids).
    """
    rng = np.random.Generator(np.random.PCG64DXSM(np.random.SeedSequence([seed, 7919, stream])))
    return rng.integers(0, vocab, size=(batch, length), dtype=np.int64).astype(np.int32)
