"""Plain numpy forward of standard and Ladder Residual Transformer blocks (test infrastructure).

Sources (pages on arXiv 2501.06589, "Ladder-residual: parallelism-aware
architecture for accelerating large model inference with communication
overlapping"):

* Paper-Notes page "Ladder Residual: Parallelism-Aware Architecture for
  Accelerating Large Model Inference" (ICML 2025 notes), sections
  "research background and motivation / core idea" and "method details /
  key design: staggered residual connection": the ladder rule
  x_{i+1} = h_{i+1}(x_{i-1}) + x_i against the standard x_{i+1} = h_{i+1}(x_i) + x_i;
  section "method details / overall framework": every Attention and every
  MLP is one module h, the residual stream keeps accumulating every module's
  output and only the module inputs are one step stale;
  section "asynchronous AllReduce implementation": within a layer the
  attention module runs first, then the MLP;
  section "hybrid Ladder adaptation": the lower layers of a model may stay
  standard while the upper ones are ladder.
* ICML 2025 poster page and the codewithpapers record: the models are
  Llama-3.1 shaped (RMSNorm, rotary embeddings with ``precompute_freqs_cis``
  / ``apply_rotary_emb``, grouped-query attention with ``repeat_kv``, SwiGLU
  MLP).

Readings where the pages are silent (each is listed with its reason in the
design notes of the repository):
  * the first module has no x_{-1}; it is taken to be x_0, so the first
    attention and the first MLP both read the embedding;
  * a layer's flag covers both of its modules; the rule is applied per module,
    so at a standard->ladder boundary the first ladder module reads x_{m-1};
  * pre-norm RMSNorm with eps 1e-5, gains stored with the weights;
  * rotary pairs are adjacent elements (2j, 2j+1), angle p * theta^(-2j/hd);
  * where a model config carries ``rope_scaling`` (Llama-3.1 shapes: factor 8,
    low_freq_factor 1, high_freq_factor 4, original context 8192), the frequencies
    theta^(-2j/hd) first go through Llama-3.1's published band rule
    (llama3_scale_inv_freq); the pages only name the function;
  * no biases, untied LM head, greedy argmax takes the lowest index on ties;
  * the KV cache is model state kept in the model's storage type, like the
    weights it is computed from: each K and V value is rounded to that type
    (round to nearest, ties to even) when it is written, and attention reads
    the stored values.  ``kv_store_dtype=False`` keeps them unrounded.

Compute precision is float64 unless the caller asks for float32 (used only to
time the oracle and to run the largest shards within host memory).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np

# ---------------------------------------------------------------------------
# element-wise building blocks
# ---------------------------------------------------------------------------


def upcast(w: np.ndarray, dtype=np.float64) -> np.ndarray:
    """Exact value of a stored weight in ``dtype``.

    bf16 tensors arrive as uint16 bit patterns; a bf16 value is the float32
    whose upper 16 bits are that pattern and whose lower 16 bits are zero.
    Pin: known bit patterns (1.0, -2.0, 0.5, smallest normal) decode exactly.
    """
    if w.dtype == np.uint16:
        f = (w.astype(np.uint32) << np.uint32(16)).view(np.float32)
    elif w.dtype == np.float32 or w.dtype == np.float64:
        f = w
    else:
        raise TypeError(f"unsupported stored dtype {w.dtype}")
    return np.asarray(f, dtype=dtype)


def round_to_storage(x: np.ndarray, dtype_name: str) -> np.ndarray:
    """Round ``x`` to the model's storage type, keeping the array's own dtype.

    bf16 has 8 significant bits: with x = f * 2**e, 0.5 <= |f| < 1 (frexp), the
    spacing of bf16 values around x is 2**(e - 8), and 2**-133 below the smallest
    normal 2**-126; x / spacing is rounded half-to-even (numpy ``rint``) and scaled
    back, which is exact in binary floating point.  fp32 storage is numpy's own
    round-to-nearest-even conversion.  Pins: halfway cases round to the even
    neighbour; agreement with an independent bit-pattern rounding of float32 input.
    """
    if dtype_name == "bf16":
        x64 = np.asarray(x, dtype=np.float64)
        _, e = np.frexp(x64)
        q = np.ldexp(1.0, np.maximum(e, -125) - 8)
        return (np.rint(x64 / q) * q).astype(x.dtype)
    if dtype_name == "f32":
        return np.asarray(x).astype(np.float32).astype(x.dtype)
    raise ValueError(f"unknown storage dtype {dtype_name!r}")


def rms_norm(x: np.ndarray, gain: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm over the last axis: x / sqrt(mean(x^2) + eps) * gain.

    Pin: equals torch.nn.functional.rms_norm; scale invariance for c > 0.
    """
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * gain


def llama3_scale_inv_freq(inv_freq: np.ndarray, factor: float, low_freq_factor: float,
                          high_freq_factor: float, original_max_pos: int) -> np.ndarray:
    """Llama-3.1 rotary frequency scaling (the function the method's inference code calls
    ``apply_rope_scaling``, named on the codewithpapers record; the pages give no
    constants, so the rule and its constants are those Llama-3.1 publishes, see the
    readings in the module docstring).

    With the wavelength w = 2 pi / f of a pair's frequency f and the original context
    length N: a pair with w < N / high_freq_factor keeps f; a pair with
    w > N / low_freq_factor gets f / factor; in between, with
    s = (N / w - low_freq_factor) / (high_freq_factor - low_freq_factor) in [0, 1],
    f becomes (1 - s) f / factor + s f, which meets both sides at the band edges.
    Pins: the closed forms at chosen wavelengths (f, f, 5f/12 at w = N/2 for the
    Llama-3.1 constants, f / factor), continuity at both edges, monotonicity in w and
    the identity for factor 1.
    """
    f = np.asarray(inv_freq, dtype=np.float64)
    wavelen = 2.0 * np.pi / f
    low_wavelen = original_max_pos / low_freq_factor      # longer: fully scaled
    high_wavelen = original_max_pos / high_freq_factor    # shorter: unchanged
    s = (original_max_pos / wavelen - low_freq_factor) / (high_freq_factor - low_freq_factor)
    mid = (1.0 - s) * f / factor + s * f
    return np.where(wavelen < high_wavelen, f, np.where(wavelen > low_wavelen, f / factor, mid))


def rope_inv_freq(head_dim: int, theta: float, scaling=None) -> np.ndarray:
    """Frequency of pair j: theta^(-2j/head_dim), j < head_dim/2; with ``scaling`` =
    (factor, low_freq_factor, high_freq_factor, original_max_pos) passed through
    llama3_scale_inv_freq."""
    j = np.arange(head_dim // 2, dtype=np.float64)
    inv_freq = np.power(float(theta), -2.0 * j / head_dim)
    if scaling is not None:
        inv_freq = llama3_scale_inv_freq(inv_freq, *scaling)
    return inv_freq


def rope_angles(positions: np.ndarray, head_dim: int, theta: float, scaling=None) -> np.ndarray:
    """Rotation angle of pair j at position p: p * f_j (rope_inv_freq), shape [P, head_dim/2]."""
    return np.outer(np.asarray(positions, dtype=np.float64), rope_inv_freq(head_dim, theta, scaling))


def apply_rope(x: np.ndarray, positions: np.ndarray, theta: float, scaling=None) -> np.ndarray:
    """Rotate adjacent pairs (x[2j], x[2j+1]) of the last axis by their angle.

    ``x`` has shape [..., P, head_dim] with positions along axis -2.
    Pin: equals multiplication by the complex phase e^{i*angle} (torch.polar);
    identity at p = 0; preserves norms; q_p . k_s depends only on p - s.
    """
    hd = x.shape[-1]
    ang = rope_angles(positions, hd, theta, scaling)
    c = np.cos(ang).astype(x.dtype)
    s = np.sin(ang).astype(x.dtype)
    x0 = x[..., 0::2]
    x1 = x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


def gqa_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                  q_pos: np.ndarray, k_pos: np.ndarray) -> np.ndarray:
    """Causal grouped-query softmax attention.

    q: [B, nq, T, hd]; k, v: [B, nkv, S, hd]; query head h reads key/value head
    h // (nq / nkv).  A query at position p sees the keys at positions <= p.
    Scale 1/sqrt(hd).  Returns [B, nq, T, hd].
    Pin: equals torch's scaled_dot_product_attention (is_causal) with repeated
    KV heads; with a single key it returns that key's value exactly.
    """
    B, nq, T, hd = q.shape
    nkv = k.shape[1]
    group = nq // nkv
    allowed = np.asarray(k_pos)[None, :] <= np.asarray(q_pos)[:, None]     # [T, S]
    scale = 1.0 / np.sqrt(hd)
    out = np.empty_like(q)
    for h in range(nq):
        kv = h // group
        scores = np.matmul(q[:, h], np.swapaxes(k[:, kv], -1, -2)) * scale   # [B, T, S]
        scores = np.where(allowed[None], scores, -np.inf)
        scores = scores - scores.max(axis=-1, keepdims=True)
        p = np.exp(scores)
        p = p / p.sum(axis=-1, keepdims=True)
        out[:, h] = np.matmul(p, v[:, kv])
    return out


def silu(z: np.ndarray) -> np.ndarray:
    """SiLU z * sigmoid(z) = z / (1 + e^{-z}).  Pin: torch silu; silu(0) = 0; silu(z) -> z."""
    return z / (1.0 + np.exp(-z))


def swiglu_mlp(u: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray, w_down: np.ndarray) -> np.ndarray:
    """SwiGLU MLP (silu(u Wg^T) * (u Wu^T)) Wd^T on normalised input u.  Pin: torch textbook model."""
    g = np.matmul(u, w_gate.T)
    a = silu(g) * np.matmul(u, w_up.T)
    return np.matmul(a, w_down.T)


def module_input_index(m: int, ladder_mask) -> int:
    """Index j of the residual x_j that module m (0-based) reads.

    Modules are numbered m = 0..2L-1: m = 2l is layer l's attention, m = 2l+1
    its MLP, and x_{m+1} = x_m + out_m.  The layer's mask value picks the rule:

    * 0, standard: every module reads x_m, the residual right before it;
    * 1, ladder (Paper-Notes page, "method details / key design: staggered residual
      connection"): every module reads x_{m-1}, one step earlier, with x_{-1}
      taken as x_0;
    * 2, parallel block (the "Parallel" baseline the paper compares against,
      which it does not define; read as the GPT-J style block): both modules
      of the layer read the layer input x_{2l}, so the attention follows the
      standard rule and the MLP the ladder one.

    Pins: the hand-expanded two-layer formulas for every mask over {0, 1, 2};
    the parallel block's closed form x_{2l+2} = x_{2l} + A(x_{2l}) + M(x_{2l});
    a parallel first layer equals a ladder first layer.
    """
    mode = ladder_mask[m // 2]
    if mode == 1 or (mode == 2 and m % 2 == 1):
        return max(m - 1, 0)
    return m


# ---------------------------------------------------------------------------
# the model
# ---------------------------------------------------------------------------


@dataclasses.dataclass
class ForwardResult:
    hidden: np.ndarray                    # final residual x_{2L}, [B, T, H]
    logits: Optional[np.ndarray]          # [B, T or 1, V] (None if not requested)
    module_outputs: Optional[List[np.ndarray]] = None   # out_m, when recorded
    residuals: Optional[List[np.ndarray]] = None        # x_0 .. x_{2L}, when recorded


class LadderOracle:
    """Forward pass over a chunk of tokens with an explicit per-layer KV cache.

    ``weights`` is a ``synth.ModelWeights``-like object (attributes tok_embed,
    final_norm, lm_head, layers[...] with attn_norm, wq, wk, wv, wo, mlp_norm,
    w_gate, w_up, w_down) holding the stored arrays; ``cfg`` provides the
    shapes (hidden, n_q_heads, n_kv_heads, head_dim, n_layers, rope_theta,
    norm_eps, ladder_mask, dtype).  Weights are upcast exactly from their stored
    values, one layer at a time unless ``cache_weights`` keeps them.  New K and V
    rows are rounded to ``cfg.dtype`` before they enter the cache unless
    ``kv_store_dtype`` is False.
    """

    def __init__(self, cfg, weights, dtype=np.float64, cache_weights: bool = False,
                 ladder_mask=None, kv_store_dtype: bool = True):
        self.cfg = cfg
        self.kv_store_dtype = kv_store_dtype
        self.w = weights
        self.dtype = np.dtype(dtype)
        self.mask = tuple(int(v) for v in (cfg.ladder_mask if ladder_mask is None else ladder_mask))
        if len(self.mask) != cfg.n_layers:
            raise ValueError("one mask entry per layer")
        if any(v not in (0, 1, 2) for v in self.mask):
            raise ValueError("mask entries are 0 (standard), 1 (ladder) or 2 (parallel)")
        self.cache_weights = cache_weights
        self._cache: Dict[int, dict] = {}
        self._head: Optional[dict] = None

    # -- weights --------------------------------------------------------
    def layer(self, li: int) -> dict:
        if li in self._cache:
            return self._cache[li]
        lw = self.w.layers[li]
        d = {name: upcast(getattr(lw, name), self.dtype) for name in
             ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate", "w_up", "w_down")}
        if self.cache_weights:
            self._cache[li] = d
        return d

    def head(self) -> dict:
        if self._head is not None:
            return self._head
        d = {"final_norm": upcast(self.w.final_norm, self.dtype),
             "lm_head": upcast(self.w.lm_head, self.dtype)}
        if self.cache_weights:
            self._head = d
        return d

    def embed(self, ids: np.ndarray) -> np.ndarray:
        return upcast(self.w.tok_embed[np.asarray(ids)], self.dtype)

    # -- KV cache ---------------------------------------------------------
    def new_cache(self) -> dict:
        return {"k": [None] * self.cfg.n_layers, "v": [None] * self.cfg.n_layers, "len": 0}

    # -- modules ----------------------------------------------------------
    def attention(self, li: int, x_in: np.ndarray, cache: dict, start_pos: int) -> np.ndarray:
        """Layer li's attention module on input x_in [B, T, H] at positions start_pos.. ."""
        cfg = self.cfg
        W = self.layer(li)
        B, T, _ = x_in.shape
        nq, nkv, hd = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
        u = rms_norm(x_in, W["attn_norm"], cfg.norm_eps)
        q = np.matmul(u, W["wq"].T).reshape(B, T, nq, hd).transpose(0, 2, 1, 3)
        k = np.matmul(u, W["wk"].T).reshape(B, T, nkv, hd).transpose(0, 2, 1, 3)
        v = np.matmul(u, W["wv"].T).reshape(B, T, nkv, hd).transpose(0, 2, 1, 3)
        pos = start_pos + np.arange(T)
        scaling = getattr(cfg, "rope_scaling", None)
        q = apply_rope(q, pos, cfg.rope_theta, scaling)
        k = apply_rope(k, pos, cfg.rope_theta, scaling)
        if self.kv_store_dtype:
            k = round_to_storage(k, cfg.dtype)
            v = round_to_storage(v, cfg.dtype)
        prev_k, prev_v = cache["k"][li], cache["v"][li]
        if start_pos == 0 or prev_k is None:
            if start_pos != 0:
                raise ValueError("cache is empty but start_pos > 0")
            k_all, v_all = k, v
        else:
            if prev_k.shape[2] != start_pos:
                raise ValueError("cache length does not match start_pos")
            k_all = np.concatenate([prev_k, k], axis=2)
            v_all = np.concatenate([prev_v, v], axis=2)
        cache["k"][li], cache["v"][li] = k_all, v_all
        o = gqa_attention(q, k_all, v_all, pos, np.arange(start_pos + T))
        o = o.transpose(0, 2, 1, 3).reshape(B, T, nq * hd)
        return np.matmul(o, W["wo"].T)

    def mlp(self, li: int, x_in: np.ndarray) -> np.ndarray:
        """Layer li's SwiGLU MLP module on input x_in [B, T, H]."""
        W = self.layer(li)
        u = rms_norm(x_in, W["mlp_norm"], self.cfg.norm_eps)
        return swiglu_mlp(u, W["w_gate"], W["w_up"], W["w_down"])

    # -- whole model ------------------------------------------------------
    def forward(self, ids: np.ndarray, cache: Optional[dict] = None, start_pos: int = 0,
                logits: str = "all", record: bool = False) -> ForwardResult:
        """Run tokens ``ids`` [B, T] at positions start_pos..start_pos+T-1.

        The module loop is the ladder rule itself: module m reads
        x_{module_input_index(m)} and the stream adds its output,
        x_{m+1} = x_m + out_m.
        """
        ids = np.asarray(ids)
        if ids.ndim != 2:
            raise ValueError("ids must be [B, T]")
        cfg = self.cfg
        if cache is None:
            cache = self.new_cache()
        if cache["len"] != start_pos:
            raise ValueError("start_pos must equal the number of cached positions")
        xs: Dict[int, np.ndarray] = {0: self.embed(ids)}
        outs: List[np.ndarray] = []
        kept: List[np.ndarray] = [xs[0]] if record else []
        for m in range(2 * cfg.n_layers):
            li = m // 2
            x_in = xs[module_input_index(m, self.mask)]
            if m % 2 == 0:
                out = self.attention(li, x_in, cache, start_pos)
            else:
                out = self.mlp(li, x_in)
            xs[m + 1] = xs[m] + out
            if record:
                outs.append(out)
                kept.append(xs[m + 1])
            xs.pop(m - 1, None)          # no later module reads x_{m-1}
        cache["len"] = start_pos + ids.shape[1]
        hidden = xs[2 * cfg.n_layers]
        lg = None
        if logits in ("all", "last"):
            h = hidden if logits == "all" else hidden[:, -1:]
            hd = self.head()
            lg = np.matmul(rms_norm(h, hd["final_norm"], cfg.norm_eps), hd["lm_head"].T)
        elif logits is not None and logits != "none":
            raise ValueError("logits must be 'all', 'last' or None")
        return ForwardResult(hidden, lg, outs if record else None, kept if record else None)


def _top2_margin(logits: np.ndarray):
    """argmax (lowest index on exact ties) and the gap to the runner-up, per row."""
    idx = np.argmax(logits, axis=-1)
    top = np.take_along_axis(logits, idx[:, None], axis=-1)[:, 0]
    masked = logits.copy()
    np.put_along_axis(masked, idx[:, None], -np.inf, axis=-1)
    return idx, top - masked.max(axis=-1)


def greedy_generate(oracle: LadderOracle, prompt: np.ndarray, n_decode: int) -> dict:
    """Free-running greedy decoding.

    Prefill ``prompt`` [B, T] (its last logits give token 0), then ``n_decode``
    single-token steps at positions T..T+n_decode-1, each feeding the previous
    token.  Returns the produced tokens [B, n_decode+1], the top-1/top-2 margin
    of every choice, and the final hidden state and logits of each step
    (index 0 = prefill's last position).
    """
    B, T = prompt.shape
    cache = oracle.new_cache()
    r = oracle.forward(prompt, cache, 0, logits="last")
    tokens, margins, hiddens, logits = [], [], [r.hidden[:, -1]], [r.logits[:, -1]]
    for step in range(n_decode + 1):
        tok, mar = _top2_margin(logits[-1])
        tokens.append(tok)
        margins.append(mar)
        if step == n_decode:
            break
        r = oracle.forward(tok[:, None].astype(np.int64), cache, T + step, logits="last")
        hiddens.append(r.hidden[:, -1])
        logits.append(r.logits[:, -1])
    return {"tokens": np.stack(tokens, axis=1), "margins": np.stack(margins, axis=1),
            "hidden": np.stack(hiddens, axis=1), "logits": np.stack(logits, axis=1)}


def teacher_forced(oracle: LadderOracle, prompt: np.ndarray, cont: np.ndarray,
                   logits: str = "all") -> ForwardResult:
    """One pass over prompt followed by the given continuation ids.

    Position T-1+k of the result is what decode step k (k >= 1, fed
    cont[:, k-1] at position T+k-1) must produce.
    """
    ids = np.concatenate([prompt, cont], axis=1) if cont is not None and cont.size else prompt
    return oracle.forward(ids, None, 0, logits=logits)
