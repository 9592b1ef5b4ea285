"""ladder_decode_step_static (the decode step whose per-step buffers live in the library's
static scratch, for callers that cannot allocate) against ladder_decode_step.

Two contexts with the same weights and prompt run the same decode steps, one through each
entry point; the static one must give the same logits, hidden state and next tokens bit
for bit (same kernels, same arguments apart from the buffer addresses), call after call,
with the batch shrinking from one call to the next so that every call inherits a scratch
array that a larger call left behind.  All calls go through the C ABI.
"""
import numpy as np
import pytest
import torch

import synth
from gpu_helpers import log, make_model

from ladder_residual_transformer_amd import abi

pytestmark = pytest.mark.gpu

# bf16 model with ragged shapes and every layer kind (standard, parallel, ladder): batch 5
# takes the matrix-core decode route (split-K partials in the scratch), batch 2 the
# row-wave GEMV, batch 1 the two streaming launches per ladder layer (tagged handoff words
# and attention chunk records in the scratch).
MIXED = synth.ModelConfig("mixed", 4, 2112, 6, 2, 64, 1344, 1001, 1e4, "bf16", (0, 2, 1, 2))


def _outs(model, B):
    cfg = model.cfg
    return (torch.empty(B, cfg.vocab, device="cuda", dtype=torch.float32),
            torch.empty(B, device="cuda", dtype=torch.int32),
            torch.empty(B, cfg.hidden, device="cuda", dtype=torch.float32))


def _pair(cfg, w, max_batch, max_seq, prompt):
    ids = torch.from_numpy(np.ascontiguousarray(prompt, dtype=np.int32)).cuda()
    models = []
    for _ in range(2):
        m = make_model(cfg, w, max_batch, max_seq)
        m.prefill(ids)
        models.append(m)
    return models


def _run_steps(ref, new, steps, vocab, seed):
    """Decode with ref (ladder_decode_step) and new (ladder_decode_step_static) at the
    (batch, position) pairs of `steps` and compare every output.  A step never reads a
    position of a sequence that no earlier call wrote: after a smaller batch, a larger one
    repeats the smaller one's position (rewriting those rows)."""
    for k, (B, pos) in enumerate(steps):
        ids = torch.from_numpy(synth.gen_ids(B, 1, vocab, seed=seed, stream=k)[:, 0].astype(np.int32)).cuda()
        log(f"  step {k}: B={B} pos={pos}")
        a = ref.decode_step(ids, pos, out=_outs(ref, B))
        b = new.decode_step_static(ids, pos, _outs(new, B))
        torch.cuda.synchronize()
        for name, x, y in zip(("logits", "next", "hidden"), a, b):
            x, y = x.cpu().numpy(), y.cpu().numpy()
            assert np.isfinite(x).all() if x.dtype != np.int32 else True
            assert np.array_equal(x, y), f"{name} differs at step {k} (B={B})"
    ref.sync()
    new.sync()


def test_static_step_matches_decode_step_bf16():
    cfg = MIXED
    w = synth.gen_weights(cfg, seed=3)
    T = 19
    prompt = synth.gen_ids(5, T, cfg.vocab, seed=11)
    ref, new = _pair(cfg, w, 5, 48, prompt)
    steps = [(5, T), (2, T + 1), (1, T + 2), (1, T + 3), (5, T + 1), (1, T + 2)]
    log("mixed bf16: (batch, position)", steps)
    _run_steps(ref, new, steps, cfg.vocab, seed=12)
    ref.free()
    new.free()


def test_static_step_matches_decode_step_fp32():
    """fp32 model: batch 8 on the K-sliced GEMV (last-arriver counters in the scratch),
    then batch 3 and 1 on the row-wave GEMV."""
    cfg = synth.CONFIGS["tiny"]
    w = synth.gen_weights(cfg, seed=0)
    T = 13
    prompt = synth.gen_ids(8, T, cfg.vocab, seed=21)
    ref, new = _pair(cfg, w, 8, 32, prompt)
    steps = [(8, T), (3, T + 1), (1, T + 2)]
    log("tiny fp32: (batch, position)", steps)
    _run_steps(ref, new, steps, cfg.vocab, seed=22)
    ref.free()
    new.free()


def test_static_step_leaves_the_context_and_other_contexts_intact():
    """The context's own entry point still works between static calls (its per-step
    buffers point back at its workspace), two contexts may take turns on the scratch on
    one stream, and a stochastic draw gives the same tokens through both entry points."""
    cfg = MIXED
    w = synth.gen_weights(cfg, seed=3)
    T = 9
    prompt = synth.gen_ids(2, T, cfg.vocab, seed=31)
    ids = torch.from_numpy(np.ascontiguousarray(prompt, dtype=np.int32)).cuda()
    ref = make_model(cfg, w, 2, 24)
    a = make_model(cfg, w, 2, 24)
    b = make_model(cfg, w, 2, 24)
    for m in (ref, a, b):
        m.prefill(ids)
        m.set_sampling(0.8, top_k=50, seed=5)
    log("three contexts, batch 2 then 1 then 2, sampling on")
    for k, (B, pos) in enumerate([(2, T), (1, T + 1), (2, T + 1)]):
        tok = torch.from_numpy(synth.gen_ids(B, 1, cfg.vocab, seed=32, stream=k)[:, 0].astype(np.int32)).cuda()
        r = ref.decode_step(tok, pos, out=_outs(ref, B))
        x = a.decode_step_static(tok, pos, _outs(a, B))
        y = b.decode_step_static(tok, pos, _outs(b, B)) if k != 1 else b.decode_step(tok, pos, out=_outs(b, B))
        torch.cuda.synchronize()
        for got in (x, y):
            for u, v in zip(r, got):
                assert torch.equal(u, v), f"step {k}"
    for m in (ref, a, b):
        m.sync()
        m.free()


def test_static_step_rejects_a_step_beyond_the_scratch():
    """A step whose per-step buffers exceed the 64 MiB array (the logits alone of 64
    sequences over 300000 rows take 76.8 MB) is refused with LADDER_ERR_CAPACITY and the
    bytes it needs; the context stays usable through both entry points."""
    cfg = synth.ModelConfig("wide_vocab", 1, 64, 1, 1, 64, 128, 300_000, 1e4, "bf16", (1,))
    w = synth.gen_weights(cfg, seed=4)
    prompt = synth.gen_ids(64, 3, cfg.vocab, seed=41)
    ref, new = _pair(cfg, w, 64, 8, prompt)
    tok = torch.from_numpy(synth.gen_ids(64, 1, cfg.vocab, seed=42)[:, 0].astype(np.int32)).cuda()
    log("wide vocab: batch 64 refused, then batch 64 through ladder_decode_step, then batch 1")
    with pytest.raises(abi.LadderError) as e:
        new.decode_step_static(tok, 3, _outs(new, 64))
    assert e.value.status == abi.LADDER_ERR_CAPACITY
    assert "static scratch" in str(e.value)
    a = ref.decode_step(tok, 3, out=_outs(ref, 64))
    b = new.decode_step(tok, 3, out=_outs(new, 64))
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u, v)
    _run_steps(ref, new, [(1, 4)], cfg.vocab, seed=43)
    ref.free()
    new.free()
