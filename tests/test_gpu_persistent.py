"""The persistent decode step (the whole layer stack in one launch of resident
workgroups that signal each other) against the per-layer launches and the oracle.

Every layer must follow the ladder rule and the batch be at most 4; other models and
batches take the per-layer path under the same schedule, which is checked too.
"""
import numpy as np
import pytest
import torch

import synth
from gpu_helpers import (TOL, check_against_oracle, gpu_free_running, gpu_teacher_forced, log, make_model,
                         oracle_record, step_rel_err)
from oracle import LadderOracle, teacher_forced

pytestmark = pytest.mark.gpu

FUSED, PERSISTENT = 3, 4

# ragged bf16 shapes, every layer ladder: H = 2112, 6 query / 2 kv heads of 64, F = 1344
LADDER_EDGE = synth.ModelConfig("ladder_edge", 3, 2112, 6, 2, 64, 1344, 1001, 1e4, "bf16", (1, 1, 1))
# one tensor-parallel rank of a large model, scaled down: 8 query heads of 128 over one kv head
SHARD_LIKE = synth.ModelConfig("shard_like", 4, 1024, 8, 1, 128, 768, 1000, 5e5, "bf16", (1, 1, 1, 1))


@pytest.fixture(scope="module", params=[LADDER_EDGE, SHARD_LIKE], ids=lambda c: c.name)
def model_w(request):
    cfg = request.param
    return cfg, synth.gen_weights(cfg, seed=21)


def run(cfg, w, sched, prompt, cont, max_seq, use_graph=True, trace=None):
    m = make_model(cfg, w, prompt.shape[0], max_seq)
    m.set_schedule(sched, use_graph)
    if trace:
        m.trace_kernel(trace)
    out = gpu_teacher_forced(m, prompt, cont)
    res = m.trace_result() if trace else None
    m.free()
    return out, res


@pytest.mark.parametrize("B", [1, 2, 3, 4])
@pytest.mark.parametrize("use_graph", [False, True])
def test_persistent_is_bitwise_the_per_layer_path(model_w, B, use_graph):
    """Same kernels per row, same merge order: the persistent launch must reproduce the
    per-layer launches bit for bit (a missing wait would read a stale residual, q, K/V
    row or attention output), and both match the oracle."""
    cfg, w = model_w
    prompt = synth.gen_ids(B, 19, cfg.vocab, seed=22)
    cont = synth.gen_ids(B, 5, cfg.vocab, seed=22, stream=1)
    log(f"persistent {cfg.name} B={B} graph={use_graph}")
    ref, _ = run(cfg, w, FUSED, prompt, cont, 32, use_graph)
    # eager runs also time the launch (one per step)
    got, tr = run(cfg, w, PERSISTENT, prompt, cont, 32, use_graph, trace=None if use_graph else "layer_stack")
    if tr is not None:
        assert tr[1] == 1 and tr[0] > 0.0
    for a, b in zip(ref, got):
        assert np.array_equal(a, b)
    o = teacher_forced(LadderOracle(cfg, w), prompt, cont)
    el = step_rel_err(got[0], o.logits[:, prompt.shape[1] - 1:])
    eh = step_rel_err(got[1], o.hidden[:, prompt.shape[1] - 1:])
    log(f"  vs oracle: logits {el:.3g} hidden {eh:.3g}")
    assert el <= TOL["bf16"] and eh <= TOL["bf16"]


def test_persistent_long_context(model_w):
    """2100 cached keys: 16 key chunks of three tiles each, merged across chunks."""
    cfg, w = model_w
    prompt = synth.gen_ids(1, 2100, cfg.vocab, seed=23)
    cont = synth.gen_ids(1, 3, cfg.vocab, seed=23, stream=1)
    log(f"persistent long context {cfg.name}")
    ref, _ = run(cfg, w, FUSED, prompt, cont, 2200)
    got, _ = run(cfg, w, PERSISTENT, prompt, cont, 2200)
    for a, b in zip(ref, got):
        assert np.array_equal(a, b)
    o = teacher_forced(LadderOracle(cfg, w), prompt, cont)
    assert step_rel_err(got[0], o.logits[:, 2099:]) <= TOL["bf16"]


def test_persistent_greedy_generation(model_w):
    """The oracle's greedy record fed teacher-forced matches within tolerance (argmax
    equal outside near-ties), and free-running decoding (each step's argmax fed back on
    the device) reproduces the tokens of the same path fed those tokens."""
    cfg, w = model_w
    prompt = synth.gen_ids(2, 9, cfg.vocab, seed=24)
    ref = oracle_record(cfg, w, prompt, 8)
    m = make_model(cfg, w, 2, 24)
    m.set_schedule(PERSISTENT, True)
    gl, gh, gt = gpu_teacher_forced(m, prompt, ref["tokens"][:, :-1])
    m.free()
    check_against_oracle(cfg, gl, gh, gt, ref, TOL["bf16"], f"persistent greedy {cfg.name}")
    m = make_model(cfg, w, 2, 24)
    m.set_schedule(PERSISTENT, True)
    toks = gpu_free_running(m, prompt, 8)
    m.free()
    m = make_model(cfg, w, 2, 24)
    m.set_schedule(PERSISTENT, True)
    _, _, again = gpu_teacher_forced(m, prompt, toks[:, :-1])
    m.free()
    assert np.array_equal(toks, again)


def test_persistent_falls_back_where_it_cannot_run():
    """A standard layer in the stack, or a batch above 4: the schedule takes the
    per-layer launches (bitwise those of FUSED), and the kernel timer reports -1."""
    cfg = synth.ModelConfig("mixed", 3, 2112, 6, 2, 64, 1344, 1001, 1e4, "bf16", (0, 1, 1))
    w = synth.gen_weights(cfg, seed=25)
    prompt = synth.gen_ids(2, 11, cfg.vocab, seed=25)
    cont = synth.gen_ids(2, 3, cfg.vocab, seed=25, stream=1)
    ref, _ = run(cfg, w, FUSED, prompt, cont, 16)
    got, _ = run(cfg, w, PERSISTENT, prompt, cont, 16)
    for a, b in zip(ref, got):
        assert np.array_equal(a, b)
    m = make_model(cfg, w, 2, 16)
    m.prefill(torch.from_numpy(prompt).cuda())
    us = m.time_kernels(2, 1)
    assert us["layer_stack"] == -1.0
    m.free()
    cfg5 = LADDER_EDGE
    w5 = synth.gen_weights(cfg5, seed=26)
    prompt5 = synth.gen_ids(5, 7, cfg5.vocab, seed=26)
    cont5 = synth.gen_ids(5, 2, cfg5.vocab, seed=26, stream=1)
    ref, _ = run(cfg5, w5, FUSED, prompt5, cont5, 16)
    got, _ = run(cfg5, w5, PERSISTENT, prompt5, cont5, 16)
    for a, b in zip(ref, got):
        assert np.array_equal(a, b)


def test_persistent_kernel_timer(model_w):
    cfg, w = model_w
    prompt = synth.gen_ids(1, 9, cfg.vocab, seed=27)
    m = make_model(cfg, w, 1, 16)
    m.set_schedule(PERSISTENT, True)
    m.prefill(torch.from_numpy(prompt).cuda())
    m.decode_step(torch.zeros(1, dtype=torch.int32, device="cuda"), 9)
    us = m.time_kernels(1, 2)
    m.sync()
    m.free()
    log(f"persistent timer {cfg.name}: {us['layer_stack']:.1f} us per stack")
    assert us["layer_stack"] > 0.0
