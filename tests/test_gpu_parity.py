"""HIP path vs the oracle on small models: every kernel, schedule, mask and edge case.

All calls go through the C ABI (libladder.so via ctypes); inputs are the seeded synth
arrays, expected values come from oracle/ only.
"""
import dataclasses

import numpy as np
import pytest
import torch

import synth
from gpu_helpers import (TOL, check_against_oracle, gpu_free_running, gpu_teacher_forced, log, make_model,
                         oracle_record, rel_err, small_config, step_rel_err)
from oracle import LadderOracle, teacher_forced

pytestmark = pytest.mark.gpu

SERIAL, SIDE, DUAL, FUSED, PERSISTENT, LATE = 0, 1, 2, 3, 4, 5

# bf16 model with ragged shapes: H = 2112 (264 vectors: two K slices at batch > 4, the
# second one short), 6 query / 2 kv heads of 64, F = 1344, vocab 1001 (ragged row
# tiles), standard layer 0 then ladder layers 1-2.
EDGE = synth.ModelConfig("edge", 3, 2112, 6, 2, 64, 1344, 1001, 1e4, "bf16", (0, 1, 1))


@pytest.fixture(scope="module")
def tiny():
    cfg = synth.CONFIGS["tiny"]
    return cfg, synth.gen_weights(cfg, seed=0)


def test_tiny_fp32_matches_oracle_and_greedy_is_identical(tiny):
    cfg, w = tiny
    wl = synth.WORKLOADS["tiny"]
    prompt = synth.gen_ids(1, wl.prompt_len, cfg.vocab, seed=1)
    log("tiny fp32: B=1 prompt", wl.prompt_len, "decode", wl.decode_len)
    ref = oracle_record(cfg, w, prompt, wl.decode_len)
    model = make_model(cfg, w, 1, wl.max_seq)
    gl, gh, gt = gpu_teacher_forced(model, prompt, ref["tokens"][:, :-1])
    check_against_oracle(cfg, gl, gh, gt, ref, TOL["f32"], "tiny teacher-forced")
    assert np.array_equal(gt, ref["tokens"])
    free = gpu_free_running(model, prompt, wl.decode_len)
    assert np.array_equal(free, ref["tokens"]), (free, ref["tokens"])
    model.free()


@pytest.mark.parametrize("mask", [(0, 0), (0, 1), (1, 0), (2, 2), (0, 2), (2, 1)])
def test_tiny_every_mask(tiny, mask):
    cfg, w = tiny
    cfg = cfg.with_mask(mask)
    prompt = synth.gen_ids(1, 9, cfg.vocab, seed=2)
    log("tiny mask", mask)
    ref = oracle_record(cfg, w, prompt, 6)
    model = make_model(cfg, w, 1, 16)
    gl, gh, gt = gpu_teacher_forced(model, prompt, ref["tokens"][:, :-1])
    check_against_oracle(cfg, gl, gh, gt, ref, TOL["f32"], f"tiny {mask}")
    assert np.array_equal(gt, ref["tokens"])
    model.free()


@pytest.mark.parametrize("B", [3, 8, 16])
def test_tiny_fp32_batches(tiny, B):
    """fp32 model beyond batch 2: B=3 on the row-wave GEMV (three batch rows staged per
    workgroup), B=8 and 16 on the K-sliced GEMV (gemv.hip) with its last-arriver tickets,
    and the VALU attention over 3-16 sequences.  Teacher-forced within 1e-5 of the fp64
    oracle with every row's argmax equal to the oracle's greedy token, and free-running
    greedy decoding identical to the oracle's."""
    cfg, w = tiny
    prompt = synth.gen_ids(B, 11, cfg.vocab, seed=40 + B)
    n_dec = 6
    log(f"tiny fp32 B={B}: prompt 11, decode {n_dec}")
    ref = oracle_record(cfg, w, prompt, n_dec)
    model = make_model(cfg, w, B, 24)
    gl, gh, gt = gpu_teacher_forced(model, prompt, ref["tokens"][:, :-1])
    check_against_oracle(cfg, gl, gh, gt, ref, TOL["f32"], f"tiny fp32 B={B}")
    assert np.array_equal(gt, ref["tokens"])
    free = gpu_free_running(model, prompt, n_dec)
    assert np.array_equal(free, ref["tokens"]), (free, ref["tokens"])
    model.free()


@pytest.mark.parametrize("sched", [SERIAL, FUSED])
def test_llama31_rope_scaling(tiny, sched):
    """Llama-3.1 rotary frequency scaling (factor 8, low 1, high 4, original context 8192)
    on the tiny fp32 model with theta 5e5: with head_dim 64, pairs 0..14 keep their
    frequency, 15..17 are blended and 18..31 divided by 8.  Prefill and decode match the
    oracle within 1e-5 with greedy tokens identical, and the scaling moves the oracle's
    logits by more than ten times that tolerance (2.5e-4 here: random weights keep the
    attention nearly uniform), so the test sees it."""
    cfg, w = tiny
    cfg = dataclasses.replace(cfg, rope_theta=5e5, rope_scaling=synth.LLAMA31_ROPE_SCALING)
    prompt = synth.gen_ids(2, 40, cfg.vocab, seed=15)
    log(f"tiny fp32 + Llama-3.1 RoPE scaling, schedule {sched}: B=2 prompt 40, decode 6")
    ref = oracle_record(cfg, w, prompt, 6)
    plain = oracle_record(dataclasses.replace(cfg, rope_scaling=None), w, prompt, 6)
    assert rel_err(plain["logits"], ref["logits"]) > 10 * TOL["f32"]
    model = make_model(cfg, w, 2, 64)
    model.set_schedule(sched)
    gl, gh, gt = gpu_teacher_forced(model, prompt, ref["tokens"][:, :-1])
    check_against_oracle(cfg, gl, gh, gt, ref, TOL["f32"], "rope scaling")
    assert np.array_equal(gt, ref["tokens"])
    model.free()


def test_single_key_prompt(tiny):
    """A one-token prompt: attention sees exactly one key (position 0)."""
    cfg, w = tiny
    prompt = synth.gen_ids(2, 1, cfg.vocab, seed=3)
    ref = oracle_record(cfg, w, prompt, 3)
    model = make_model(cfg, w, 2, 8)
    gl, gh, gt = gpu_teacher_forced(model, prompt, ref["tokens"][:, :-1])
    check_against_oracle(cfg, gl, gh, gt, ref, TOL["f32"], "single key")
    model.free()


@pytest.mark.parametrize("B", [1, 2])
def test_narrow_bf16_model(B):
    """hidden 64, one query head: too narrow for the batch-1 streaming launches (their back
    launch needs at least 128 output rows), so batch 1 takes the row-wave launches of the
    FUSED schedule instead, as batch 2 does."""
    cfg = synth.ModelConfig("narrow", 2, 64, 1, 1, 64, 128, 777, 1e4, "bf16", (1, 1))
    w = synth.gen_weights(cfg, seed=8)
    prompt = synth.gen_ids(B, 7, cfg.vocab, seed=9)
    log(f"narrow bf16 B={B}: prompt 7, decode 5")
    ref = oracle_record(cfg, w, prompt, 5)
    model = make_model(cfg, w, B, 16)
    gl, gh, gt = gpu_teacher_forced(model, prompt, ref["tokens"][:, :-1])
    check_against_oracle(cfg, gl, gh, gt, ref, TOL["bf16"], f"narrow B={B}")
    model.free()


@pytest.fixture(scope="module")
def edge():
    return EDGE, synth.gen_weights(EDGE, seed=5)


@pytest.mark.parametrize("B, T, chunk", [(1, 37, 0), (5, 37, 64), (3, 20, 0)])
def test_edge_shapes_bf16(edge, B, T, chunk):
    """Ragged tiles everywhere; B=5 splits K of the 2112-wide projections; chunk=64
    cuts the 5x37 prompt into 12-token prefill chunks."""
    cfg, w = edge
    prompt = synth.gen_ids(B, T, cfg.vocab, seed=6)
    log(f"edge bf16 B={B} T={T} chunk={chunk}")
    ref = oracle_record(cfg, w, prompt, 5, dtype=np.float64)
    model = make_model(cfg, w, B, T + 8, max_prefill_tokens=chunk)
    gl, gh, gt = gpu_teacher_forced(model, prompt, ref["tokens"][:, :-1])
    check_against_oracle(cfg, gl, gh, gt, ref, TOL["bf16"], f"edge B={B}")
    model.free()


@pytest.mark.parametrize("B", [1, 2, 5])
@pytest.mark.parametrize("use_graph", [False, True])
def test_schedules_are_bitwise_identical(edge, use_graph, B):
    """Race check: the side-stream, two-stream and fused-ladder schedules must reproduce
    the serial one bit for bit (any missing wait would read a stale or half-written
    residual).  B=1: the fused schedule's ladder layers take the two streaming launches
    (tagged QKV hand-over, attention records merged in the back launch); B=2 the row-wave
    kernels; B=5 the matrix-core decode route."""
    cfg, w = edge
    prompt = synth.gen_ids(B, 21, cfg.vocab, seed=7)
    cont = synth.gen_ids(B, 4, cfg.vocab, seed=7, stream=1)
    outs = {}
    for sched in (SERIAL, SIDE, DUAL, FUSED, LATE):
        model = make_model(cfg, w, B, 32)
        model.set_schedule(sched, use_graph)
        outs[sched] = gpu_teacher_forced(model, prompt, cont)
        model.free()
    for sched in (SIDE, DUAL, FUSED, LATE):
        for a, b in zip(outs[SERIAL], outs[sched]):
            assert np.array_equal(a, b), f"schedule {sched} differs from serial"


# The edge shapes with four layers mixing every layer kind: standard, then parallel blocks
# around a ladder layer (a parallel block after a standard or ladder layer and a ladder
# layer after a parallel block).
MIXED = synth.ModelConfig("mixed", 4, 2112, 6, 2, 64, 1344, 1001, 1e4, "bf16", (0, 2, 1, 2))


@pytest.fixture(scope="module")
def mixed():
    return MIXED, synth.gen_weights(MIXED, seed=9)


@pytest.mark.parametrize("B", [1, 5])
def test_mixed_layer_kinds_match_oracle(mixed, B):
    cfg, w = mixed
    prompt = synth.gen_ids(B, 23, cfg.vocab, seed=13)
    log(f"mixed mask {cfg.ladder_mask} bf16 B={B}")
    ref = oracle_record(cfg, w, prompt, 5, dtype=np.float64)
    model = make_model(cfg, w, B, 32)
    gl, gh, gt = gpu_teacher_forced(model, prompt, ref["tokens"][:, :-1])
    check_against_oracle(cfg, gl, gh, gt, ref, TOL["bf16"], f"mixed B={B}")
    model.free()


@pytest.mark.parametrize("B", [2, 5])
@pytest.mark.parametrize("use_graph", [False, True])
def test_mixed_layer_kinds_schedules_bitwise(mixed, use_graph, B):
    """Every schedule, including the persistent one (which falls back to the fused layers
    when not every layer is ladder), reproduces the serial result bit for bit."""
    cfg, w = mixed
    prompt = synth.gen_ids(B, 19, cfg.vocab, seed=14)
    cont = synth.gen_ids(B, 4, cfg.vocab, seed=14, stream=1)
    outs = {}
    for sched in (SERIAL, SIDE, DUAL, FUSED, PERSISTENT, LATE):
        model = make_model(cfg, w, B, 32)
        model.set_schedule(sched, use_graph)
        outs[sched] = gpu_teacher_forced(model, prompt, cont)
        model.free()
    for sched in (SIDE, DUAL, FUSED, PERSISTENT, LATE):
        for a, b in zip(outs[SERIAL], outs[sched]):
            assert np.array_equal(a, b), f"schedule {sched} differs from serial"


def test_large_batch_matches_oracle_and_rows(edge):
    """Batch 24 (beyond the K-sliced GEMV's 16 rows, so only the matrix-core decode route
    can take it): against the oracle, and the graph replays bit for bit equal to eager
    launches."""
    cfg, w = edge
    B = 24
    prompt = synth.gen_ids(B, 9, cfg.vocab, seed=21)
    cont = synth.gen_ids(B, 3, cfg.vocab, seed=21, stream=1)
    ref = oracle_record(cfg, w, prompt, 4, dtype=np.float64)
    res = []
    for g in (False, True):
        model = make_model(cfg, w, B, 16)
        model.set_schedule(FUSED, g)
        gl, gh, gt = gpu_teacher_forced(model, prompt, ref["tokens"][:, :-1])
        model.free()
        check_against_oracle(cfg, gl, gh, gt, ref, TOL["bf16"], f"edge B={B} graph={g}")
        res.append((gl, gh, gt))
    for a, b in zip(*res):
        assert np.array_equal(a, b), "graph replay differs from eager launches"


def test_graph_replay_matches_eager(edge):
    cfg, w = edge
    prompt = synth.gen_ids(2, 11, cfg.vocab, seed=8)
    cont = synth.gen_ids(2, 6, cfg.vocab, seed=8, stream=1)
    res = []
    for g in (False, True):
        model = make_model(cfg, w, 2, 24)
        model.set_schedule(FUSED, g)
        res.append(gpu_teacher_forced(model, prompt, cont))
        model.free()
    for a, b in zip(*res):
        assert np.array_equal(a, b)


def test_chunked_prefill_equals_prefill_then_decode(edge):
    """prefill(n) followed by single decode steps equals prefill(n+k) at the last position
    (both against the oracle), and a prefill that starts at start_pos > 0 continues the cache."""
    cfg, w = edge
    ids = synth.gen_ids(1, 24, cfg.vocab, seed=9)
    o = LadderOracle(cfg, w)
    ref = o.forward(ids)
    model = make_model(cfg, w, 1, 32)
    t = torch.from_numpy(ids).cuda()
    model.prefill(t[:, :16].contiguous())
    lg, nx, hd = model.prefill(t[:, 16:24].contiguous(), start_pos=16)
    torch.cuda.synchronize()
    assert rel_err(lg.cpu().numpy(), ref.logits[:, 23]) <= TOL["bf16"]
    assert rel_err(hd.cpu().numpy(), ref.hidden[:, 23]) <= TOL["bf16"]
    model.free()


def test_split_key_prefill_continuing_a_cache(edge):
    """A long prefill that continues an existing cache (start_pos 300, 1000 more tokens:
    its query tiles' keys are cut into chunks and merged) against the oracle at every
    position of the second chunk."""
    cfg, w = edge
    ids = synth.gen_ids(1, 1300, cfg.vocab, seed=17)
    ref = LadderOracle(cfg, w).forward(ids, logits="all")
    model = make_model(cfg, w, 1, 1310)
    t = torch.from_numpy(ids).cuda()
    model.prefill(t[:, :300].contiguous())
    lg, nx, hd = model.prefill(t[:, 300:].contiguous(), start_pos=300)
    torch.cuda.synchronize()
    log(f"split-key prefill: rel err logits {rel_err(lg.cpu().numpy(), ref.logits[:, 1299]):.3g}")
    assert rel_err(lg.cpu().numpy(), ref.logits[:, 1299]) <= TOL["bf16"]
    assert rel_err(hd.cpu().numpy(), ref.hidden[:, 1299]) <= TOL["bf16"]
    # the next decode step reads every cached key written by both prefills
    step = torch.from_numpy(synth.gen_ids(1, 1, cfg.vocab, seed=18)[:, 0].copy()).cuda()
    lg2, _, _ = model.decode_step(step, 1300)
    torch.cuda.synchronize()
    ids2 = np.concatenate([ids, step.cpu().numpy()[:, None].astype(ids.dtype)], axis=1)
    ref2 = LadderOracle(cfg, w).forward(ids2, logits="last")
    assert rel_err(lg2.cpu().numpy(), ref2.logits[:, -1]) <= TOL["bf16"]
    model.free()


def test_resume_on_existing_cache_is_bitwise(edge):
    """Prefill and two decode steps in one context, then a fresh context on the same KV
    cache (kv_filled) continues exactly like the uninterrupted one."""
    cfg, w = edge
    prompt = synth.gen_ids(1, 12, cfg.vocab, seed=10)
    cont = synth.gen_ids(1, 5, cfg.vocab, seed=10, stream=1)
    a = make_model(cfg, w, 1, 24)
    full = gpu_teacher_forced(a, prompt, cont)
    a.free()
    b = make_model(cfg, w, 1, 24)
    gpu_teacher_forced(b, prompt, cont[:, :2])
    kv = (b.k_cache, b.v_cache)
    c = make_model(cfg, w, 1, 24, kv=kv, kv_filled=12 + 2)
    outs = []
    for k in range(2, 5):
        lg, nx, hd = c.decode_step(torch.from_numpy(cont[:, k].copy()).cuda(), 12 + k)
        outs.append(lg)
    torch.cuda.synchronize()
    for k, lg in zip(range(2, 5), outs):
        assert np.array_equal(lg.cpu().numpy(), full[0][:, k + 1])
    b.free()
    c.free()


def test_error_paths_on_device(edge):
    from ladder_residual_transformer_amd import LadderError, abi
    cfg, w = edge
    m = make_model(cfg, w, 2, 16)
    ids1 = torch.zeros(1, dtype=torch.int32, device="cuda")
    with pytest.raises(LadderError) as e:
        m.decode_step(ids1, 3)                    # nothing prefilled yet
    assert e.value.status == abi.LADDER_ERR_STATE
    with pytest.raises(LadderError) as e:
        m.decode_step(torch.zeros(3, dtype=torch.int32, device="cuda"), 0)
    assert e.value.status == abi.LADDER_ERR_CAPACITY
    with pytest.raises(LadderError) as e:
        m.prefill(torch.zeros((1, 17), dtype=torch.int32, device="cuda"))
    assert e.value.status == abi.LADDER_ERR_CAPACITY
    m.prefill(torch.zeros((1, 16), dtype=torch.int32, device="cuda"))
    with pytest.raises(LadderError) as e:
        m.decode_step(ids1, 16)                   # pos == max_seq
    assert e.value.status == abi.LADDER_ERR_CAPACITY
    assert m.filled() == 16
    m.decode_step(ids1, 15)                       # rewriting the last position is allowed
    torch.cuda.synchronize()
    m.free()


def test_batch_rows_match_single_sequence(edge):
    cfg, w = edge
    prompt = synth.gen_ids(3, 10, cfg.vocab, seed=11)
    cont = synth.gen_ids(3, 3, cfg.vocab, seed=11, stream=1)
    m3 = make_model(cfg, w, 3, 16)
    l3 = gpu_teacher_forced(m3, prompt, cont)[0]
    m3.free()
    for b in range(3):
        m1 = make_model(cfg, w, 1, 16)
        l1 = gpu_teacher_forced(m1, prompt[b:b + 1], cont[b:b + 1])[0]
        m1.free()
        assert rel_err(l3[b], l1[0]) <= 2e-3


def test_kernel_tracing_keeps_results_and_counts_launches(edge):
    """Event-bracketed decode graphs give the same bits as plain ones and one timed
    launch per ladder layer for a fused kind (the standard layer 0 has none), under the
    default schedule and the one with the attention in the down projection's launch."""
    from ladder_residual_transformer_amd import LadderError, abi
    cfg, w = edge
    prompt = synth.gen_ids(1, 9, cfg.vocab, seed=12)
    cont = synth.gen_ids(1, 3, cfg.vocab, seed=12, stream=1)
    m = make_model(cfg, w, 1, 16)
    plain = gpu_teacher_forced(m, prompt, cont)
    m.free()
    m = make_model(cfg, w, 1, 16)
    with pytest.raises(LadderError) as e:
        m.trace_result()
    assert e.value.status == abi.LADDER_ERR_STATE
    m.trace_kernel("qkv_attn_gateup")
    traced = gpu_teacher_forced(m, prompt, cont)
    us, n = m.trace_result()
    assert n == sum(1 for v in cfg.ladder_mask if v) and us > 0.0
    m.trace_kernel("lmhead")
    m.decode_step(torch.from_numpy(cont[:, 0].copy()).cuda(), 9)
    us2, n2 = m.trace_result()
    assert n2 == 1 and us2 > 0.0
    m.free()
    for a, b in zip(plain, traced):
        assert np.array_equal(a, b)
    m = make_model(cfg, w, 1, 16)
    m.set_schedule(LATE, True)
    m.trace_kernel("qkv_gateup")
    late = gpu_teacher_forced(m, prompt, cont)
    us3, n3 = m.trace_result()
    assert n3 == sum(1 for v in cfg.ladder_mask if v) and us3 > 0.0
    m.free()
    for a, b in zip(plain, late):
        assert np.array_equal(a, b)


def test_matrix_core_layer_launch_is_traced_with_its_attention(edge):
    """Batch 5 decodes on the matrix cores: the first launch of each ladder layer is the
    skinny [QKV + RoPE/KV | attention | gate/up] launch, whose attention workgroups wait for
    the QKV tiles' progress words; it is traced as the qkv_attn_gateup kind once per ladder
    layer, no wait gives up (sync reports one that did), and tracing leaves every result
    unchanged."""
    cfg, w = edge
    B = 5
    prompt = synth.gen_ids(B, 9, cfg.vocab, seed=13)
    cont = synth.gen_ids(B, 3, cfg.vocab, seed=13, stream=1)
    m = make_model(cfg, w, B, 16)
    plain = gpu_teacher_forced(m, prompt, cont)
    m.free()
    m = make_model(cfg, w, B, 16)
    m.trace_kernel("qkv_attn_gateup")
    traced = gpu_teacher_forced(m, prompt, cont)
    us, n = m.trace_result()
    assert n == sum(1 for v in cfg.ladder_mask if v) and us > 0.0
    m.free()
    for a, b in zip(plain, traced):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("B", [33, 40, 64])
def test_tiled_paired_launches_match_module_order(B):
    """Batches 33-64 decode through the tiled split-K GEMMs (batch 33: 31 rows of
    padding in the 64-row tiles).  Under the fused schedule a
    ladder layer's [QKV | gate/up] run in one launch with one reduction (RMSNorm, RoPE + KV,
    SwiGLU) and [attention | down | O] in one launch (the O workgroups wait for the
    attention's signal) whose reduction writes both residual adds; module order (serial)
    launches the attention, each GEMM and its reduction alone.  The two must give the same
    bits (70B shard widths, two ladder layers, so that K splits), the paired launch must be
    traced once per layer, and tracing must leave every result unchanged."""
    cfg = synth.scaled_config(synth.CONFIGS["70b_tp8_shard"], 2)
    w = synth.gen_weights(cfg, seed=21)
    prompt = synth.gen_ids(B, 6, cfg.vocab, seed=22)
    cont = synth.gen_ids(B, 3, cfg.vocab, seed=22, stream=1)
    outs = {}
    for sched in (SERIAL, FUSED):
        model = make_model(cfg, w, B, 16)
        model.set_schedule(sched, True)
        outs[sched] = gpu_teacher_forced(model, prompt, cont)
        model.free()
    for a, b in zip(outs[SERIAL], outs[FUSED]):
        assert np.array_equal(a, b), "paired launches differ from module order"
    model = make_model(cfg, w, B, 16)
    model.trace_kernel("qkv_gateup")
    traced = gpu_teacher_forced(model, prompt, cont)
    us, n = model.trace_result()
    log(f"tiled pairs B={B}: qkv_gateup launch {us:.1f} us over {n} launches")
    assert n == cfg.n_layers and us > 0.0
    model.free()
    for a, b in zip(outs[FUSED], traced):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("B, T, max_seq, n_dec", [(2, 150, 256, 6), (1, 2100, 2200, 3)])
def test_long_context_split_kv(edge, B, T, max_seq, n_dec):
    """Decode attention over several key chunks (150 keys in 64-key chunks, merged across
    chunks) and over chunks of several tiles (2100 keys: 16 chunks of three tiles, the
    newest key in a later tile of the last chunk), against the oracle; and the default
    schedule (attention inside the fused launch) bit for bit against the serial one (the
    stand-alone attention kernel), which the tolerance alone would not see if one key
    were read wrongly."""
    cfg, w = edge
    prompt = synth.gen_ids(B, T, cfg.vocab, seed=13)
    cont = synth.gen_ids(B, n_dec, cfg.vocab, seed=13, stream=1)
    log(f"edge long context B={B} T={T} max_seq={max_seq}")
    ref = teacher_forced(LadderOracle(cfg, w), prompt, cont)
    outs = {}
    for sched in (FUSED, SERIAL):
        model = make_model(cfg, w, B, max_seq)
        model.set_schedule(sched, True)
        outs[sched] = gpu_teacher_forced(model, prompt, cont)
        model.free()
    gl, gh, _ = outs[FUSED]
    el = step_rel_err(gl, ref.logits[:, T - 1:])
    eh = step_rel_err(gh, ref.hidden[:, T - 1:])
    log(f"edge long context: rel err logits {el:.3g} hidden {eh:.3g}")
    assert el <= TOL["bf16"] and eh <= TOL["bf16"]
    for a, b in zip(outs[SERIAL], outs[FUSED]):
        assert np.array_equal(a, b), "fused schedule differs from serial"



def test_read_probe_reports_a_plausible_ceiling():
    """The streaming-read probe runs and reports a rate between 1 TB/s and the 8 TB/s peak."""
    from ladder_residual_transformer_amd import abi
    g = abi.ladder_read_probe(torch.cuda.current_stream().cuda_stream, 256 << 20, 2)
    log(f"streaming-read ceiling over 256 MiB: {g:.0f} GB/s")
    assert 1000.0 < g < 8000.0
