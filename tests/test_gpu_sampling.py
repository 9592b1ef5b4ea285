"""HIP sampling path vs the oracle's draw (oracle/sampling.py), through the C ABI.

The draw is decided in float32 on both sides from the same Philox uniforms; the two
implementations of log may differ in the last bit, so a token may legitimately differ
where the oracle's two best Gumbel scores are within a few ulps of each other (a near
tie): every other draw must be identical, and every GPU token must lie in the kept set.
The logits fed to the context-free draw are seeded test inputs; in the model tests both
sides draw from their own logits (teacher forcing with the oracle's tokens).
"""
import numpy as np
import pytest
import torch

import synth
from gpu_helpers import gpu_teacher_forced, log, make_model
from oracle import LadderOracle, teacher_forced
from oracle.sampling import sample_rows, sample_scores, sampling_uniforms, topk_keep

pytestmark = pytest.mark.gpu


def check_draws(gpu, logits, temperature, top_k, seed, pos, margin):
    """gpu [B] tokens against the oracle's draws of logits [B][V]; returns the number of
    near-tie disagreements (allowed when the oracle's scores of the two tokens differ by at
    most `margin`)."""
    B, V = logits.shape
    ref = sample_rows(logits, temperature, top_k, seed, pos)
    flips = 0
    for b in range(B):
        g, r = int(gpu[b]), int(ref[b])
        assert 0 <= g < V
        assert topk_keep(logits[b].astype(np.float32), top_k)[g], f"token {g} outside the top {top_k}"
        if g != r:
            s = sample_scores(logits[b], temperature, top_k, sampling_uniforms(seed, pos, b, V))
            assert s[r] - s[g] <= margin, (b, g, r, float(s[r] - s[g]))
            flips += 1
    return flips


@pytest.mark.parametrize("B, V", [(1, 16032), (4, 1001), (3, 128256), (16, 8016), (2, 5)])
def test_draw_matches_oracle(B, V):
    rng = np.random.default_rng(V + B)
    logits = (rng.standard_normal((B, V)) * 1.5).astype(np.float32)
    # ties at a top-k cut: copy the 3rd largest value of each row into two more entries
    for b in range(B):
        order = np.argsort(-logits[b])
        if V > 8:
            logits[b, order[5]] = logits[b, order[6]] = logits[b, order[2]]
    ld = V + 3                                          # a row pitch wider than V
    buf = np.zeros((B, ld), np.float32)
    buf[:, :V] = logits
    d_logits = torch.from_numpy(buf).cuda()
    d_next = torch.empty(B, dtype=torch.int32, device="cuda")
    from ladder_residual_transformer_amd import abi
    flips = total = 0
    for temperature in (0.7, 1.3):
        for top_k in sorted({0, 1, 3, 40, V - 1, V}):
            for pos in (0, 1, 77, 4095):
                seed = 0x1234_5678_9ABC + pos
                abi.ladder_sample(d_logits.data_ptr(), B, V, ld, temperature, top_k, seed, pos, d_next.data_ptr())
                torch.cuda.synchronize()
                got = d_next.cpu().numpy()
                flips += check_draws(got, logits, temperature, top_k, seed, pos, margin=1e-5)
                total += B
    log(f"draws B={B} V={V}: {total} draws, {flips} near-tie disagreements")
    assert flips <= max(1, total // 500)


def test_draws_are_stochastic_and_greedy_at_top1():
    """Different positions draw different tokens (not the argmax every time); top-k 1 is
    the argmax."""
    from ladder_residual_transformer_amd import abi
    rng = np.random.default_rng(5)
    logits = rng.standard_normal((1, 1000)).astype(np.float32)
    d_logits = torch.from_numpy(logits).cuda()
    d_next = torch.empty(1, dtype=torch.int32, device="cuda")
    seen = set()
    for pos in range(64):
        abi.ladder_sample(d_logits.data_ptr(), 1, 1000, 1000, 2.0, 0, 7, pos, d_next.data_ptr())
        torch.cuda.synchronize()
        seen.add(int(d_next.cpu()[0]))
        abi.ladder_sample(d_logits.data_ptr(), 1, 1000, 1000, 2.0, 1, 7, pos, d_next.data_ptr())
        torch.cuda.synchronize()
        assert int(d_next.cpu()[0]) == int(np.argmax(logits[0]))
    assert len(seen) > 20


@pytest.mark.parametrize("use_graph", [False, True])
def test_tiny_decode_with_sampling_matches_oracle(use_graph):
    """fp32 tiny model, teacher forcing: the prefill's and every decode step's draw equal
    the oracle's draw from its own logits at the same position; with sampling switched
    off again the tokens are greedy."""
    cfg = synth.CONFIGS["tiny"]
    w = synth.gen_weights(cfg, seed=0)
    prompt = synth.gen_ids(2, 12, cfg.vocab, seed=31)
    cont = synth.gen_ids(2, 8, cfg.vocab, seed=31, stream=1)
    T = prompt.shape[1]
    ref = teacher_forced(LadderOracle(cfg, w), prompt, cont)
    model = make_model(cfg, w, 2, 32)
    model.set_schedule(3, use_graph)
    temperature, top_k, seed = 0.9, 20, 2024
    model.set_sampling(temperature, top_k, seed)
    gl, gh, gt = gpu_teacher_forced(model, prompt, cont)
    flips = 0
    for k in range(cont.shape[1] + 1):
        pos = T - 1 + k
        flips += check_draws(gt[:, k], ref.logits[:, pos].astype(np.float32), temperature, top_k, seed, pos, 1e-4)
    assert flips == 0
    model.set_sampling(0.0)
    gl2, _, gt2 = gpu_teacher_forced(model, prompt, cont)
    model.free()
    assert np.array_equal(gt2, np.argmax(gl2, axis=-1))
    assert np.array_equal(gl, gl2)                     # the logits do not depend on the rule


def test_bf16_decode_with_sampling_matches_oracle():
    """bf16 edge-shaped model, batch 3, the default schedule: draws equal the oracle's
    except where the oracle's two scores are closer than the logits' measured error allows."""
    cfg = synth.ModelConfig("edge_s", 3, 2112, 6, 2, 64, 1344, 1001, 1e4, "bf16", (0, 1, 1))
    w = synth.gen_weights(cfg, seed=3)
    prompt = synth.gen_ids(3, 17, cfg.vocab, seed=32)
    cont = synth.gen_ids(3, 6, cfg.vocab, seed=32, stream=1)
    T = prompt.shape[1]
    ref = teacher_forced(LadderOracle(cfg, w), prompt, cont)
    model = make_model(cfg, w, 3, 32)
    temperature, top_k, seed = 0.8, 0, 99
    model.set_sampling(temperature, top_k, seed)
    gl, _, gt = gpu_teacher_forced(model, prompt, cont)
    model.free()
    ref_l = ref.logits[:, T - 1:]
    err = float(np.max(np.abs(gl - ref_l)))
    margin = 2.0 * err / temperature + 1e-5
    flips = 0
    for k in range(cont.shape[1] + 1):
        flips += check_draws(gt[:, k], ref_l[:, k].astype(np.float32), temperature, top_k, seed, T - 1 + k, margin)
    log(f"bf16 sampling: max logit error {err:.3g}, {flips} near-tie disagreements of {gt.size}")
    assert flips <= 2
