"""The seeded input generator: reproducible, thread-count independent, correctly rounded."""
import numpy as np
import torch

import synth


def test_bf16_rounding_matches_torch_round_to_nearest_even():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(10000).astype(np.float32) * 0.02,
                        np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 3.0, 0.0, -0.0],
                                 dtype=np.float32)])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = synth.f32_to_bf16_bits(x)
    assert np.array_equal(got, want)
    assert got[-6] == 0x3F80 and got[-5] == 0x3F82      # ties go to even


def test_weights_reproducible_and_thread_independent():
    cfg = synth.ModelConfig("t", 2, 64, 4, 2, 16, 96, 50, 1e4, "bf16", (1, 1))
    a = synth.gen_weights(cfg, seed=3, threads=1)
    b = synth.gen_weights(cfg, seed=3, threads=4)
    c = synth.gen_weights(cfg, seed=4, threads=2)
    for name in synth.LayerWeights.FIELDS:
        assert np.array_equal(getattr(a.layers[1], name), getattr(b.layers[1], name))
    assert np.array_equal(a.lm_head, b.lm_head)
    assert not np.array_equal(a.layers[0].wq, c.layers[0].wq)
    assert not np.array_equal(a.layers[0].wq, a.layers[1].wq)
    assert a.layers[0].wq.dtype == np.uint16 and a.layers[0].wq.shape == (64, 64)
    assert np.all(a.layers[0].attn_norm == 0x3F80) and np.all(a.final_norm == 0x3F80)


def test_layer_subset_matches_full_generation():
    cfg = synth.ModelConfig("t", 3, 64, 4, 2, 16, 96, 50, 1e4, "f32", (1, 1, 1))
    full = synth.gen_weights(cfg, seed=5, threads=2)
    part = synth.gen_weights(cfg, seed=5, threads=2, layers=[2])
    assert part.layers[0] is None and part.layers[1] is None
    assert np.array_equal(full.layers[2].w_down, part.layers[2].w_down)


def test_distribution_and_ids():
    cfg = synth.ModelConfig("t", 1, 512, 4, 2, 128, 1024, 64, 1e4, "f32", (1,))
    w = synth.gen_weights(cfg, seed=0, threads=2)
    s = w.layers[0].w_gate.std()
    assert abs(s - 0.02) < 0.0005 and abs(w.layers[0].w_gate.mean()) < 0.0005
    ids = synth.gen_ids(4, 100, 1000, seed=1)
    assert ids.dtype == np.int32 and ids.shape == (4, 100)
    assert ids.min() >= 0 and ids.max() < 1000
    assert np.array_equal(ids, synth.gen_ids(4, 100, 1000, seed=1))
    assert not np.array_equal(ids, synth.gen_ids(4, 100, 1000, seed=1, stream=1))


def test_config_shapes():
    c = synth.CONFIGS["70b_tp8_shard"]
    assert c.weight_bytes() == 2 * (80 * (8192 * 1280 + 1024 * 8192 + 3 * 8192 * 3584 + 2 * 8192)
                                    + 2 * 16032 * 8192 + 8192)
    # a decode step reads one embedding row per sequence, not the table
    assert c.decode_weight_bytes(1) == c.weight_bytes() - 2 * 16031 * 8192
    assert synth.CONFIGS["8b_hybrid"].ladder_mask == tuple([0] * 16 + [1] * 16)
    assert synth.CONFIGS["8b_hybrid20"].ladder_mask == tuple([0] * 12 + [1] * 20)
    assert synth.scaled_config(c, 4).n_layers == 4
