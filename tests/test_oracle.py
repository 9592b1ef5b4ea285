"""Pins of the CPU oracle against things other than itself.

Each test fixes the oracle to a library routine, a closed form, an invariant
the pages imply, or a hand expansion of the ladder rule, so that a dropped
term, a wrong sign or index, or a transposed operand in ``oracle/`` fails at
least one of them.  CPU only.
"""
import dataclasses
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import synth
from oracle import (LadderOracle, apply_rope, gqa_attention, greedy_generate, llama3_scale_inv_freq,
                    module_input_index, rope_inv_freq,
                    rms_norm, rope_angles, round_to_storage, silu, swiglu_mlp, teacher_forced, upcast)

torch.set_default_dtype(torch.float64)


def small_cfg(mask=(1, 1), dtype="f32", H=64, nq=4, nkv=2, hd=16, F_=96, V=50, theta=1e4):
    return synth.ModelConfig("small", len(mask), H, nq, nkv, hd, F_, V, theta, dtype, tuple(mask))


def model(cfg, seed=0):
    return synth.gen_weights(cfg, seed=seed, threads=2)


# ---------------------------------------------------------------------------
# building blocks against library routines and closed forms
# ---------------------------------------------------------------------------

def test_upcast_bit_patterns():
    bits = np.array([0x3F80, 0xC000, 0x3F00, 0x0080, 0x0000, 0x8000, 0x4049], dtype=np.uint16)
    want = np.array([1.0, -2.0, 0.5, 2.0 ** -126, 0.0, -0.0, 3.140625])
    got = upcast(bits)
    assert np.array_equal(got, want)
    assert np.signbit(got[5])
    f = np.array([1.5, -3.25], dtype=np.float32)
    assert np.array_equal(upcast(f), f.astype(np.float64))


def test_round_to_storage_bf16_halfway_cases():
    e = 2.0 ** -8                                   # half a bf16 spacing in [1, 2)
    x = np.array([1 + e, 1 + 3 * e, -(1 + e), 1 + e + 2.0 ** -30, 1 - e / 2, 0.0,
                  2.0 ** -130 + 2.0 ** -134, 2.0 ** -130 + 3 * 2.0 ** -134, 3.0 * 2 ** 100])
    want = np.array([1.0, 1 + 4 * e, -1.0, 1 + 2 * e, 1.0, 0.0,
                     2.0 ** -130, 2.0 ** -130 + 2 * 2.0 ** -133, 3.0 * 2 ** 100])
    got = round_to_storage(x, "bf16")
    assert got.dtype == np.float64
    assert np.array_equal(got, want)


def test_round_to_storage_matches_bit_rounding_and_torch():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(20000) * np.exp2(rng.integers(-30, 30, 20000))).astype(np.float32)
    got = round_to_storage(x.astype(np.float64), "bf16")
    assert np.array_equal(got, upcast(synth.f32_to_bf16_bits(x)))            # bit-pattern RNE
    assert np.array_equal(got, torch.from_numpy(x).to(torch.bfloat16).double().numpy())
    y = rng.standard_normal(1000)
    assert np.array_equal(round_to_storage(y, "f32"), y.astype(np.float32).astype(np.float64))
    with pytest.raises(ValueError):
        round_to_storage(y, "fp8")


def test_kv_cache_holds_values_of_the_storage_type():
    """Layer 0's cached K/V are the unrounded ones rounded once; every cached value is
    a bf16 value; attention reads the cache (rounding changes the output)."""
    cfg = small_cfg(mask=(1, 0), dtype="bf16")
    w = model(cfg, seed=12)
    ids = synth.gen_ids(2, 7, cfg.vocab, seed=4)
    ca, cb = None, None
    oa, ob = LadderOracle(cfg, w), LadderOracle(cfg, w, kv_store_dtype=False)
    ca, cb = oa.new_cache(), ob.new_cache()
    ra, rb = oa.forward(ids, ca), ob.forward(ids, cb)
    for key in ("k", "v"):
        assert np.array_equal(ca[key][0], round_to_storage(cb[key][0], "bf16"))
        for li in range(cfg.n_layers):
            assert np.array_equal(ca[key][li], round_to_storage(ca[key][li], "bf16"))
    assert not np.array_equal(ra.hidden, rb.hidden)
    assert np.max(np.abs(ra.hidden - rb.hidden)) / np.max(np.abs(rb.hidden)) < 1e-2


def test_rms_norm_matches_torch_and_scale_invariance():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((3, 5, 40))
    g = rng.standard_normal(40)
    want = F.rms_norm(torch.from_numpy(x), (40,), torch.from_numpy(g), eps=1e-5).numpy()
    np.testing.assert_allclose(rms_norm(x, g, 1e-5), want, rtol=1e-13, atol=1e-13)
    # RMSNorm(c x) == RMSNorm(x) when eps is negligible against mean(x^2)
    np.testing.assert_allclose(rms_norm(7.5 * x, g, 0.0), rms_norm(x, g, 0.0), rtol=1e-12)
    # unit gain and a constant vector give all ones
    np.testing.assert_allclose(rms_norm(np.full((1, 8), 3.0), np.ones(8), 0.0), np.ones((1, 8)))


def test_rope_is_complex_phase_multiplication():
    """Adjacent pairs as complex numbers times e^{i p theta^{-2j/hd}} (torch.polar)."""
    rng = np.random.default_rng(1)
    hd, P, theta = 16, 9, 500.0
    x = rng.standard_normal((2, 3, P, hd))
    pos = np.arange(P) + 4
    freqs = 1.0 / (theta ** (torch.arange(0, hd, 2, dtype=torch.float64) / hd))
    ang = torch.outer(torch.from_numpy(pos).double(), freqs)
    phase = torch.polar(torch.ones_like(ang), ang)
    xc = torch.view_as_complex(torch.from_numpy(x).reshape(2, 3, P, hd // 2, 2).contiguous())
    want = torch.view_as_real(xc * phase).reshape(2, 3, P, hd).numpy()
    np.testing.assert_allclose(apply_rope(x, pos, theta), want, rtol=1e-12, atol=1e-12)
    assert rope_angles(np.array([3]), hd, theta).shape == (1, hd // 2)


def test_rope_properties():
    rng = np.random.default_rng(2)
    hd, theta = 32, 1e4
    x = rng.standard_normal((1, 1, 1, hd))
    assert np.array_equal(apply_rope(x, np.array([0]), theta), x)            # identity at p = 0
    y = apply_rope(np.repeat(x, 5, axis=2), np.arange(5) * 37, theta)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x), rtol=1e-12)
    q = rng.standard_normal(hd)
    k = rng.standard_normal(hd)

    def dot(p, s):
        qp = apply_rope(q[None, None, None, :], np.array([p]), theta)[0, 0, 0]
        ks = apply_rope(k[None, None, None, :], np.array([s]), theta)[0, 0, 0]
        return qp @ ks
    assert dot(9, 4) == pytest.approx(dot(105, 100), rel=1e-10)             # depends on p - s only
    assert dot(9, 4) != pytest.approx(dot(9, 5), rel=1e-3)


LLAMA31 = (8.0, 1.0, 4.0, 8192)   # factor, low_freq_factor, high_freq_factor, original context


def test_llama3_scaling_closed_forms():
    """At wavelengths below N/4 = 2048 a frequency is kept, above N = 8192 divided by 8;
    at w = N/2 = 4096 the blend weight is s = (2 - 1) / (4 - 1) = 1/3, so the frequency
    becomes (2/3) f / 8 + f / 3 = 5 f / 12.  A dropped 1/factor, swapped band limits or an
    inverted ratio w / N each break one of these."""
    w = np.array([100.0, 1000.0, 2047.0, 4096.0, 8193.0, 20000.0, 1e6])
    f = 2 * np.pi / w
    got = llama3_scale_inv_freq(f, *LLAMA31)
    want = np.array([f[0], f[1], f[2], 5 * f[3] / 12, f[4] / 8, f[5] / 8, f[6] / 8])
    np.testing.assert_allclose(got, want, rtol=1e-14)


def test_llama3_scaling_is_continuous_and_monotone():
    """The blend meets the kept band at w = N/4 and the divided band at w = N (relative
    jumps of order the step in w), and the scaled frequency falls monotonically with the
    wavelength while its ratio to f falls from 1 to 1/8."""
    for edge in (2048.0, 8192.0):
        w = np.array([edge * (1 - 1e-9), edge, edge * (1 + 1e-9)])
        g = llama3_scale_inv_freq(2 * np.pi / w, *LLAMA31)
        assert np.all(np.abs(np.diff(g)) <= 1e-8 * g[1])
    w = np.geomspace(10.0, 1e6, 20001)
    f = 2 * np.pi / w
    g = llama3_scale_inv_freq(f, *LLAMA31)
    assert np.all(np.diff(g) < 0)
    r = g / f
    assert np.all(np.diff(r) <= 1e-15) and r[0] == 1.0 and r[-1] == pytest.approx(1 / 8, rel=1e-15)


def test_llama3_scaling_on_a_llama31_head_and_identity_at_factor_1():
    """theta 5e5, head_dim 128 (wavelength of pair j: 2 pi 5e5^(j/64)): pairs 0..28 (up to
    1956.5) keep theta^(-2j/128), pairs 35..63 (from 8218.7) are divided by 8, pairs
    29..34 (2401.7 .. 6695.1) are blended; with
    factor 1 every pair keeps its frequency.  RoPE with scaled frequencies still
    preserves norms and depends only on p - s."""
    base = rope_inv_freq(128, 5e5)
    scaled = rope_inv_freq(128, 5e5, LLAMA31)
    wl = 2 * np.pi / base
    keep, div = wl < 2048, wl > 8192
    assert np.array_equal(np.flatnonzero(keep), np.arange(29))
    assert np.array_equal(np.flatnonzero(div), np.arange(35, 64))
    np.testing.assert_array_equal(scaled[keep], base[keep])
    np.testing.assert_allclose(scaled[div], base[div] / 8, rtol=1e-15)
    mid = ~keep & ~div
    assert np.all(scaled[mid] < base[mid]) and np.all(scaled[mid] > base[mid] / 8)
    np.testing.assert_allclose(rope_inv_freq(128, 5e5, (1.0, 1.0, 4.0, 8192)), base, rtol=1e-15)
    rng = np.random.default_rng(9)
    q, k = rng.standard_normal(128), rng.standard_normal(128)

    def dot(p, s):
        qp = apply_rope(q[None, None, None, :], np.array([p]), 5e5, LLAMA31)[0, 0, 0]
        ks = apply_rope(k[None, None, None, :], np.array([s]), 5e5, LLAMA31)[0, 0, 0]
        return qp @ ks
    assert dot(30, 7) == pytest.approx(dot(1030, 1007), rel=1e-10)
    y = apply_rope(q[None, None, None, :], np.array([777]), 5e5, LLAMA31)
    assert np.linalg.norm(y) == pytest.approx(np.linalg.norm(q), rel=1e-12)
    assert not np.allclose(y, apply_rope(q[None, None, None, :], np.array([777]), 5e5), atol=1e-3)


def test_attention_matches_sdpa_with_repeated_kv():
    rng = np.random.default_rng(3)
    B, nq, nkv, T, hd = 2, 6, 2, 7, 8
    q = rng.standard_normal((B, nq, T, hd))
    k = rng.standard_normal((B, nkv, T, hd))
    v = rng.standard_normal((B, nkv, T, hd))
    got = gqa_attention(q, k, v, np.arange(T), np.arange(T))
    kr = torch.from_numpy(k).repeat_interleave(nq // nkv, dim=1)
    vr = torch.from_numpy(v).repeat_interleave(nq // nkv, dim=1)
    want = F.scaled_dot_product_attention(torch.from_numpy(q), kr, vr, is_causal=True).numpy()
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)
    # queries at positions 4..6 against keys 0..6 (a chunk after a cached prefix)
    got_tail = gqa_attention(q[:, :, 4:], k, v, np.arange(4, 7), np.arange(T))
    np.testing.assert_allclose(got_tail, want[:, :, 4:], rtol=1e-12, atol=1e-12)


def test_attention_single_key_returns_value_exactly():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((1, 4, 1, 8))
    k = rng.standard_normal((1, 1, 1, 8))
    v = rng.standard_normal((1, 1, 1, 8))
    out = gqa_attention(q, k, v, np.array([0]), np.array([0]))
    assert np.array_equal(out, np.repeat(v, 4, axis=1))


def test_silu_and_swiglu():
    z = np.linspace(-20, 20, 101)
    np.testing.assert_allclose(silu(z), F.silu(torch.from_numpy(z)).numpy(), rtol=1e-13, atol=1e-300)
    assert silu(np.array([0.0]))[0] == 0.0
    assert silu(np.array([40.0]))[0] == pytest.approx(40.0, rel=1e-15)
    rng = np.random.default_rng(5)
    u = rng.standard_normal((3, 10))
    wg, wu, wd = rng.standard_normal((7, 10)), rng.standard_normal((7, 10)), rng.standard_normal((10, 7))
    tu = torch.from_numpy(u)
    want = F.linear(F.silu(F.linear(tu, torch.from_numpy(wg))) * F.linear(tu, torch.from_numpy(wu)),
                    torch.from_numpy(wd)).numpy()
    np.testing.assert_allclose(swiglu_mlp(u, wg, wu, wd), want, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# I1: no ladder layers -> the standard pre-norm Transformer (independent torch model)
# ---------------------------------------------------------------------------

def torch_standard_transformer(cfg, w, ids, parallel=False):
    """Textbook pre-norm Llama-style decoder in torch fp64, written independently of oracle/.

    parallel=True: GPT-J style parallel blocks, the MLP normalises the block input
    instead of the residual after the attention."""
    def t(a):
        return torch.from_numpy(upcast(a))
    nq, nkv, hd = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    ids_t = torch.from_numpy(np.asarray(ids, dtype=np.int64))
    B, T = ids_t.shape
    x = F.embedding(ids_t, t(w.tok_embed))
    freqs = 1.0 / (cfg.rope_theta ** (torch.arange(0, hd, 2, dtype=torch.float64) / hd))
    phase = torch.polar(torch.ones(T, hd // 2), torch.outer(torch.arange(T, dtype=torch.float64), freqs))

    def rot(z):                                              # z: [B, T, heads, hd]
        zc = torch.view_as_complex(z.reshape(*z.shape[:-1], hd // 2, 2).contiguous())
        return torch.view_as_real(zc * phase[None, :, None, :]).flatten(3)

    for lw in w.layers:
        x_block = x
        h = F.rms_norm(x, (cfg.hidden,), t(lw.attn_norm), eps=cfg.norm_eps)
        q = rot(F.linear(h, t(lw.wq)).view(B, T, nq, hd)).transpose(1, 2)
        k = rot(F.linear(h, t(lw.wk)).view(B, T, nkv, hd)).transpose(1, 2)
        v = F.linear(h, t(lw.wv)).view(B, T, nkv, hd).transpose(1, 2)
        k = k.repeat_interleave(nq // nkv, dim=1)
        v = v.repeat_interleave(nq // nkv, dim=1)
        o = F.scaled_dot_product_attention(q, k, v, is_causal=True).transpose(1, 2).reshape(B, T, nq * hd)
        x = x + F.linear(o, t(lw.wo))
        h = F.rms_norm(x_block if parallel else x, (cfg.hidden,), t(lw.mlp_norm), eps=cfg.norm_eps)
        x = x + F.linear(F.silu(F.linear(h, t(lw.w_gate))) * F.linear(h, t(lw.w_up)), t(lw.w_down))
    logits = F.linear(F.rms_norm(x, (cfg.hidden,), t(w.final_norm), eps=cfg.norm_eps), t(w.lm_head))
    return x.numpy(), logits.numpy()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_zero_ladder_equals_standard_transformer(dtype):
    cfg = small_cfg(mask=(0, 0, 0), dtype=dtype)
    w = model(cfg, seed=11)
    ids = synth.gen_ids(2, 9, cfg.vocab, seed=3)
    r = LadderOracle(cfg, w, kv_store_dtype=False).forward(ids)
    hx, lg = torch_standard_transformer(cfg, w, ids)
    np.testing.assert_allclose(r.hidden, hx, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(r.logits, lg, rtol=1e-10, atol=1e-12)


def test_zero_ladder_equals_standard_transformer_tiny_shape():
    cfg = synth.CONFIGS["tiny"].with_mask((0, 0))
    w = synth.gen_weights(cfg, seed=0, threads=2)
    ids = synth.gen_ids(1, 16, cfg.vocab, seed=1)
    r = LadderOracle(cfg, w, kv_store_dtype=False).forward(ids)
    hx, lg = torch_standard_transformer(cfg, w, ids)
    np.testing.assert_allclose(r.hidden, hx, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(r.logits, lg, rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_all_parallel_equals_textbook_parallel_transformer(dtype):
    cfg = small_cfg(mask=(2, 2, 2), dtype=dtype)
    w = model(cfg, seed=17)
    ids = synth.gen_ids(2, 9, cfg.vocab, seed=8)
    r = LadderOracle(cfg, w, kv_store_dtype=False).forward(ids)
    hx, lg = torch_standard_transformer(cfg, w, ids, parallel=True)
    np.testing.assert_allclose(r.hidden, hx, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(r.logits, lg, rtol=1e-10, atol=1e-12)
    # and the textbook parallel model is not the sequential one on these weights
    hs, _ = torch_standard_transformer(cfg, w, ids)
    assert np.max(np.abs(hx - hs)) > 1e-6


def test_ladder_differs_from_standard():
    cfg = small_cfg(mask=(1, 1))
    w = model(cfg, seed=12)
    ids = synth.gen_ids(1, 5, cfg.vocab, seed=4)
    a = LadderOracle(cfg, w).forward(ids).hidden
    b = LadderOracle(cfg, w, ladder_mask=(0, 0)).forward(ids).hidden
    assert np.max(np.abs(a - b)) > 1e-6


# ---------------------------------------------------------------------------
# the ladder rule: hand expansion, sum invariant, zero weights, closed forms
# ---------------------------------------------------------------------------

def _module_fns(cfg, w):
    """Stand-alone A_l(x), M_l(x) on a whole sequence from position 0 (fresh cache each call)."""
    o = LadderOracle(cfg, w)

    def A(li, x):
        return o.attention(li, x, o.new_cache(), 0)

    def M(li, x):
        return o.mlp(li, x)
    return o, A, M


@pytest.mark.parametrize("mask", [(a, b) for a in (0, 1, 2) for b in (0, 1, 2)])
def test_two_layer_brute_force_all_masks(mask):
    cfg = small_cfg(mask=mask)
    w = model(cfg, seed=13)
    ids = synth.gen_ids(2, 6, cfg.vocab, seed=5)
    o, A, M = _module_fns(cfg, w)
    x0 = o.embed(ids)
    # written out by hand from x_{i+1} = h_{i+1}(x_{i-1}) + x_i (ladder, 1),
    # x_{i+1} = h_{i+1}(x_i) + x_i (standard, 0), with x_{-1} = x_0, and the parallel
    # block (2) x_{2l+2} = x_{2l} + A(x_{2l}) + M(x_{2l})
    x1 = x0 + A(0, x0)
    x2 = x1 + {0: M(0, x1), 1: M(0, x0), 2: M(0, x0)}[mask[0]]
    x3 = x2 + {0: A(1, x2), 1: A(1, x1), 2: A(1, x2)}[mask[1]]
    x4 = x3 + {0: M(1, x3), 1: M(1, x2), 2: M(1, x2)}[mask[1]]
    r = o.forward(ids, record=True)
    np.testing.assert_array_equal(r.hidden, x4)
    np.testing.assert_array_equal(r.residuals[2], x2)
    per_layer = {0: lambda l: [2 * l, 2 * l + 1], 1: lambda l: [max(2 * l - 1, 0), 2 * l],
                 2: lambda l: [2 * l, 2 * l]}
    assert [module_input_index(m, mask) for m in range(4)] == per_layer[mask[0]](0) + per_layer[mask[1]](1)


@pytest.mark.parametrize("rest", [(0,), (1,), (2,), (2, 1)])
def test_parallel_first_layer_equals_ladder_first_layer(rest):
    """At layer 0 the ladder rule's x_{-1} = x_0 makes both modules read x_0, which is
    exactly the parallel block."""
    cfg = small_cfg(mask=(1,) + rest)
    w = model(cfg, seed=18)
    ids = synth.gen_ids(2, 5, cfg.vocab, seed=9)
    a = LadderOracle(cfg, w).forward(ids)
    b = LadderOracle(cfg, w, ladder_mask=(2,) + rest).forward(ids)
    np.testing.assert_array_equal(a.hidden, b.hidden)
    np.testing.assert_array_equal(a.logits, b.logits)


def test_parallel_block_closed_form_in_mixed_stack():
    """x_{2l+2} = x_{2l} + A_l(x_{2l}) + M_l(x_{2l}) for every parallel layer of a mixed
    stack; the ladder and standard layers around it leave it whole."""
    mask = (0, 2, 1, 2)
    cfg = small_cfg(mask=mask)
    w = model(cfg, seed=19)
    ids = synth.gen_ids(1, 6, cfg.vocab, seed=10)
    o, A, M = _module_fns(cfg, w)
    r = o.forward(ids, record=True)
    xs = r.residuals
    for l in (1, 3):
        xin = xs[2 * l]
        np.testing.assert_allclose(xs[2 * l + 2], xin + A(l, xin) + M(l, xin), rtol=1e-13, atol=1e-14)
    # the ladder layer 2 reads x_3 and x_4: not the parallel closed form
    assert np.max(np.abs(xs[6] - (xs[4] + A(2, xs[4]) + M(2, xs[4])))) > 1e-8


def test_mask_values_beyond_parallel_rejected():
    cfg = small_cfg(mask=(1, 1))
    w = model(cfg, seed=20)
    with pytest.raises(ValueError):
        LadderOracle(cfg, w, ladder_mask=(1, 3))
    with pytest.raises(ValueError):
        cfg.with_mask((0, 3))


@pytest.mark.parametrize("mask", [(1, 1, 1), (0, 1, 1), (1, 0, 1), (0, 0, 0), (2, 2, 2), (0, 2, 1)])
def test_sum_invariant(mask):
    """The stream accumulates every module output: x_{2L} = x_0 + sum_m out_m."""
    cfg = small_cfg(mask=mask)
    w = model(cfg, seed=14)
    ids = synth.gen_ids(1, 5, cfg.vocab, seed=6)
    r = LadderOracle(cfg, w).forward(ids, record=True)
    total = r.residuals[0] + sum(r.module_outputs)
    np.testing.assert_allclose(r.hidden, total, rtol=1e-13, atol=1e-14)
    for m, out in enumerate(r.module_outputs):
        np.testing.assert_array_equal(r.residuals[m + 1], r.residuals[m] + out)


@pytest.mark.parametrize("mask", [(1, 1), (0, 1), (0, 0)])
def test_zero_output_matrices_leave_residual_unchanged(mask):
    cfg = small_cfg(mask=mask, dtype="bf16")
    w = model(cfg, seed=15)
    for lw in w.layers:
        lw.wo[:] = 0
        lw.w_down[:] = 0
    ids = synth.gen_ids(2, 4, cfg.vocab, seed=7)
    o = LadderOracle(cfg, w)
    r = o.forward(ids, record=True)
    assert np.array_equal(r.hidden, o.embed(ids))
    for out in r.module_outputs:
        assert not np.any(out)


def test_zeroing_one_module_matrix_zeroes_that_output_only():
    cfg = small_cfg(mask=(1, 1))
    w = model(cfg, seed=16)
    w.layers[1].wo[:] = 0                                    # module m = 2
    r = LadderOracle(cfg, w).forward(synth.gen_ids(1, 5, cfg.vocab, seed=8), record=True)
    assert not np.any(r.module_outputs[2])
    assert all(np.any(r.module_outputs[m]) for m in (0, 1, 3))


def test_one_ladder_layer_is_parallel_block():
    """With one ladder layer both modules read x_0: x_2 = x_0 + A(x_0) + M(x_0)."""
    cfg = small_cfg(mask=(1,))
    w = model(cfg, seed=17)
    ids = synth.gen_ids(2, 7, cfg.vocab, seed=9)
    o, A, M = _module_fns(cfg, w)
    x0 = o.embed(ids)
    np.testing.assert_allclose(o.forward(ids).hidden, x0 + A(0, x0) + M(0, x0), rtol=1e-14, atol=1e-15)


# ---------------------------------------------------------------------------
# decoding consistency
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("mask", [(1, 1), (0, 1)])
def test_decode_equals_prefill(mask):
    cfg = small_cfg(mask=mask)
    w = model(cfg, seed=18)
    ids = synth.gen_ids(2, 8, cfg.vocab, seed=10)
    o = LadderOracle(cfg, w)
    full = o.forward(ids)
    cache = o.new_cache()
    o.forward(ids[:, :5], cache, 0)
    o.forward(ids[:, 5:7], cache, 5)                         # a two-token chunk
    step = o.forward(ids[:, 7:8], cache, 7)                  # a single decode step
    np.testing.assert_allclose(step.logits[:, 0], full.logits[:, 7], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(step.hidden[:, 0], full.hidden[:, 7], rtol=1e-10, atol=1e-12)


def test_batch_rows_are_independent():
    cfg = small_cfg(mask=(1, 0))
    w = model(cfg, seed=19)
    ids = synth.gen_ids(3, 6, cfg.vocab, seed=11)
    o = LadderOracle(cfg, w)
    full = o.forward(ids)
    for b in range(3):
        one = o.forward(ids[b:b + 1])
        np.testing.assert_allclose(one.logits[0], full.logits[b], rtol=1e-12, atol=1e-13)


def test_greedy_generate_is_argmax_of_teacher_forced_logits():
    cfg = small_cfg(mask=(1, 1))
    w = model(cfg, seed=20)
    prompt = synth.gen_ids(2, 5, cfg.vocab, seed=12)
    g = greedy_generate(LadderOracle(cfg, w), prompt, 6)
    assert g["tokens"].shape == (2, 7)
    tf = teacher_forced(LadderOracle(cfg, w), prompt, g["tokens"][:, :-1])
    np.testing.assert_array_equal(np.argmax(tf.logits[:, 4:], axis=-1), g["tokens"])
    np.testing.assert_allclose(g["logits"], tf.logits[:, 4:], rtol=1e-10, atol=1e-12)
    assert np.all(g["margins"] >= 0)


def test_argmax_takes_lowest_index_on_ties():
    from oracle.ladder import _top2_margin
    idx, mar = _top2_margin(np.array([[1.0, 3.0, 3.0, 2.0], [0.0, -1.0, 5.0, 4.5]]))
    assert idx.tolist() == [1, 2]
    assert mar.tolist() == [0.0, 0.5]


# ---------------------------------------------------------------------------
# I12: one rank's shard -- rank outputs sum to the unsharded module
# ---------------------------------------------------------------------------

def test_simulated_tensor_parallel_shards_sum_to_full_module():
    """Column-split QKV / gate / up by heads and ffn, row-split O / down: the
    per-rank partial outputs (what an all-reduce would sum) add up to the
    unsharded module output.  This is the reading under which one rank's
    shard, with identity in place of the all-reduce, is the workload."""
    ranks = 2
    cfg = small_cfg(mask=(1,), H=64, nq=4, nkv=2, hd=16, F_=96)
    w = model(cfg, seed=21)
    ids = synth.gen_ids(1, 6, cfg.vocab, seed=13)
    o = LadderOracle(cfg, w)
    x = o.embed(ids)
    full_a = o.attention(0, x, o.new_cache(), 0)
    full_m = o.mlp(0, x)
    lw = w.layers[0]
    qs, kvs, fs = cfg.n_q_heads // ranks * cfg.head_dim, cfg.n_kv_heads // ranks * cfg.head_dim, cfg.ffn // ranks
    sum_a = 0
    sum_m = 0
    for r in range(ranks):
        shard_cfg = dataclasses.replace(cfg, n_q_heads=cfg.n_q_heads // ranks,
                                        n_kv_heads=cfg.n_kv_heads // ranks, ffn=fs)
        sl = synth.LayerWeights(lw.attn_norm, lw.wq[r * qs:(r + 1) * qs], lw.wk[r * kvs:(r + 1) * kvs],
                                lw.wv[r * kvs:(r + 1) * kvs], np.ascontiguousarray(lw.wo[:, r * qs:(r + 1) * qs]),
                                lw.mlp_norm, lw.w_gate[r * fs:(r + 1) * fs], lw.w_up[r * fs:(r + 1) * fs],
                                np.ascontiguousarray(lw.w_down[:, r * fs:(r + 1) * fs]))
        ws = synth.ModelWeights(w.dtype, w.tok_embed, w.final_norm, w.lm_head, [sl])
        os_ = LadderOracle(shard_cfg, ws)
        sum_a = sum_a + os_.attention(0, x, os_.new_cache(), 0)
        sum_m = sum_m + os_.mlp(0, x)
    np.testing.assert_allclose(sum_a, full_a, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(sum_m, full_m, rtol=1e-12, atol=1e-14)


def test_float32_mode_tracks_float64():
    cfg = small_cfg(mask=(1, 1), dtype="bf16")
    w = model(cfg, seed=22)
    ids = synth.gen_ids(1, 6, cfg.vocab, seed=14)
    a = LadderOracle(cfg, w, dtype=np.float32).forward(ids)
    b = LadderOracle(cfg, w).forward(ids)
    assert a.hidden.dtype == np.float32
    assert np.max(np.abs(a.logits - b.logits)) / np.max(np.abs(b.logits)) < 1e-5
