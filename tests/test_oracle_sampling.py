"""Pins of the oracle's stochastic sampling (oracle/sampling.py) against what the
generator's definition and the mathematics fix: the published known-answer vectors of
Philox4x32-10, the categorical distribution the Gumbel-max draw must follow, and the
special cases that reduce to greedy decoding."""
import os

import numpy as np
import pytest

from oracle.sampling import (philox4x32, sample_scores, sample_token, sampling_probs, sampling_uniforms,
                             topk_keep)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.txt")


def kat_rows():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                rows.append([int(x, 16) for x in line.split()])
    return rows


@pytest.mark.parametrize("row", kat_rows())
def test_philox_known_answers(row):
    c, k, want = row[:4], row[4:6], row[6:]
    got = [int(x) for x in philox4x32(*c, *k)]
    assert got == want, [hex(x) for x in got]


def test_uniforms_are_exact_and_inside_the_open_interval():
    u = sampling_uniforms(seed=12345, pos=7, b=1, V=4099)
    assert u.dtype == np.float32 and u.shape == (4099,)
    assert np.all(u > 0.0) and np.all(u < 1.0)
    # U = (2 (word >> 9) + 1) * 2^-24: an odd multiple of 2^-24, exact in float32
    scaled = u.astype(np.float64) * 2.0 ** 24
    assert np.array_equal(scaled, np.round(scaled)) and np.all(scaled.astype(np.int64) % 2 == 1)
    assert abs(float(u.mean()) - 0.5) < 0.02
    # a different position, sequence or seed gives different numbers
    assert not np.array_equal(u, sampling_uniforms(12345, 8, 1, 4099))
    assert not np.array_equal(u, sampling_uniforms(12345, 7, 0, 4099))
    assert not np.array_equal(u, sampling_uniforms(12346, 7, 1, 4099))


def draws(z, temperature, top_k, n, seed=99):
    """n seeded draws (positions 0..n-1, sequence 0) of logits z."""
    V = z.shape[0]
    pos = np.arange(n, dtype=np.uint64)
    n4 = (V + 3) // 4
    words = np.stack([np.stack(philox4x32(j, 0, pos, 0, seed, 0), axis=1) for j in range(n4)], axis=1)
    words = words.reshape(n, -1)[:, :V]
    u = ((words >> np.uint32(9)) * np.uint32(2) + np.uint32(1)).astype(np.float32) * np.float32(2.0 ** -24)
    keep = topk_keep(z.astype(np.float32), top_k)
    s = z.astype(np.float32)[None, :] / np.float32(temperature) - np.log(-np.log(u))
    s = np.where(keep[None, :], s, -np.inf)
    return np.argmax(s, axis=1)


@pytest.mark.parametrize("temperature, top_k", [(1.0, 0), (0.6, 0), (1.7, 3)])
def test_draws_follow_the_categorical_distribution(temperature, top_k):
    """Gumbel-max: frequencies of 60 000 seeded draws against softmax(z/T) over the kept
    logits (chi-square, far beyond the 1e-6 quantile would mean a wrong draw).  A dropped
    temperature, a flipped noise sign or a wrong cut all fail this."""
    z = np.array([0.3, -1.2, 2.0, 0.9, -0.4, 1.4], dtype=np.float32)
    n = 60000
    tok = draws(z, temperature, top_k, n)
    p = sampling_probs(z, temperature, top_k)
    counts = np.bincount(tok, minlength=z.size)
    assert np.all(counts[p == 0] == 0)
    kept = p > 0
    exp = p[kept] * n
    chi2 = float(((counts[kept] - exp) ** 2 / exp).sum())
    # chi-square with <= 5 degrees of freedom: P(chi2 > 40) < 1e-6
    assert chi2 < 40.0, (counts, exp, chi2)
    # and the temperature matters: the T=1 distribution does not fit the T=0.6 draws
    if temperature != 1.0:
        p1 = sampling_probs(z, 1.0, top_k)
        e1 = p1[kept] * n
        assert float(((counts[kept] - e1) ** 2 / e1).sum()) > 200.0


def test_single_draw_matches_the_vectorized_draws():
    z = np.array([0.3, -1.2, 2.0, 0.9, -0.4, 1.4], dtype=np.float32)
    tok = draws(z, 0.8, 4, 50)
    for pos in range(50):
        assert sample_token(z, 0.8, 4, sampling_uniforms(99, pos, 0, z.size)) == tok[pos]


def test_top1_and_cold_temperature_are_greedy():
    rng = np.random.default_rng(3)
    for pos in range(200):
        z = rng.normal(size=300).astype(np.float32)
        u = sampling_uniforms(7, pos, 0, 300)
        assert sample_token(z, 1.0, 1, u) == int(np.argmax(z))
        assert sample_token(z, 1e-6, 0, u) == int(np.argmax(z))


def test_topk_cut_keeps_ties_and_never_draws_outside():
    assert topk_keep(np.array([1, 3, 3, 2], np.float32), 2).tolist() == [False, True, True, False]
    assert topk_keep(np.array([3, 2, 2, 1], np.float32), 2).tolist() == [True, True, True, False]
    assert topk_keep(np.array([3, 2, 2, 1], np.float32), 0).all()
    assert topk_keep(np.array([3, 2, 2, 1], np.float32), 4).all()
    rng = np.random.default_rng(4)
    z = rng.normal(size=1000).astype(np.float32)
    top = set(np.argsort(-z)[:10].tolist())
    for pos in range(300):
        s = sample_scores(z, 3.0, 10, sampling_uniforms(11, pos, 2, 1000))
        assert int(np.argmax(s)) in top
        assert np.isneginf(s).sum() == 990
