"""Stochastic next-token sampling (test infrastructure).

Source: the codewithpapers record of the pages (arXiv 2501.06589) lists, among the
functions of the method's released inference benchmark, ``logits_to_probs``,
``multinomial_sample_one_no_sync`` and ``sample``.  The pages give their names only.
Reading (the plainest one the names support; listed with its reason in the design
notes of the repository):

  * ``logits_to_probs``: the last position's logits are divided by a temperature T > 0;
    optionally only the top-k logits are kept (every logit >= the k-th largest one, so
    ties at the cut are kept); the kept ones are turned into probabilities by a softmax;
  * ``multinomial_sample_one_no_sync``: one token is drawn from those probabilities
    without a host synchronisation.  Read as the exponential race: with E_i ~ Exp(1)
    independent, argmax_i p_i / E_i is distributed as the categorical p.  Taking logs,
    that is argmax_i (z_i / T + G_i) over the kept i, with G_i = -log(E_i) = -log(-log U_i)
    Gumbel noise from uniforms U_i (the softmax normaliser cancels);
  * ``sample``: the two together for the last position of each sequence.

The uniforms come from a counter-based generator so that a draw is a pure function of
(seed, position, sequence, vocabulary index): Philox4x32 with 10 rounds (Salmon, Moraes,
Dror and Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC 2011), written here
from its published definition.  Counter (i // 4, b, pos, 0), key (seed low word, seed
high word); vocabulary entry i takes output word i % 4, and U = (2 (word >> 9) + 1) / 2^24,
an odd multiple of 2^-24: an exact float32 strictly inside (0, 1).

Pins (tests/test_oracle_sampling.py): the generator against the published known-answer
vectors; the Gumbel-max draw against the categorical distribution it must follow (many
seeded draws on a small vocabulary, chi-square bound); top-k = 1 and a vanishing
temperature reduce to greedy argmax; tokens outside the top k are never drawn.
"""
from __future__ import annotations

import numpy as np

# Philox4x32 constants from the published definition: round multipliers and the Weyl
# sequence that bumps the key between rounds.
PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
_MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32(c0, c1, c2, c3, k0, k1, rounds: int = 10):
    """Philox4x32-R on arrays of counters (uint32 values, any broadcastable shapes).

    One round: (hi0, lo0) = M0 * c0 and (hi1, lo1) = M1 * c2 as 64-bit products, then
    (c0, c1, c2, c3) <- (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0); the key is bumped by
    the Weyl constants before every round but the first.  Returns four uint32 arrays.
    Pin: the published known-answer vectors.
    """
    c = [np.asarray(x, dtype=np.uint64) & _MASK32 for x in (c0, c1, c2, c3)]
    k = [np.asarray(x, dtype=np.uint64) & _MASK32 for x in (k0, k1)]
    for r in range(rounds):
        if r > 0:
            k = [(k[0] + np.uint64(PHILOX_W0)) & _MASK32, (k[1] + np.uint64(PHILOX_W1)) & _MASK32]
        p0 = np.uint64(PHILOX_M0) * c[0]
        p1 = np.uint64(PHILOX_M1) * c[2]
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK32
        c = [hi1 ^ c[1] ^ k[0], lo1, hi0 ^ c[3] ^ k[1], lo0]
    return [x.astype(np.uint32) for x in c]


def sampling_uniforms(seed: int, pos: int, b: int, V: int) -> np.ndarray:
    """float32 [V]: the uniform of vocabulary entry i for sequence b at position pos.

    Counter (i // 4, b, pos, 0), key (seed & 0xffffffff, seed >> 32), word i % 4,
    U = (2 (word >> 9) + 1) * 2^-24 (exact in float32, strictly inside (0, 1)).
    """
    n4 = (V + 3) // 4
    j = np.arange(n4, dtype=np.uint64)
    w = philox4x32(j, b, pos, 0, seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)
    words = np.stack(w, axis=1).reshape(-1)[:V]
    return ((words >> np.uint32(9)) * np.uint32(2) + np.uint32(1)).astype(np.float32) * np.float32(2.0 ** -24)


def topk_keep(z: np.ndarray, top_k: int) -> np.ndarray:
    """Boolean [V]: the logits kept by a top-k cut (every z_i >= the k-th largest z);
    all of them when top_k <= 0 or top_k >= V."""
    V = z.shape[-1]
    if top_k <= 0 or top_k >= V:
        return np.ones(V, dtype=bool)
    kth = np.sort(z)[::-1][top_k - 1]
    return z >= kth


def sampling_probs(logits: np.ndarray, temperature: float, top_k: int) -> np.ndarray:
    """float64 [V]: softmax(z / T) over the kept logits, 0 elsewhere (the distribution a
    draw follows)."""
    z = np.asarray(logits, dtype=np.float64)
    keep = topk_keep(np.asarray(logits, dtype=np.float32), top_k)
    s = np.where(keep, z / temperature, -np.inf)
    s = s - s.max()
    p = np.exp(s)
    return p / p.sum()


def sample_scores(logits: np.ndarray, temperature: float, top_k: int, u: np.ndarray) -> np.ndarray:
    """float32 [V]: z_i / T + G_i with G_i = -log(-log U_i) on the kept entries, -inf on
    the others.  All arithmetic in float32 (the precision the draw is decided in)."""
    z = np.asarray(logits, dtype=np.float32)
    keep = topk_keep(z, top_k)
    g = -np.log(-np.log(u.astype(np.float32)))
    s = z / np.float32(temperature) + g
    return np.where(keep, s, np.float32(-np.inf)).astype(np.float32)


def sample_token(logits: np.ndarray, temperature: float, top_k: int, u: np.ndarray) -> int:
    """The drawn token: argmax of ``sample_scores`` (lowest index on exact ties)."""
    return int(np.argmax(sample_scores(logits, temperature, top_k, u)))


def sample_rows(logits: np.ndarray, temperature: float, top_k: int, seed: int, pos: int) -> np.ndarray:
    """int64 [B]: the draw of every batch row b of logits [B][V] at position pos."""
    B, V = logits.shape
    return np.array([sample_token(logits[b], temperature, top_k, sampling_uniforms(seed, pos, b, V))
                     for b in range(B)], dtype=np.int64)
