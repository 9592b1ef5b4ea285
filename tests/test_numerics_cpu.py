"""Number formats the GPU path relies on, emulated on the CPU.

The GEMMs on the matrix cores (prefill projections, decode at batch > 4) carry each fp32
activation a as a bf16 pair hi = bf16(a), lo = bf16(a - hi); the decode route folds
RMSNorm into those GEMMs by feeding the raw residual times the gain through such pairs,
so the pair's range is that path's range.  The attention kernels carry q and the softmax
probabilities as fp16 pairs hi = fp16(a), lo = fp16(a - hi) (numpy's IEEE fp16).
"""
import numpy as np


def to_bf16(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even), returned as fp32: the top 16 bits of the
    fp32 encoding after adding half an ulp of bf16 plus the kept bit's parity."""
    u = np.asarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return r.astype(np.uint32).view(np.float32)


def split_bf_pair(a: np.ndarray):
    a = np.asarray(a, dtype=np.float32)
    hi = to_bf16(a)
    return hi, to_bf16(a - hi)


def split_pair(a: np.ndarray):
    a = np.asarray(a, dtype=np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        hi = a.astype(np.float16)
        lo = (a - hi.astype(np.float32)).astype(np.float16)
    return hi, lo


def test_bf16_rounding_matches_known_values():
    """1 + 2^-8 is a tie between 1 and 1 + 2^-7 and goes to the even 1; 1 + 3*2^-8 goes
    up to 1 + 2^-6; the largest finite fp32 rounds to infinity; small integers stay."""
    a = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 1 + 2.0 ** -8 + 2.0 ** -20, 255.0, -3.0],
                 dtype=np.float32)
    assert to_bf16(a).tolist() == [1.0, 1 + 2.0 ** -6, 1 + 2.0 ** -7, 255.0, -3.0]
    with np.errstate(over="ignore"):
        assert np.isinf(to_bf16(np.array([np.finfo(np.float32).max], np.float32)))[0]


def test_bf16_pair_holds_fp32_values_over_fp32_range():
    """From 2^-100 to 2^100 the pair reproduces an fp32 value to about 16 significant
    bits: hi rounds to 8 bits (error at most half of bf16's spacing, 2^-8 |a|), a - hi
    is exact in fp32 and lo rounds it to 8 bits (error at most 2^-8 |a - hi|, so
    2^-16 |a|)."""
    rng = np.random.default_rng(0)
    a = (2.0 ** rng.uniform(-100, 100, 200_000)).astype(np.float32)
    a *= rng.choice([-1.0, 1.0], a.size).astype(np.float32)
    hi, lo = split_bf_pair(a)
    back = hi.astype(np.float64) + lo.astype(np.float64)
    rel = np.abs(back - a) / np.abs(a)
    assert rel.max() <= 2.0 ** -16
    assert rel.max() > 2.0 ** -18                      # not fp32-exact: 16 bits, not 24
    assert np.all(np.abs(lo.astype(np.float64)) <= np.abs(hi.astype(np.float64)) * 2.0 ** -8)


def test_bf16_pair_range_covers_fp16_overflow():
    """The folded decode RMSNorm passes |x g| far beyond fp16's largest finite value:
    the bf16 pair stays finite and precise there."""
    a = np.array([65520.0, 1.0e5, 3.0e30, -7.5e37], dtype=np.float32)
    hi, lo = split_bf_pair(a)
    back = hi.astype(np.float64) + lo.astype(np.float64)
    assert np.all(np.isfinite(back))
    assert np.all(np.abs(back - a) <= 2.0 ** -16 * np.abs(a))


def test_fp16_pair_holds_fp32_values_in_its_range():
    """From 2^-3 to fp16's largest finite value the pair reproduces an fp32 value to
    about 22 significant bits (each half rounds to 11; lo stays a normal fp16 number)."""
    rng = np.random.default_rng(0)
    a = (2.0 ** rng.uniform(-3, 15.99, 200_000)).astype(np.float32)
    a *= rng.choice([-1.0, 1.0], a.size).astype(np.float32)
    hi, lo = split_pair(a)
    back = hi.astype(np.float64) + lo.astype(np.float64)
    rel = np.abs(back - a) / np.abs(a)
    assert rel.max() <= 2.0 ** -21
    assert np.all(np.abs(lo.astype(np.float64)) <= np.abs(hi.astype(np.float64)) * 2.0 ** -10)


def test_fp16_pair_range_limit():
    """The fp16 pair's limits: at or above 65520 (fp16's largest finite value rounds up
    there) the pair is infinite, just below it finite; far below its range the pair keeps
    only fp16's subnormal grid (an absolute error of at most 2^-25)."""
    hi, _ = split_pair(np.array([65504.0, 65519.0, 65520.0, 1.0e5], dtype=np.float32))
    assert np.all(np.isfinite(hi[:2])) and np.all(np.isinf(hi[2:]))
    a = np.array([3.0e-6, 1.0e-7], dtype=np.float32) * np.float32(1.0 + 2.0 ** -20)
    hi, lo = split_pair(a)
    err = np.abs(hi.astype(np.float64) + lo.astype(np.float64) - a)
    assert np.all(err / a > 2.0 ** -21)                      # fp32-grade precision lost ...
    assert np.all(err <= 2.0 ** -25)                         # ... to the subnormal grid
