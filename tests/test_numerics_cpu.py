"""Number formats the GPU path relies on, emulated on the CPU with numpy's IEEE fp16.

The matrix-core paths (prefill GEMMs, decode at batch > 4, the decode attention) carry
each fp32 activation a as an fp16 pair hi = fp16(a), lo = fp16(a - hi).  The decode
route folds RMSNorm into its GEMMs by feeding the raw residual times the gain through
such pairs, so the pair's range is that path's range.
"""
import numpy as np


def split_pair(a: np.ndarray):
    a = np.asarray(a, dtype=np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        hi = a.astype(np.float16)
        lo = (a - hi.astype(np.float32)).astype(np.float16)
    return hi, lo


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
    """The limits of the folded decode RMSNorm: |x g| at or above 65520 (fp16's largest
    finite value rounds up there) turns the pair infinite, just below it the pair is
    finite; far below the range the pair keeps only fp16's subnormal grid (an absolute
    error of at most 2^-25)."""
    hi, _ = split_pair(np.array([65504.0, 65519.0, 65520.0, 1.0e5], dtype=np.float32))
    assert np.all(np.isfinite(hi[:2])) and np.all(np.isinf(hi[2:]))
    a = np.array([3.0e-6, 1.0e-7], dtype=np.float32) * np.float32(1.0 + 2.0 ** -20)
    hi, lo = split_pair(a)
    err = np.abs(hi.astype(np.float64) + lo.astype(np.float64) - a)
    assert np.all(err / a > 2.0 ** -21)                      # fp32-grade precision lost ...
    assert np.all(err <= 2.0 ** -25)                         # ... to the subnormal grid
