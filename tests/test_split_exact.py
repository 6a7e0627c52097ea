"""The three-term bf16 split the backward kernels use for fp32 factors.

An fp32 value x is cut into hi = x with its low 16 bits cleared, then the
remainder r = x - hi (exact in fp32) is cut the same way into mid, and
lo = r - mid.  Each term must be a bf16 value (low 16 bits zero) and
hi + mid + lo must equal x exactly, so that a product with a bf16 factor
taken as three bf16 products loses nothing.  Checked here with numpy's fp32
arithmetic (round to nearest even, as on the GPU) over a wide magnitude range.
"""
import numpy as np


def _cut(v):
    return (v.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)


def test_three_term_split_is_exact():
    rng = np.random.default_rng(2024)
    x = (rng.standard_normal(1 << 20) * np.exp(rng.uniform(-40.0, 40.0, 1 << 20))).astype(np.float32)
    x = np.concatenate([x, np.array([0.0, -0.0, 1.0, -1.0, 3.1415927, 65504.0, 1e-30, -7.5e20,
                                     np.finfo(np.float32).max, np.finfo(np.float32).tiny], np.float32)])
    hi = _cut(x)
    r = (x - hi).astype(np.float32)
    mid = _cut(r)
    lo = (r - mid).astype(np.float32)
    for t in (hi, mid, lo):
        assert np.all((t.view(np.uint32) & np.uint32(0xFFFF)) == 0), "a term is not a bf16 value"
    total = hi.astype(np.float64) + mid.astype(np.float64) + lo.astype(np.float64)
    assert np.array_equal(total, x.astype(np.float64))


def test_two_terms_are_not_enough():
    """The third term matters: hi + mid alone misses bits of a typical value."""
    x = np.array([1.0 + 2.0 ** -9 + 2.0 ** -20 + 2.0 ** -23], np.float32)   # bits in all three parts
    hi = _cut(x)
    mid = _cut((x - hi).astype(np.float32))
    assert float(hi[0]) + float(mid[0]) != float(x[0])
