"""The threshold kernel's fixed-point masses, checked on the host: the kernel
forms trunc(f * 2^42) for a weight f = 2^e in fp32 as two 32-bit halves,
hi = trunc(f * 2^10) and lo = trunc((f * 2^10 - hi) * 2^32).  Emulated here
with numpy's fp32 arithmetic (the same IEEE single operations, no fused
multiply-add) against the exact value in double, over every exponent of
the floats below 2 (subnormals included) with random and extreme
significands."""
import numpy as np


def _split(f32):
    fs = f32 * np.float32(1024.0)
    hi = fs.astype(np.uint32)
    fr = fs - hi.astype(np.float32)
    lo = (fr * np.float32(4294967296.0)).astype(np.uint32)
    return (hi.astype(np.uint64) << np.uint64(32)) | lo.astype(np.uint64)


def test_fixed_mass_split_is_exact():
    rng = np.random.default_rng(5)
    exps = np.arange(0, 128, dtype=np.uint32)            # biased exponents of floats below 2
    mant = np.concatenate([rng.integers(0, 1 << 23, 4096, dtype=np.uint32),
                           np.array([0, 1, 2, (1 << 23) - 2, (1 << 23) - 1], dtype=np.uint32)])
    u = (exps[:, None] << np.uint32(23)) | mant[None, :]
    f = u.ravel().view(np.float32)
    want = np.trunc(f.astype(np.float64) * 2.0 ** 42).astype(np.uint64)
    got = _split(f)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, (f[bad[:5]], got[bad[:5]], want[bad[:5]])


def test_fixed_mass_split_planted_mistake_is_caught():
    # the low half rounded to nearest instead of truncated: the check above
    # sees it on the same inputs
    rng = np.random.default_rng(5)
    f = (rng.random(4096) * 2.0 ** -20).astype(np.float32)
    fs = f * np.float32(1024.0)
    hi = fs.astype(np.uint32)
    lo = np.rint((fs - hi.astype(np.float32)) * np.float32(4294967296.0)).astype(np.uint64)
    wrong = (hi.astype(np.uint64) << np.uint64(32)) | lo
    want = np.trunc(f.astype(np.float64) * 2.0 ** 42).astype(np.uint64)
    assert np.any(wrong != want)
    np.testing.assert_array_equal(_split(f), want)
