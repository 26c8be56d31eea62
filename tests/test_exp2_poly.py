"""The double-precision 2^x of the draw kernel, checked on the host: its
polynomial is the one the Remez generator beside the kernel derives, and
2^n p(x - n) with n the nearest integer is within 5e-11 relative of 2^x
over the arguments the kernel sees (x <= 0, down to the underflow)."""
import os
import re
import runpy

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "..", "speculative_decoding_verification_07_amd", "csrc")


def _kernel_coefficients():
    src = open(os.path.join(CSRC, "spec_verify.hip")).read()
    body = re.search(r"constexpr double kExp2Poly\[8\] = \{(.*?)\};", src, re.S).group(1)
    return np.array([float(v) for v in re.findall(r"[-+0-9.eE]+", body)])


def test_kernel_polynomial_is_the_remez_one():
    gen = runpy.run_path(os.path.join(CSRC, "exp2_poly.py"))
    coef, err = gen["remez"]()
    assert err < 4.5e-11
    np.testing.assert_allclose(_kernel_coefficients(), coef, rtol=1e-12, atol=0)


def test_kernel_exp2_relative_error():
    c = _kernel_coefficients()
    x = np.concatenate([np.linspace(-0.5, 0.5, 100_001), -np.geomspace(1e-12, 1020.0, 100_001)])
    n = np.rint(x)
    r = x - n
    p = np.zeros_like(r) + c[7]
    for k in range(6, -1, -1):
        p = p * r + c[k]
    got = np.ldexp(p, n.astype(np.int64))
    want = np.exp2(x.astype(np.longdouble))
    rel = np.abs((got - want) / want).astype(np.float64)
    assert rel.max() < 5e-11, rel.max()
