"""Coefficients of the polynomial the verify kernel evaluates for 2^r.

The kernel computes 2^x in double precision as 2^n * p(r), with n the
nearest integer to x and r = x - n in [-1/2, 1/2].  p is the degree-7
polynomial that minimises the largest relative error |p(r) / 2^r - 1| on
[-1/2, 1/2], found here with the Remez exchange algorithm: solve for the
polynomial whose relative error alternates in sign with equal magnitude on
n + 2 reference points, move the reference points to the extrema of the
resulting error, and repeat until the extrema are level.

Run as a script to print the coefficients (lowest degree first) and the
largest relative error on a dense grid.
"""
from __future__ import annotations

import numpy as np

DEGREE = 7
LO, HI = -0.5, 0.5


def _extrema(err: np.ndarray) -> np.ndarray:
    """Indices of the local extrema of err, endpoints included."""
    d = np.diff(err)
    inner = np.nonzero(d[:-1] * d[1:] <= 0)[0] + 1
    return np.concatenate([[0], inner, [len(err) - 1]])


def remez(degree: int = DEGREE, iters: int = 40, grid: int = 400_001):
    m = degree + 2
    # start from the Chebyshev extrema
    x = 0.5 * (LO + HI) + 0.5 * (HI - LO) * np.cos(np.pi * np.arange(m)[::-1] / (m - 1))
    g = np.linspace(LO, HI, grid)
    fg = np.exp2(g)
    c = None
    for _ in range(iters):
        # p(x_i) - 2^x_i = (-1)^i E 2^x_i for the unknowns c_0..c_n, E
        a = np.zeros((m, m))
        a[:, :degree + 1] = x[:, None] ** np.arange(degree + 1)[None, :]
        a[:, degree + 1] = (-1.0) ** np.arange(m) * np.exp2(x)
        sol = np.linalg.solve(a, np.exp2(x))
        c = sol[:degree + 1]
        err = np.polynomial.polynomial.polyval(g, c) / fg - 1.0
        idx = _extrema(err)
        # keep one extremum per run of equal sign (the largest), then the m largest
        pts = []
        for i in idx:
            if pts and np.sign(err[i]) == np.sign(err[pts[-1]]):
                if abs(err[i]) > abs(err[pts[-1]]):
                    pts[-1] = i
            else:
                pts.append(i)
        while len(pts) > m:
            if abs(err[pts[0]]) < abs(err[pts[-1]]):
                pts.pop(0)
            else:
                pts.pop()
        if len(pts) < m:
            break
        x = g[np.array(pts)]
    err = np.polynomial.polynomial.polyval(g, c) / fg - 1.0
    return c, float(np.abs(err).max())


if __name__ == "__main__":
    coef, e = remez()
    print(f"degree {DEGREE}, largest relative error {e:.3e}")
    for k, v in enumerate(coef):
        print(f"  r^{k}: {float(v)!r}")
