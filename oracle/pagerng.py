"""The self-test generator printed on "Speculative decoding" (mhtirogla.ai),
section "Code": xorshift64* with a 24-bit float in [0, 1).  Test
infrastructure only: it replays that page's statistical self-test against the
oracle.  Production uniforms are an input of the verify step (numpy Philox).

Written from the published definition of xorshift64* (shift triple 12, 25,
27, multiplier 0x2545F4914F6CDD1D, top bits of the product) and the page's
conversion of the top 24 bits to a float.
"""
from __future__ import annotations

import numpy as np

_MASK = (1 << 64) - 1
_MULT = 0x2545F4914F6CDD1D


class XorShift64Star:
    def __init__(self, seed: int):
        if seed == 0:
            raise ValueError("xorshift64* needs a non-zero state")
        self.state = seed & _MASK

    def next_u64(self) -> int:
        s = self.state
        s ^= s >> 12
        s ^= (s << 25) & _MASK
        s ^= s >> 27
        self.state = s
        return (s * _MULT) & _MASK

    def uniform24(self) -> float:
        """Top 24 bits of the scrambled output divided by 2^24."""
        return (self.next_u64() >> 40) / float(1 << 24)

    def uniforms(self, n: int) -> np.ndarray:
        out = np.empty(n, np.float32)
        for k in range(n):
            out[k] = self.uniform24()
        return out
