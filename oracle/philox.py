"""Philox4x32-10 and the Gumbel noise of the sampled walk.  TEST INFRASTRUCTURE ONLY.

Philox4x32-10 is the counter-based generator of Salmon, Moraes, Dror and Shaw,
"Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11): a 4x32-bit counter is
mixed by ten rounds of two 32x32->64-bit multiplies and xors with a 2x32-bit
key that is advanced by two Weyl constants between rounds.  Written here with
Python integers, one output block per call.

The pages fix only that sampling draws from the same scores as greedy
(DFlash 2: Keep Drafting Parallel, wpnews.pro, section "A Lightweight Path
Selector").  The stream layout is this implementation's reading: key =
(seed low 32 bits, seed high 32 bits), counter = (candidate slot j, position t,
sequence b, 0), output word 0 is used.
"""
from __future__ import annotations

import math

_MASK = 0xFFFFFFFF
# Multipliers and Weyl key increments of Philox4x32 (Salmon et al., SC'11).
_M0 = 0xD2511F53
_M1 = 0xCD9E8D57
_W0 = 0x9E3779B9
_W1 = 0xBB67AE85


def philox4x32_10(counter: tuple[int, int, int, int], key: tuple[int, int]) -> tuple[int, int, int, int]:
    """Ten Philox rounds on ``counter`` under ``key``; returns the 4 output words."""
    c0, c1, c2, c3 = (int(c) & _MASK for c in counter)
    k0, k1 = (int(k) & _MASK for k in key)
    for _ in range(10):
        p0 = _M0 * c0
        p1 = _M1 * c2
        c0, c1, c2, c3 = ((p1 >> 32) ^ c1 ^ k0) & _MASK, p1 & _MASK, ((p0 >> 32) ^ c3 ^ k1) & _MASK, p0 & _MASK
        k0 = (k0 + _W0) & _MASK
        k1 = (k1 + _W1) & _MASK
    return c0, c1, c2, c3


def uniform_from_word(x: int) -> float:
    """Map a 32-bit word to u in (0, 1): the top 23 bits plus one half, times 2^-23.

    The result is exactly representable in fp32 and fp64 and never 0 or 1.
    """
    return ((int(x) >> 9) + 0.5) * 2.0 ** -23


def gumbel(seed: int, b: int, t: int, j: int) -> float:
    """Standard Gumbel noise -log(-log u) for (sequence b, position t, slot j), in fp64."""
    key = (seed & _MASK, (seed >> 32) & _MASK)
    x = philox4x32_10((j, t, b, 0), key)[0]
    u = uniform_from_word(x)
    return -math.log(-math.log(u))
