"""Constructed FFN inputs shared by the oracle pins and the GPU parity tests.

No arithmetic of the method lives here: these functions only choose gate/up
values (as IEEE fp32/binary64 facts) for cases that a summation order would
decide.
"""
from __future__ import annotations

import math

import numpy as np


def _factor(ss: float, F: int, eps: float) -> np.float32:
    # fp32(1 / sqrt(ss / F + eps)), every step one IEEE binary64 operation
    return np.float32(1.0 / math.sqrt(ss / F + eps))


def order_sensitive_token(F: int = 128):
    """(g, u, eps, c_exact, c_left_to_right) for one token of F channels.

    The squares h^2 (h = relu(g)^2 * u with g = 1, so h = u) are 11^2, powers
    of two that spell out the rest of a double S below 128, and four squares
    of 2^-24 (2^-48 each).  Summed exactly the four add one binary64 ulp
    (2^-46) to S; summed left to right each is below half an ulp and is
    dropped.  S is chosen as the double just below a point where the fp32
    factor 1/sqrt(ss/F + eps) changes, so the two sums give different
    factors.  eps is the smallest fp32 subnormal, which vanishes next to
    ss/F ~ 1.
    """
    eps = float(np.float32(1.4e-45))
    lo, hi = 127.99, 128.0
    assert _factor(lo, F, eps) != _factor(hi, F, eps)
    a = np.array([lo, hi]).view(np.int64)
    ia, ib = int(a[0]), int(a[1])
    while ib - ia > 1:                       # bisect over adjacent doubles
        im = (ia + ib) // 2
        vm = float(np.array([im], np.int64).view(np.float64)[0])
        if _factor(vm, F, eps) == _factor(lo, F, eps):
            ia = im
        else:
            ib = im
    s_below = float(np.array([ia], np.int64).view(np.float64)[0])
    s_exact = float(np.array([ib], np.int64).view(np.float64)[0])
    assert s_exact - s_below == 2.0 ** -46
    h = [11.0]
    rest = s_below - 121.0                   # a multiple of 2^-46 in (6, 7)
    for j in range(2, -47, -1):              # its binary digits, each as one or two squares
        bit = 2.0 ** j
        if rest >= bit:
            rest -= bit
            if j % 2 == 0:
                h.append(2.0 ** (j // 2))
            else:
                h += [2.0 ** ((j - 1) // 2)] * 2
    assert rest == 0.0
    h += [2.0 ** -24] * 4
    assert len(h) <= F
    u = np.zeros((1, F), np.float32)
    u[0, :len(h)] = np.array(h, np.float32)
    g = np.ones((1, F), np.float32)
    return g, u, eps, _factor(s_exact, F, eps), _factor(s_below, F, eps)


def _powers_as_squares(j0: int, j1: int) -> list:
    """h values whose squares are 2^-j for j0 <= j < j1: 2^-(j/2) for even j,
    two copies of 2^-((j+1)/2) for odd j."""
    h = []
    for j in range(j0, j1):
        if j % 2 == 0:
            h.append(2.0 ** (-j // 2))
        else:
            h += [2.0 ** (-(j + 1) // 2)] * 2
    return h


def _token(h: list):
    F = (len(h) + 127) // 128 * 128
    u = np.zeros((1, F), np.float32)
    u[0, :len(h)] = np.array(h, np.float32)
    return np.ones((1, F), np.float32), u


def carry_token(extra: int = 0):
    """(g, u) of a token with squares 1, 2^-54 .. 2^-112 (every bit once) and
    256 + extra squares of 2^-120.  The sum is 1 + 2^-53 - 2^-112 + (256 +
    extra) * 2^-120: at extra = 0 exactly the midpoint 1 + 2^-53 (ties to
    even: 1), above it for extra > 0 (1 + 2^-52), below for extra < 0 (1).
    A sum that keeps 112 bits below 1 sees a run of ones down to the round
    bit and only a count of the 2^-120 squares below it."""
    return _token([1.0] + _powers_as_squares(54, 113) + [2.0 ** -60] * (256 + extra))


def deep_carry_token():
    """Squares 1, then every power 2^-54 .. 2^-224, then four of 2^-226: the
    run of ones spans two 112-bit windows and the last four squares complete
    the carry to exactly 1 + 2^-53 (a tie: rounds to 1)."""
    return _token([1.0] + _powers_as_squares(54, 225) + [2.0 ** -113] * 4)
