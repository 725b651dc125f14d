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
