"""CPU oracle for the BitNet b1.58 W2A8 (I2_S) matmul -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline
leg may import this package.  It is a thin numpy/ctypes wrapper around the
plain C in ``bitnet_oracle.c`` (built by ``build()`` below or by the repo's
``__graft_entry__.build()``) and shares no code with the GPU library.  Page
keys [P1]..[P4] are listed in ``bitnet_oracle.h``; each wrapper cites the
passage its C function follows.

Every function here is pinned by ``tests/test_oracle_pins.py`` against facts
the pages print (worked examples under ``tests/golden/``), closed forms,
library routines (numpy's int64 matmul, IEEE float32 division and rint) and
brute force on tiny inputs.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "bitnet_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_i64 = ctypes.c_int64
_p = ctypes.c_void_p


def build() -> str:
    """Compile the oracle with gcc (no FMA contraction, no fast-math)."""
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-ffp-contract=off",
           "-fno-fast-math", "-fPIC", "-shared", _SRC, "-o", _LIB,
           "-lpthread", "-lm"]
    subprocess.run(cmd, check=True)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            raise RuntimeError(f"oracle library {_LIB} is not built; run "
                               "__graft_entry__.build() (or oracle.build())")
        L = ctypes.CDLL(_LIB)
        L.orc_code_of_weight.argtypes = [ctypes.c_int]
        L.orc_code_of_weight.restype = ctypes.c_int
        L.orc_weight_of_code.argtypes = [ctypes.c_int]
        L.orc_weight_of_code.restype = ctypes.c_int
        L.orc_pack_i2s.argtypes = [_p, _i64, _i64, _p]
        L.orc_pack_i2s.restype = _i64
        L.orc_unpack_i2s.argtypes = [_p, _i64, _i64, _p]
        L.orc_unpack_i2s.restype = _i64
        L.orc_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.orc_bf16_to_f32.restype = ctypes.c_float
        L.orc_exact_sum.argtypes = [_p, _i64]
        L.orc_exact_sum.restype = ctypes.c_double
        L.orc_absmean_alpha_f32.argtypes = [_p, _i64]
        L.orc_absmean_alpha_f32.restype = ctypes.c_float
        L.orc_absmean_alpha_bf16.argtypes = [_p, _i64]
        L.orc_absmean_alpha_bf16.restype = ctypes.c_float
        L.orc_absmean_ternary_f32.argtypes = [_p, _i64, ctypes.c_float, _p]
        L.orc_absmean_ternary_bf16.argtypes = [_p, _i64, ctypes.c_float, _p]
        L.orc_sign_ternary_f32.argtypes = [_p, _i64, _p, _p]
        L.orc_sign_ternary_f32.restype = _i64
        L.orc_ffn_act_quant.argtypes = [_p, _p, _p, ctypes.c_float, _i64, _i64, _p, _p, _p, _p]
        L.orc_quant_act_f32.argtypes = [_p, _i64, _i64, _p, _p, _p]
        L.orc_quant_act_f32.restype = None
        L.orc_quant_act_bf16.argtypes = [_p, _i64, _i64, _p, _p, _p]
        L.orc_quant_act_bf16.restype = None
        L.orc_dot_def.argtypes = [_p, _p, _i64, _i64, _i64, _p]
        L.orc_dot_def.restype = None
        L.orc_dot_raw.argtypes = [_p, _p, _p, _i64, _i64, _i64, _p, _p]
        L.orc_dot_raw.restype = None
        L.orc_lut_tables.argtypes = [_p, _i64, _p]
        L.orc_lut_tables.restype = None
        L.orc_dot_lut.argtypes = [_p, _p, _p, _i64, _i64, _i64, _p, _p]
        L.orc_dot_lut.restype = None
        L.orc_epilogue.argtypes = [_p, ctypes.c_double, _p, _i64, _i64, _p]
        L.orc_epilogue.restype = None
        L.orc_linear_i2s.argtypes = [_p, _i64, _i64, _p, _i64, _p, ctypes.c_float,
                                     _i64, _i64, _p, _p, ctypes.c_int]
        L.orc_linear_i2s.restype = _i64
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data


def code_of_weight(w: int) -> int:
    """[P1 §1-1] weight -> 2-bit code (-1 if the weight is not ternary)."""
    return lib().orc_code_of_weight(int(w))


def weight_of_code(c: int) -> int:
    """[P1 §1-1, §8] code -> weight (99 for code 3)."""
    return lib().orc_weight_of_code(int(c))


def pack_i2s(w: np.ndarray) -> tuple[np.ndarray, int]:
    """[P1 §4-2] int8 W[M][K] -> (uint8 packed[M][K/4], number of non-ternary weights)."""
    w = np.ascontiguousarray(w, dtype=np.int8)
    M, K = w.shape
    if K % 128:
        raise ValueError("K must be a multiple of 128")
    out = np.zeros((M, K // 4), dtype=np.uint8)
    bad = lib().orc_pack_i2s(_ptr(w), M, K, _ptr(out))
    return out, int(bad)


def unpack_i2s(packed: np.ndarray, K: int) -> tuple[np.ndarray, int]:
    """[P1 §8; P2 §3] packed[M][K/4] -> (int8 W[M][K], number of code-3 slots)."""
    packed = np.ascontiguousarray(packed, dtype=np.uint8).reshape(-1, K // 4)
    M = packed.shape[0]
    w = np.zeros((M, K), dtype=np.int8)
    bad = lib().orc_unpack_i2s(_ptr(packed), M, K, _ptr(w))
    return w, int(bad)


def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    return np.array([lib().orc_bf16_to_f32(int(v)) for v in h.ravel()],
                    dtype=np.float32).reshape(h.shape)


def quant_act(x: np.ndarray):
    """[P1 §4-5; P4] per-token absmax int8 quantisation.

    ``x`` is float32 [N][K] or bf16 bits as uint16 [N][K].  Returns
    (int8 q[N][K], float32 s[N], int32 qsum[N]) with s = 127/max(absmax, 1e-5).
    """
    x = np.ascontiguousarray(x)
    if x.ndim == 1:
        x = x[None, :]
    N, K = x.shape
    q = np.zeros((N, K), dtype=np.int8)
    s = np.zeros(N, dtype=np.float32)
    qs = np.zeros(N, dtype=np.int32)
    if x.dtype == np.float32:
        lib().orc_quant_act_f32(_ptr(x), N, K, _ptr(q), _ptr(s), _ptr(qs))
    elif x.dtype == np.uint16:
        lib().orc_quant_act_bf16(_ptr(x), N, K, _ptr(q), _ptr(s), _ptr(qs))
    else:
        raise TypeError("x must be float32 or bf16 bits (uint16)")
    return q, s, qs


def dot_def(w: np.ndarray, q: np.ndarray) -> np.ndarray:
    """[P1 §1-1; P4] D[n][m] = sum_k W[m][k]*q[n][k] (int64), the definition."""
    w = np.ascontiguousarray(w, dtype=np.int8)
    q = np.ascontiguousarray(q, dtype=np.int8)
    if q.ndim == 1:
        q = q[None, :]
    M, K = w.shape
    N = q.shape[0]
    assert q.shape[1] == K
    D = np.zeros((N, M), dtype=np.int64)
    lib().orc_dot_def(_ptr(w), _ptr(q), M, K, N, _ptr(D))
    return D


def dot_raw(packed: np.ndarray, q: np.ndarray, qsum: np.ndarray, K: int):
    """[P2 §3; P3 §3.2, §4] raw-code dot R and corrected D = R - qsum."""
    packed = np.ascontiguousarray(packed, dtype=np.uint8).reshape(-1, K // 4)
    q = np.ascontiguousarray(q, dtype=np.int8)
    if q.ndim == 1:
        q = q[None, :]
    qsum = np.ascontiguousarray(qsum, dtype=np.int32)
    M = packed.shape[0]
    N = q.shape[0]
    R = np.zeros((N, M), dtype=np.int64)
    D = np.zeros((N, M), dtype=np.int64)
    lib().orc_dot_raw(_ptr(packed), _ptr(q), _ptr(qsum), M, K, N, _ptr(R), _ptr(D))
    return R, D


def lut_tables(q: np.ndarray, K: int) -> np.ndarray:
    """[P1 §4-4, §11-2] per-group lookup tables of one token: int32 [K/2][16],
    entry 4*c_hi + c_lo = c_hi*x_first + c_lo*x_second over raw codes 0..3."""
    q = np.ascontiguousarray(q, dtype=np.int8).reshape(K)
    t = np.zeros((K // 2, 16), dtype=np.int32)
    lib().orc_lut_tables(_ptr(q), K, _ptr(t))
    return t


def dot_lut(packed: np.ndarray, q: np.ndarray, qsum: np.ndarray, K: int):
    """[P1 §4-3, §4-4] raw-code dot by table lookup (tables first, then one
    lookup per nibble); returns (R, D) like dot_raw."""
    packed = np.ascontiguousarray(packed, dtype=np.uint8).reshape(-1, K // 4)
    q = np.ascontiguousarray(q, dtype=np.int8)
    if q.ndim == 1:
        q = q[None, :]
    qsum = np.ascontiguousarray(qsum, dtype=np.int32)
    M = packed.shape[0]
    N = q.shape[0]
    R = np.zeros((N, M), dtype=np.int64)
    D = np.zeros((N, M), dtype=np.int64)
    lib().orc_dot_lut(_ptr(packed), _ptr(q), _ptr(qsum), M, K, N, _ptr(R), _ptr(D))
    return R, D


def epilogue(D: np.ndarray, alpha: float, s: np.ndarray) -> np.ndarray:
    """[P2 §3; P1 §4-5, §6-2] y = D*alpha/s in float64."""
    D = np.ascontiguousarray(D, dtype=np.int64)
    if D.ndim == 1:
        D = D[None, :]
    s = np.ascontiguousarray(s, dtype=np.float32)
    N, M = D.shape
    y = np.zeros((N, M), dtype=np.float64)
    lib().orc_epilogue(_ptr(D), float(alpha), _ptr(s), M, N, _ptr(y))
    return y


def linear_i2s(packed: np.ndarray, K: int, q: np.ndarray, s: np.ndarray,
               alpha: float, rows=None, nthreads: int = 1, want_y: bool = True):
    """Threaded whole matmul on packed weights (unpack + definition + epilogue).

    ``rows`` = (row0, nrows) restricts the work to those output rows; the
    returned D / y are then [N][nrows].  Returns (D int64, y float64 or None).
    """
    packed = np.ascontiguousarray(packed, dtype=np.uint8).reshape(-1, K // 4)
    q = np.ascontiguousarray(q, dtype=np.int8)
    if q.ndim == 1:
        q = q[None, :]
    s = np.ascontiguousarray(s, dtype=np.float32)
    M = packed.shape[0]
    N = q.shape[0]
    r0, nr = (0, M) if rows is None else rows
    D = np.zeros((N, M), dtype=np.int64)
    y = np.zeros((N, M), dtype=np.float64) if want_y else None
    bad = lib().orc_linear_i2s(_ptr(packed), M, K, _ptr(q), N, _ptr(s),
                               float(alpha), r0, nr, _ptr(D),
                               _ptr(y) if want_y else None, int(nthreads))
    if bad:
        raise ValueError(f"packed weights hold {bad} code-3 slots")
    D = np.ascontiguousarray(D[:, r0:r0 + nr])
    if want_y:
        y = np.ascontiguousarray(y[:, r0:r0 + nr])
    return D, y


def exact_sum(x: np.ndarray) -> float:
    """Exactly rounded binary64 sum of finite, non-negative values (order-free).

    The AbsMean scale [P1 §6-2; P4] and the FFN sub-norm [P4 "Forward Pass"]
    both sum non-negative values whose order the pages do not fix; the oracle
    takes the exact sum, rounded once.  Raises on a negative or non-finite value.
    """
    x = np.ascontiguousarray(x, dtype=np.float64).ravel()
    r = lib().orc_exact_sum(_ptr(x), x.size)
    if r < 0:
        raise ValueError("exact_sum takes finite, non-negative values")
    return float(r)


def absmean_alpha(w: np.ndarray) -> float:
    """AbsMean scale of a whole tensor [P1 §6-2; P4 "Ternary Weight
    Quantisation (AbsMean)"]: fp32 (float32 array) or bf16 bits (uint16)."""
    w = np.ascontiguousarray(w)
    if w.dtype == np.uint16:
        return float(np.float32(lib().orc_absmean_alpha_bf16(_ptr(w), w.size)))
    w = np.ascontiguousarray(w, dtype=np.float32)
    return float(np.float32(lib().orc_absmean_alpha_f32(_ptr(w), w.size)))


def absmean_ternary(w: np.ndarray, alpha: float) -> np.ndarray:
    """q = clip(round-half-even(w / alpha), -1, 1) with one fp32 division
    [P1 §6-2; P4]; same shape as w, int8."""
    w = np.ascontiguousarray(w)
    q = np.empty(w.shape, dtype=np.int8)
    if w.dtype == np.uint16:
        lib().orc_absmean_ternary_bf16(_ptr(w), w.size, np.float32(alpha), _ptr(q))
    else:
        w = np.ascontiguousarray(w, dtype=np.float32)
        lib().orc_absmean_ternary_f32(_ptr(w), w.size, np.float32(alpha), _ptr(q))
    return q


def absmean_i2s(w: np.ndarray) -> tuple[np.ndarray, float, np.ndarray]:
    """AbsMean ternarise a [M][K] weight tensor and pack it to I2_S:
    returns (packed, alpha, q)."""
    alpha = absmean_alpha(w)
    q = absmean_ternary(w, alpha)
    packed, bad = pack_i2s(q)
    assert bad == 0
    return packed, alpha, q


def sign_ternary(w: np.ndarray) -> tuple[np.ndarray, float, int]:
    """Sign/threshold ternary of float weights [P1 §4-2]: (q, max|w|, number
    of non-finite weights)."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    q = np.empty(w.shape, dtype=np.int8)
    wmax = ctypes.c_float(0.0)
    bad = lib().orc_sign_ternary_f32(_ptr(w), w.size, _ptr(q), ctypes.byref(wmax))
    return q, float(np.float32(wmax.value)), int(bad)


def ffn_act_quant(g: np.ndarray, u: np.ndarray, gamma, eps: float):
    """sqrelu(g) * u -> RMS sub-norm (the exactly rounded binary64 sum of the
    squares, gain gamma or 1) -> per-token int8 quantisation [P4 "Forward
    Pass"; P1 §4-5].  g, u: fp32 [N][F].  Returns (q, s, qsum, v)."""
    g = np.ascontiguousarray(g, dtype=np.float32)
    u = np.ascontiguousarray(u, dtype=np.float32)
    N, F = g.shape
    assert u.shape == (N, F) and F % 32 == 0
    gm = None if gamma is None else np.ascontiguousarray(gamma, dtype=np.float32)
    q = np.empty((N, F), dtype=np.int8)
    s = np.empty((N,), dtype=np.float32)
    qs = np.empty((N,), dtype=np.int32)
    v = np.empty((N, F), dtype=np.float32)
    lib().orc_ffn_act_quant(_ptr(g), _ptr(u), None if gm is None else _ptr(gm),
                            np.float32(eps), N, F, _ptr(q), _ptr(s), _ptr(qs), _ptr(v))
    return q, s, qs, v
