"""ctypes binding of libbitnet_i2s.so (C ABI in include/bitnet_i2s.h).

Argument marshalling only: each function checks the dtype, shape, device
and contiguity of every torch tensor it is given (so a wrong K or a short
output buffer is refused on the host, never read or written out of bounds),
passes ``data_ptr()`` and the current HIP stream, and raises ``BitnetError``
on a non-zero status.  Every step of the computation
runs in the library's HIP kernels; nothing here computes a result.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libbitnet_i2s.so")
# the same library built with per-launch start/end stamps of the decode GEMV
# (include/bitnet_i2s_stamps.h); a measurement aid, never loaded by default
_STAMPS_PATH = os.path.join(_HERE, "libbitnet_i2s_stamps.so")

OK, E_NULL, E_SHAPE, E_ALIGN, E_DTYPE, E_VALUE, E_HIP = range(7)
F32, BF16 = 0, 1
GEMV_MAX_N = 64
LINEAR_FUSED_MAX_N = 2     # bitnet_linear_i2s: one fused launch up to this N


MAX_GROUP = 8


class I2SMatrix(ctypes.Structure):
    """Mirror of bitnet_i2s_matrix."""
    _fields_ = [("packed", ctypes.c_void_p), ("M", ctypes.c_int64),
                ("w_scale", ctypes.c_float), ("dot", ctypes.c_void_p),
                ("y", ctypes.c_void_p)]


class BitnetError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"bitnet status {status}: {msg}")
        self.status = status


_lib = None


def lib_path() -> str:
    return _LIB_PATH


def load() -> ctypes.CDLL:
    """Load the HIP library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    _lib = _open(_LIB_PATH)
    return _lib


def use_library(which: str) -> None:
    """Route every call through the product library ("main") or its
    instrumented twin ("stamps", which also records per-launch start/end
    stamps of the decode GEMV).  Both must have been built."""
    global _lib
    if which == "main":
        _lib = _open(_LIB_PATH)
    elif which == "stamps":
        L = _open(_STAMPS_PATH)
        L.bitnet_stamps_reset.argtypes = [ctypes.c_int, ctypes.c_void_p]
        L.bitnet_stamps_reset.restype = ctypes.c_int
        L.bitnet_stamps_read.argtypes = [ctypes.POINTER(ctypes.c_uint64), ctypes.c_int]
        L.bitnet_stamps_read.restype = ctypes.c_int
        _lib = L
    else:
        raise ValueError(which)


def stamps_reset(rewind: bool = False) -> None:
    """Clear the stamp slots on the current stream (instrumented library)."""
    import torch
    _check(load().bitnet_stamps_reset(int(rewind), torch.cuda.current_stream().cuda_stream))


def stamps_read(max_launches: int) -> list[tuple[int, int]]:
    """[(start, end)] in 100 MHz ticks for the launches since the last rewind."""
    buf = (ctypes.c_uint64 * (2 * max_launches))()
    n = load().bitnet_stamps_read(buf, max_launches)
    if n < 0:
        raise BitnetError(E_HIP, "bitnet_stamps_read failed")
    return [(buf[2 * i], buf[2 * i + 1]) for i in range(n)]


def _open(path: str) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with __graft_entry__.build() "
            "(there is no fallback implementation)")
    L = ctypes.CDLL(path)
    p, i64, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float
    L.bitnet_pack_i2s.argtypes = [p, i64, i64, p, p]
    L.bitnet_quant_act_i8.argtypes = [p, ctypes.c_int, i64, i64, p, p, p, p]
    sig = [p, f32, i64, i64, p, p, p, i64, p, p, p]
    L.bitnet_gemv_i2s_i8.argtypes = sig
    L.bitnet_gemm_i2s_i8.argtypes = sig
    L.bitnet_gemv_i2s_lut.argtypes = sig
    L.bitnet_linear_i2s.argtypes = [p, ctypes.c_int, i64, i64, ctypes.POINTER(I2SMatrix),
                                    ctypes.c_int, p, p, p, p]
    L.bitnet_linear_i2s.restype = ctypes.c_int
    L.bitnet_gemm_i2s_i8_group.argtypes = [ctypes.POINTER(I2SMatrix), ctypes.c_int, i64, p, p, p,
                                           i64, p]
    L.bitnet_gemm_i2s_i8_group.restype = ctypes.c_int
    L.bitnet_gemv_i2s_i8_group.argtypes = L.bitnet_gemm_i2s_i8_group.argtypes
    L.bitnet_gemv_i2s_i8_group.restype = ctypes.c_int
    L.bitnet_ffn_act_quant_i8.argtypes = [p, p, p, f32, i64, i64, p, p, p, p]
    L.bitnet_ffn_act_quant_i8.restype = ctypes.c_int
    L.bitnet_absmean_i2s.argtypes = [p, ctypes.c_int, i64, i64, p, ctypes.POINTER(ctypes.c_float), p]
    L.bitnet_absmean_i2s.restype = ctypes.c_int
    L.bitnet_pack_i2s_f32.argtypes = [p, i64, i64, p, ctypes.POINTER(ctypes.c_float), p]
    L.bitnet_pack_i2s_f32.restype = ctypes.c_int
    for fn in ("bitnet_pack_i2s", "bitnet_quant_act_i8", "bitnet_gemv_i2s_i8",
               "bitnet_gemm_i2s_i8", "bitnet_gemv_i2s_lut", "bitnet_abi_version"):
        getattr(L, fn).restype = ctypes.c_int
    L.bitnet_abi_version.argtypes = []
    L.bitnet_last_error.argtypes = []
    L.bitnet_last_error.restype = ctypes.c_char_p
    return L


def _check(status: int) -> None:
    if status != OK:
        msg = load().bitnet_last_error().decode(errors="replace")
        raise BitnetError(status, msg)


def _stream(t) -> int:
    import torch
    return torch.cuda.current_stream(t.device).cuda_stream


def _ptr(t) -> int | None:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _expect(t, name, dtype, shape, device=None):
    """Refuse a tensor of the wrong dtype, shape or device before any launch."""
    if t is None:
        raise ValueError(f"{name} is required")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, the other operands on {device}")


def _expect_tokens(xq, x_scale, x_sum):
    """Quantised tokens xq[N][K] int8 with s[N] fp32 and sum[N] int32 -> (N, K)."""
    import torch
    if xq is None or xq.dim() != 2:
        raise ValueError("xq must be a 2-D [N][K] tensor")
    N, K = xq.shape
    _expect(xq, "xq", torch.int8, (N, K))
    _expect(x_scale, "x_scale", torch.float32, (N,), xq.device)
    _expect(x_sum, "x_sum", torch.int32, (N,), xq.device)
    return N, K


def _expect_packed(P, K, device, name="packed"):
    """I2_S weights [M][K/4] uint8 for reduction length K -> M."""
    import torch
    if P is None or P.dim() != 2:
        raise ValueError(f"{name} must be a 2-D [M][K/4] tensor")
    if K % 4:
        raise ValueError(f"K={K} is not a multiple of 4")
    _expect(P, name, torch.uint8, (P.shape[0], K // 4), device)
    return P.shape[0]


def _expect_outputs(dot, y, N, M, device, name=""):
    import torch
    if dot is not None:
        _expect(dot, f"{name}dot", torch.int32, (N, M), device)
    if y is not None:
        _expect(y, f"{name}y", torch.float32, (N, M), device)


def abi_version() -> int:
    return load().bitnet_abi_version()


def pack(w):
    """int8 ternary W[M][K] (cuda) -> uint8 I2_S packed[M][K/4]."""
    import torch
    if w.dtype != torch.int8 or w.dim() != 2:
        raise TypeError("w must be a 2-D int8 tensor")
    M, K = w.shape
    if K % 4:
        raise ValueError(f"K={K} is not a multiple of 4")
    out = torch.empty((M, K // 4), dtype=torch.uint8, device=w.device)
    _check(load().bitnet_pack_i2s(_ptr(w), M, K, _ptr(out), _stream(w)))
    return out


def absmean_pack(w, out=None):
    """fp32 or bf16 weights W[M][K] (cuda) -> (uint8 I2_S packed[M][K/4], AbsMean
    scale alpha as a Python float)."""
    import torch
    if w.dim() != 2:
        raise TypeError("w must be 2-D [M][K]")
    dt = {torch.float32: F32, torch.bfloat16: BF16}.get(w.dtype)
    if dt is None:
        raise TypeError("w must be float32 or bfloat16")
    M, K = w.shape
    if K % 4:
        raise ValueError(f"K={K} is not a multiple of 4")
    packed = out if out is not None else torch.empty((M, K // 4), dtype=torch.uint8,
                                                     device=w.device)
    _expect(packed, "out", torch.uint8, (M, K // 4), w.device)
    alpha = ctypes.c_float(0.0)
    _check(load().bitnet_absmean_i2s(_ptr(w), dt, M, K, _ptr(packed), ctypes.byref(alpha),
                                     _stream(w)))
    return packed, alpha.value


def pack_f32(w, out=None):
    """fp32 weights already ternary in value, W[M][K] (cuda) -> (packed I2_S by
    sign with the 1e-6 zero threshold, max|w| as a Python float)."""
    import torch
    if w.dtype != torch.float32 or w.dim() != 2:
        raise TypeError("w must be a 2-D float32 tensor")
    M, K = w.shape
    if K % 4:
        raise ValueError(f"K={K} is not a multiple of 4")
    packed = out if out is not None else torch.empty((M, K // 4), dtype=torch.uint8,
                                                     device=w.device)
    _expect(packed, "out", torch.uint8, (M, K // 4), w.device)
    wmax = ctypes.c_float(0.0)
    _check(load().bitnet_pack_i2s_f32(_ptr(w), M, K, _ptr(packed), ctypes.byref(wmax),
                                      _stream(w)))
    return packed, wmax.value


def quant_act(x, out=None):
    """fp32 or bf16 x[N][K] (cuda) -> (int8 xq[N][K], fp32 s[N], int32 xsum[N])."""
    import torch
    if x.dim() != 2:
        raise TypeError("x must be 2-D [N][K]")
    dt = {torch.float32: F32, torch.bfloat16: BF16}.get(x.dtype)
    if dt is None:
        raise TypeError("x must be float32 or bfloat16")
    N, K = x.shape
    if out is None:
        xq = torch.empty((N, K), dtype=torch.int8, device=x.device)
        s = torch.empty((N,), dtype=torch.float32, device=x.device)
        xs = torch.empty((N,), dtype=torch.int32, device=x.device)
    else:
        xq, s, xs = out
        _expect(xq, "xq", torch.int8, (N, K), x.device)
        _expect(s, "x_scale", torch.float32, (N,), x.device)
        _expect(xs, "x_sum", torch.int32, (N,), x.device)
    _check(load().bitnet_quant_act_i8(_ptr(x), dt, N, K, _ptr(xq), _ptr(s),
                                      _ptr(xs), _stream(x)))
    return xq, s, xs


def _matmul(fn, packed, w_scale, xq, x_scale, x_sum, want_dot, want_y, out):
    import torch
    N, K = _expect_tokens(xq, x_scale, x_sum)
    M = _expect_packed(packed, K, xq.device)
    if out is not None:
        dot, y = out
        _expect_outputs(dot, y, N, M, xq.device)
    else:
        dot = torch.empty((N, M), dtype=torch.int32, device=xq.device) if want_dot else None
        y = torch.empty((N, M), dtype=torch.float32, device=xq.device) if want_y else None
    _check(fn(_ptr(packed), float(w_scale), M, K, _ptr(xq), _ptr(x_scale),
              _ptr(x_sum), N, _ptr(dot), _ptr(y), _stream(xq)))
    return dot, y


def gemv(packed, w_scale, xq, x_scale, x_sum, want_dot=True, want_y=True, out=None):
    """Decode matmul (1..64 tokens) -> (int32 dot[N][M] | None, fp32 y[N][M] | None)."""
    return _matmul(load().bitnet_gemv_i2s_i8, packed, w_scale, xq, x_scale, x_sum,
                   want_dot, want_y, out)


def gemv_lut(packed, w_scale, xq, x_scale, x_sum, want_dot=True, want_y=True, out=None):
    """Decode matmul by table lookup (K <= 8192) -> (dot | None, y | None),
    the same values as gemv."""
    return _matmul(load().bitnet_gemv_i2s_lut, packed, w_scale, xq, x_scale, x_sum,
                   want_dot, want_y, out)


def gemm(packed, w_scale, xq, x_scale, x_sum, want_dot=True, want_y=True, out=None):
    """Prefill matmul (any token count, int8 MFMA) -> (dot | None, y | None)."""
    return _matmul(load().bitnet_gemm_i2s_i8, packed, w_scale, xq, x_scale, x_sum,
                   want_dot, want_y, out)


def _mats_out(mats, N, K, device, want_dot, want_y, out):
    import torch
    if not 1 <= len(mats) <= MAX_GROUP:
        raise ValueError(f"{len(mats)} matrices; a call takes 1..{MAX_GROUP}")
    for i, (P, _) in enumerate(mats):
        _expect_packed(P, K, device, f"mats[{i}] packed")
    if out is not None:
        if len(out) != len(mats):
            raise ValueError("out must hold one (dot, y) pair per matrix")
        for i, ((P, _), (d, y)) in enumerate(zip(mats, out)):
            _expect_outputs(d, y, N, P.shape[0], device, f"out[{i}] ")
        return out
    res = []
    for P, _ in mats:
        M = P.shape[0]
        res.append((torch.empty((N, M), dtype=torch.int32, device=device) if want_dot else None,
                    torch.empty((N, M), dtype=torch.float32, device=device) if want_y else None))
    return res


def _mat_array(mats, out):
    arr = (I2SMatrix * len(mats))()
    for i, ((P, ws), (d, y)) in enumerate(zip(mats, out)):
        arr[i] = I2SMatrix(_ptr(P), P.shape[0], float(ws), _ptr(d), _ptr(y))
    return arr


def gemm_group(mats, xq, x_scale, x_sum, want_dot=True, want_y=True, out=None):
    """Prefill matmul of every (packed, w_scale) in ``mats`` by the same
    quantised tokens, one MFMA launch -> [(dot | None, y | None) per matrix]."""
    N, K = _expect_tokens(xq, x_scale, x_sum)
    out = _mats_out(mats, N, K, xq.device, want_dot, want_y, out)
    _check(load().bitnet_gemm_i2s_i8_group(_mat_array(mats, out), len(mats), K, _ptr(xq),
                                           _ptr(x_scale), _ptr(x_sum), N, _stream(xq)))
    return out


def gemv_group(mats, xq, x_scale, x_sum, want_dot=True, want_y=True, out=None):
    """Decode matmul (N <= 64 quantised tokens) of every (packed, w_scale) in
    ``mats`` -> [(dot | None, y | None) per matrix]."""
    N, K = _expect_tokens(xq, x_scale, x_sum)
    out = _mats_out(mats, N, K, xq.device, want_dot, want_y, out)
    _check(load().bitnet_gemv_i2s_i8_group(_mat_array(mats, out), len(mats), K, _ptr(xq),
                                           _ptr(x_scale), _ptr(x_sum), N, _stream(xq)))
    return out


def ffn_act_quant(g, u, gamma=None, eps=1e-5, out=None):
    """sqrelu(g) * u -> RMS sub-norm (gain gamma or 1, eps) -> int8 tokens for
    the down projection: fp32 g, u [N][F] (cuda) -> (xq, s, xsum)."""
    import torch
    if g.dtype != torch.float32 or u.dtype != torch.float32 or g.shape != u.shape or g.dim() != 2:
        raise TypeError("g and u must be float32 tensors of the same 2-D shape")
    N, F = g.shape
    if u.device != g.device:
        raise ValueError("g and u must be on the same device")
    if gamma is not None:
        _expect(gamma, "gamma", torch.float32, (F,), g.device)
    if out is None:
        out = (torch.empty((N, F), dtype=torch.int8, device=g.device),
               torch.empty((N,), dtype=torch.float32, device=g.device),
               torch.empty((N,), dtype=torch.int32, device=g.device))
    xq, xs, xsum = out
    _expect(xq, "xq", torch.int8, (N, F), g.device)
    _expect(xs, "x_scale", torch.float32, (N,), g.device)
    _expect(xsum, "x_sum", torch.int32, (N,), g.device)
    _check(load().bitnet_ffn_act_quant_i8(_ptr(g), _ptr(u), _ptr(gamma), float(eps), N, F,
                                          _ptr(xq), _ptr(xs), _ptr(xsum), _stream(g)))
    return xq, xs, xsum


def ffn(x, gate, up, down, gamma=None, eps=1e-5):
    """The squared-ReLU gated FFN block on I2_S weights, as three library calls:
    bitnet_linear_i2s(x, [gate, up]) -> bitnet_ffn_act_quant_i8 -> the down
    projection (decode or prefill kernel by N).  gate/up/down are
    (packed, w_scale) pairs; x is fp32/bf16 [N][K] (cuda).
    Returns (dot, y) of the down projection."""
    outs, _ = linear(x, [gate, up])
    (_, g), (_, u) = outs
    xq, xs, xsum = ffn_act_quant(g, u, gamma, eps)
    P, ws = down
    if xq.shape[0] <= GEMV_MAX_N:
        return gemv(P, ws, xq, xs, xsum)
    return gemm(P, ws, xq, xs, xsum)


def linear(x, mats, want_dot=True, want_y=True, out=None, qout=None):
    """Linear layer step: quantise tokens x[N][K] (fp32/bf16, cuda) and multiply
    them by every (packed, w_scale) in ``mats`` -- one fused launch for N <= 2;
    for N > 2 the library quantises into ``qout`` first (allocated here if
    None), then runs the batched-decode (N <= 64) or grouped prefill kernels.

    Returns ([(dot | None, y | None) per matrix], (xq, s, xsum) | None)."""
    import torch
    if x.dim() != 2:
        raise TypeError("x must be 2-D [N][K]")
    dt = {torch.float32: F32, torch.bfloat16: BF16}.get(x.dtype)
    if dt is None:
        raise TypeError("x must be float32 or bfloat16")
    N, K = x.shape
    out = _mats_out(mats, N, K, x.device, want_dot, want_y, out)
    if qout is None and N > LINEAR_FUSED_MAX_N:
        qout = (torch.empty((N, K), dtype=torch.int8, device=x.device),
                torch.empty((N,), dtype=torch.float32, device=x.device),
                torch.empty((N,), dtype=torch.int32, device=x.device))
    xq, xs, xsum = qout if qout is not None else (None, None, None)
    if qout is not None:
        _expect(xq, "qout xq", torch.int8, (N, K), x.device)
        _expect(xs, "qout x_scale", torch.float32, (N,), x.device)
        _expect(xsum, "qout x_sum", torch.int32, (N,), x.device)
    _check(load().bitnet_linear_i2s(_ptr(x), dt, N, K, _mat_array(mats, out), len(mats),
                                    _ptr(xq), _ptr(xs), _ptr(xsum), _stream(x)))
    return out, qout
