"""Host-side checks of the C ABI (CPU only: nothing is launched).

The library must load, export every function include/bitnet_i2s.h declares,
and reject bad arguments with the documented status before touching the
device.  Fake pointer values are never dereferenced: every case below fails
validation first.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bitnet_i2s.h")
STAMPS_HEADER = os.path.join(ROOT, "include", "bitnet_i2s_stamps.h")

OK, E_NULL, E_SHAPE, E_ALIGN, E_DTYPE, E_VALUE, E_HIP = range(7)
FAKE = 0x10000          # 64 KiB-aligned non-null value, never dereferenced
MIS = 0x10004           # 4- but not 16-byte aligned


@pytest.fixture(scope="module")
def L():
    from ternary_weight_i2_amd import _binding
    return _binding.load()


def declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(bitnet_\w+)\s*\(", text, flags=re.M)


def test_header_declares_the_boundary():
    fns = set(declared_functions())
    assert {"bitnet_pack_i2s", "bitnet_quant_act_i8", "bitnet_gemv_i2s_i8",
            "bitnet_gemm_i2s_i8", "bitnet_gemm_i2s_i8_group", "bitnet_gemv_i2s_i8_group",
            "bitnet_linear_i2s", "bitnet_gemv_i2s_lut",
            "bitnet_absmean_i2s", "bitnet_pack_i2s_f32", "bitnet_ffn_act_quant_i8",
            "bitnet_last_error",
            "bitnet_abi_version"} <= fns


def test_library_exports_every_declared_symbol(L):
    for fn in declared_functions():
        assert hasattr(L, fn), fn


def test_stamps_build_exports_both_headers_and_the_product_build_neither(L):
    """The instrumented twin exports the whole ABI plus the stamp calls; the
    product library has no stamp calls."""
    from ternary_weight_i2_amd import _binding
    S = ctypes.CDLL(_binding._STAMPS_PATH)
    stamps = declared_functions(STAMPS_HEADER)
    assert set(stamps) == {"bitnet_stamps_reset", "bitnet_stamps_read"}
    for fn in declared_functions() + stamps:
        assert hasattr(S, fn), fn
    for fn in stamps:
        assert not hasattr(L, fn), fn


def test_abi_version(L):
    text = open(HEADER).read()
    v = int(re.search(r"#define BITNET_ABI_VERSION (\d+)", text).group(1))
    assert L.bitnet_abi_version() == v


def _err(L):
    return L.bitnet_last_error().decode()


def test_pack_validation(L):
    assert L.bitnet_pack_i2s(FAKE, 4, 100, FAKE, None) == E_SHAPE
    assert "multiple of 128" in _err(L)
    assert L.bitnet_pack_i2s(FAKE, -1, 128, FAKE, None) == E_SHAPE
    assert L.bitnet_pack_i2s(FAKE, 4, 0, FAKE, None) == E_SHAPE
    assert L.bitnet_pack_i2s(FAKE, 4, 32768 + 128, FAKE, None) == E_SHAPE
    assert L.bitnet_pack_i2s(None, 4, 128, FAKE, None) == E_NULL
    assert L.bitnet_pack_i2s(FAKE, 4, 128, None, None) == E_NULL
    assert L.bitnet_pack_i2s(FAKE + 1, 4, 128, FAKE, None) == E_ALIGN
    assert L.bitnet_pack_i2s(FAKE, 4, 128, MIS, None) == E_ALIGN
    # M == 0 is a no-op, even with NULL pointers
    assert L.bitnet_pack_i2s(None, 0, 128, None, None) == OK


def test_quant_validation(L):
    q = L.bitnet_quant_act_i8
    assert q(FAKE, 2, 1, 128, FAKE, FAKE, FAKE, None) == E_DTYPE
    assert q(FAKE, 0, 1, 96, FAKE, FAKE, FAKE, None) == E_SHAPE
    assert q(FAKE, 0, -2, 128, FAKE, FAKE, FAKE, None) == E_SHAPE
    assert q(None, 0, 1, 128, FAKE, FAKE, FAKE, None) == E_NULL
    assert q(FAKE, 1, 1, 128, FAKE, None, FAKE, None) == E_NULL
    assert q(MIS, 1, 1, 128, FAKE, FAKE, FAKE, None) == E_ALIGN
    assert q(FAKE, 1, 1, 128, MIS, FAKE, FAKE, None) == E_ALIGN
    assert q(FAKE, 1, 1, 128, FAKE, FAKE + 2, FAKE, None) == E_ALIGN
    assert q(None, 1, 0, 128, None, None, None, None) == OK


@pytest.mark.parametrize("name,maxn", [("bitnet_gemv_i2s_i8", 64),
                                       ("bitnet_gemm_i2s_i8", 1 << 21),
                                       ("bitnet_gemv_i2s_lut", 64)])
def test_matmul_validation(L, name, maxn):
    f = getattr(L, name)
    a = dict(packed=FAKE, s=0.05, M=16, K=256, xq=FAKE, xs=FAKE, xsum=FAKE, N=1,
             dot=FAKE, y=FAKE)

    def call(**kw):
        b = dict(a, **kw)
        return f(b["packed"], b["s"], b["M"], b["K"], b["xq"], b["xs"], b["xsum"],
                 b["N"], b["dot"], b["y"], None)

    assert call(K=200) == E_SHAPE
    assert call(K=0) == E_SHAPE
    assert call(M=-1) == E_SHAPE
    assert call(N=-1) == E_SHAPE
    assert call(N=maxn + 1) == E_SHAPE
    assert call(M=1 << 31) == E_SHAPE
    assert call(packed=None) == E_NULL
    assert call(xq=None) == E_NULL
    assert call(xs=None) == E_NULL
    assert call(xsum=None) == E_NULL
    assert call(dot=None, y=None) == E_NULL
    assert call(packed=MIS) == E_ALIGN
    assert call(xq=MIS) == E_ALIGN
    assert call(y=FAKE + 2) == E_ALIGN
    assert call(dot=FAKE + 1) == E_ALIGN
    assert call(M=0, packed=None, xq=None) == OK
    assert call(N=0, packed=None, xq=None) == OK
    assert _err(L) == ""
    if name == "bitnet_gemv_i2s_lut":
        # the tables of one token take 16*K bytes of LDS: K <= 8192
        assert call(K=8192 + 128) == E_SHAPE
        assert "8192" in _err(L)
        assert call(K=8192 + 128, M=0) == E_SHAPE


def test_linear_validation(L):
    from ternary_weight_i2_amd._binding import I2SMatrix
    f = L.bitnet_linear_i2s

    def mats(*ms):
        arr = (I2SMatrix * len(ms))()
        for i, m in enumerate(ms):
            arr[i] = m
        return arr
    good = I2SMatrix(FAKE, 64, 0.1, FAKE, FAKE)
    g1 = mats(good)
    assert f(FAKE, 5, 1, 256, g1, 1, None, None, None, None) == E_DTYPE
    assert f(FAKE, 1, (1 << 21) + 1, 256, g1, 1, None, None, None, None) == E_SHAPE
    assert f(FAKE, 1, 65, 256, g1, 1, None, None, None, None) == E_NULL   # prefill needs xq
    assert f(FAKE, 1, -1, 256, g1, 1, None, None, None, None) == E_SHAPE
    assert f(FAKE, 1, 1, 200, g1, 1, None, None, None, None) == E_SHAPE
    assert f(FAKE, 1, 1, 256, g1, 0, None, None, None, None) == E_SHAPE
    assert f(FAKE, 1, 1, 256, mats(*[good] * 9), 9, None, None, None, None) == E_SHAPE
    assert f(FAKE, 1, 1, 256, None, 1, None, None, None, None) == E_NULL
    assert f(None, 1, 1, 256, g1, 1, None, None, None, None) == E_NULL
    assert f(FAKE, 1, 1, 256, mats(I2SMatrix(None, 64, 0.1, FAKE, FAKE)), 1,
             None, None, None, None) == E_NULL
    assert f(FAKE, 1, 1, 256, mats(I2SMatrix(FAKE, 64, 0.1, None, None)), 1,
             None, None, None, None) == E_NULL
    assert f(FAKE, 1, 1, 256, mats(good, I2SMatrix(MIS, 64, 0.1, FAKE, FAKE)), 2,
             None, None, None, None) == E_ALIGN
    assert f(FAKE, 1, 1, 256, mats(I2SMatrix(FAKE, -3, 0.1, FAKE, FAKE)), 1,
             None, None, None, None) == E_SHAPE
    assert f(MIS, 1, 1, 256, g1, 1, None, None, None, None) == E_ALIGN
    assert f(FAKE, 1, 1, 256, g1, 1, MIS, None, None, None) == E_ALIGN
    # N > BITNET_LINEAR_FUSED_MAX_N (2) needs the token buffers
    assert f(FAKE, 1, 3, 256, g1, 1, None, None, None, None) == E_NULL
    assert f(FAKE, 1, 9, 256, g1, 1, None, None, None, None) == E_NULL
    # N == 0 and matrices with M == 0 are no-ops
    assert f(None, 1, 0, 256, g1, 1, None, None, None, None) == OK
    assert f(None, 1, 0, 256, mats(I2SMatrix(None, 0, 0.1, None, None)), 1,
             None, None, None, None) == OK


@pytest.mark.parametrize("name,maxn", [("bitnet_gemm_i2s_i8_group", 1 << 21),
                                       ("bitnet_gemv_i2s_i8_group", 64)])
def test_group_validation(L, name, maxn):
    from ternary_weight_i2_amd._binding import I2SMatrix
    f = getattr(L, name)

    def mats(*ms):
        arr = (I2SMatrix * len(ms))()
        for i, m in enumerate(ms):
            arr[i] = m
        return arr
    good = I2SMatrix(FAKE, 64, 0.1, FAKE, FAKE)
    g1 = mats(good)
    assert f(g1, 0, 256, FAKE, FAKE, FAKE, 4, None) == E_SHAPE
    assert f(mats(*[good] * 9), 9, 256, FAKE, FAKE, FAKE, 4, None) == E_SHAPE
    assert f(None, 1, 256, FAKE, FAKE, FAKE, 4, None) == E_NULL
    assert f(g1, 1, 200, FAKE, FAKE, FAKE, 4, None) == E_SHAPE
    assert f(g1, 1, 256, FAKE, FAKE, FAKE, -1, None) == E_SHAPE
    assert f(g1, 1, 256, FAKE, FAKE, FAKE, maxn + 1, None) == E_SHAPE
    assert f(g1, 1, 256, None, FAKE, FAKE, 4, None) == E_NULL
    assert f(g1, 1, 256, FAKE, None, FAKE, 4, None) == E_NULL
    assert f(g1, 1, 256, MIS, FAKE, FAKE, 4, None) == E_ALIGN
    assert f(g1, 1, 256, FAKE, FAKE + 2, FAKE, 4, None) == E_ALIGN
    assert f(mats(good, I2SMatrix(None, 64, 0.1, FAKE, FAKE)), 2, 256, FAKE, FAKE, FAKE, 4,
             None) == E_NULL
    assert f(mats(I2SMatrix(FAKE, 64, 0.1, None, None)), 1, 256, FAKE, FAKE, FAKE, 4,
             None) == E_NULL
    assert f(mats(I2SMatrix(MIS, 64, 0.1, FAKE, FAKE)), 1, 256, FAKE, FAKE, FAKE, 4,
             None) == E_ALIGN
    assert f(mats(I2SMatrix(FAKE, 64, 0.1, FAKE + 1, None)), 1, 256, FAKE, FAKE, FAKE, 4,
             None) == E_ALIGN
    assert f(mats(I2SMatrix(FAKE, -2, 0.1, FAKE, FAKE)), 1, 256, FAKE, FAKE, FAKE, 4,
             None) == E_SHAPE
    assert name in _err(L)
    # no-ops: N == 0, or every matrix empty
    assert f(g1, 1, 256, None, None, None, 0, None) == OK
    assert f(mats(I2SMatrix(None, 0, 0.1, None, None)), 1, 256, None, None, None, 4, None) == OK
    assert _err(L) == ""


def test_conversion_validation(L):
    import ctypes
    a = ctypes.c_float(0.0)
    f = L.bitnet_absmean_i2s
    assert f(FAKE, 3, 4, 128, FAKE, ctypes.byref(a), None) == E_DTYPE
    assert f(FAKE, 0, 0, 128, FAKE, ctypes.byref(a), None) == E_SHAPE   # no rows: no scale
    assert "at least one row" in _err(L)
    assert f(FAKE, 0, 4, 100, FAKE, ctypes.byref(a), None) == E_SHAPE
    assert f(FAKE, 1, 4, 32768 + 128, FAKE, ctypes.byref(a), None) == E_SHAPE
    assert f(None, 0, 4, 128, FAKE, ctypes.byref(a), None) == E_NULL
    assert f(FAKE, 0, 4, 128, None, ctypes.byref(a), None) == E_NULL
    assert f(FAKE, 0, 4, 128, FAKE, None, None) == E_NULL
    assert f(FAKE + 8, 1, 4, 128, FAKE, ctypes.byref(a), None) == E_ALIGN
    assert f(FAKE, 0, 4, 128, MIS, ctypes.byref(a), None) == E_ALIGN
    g = L.bitnet_pack_i2s_f32
    assert g(FAKE, -1, 128, FAKE, None, None) == E_SHAPE
    assert g(FAKE, 4, 96, FAKE, None, None) == E_SHAPE
    assert g(None, 4, 128, FAKE, None, None) == E_NULL
    assert g(FAKE, 4, 128, None, None, None) == E_NULL
    assert g(FAKE + 4, 4, 128, FAKE, None, None) == E_ALIGN
    assert g(FAKE, 4, 128, MIS, None, None) == E_ALIGN
    a.value = 7.0
    assert g(None, 0, 128, None, ctypes.byref(a), None) == OK and a.value == 0.0
    assert _err(L) == ""


def test_ffn_act_quant_validation(L):
    f = L.bitnet_ffn_act_quant_i8
    assert f(FAKE, FAKE, None, 1e-5, -1, 256, FAKE, FAKE, FAKE, None) == E_SHAPE
    assert f(FAKE, FAKE, None, 1e-5, 2, 200, FAKE, FAKE, FAKE, None) == E_SHAPE
    assert f(FAKE, FAKE, None, 1e-5, 2, 32768 + 128, FAKE, FAKE, FAKE, None) == E_SHAPE
    assert f(FAKE, FAKE, None, 0.0, 2, 256, FAKE, FAKE, FAKE, None) == E_VALUE
    assert f(FAKE, FAKE, None, -1e-5, 2, 256, FAKE, FAKE, FAKE, None) == E_VALUE
    assert f(FAKE, FAKE, None, float("inf"), 2, 256, FAKE, FAKE, FAKE, None) == E_VALUE
    assert f(FAKE, FAKE, None, float("nan"), 2, 256, FAKE, FAKE, FAKE, None) == E_VALUE
    assert f(None, FAKE, None, 1e-5, 2, 256, FAKE, FAKE, FAKE, None) == E_NULL
    assert f(FAKE, FAKE, None, 1e-5, 2, 256, FAKE, None, FAKE, None) == E_NULL
    assert f(MIS, FAKE, None, 1e-5, 2, 256, FAKE, FAKE, FAKE, None) == E_ALIGN
    assert f(FAKE, FAKE, FAKE + 4, 1e-5, 2, 256, FAKE, FAKE, FAKE, None) == E_ALIGN
    assert f(FAKE, FAKE, None, 1e-5, 2, 256, MIS, FAKE, FAKE, None) == E_ALIGN
    assert "bitnet_ffn_act_quant_i8" in _err(L)
    assert f(None, None, None, 1e-5, 0, 256, None, None, None, None) == OK


def test_last_error_is_per_thread(L):
    import threading
    assert L.bitnet_pack_i2s(FAKE, 4, 100, FAKE, None) == E_SHAPE
    seen = {}

    def other():
        seen["msg"] = L.bitnet_last_error().decode()

    t = threading.Thread(target=other)
    t.start()
    t.join()
    assert seen["msg"] == ""
    assert "multiple of 128" in _err(L)


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    from ternary_weight_i2_amd import _binding
    monkeypatch.setattr(_binding, "_lib", None)
    monkeypatch.setattr(_binding, "_LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="no fallback"):
        _binding.load()


def test_product_path_does_not_touch_the_oracle():
    # the package and the C sources must not import, link or name the oracle
    pkg = os.path.join(ROOT, "ternary_weight_i2_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, fn), encoding="utf-8").read()
                assert "import oracle" not in text and "from oracle" not in text, fn
                assert "bitnet_oracle" not in text and "liboracle" not in text, fn


def test_binding_limits_match_header():
    from ternary_weight_i2_amd import _binding
    text = open(HEADER).read()
    for name, value in (("BITNET_GEMV_MAX_N", _binding.GEMV_MAX_N),
                        ("BITNET_LINEAR_FUSED_MAX_N", _binding.LINEAR_FUSED_MAX_N)):
        m = re.search(r"#define %s (\d+)" % name, text)
        assert m and int(m.group(1)) == value, name


# ------------------------------------------- binding argument checks (no GPU)
def _binding_cases():
    import torch
    import ternary_weight_i2_amd as bn
    i8, u8, f32, i32 = torch.int8, torch.uint8, torch.float32, torch.int32
    N, K, M = 3, 256, 40
    xq = torch.zeros((N, K), dtype=i8)
    xs = torch.zeros((N,), dtype=f32)
    xsum = torch.zeros((N,), dtype=i32)
    P = torch.zeros((M, K // 4), dtype=u8)
    g = torch.zeros((N, 512), dtype=f32)
    x = torch.zeros((N, K), dtype=f32)
    return bn, [
        # K of the weights does not match the tokens
        lambda: bn.gemv(torch.zeros((M, K // 4 + 32), dtype=u8), 1.0, xq, xs, xsum),
        lambda: bn.gemm(torch.zeros((M, K // 4), dtype=i8), 1.0, xq, xs, xsum),
        lambda: bn.gemv_lut(P, 1.0, xq.to(f32), xs, xsum),
        lambda: bn.gemv(P, 1.0, xq, xs[:2], xsum),
        lambda: bn.gemv(P, 1.0, xq, xs, xsum.to(torch.int64)),
        # short or mistyped caller outputs
        lambda: bn.gemv(P, 1.0, xq, xs, xsum, out=(torch.zeros((N, M - 1), dtype=i32), None)),
        lambda: bn.gemm(P, 1.0, xq, xs, xsum, out=(None, torch.zeros((N, M), dtype=torch.float64))),
        lambda: bn.quant_act(x, out=(xq[:, :128], xs, xsum)),
        lambda: bn.ffn_act_quant(g, g, gamma=torch.zeros(256, dtype=f32)),
        lambda: bn.ffn_act_quant(g, g, out=(torch.zeros((N, 256), dtype=i8), xs, xsum)),
        lambda: bn.gemm_group([(P, 1.0), (torch.zeros((7, K // 8), dtype=u8), 1.0)], xq, xs, xsum),
        lambda: bn.gemv_group([(P, 1.0)], xq, xs, xsum, out=[(None, torch.zeros((N + 1, M), dtype=f32))]),
        lambda: bn.gemv_group([(P, 1.0)] * 9, xq, xs, xsum),
        lambda: bn.linear(x, [(torch.zeros((M, K // 2), dtype=u8), 1.0)]),
        lambda: bn.linear(x, [(P, 1.0)], qout=(xq, xs, xsum[:1])),
        lambda: bn.absmean_pack(x, out=torch.zeros((N, K // 8), dtype=u8)),
        lambda: bn.pack(torch.zeros((2, 130), dtype=i8)),
    ]


def test_binding_refuses_bad_tensors_before_any_launch():
    """Every malformed tensor (wrong K, dtype or length, short output buffer)
    raises in the binding on the host -- these are CPU tensors, so reaching
    data_ptr() or the library would raise a different error."""
    bn, cases = _binding_cases()
    for i, case in enumerate(cases):
        with pytest.raises((TypeError, ValueError)) as e:
            case()
        assert "must live on the GPU" not in str(e.value), (i, str(e.value))
