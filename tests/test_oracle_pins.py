"""Pins of the CPU oracle to facts outside itself (CPU only).

Each test ties an oracle function to something the pages print (fixtures in
tests/golden/, each carrying its citation), a closed form, an invariant of
the mathematics, or brute force on tiny inputs.  The set is chosen so that a
dropped term, a wrong sign, a wrong shift or index, or a transposed operand in
the oracle fails at least one test.
"""
import os

import numpy as np
import pytest

from ternary_weight_i2_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _fixture(name):
    rows, kv = [], {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if ":" in line:
                k, v = line.split(":", 1)
                kv[k.strip()] = [int(t) for t in v.split()]
            else:
                rows.append([t for t in line.split()])
    return rows, kv


# ---------------------------------------------------------------- code map
def test_code_map_matches_page_table(orc):
    rows, _ = _fixture("p1_code_map.txt")
    assert len(rows) == 3
    for w, code, bits in rows:
        assert orc.code_of_weight(int(w)) == int(code)
        assert format(int(code), "02b") == bits
        assert orc.weight_of_code(int(code)) == int(w)
    # no other weight has a code, and code 3 has no weight
    for w in (-3, -2, 2, 3, 127, -128):
        assert orc.code_of_weight(w) == -1
    assert orc.weight_of_code(3) == 99


# ------------------------------------------------------- worked byte (P1 §8)
def test_worked_byte_pack(orc):
    _, kv = _fixture("p1_worked_byte.txt")
    w_top_first = kv["weights_top_first"]
    # the four weights that share byte 0 of a block are elements 0/32/64/96
    W = np.full((1, 128), 0, dtype=np.int8)
    for g, wv in enumerate(w_top_first):
        W[0, 32 * g] = wv
    P, bad = orc.pack_i2s(W)
    assert bad == 0
    assert int(P[0, 0]) == kv["byte"][0]
    # every other byte holds four zero weights = four codes 1 = 0b01010101
    assert all(int(b) == 0x55 for b in P[0, 1:])


def test_worked_byte_unpack(orc):
    _, kv = _fixture("p1_worked_byte.txt")
    P = np.full((1, 32), 0x55, dtype=np.uint8)
    P[0, 0] = kv["byte"][0]
    W, bad = orc.unpack_i2s(P, 128)
    assert bad == 0
    assert [int(W[0, 32 * g]) for g in range(4)] == kv["weights_top_first"]
    codes = [orc.code_of_weight(int(W[0, 32 * g])) for g in range(4)]
    assert codes == kv["codes_top_first"]


# ------------------------------------------------------ interleave (P1 §4-2)
def test_interleave_positions(orc):
    rows, _ = _fixture("p1_interleave.txt")
    for row in rows:
        byte_idx = int(row[0])
        elems = [int(t) for t in row[1:]]
        for slot, e in enumerate(elems):
            # one +1 (code 2) among -1s (code 0): exactly one non-zero byte
            W = np.full((1, 128), -1, dtype=np.int8)
            W[0, e] = 1
            P, _ = orc.pack_i2s(W)
            nz = np.nonzero(P[0])[0].tolist()
            assert nz == [byte_idx]
            # first listed element sits in the top two bits
            assert int(P[0, byte_idx]) == 2 << (6 - 2 * slot)


def test_blocks_and_rows_are_contiguous(orc):
    # A +1 at (m, k) with -1 elsewhere lights exactly one byte; its index must
    # grow by 32 per 128-block along k and by K/4 per row (rows back to back).
    M, K = 3, 384
    seen = []
    for m in range(M):
        for k in (0, 127, 128, 200, 383):
            W = np.full((M, K), -1, dtype=np.int8)
            W[m, k] = 1
            P, _ = orc.pack_i2s(W)
            nz = np.flatnonzero(P)
            assert len(nz) == 1
            seen.append((m, k, int(nz[0])))
    byte = {(m, k): b for m, k, b in seen}
    for m in range(M):
        assert byte[(m, 128)] - byte[(m, 0)] == 32
        assert byte[(m, 383)] - byte[(m, 0)] == 2 * 32 + 31
    for k in (0, 127, 128, 200, 383):
        assert byte[(1, k)] - byte[(0, k)] == K // 4
        assert byte[(2, k)] - byte[(1, k)] == K // 4


# -------------------------------------------------------- round trips
@pytest.mark.parametrize("M,K", [(1, 128), (5, 256), (17, 640), (64, 384)])
def test_pack_unpack_roundtrip(orc, M, K):
    rng = np.random.default_rng(M * 1000 + K)
    for dist in ("uniform", "half_zero"):
        W = synth.ternary(rng, M, K, dist)
        P, bad = orc.pack_i2s(W)
        assert bad == 0 and P.shape == (M, K // 4)
        W2, bad2 = orc.unpack_i2s(P, K)
        assert bad2 == 0
        np.testing.assert_array_equal(W, W2)


def test_all_valid_bytes_roundtrip(orc):
    # 3^4 = 81 bytes hold four valid codes; unpack then pack restores each.
    valid = [(a << 6) | (b << 4) | (c << 2) | d
             for a in range(3) for b in range(3) for c in range(3) for d in range(3)]
    assert len(valid) == 81
    P = np.full((81, 32), 0x55, dtype=np.uint8)
    for i, v in enumerate(valid):
        P[i, i % 32] = v
    W, bad = orc.unpack_i2s(P, 128)
    assert bad == 0
    P2, bad2 = orc.pack_i2s(W)
    assert bad2 == 0
    np.testing.assert_array_equal(P, P2)


def test_nonternary_and_code3_detected(orc):
    W = np.zeros((2, 128), dtype=np.int8)
    W[1, 77] = 2
    W[0, 3] = -5
    P, bad = orc.pack_i2s(W)
    assert bad == 2
    _, bad_codes = orc.unpack_i2s(P, 128)
    assert bad_codes == 2


# ---------------------------------------------------- worked dot (P1 §1-1)
def test_worked_dot_definition(orc):
    _, kv = _fixture("p1_worked_dot.txt")
    x = np.zeros((1, 128), dtype=np.int8)
    w = np.zeros((1, 128), dtype=np.int8)
    x[0, :4] = kv["x"]
    w[0, :4] = kv["w"]
    assert int(orc.dot_def(w, x)[0, 0]) == kv["dot"][0]


def test_worked_dot_raw_code_identity(orc):
    # sum(code*x) = sum(w*x) + sum(x): with the page's numbers 25 = 7 + 18.
    _, kv = _fixture("p1_worked_dot.txt")
    x = np.zeros((1, 128), dtype=np.int8)
    w = np.zeros((1, 128), dtype=np.int8)
    x[0, :4] = kv["x"]
    w[0, :4] = kv["w"]
    P, _ = orc.pack_i2s(w)
    qsum = np.array([sum(kv["x"])], dtype=np.int32)
    R, D = orc.dot_raw(P, x, qsum, 128)
    assert int(D[0, 0]) == kv["dot"][0]
    assert int(R[0, 0]) == kv["dot"][0] + sum(kv["x"]) == 25


# ------------------------------------------------------- brute force
@pytest.mark.parametrize("M,K,N", [(1, 128, 1), (7, 256, 3), (64, 384, 8), (33, 128, 5)])
def test_dot_def_vs_numpy_int64_matmul(orc, M, K, N):
    rng = np.random.default_rng(7 * M + K + N)
    W = synth.ternary(rng, M, K)
    q = rng.integers(-128, 128, size=(N, K), dtype=np.int8)
    ref = q.astype(np.int64) @ W.astype(np.int64).T
    np.testing.assert_array_equal(orc.dot_def(W, q), ref)


@pytest.mark.parametrize("M,K,N", [(3, 128, 1), (16, 512, 4), (9, 1152, 2)])
def test_dot_raw_equals_definition(orc, M, K, N):
    rng = np.random.default_rng(M + 11 * K + N)
    for dist in ("uniform", "half_zero"):
        W = synth.ternary(rng, M, K, dist)
        q = rng.integers(-128, 128, size=(N, K), dtype=np.int8)
        qsum = q.astype(np.int64).sum(1).astype(np.int32)
        P, _ = orc.pack_i2s(W)
        R, D = orc.dot_raw(P, q, qsum, K)
        Dd = orc.dot_def(W, q)
        np.testing.assert_array_equal(D, Dd)
        np.testing.assert_array_equal(R, Dd + qsum[:, None])


# ------------------------------------------------------- closed forms
def test_closed_forms(orc):
    rng = np.random.default_rng(99)
    M, K, N = 6, 256, 3
    q = rng.integers(-128, 128, size=(N, K), dtype=np.int8)
    qsum = q.astype(np.int64).sum(1)
    for fill, expect in ((0, 0 * qsum), (1, qsum), (-1, -qsum)):
        W = np.full((M, K), fill, dtype=np.int8)
        D = orc.dot_def(W, q)
        assert (D == expect[:, None]).all()
        P, _ = orc.pack_i2s(W)
        R, D2 = orc.dot_raw(P, q, qsum.astype(np.int32), K)
        np.testing.assert_array_equal(D2, D)
        if fill == 0:
            assert (R == qsum[:, None]).all()
    # one-hot token picks a column of W
    W = synth.ternary(rng, M, K)
    for k in (0, 31, 32, 127, 128, 255):
        e = np.zeros((1, K), dtype=np.int8)
        e[0, k] = 1
        np.testing.assert_array_equal(orc.dot_def(W, e)[0], W[:, k].astype(np.int64))
        e[0, k] = -3
        np.testing.assert_array_equal(orc.dot_def(W, e)[0], -3 * W[:, k].astype(np.int64))
    # duplicated token rows give identical outputs
    qq = np.concatenate([q[:1], q[:1]])
    D = orc.dot_def(W, qq)
    np.testing.assert_array_equal(D[0], D[1])


# ------------------------------------------------------- lookup-table route
@pytest.mark.parametrize("M,K,N", [(5, 128, 1), (16, 384, 3), (7, 1280, 2)])
def test_lut_dot_equals_definition(orc, M, K, N):
    # The table route must reach the definition's integers exactly.
    rng = np.random.default_rng(7 * M + K + N)
    for dist in ("uniform", "half_zero"):
        W = synth.ternary(rng, M, K, dist)
        q = rng.integers(-128, 128, size=(N, K), dtype=np.int8)
        qsum = q.astype(np.int64).sum(1).astype(np.int32)
        P, _ = orc.pack_i2s(W)
        R, D = orc.dot_lut(P, q, qsum, K)
        Dd = orc.dot_def(W, q)
        np.testing.assert_array_equal(D, Dd)
        np.testing.assert_array_equal(R, Dd + qsum[:, None])


def test_lut_one_hot_token_reads_each_code(orc):
    # A one-hot token x = v*e_k makes R[m] = code(W[m][k]) * v: every position
    # of a block must reach its own weight through its group and nibble half
    # (a swapped pair, a swapped nibble or a transposed table index fails).
    rng = np.random.default_rng(123)
    M, K = 6, 256
    W = synth.ternary(rng, M, K)
    P, _ = orc.pack_i2s(W)
    for k in range(K):
        for v in (1, -7):
            e = np.zeros((1, K), dtype=np.int8)
            e[0, k] = v
            R, D = orc.dot_lut(P, e, np.array([v], dtype=np.int32), K)
            np.testing.assert_array_equal(R[0], (W[:, k].astype(np.int64) + 1) * v)
            np.testing.assert_array_equal(D[0], W[:, k].astype(np.int64) * v)


def test_lut_tables_closed_forms(orc):
    rng = np.random.default_rng(321)
    K = 384
    q = rng.integers(-128, 128, size=K, dtype=np.int8)
    T = orc.lut_tables(q, K).astype(np.int64)
    assert T.shape == (K // 2, 16)
    # both codes 0 contribute nothing
    assert (T[:, 0] == 0).all()
    # every activation sits in exactly one group: the all-zero-weight entries
    # (codes 1,1) add up to the token sum, and so do the lone-first plus
    # lone-second entries (codes 1,0 and 0,1)
    assert T[:, 5].sum() == q.astype(np.int64).sum()
    assert T[:, 4].sum() + T[:, 1].sum() == q.astype(np.int64).sum()
    # each table is bilinear in the two codes: entry(a,b) = a*entry(1,0) + b*entry(0,1)
    for a in range(4):
        for b in range(4):
            np.testing.assert_array_equal(T[:, 4 * a + b], a * T[:, 4] + b * T[:, 1])
    # the first activation of the high-nibble group of byte t is the one at
    # block start + t mod 32 (one-hot probes)
    for k in (0, 5, 31, 32, 63, 64, 96, 127, 128, 200, 383):
        e = np.zeros(K, dtype=np.int8)
        e[k] = 3
        Te = orc.lut_tables(e, K)
        nz = np.nonzero(Te[:, 4] + Te[:, 1])[0]
        blk, p = divmod(k, 128)
        t = blk * 32 + p % 32
        g = 2 * t + (1 if p >= 64 else 0)
        assert list(nz) == [g]
        first = (p % 64) < 32
        assert Te[g, 4] == (3 if first else 0) and Te[g, 1] == (0 if first else 3)


def test_lut_counts_code3_like_the_raw_dot(orc):
    # Any nibble is a valid table index: a code-3 slot contributes 3*x, as in
    # the raw-code walk (both routes give the same R on arbitrary bytes).
    rng = np.random.default_rng(77)
    M, K, N = 9, 512, 2
    P = rng.integers(0, 256, size=(M, K // 4), dtype=np.uint8)
    q = rng.integers(-128, 128, size=(N, K), dtype=np.int8)
    qsum = q.astype(np.int64).sum(1).astype(np.int32)
    R1, D1 = orc.dot_lut(P, q, qsum, K)
    R2, D2 = orc.dot_raw(P, q, qsum, K)
    np.testing.assert_array_equal(R1, R2)
    np.testing.assert_array_equal(D1, D2)
    # all bytes 0xFF: every weight has code 3, so R = 3 * sum(x)
    P3 = np.full((1, K // 4), 0xFF, dtype=np.uint8)
    R3, _ = orc.dot_lut(P3, q, qsum, K)
    np.testing.assert_array_equal(R3[:, 0], 3 * q.astype(np.int64).sum(1))


# ------------------------------------------------------- quantisation
def test_quant_absmax_maps_to_127(orc):
    rng = np.random.default_rng(5)
    x = rng.standard_normal((4, 512), dtype=np.float32)
    q, s, qs = orc.quant_act(x)
    for n in range(4):
        k = int(np.argmax(np.abs(x[n])))
        assert int(q[n, k]) == (127 if x[n, k] > 0 else -127)
        assert np.abs(q[n]).max() == 127
        assert int(qs[n]) == int(q[n].astype(np.int64).sum())


def test_quant_constant_and_zero_rows(orc):
    x = np.zeros((3, 256), dtype=np.float32)
    x[0, :] = 0.37
    x[1, :] = -2.5
    q, s, qs = orc.quant_act(x)
    assert (q[0] == 127).all() and int(qs[0]) == 127 * 256
    assert (q[1] == -127).all() and int(qs[1]) == -127 * 256
    # all-zero token: floor 1e-5 (fp32) -> s ~ 1.27e7, q = 0, sum 0
    assert (q[2] == 0).all() and int(qs[2]) == 0
    assert abs(float(s[2]) * 1e-5 - 127.0) < 127.0 * 1e-6
    # tiny but non-zero token below the floor: still divided by the floor
    xt = np.full((1, 128), 1e-7, dtype=np.float32)
    qt, st, _ = orc.quant_act(xt)
    assert st[0] == s[2] and (qt == 1).all()   # 1e-7 * 1.27e7 = 1.27 -> 1


def test_quant_scale_is_exact_division(orc):
    # s is the correctly rounded fp32 value of 127 / max|x| (IEEE division):
    # exactly representable cases pin it without retyping the formula.
    for amax, s_exact in ((127.0, 1.0), (254.0, 0.5), (2.0, 63.5), (0.5, 254.0)):
        x = np.zeros((1, 128), dtype=np.float32)
        x[0, 5] = amax
        _, s, _ = orc.quant_act(x)
        assert float(s[0]) == s_exact


def test_quant_round_half_even(orc):
    # amax 127 -> s = 1 exactly, so q = round(x) on exact halves.
    x = np.zeros((1, 128), dtype=np.float32)
    x[0, 0] = 127.0
    halves = [0.5, 1.5, 2.5, 3.5, -0.5, -1.5, -2.5, 126.5]
    expect = [0, 2, 2, 4, 0, -2, -2, 126]
    x[0, 1:1 + len(halves)] = halves
    q, _, _ = orc.quant_act(x)
    assert q[0, 1:1 + len(halves)].tolist() == expect
    # amax 2 -> s = 63.5: x = 1 gives 63.5 -> 64, x = -1 -> -64, x = 0.5 -> 31.75 -> 32
    x = np.zeros((1, 128), dtype=np.float32)
    x[0, :4] = [2.0, 1.0, -1.0, 0.5]
    q, _, _ = orc.quant_act(x)
    assert q[0, :4].tolist() == [127, 64, -64, 32]


def test_quant_multiply_form_not_divide(orc):
    """"BitNet 딥다이브" §4-5 quantises with the multiplier s = 127/absmax
    (q = round(x*s)); "bitnet.rs" divides by alpha = absmax/127.  On the stored
    elements the two fp32 forms round to codes one apart; the oracle must give
    the multiply form's code (reading: the multiplier of §4-5)."""
    rows = []
    with open(os.path.join(GOLDEN, "quant_mul_vs_div.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                a, x = (int(t, 16) for t in line.split())
                rows.append((np.uint32(a).view(np.float32), np.uint32(x).view(np.float32)))
    assert len(rows) >= 2
    for amax, xv in rows:
        tok = np.zeros((1, 128), np.float32)
        tok[0, 0] = amax
        tok[0, 1] = xv
        s_mul = np.float32(127.0 / np.float64(amax))          # correctly rounded quotient
        alpha = np.float32(np.float64(amax) / 127.0)
        q_mul = int(np.rint(np.float32(xv) * s_mul))
        q_div = int(np.rint(np.float32(xv) / alpha))
        assert abs(q_mul - q_div) == 1                        # the forms disagree here
        q, s, _ = orc.quant_act(tok)
        assert s[0] == s_mul
        assert int(q[0, 1]) == q_mul


def test_quant_rounding_error_bound(orc):
    # |x - q/s| <= 0.5/s elementwise (rounding to nearest), q within [-127,127].
    rng = np.random.default_rng(17)
    x = rng.standard_normal((8, 2560), dtype=np.float32) * np.float32(3.0)
    q, s, _ = orc.quant_act(x)
    err = np.abs(x.astype(np.float64) - q.astype(np.float64) / s[:, None].astype(np.float64))
    assert (err <= 0.5 / s[:, None].astype(np.float64) * (1 + 1e-6)).all()
    assert np.abs(q.astype(np.int32)).max() <= 127


def test_quant_outlier_row(orc):
    rng = synth.rng_for("b2_sparse", 0, "q", "act")
    xb = synth.tokens_bf16(rng, 4, 2560, outliers=True,
                           orng=synth.rng_for("b2_sparse", 0, "q", "outlier"))
    x = synth.bf16_bits_to_f32(xb)
    q, s, _ = orc.quant_act(xb)
    for n in (1, 3):
        k = int(np.argmax(np.abs(x[n])))
        assert abs(float(x[n, k])) == 20.0
        assert abs(int(q[n, k])) == 127
        rest = np.delete(np.abs(q[n].astype(np.int32)), k)
        bound = int(np.ceil(127 * np.delete(np.abs(x[n]), k).max() / 20.0))
        assert rest.max() <= bound <= 30


def test_quant_bf16_equals_exact_f32(orc):
    rng = np.random.default_rng(3)
    xb = synth.f32_to_bf16_bits(rng.standard_normal((5, 640), dtype=np.float32))
    xf = synth.bf16_bits_to_f32(xb)
    np.testing.assert_array_equal(orc.bf16_to_f32(xb[0, :16]), xf[0, :16])
    a = orc.quant_act(xb)
    b = orc.quant_act(np.ascontiguousarray(xf))
    for u, v in zip(a, b):
        np.testing.assert_array_equal(u, v)


# ------------------------------------------------------- epilogue
def test_epilogue_closed_forms(orc):
    D = np.array([[0, 1, -1, 1000, -3641344]], dtype=np.int64)
    s = np.array([2.0], dtype=np.float32)
    y = orc.epilogue(D, 0.25, s)
    assert y[0, 0] == 0.0
    # alpha/s = 1/8 exactly, so every value is exact in binary64
    assert y[0, 1:].tolist() == [0.125, -0.125, 125.0, -455168.0]


def test_epilogue_dequantises_the_float_product(orc):
    # y approximates alpha * W @ x: the only error is the activation rounding,
    # |y - alpha * sum_k w x| <= alpha * sum_k |w| * 0.5 / s.  Swapping the
    # roles of alpha and s, or multiplying by s, breaks this bound.
    rng = np.random.default_rng(23)
    M, K, N = 40, 1024, 3
    W = synth.ternary(rng, M, K)
    alpha = 0.0625
    x = rng.standard_normal((N, K), dtype=np.float32)
    q, s, _ = orc.quant_act(x)
    y = orc.epilogue(orc.dot_def(W, q), alpha, s)
    exact = alpha * (x.astype(np.float64) @ W.astype(np.float64).T)
    bound = alpha * np.abs(W).sum(1)[None, :] * 0.5 / s[:, None].astype(np.float64)
    assert (np.abs(y - exact) <= bound * (1 + 1e-9)).all()
    assert np.abs(y - exact).max() > 0  # the bound is not vacuous


# ------------------------------------------------------- threaded driver
def test_linear_driver_matches_pieces(orc):
    rng = np.random.default_rng(31)
    M, K, N = 57, 640, 4
    W = synth.ternary(rng, M, K)
    P, _ = orc.pack_i2s(W)
    x = rng.standard_normal((N, K), dtype=np.float32)
    q, s, qs = orc.quant_act(x)
    D = orc.dot_def(W, q)
    y = orc.epilogue(D, 0.03, s)
    for nt in (1, 3, 8):
        D2, y2 = orc.linear_i2s(P, K, q, s, np.float32(0.03), nthreads=nt)
        np.testing.assert_array_equal(D2, D)
        np.testing.assert_allclose(y2, orc.epilogue(D, float(np.float32(0.03)), s), rtol=1e-15)
    D3, _ = orc.linear_i2s(P, K, q, s, np.float32(0.03), rows=(10, 20), nthreads=2)
    np.testing.assert_array_equal(D3, D[:, 10:30])
    assert y.shape == (N, M)


# ------------------------------------------------------- stored regression
def test_stored_regression_values(orc):
    """Values written by tests/golden/make_golden.py (oracle only)."""
    path = os.path.join(GOLDEN, "oracle_single_rows.txt")
    _, kv = _fixture("oracle_single_rows.txt")
    W, alpha = synth.matrix("single", "w")
    x = synth.activations("single", "w", 1)
    q, s, qs = orc.quant_act(x)
    assert int(qs[0]) == kv["qsum"][0]
    P, _ = orc.pack_i2s(W)
    assert [int(b) for b in P[0, :16]] == kv["packed_row0_first16"]
    R, D = orc.dot_raw(P, q, qs, W.shape[1])
    rows = kv["rows"]
    assert [int(D[0, r]) for r in rows] == kv["dot"]
    assert os.path.exists(path)


# ------------------------------------------------------- AbsMean ternariser
def _float_fixture(name):
    kv = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#") and ":" in line:
                k, v = line.split(":", 1)
                kv[k.strip()] = [float(t) for t in v.split()]
    return kv


def test_absmean_worked_example(orc):
    """[P1 §6-2]: mean |w| = 0.4 and w / 0.4 = +-0.5, +-1.5 -- exact ties in
    fp32, so q is decided by the rounding rule (reading: half to even)."""
    kv = _float_fixture("p1_absmean_example.txt")
    w = np.array(kv["w"], dtype=np.float32)
    alpha = orc.absmean_alpha(w)
    assert np.float32(alpha) == np.float32(kv["mean_abs"][0])
    ratio = w / np.float32(alpha)                 # IEEE fp32 division
    np.testing.assert_array_equal(ratio, np.array(kv["ratio"], dtype=np.float32))
    q = orc.absmean_ternary(w, alpha)
    np.testing.assert_array_equal(q, np.clip(np.rint(ratio), -1, 1).astype(np.int8))
    np.testing.assert_array_equal(q, [-1, 0, 0, 1])   # half away from zero: [-1,-1,1,1]


def test_absmean_floor_and_constant_tensors(orc):
    z = np.zeros((4, 128), np.float32)
    assert orc.absmean_alpha(z) == np.float32(1e-5)
    assert not orc.absmean_ternary(z, orc.absmean_alpha(z)).any()
    tiny = np.full((2, 128), 1e-7, np.float32)      # mean below the floor
    a = orc.absmean_alpha(tiny)
    assert a == np.float32(1e-5)
    assert not orc.absmean_ternary(tiny, a).any()
    c = np.full((8, 128), -0.25, np.float32)
    a = orc.absmean_alpha(c)
    assert a == np.float32(0.25)
    assert (orc.absmean_ternary(c, a) == -1).all()


def test_absmean_of_scaled_ternary_is_identity(orc):
    """W = c*T: mean |W| = c * (nonzero fraction) <= c, so W / alpha rounds
    to T for every element."""
    rng = np.random.default_rng(3)
    T = synth.ternary(rng, 16, 256)
    frac = np.count_nonzero(T) / T.size
    for c in (0.01, 0.37, 3.0):
        W = T.astype(np.float32) * np.float32(c)
        a = orc.absmean_alpha(W)
        assert abs(a - c * frac) <= 1e-6 * c
        np.testing.assert_array_equal(orc.absmean_ternary(W, a), T)


def test_absmean_symmetry_and_power_of_two_scaling(orc):
    rng = np.random.default_rng(4)
    W = (rng.standard_normal((32, 384)) * 0.02).astype(np.float32)
    a = orc.absmean_alpha(W)
    q = orc.absmean_ternary(W, a)
    assert orc.absmean_alpha(-W) == a
    np.testing.assert_array_equal(orc.absmean_ternary(-W, a), -q)
    for k in (-3, 5):
        s = np.float32(2.0 ** k)
        assert orc.absmean_alpha(W * s) == np.float32(a) * s
        np.testing.assert_array_equal(orc.absmean_ternary(W * s, orc.absmean_alpha(W * s)), q)


def test_absmean_half_normal_statistics(orc):
    """For N(0, sigma^2) weights mean |w| -> sigma*sqrt(2/pi), and q = 0 exactly
    when |z| < 0.5*sqrt(2/pi), which has probability erf(0.5/sqrt(pi))."""
    import math
    rng = np.random.default_rng(5)
    sigma = 0.02
    W = (rng.standard_normal((512, 1024)) * sigma).astype(np.float32)
    a = orc.absmean_alpha(W)
    assert abs(a / (sigma * math.sqrt(2 / math.pi)) - 1) < 3e-3
    zero = np.mean(orc.absmean_ternary(W, a) == 0)
    assert abs(zero - math.erf(0.5 / math.sqrt(math.pi))) < 3e-3


def test_absmean_matches_numpy_on_random_tensors(orc):
    rng = np.random.default_rng(6)
    for shape in ((3, 128), (17, 640), (64, 1024)):
        W = (rng.standard_normal(shape) * 0.05).astype(np.float32)
        a_ref = np.float32(np.abs(W.astype(np.float64)).sum() / W.size)
        a = orc.absmean_alpha(W)
        assert a == max(a_ref, np.float32(1e-5))
        q_ref = np.clip(np.rint(W / np.float32(a)), -1, 1).astype(np.int8)
        np.testing.assert_array_equal(orc.absmean_ternary(W, a), q_ref)


def test_absmean_bf16_is_f32_of_widened_bits(orc):
    rng = np.random.default_rng(7)
    W = (rng.standard_normal((16, 256)) * 0.03).astype(np.float32)
    bits = synth.f32_to_bf16_bits(W)
    wide = orc.bf16_to_f32(bits)
    assert orc.absmean_alpha(bits) == orc.absmean_alpha(wide)
    np.testing.assert_array_equal(orc.absmean_ternary(bits, orc.absmean_alpha(bits)),
                                  orc.absmean_ternary(wide, orc.absmean_alpha(wide)))


def test_absmean_equals_fsum_definition(orc):
    """alpha = fp32(S / n) with S the exactly rounded binary64 sum of |w|:
    checked against math.fsum (an independent exactly rounded sum) on random
    tensors, fp32 and bf16."""
    import math
    rng = np.random.default_rng(61)
    for shape in ((3, 128), (17, 640), (64, 1024)):
        W = (rng.standard_normal(shape) * 0.05).astype(np.float32)
        S = math.fsum(np.abs(W.astype(np.float64)).ravel())
        assert orc.absmean_alpha(W) == max(np.float32(S / W.size), np.float32(1e-5))
        bits = synth.f32_to_bf16_bits(W)
        Sb = math.fsum(np.abs(synth.bf16_bits_to_f32(bits).astype(np.float64)).ravel())
        assert orc.absmean_alpha(bits) == max(np.float32(Sb / W.size), np.float32(1e-5))


def test_absmean_sum_is_order_free(orc):
    """w = [4, 2^-22, 2^-51, 2^-51]: the exact sum is 4 + 2^-22 + 2^-50 (one
    binary64 ulp above 4 + 2^-22), so the mean 1 + 2^-24 + 2^-52 lies above
    the fp32 midpoint 1 + 2^-24 and alpha = 1 + 2^-23.  Summed left to right in
    binary64 each 2^-51 is a tie that rounds away (mean exactly the midpoint,
    alpha = 1); summed right to left they survive.  The oracle gives
    1 + 2^-23 for every order."""
    import itertools
    base = np.array([4.0, 2.0 ** -22, 2.0 ** -51, 2.0 ** -51], np.float32)
    want = np.float32(1 + 2.0 ** -23)
    naive = set()
    for perm in itertools.permutations(range(4)):
        w = base[list(perm)]
        assert orc.absmean_alpha(w) == want
        acc = 0.0
        for v in w.astype(np.float64):
            acc += v
        naive.add(float(np.float32(acc / 4)))
    assert naive == {1.0, float(want)}      # a fixed-order binary64 sum depends on the order
    # the same weights in a 1 x 128 tensor (the rest zero): alpha = (1 + 2^-23) / 32
    w128 = np.zeros((1, 128), np.float32)
    w128[0, :4] = base
    assert orc.absmean_alpha(w128) == want / np.float32(32)


# ------------------------------------------- sign/threshold float packer
def test_sign_ternary_threshold_edges(orc):
    """[P1 §4-2]: |v| < 1e-6 is zero, positive -> +1, negative -> -1; the
    comparison is against the binary64 constant, so fp32(1e-6), which lies
    just below it, still counts as zero."""
    one_e6 = np.float32(1e-6)
    above = np.nextafter(one_e6, np.float32(1))
    v = np.array([0.0, -0.0, 5e-7, -5e-7, one_e6, -one_e6, above, -above, 2.0, -3.0],
                 dtype=np.float32)
    q, wmax, bad = orc.sign_ternary(v)
    np.testing.assert_array_equal(q, [0, 0, 0, 0, 0, 0, 1, -1, 1, -1])
    assert wmax == 3.0 and bad == 0
    q, wmax, bad = orc.sign_ternary(np.array([1.0, np.nan, -np.inf, 0.5], np.float32))
    assert bad == 2 and wmax == 1.0
    np.testing.assert_array_equal(q, [1, 0, 0, 1])


def test_sign_ternary_of_scaled_ternary_round_trips(orc):
    rng = np.random.default_rng(8)
    T = synth.ternary(rng, 8, 384)
    W = T.astype(np.float32) * np.float32(0.0731)
    q, wmax, bad = orc.sign_ternary(W)
    np.testing.assert_array_equal(q, T)
    assert bad == 0 and wmax == np.float32(0.0731)


# ------------------------------------------- exactly rounded sums
def test_exact_sum_matches_fsum(orc):
    """orc_exact_sum against math.fsum (Shewchuk's exactly rounded sum in the
    Python library) on non-negative values spanning the whole binary64 range,
    subnormals included."""
    import math
    rng = np.random.default_rng(71)
    for trial in range(300):
        n = int(rng.integers(1, 400))
        e = rng.integers(-1074, 1000, size=n) if trial % 3 == 0 else rng.integers(-80, 40, size=n)
        x = np.ldexp(rng.random(n) + 0.5, e)
        x[rng.random(n) < 0.1] = 0.0
        assert orc.exact_sum(x) == math.fsum(x)
    # squares of fp32 values, as the FFN sub-norm forms them
    h = (rng.standard_normal(6912) * np.exp2(rng.integers(-30, 10, 6912))).astype(np.float32)
    sq = h.astype(np.float64) ** 2
    assert orc.exact_sum(sq) == math.fsum(sq)


def test_exact_sum_rounds_half_to_even(orc):
    one = 1.0
    ulp = 2.0 ** -52
    tiny = 5e-324
    # 1 + 2^-53 is a midpoint: ties to even keep 1; anything above goes up
    assert orc.exact_sum(np.array([one, 2.0 ** -53])) == one
    assert orc.exact_sum(np.array([one, 2.0 ** -53, tiny])) == one + ulp
    # (1 + 2^-52) + 2^-53: the tie goes to the even neighbour 1 + 2^-51
    assert orc.exact_sum(np.array([one + ulp, 2.0 ** -53])) == one + 2 * ulp
    # below half an ulp: down, however many tiny addends leave it below
    assert orc.exact_sum(np.array([one] + [2.0 ** -60] * 127)) == one
    assert orc.exact_sum(np.array([one] + [2.0 ** -60] * 129)) == one + ulp
    # subnormal and overflow-edge sums are exact
    assert orc.exact_sum(np.array([tiny] * 3)) == 3 * tiny
    big = np.finfo(np.float64).max / 2
    assert orc.exact_sum(np.array([big, big])) == np.finfo(np.float64).max
    assert orc.exact_sum(np.zeros(5)) == 0.0
    with pytest.raises(ValueError):
        orc.exact_sum(np.array([1.0, -1.0]))


def test_exact_sum_is_order_free(orc):
    """Random orders of an array whose left-to-right binary64 sums differ
    give one exactly rounded sum."""
    import math
    rng = np.random.default_rng(72)
    x = np.concatenate([[1.0], np.full(300, 2.0 ** -54), rng.random(50) * 1e-3])
    seen = set()
    for _ in range(20):
        p = rng.permutation(x)
        acc = 0.0
        for v in p:
            acc += v
        seen.add(acc)
        assert orc.exact_sum(p) == math.fsum(x)
    assert len(seen) > 1


# ------------------------------------------- squared-ReLU gated FFN glue
def _rms_ref(h, gamma, eps):
    """h / sqrt(mean(h^2) + eps) * gamma, float64 (numpy's own sum order)."""
    h = h.astype(np.float64)
    r = h / np.sqrt(np.mean(h * h, axis=1, keepdims=True) + eps)
    return r if gamma is None else r * gamma.astype(np.float64)


def test_ffn_sqrelu_gate_and_norm(orc):
    """[P4 "Forward Pass"]: sqrelu(gate) (x) up, then the sub-norm: channels
    with gate <= 0 are exactly zero, the rest follow h / rms(h) * gamma."""
    rng = np.random.default_rng(11)
    N, F = 3, 256
    g = rng.standard_normal((N, F)).astype(np.float32)
    u = rng.standard_normal((N, F)).astype(np.float32)
    gamma = rng.uniform(0.5, 1.5, F).astype(np.float32)
    q, s, qs, v = orc.ffn_act_quant(g, u, gamma, 1e-5)
    assert (v[g <= 0] == 0).all() and (q[g <= 0] == 0).all()
    h = np.maximum(g, 0).astype(np.float64) ** 2 * u
    np.testing.assert_allclose(v, _rms_ref(h, gamma, 1e-5), rtol=2e-6, atol=1e-30)
    # the quantisation step is the activation quantiser's
    q2, s2, qs2 = orc.quant_act(v)
    np.testing.assert_array_equal(q, q2)
    np.testing.assert_array_equal(s.view(np.uint32), s2.view(np.uint32))
    np.testing.assert_array_equal(qs, qs2)


def test_ffn_unit_rms_and_constant_rows(orc):
    rng = np.random.default_rng(12)
    g = np.abs(rng.standard_normal((4, 512))).astype(np.float32) + 0.1
    u = rng.standard_normal((4, 512)).astype(np.float32)
    _, _, _, v = orc.ffn_act_quant(g, u, None, 0.0)
    np.testing.assert_allclose(np.mean(v.astype(np.float64) ** 2, axis=1), 1.0, rtol=1e-6)
    g = np.full((2, 128), 0.75, np.float32)
    u = np.ones((2, 128), np.float32)
    q, s, qs, v = orc.ffn_act_quant(g, u, None, 0.0)
    np.testing.assert_allclose(v, 1.0, rtol=1.2e-7)
    assert (q == 127).all() and (qs == 127 * 128).all()


def test_ffn_power_of_two_invariances(orc):
    """Scaling the gate by 2 scales h by exactly 4 and the sum of squares by
    16, so (eps = 0) the normalised values and codes are unchanged bit for
    bit; doubling gamma doubles v and halves s exactly."""
    rng = np.random.default_rng(13)
    g = rng.standard_normal((5, 384)).astype(np.float32)
    u = rng.standard_normal((5, 384)).astype(np.float32)
    gamma = rng.uniform(0.5, 1.5, 384).astype(np.float32)
    q, s, qs, v = orc.ffn_act_quant(g, u, gamma, 0.0)
    q2, s2, qs2, v2 = orc.ffn_act_quant(g * np.float32(2), u, gamma, 0.0)
    np.testing.assert_array_equal(v, v2)
    np.testing.assert_array_equal(q, q2)
    q3, s3, qs3, v3 = orc.ffn_act_quant(g, u, gamma * np.float32(2), 0.0)
    np.testing.assert_array_equal(v3, v * np.float32(2))
    np.testing.assert_array_equal(q3, q)
    np.testing.assert_array_equal(s3, s / np.float32(2))


def test_ffn_eps_dominates_tiny_activations(orc):
    g = np.full((1, 128), 1e-3, np.float32)
    u = np.ones((1, 128), np.float32)
    _, _, _, v = orc.ffn_act_quant(g, u, None, 1e-5)
    h = np.float64(np.float32(1e-3)) ** 2
    np.testing.assert_allclose(v, h / np.sqrt(h * h + 1e-5), rtol=2e-7)
    # a token whose gate is never positive normalises to zero (eps > 0)
    q, s, qs, v = orc.ffn_act_quant(-np.abs(g), u, None, 1e-5)
    assert not v.any() and not q.any() and qs[0] == 0
    assert s[0] == np.float32(127.0 / 1e-5)


def test_ffn_norm_factor_from_exact_sum(orc):
    """The factor is fp32(1 / sqrt(S / F + eps)) with S the exactly rounded
    sum of the (exact) squares: with S from math.fsum, v = (h * c) * gamma in
    fp32 must equal the oracle's v bit for bit."""
    import math
    rng = np.random.default_rng(73)
    N, F = 4, 640
    g = (rng.standard_normal((N, F)) * np.exp2(rng.integers(-12, 3, (N, F)))).astype(np.float32)
    u = rng.standard_normal((N, F)).astype(np.float32)
    gamma = rng.uniform(0.5, 1.5, F).astype(np.float32)
    for eps in (1e-5, 1e-6):
        _, _, _, v = orc.ffn_act_quant(g, u, gamma, eps)
        for n in range(N):
            r = np.maximum(g[n], np.float32(0))
            h = (r * r) * u[n]
            S = math.fsum(h.astype(np.float64) ** 2)
            c = np.float32(1.0 / math.sqrt(S / F + float(np.float32(eps))))
            np.testing.assert_array_equal(v[n].view(np.uint32), ((h * c) * gamma).view(np.uint32))


def test_ffn_is_channel_order_free(orc):
    """Permuting the channels of g, u and gamma permutes v and the codes and
    leaves s and the code sum unchanged, bit for bit (the sub-norm's sum has
    no order)."""
    rng = np.random.default_rng(74)
    N, F = 3, 6912
    g = (rng.standard_normal((N, F)) * np.exp2(rng.integers(-20, 4, (N, F)))).astype(np.float32)
    u = rng.standard_normal((N, F)).astype(np.float32)
    gamma = rng.uniform(0.5, 1.5, F).astype(np.float32)
    q, s, qs, v = orc.ffn_act_quant(g, u, gamma, 1e-6)
    p = rng.permutation(F)
    q2, s2, qs2, v2 = orc.ffn_act_quant(np.ascontiguousarray(g[:, p]), np.ascontiguousarray(u[:, p]),
                                        np.ascontiguousarray(gamma[p]), 1e-6)
    np.testing.assert_array_equal(v2.view(np.uint32), v[:, p].view(np.uint32))
    np.testing.assert_array_equal(q2, q[:, p])
    np.testing.assert_array_equal(s2.view(np.uint32), s.view(np.uint32))
    np.testing.assert_array_equal(qs2, qs)


def test_ffn_factor_takes_the_exact_sum(orc):
    """A token (tests/ffn_cases.py) whose left-to-right binary64 sum of
    squares drops one ulp that the exact sum keeps, at a point where that ulp
    changes the fp32 factor: the oracle's v follows the exact sum."""
    import ffn_cases
    g, u, eps, c_exact, c_ltr = ffn_cases.order_sensitive_token()
    assert c_exact != c_ltr
    q, s, qs, v = orc.ffn_act_quant(g, u, None, eps)
    assert v[0, 0] == np.float32(11.0) * c_exact
    assert v[0, 0] != np.float32(11.0) * c_ltr


def test_ffn_carry_tokens_follow_the_exact_sum(orc):
    """Constructed tokens (tests/ffn_cases.py) whose sum of squares is the
    midpoint 1 + 2^-53 or just beside it: the oracle's factor is the one of
    math.fsum's sum (ties to even), checked through v = h * c."""
    import math
    import ffn_cases
    eps = float(np.float32(1.4e-45))
    cases = [ffn_cases.carry_token(e) for e in (-1, 0, 1)] + [ffn_cases.deep_carry_token()]
    sums = []
    for g, u in cases:
        F = u.shape[1]
        S = math.fsum(u[0].astype(np.float64) ** 2)
        sums.append(S)
        c = np.float32(1.0 / math.sqrt(S / F + eps))
        _, _, _, v = orc.ffn_act_quant(g, u, None, eps)
        np.testing.assert_array_equal(v[0].view(np.uint32), (u[0] * c).view(np.uint32))
    assert sums == [1.0, 1.0, 1.0 + 2.0 ** -52, 1.0]
