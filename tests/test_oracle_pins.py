"""Pins of the CPU oracle against what the pages and the mathematics fix.

Nothing here re-types the oracle's own formulas: each test checks it against an independent
construction (the Kronecker definition of the Hadamard matrix and its closed-form entries,
the other page's recursive transform written out as its matrix, hand-worked fixtures under tests/golden/, closed forms, invariants, brute force,
torch's float8 conversions).
"""
import os

import numpy as np
import pytest

import oracle as O
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# independent constructions
# ---------------------------------------------------------------------------

def sylvester(n):
    """Unnormalised Hadamard matrix by the Kronecker recursion H_2n = [[H, H], [H, -H]]
    ("QWHA方法：基于Walsh-Hadamard变换的高效大模型微调技术", s2.1)."""
    h = np.ones((1, 1), dtype=np.int64)
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def bit_reversed_sylvester(n):
    """Matrix of the recursive even/odd transform described on the HALO overview page
    ("企业官网建设流程全解析", s2.1): the two halves of its output are the sum and the
    difference of the transforms of the even- and odd-indexed inputs, so the output's top
    index bit pairs with the input's lowest bit, and so on down; written out, entry (i, j) is
    (-1)^popcount(rev(i) & j) with rev the reversal of i's log2(n) bits.  Unnormalised."""
    bits = n.bit_length() - 1
    rev = bit_reverse_perm(n)
    i = rev[:, None]
    j = np.arange(n)[None, :]
    pc = np.vectorize(lambda v: bin(int(v)).count("1"))(i & j)
    return np.where(pc % 2 == 0, 1, -1).astype(np.int64) if bits else np.ones((1, 1), np.int64)


def bit_reverse_perm(n):
    bits = n.bit_length() - 1
    return np.array([int(format(i, f"0{bits}b")[::-1], 2) if bits else 0 for i in range(n)])


def _rows(line):
    return [np.array([float(t) for t in part.split()]) for part in line.split(";")]


def _golden(name):
    out = []
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                out.append(line)
    return out


# ---------------------------------------------------------------------------
# the transform
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n", [1, 2, 4, 8, 16, 32, 64])
def test_sylvester_integer_orthogonality(n):
    h = sylvester(n)
    assert np.array_equal(h @ h.T, n * np.eye(n, dtype=np.int64))


@pytest.mark.parametrize("n", [1, 2, 4, 8, 16, 32, 64])
def test_fwht_equals_sylvester_matrix(n):
    rng = np.random.default_rng(n)
    x = rng.standard_normal((5, n))
    y = O.fwht(x, n)
    ref = x @ sylvester(n).T.astype(np.float64) / np.sqrt(n)
    np.testing.assert_allclose(y, ref, rtol=0, atol=1e-13 * max(1.0, np.abs(ref).max()))


@pytest.mark.parametrize("n", [1, 2, 4, 8, 16, 32, 64])
def test_kronecker_power_entries(n):
    # the Kronecker recursion of the QWHA page (s2.1) has entries (-1)^popcount(i & j)
    i, j = np.meshgrid(np.arange(n), np.arange(n), indexing="ij")
    pc = np.vectorize(lambda v: bin(int(v)).count("1"))(i & j)
    assert np.array_equal(sylvester(n), np.where(pc % 2 == 0, 1, -1))


@pytest.mark.parametrize("n", [2, 4, 8, 16, 32, 64])
def test_recursive_page_transform_is_bit_reversed_sylvester(n):
    # cross-pin between two pages: the overview page's recursive even/odd transform gives the
    # Sylvester (natural-order) result in bit-reversed order, unnormalised.
    rng = np.random.default_rng(100 + n)
    x = rng.standard_normal(n)
    rec = bit_reversed_sylvester(n).astype(np.float64) @ x
    nat = O.fwht(x, n) * np.sqrt(n)
    np.testing.assert_allclose(rec, nat[bit_reverse_perm(n)], rtol=0, atol=1e-12)


def test_fwht_worked_values():
    for line in _golden("fwht_worked.txt"):
        b, xin, yout = [p.strip() for p in line.split("|")]
        x = np.array([float(t) for t in xin.split()])
        y = np.array([float(t) for t in yout.split()])
        np.testing.assert_allclose(O.fwht(x, int(b)), y, rtol=0, atol=1e-15)


@pytest.mark.parametrize("b", [16, 128, 256, 1024, 4096])
def test_fwht_round_trip_and_parseval(b):
    rng = np.random.default_rng(b)
    x = rng.standard_normal(3 * b)
    y = O.fwht(x, b)
    # natural-order Sylvester is symmetric and orthonormal: applying it twice is the identity
    np.testing.assert_allclose(O.fwht(y, b), x, rtol=0, atol=1e-13 * np.abs(x).max())
    assert abs(np.linalg.norm(y) - np.linalg.norm(x)) <= 1e-13 * np.linalg.norm(x)


@pytest.mark.parametrize("b", [2, 64, 512])
def test_fwht_special_vectors(b):
    e0 = np.zeros(b); e0[0] = 1.0
    np.testing.assert_allclose(O.fwht(e0, b), np.full(b, 1 / np.sqrt(b)), rtol=1e-15)
    ones = np.ones(b)
    expect = np.zeros(b); expect[0] = np.sqrt(b)
    np.testing.assert_allclose(O.fwht(ones, b), expect, rtol=0, atol=1e-12)


def test_fwht_blocks_are_independent():
    rng = np.random.default_rng(3)
    b, nb = 32, 5
    x = rng.standard_normal(b * nb)
    y = O.fwht(x, b)
    for j in range(nb):
        np.testing.assert_array_equal(y[j * b:(j + 1) * b], O.fwht(x[j * b:(j + 1) * b], b))
    # block-diagonal matrix I (x) H_b / sqrt(b)
    big = np.kron(np.eye(nb), sylvester(b).astype(np.float64)) / np.sqrt(b)
    np.testing.assert_allclose(y, big @ x, rtol=0, atol=1e-13)


def test_rotation_preserves_products():
    # "the transform matrix should be orthogonal" (QWHA page, s6): (XH)(WH)^T = X W^T
    rng = np.random.default_rng(4)
    m, n, k, b = 24, 20, 512, 128
    x = rng.standard_normal((m, k)).astype(np.float32)
    w = rng.standard_normal((n, k)).astype(np.float32)
    xr, _ = O.fwht_quant(x, O.ROWS, b, O.F64)
    wr, _ = O.fwht_quant(w, O.ROWS, b, O.F64)
    exact = x.astype(np.float64) @ w.astype(np.float64).T
    rot = O.matmul_f64(xr, wr)
    assert np.linalg.norm(rot - exact) <= 1e-12 * np.linalg.norm(exact)


def test_fwht_quant_f64_mode_is_the_transform_rows_and_cols():
    rng = np.random.default_rng(5)
    a = rng.standard_normal((64, 96)).astype(np.float32)
    r, s = O.fwht_quant(a, O.ROWS, 32, O.F64)
    np.testing.assert_allclose(r, O.fwht(a.astype(np.float64), 32), rtol=0, atol=1e-14)
    np.testing.assert_allclose(s, np.abs(r).max(axis=1), rtol=0)
    c, _ = O.fwht_quant(a, O.COLS, 16, O.F64)
    np.testing.assert_allclose(c, O.fwht(a.astype(np.float64).T, 16), rtol=0, atol=1e-14)


def test_bf16_inputs_are_read_exactly():
    rng = np.random.default_rng(6)
    a = rng.standard_normal((8, 64)).astype(np.float32)
    bits = synth.bf16_bits(a)
    vals = synth.bf16_to_f32(bits)
    r1, _ = O.fwht_quant(bits, O.ROWS, 64, O.F64)
    r2, _ = O.fwht_quant(vals, O.ROWS, 64, O.F64)
    np.testing.assert_array_equal(r1, r2)


def test_bf16_cast_is_nearest_even():
    # 1 + 2^-8 is a tie between bf16 1.0 and 1 + 2^-7: it rounds to the even 1.0;
    # 1 + 3*2^-8 is a tie between 1 + 2^-7 (odd) and 1 + 2^-6: it rounds to 1 + 2^-6.
    v = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -2.5, 3.0e38], dtype=np.float32)
    got = synth.bf16_to_f32(synth.bf16_bits(v))
    assert got[0] == 1.0 and got[1] == 1 + 2.0 ** -6 and got[2] == -2.5
    import torch
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(got, ref)


# ---------------------------------------------------------------------------
# the quantiser
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("precision", [64, 32])
def test_quantiser_hand_rows(precision):
    for line in _golden("quant_ties.txt"):
        xin, qout, sc = [p.strip() for p in line.split("|")]
        x = np.array([[float(t) for t in xin.split()]], dtype=np.float32)
        q, s = O.fwht_quant(x, O.ROWS, 1, O.I8, precision=precision)
        assert q[0].tolist() == [int(t) for t in qout.split()]
        assert s[0] == float(sc)


@pytest.mark.parametrize("qtype", [O.I8, O.E4M3, O.E5M2])
def test_quantiser_invariants(qtype):
    rng = np.random.default_rng(7)
    x = synth.activations(rng, 16, 256)
    q, s = O.fwht_quant(x, O.ROWS, 64, qtype)
    y, _ = O.fwht_quant(x, O.ROWS, 64, O.F64)
    qmax = O.QMAX[qtype]
    if qtype == O.I8:
        dq = q.astype(np.float64)
        assert np.abs(q).max() <= 127
        assert (q != -128).all()
        # the argmax of every row maps to +-qmax
        am = np.abs(y).argmax(axis=1)
        assert (np.abs(dq[np.arange(16), am]) == 127).all()
        # rounding error at most half a step
        assert (np.abs(dq * s[:, None] - y) <= s[:, None] / 2 * (1 + 1e-12)).all()
    else:
        tab = O.fp8_table(qtype)
        dq = tab[q]
        assert np.isfinite(dq).all() and np.abs(dq).max() <= qmax
        am = np.abs(y).argmax(axis=1)
        assert (np.abs(dq[np.arange(16), am]) == qmax).all()
        # relative error of a normal fp8 value is at most half an ulp: 2^-(mbits+1)
        mb = 3 if qtype == O.E4M3 else 2
        t = y / s[:, None]
        normal = np.abs(t) >= (2.0 ** -6 if qtype == O.E4M3 else 2.0 ** -14)
        err = np.abs(dq - t)[normal] / np.abs(t)[normal]
        assert err.max() <= 2.0 ** -(mb + 1) * (1 + 1e-12)
    np.testing.assert_allclose(s, np.abs(y).max(axis=1) / qmax, rtol=1e-15)
    # a power-of-two rescale of the input leaves the codes unchanged and rescales the scale
    q2, s2 = O.fwht_quant(x * np.float32(8.0), O.ROWS, 64, qtype)
    assert np.array_equal(q, q2)
    np.testing.assert_array_equal(s2, s * 8.0)


def test_zero_vector():
    x = np.zeros((3, 64), dtype=np.float32)
    x[1, 5] = 2.0
    for qt in (O.I8, O.E4M3, O.E5M2):
        q, s = O.fwht_quant(x, O.ROWS, 32, qt)
        assert s[0] == 0 and s[2] == 0 and s[1] > 0
        assert not q[0].any() and not q[2].any()


@pytest.mark.parametrize("precision", [32, 64])
def test_signed_zeros(precision):
    # reading: an exactly zero scaled value takes the +0 code (0x00); a nonzero value that
    # rounds to zero keeps its sign (OCP conversion: 0x80 for a tiny negative)
    x = np.zeros((1, 16), dtype=np.float32)
    x[0, :8] = -0.0                      # a block of -0: its sum butterfly stays -0
    x[0, 8:] = [448.0, -1e-9, 3.0, -0.0, 1.0, 2.0, 0.0, -5.0]
    for qt in (O.E4M3, O.E5M2):
        q1, _ = O.fwht_quant(x, O.ROWS, 1, qt, precision=precision)    # no rotation
        assert (q1[0, :8] == 0).all() and q1[0, 11] == 0 and q1[0, 14] == 0
        assert q1[0, 9] == 0x80            # -1e-9 * qmax / 448 underflows to -0
        q8, _ = O.fwht_quant(x, O.ROWS, 8, qt, precision=precision)
        assert (q8[0, :8] == 0).all()
    # fp32 output mode: zeros come out as +0 too
    y, _ = O.fwht_quant(x, O.ROWS, 8, O.F64, precision=precision)
    assert not np.signbit(y[0, :8]).any()


@pytest.mark.parametrize("block", [16, 128, 256, 1024, 4096])
def test_precision32_agrees_with_precision64(block):
    # the fp32 decision against the plain fp64 definition, at the code bar: |dq| <= 1 and at
    # most 1e-4 of the codes off by one; scales far inside 1e-5 relative
    rng = np.random.default_rng(8)
    x = synth.bf16_bits(synth.activations(rng, 128, 4096))
    for qt in (O.I8, O.E4M3, O.E5M2):
        q64, s64 = O.fwht_quant(x, O.ROWS, block, qt, precision=64)
        q32, s32 = O.fwht_quant(x, O.ROWS, block, qt, precision=32)
        np.testing.assert_allclose(s32, s64, rtol=1e-6)
        if qt == O.I8:
            d = np.abs(q64.astype(np.int32) - q32.astype(np.int32))
        else:
            d = np.abs(_fp8_ordinal(q64) - _fp8_ordinal(q32))
        assert d.max() <= 1 and (d == 1).mean() <= 1e-4


def _fp8_ordinal(c):
    c = c.astype(np.int32)
    return np.where(c & 0x80, -(c & 0x7F), c & 0x7F)


# ---------------------------------------------------------------------------
# FP8 codec
# ---------------------------------------------------------------------------

def test_fp8_spec_values():
    for line in _golden("fp8_spec.txt"):
        fmt, code, val = line.split()
        f = O.E4M3 if fmt == "e4m3" else O.E5M2
        v = O.fp8_decode(int(code, 16), f)
        assert v == float(val) and np.signbit(v) == val.startswith("-")
        assert O.fp8_encode(float(val), f) == int(code, 16)


@pytest.mark.parametrize("fmt", [O.E4M3, O.E5M2])
def test_fp8_exhaustive_round_trip(fmt):
    tab = O.fp8_table(fmt)
    for c in range(256):
        if np.isfinite(tab[c]):
            assert O.fp8_encode(tab[c], fmt) == c
    # exactly 254 (E4M3FN) or 248 (E5M2) finite codes, symmetric, strictly monotone magnitudes
    fin = np.isfinite(tab)
    assert fin.sum() == (254 if fmt == O.E4M3 else 248)
    pos = tab[:128][fin[:128]]
    assert (np.diff(pos) > 0).all()


@pytest.mark.parametrize("fmt", [O.E4M3, O.E5M2])
def test_fp8_ties_to_even_and_saturation(fmt):
    tab = O.fp8_table(fmt)
    pos = [(c, tab[c]) for c in range(128) if np.isfinite(tab[c])]
    for (c0, v0), (c1, v1) in zip(pos[:-1], pos[1:]):
        mid = (v0 + v1) / 2
        want = c0 if c0 % 2 == 0 else c1  # the even mantissa wins a tie
        assert O.fp8_encode(mid, fmt) == want
        assert O.fp8_encode(-mid, fmt) == want | 0x80
        assert O.fp8_encode(np.nextafter(mid, 0), fmt) == c0
        assert O.fp8_encode(np.nextafter(mid, np.inf), fmt) == c1
    mx = 448.0 if fmt == O.E4M3 else 57344.0
    top = 0x7E if fmt == O.E4M3 else 0x7B
    for v in (mx, mx * 1.01, 1e6, 1e30):
        assert O.fp8_encode(v, fmt) == top
        assert O.fp8_encode(-v, fmt) == top | 0x80


@pytest.mark.parametrize("fmt", [O.E4M3, O.E5M2])
def test_fp8_matches_torch_conversion(fmt):
    import torch
    tdt = torch.float8_e4m3fn if fmt == O.E4M3 else torch.float8_e5m2
    mx = 448.0 if fmt == O.E4M3 else 57344.0
    rng = np.random.default_rng(9)
    mag = np.exp2(rng.uniform(-20, np.log2(mx), 20000))
    v = (mag * rng.choice([-1.0, 1.0], 20000)).astype(np.float32)
    ref = torch.from_numpy(v).to(tdt).view(torch.uint8).numpy()
    got = np.array([O.fp8_encode(float(t), fmt) for t in v], dtype=np.uint8)
    assert np.array_equal(got, ref)
    dec = torch.arange(256, dtype=torch.uint8).view(tdt).to(torch.float64).numpy()
    tab = O.fp8_table(fmt)
    fin = np.isfinite(tab)
    np.testing.assert_array_equal(tab[fin], dec[fin])


# ---------------------------------------------------------------------------
# products
# ---------------------------------------------------------------------------

def test_gemm_i8_brute_force():
    rng = np.random.default_rng(10)
    for (m, n, k) in [(1, 1, 1), (3, 5, 7), (4, 6, 64)]:
        a = rng.integers(-127, 128, (m, k), dtype=np.int8)
        b = rng.integers(-127, 128, (n, k), dtype=np.int8)
        acc = O.gemm_i8(a, b)
        for i in range(m):
            for j in range(n):
                s = 0
                for t in range(k):
                    s += int(a[i, t]) * int(b[j, t])
                assert acc[i, j] == s


def test_gemm_i8_identity_and_bound():
    k = 64
    eye = np.eye(k, dtype=np.int8)
    rng = np.random.default_rng(11)
    a = rng.integers(-127, 128, (9, k), dtype=np.int8)
    assert np.array_equal(O.gemm_i8(a, eye), a.astype(np.int64))
    full = np.full((2, 4096), 127, dtype=np.int8)
    acc = O.gemm_i8(full, -full)
    assert (acc == -127 * 127 * 4096).all() and np.abs(acc).max() < 2 ** 31


def test_gemm_fp8_against_torch_decode():
    import torch
    rng = np.random.default_rng(12)
    tab4, tab5 = O.fp8_table(O.E4M3), O.fp8_table(O.E5M2)
    fin4 = np.nonzero(np.isfinite(tab4))[0].astype(np.uint8)
    fin5 = np.nonzero(np.isfinite(tab5))[0].astype(np.uint8)
    a = rng.choice(fin5, (7, 128))
    b = rng.choice(fin4, (5, 128))
    got = O.gemm_fp8(a, O.E5M2, b, O.E4M3)
    da = torch.from_numpy(a).view(torch.float8_e5m2).to(torch.float64).numpy()
    db = torch.from_numpy(b).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ref = da @ db.T
    np.testing.assert_allclose(got, ref, rtol=1e-15, atol=1e-300)


# ---------------------------------------------------------------------------
# the layer
# ---------------------------------------------------------------------------

def _golden_kv():
    kv = {}
    for line in _golden("layer_2x2.txt"):
        k, v = line.split("=", 1)
        kv[k.strip()] = np.array(_rows(v))
    return kv


@pytest.mark.parametrize("precision", [64, 32])
def test_layer_worked_example(precision):
    g = _golden_kv()
    f32 = np.float32
    x, w = g["fwd.x"].astype(f32), g["fwd.w"].astype(f32)
    qx, _ = O.fwht_quant(x, O.ROWS, 2, O.I8, precision)
    qw, _ = O.fwht_quant(w, O.ROWS, 2, O.I8, precision)
    assert np.array_equal(qx, g["fwd.qx"].astype(np.int8))
    assert np.array_equal(qw, g["fwd.qw"].astype(np.int8))
    assert np.array_equal(O.gemm_i8(qx, qw), g["fwd.acc"].astype(np.int64))
    tol = 1e-15 if precision == 64 else 3e-7
    np.testing.assert_allclose(O.linear_fwd(x, w, 2, O.I8, precision), g["fwd.y"], rtol=tol)
    dx, dw = O.linear_bwd(g["bwd.dy"].astype(f32), g["bwd.x"].astype(f32),
                          g["bwd.w"].astype(f32), 2, O.I8, O.I8, precision)
    np.testing.assert_allclose(dx, g["bwd.dx"], rtol=tol)
    np.testing.assert_allclose(dw, g["bwd.dw"], rtol=tol)


def _grid_matrix(rng, r, c):
    """Integers in [-127, 127] whose every row and every column holds a +-127."""
    a = rng.integers(-126, 127, (r, c)).astype(np.float32)
    for i in range(r):
        a[i, rng.integers(c)] = 127.0 * rng.choice([-1, 1])
    for j in range(c):
        a[rng.integers(r), j] = 127.0 * rng.choice([-1, 1])
    return a


def test_unrotated_exact_grid_layer_is_the_plain_product():
    # block 1 and inputs on the integer grid with absmax 127 in every row and column: each
    # scale is 1 and each code equals its input, so every pass reduces to the plain product
    rng = np.random.default_rng(13)
    m, n, k = 12, 10, 8
    x, w, dy = _grid_matrix(rng, m, k), _grid_matrix(rng, n, k), _grid_matrix(rng, m, n)
    y = O.linear_fwd(x, w, 1)
    dx, dw = O.linear_bwd(dy, x, w, 1)
    xd, wd, dyd = (t.astype(np.float64) for t in (x, w, dy))
    np.testing.assert_array_equal(y, xd @ wd.T)
    np.testing.assert_array_equal(dx, dyd @ wd)
    np.testing.assert_array_equal(dw, dyd.T @ xd)


def test_rotation_reduces_outlier_error():
    # rotations spread the outlier channels (HALO paper, abstract), so the rotated INT8
    # product is far closer to the exact one than the unrotated (block 1) product
    x, w, dy = synth.layer(128, 256, 1024, seed=14, io=synth.F32)
    exact = x.astype(np.float64) @ w.astype(np.float64).T
    e_rot = np.linalg.norm(O.linear_fwd(x, w, 256) - exact) / np.linalg.norm(exact)
    e_raw = np.linalg.norm(O.linear_fwd(x, w, 1) - exact) / np.linalg.norm(exact)
    assert e_rot < 0.03 and e_raw > 2.5 * e_rot
    dx_ex = dy.astype(np.float64) @ w.astype(np.float64)
    dw_ex = dy.astype(np.float64).T @ x.astype(np.float64)
    dx, dw = O.linear_bwd(dy, x, w, 128)
    assert np.linalg.norm(dx - dx_ex) / np.linalg.norm(dx_ex) < 0.05
    assert np.linalg.norm(dw - dw_ex) / np.linalg.norm(dw_ex) < 0.05


def test_fp8_layer_close_to_exact():
    x, w, dy = synth.layer(64, 128, 512, seed=15, io=synth.BF16)
    xf, wf, dyf = (synth.bf16_to_f32(t).astype(np.float64) for t in (x, w, dy))
    y = O.linear_fwd(x, w, 128, O.E4M3)
    assert np.linalg.norm(y - xf @ wf.T) / np.linalg.norm(xf @ wf.T) < 0.08
    dx, dw = O.linear_bwd(dy, x, w, 64, O.E4M3, O.E5M2)
    assert np.linalg.norm(dx - dyf @ wf) / np.linalg.norm(dyf @ wf) < 0.15
    assert np.linalg.norm(dw - dyf.T @ xf) / np.linalg.norm(dyf.T @ xf) < 0.15


def test_sampled_vectors_match_full():
    rng = np.random.default_rng(16)
    a = synth.bf16_bits(rng.standard_normal((48, 256)).astype(np.float32))
    qa, sa = O.fwht_quant(a, O.COLS, 16, O.I8)
    idx = np.array([0, 7, 255, 3])
    qs, ss = O.fwht_quant(a, O.COLS, 16, O.I8, vec_idx=idx)
    assert np.array_equal(qs, qa[idx]) and np.array_equal(ss, sa[idx])


def test_oracle_rejects_bad_arguments():
    x = np.zeros((4, 48), dtype=np.float32)
    with pytest.raises(ValueError):
        O.fwht_quant(x, O.ROWS, 3, O.I8)  # not a power of two
    with pytest.raises(ValueError):
        O.fwht_quant(x, O.ROWS, 16, O.F64, rounding=O.STOCHASTIC)  # rounding of values
    with pytest.raises(ValueError):
        O.fwht_quant(x, O.ROWS, 16, O.I8, rounding=2)
