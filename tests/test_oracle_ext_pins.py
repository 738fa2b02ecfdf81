"""Pins of the oracle's randomised transform H D, its zero padding and its stochastic rounding.

Each test checks the oracle against something other than itself: the explicit Sylvester
matrix with an explicit sign diagonal, the page's own padding to a power of two, the
invariance of the products under an orthogonal transform, the generator's published
known-answer vectors (tests/golden/philox_kat.txt), and the properties stochastic rounding is
defined by (only the two neighbouring grid points, unbiased, independent draws, exact values
kept).  Pages: "QWHA方法：基于Walsh-Hadamard变换的高效大模型微调技术" s2.1 (Sylvester definition),
s5 (padding to a power of two, stochastic rounding); "企业官网建设流程全解析" s4.2 (one random
seed for the Hadamard matrix on every node).
"""
import os

import numpy as np
import pytest

import oracle as O
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
QTYPES = [O.I8, O.E4M3, O.E5M2]


def sylvester(n):
    """Unnormalised Hadamard matrix by the Kronecker recursion H_2n = [[H, H], [H, -H]]."""
    h = np.ones((1, 1), dtype=np.int64)
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def sign_vector(words, n):
    """+1 / -1 per element from packed sign words (bit i of the little-endian bit stream)."""
    bits = np.unpackbits(np.ascontiguousarray(words, dtype=np.uint32).view(np.uint8),
                         bitorder="little")[:n]
    return 1.0 - 2.0 * bits.astype(np.float64)


def grid(qtype):
    """Sorted non-negative values of the target grid (INT8 integers or the finite FP8 values)."""
    if qtype == O.I8:
        return np.arange(0, 128, dtype=np.float64)
    t = O.fp8_table(qtype)
    t = t[np.isfinite(t) & (t >= 0)]
    return np.unique(t[t <= O.QMAX[qtype]])


def decode(codes, qtype):
    if qtype == O.I8:
        return codes.astype(np.float64)
    return O.fp8_table(qtype)[codes]


# ---------------------------------------------------------------------------
# Philox4x32-10
# ---------------------------------------------------------------------------

def test_philox_known_answers():
    n = 0
    with open(os.path.join(GOLDEN, "philox_kat.txt"), encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            ctr, key, out = ([int(t, 16) for t in part.split()] for part in line.split("|"))
            assert list(O.philox4x32_10(ctr, key)) == out
            n += 1
    assert n == 3


# ---------------------------------------------------------------------------
# randomised transform H D
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n", [1, 2, 4, 8, 16, 32, 64])
def test_signed_transform_equals_explicit_matrix(n):
    rng = np.random.default_rng(100 + n)
    x = rng.standard_normal((3, n)).astype(np.float32)
    words = synth.sign_words(n, seed=n)
    d = sign_vector(words, n)
    want = (sylvester(n) @ (d[:, None] * x.T.astype(np.float64))).T / np.sqrt(n)
    got, _ = O.fwht_quant(x, O.ROWS, n, O.F64, signs=words)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)
    # the columns axis applies the same signs along the rows
    got_c, _ = O.fwht_quant(np.ascontiguousarray(x.T), O.COLS, n, O.F64, signs=words)
    np.testing.assert_allclose(got_c, want, rtol=1e-12, atol=1e-12)


def test_sign_bit_order():
    # bit i of the stream (word i / 32, bit i % 32) negates element i and nothing else
    rng = np.random.default_rng(7)
    x = rng.standard_normal((2, 96)).astype(np.float32)
    plain, _ = O.fwht_quant(x, O.ROWS, 32, O.F64)
    for i in (0, 5, 31, 32, 63, 70, 95):
        words = np.zeros(3, dtype=np.uint32)
        words[i // 32] = np.uint32(1) << np.uint32(i % 32)
        xn = x.copy()
        xn[:, i] = -xn[:, i]
        want, _ = O.fwht_quant(xn, O.ROWS, 32, O.F64)
        got, _ = O.fwht_quant(x, O.ROWS, 32, O.F64, signs=words)
        assert np.array_equal(got, want)
        assert not np.array_equal(got, plain)


def test_signed_transform_preserves_products():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((8, 256)).astype(np.float32)
    w = rng.standard_normal((6, 256)).astype(np.float32)
    words = synth.sign_words(256, seed=3)
    yx, _ = O.fwht_quant(x, O.ROWS, 64, O.F64, signs=words)
    yw, _ = O.fwht_quant(w, O.ROWS, 64, O.F64, signs=words)
    exact = x.astype(np.float64) @ w.astype(np.float64).T
    assert np.abs(yx @ yw.T - exact).max() <= 1e-12 * np.abs(exact).max()


@pytest.mark.parametrize("precision", [32, 64])
@pytest.mark.parametrize("qtype", QTYPES)
def test_all_signs_negate_the_codes(qtype, precision):
    rng = np.random.default_rng(9)
    x = synth.bf16_bits(rng.standard_normal((16, 128)).astype(np.float32))
    q0, s0 = O.fwht_quant(x, O.ROWS, 128, qtype, precision=precision)
    q1, s1 = O.fwht_quant(x, O.ROWS, 128, qtype, precision=precision,
                          signs=np.full(4, 0xFFFFFFFF, dtype=np.uint32))
    assert np.array_equal(s0, s1)
    if qtype == O.I8:
        assert np.array_equal(q1, -q0)
    else:
        want = np.where(q0 == 0, q0, q0 ^ np.uint8(0x80))
        assert np.array_equal(q1, want)


# ---------------------------------------------------------------------------
# zero padding
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("qtype", [O.I8, O.E5M2, O.F64])
@pytest.mark.parametrize("axis,L,block", [(O.ROWS, 100, 32), (O.ROWS, 200, 256),
                                          (O.COLS, 72, 64), (O.COLS, 1000, 128)])
def test_padding_equals_explicit_zero_padding(axis, L, block, qtype):
    rng = np.random.default_rng(L + block)
    nvec = 5
    shape = (nvec, L) if axis == O.ROWS else (L, nvec)
    x = synth.bf16_bits(rng.standard_normal(shape).astype(np.float32))
    Lp = O.padded_len(L, block)
    pad = np.zeros((nvec, Lp) if axis == O.ROWS else (Lp, nvec), dtype=np.uint16)
    pad[:shape[0], :shape[1]] = x
    for precision in (32, 64):
        got, gs = O.fwht_quant(x, axis, block, qtype, precision=precision)
        want, ws = O.fwht_quant(pad, axis, block, qtype, precision=precision)
        assert got.shape == (nvec, Lp)
        assert np.array_equal(got, want) and np.array_equal(gs, ws)


def test_single_block_padding_is_the_pages_power_of_two_padding():
    # one block of the next power of two: the page pads the vector with zeros to 2^ceil(log2 L)
    # and applies the whole transform
    rng = np.random.default_rng(11)
    x = rng.standard_normal((4, 100)).astype(np.float32)
    padded = np.concatenate([x, np.zeros((4, 28), dtype=np.float32)], axis=1).astype(np.float64)
    want = (sylvester(128) @ padded.T).T / np.sqrt(128)
    got, _ = O.fwht_quant(x, O.ROWS, 128, O.F64)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_padded_rotation_preserves_products():
    rng = np.random.default_rng(12)
    x = rng.standard_normal((5, 100)).astype(np.float32)
    w = rng.standard_normal((7, 100)).astype(np.float32)
    yx, _ = O.fwht_quant(x, O.ROWS, 32, O.F64, signs=synth.sign_words(128, seed=1))
    yw, _ = O.fwht_quant(w, O.ROWS, 32, O.F64, signs=synth.sign_words(128, seed=1))
    assert yx.shape == (5, 128)
    exact = x.astype(np.float64) @ w.astype(np.float64).T
    assert np.abs(yx @ yw.T - exact).max() <= 1e-12 * np.abs(exact).max()


def test_padded_layer_equals_layer_on_padded_operands():
    cfg = synth.layer(24, 40, 200, seed=5)
    x, w, dy = cfg
    k = 200
    kp = O.padded_len(k, 64)
    xp = np.zeros((24, kp), dtype=np.uint16)
    wp = np.zeros((40, kp), dtype=np.uint16)
    xp[:, :k], wp[:, :k] = x, w
    for precision in (32, 64):
        assert np.array_equal(O.linear_fwd(x, w, 64, precision=precision),
                              O.linear_fwd(xp, wp, 64, precision=precision))
    # backward: pad M (dY and X rows) and N (dY columns, W rows)
    m, n = 24, 40
    dx, dw = O.linear_bwd(dy, x, w, 16)
    mp, npad = O.padded_len(m, 16), O.padded_len(n, 16)
    assert (mp, npad) == (32, 48)
    dyp = np.zeros((mp, npad), dtype=np.uint16)
    dyp[:m, :n] = dy
    xq = np.zeros((mp, k), dtype=np.uint16)
    xq[:m] = x
    wq = np.zeros((npad, k), dtype=np.uint16)
    wq[:n] = w
    dxp, dwp = O.linear_bwd(dyp, xq, wq, 16)
    assert np.array_equal(dx, dxp[:m]) and np.array_equal(dw, dwp[:n])


# ---------------------------------------------------------------------------
# stochastic rounding
# ---------------------------------------------------------------------------

def _scaled(x, axis, block, qtype, signs=None):
    """t = y * qmax / absmax of every rotated element (fp64)."""
    y, a = O.fwht_quant(x, axis, block, O.F64, signs=signs)
    return y * (O.QMAX[qtype] / np.where(a > 0, a, 1.0))[:, None]


@pytest.mark.parametrize("qtype", QTYPES)
def test_sr_exact_grid_values_are_kept(qtype):
    # block 1 is the identity; vectors whose absmax is qmax hold grid values exactly
    rng = np.random.default_rng(20)
    g = grid(qtype)
    vals = rng.choice(g, size=(6, 64)) * rng.choice([-1.0, 1.0], size=(6, 64))
    vals[:, 3] = g[-1]
    x = vals.astype(np.float32)
    want, _ = O.fwht_quant(x, O.ROWS, 1, qtype)
    for key in [(0, 0), (1, 2), (0xDEADBEEF, 77)]:
        got, _ = O.fwht_quant(x, O.ROWS, 1, qtype, rounding=O.STOCHASTIC, key=key)
        assert np.array_equal(got, want)


@pytest.mark.parametrize("precision", [32, 64])
@pytest.mark.parametrize("qtype", QTYPES)
def test_sr_rounds_to_a_neighbouring_grid_point(qtype, precision):
    rng = np.random.default_rng(21)
    x = synth.bf16_bits(rng.standard_normal((32, 256)).astype(np.float32))
    t = _scaled(x, O.ROWS, 64, qtype)
    q, _ = O.fwht_quant(x, O.ROWS, 64, qtype, precision=precision, rounding=O.STOCHASTIC,
                        key=(5, 6), ctr_hi=(7, 8))
    v = decode(q, qtype)
    g = np.concatenate([-grid(qtype)[::-1], grid(qtype)])
    lo = g[np.searchsorted(g, t, side="right") - 1]
    hi = g[np.minimum(np.searchsorted(g, t, side="left"), g.size - 1)]
    tol = 1e-6 * np.abs(t) if precision == 32 else 0.0  # fp32 t may sit a hair off t64
    ok = (v == lo) | (v == hi) | (np.abs(v - t) <= tol)
    assert ok.all(), f"{int((~ok).sum())} codes off the neighbouring grid points"
    assert (v == hi).any() and (v == lo).any() and (lo != hi).any()


@pytest.mark.parametrize("qtype", QTYPES)
def test_sr_is_unbiased(qtype):
    # 4000 copies of one vector draw independently (the vector index is in the counter):
    # the mean of the dequantised codes converges to the rotated value itself
    rng = np.random.default_rng(22)
    v = (rng.standard_normal(128) * np.where(rng.random(128) < 0.05, 30.0, 1.0)).astype(np.float32)
    n = 4000
    x = np.tile(v, (n, 1))
    y, a = O.fwht_quant(x[:1], O.ROWS, 128, O.F64)
    q, s = O.fwht_quant(x, O.ROWS, 128, qtype, rounding=O.STOCHASTIC, key=(123, 456))
    assert np.allclose(s, s[0])
    deq = decode(q, qtype) * s[0]
    mean = deq.mean(axis=0)
    # per-element spread: half the local grid step
    t = y[0] * O.QMAX[qtype] / a[0]
    g = np.concatenate([-grid(qtype)[::-1], grid(qtype)])
    lo = g[np.searchsorted(g, t, side="right") - 1]
    hi = g[np.minimum(np.searchsorted(g, t, side="left"), g.size - 1)]
    # (an element on a grid point has no spread: only summation rounding in the mean)
    sigma = np.maximum((hi - lo) * s[0] / 2, 1e-9 * np.abs(y[0]) + 1e-30)
    z = np.abs(mean - y[0]) / (sigma / np.sqrt(n))
    assert z.max() < 5.5, f"max z-score {z.max():.2f}"
    # nearest-even rounding of the same vector is biased far beyond that on some elements
    qr, _ = O.fwht_quant(x[:1], O.ROWS, 128, qtype)
    zr = np.abs(decode(qr[0], qtype) * s[0] - y[0]) / (sigma / np.sqrt(n))
    assert zr.max() > 20


def test_sr_draws_are_independent():
    # t = 0.5 exactly on every element but the first: each draw is a fair coin, and the coins
    # of neighbouring positions (same and different Philox calls) and of neighbouring
    # vectors are uncorrelated
    nvec, L = 512, 256
    x = np.full((nvec, L), 0.5, dtype=np.float32)
    x[:, 0] = 127.0  # absmax 127: the multiplier is exactly 1 (block 1 = identity)
    q, _ = O.fwht_quant(x, O.ROWS, 1, O.I8, rounding=O.STOCHASTIC, key=(9, 9), ctr_hi=(1, 0))
    up = q[:, 1:].astype(np.float64)  # 1 = rounded up, 0 = down
    assert set(np.unique(up)) == {0.0, 1.0}
    assert abs(up.mean() - 0.5) < 5 * 0.5 / np.sqrt(up.size)
    c = up - up.mean()
    lim = 5 / np.sqrt(c.size)
    for dp in (1, 2, 3, 4, 5, 8):
        r = (c[:, :-dp] * c[:, dp:]).mean() / c.var()
        assert abs(r) < lim, f"lag {dp}: correlation {r:.4f}"
    r = (c[:-1] * c[1:]).mean() / c.var()
    assert abs(r) < lim, f"vector lag 1: correlation {r:.4f}"


def test_sr_counter_layout():
    # the uniform of element p of vector v is the top 24 bits of word p % 4 of
    # Philox4x32-10(counter (p / 4, v, c2, c3), key): checked with t known exactly (block 1,
    # absmax 127, so t = x)
    rng = np.random.default_rng(23)
    x = (np.round(rng.uniform(-126, 126, size=(3, 40)) * 64) / 64).astype(np.float32)
    x[:, 0] = 127.0
    key, chi = (0x1234, 0x5678), (0x9ABC, 0xDEF0)
    q, _ = O.fwht_quant(x, O.ROWS, 1, O.I8, rounding=O.STOCHASTIC, key=key, ctr_hi=chi)
    for v in range(3):
        for p in range(40):
            w = int(O.philox4x32_10([p // 4, v, chi[0], chi[1]], key)[p % 4]) >> 8
            t = float(x[v, p])
            fl = np.floor(t)
            want = fl + (1.0 if w < (t - fl) * 2.0 ** 24 else 0.0)
            assert q[v, p] == want, (v, p)


def test_sr_is_deterministic_and_keyed():
    rng = np.random.default_rng(24)
    x = synth.bf16_bits(rng.standard_normal((16, 512)).astype(np.float32))
    a, _ = O.fwht_quant(x, O.COLS, 16, O.E5M2, rounding=O.STOCHASTIC, key=(1, 2), ctr_hi=(3, 4))
    b, _ = O.fwht_quant(x, O.COLS, 16, O.E5M2, rounding=O.STOCHASTIC, key=(1, 2), ctr_hi=(3, 4))
    c, _ = O.fwht_quant(x, O.COLS, 16, O.E5M2, rounding=O.STOCHASTIC, key=(1, 3), ctr_hi=(3, 4))
    d, _ = O.fwht_quant(x, O.COLS, 16, O.E5M2, rounding=O.STOCHASTIC, key=(1, 2), ctr_hi=(3, 5))
    assert np.array_equal(a, b)
    assert (a != c).mean() > 0.1 and (a != d).mean() > 0.1


@pytest.mark.parametrize("qtype", QTYPES)
def test_sr_precision32_agrees_with_precision64(qtype):
    rng = np.random.default_rng(25)
    x = synth.bf16_bits(rng.standard_normal((64, 1024)).astype(np.float32))
    k = dict(rounding=O.STOCHASTIC, key=(77, 88), ctr_hi=(0, 1))
    q32, s32 = O.fwht_quant(x, O.ROWS, 256, qtype, precision=32, **k)
    q64, s64 = O.fwht_quant(x, O.ROWS, 256, qtype, precision=64, **k)
    np.testing.assert_allclose(s32, s64, rtol=1e-6)
    diff = (q32 != q64).sum()
    assert diff <= max(2, 1e-4 * q32.size), f"{diff} codes differ"


def test_layer_with_options_stays_close_to_the_exact_product():
    x, w, dy = synth.layer(64, 96, 200, seed=6)
    xf, wf, dyf = (synth.bf16_to_f32(a).astype(np.float64) for a in (x, w, dy))
    sk = synth.sign_words(O.padded_len(200, 64), seed=1)
    sn = synth.sign_words(O.padded_len(96, 64), seed=2)
    sm = synth.sign_words(O.padded_len(64, 64), seed=3)
    y = O.linear_fwd(x, w, 64, signs_k=sk)
    exact = xf @ wf.T
    assert np.linalg.norm(y - exact) <= 0.05 * np.linalg.norm(exact)
    dx, dw = O.linear_bwd(dy, x, w, 64, signs_n=sn, signs_m=sm, grad_rounding=O.STOCHASTIC,
                          key=(4, 5), ctr_hi=(6, 7))
    for got, ref in ((dx, dyf @ wf), (dw, dyf.T @ xf)):
        assert np.linalg.norm(got - ref) <= 0.05 * np.linalg.norm(ref)


def test_layer_sr_uses_distinct_draws_for_rows_and_columns_of_dy():
    # the columns pass of dY draws with counter word 3 ^ 2^31: its codes are those of a
    # standalone columns pass with that counter
    x, w, dy = synth.layer(64, 64, 64, seed=7)
    key, chi = (11, 12), (13, 14)
    _, dw = O.linear_bwd(dy, x, w, 64, grad_rounding=O.STOCHASTIC, key=key, ctr_hi=chi,
                         want_dx=False)
    qa, sa = O.fwht_quant(dy, O.COLS, 64, O.I8, rounding=O.STOCHASTIC, key=key,
                          ctr_hi=(chi[0], chi[1] ^ 0x80000000))
    qb, sb = O.fwht_quant(x, O.COLS, 64, O.I8)
    assert np.array_equal(dw, O.dequant(O.gemm_i8(qa, qb).astype(np.float64), sa, sb))
    qr, _ = O.fwht_quant(dy, O.COLS, 64, O.I8, rounding=O.STOCHASTIC, key=key, ctr_hi=chi)
    assert not np.array_equal(qr, qa)


# ---------------------------------------------------------------------------
# vectors of tiny values (absmax scale invariance)
# ---------------------------------------------------------------------------

def _tiny_and_scaled(seed, rows=3, cols=512):
    """fp32 inputs v_big = integer * 2^-85 (normal, about 2^-70) and v_tiny = v_big * 2^-64
    (integer multiples of 2^-149: subnormal, exact).  A rotated tiny vector's absmax is about
    2^-124, so fp32 qmax / absmax overflows for every code type."""
    rng = np.random.default_rng(seed)
    ints = np.rint(rng.standard_normal((rows, cols)) * 2.0 ** 15)
    big = (ints * 2.0 ** -85).astype(np.float32)
    tiny = (ints * 2.0 ** -149).astype(np.float32)
    assert np.array_equal(tiny.astype(np.float64) * 2.0 ** 64, big.astype(np.float64))
    assert np.abs(tiny).max() < np.finfo(np.float32).tiny
    return tiny, big


@pytest.mark.parametrize("qtype", [O.I8, O.E4M3, O.E5M2])
@pytest.mark.parametrize("axis", [O.ROWS, O.COLS])
def test_tiny_vector_codes_equal_those_of_the_scaled_vector(qtype, axis):
    # Absmax quantisation is invariant under scaling a vector: its codes are those of the same
    # vector times 2^64.  That holds in exact arithmetic (the fp64 path) and must hold in the
    # fp32 decision too, even where fp32 qmax / absmax overflows for the tiny vector.
    tiny, big = _tiny_and_scaled(11)
    if axis == O.COLS:
        tiny, big = np.ascontiguousarray(tiny.T), np.ascontiguousarray(big.T)
    qmax = {O.I8: 127.0, O.E4M3: 448.0, O.E5M2: 57344.0}[qtype]
    for precision in (64, 32):
        qt, st = O.fwht_quant(tiny, axis, 256, qtype, precision=precision)
        qb, sb = O.fwht_quant(big, axis, 256, qtype, precision=precision)
        assert np.array_equal(qt, qb), f"precision {precision}"
        assert (np.abs(qb.astype(np.int64)) > 0).any()  # not the zero vector's codes
        # scales: absmax / qmax, scaled back by 2^-64 (the tiny scales are subnormal in fp32)
        np.testing.assert_allclose(st, sb * 2.0 ** -64, rtol=1e-6, atol=2.0 ** -149)
    # the tiny vector really is in the range where fp32 qmax / absmax overflows
    y = O.fwht_quant(tiny, axis, 256, O.F64, precision=32)[1] * 16.0  # absmax of unnormalised y
    with np.errstate(over="ignore"):
        assert (np.float32(qmax) / y.astype(np.float32) == np.inf).all()


@pytest.mark.parametrize("qtype", [O.I8, O.E4M3, O.E5M2])
def test_tiny_vector_stochastic_codes_equal_those_of_the_scaled_vector(qtype):
    # with stochastic rounding the same uniforms meet the same scaled values
    tiny, big = _tiny_and_scaled(12)
    kw = dict(rounding=O.STOCHASTIC, key=(7, 8), ctr_hi=(1, 2))
    for precision in (64, 32):
        qt, _ = O.fwht_quant(tiny, O.ROWS, 256, qtype, precision=precision, **kw)
        qb, _ = O.fwht_quant(big, O.ROWS, 256, qtype, precision=precision, **kw)
        assert np.array_equal(qt, qb), f"precision {precision}"
