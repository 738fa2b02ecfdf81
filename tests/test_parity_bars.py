"""CPU checks of the parity bars themselves (tests/parity_util.py), with the oracle standing in
for the GPU: a bar must accept what a correct fp32 computation gives and reject planted errors.

The FP8 code bar: where the fp32 butterflies round (fp32 input; bf16 input too once a block's
sums need more than 24 bits), near zero the E5M2 grid (2^-16 code units apart) is much finer
than that rounding, so the oracle's own fp32-decision codes may sit several grid steps from its
fp64 decision there.  The bar holds every code to the exact value within half a grid step plus
an a-priori bound on the fp32 rotation's error; it must accept those codes and still reject a
code moved by a few steps.
"""
import numpy as np
import pytest

import oracle as O
import synth
import parity_util as P


def _case(rows, cols, block, qt, signs, seed):
    rng = np.random.default_rng(seed)
    x = synth.activations(rng, rows, cols)                      # fp32
    words = synth.sign_words(O.padded_len(rows, block), seed=rows + block) if signs else None
    opts = dict(signs=words, rounding=O.RNE)
    q32, _ = O.fwht_quant(x, O.COLS, block, qt, precision=32, **opts)
    q64, _ = O.fwht_quant(x, O.COLS, block, qt, precision=64, **opts)
    return x, opts, q32, q64


def test_fp32_input_e5m2_bar_accepts_the_fp32_path():
    # 5000 x 72 fp32, block 128, signs: one code of the fp32 path is 5 E5M2 steps from fp64
    x, opts, q32, q64 = _case(5000, 72, 128, O.E5M2, True, 5000 + 3 * 72 + 128)
    d = P.code_distance(q32, q64, O.E5M2)
    assert d.max() > 1                  # the case the bar exists for
    P.assert_codes_close_to_fp64(q32, q64, O.E5M2, 128, x=x, oaxis=O.COLS, opts=opts)
    with pytest.raises(AssertionError):  # the one-step ordinal bar rejects it
        P.assert_codes_close_to_fp64(q32, q64, O.E5M2, 128)


@pytest.mark.parametrize("qt,steps", [(O.E5M2, 3), (O.E4M3, 2)])
def test_fp32_input_fp8_bar_rejects_moved_codes(qt, steps):
    x, opts, q32, q64 = _case(2048, 40, 256, qt, False, 17)
    P.assert_codes_close_to_fp64(q32, q64, qt, 256, x=x, oaxis=O.COLS, opts=opts)
    vals = np.abs(O.fp8_table(qt)[q32])
    for target in (vals.argmax(), np.argsort(vals.ravel())[vals.size // 2]):  # largest, median
        bad = q32.copy().ravel()
        c = int(bad[target])
        bad[target] = (c - steps) if (c & 0x7F) >= steps else (c + steps)  # same sign, |.| moved
        with pytest.raises(AssertionError):
            P.assert_codes_close_to_fp64(bad.reshape(q32.shape), q64, qt, 256, x=x,
                                         oaxis=O.COLS, opts=opts)


def test_ties_repeated_by_padding_do_not_count():
    # 16 bf16 rows padded to one block of 4096: each rotated column holds 16 distinct values,
    # each 256 times.  Three of them are exact ties (t = k + 1/2) that the fp32 decision
    # (m = fl32(127 / a)) rounds away from even: 768 codes differ from fp64, 0.15 %, all
    # undecidable in fp32.  The bar accepts them; a moved code elsewhere still fails.
    rng = np.random.default_rng(5617)
    x = synth.bf16_bits(synth.activations(rng, 16, 128))
    q32, _ = O.fwht_quant(x, O.COLS, 4096, O.I8, precision=32)
    q64, _ = O.fwht_quant(x, O.COLS, 4096, O.I8, precision=64)
    d = P.code_distance(q32, q64, O.I8)
    t, e = P.fp32_rotation_code_bound(x, O.COLS, 4096, O.I8)
    und = P.undecidable_in_fp32(t, e, O.I8)
    assert (d == 1).sum() > 1e-4 * d.size and (d[~und] == 0).all()
    assert np.all(np.abs(t[d == 1] - np.floor(t[d == 1]) - 0.5) == 0.0)  # exact ties
    P.assert_codes_close_to_fp64(q32, q64, O.I8, 4096, x=x, oaxis=O.COLS)
    with pytest.raises(AssertionError):  # the plain fraction rejects them
        P.assert_codes_close_to_fp64(q32, q64, O.I8, 4096)
    bad = q32.copy()
    far = np.argwhere(~und & (np.abs(t) < 120))
    for i, j in far[:60]:            # 60 decidable codes moved by one: over the 52 allowed
        bad[i, j] += 1
    with pytest.raises(AssertionError):
        P.assert_codes_close_to_fp64(bad, q64, O.I8, 4096, x=x, oaxis=O.COLS)


def test_bf16_input_fp8_code_near_zero():
    # random rotation case 1902: 41 bf16 rows of 4160 with outlier channels, block 4096 (rows
    # padded to 8192), E5M2 codes, signs.  The block's sums need more than fp32's 24 bits, so
    # the fp32 butterflies round; one code's exact value is -0.0017 code units against an fp32
    # bound of 0.42, and the fp32 decision (the GPU's, bit for bit) lands 23 E5M2 steps from
    # the fp64 one.  The value bar accepts it; a code moved beyond the bound still fails.
    c = P.random_rotation_case(1902)
    x, b, qt, words = c["x"], c["block"], c["qt"], c["words"]
    assert c["axis"] == 0 and x.dtype == np.uint16 and qt == O.E5M2 and not c["sr"]
    opts = dict(signs=words, rounding=O.RNE)
    q32, _ = O.fwht_quant(x, O.ROWS, b, qt, precision=32, **opts)
    q64, _ = O.fwht_quant(x, O.ROWS, b, qt, precision=64, **opts)
    d = P.code_distance(q32, q64, qt)
    assert d.max() > 1                  # the case the bar exists for
    P.assert_codes_close_to_fp64(q32, q64, qt, b, x=x, oaxis=O.ROWS, opts=opts)
    i = np.unravel_index(np.argmax(d), d.shape)
    t, e = P.fp32_rotation_code_bound(x, O.ROWS, b, qt, opts)
    assert abs(t[i]) < e[i]             # undecidable in fp32: the bound exceeds the value
    table = O.fp8_table(qt)
    far = t[i] + 4 * e[i] + 1.0         # a value well beyond the bound
    bad = q32.copy()
    bad[i] = int(np.nanargmin(np.abs(table - far)))
    with pytest.raises(AssertionError):
        P.assert_codes_close_to_fp64(bad, q64, qt, b, x=x, oaxis=O.ROWS, opts=opts)
