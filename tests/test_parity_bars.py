"""CPU checks of the parity bars themselves (tests/parity_util.py), with the oracle standing in
for the GPU: a bar must accept what a correct fp32 computation gives and reject planted errors.

The fp32-input FP8 code bar: with fp32 input the butterflies round (bf16 sums do not), and near
zero the E5M2 grid (2^-16 code units apart) is much finer than that rounding, so the oracle's
own fp32-decision codes may sit several grid steps from its fp64 decision there.  The bar
holds every code to the exact value within half a grid step plus an a-priori bound on the fp32
rotation's error; it must accept those codes and still reject a code moved by a few steps.
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
