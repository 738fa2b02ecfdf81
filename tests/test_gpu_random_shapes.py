"""GPU parity on seeded random shapes: random valid sizes, blocks, code types, input types,
sign arrays and rounding modes through halo_fwht_quant (both axes, including columns long
enough to exchange partial maxima) and through the layer calls, each against the oracle with
the bars of the fixed-shape tests (codes and scales bit-exact to the fp32 decision and within
the code bar of the fp64 definition; layer
outputs within 1e-2 relative Frobenius of the fp64 path and within one output rounding, plus
the FP8 accumulation bound, of the fp32-decision path).  Case i draws everything from its own
generator, so a failing case is reproduced by its index alone.
"""
import numpy as np
import pytest
import torch

import hadamard_rotated_precision_halo_amd as H
import oracle as O
import synth
from parity_util import COUNTER64, CTR, KEY, Q_TORCH, SEED64, bound_ok, check_fq_parity, \
    codes_to_np, fp8_extra, random_rotation_case, rel_fro, signs_dev, to_dev, to_np64

pytestmark = pytest.mark.gpu

def _block(rng):
    return 1 << int(rng.integers(0, 13))


@pytest.mark.parametrize("case", range(24))
def test_random_rotation_pass(case):
    c = random_rotation_case(case)
    axis, b, qt, x, words, sr = c["axis"], c["block"], c["qt"], c["x"], c["words"], c["sr"]
    print(f"case {case}: axis {axis} io {c['io']} {c['rows']}x{c['cols']} block {b} code {qt} "
          f"signs {words is not None} sr {sr}", flush=True)
    q, s = H.fwht_quant(to_dev(x), axis=H.ROWS if axis == 0 else H.COLS, block=b,
                        q_dtype=Q_TORCH[qt], signs=signs_dev(words) if words is not None else None,
                        rounding="stochastic" if sr else "nearest", seed=SEED64,
                        counter=COUNTER64)
    torch.cuda.synchronize()
    check_fq_parity(codes_to_np(q), s.cpu().numpy(), x, O.ROWS if axis == 0 else O.COLS, b, qt,
                    signs=words, rounding=O.STOCHASTIC if sr else O.RNE, key=KEY, ctr_hi=CTR)


@pytest.mark.parametrize("case", range(24))
def test_random_layer(case):
    rng = np.random.default_rng(6000 + case)
    io = synth.BF16 if rng.random() < 0.8 else synth.F32
    q = ["i8", "e4m3"][int(rng.integers(0, 2))]
    gq = q if q == "i8" else ["e4m3", "e5m2"][int(rng.integers(0, 2))]
    code = {"i8": O.I8, "e4m3": O.E4M3, "e5m2": O.E5M2}
    qt, gt, b = code[q], code[gq], _block(rng)
    long_m = rng.random() < 0.15  # dY and X columns longer than 4096
    m = int(rng.integers(4097, 8500) if long_m else rng.integers(1, 700))
    n = 8 * int(rng.integers(1, 16 if long_m else 100))
    k = 8 * int(rng.integers(1, 16 if long_m else 150))
    signs, sr, fwd = rng.random() < 0.4, rng.random() < 0.3, rng.random() < 0.4
    print(f"case {case}: {'fwd' if fwd else 'bwd'} io {io} m {m} n {n} k {k} block {b} "
          f"{q}/{gq} signs {signs} sr {sr}", flush=True)
    x, w, dy = synth.layer(m, n, k, seed=7000 + case, io=io, with_grad=not fwd)
    rel = 4 * 2.0 ** -24 if io == synth.F32 else 2.0 ** -8 + 4 * 2.0 ** -24
    if fwd:
        sk = synth.sign_words(O.padded_len(k, b), seed=case) if signs else None
        y = H.linear_fwd(to_dev(x), to_dev(w), b, q_dtype=Q_TORCH[qt],
                         signs_k=signs_dev(sk) if signs else None,
                         y_dtype=torch.float32 if io == synth.F32 else torch.bfloat16)
        torch.cuda.synchronize()
        got = to_np64(y)
        assert rel_fro(got, O.linear_fwd(x, w, b, qt, precision=64, signs_k=sk)) <= 1e-2
        r32 = O.linear_fwd(x, w, b, qt, precision=32, signs_k=sk)
        ex = 0.0
        if qt != O.I8:
            ex = fp8_extra(x, O.ROWS, qt, w, O.ROWS, qt, b, dict(signs=sk), dict(signs=sk))
        ok, nbad = bound_ok(got, r32, rel, ex)
        assert ok, f"{nbad} outputs outside the bound"
        return
    sn = synth.sign_words(O.padded_len(n, b), seed=case + 1) if signs else None
    sm = synth.sign_words(O.padded_len(m, b), seed=case + 2) if signs else None
    dx, dw = H.linear_bwd(to_dev(dy), to_dev(x), to_dev(w), b, q_dtype=Q_TORCH[qt],
                          grad_q_dtype=Q_TORCH[gt], signs_n=signs_dev(sn) if signs else None,
                          signs_m=signs_dev(sm) if signs else None,
                          grad_rounding="stochastic" if sr else "nearest", seed=SEED64,
                          counter=COUNTER64)
    torch.cuda.synchronize()
    gdx, gdw = to_np64(dx), to_np64(dw)
    o = dict(signs_n=sn, signs_m=sm, grad_rounding=O.STOCHASTIC if sr else O.RNE, key=KEY,
             ctr_hi=CTR)
    r64 = O.linear_bwd(dy, x, w, b, qt, gt, precision=64, **o)
    assert rel_fro(gdx, r64[0]) <= 1e-2 and rel_fro(gdw, r64[1]) <= 1e-2
    r32 = O.linear_bwd(dy, x, w, b, qt, gt, precision=32, **o)
    ex_dx = ex_dw = 0.0
    if qt != O.I8:
        g_rows = dict(signs=sn, rounding=o["grad_rounding"], key=KEY, ctr_hi=CTR)
        g_cols = dict(signs=sm, rounding=o["grad_rounding"], key=KEY,
                      ctr_hi=(CTR[0], CTR[1] ^ 0x80000000))
        ex_dx = fp8_extra(dy, O.ROWS, gt, w, O.COLS, qt, b, g_rows, dict(signs=sn))
        ex_dw = fp8_extra(dy, O.COLS, gt, x, O.COLS, qt, b, g_cols, dict(signs=sm))
    ok, nbad = bound_ok(gdx, r32[0], rel, ex_dx)
    assert ok, f"dX: {nbad} outputs outside the bound"
    ok, nbad = bound_ok(gdw, r32[1], rel, ex_dw)
    assert ok, f"dW: {nbad} outputs outside the bound"
