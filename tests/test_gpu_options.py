"""GPU parity of the randomised transform H D, the zero padding and the stochastic rounding
(halo_fwht_quant_ex, halo_linear_fwd_ex, halo_linear_bwd_ex) against the CPU oracle.

Bars as for the plain calls: codes and scales bit-identical to the oracle's fp32-decision
path, which draws the same Philox4x32-10 uniforms from the same key and counter; codes within
the +-1 / 0.01 % budget of its fp64 path; layer outputs within 1e-2 relative Frobenius of the
fp64 path and within one output rounding (plus the FP8 accumulation bound) of the fp32 path.
Cases cover every kernel that serves these shapes: the wave-slice rows kernel (one or several
rows per wave, several waves per row), the single-read columns kernel (one or several parts
per column), the backward batch launch, and the older rows / two-read columns kernels (fp32
input, short or odd padded lengths).
"""
import numpy as np
import pytest
import torch

import hadamard_rotated_precision_halo_amd as H
import oracle as O
import synth
from parity_util import COUNTER64, CTR, DEV, KEY, Q_TORCH, SEED64, assert_codes_close_to_fp64, \
    check_fq_parity, \
    codes_to_np, rel_fro, to_dev
from parity_util import bound_ok as _bound_ok, fp8_extra as _fp8_extra, signs_dev as _signs_dev, \
    to_np64 as _np

pytestmark = pytest.mark.gpu

QT = {"i8": O.I8, "e4m3": O.E4M3, "e5m2": O.E5M2}


def _input(rows, cols, io, seed):
    rng = np.random.default_rng(seed)
    a = synth.activations(rng, rows, cols)
    return synth.bf16_bits(a) if io == "bf16" else a


ROT_CASES = [
    # axis, io, block, rows, cols, qtype, signs, stochastic, workspace
    ("rows", "bf16", 256, 37, 4096, "i8", True, True, None),       # wave slice, one row per wave
    ("rows", "bf16", 128, 19, 1000, "e4m3", True, True, None),     # padded 1000 -> 1024
    ("rows", "bf16", 64, 21, 200, "e5m2", False, True, None),      # padded 200 -> 256
    ("rows", "bf16", 256, 64, 4096, "i8", True, False, None),      # signs only
    ("rows", "bf16", 128, 16, 1000, "i8", False, False, None),     # padding only
    ("rows", "bf16", 4096, 3, 5000, "e4m3", True, True, None),     # padded 5000 -> 8192, 2 waves
    ("rows", "bf16", 512, 5, 14336, "e5m2", True, True, None),     # four waves per row
    ("rows", "f32", 256, 9, 1000, "i8", True, True, None),         # fp32: older rows kernel
    ("rows", "bf16", 16, 33, 1000, "i8", True, True, None),        # padded 1008: older kernel
    ("rows", "f32", 1024, 4, 3000, "e5m2", True, True, None),      # padded 3072: older kernel
    ("rows", "bf16", 256, 3, 20480, "e5m2", True, True, None),     # five waves per row
    ("rows", "f32", 512, 2, 16384, "i8", True, True, None),        # fp32 SR: older kernel, longest
    ("cols", "bf16", 256, 4096, 64, "i8", True, True, None),       # 4 parts per column
    ("cols", "bf16", 128, 1000, 200, "i8", True, True, None),      # padded 1000 -> 1024, 1 part
    ("cols", "bf16", 128, 5000, 72, "e5m2", True, True, None),     # padded 5120, 5 parts
    ("cols", "bf16", 512, 3000, 40, "e4m3", False, True, None),    # padded 3072, 3 parts
    ("cols", "bf16", 4096, 5000, 16, "e4m3", True, True, None),    # padded 8192, 2 parts
    ("cols", "bf16", 256, 4096, 64, "i8", True, False, None),      # signs only
    ("cols", "f32", 256, 700, 24, "i8", True, True, None),         # fp32 SR: two-read kernel
    ("cols", "f32", 256, 4096, 64, "i8", True, False, None),       # fp32: single read, signs
    ("cols", "f32", 128, 5000, 72, "e5m2", True, False, None),     # fp32: padded 5120, 5 parts
    ("cols", "f32", 4096, 5000, 16, "e4m3", False, False, None),   # fp32: padded 8192, 2 parts
    ("cols", "bf16", 16, 13, 64, "i8", True, True, None),          # 13 rows padded to 16
    ("cols", "bf16", 256, 2000, 64, "e5m2", True, True, False),    # no scratch: two-read kernel
]


@pytest.mark.parametrize("axis,io,block,rows,cols,q,signs,sr,ws", ROT_CASES)
def test_rotation_options_match_oracle(axis, io, block, rows, cols, q, signs, sr, ws):
    qt = QT[q]
    ax_h, ax_o = (H.ROWS, O.ROWS) if axis == "rows" else (H.COLS, O.COLS)
    x = _input(rows, cols, io, seed=rows + 3 * cols + block)
    L = cols if axis == "rows" else rows
    Lp = O.padded_len(L, block)
    words = synth.sign_words(Lp, seed=L + block) if signs else None
    kw = dict(signs=_signs_dev(words) if signs else None,
              rounding="stochastic" if sr else "nearest", seed=SEED64, counter=COUNTER64)
    if ws is False:
        kw["workspace"] = False
    print(f"{axis} {io} block {block} {rows}x{cols} {q} signs={signs} sr={sr}", flush=True)
    qg, sg = H.fwht_quant(to_dev(x), axis=ax_h, block=block, q_dtype=Q_TORCH[qt], **kw)
    torch.cuda.synchronize()
    got, gs = codes_to_np(qg), sg.cpu().numpy().astype(np.float64)
    assert got.shape == ((rows if axis == "rows" else cols), Lp)
    ok = dict(signs=words, rounding=O.STOCHASTIC if sr else O.RNE, key=KEY, ctr_hi=CTR)
    r32, s32 = O.fwht_quant(x, ax_o, block, qt, precision=32, **ok)
    assert np.array_equal(got, r32), f"{int((got != r32).sum())} codes differ from the fp32 path"
    assert np.array_equal(gs, s32)
    r64, s64 = O.fwht_quant(x, ax_o, block, qt, precision=64, **ok)
    assert_codes_close_to_fp64(got, r64, qt, block, x=x, oaxis=ax_o, opts=ok)
    np.testing.assert_allclose(gs, s64, rtol=1e-5)


def test_stochastic_rounding_is_unbiased_on_the_gpu():
    # many identical rows draw independently: the mean of the dequantised codes approaches the
    # rotated values, while nearest-even rounding keeps its bias
    n = 4096
    rng = np.random.default_rng(5)
    v = rng.standard_normal(256).astype(np.float32)
    x = np.tile(v, (n, 1))
    qg, sg = H.fwht_quant(to_dev(x), axis=H.ROWS, block=256, rounding="stochastic", seed=99)
    torch.cuda.synchronize()
    deq = qg.float().cpu().numpy().astype(np.float64) * sg.cpu().numpy()[:, None]
    y, _ = O.fwht_quant(x[:1], O.ROWS, 256, O.F64)
    s = float(sg[0])
    z = np.abs(deq.mean(axis=0) - y[0]) / (0.5 * s / np.sqrt(n))
    assert z.max() < 5.5, f"max z-score {z.max():.2f}"


def test_signs_from_a_seed_are_shared_and_orthogonal():
    # hadamard_signs draws the same words from the same seed; the signed transform keeps the
    # rotated product equal to the plain one (fp32 value mode)
    a = H.hadamard_signs(4096, seed=1234)
    b = H.hadamard_signs(4096, seed=1234)
    assert torch.equal(a, b) and a.shape == (128,)
    assert not torch.equal(a, H.hadamard_signs(4096, seed=1235))
    rng = np.random.default_rng(6)
    x = rng.standard_normal((64, 4096)).astype(np.float32)
    w = rng.standard_normal((48, 4096)).astype(np.float32)
    sgn = a.to(DEV)
    yx, ax_ = H.fwht_quant(to_dev(x), axis=H.ROWS, block=256, q_dtype=torch.float32, signs=sgn)
    yw, aw_ = H.fwht_quant(to_dev(w), axis=H.ROWS, block=256, q_dtype=torch.float32, signs=sgn)
    prod = (yx.double() @ yw.double().T).cpu().numpy()
    exact = x.astype(np.float64) @ w.astype(np.float64).T
    assert rel_fro(prod, exact) < 1e-6


FWD = [  # m, n, k, block, io, q, signs
    (96, 80, 200, 64, synth.BF16, "i8", True),      # k padded 200 -> 256
    (64, 48, 200, 16, synth.BF16, "i8", True),      # k padded to 208 (224 on the device)
    (128, 96, 1000, 256, synth.BF16, "e4m3", True),
    (256, 512, 4096, 256, synth.BF16, "i8", True),  # signs only, no padding
    (40, 64, 3000, 1024, synth.F32, "i8", False),   # fp32, padded 3072: older rows kernel
]


@pytest.mark.parametrize("m,n,k,block,io,q,signs", FWD)
def test_linear_fwd_options(m, n, k, block, io, q, signs):
    qt = QT[q]
    x, w, _ = synth.layer(m, n, k, seed=m + 2 * n + k, io=io, with_grad=False)
    words = synth.sign_words(O.padded_len(k, block), seed=k) if signs else None
    y = H.linear_fwd(to_dev(x), to_dev(w), block, q_dtype=Q_TORCH[qt],
                     signs_k=_signs_dev(words) if signs else None)
    torch.cuda.synchronize()
    got = _np(y)
    ref64 = O.linear_fwd(x, w, block, qt, precision=64, signs_k=words)
    assert rel_fro(got, ref64) <= 1e-2
    ref32 = O.linear_fwd(x, w, block, qt, precision=32, signs_k=words)
    rel = 4 * 2.0 ** -24 if io == synth.F32 else 2.0 ** -8 + 4 * 2.0 ** -24
    extra = 0.0
    if qt != O.I8:
        o = dict(signs=words)
        extra = _fp8_extra(x, O.ROWS, qt, w, O.ROWS, qt, block, o, o)
    ok, nbad = _bound_ok(got, ref32, rel, extra)
    assert ok, f"{nbad} outputs outside the bound"


BWD = [  # m, n, k, block, io, q, gq, signs, sr
    (200, 136, 96, 64, synth.BF16, "i8", "i8", True, True),        # m, n padded
    (1024, 1024, 512, 256, synth.BF16, "i8", "i8", True, True),    # the batch launch
    (1024, 1024, 512, 256, synth.BF16, "i8", "i8", False, True),   # batch, rounding only
    (512, 256, 256, 128, synth.BF16, "e4m3", "e5m2", True, True),  # FP8, batch launch
    (300, 264, 128, 128, synth.BF16, "e4m3", "e4m3", True, True),  # same code types, padded
    (2048, 2048, 256, 256, synth.BF16, "i8", "i8", True, True),    # column passes in 2 parts
    (256, 200, 64, 64, synth.F32, "i8", "i8", True, True),         # fp32: older kernels
    (96, 5000, 64, 4096, synth.BF16, "i8", "i8", True, True),      # n padded to 8192: long rows
    (64, 20480, 64, 256, synth.BF16, "i8", "i8", True, True),      # dY rows of 20480
]


@pytest.mark.parametrize("m,n,k,block,io,q,gq,signs,sr", BWD)
def test_linear_bwd_options(m, n, k, block, io, q, gq, signs, sr):
    qt, gt = QT[q], QT[gq]
    x, w, dy = synth.layer(m, n, k, seed=5 * m + n + k, io=io)
    sn = synth.sign_words(O.padded_len(n, block), seed=n + 1) if signs else None
    sm = synth.sign_words(O.padded_len(m, block), seed=m + 2) if signs else None
    print(f"bwd {m}x{n}x{k} block {block} {q}/{gq} signs={signs} sr={sr}", flush=True)
    dx, dw = H.linear_bwd(to_dev(dy), to_dev(x), to_dev(w), block, q_dtype=Q_TORCH[qt],
                          grad_q_dtype=Q_TORCH[gt],
                          signs_n=_signs_dev(sn) if signs else None,
                          signs_m=_signs_dev(sm) if signs else None,
                          grad_rounding="stochastic" if sr else "nearest", seed=SEED64,
                          counter=COUNTER64)
    torch.cuda.synchronize()
    gdx, gdw = _np(dx), _np(dw)
    o = dict(signs_n=sn, signs_m=sm, grad_rounding=O.STOCHASTIC if sr else O.RNE, key=KEY,
             ctr_hi=CTR)
    r64 = O.linear_bwd(dy, x, w, block, qt, gt, precision=64, **o)
    assert rel_fro(gdx, r64[0]) <= 1e-2
    assert rel_fro(gdw, r64[1]) <= 1e-2
    r32 = O.linear_bwd(dy, x, w, block, qt, gt, precision=32, **o)
    rel = 4 * 2.0 ** -24 if io == synth.F32 else 2.0 ** -8 + 4 * 2.0 ** -24
    ex_dx = ex_dw = 0.0
    if qt != O.I8:
        g_rows = dict(signs=sn, rounding=o["grad_rounding"], key=KEY, ctr_hi=CTR)
        g_cols = dict(signs=sm, rounding=o["grad_rounding"], key=KEY,
                      ctr_hi=(CTR[0], CTR[1] ^ 0x80000000))
        ex_dx = _fp8_extra(dy, O.ROWS, gt, w, O.COLS, qt, block, g_rows, dict(signs=sn))
        ex_dw = _fp8_extra(dy, O.COLS, gt, x, O.COLS, qt, block, g_cols, dict(signs=sm))
    ok, nbad = _bound_ok(gdx, r32[0], rel, ex_dx)
    assert ok, f"dX: {nbad} outputs outside the bound"
    ok, nbad = _bound_ok(gdw, r32[1], rel, ex_dw)
    assert ok, f"dW: {nbad} outputs outside the bound"


def test_fullsize_rotation_with_options():
    # the 4096 x 4096 bf16 gradient at block 256 with signs and stochastic rounding, in the
    # launch configuration of the benchmark's option leg: every vector, both bars
    _, x, w, dy = synth.workload("c3_bwd_4096x4096x4096_bf16_b256_i8")
    t = to_dev(dy)
    words = synth.sign_words(4096, seed=77)
    sg = _signs_dev(words)
    for axis, oax in ((H.ROWS, O.ROWS), (H.COLS, O.COLS)):
        ws = torch.empty(max(H.fwht_quant_workspace_bytes(4096, 4096, axis, 256), 256),
                         dtype=torch.uint8, device=DEV)
        qg, sc = H.fwht_quant(t, axis=axis, block=256, signs=sg, rounding="stochastic",
                              seed=SEED64, counter=COUNTER64, workspace=ws)
        torch.cuda.synchronize()
        check_fq_parity(codes_to_np(qg), sc.cpu().numpy(), dy, oax, 256, O.I8, signs=words,
                        rounding=O.STOCHASTIC, key=KEY, ctr_hi=CTR)
