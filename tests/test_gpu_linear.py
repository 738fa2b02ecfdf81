"""GPU parity of the layer entry points halo_linear_fwd / halo_linear_bwd against the oracle.

Bars: relative Frobenius error <= 1e-2 against the oracle's fp64 quantised path; against the oracle's fp32-decision path the codes are identical, so the only
difference left is the output rounding (bf16: 2^-8 relative per element, with slack for the
fp32 epilogue).  Workloads are the synth layer tensors (outlier channels, Student-t grads).
"""
import numpy as np
import pytest
import torch

import hadamard_rotated_precision_halo_amd as H
import oracle as O
import synth
from parity_util import Q_TORCH, bound_ok, rel_fro, to_dev
from parity_util import fp8_extra as _fp8_extra, to_np64 as _np

pytestmark = pytest.mark.gpu

QT = {"i8": O.I8, "e4m3": O.E4M3, "e5m2": O.E5M2}


def _elementwise_bound(got, ref, rel, extra=0.0):
    return bound_ok(got, ref, rel, extra)[0]


FWD = [  # m, n, k, block, io, q
    (256, 1024, 1024, 1024, synth.F32, "i8"),     # the single-linear workload, full size (4 x50 channels)
    (320, 384, 1024, 256, synth.BF16, "i8"),
    (96, 200, 11008, 128, synth.BF16, "i8"),      # ragged n, 86 blocks along k
    (256, 512, 4096, 512, synth.BF16, "e4m3"),
    (64, 64, 512, 1, synth.BF16, "i8"),           # block 1: no rotation
    (0, 256, 256, 256, synth.BF16, "i8"),         # no tokens
    (64, 96, 20000, 128, synth.BF16, "i8"),       # k padded to 20096: five waves per row
    (32, 64, 28672, 256, synth.F32, "e4m3"),      # fp32 rows of 28672: seven waves per row
]


@pytest.mark.parametrize("m,n,k,block,io,q", FWD)
def test_linear_fwd(m, n, k, block, io, q):
    # the single-linear workload states 4 outlier channels; the others take 0.1 % of k
    outliers = 4 if (m, n, k) == (256, 1024, 1024) else None
    x, w, _ = synth.layer(m, n, k, seed=m + n + k, io=io, with_grad=False, outliers=outliers)
    y = H.linear_fwd(to_dev(x), to_dev(w), block, q_dtype=Q_TORCH[QT[q]])
    torch.cuda.synchronize()
    got = _np(y)
    assert got.shape == (m, n)
    if m == 0:
        return
    ref64 = O.linear_fwd(x, w, block, QT[q], precision=64)
    assert rel_fro(got, ref64) <= 1e-2
    ref32 = O.linear_fwd(x, w, block, QT[q], precision=32)
    rel = 4 * 2.0 ** -24 if io == synth.F32 else 2.0 ** -8 + 4 * 2.0 ** -24
    extra = 0.0
    if QT[q] != O.I8:  # grouped accumulation of the FP8 matrix cores
        extra = _fp8_extra(x, O.ROWS, QT[q], w, O.ROWS, QT[q], block)
    assert _elementwise_bound(got, ref32, rel, extra)


BWD = [  # m, n, k, block, io, q, gq
    (512, 384, 256, 128, synth.BF16, "i8", "i8"),
    (256, 512, 768, 256, synth.BF16, "i8", "i8"),
    (1024, 512, 256, 512, synth.BF16, "e4m3", "e5m2"),
    (256, 256, 128, 64, synth.F32, "i8", "i8"),
    (512, 512, 256, 256, synth.BF16, "e4m3", "e4m3"),
    (2048, 2048, 256, 256, synth.BF16, "i8", "i8"),    # every column pass split over 2 tasks
    (2048, 512, 256, 512, synth.BF16, "e4m3", "e5m2"),  # split dY / X passes, separate launches
    (64, 28672, 64, 256, synth.BF16, "i8", "i8"),      # dY rows of 28672 (dX of a wide layer)
]


@pytest.mark.parametrize("m,n,k,block,io,q,gq", BWD)
def test_linear_bwd(m, n, k, block, io, q, gq):
    x, w, dy = synth.layer(m, n, k, seed=7 * m + n + k, io=io)
    dx, dw = H.linear_bwd(to_dev(dy), to_dev(x), to_dev(w), block, q_dtype=Q_TORCH[QT[q]],
                          grad_q_dtype=Q_TORCH[QT[gq]])
    torch.cuda.synchronize()
    gdx, gdw = _np(dx), _np(dw)
    r64 = O.linear_bwd(dy, x, w, block, QT[q], QT[gq], precision=64)
    assert rel_fro(gdx, r64[0]) <= 1e-2
    assert rel_fro(gdw, r64[1]) <= 1e-2
    r32 = O.linear_bwd(dy, x, w, block, QT[q], QT[gq], precision=32)
    rel = 4 * 2.0 ** -24 if io == synth.F32 else 2.0 ** -8 + 4 * 2.0 ** -24
    ex_dx = ex_dw = 0.0
    if QT[q] != O.I8:
        ex_dx = _fp8_extra(dy, O.ROWS, QT[gq], w, O.COLS, QT[q], block)
        ex_dw = _fp8_extra(dy, O.COLS, QT[gq], x, O.COLS, QT[q], block)
    assert _elementwise_bound(gdx, r32[0], rel, ex_dx)
    assert _elementwise_bound(gdw, r32[1], rel, ex_dw)


def test_linear_bwd_single_outputs():
    m, n, k, b = 256, 256, 512, 128
    x, w, dy = synth.layer(m, n, k, seed=11)
    dxo, dwo = H.linear_bwd(to_dev(dy), to_dev(x), to_dev(w), b, want_dw=False)
    assert dwo is None
    dxb, dwb = H.linear_bwd(to_dev(dy), to_dev(x), to_dev(w), b, want_dx=False)
    assert dxb is None
    dx, dw = H.linear_bwd(to_dev(dy), to_dev(x), to_dev(w), b)
    assert torch.equal(dx, dxo) and torch.equal(dw, dwb)


def test_linear_bwd_dw_only_long_columns():
    # no rows pass precedes the column passes: their scratch is cleared by a fill of its own
    m, n, k, b = 4096, 256, 128, 256
    x, w, dy = synth.layer(m, n, k, seed=13)
    _, dw = H.linear_bwd(to_dev(dy), to_dev(x), to_dev(w), b, want_dx=False)
    _, dw_ref = H.linear_bwd(to_dev(dy), to_dev(x), to_dev(w), b)
    assert torch.equal(dw, dw_ref)
    r64 = O.linear_bwd(dy, x, w, b, O.I8, O.I8, precision=64)
    assert rel_fro(_np(dw), r64[1]) <= 1e-2


def test_rotation_beats_no_rotation_on_outliers():
    # the method's purpose: with outlier channels the rotated INT8 layer is closer to the
    # exact product than the same layer without rotation (block 1)
    m, n, k = 512, 512, 4096
    x, w, _ = synth.layer(m, n, k, seed=21, io=synth.BF16, with_grad=False)
    xf, wf = synth.bf16_to_f32(x).astype(np.float64), synth.bf16_to_f32(w).astype(np.float64)
    exact = xf @ wf.T
    rot = _np(H.linear_fwd(to_dev(x), to_dev(w), 256))
    raw = _np(H.linear_fwd(to_dev(x), to_dev(w), 1))
    assert rel_fro(rot, exact) * 2.5 < rel_fro(raw, exact)


def test_repeat_runs_bit_identical():
    m, n, k, b = 512, 768, 1024, 256
    x, w, dy = synth.layer(m, n, k, seed=31)
    X, W, DY = to_dev(x), to_dev(w), to_dev(dy)
    y0 = H.linear_fwd(X, W, b)
    dx0, dw0 = H.linear_bwd(DY, X, W, b)
    for _ in range(5):
        assert torch.equal(H.linear_fwd(X, W, b), y0)
        dx, dw = H.linear_bwd(DY, X, W, b)
        assert torch.equal(dx, dx0) and torch.equal(dw, dw0)


def test_concurrent_host_threads():
    # Calls are documented as thread-safe: four host threads, each on its own stream, run
    # forward + backward on their own inputs at the same time (ctypes releases the GIL around
    # the C calls); every result equals the same call made alone, bit for bit.
    import threading
    m, n, k, b = 512, 512, 1024, 256
    cases = []
    for t in range(4):
        x, w, dy = synth.layer(m, n, k, seed=60 + t)
        cases.append((to_dev(x), to_dev(w), to_dev(dy)))
    ref = []
    for X, W, DY in cases:
        y = H.linear_fwd(X, W, b)
        dx, dw = H.linear_bwd(DY, X, W, b)
        ref.append((y, dx, dw))
    torch.cuda.synchronize()
    out, errs = [None] * len(cases), []
    start = threading.Barrier(len(cases))

    def work(i):
        try:
            s = torch.cuda.Stream()
            X, W, DY = cases[i]
            start.wait(timeout=30)
            res = []
            with torch.cuda.stream(s):
                for _ in range(3):
                    y = H.linear_fwd(X, W, b)
                    dx, dw = H.linear_bwd(DY, X, W, b)
                    res.append((y, dx, dw))
            s.synchronize()
            out[i] = res
        except Exception as e:  # reported below, in the test's own thread
            errs.append(e)

    threads = [threading.Thread(target=work, args=(i,)) for i in range(len(cases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=60)
    assert not errs, errs
    for i, res in enumerate(out):
        assert res is not None, f"thread {i} did not finish"
        for y, dx, dw in res:
            assert torch.equal(y, ref[i][0])
            assert torch.equal(dx, ref[i][1]) and torch.equal(dw, ref[i][2])


def test_non_default_stream():
    m, n, k, b = 256, 256, 1024, 256
    x, w, _ = synth.layer(m, n, k, seed=41, with_grad=False)
    X, W = to_dev(x), to_dev(w)
    ref = H.linear_fwd(X, W, b)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        y = H.linear_fwd(X, W, b)
    s.synchronize()
    assert torch.equal(y, ref)
