"""Parity at the workloads' full sizes, through the same entry points and launch configuration
the benchmark times (halo_linear_fwd / halo_linear_bwd, halo_fwht_quant with its scratch).

The GPU computes every output; the oracle recomputes a seeded sample of output rows (first,
last and random ones) from its own codes: the sampled rows' operand vectors and all vectors of
the other operand, quantised by the oracle, multiplied in int64 / fp64 and dequantised.  Bars
as in the small-size tests: relative Frobenius error <= 1e-2 against the fp64 path, and
elementwise within one output rounding of the fp32-decision path (plus the FP8 matrix cores'
accumulation bound).  Rotation passes: sampled vectors' codes and scales bit-exact to the
fp32-decision oracle.
"""
import numpy as np
import pytest
import torch

import hadamard_rotated_precision_halo_amd as H
import oracle as O
import synth
from parity_util import Q_TORCH, codes_to_np, fp8_acc_bound, rel_fro, to_dev

pytestmark = pytest.mark.gpu

QT = {"i8": O.I8, "e4m3": O.E4M3, "e5m2": O.E5M2}
NAMES = list(synth.WORKLOADS)
_CACHE = {}


def _workload(name):
    if name not in _CACHE:
        _CACHE.clear()  # one workload resident at a time (the largest is ~0.7 GB of inputs)
        cfg, x, w, dy = synth.workload(name)
        dev = {"x": to_dev(x), "w": to_dev(w), "dy": to_dev(dy) if dy is not None else None}
        _CACHE[name] = (cfg, x, w, dy, dev)
    return _CACHE[name]


def _sample_rows(n, count, seed):
    rng = np.random.default_rng(seed)
    pick = rng.choice(n, size=min(count, n), replace=False)
    return np.unique(np.concatenate([[0, n - 1], pick])).astype(np.int64)


def _np(t):
    return t.float().cpu().numpy().astype(np.float64)


def _check_rows(got, a_src, a_axis, a_qt, b_src, b_axis, b_qt, block, rows, io):
    """got: GPU output rows `rows` [len(rows) x Q]; the product's A vectors `rows` come from
    a_src along a_axis, its B vectors are all vectors of b_src along b_axis."""
    for precision in (64, 32):
        qa, sa = O.fwht_quant(a_src, a_axis, block, a_qt, precision=precision, vec_idx=rows)
        qb, sb = O.fwht_quant(b_src, b_axis, block, b_qt, precision=precision)
        if a_qt == O.I8:
            acc = O.gemm_i8(qa, qb).astype(np.float64)
        else:
            acc = O.gemm_fp8(qa, a_qt, qb, b_qt)
        ref = O.dequant(acc, sa, sb)
        if precision == 64:
            assert rel_fro(got, ref) <= 1e-2, f"relative Frobenius error {rel_fro(got, ref)}"
            continue
        rel = 4 * 2.0 ** -24 if io == synth.F32 else 2.0 ** -8 + 4 * 2.0 ** -24
        extra = 0.0
        if a_qt != O.I8:
            absum = O.matmul_f64(np.abs(O.fp8_table(a_qt)[qa]), np.abs(O.fp8_table(b_qt)[qb]))
            extra = fp8_acc_bound(absum, qa.shape[1]) * np.outer(sa, sb) * (1 + 1e-6)
        scale = np.abs(ref) + 1e-6 * np.abs(ref).max()
        bad = np.abs(got - ref) > rel * scale + extra
        assert not bad.any(), f"{int(bad.sum())} of {bad.size} sampled outputs outside the bound"


@pytest.mark.parametrize("name", NAMES)
def test_fullsize_layer(name):
    cfg, x, w, dy, dev = _workload(name)
    q, gq, b = QT[cfg["q"]], QT[cfg["gq"]], cfg["block"]
    if cfg["fwd"]:
        y = H.linear_fwd(dev["x"], dev["w"], b, q_dtype=Q_TORCH[q],
                         y_dtype=torch.float32 if cfg["io"] == synth.F32 else torch.bfloat16)
        torch.cuda.synchronize()
        rows = _sample_rows(cfg["m"], 14, seed=cfg["m"] + 1)
        got = _np(y[torch.from_numpy(rows).to(y.device)])
        print(f"{name}: Y {tuple(y.shape)}, {len(rows)} sampled rows", flush=True)
        _check_rows(got, x, O.ROWS, q, w, O.ROWS, q, b, rows, cfg["io"])
        del y
    if cfg["bwd"]:
        dx, dw = H.linear_bwd(dev["dy"], dev["x"], dev["w"], b, q_dtype=Q_TORCH[q],
                              grad_q_dtype=Q_TORCH[gq])
        torch.cuda.synchronize()
        # dX[m x k] = dY . W: dY rows along n, W columns along n
        rows = _sample_rows(cfg["m"], 8, seed=cfg["m"] + 2)
        got = _np(dx[torch.from_numpy(rows).to(dx.device)])
        print(f"{name}: dX {tuple(dx.shape)}, {len(rows)} sampled rows", flush=True)
        _check_rows(got, dy, O.ROWS, gq, w, O.COLS, q, b, rows, cfg["io"])
        # dW[n x k] = dY^T . X: dY columns along m, X columns along m
        rows = _sample_rows(cfg["n"], 8, seed=cfg["n"] + 3)
        got = _np(dw[torch.from_numpy(rows).to(dw.device)])
        print(f"{name}: dW {tuple(dw.shape)}, {len(rows)} sampled rows", flush=True)
        _check_rows(got, dy, O.COLS, gq, x, O.COLS, q, b, rows, cfg["io"])


@pytest.mark.parametrize("axis,src", [(H.ROWS, "x"), (H.COLS, "dy"), (H.COLS, "x"), (H.ROWS, "dy")])
def test_fullsize_rotation_passes(axis, src):
    # the benchmark's rotation launches (4096 x 4096 bf16, block 256, INT8; the columns pass
    # with its scratch), sampled vectors bit-exact to the fp32-decision oracle
    name = "c3_bwd_4096x4096x4096_bf16_b256_i8"
    cfg, x, w, dy, dev = _workload(name)
    a = {"x": x, "dy": dy}[src]
    t = dev[src]
    ws = torch.empty(max(H.fwht_quant_workspace_bytes(*t.shape, axis, cfg["block"]), 256),
                     dtype=torch.uint8, device=t.device)
    qg, sg = H.fwht_quant(t, axis=axis, block=cfg["block"], workspace=ws)
    torch.cuda.synchronize()
    oax = O.ROWS if axis == H.ROWS else O.COLS
    idx = _sample_rows(qg.shape[0], 48, seed=7 + axis)
    r32, s32 = O.fwht_quant(a, oax, cfg["block"], O.I8, precision=32, vec_idx=idx)
    sel = torch.from_numpy(idx).to(qg.device)
    assert np.array_equal(codes_to_np(qg[sel]), r32)
    assert np.array_equal(sg[sel].cpu().numpy().astype(np.float64), s32)
