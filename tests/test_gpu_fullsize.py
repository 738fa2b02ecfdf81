"""Parity at the workloads' full sizes, through the same entry points and launch configuration
the benchmark times (halo_linear_fwd / halo_linear_bwd, halo_fwht_quant with its scratch,
halo_gemm_i8 / halo_gemm_fp8).

Bars:
  * layer outputs Y, dX, dW: relative Frobenius error <= 1e-2 against the oracle's fp64 path,
    and elementwise within one output rounding of its fp32-decision path (whose codes are the
    GPU's), plus the FP8 matrix cores' accumulation bound for FP8;
  * rotation passes: codes and scales bit-exact to the fp32 decision and within the code bar
    of the fp64 definition (|dq| <= 1 on at most 1e-4 of the codes, scales within 1e-5);
  * products on identical codes (the oracle's own): INT8 int32 accumulators bit-exact, FP8
    within the accumulation bound.

The 4096^3 workloads and the 256 x 1024 x 1024 single forward compare every element; the two
largest (8192 x 4096 x 11008, 16384 x 14336 x 4096) compare seeded samples of output rows and
columns (first, last and random ones) that the oracle recomputes from its own codes.
"""
import numpy as np
import pytest
import torch

import hadamard_rotated_precision_halo_amd as H
import oracle as O
import synth
from parity_util import Q_TORCH, bound_ok, check_fq_parity, codes_to_dev, codes_to_np, \
    fp8_acc_bound, rel_fro, to_dev

pytestmark = pytest.mark.gpu

QT = {"i8": O.I8, "e4m3": O.E4M3, "e5m2": O.E5M2}
FULL = ["c1_fwd_256x1024x1024_f32_b1024_i8", "c2_fwd_4096x4096x4096_bf16_b256_i8",
        "c3_bwd_4096x4096x4096_bf16_b256_i8", "c3_bwd_4096x4096x4096_bf16_b4096_i8"]
SAMPLED = ["c4_fwdbwd_8192x4096x11008_bf16_b128_i8", "c5_fwdbwd_16384x14336x4096_bf16_b512_fp8"]
_CACHE = {}


def _workload(name):
    if name not in _CACHE:
        _CACHE.clear()  # one workload resident at a time (the largest is ~0.7 GB of inputs)
        cfg, x, w, dy = synth.workload(name)
        dev = {"x": to_dev(x), "w": to_dev(w), "dy": to_dev(dy) if dy is not None else None}
        _CACHE[name] = (cfg, x, w, dy, dev)
    return _CACHE[name]


def _sample(n, count, seed):
    rng = np.random.default_rng(seed)
    pick = rng.choice(n, size=min(count, n), replace=False)
    return np.unique(np.concatenate([[0, n - 1], pick])).astype(np.int64)


def _np(t):
    return t.float().cpu().numpy().astype(np.float64)


def _rel_bound(io):
    # one output rounding (bf16: 2^-8 relative) plus a few fp32 roundings of the epilogue
    return 4 * 2.0 ** -24 if io == synth.F32 else 2.0 ** -8 + 4 * 2.0 ** -24


def _fp8_extra(qa, at, sa, qb, bt, sb):
    absum = O.matmul_f64(np.abs(O.fp8_table(at)[qa]), np.abs(O.fp8_table(bt)[qb]))
    return fp8_acc_bound(absum, qa.shape[1]) * np.outer(sa, sb) * (1 + 1e-6)


def _product(qa, at, qb, bt):
    if at == O.I8:
        return O.gemm_i8(qa, qb).astype(np.float64)
    return O.gemm_fp8(qa, at, qb, bt)


def _check_product(got, a_src, a_axis, a_qt, b_src, b_axis, b_qt, block, io, rows=None,
                   cols=None):
    """got: the GPU output (rows `rows` of it, or columns `cols`, or all of it) of the product
    whose A vectors come from a_src along a_axis and B vectors from b_src along b_axis."""
    for precision in (64, 32):
        qa, sa = O.fwht_quant(a_src, a_axis, block, a_qt, precision=precision, vec_idx=rows)
        qb, sb = O.fwht_quant(b_src, b_axis, block, b_qt, precision=precision, vec_idx=cols)
        ref = O.dequant(_product(qa, a_qt, qb, b_qt), sa, sb)
        if precision == 64:
            assert rel_fro(got, ref) <= 1e-2, f"relative Frobenius error {rel_fro(got, ref)}"
            continue
        extra = 0.0 if a_qt == O.I8 else _fp8_extra(qa, a_qt, sa, qb, b_qt, sb)
        ok, nbad = bound_ok(got, ref, _rel_bound(io), extra)
        assert ok, f"{nbad} of {got.size} outputs outside the bound"


@pytest.mark.parametrize("name", FULL)
def test_fullsize_layer_every_element(name):
    cfg, x, w, dy, dev = _workload(name)
    q, gq, b = QT[cfg["q"]], QT[cfg["gq"]], cfg["block"]
    if cfg["fwd"]:
        y = H.linear_fwd(dev["x"], dev["w"], b, q_dtype=Q_TORCH[q],
                         y_dtype=torch.float32 if cfg["io"] == synth.F32 else torch.bfloat16)
        torch.cuda.synchronize()
        print(f"{name}: Y {tuple(y.shape)}, every element", flush=True)
        _check_product(_np(y), x, O.ROWS, q, w, O.ROWS, q, b, cfg["io"])
        del y
    if cfg["bwd"]:
        dx, dw = H.linear_bwd(dev["dy"], dev["x"], dev["w"], b, q_dtype=Q_TORCH[q],
                              grad_q_dtype=Q_TORCH[gq])
        torch.cuda.synchronize()
        print(f"{name}: dX {tuple(dx.shape)}, every element", flush=True)
        _check_product(_np(dx), dy, O.ROWS, gq, w, O.COLS, q, b, cfg["io"])   # dY W
        print(f"{name}: dW {tuple(dw.shape)}, every element", flush=True)
        _check_product(_np(dw), dy, O.COLS, gq, x, O.COLS, q, b, cfg["io"])   # dY^T X


@pytest.mark.parametrize("name", SAMPLED)
def test_fullsize_layer_sampled(name):
    cfg, x, w, dy, dev = _workload(name)
    q, gq, b = QT[cfg["q"]], QT[cfg["gq"]], cfg["block"]
    y = H.linear_fwd(dev["x"], dev["w"], b, q_dtype=Q_TORCH[q])
    torch.cuda.synchronize()
    rows, cols = _sample(cfg["m"], 24, seed=cfg["m"] + 1), _sample(cfg["n"], 24, seed=cfg["n"] + 1)
    print(f"{name}: Y {tuple(y.shape)}, {len(rows)} rows and {len(cols)} columns", flush=True)
    yr = _np(y[torch.from_numpy(rows).to(y.device)])
    _check_product(yr, x, O.ROWS, q, w, O.ROWS, q, b, cfg["io"], rows=rows)
    yc = _np(y[:, torch.from_numpy(cols).to(y.device)])
    _check_product(yc, x, O.ROWS, q, w, O.ROWS, q, b, cfg["io"], cols=cols)
    del y, yr, yc
    dx, dw = H.linear_bwd(dev["dy"], dev["x"], dev["w"], b, q_dtype=Q_TORCH[q],
                          grad_q_dtype=Q_TORCH[gq])
    torch.cuda.synchronize()
    # dX[m x k] = dY . W: dY rows along n, W columns along n
    rows, cols = _sample(cfg["m"], 12, seed=cfg["m"] + 2), _sample(cfg["k"], 12, seed=cfg["k"] + 2)
    print(f"{name}: dX {tuple(dx.shape)}, {len(rows)} rows and {len(cols)} columns", flush=True)
    _check_product(_np(dx[torch.from_numpy(rows).to(dx.device)]), dy, O.ROWS, gq, w, O.COLS, q,
                   b, cfg["io"], rows=rows)
    _check_product(_np(dx[:, torch.from_numpy(cols).to(dx.device)]), dy, O.ROWS, gq, w, O.COLS,
                   q, b, cfg["io"], cols=cols)
    # dW[n x k] = dY^T . X: dY columns along m, X columns along m
    rows, cols = _sample(cfg["n"], 12, seed=cfg["n"] + 3), _sample(cfg["k"], 12, seed=cfg["k"] + 3)
    print(f"{name}: dW {tuple(dw.shape)}, {len(rows)} rows and {len(cols)} columns", flush=True)
    _check_product(_np(dw[torch.from_numpy(rows).to(dw.device)]), dy, O.COLS, gq, x, O.COLS, q,
                   b, cfg["io"], rows=rows)
    _check_product(_np(dw[:, torch.from_numpy(cols).to(dw.device)]), dy, O.COLS, gq, x, O.COLS,
                   q, b, cfg["io"], cols=cols)


# the three products of each layer workload: (A source, A axis, B source, B axis, codes)
_PRODUCTS = {"fwd": ("x", O.ROWS, "w", O.ROWS), "dx": ("dy", O.ROWS, "w", O.COLS),
             "dw": ("dy", O.COLS, "x", O.COLS)}


@pytest.mark.parametrize("name,prod", [(n, p) for n in SAMPLED for p in _PRODUCTS])
def test_fullsize_products_on_oracle_codes(name, prod):
    # Given identical codes (the oracle's, fp32 decision), the INT8 product's int32
    # accumulators are bit-exact and the FP8 product within its accumulation bound: 256 seeded
    # rows x all columns and 256 columns x all rows of each product at full size.
    cfg, x, w, dy, dev = _workload(name)
    src = {"x": x, "w": w, "dy": dy}
    an, aax, bn, bax = _PRODUCTS[prod]
    qw = QT[cfg["q"]]
    at = QT[cfg["gq"]] if an == "dy" else qw
    bt = qw
    b = cfg["block"]
    qa, sa = O.fwht_quant(src[an], aax, b, at, precision=32)
    qb, sb = O.fwht_quant(src[bn], bax, b, bt, precision=32)
    P, Q, Kc = qa.shape[0], qb.shape[0], qa.shape[1]
    print(f"{name} {prod}: {P} x {Q} x {Kc} on oracle codes", flush=True)
    A, B = codes_to_dev(qa, at), codes_to_dev(qb, bt)
    rows, cols = _sample(P, 256, seed=P + 5), _sample(Q, 256, seed=Q + 5)
    if at == O.I8:
        acc = H.gemm_i8(A, None, B, None, out_dtype=torch.int32)
        torch.cuda.synchronize()
        got_r = acc[torch.from_numpy(rows).to(acc.device)].cpu().numpy().astype(np.int64)
        got_c = acc[:, torch.from_numpy(cols).to(acc.device)].cpu().numpy().astype(np.int64)
        assert np.array_equal(got_r, O.gemm_i8(qa[rows], qb)), "sampled rows differ"
        assert np.array_equal(got_c, O.gemm_i8(qa, qb[cols])), "sampled columns differ"
        return
    one_a = torch.ones(P, dtype=torch.float32, device=A.device)
    one_b = torch.ones(Q, dtype=torch.float32, device=A.device)
    acc = H.gemm_fp8(A, one_a, B, one_b, out_dtype=torch.float32)
    torch.cuda.synchronize()
    for sel, qa_s, qb_s, got in (
            (rows, qa[rows], qb, acc[torch.from_numpy(rows).to(acc.device)]),
            (cols, qa, qb[cols], acc[:, torch.from_numpy(cols).to(acc.device)])):
        ref = O.gemm_fp8(qa_s, at, qb_s, bt)
        absum = O.matmul_f64(np.abs(O.fp8_table(at)[qa_s]), np.abs(O.fp8_table(bt)[qb_s]))
        err = np.abs(got.cpu().numpy().astype(np.float64) - ref)
        bad = err > fp8_acc_bound(absum, Kc) * (1 + 1e-6)
        assert not bad.any(), f"{int(bad.sum())} sampled accumulators outside the bound"


def test_gemm_i8_int32_exact_4096():
    # every int32 accumulator of the 4096^3 product on the oracle's codes of the forward's X
    # and W (256 output tiles over the 8 XCDs, the grouped tile order), bit-exact
    cfg, x, w, dy, dev = _workload("c2_fwd_4096x4096x4096_bf16_b256_i8")
    qa, _ = O.fwht_quant(x, O.ROWS, 256, O.I8, precision=32)
    qb, _ = O.fwht_quant(w, O.ROWS, 256, O.I8, precision=32)
    acc = H.gemm_i8(codes_to_dev(qa, O.I8), None, codes_to_dev(qb, O.I8), None,
                    out_dtype=torch.int32)
    torch.cuda.synchronize()
    got = acc.cpu().numpy().astype(np.int64)
    ref = O.gemm_i8(qa, qb)
    assert np.array_equal(got, ref), f"{int((got != ref).sum())} accumulators differ"


@pytest.mark.parametrize("axis,src", [(H.ROWS, "x"), (H.COLS, "dy"), (H.COLS, "x"), (H.ROWS, "dy")])
def test_fullsize_rotation_passes(axis, src):
    # the benchmark's rotation launches (4096 x 4096 bf16, block 256, INT8; the columns pass
    # with its scratch): every vector, both bars
    name = "c3_bwd_4096x4096x4096_bf16_b256_i8"
    cfg, x, w, dy, dev = _workload(name)
    a = {"x": x, "dy": dy}[src]
    t = dev[src]
    ws = torch.empty(max(H.fwht_quant_workspace_bytes(*t.shape, axis, cfg["block"]), 256),
                     dtype=torch.uint8, device=t.device)
    qg, sg = H.fwht_quant(t, axis=axis, block=cfg["block"], workspace=ws)
    torch.cuda.synchronize()
    check_fq_parity(codes_to_np(qg), sg.cpu().numpy(), a, O.ROWS if axis == H.ROWS else O.COLS,
                    cfg["block"], O.I8)
