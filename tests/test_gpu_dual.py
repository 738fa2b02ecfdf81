"""GPU parity of halo_fwht_quant_dual: both rotation passes of one matrix from a single read.

Its row codes and scales must be exactly those of the rows pass and its column codes and
scales those of the columns pass: bit-exact to the oracle's fp32 decision and within the code
bar of its fp64 definition, on every vector.  Shapes that the single read does not take
(sizes that are not multiples of 256, fp32 input, stochastic rounding, no scratch) run the two
passes and must give the same.  The single-read launch's exchanges are bounded waits like the
columns pass's; with a limit of one poll some tasks stop waiting and the repair launch stores
their strips, and every call must still give the oracle's codes.
"""
import numpy as np
import pytest
import torch

import hadamard_rotated_precision_halo_amd as H
import oracle as O
import synth
from parity_util import (CTR, DEV, KEY, Q_TORCH, check_fq_parity, codes_to_np, signs_dev,
                         to_dev)

pytestmark = pytest.mark.gpu

SEED64 = KEY[0] | (KEY[1] << 32)
CTR_R = CTR[0] | (CTR[1] << 32)
CTR_C = CTR[0] | ((CTR[1] ^ 0x80000000) << 32)


def _grad(rows, cols, io, seed):
    a = synth.grads(np.random.default_rng(seed), rows, cols)
    return synth.bf16_bits(a) if io == "bf16" else a


def _check_both(x_np, block, qt, qr, sr, qc, sc, row_opts=None, col_opts=None):
    check_fq_parity(codes_to_np(qr), sr.cpu().numpy(), x_np, O.ROWS, block, qt,
                    **(row_opts or {}))
    check_fq_parity(codes_to_np(qc), sc.cpu().numpy(), x_np, O.COLS, block, qt,
                    **(col_opts or {}))


DUAL_CASES = [
    # rows, cols, block, code type: all take the single read (multiples of 256, block <= 256)
    (4096, 4096, 256, O.I8),     # the 4096^2 gradient: 256 tiles, one per compute unit
    (1024, 2048, 128, O.E4M3),
    (512, 768, 64, O.E5M2),
    (256, 256, 16, O.I8),        # one tile
    (2048, 1024, 256, O.F64),    # the rotated values themselves (fp32)
    (768, 512, 1, O.I8),         # block 1: no rotation
]


@pytest.mark.parametrize("rows,cols,block,qt", DUAL_CASES)
def test_dual_matches_both_passes(rows, cols, block, qt):
    x_np = _grad(rows, cols, "bf16", seed=rows + 3 * cols + block)
    x = to_dev(x_np)
    assert H.fwht_quant_dual_workspace_bytes(rows, cols, block) > 0
    print(f"dual {rows}x{cols} block {block} qt {qt}", flush=True)
    qr, sr, qc, sc = H.fwht_quant_dual(x, block=block, q_dtype=Q_TORCH[qt])
    torch.cuda.synchronize()
    _check_both(x_np, block, qt, qr, sr, qc, sc)


def test_dual_with_signs_on_each_axis():
    rows, cols, block, qt = 1024, 1536, 256, O.I8
    x_np = _grad(rows, cols, "bf16", seed=77)
    sgn_r = synth.sign_words(cols, seed=5)   # along a row: the columns
    sgn_c = synth.sign_words(rows, seed=6)   # along a column: the rows
    qr, sr, qc, sc = H.fwht_quant_dual(to_dev(x_np), block=block, q_dtype=Q_TORCH[qt],
                                       row_signs=signs_dev(sgn_r), col_signs=signs_dev(sgn_c))
    torch.cuda.synchronize()
    _check_both(x_np, block, qt, qr, sr, qc, sc, dict(signs=sgn_r), dict(signs=sgn_c))


@pytest.mark.parametrize("rows,cols,block,io,rounding,ws", [
    (300, 512, 256, "bf16", "nearest", None),      # rows not a multiple of 256
    (512, 528, 8, "bf16", "nearest", None),        # cols not a multiple of 256
    (512, 512, 512, "bf16", "nearest", None),      # block above 256
    (256, 512, 128, "f32", "nearest", None),       # fp32 input
    (512, 512, 128, "bf16", "stochastic", None),   # stochastic rounding
    (512, 512, 128, "bf16", "nearest", False),     # no scratch
    (8192, 512, 256, "bf16", "nearest", None),     # columns of 8192: the exchanging columns pass
])
def test_dual_two_pass_shapes(rows, cols, block, io, rounding, ws):
    qt = O.E5M2 if rounding == "stochastic" else O.I8
    x_np = _grad(rows, cols, io, seed=rows * 5 + cols)
    print(f"dual (two passes) {rows}x{cols} block {block} {io} {rounding}", flush=True)
    qr, sr, qc, sc = H.fwht_quant_dual(to_dev(x_np), block=block, q_dtype=Q_TORCH[qt],
                                       workspace=ws, rounding=rounding, seed=SEED64,
                                       row_counter=CTR_R, col_counter=CTR_C)
    torch.cuda.synchronize()
    ro = co = None
    if rounding == "stochastic":
        ro = dict(rounding=O.STOCHASTIC, key=KEY, ctr_hi=CTR)
        co = dict(rounding=O.STOCHASTIC, key=KEY, ctr_hi=(CTR[0], CTR[1] ^ 0x80000000))
    _check_both(x_np, block, qt, qr, sr, qc, sc, ro, co)


def test_dual_exact_when_tasks_stop_waiting():
    # a limit of one poll: tasks that arrive before the rest of their tile row or column stop
    # waiting and leave their part to the repair launch; the codes must not change
    rows, cols, block, qt = 4096, 2048, 256, O.I8
    x_np = _grad(rows, cols, "bf16", seed=919)
    x = to_dev(x_np)
    r_q, r_s = O.fwht_quant(x_np, O.ROWS, block, qt, precision=32)
    c_q, c_s = O.fwht_quant(x_np, O.COLS, block, qt, precision=32)
    ws = torch.empty(H.fwht_quant_dual_workspace_bytes(rows, cols, block), dtype=torch.uint8,
                     device=DEV)
    late_total = 0
    for call in range(4):
        qr, sr, qc, sc = H.fwht_quant_dual(x, block=block, q_dtype=Q_TORCH[qt], workspace=ws,
                                           exchange_polls=1)
        torch.cuda.synchronize()
        late = int(ws[:4].view(torch.int32).item())
        late_total += late
        print(f"call {call}: {late} tasks stopped waiting", flush=True)
        assert np.array_equal(codes_to_np(qr), r_q) and np.array_equal(codes_to_np(qc), c_q)
        assert np.array_equal(sr.cpu().numpy().astype(np.float64), r_s)
        assert np.array_equal(sc.cpu().numpy().astype(np.float64), c_s)
    print(f"{late_total} tasks stopped waiting over 4 calls", flush=True)


def test_dual_guards():
    # outputs inside sentinel-filled buffers with padded leading dimensions; nothing outside
    # the outputs or past the scratch may change
    rows, cols, block, qt = 512, 768, 128, O.I8
    x_np = _grad(rows, cols, "bf16", seed=31)
    ref = H.fwht_quant_dual(to_dev(x_np), block=block, q_dtype=Q_TORCH[qt])
    S = 0x5A
    qr_buf = torch.full((rows + 4, cols + 32), S, dtype=torch.uint8, device=DEV)
    qc_buf = torch.full((cols + 4, rows + 32), S, dtype=torch.uint8, device=DEV)
    s_r = torch.full((rows + 8,), 0, dtype=torch.float32, device=DEV)
    s_c = torch.full((cols + 8,), 0, dtype=torch.float32, device=DEV)
    s_r.view(torch.uint8).fill_(S)
    s_c.view(torch.uint8).fill_(S)
    need = H.fwht_quant_dual_workspace_bytes(rows, cols, block)
    ws = torch.full((need + 4096,), S, dtype=torch.uint8, device=DEV)
    qr = qr_buf[2:2 + rows, :cols].view(torch.int8)
    qc = qc_buf[2:2 + cols, :rows].view(torch.int8)
    H.fwht_quant_dual(to_dev(x_np), block=block, q_dtype=Q_TORCH[qt], qr=qr, scale_r=s_r[4:4 + rows],
                      qc=qc, scale_c=s_c[4:4 + cols], workspace=ws[:need])
    torch.cuda.synchronize()
    assert torch.equal(qr, ref[0]) and torch.equal(qc, ref[2])
    assert torch.equal(s_r[4:4 + rows], ref[1]) and torch.equal(s_c[4:4 + cols], ref[3])
    for buf, r, c in ((qr_buf, rows, cols), (qc_buf, cols, rows)):
        assert (buf[:2] == S).all() and (buf[2 + r:] == S).all() and (buf[2:2 + r, c:] == S).all()
    for s_buf, n in ((s_r, rows), (s_c, cols)):
        b = s_buf.view(torch.uint8)
        assert (b[:16] == S).all() and (b[(4 + n) * 4:] == S).all()
    assert (ws[need:] == S).all(), "scratch written past its size"
