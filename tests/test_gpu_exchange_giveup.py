"""The bounded wait of the single-read columns pass over columns longer than 4096 rows.

The tasks of one column strip wait for each other to combine their partial maxima.  A task
that polls `exchange_polls` times (an option of the _ex calls; 2^20 by default) without seeing
the whole strip gives the strip up, and then every task of that strip does: its columns get a
NaN scale and codes that decode to zero, never codes from partial maxima.  A task gives up by
a compare-and-swap that only succeeds when no other task of its strip arrives during its round
trip, so a limit of 1 alone rarely gives anything up: the tasks of a strip arrive together.
The shapes here make one strip straddle the first wave of workgroups (one 1024-thread
workgroup per compute unit, 256 of them): columns of 49152 rows split into 48 tasks, so the
first tasks of the straddling strip arrive a whole task's time before the rest can start, and
with the limit at 1 they give it up.  Every column must then be either exactly the oracle's
(or, for the layer, the same call's with the default limit) or wholly given up, and the pass
is repeated, up to ATTEMPTS times, until some strip is.  With the default limit, and on the
same workspace right after, every column is the oracle's.
"""
import numpy as np
import pytest
import torch

import hadamard_rotated_precision_halo_amd as H
import oracle as O
import synth
from parity_util import Q_TORCH, codes_to_np, to_dev

pytestmark = pytest.mark.gpu

ATTEMPTS = 10


def _given_up_or_exact(got_q, got_s, ref_q, ref_s):
    lost = np.isnan(got_s)
    ok = ~lost
    assert np.array_equal(got_q[ok], ref_q[ok]), "codes of completed columns differ"
    assert np.array_equal(got_s[ok], ref_s[ok]), "scales of completed columns differ"
    return lost


@pytest.mark.parametrize("qt", [O.I8, O.E4M3])
def test_columns_pass_gives_up_whole_strips(qt):
    # 48 tasks per 64-column strip, 6 strips: tasks 240-287 (strip 5) straddle the first wave
    rows, cols, b = 49152, 384, 256
    rng = np.random.default_rng(808)
    x_np = synth.bf16_bits(synth.grads(rng, rows, cols))
    ref_q, ref_s = O.fwht_quant(x_np, O.COLS, b, qt, precision=32)
    x = to_dev(x_np)
    ws = torch.empty(H.fwht_quant_workspace_bytes(rows, cols, H.COLS, b), dtype=torch.uint8,
                     device=x.device)
    assert ws.numel() > 0
    for attempt in range(ATTEMPTS):
        q, s = H.fwht_quant(x, axis=H.COLS, block=b, q_dtype=Q_TORCH[qt], workspace=ws,
                            exchange_polls=1)
        torch.cuda.synchronize()
        got_q, got_s = codes_to_np(q), s.cpu().numpy().astype(np.float64)
        lost = _given_up_or_exact(got_q, got_s, ref_q, ref_s)
        # a strip is given up as a whole: 64 adjacent columns together
        assert np.array_equal(lost.reshape(-1, 64).all(axis=1), lost.reshape(-1, 64).any(axis=1))
        zero = q.view(torch.uint8).cpu().numpy()[lost] & 0x7F  # +0 or -0 codes
        assert not zero.any(), "given-up columns hold non-zero codes"
        if lost.any():
            break
    print(f"call {attempt}: {int(lost.sum())} of {cols} columns given up", flush=True)
    assert lost.any(), f"no strip was given up in {ATTEMPTS} calls with a limit of 1"

    q, s = H.fwht_quant(x, axis=H.COLS, block=b, q_dtype=Q_TORCH[qt], workspace=ws)
    torch.cuda.synchronize()
    assert np.array_equal(codes_to_np(q), ref_q)
    assert np.array_equal(s.cpu().numpy().astype(np.float64), ref_s)


def test_backward_gives_up_loudly():
    # dW = dY^T X contracts over m = 49152 rows: its dY and X column passes exchange maxima,
    # 48 tasks per strip.  The launch runs W's columns (2 tasks), dY's (4 strips, 192 tasks),
    # then X's (8 strips): X's second strip, tasks 242-289, straddles the first wave.
    m, n, k, b = 49152, 256, 512, 256
    x_np, w_np, dy_np = synth.layer(m, n, k, seed=909, with_grad=True)
    x, w, dy = to_dev(x_np), to_dev(w_np), to_dev(dy_np)
    dx_ref, dw_ref = H.linear_bwd(dy, x, w, b)
    torch.cuda.synchronize()
    dx_ref, dw_ref = dx_ref.float().cpu().numpy(), dw_ref.float().cpu().numpy()
    assert np.isfinite(dw_ref).all()
    for attempt in range(ATTEMPTS):
        dx, dw = H.linear_bwd(dy, x, w, b, exchange_polls=1)
        torch.cuda.synchronize()
        dx, dw = dx.float().cpu().numpy(), dw.float().cpu().numpy()
        assert np.array_equal(dx, dx_ref)  # W's columns (n = 256 rows) do not exchange
        bad = np.isnan(dw)
        # a given-up dY column empties a row of dW, a given-up X column a column of dW
        bad_rows, bad_cols = bad.all(axis=1), bad.all(axis=0)
        assert np.array_equal(bad, bad_rows[:, None] | bad_cols[None, :])
        assert np.array_equal(dw[~bad], dw_ref[~bad])
        if bad.any():
            break
    print(f"call {attempt}: {int(bad_rows.sum())} rows, {int(bad_cols.sum())} columns of dW "
          f"given up", flush=True)
    assert bad.any(), f"no strip was given up in {ATTEMPTS} calls with a limit of 1"


def test_two_exchanging_passes_on_two_streams():
    # The case the bound is for: two such passes overlapping on two streams, whose partly
    # dispatched strips can together fill the compute units.  With 4096 polls (far above the
    # few that a strip straddling a wave needs, far below the default) any such stall ends in
    # milliseconds; every call must still give either the oracle's columns or whole strips
    # given up.
    rows, cols, b = 49152, 384, 256
    rng = np.random.default_rng(1212)
    x_np = synth.bf16_bits(synth.grads(rng, rows, cols))
    ref_q, ref_s = O.fwht_quant(x_np, O.COLS, b, O.I8, precision=32)
    x = to_dev(x_np)
    nbytes = H.fwht_quant_workspace_bytes(rows, cols, H.COLS, b)
    ws = [torch.empty(nbytes, dtype=torch.uint8, device=x.device) for _ in range(2)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    lost_total = 0
    for _ in range(8):
        res = []
        for i, st in enumerate(streams):
            with torch.cuda.stream(st):
                res.append(H.fwht_quant(x, axis=H.COLS, block=b, workspace=ws[i], stream=st,
                                        exchange_polls=4096))
        torch.cuda.synchronize()
        for q, s in res:
            got_q, got_s = codes_to_np(q), s.cpu().numpy().astype(np.float64)
            lost = _given_up_or_exact(got_q, got_s, ref_q, ref_s)
            assert np.array_equal(lost.reshape(-1, 64).all(axis=1),
                                  lost.reshape(-1, 64).any(axis=1))
            assert not (q.view(torch.uint8).cpu().numpy()[lost] & 0x7F).any()
            lost_total += int(lost.sum())
    print(f"{lost_total} columns given up over 16 overlapping passes", flush=True)
