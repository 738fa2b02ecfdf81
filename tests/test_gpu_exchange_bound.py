"""The bounded wait of the single-read columns pass over columns longer than 4096 rows.

The tasks of one column strip wait for each other to combine their partial maxima.  A task
that polls `exchange_polls` times (an option of the _ex calls; 2^20 by default) without seeing
the whole strip stops waiting: it marks the strip late and leaves its part unstored, and so
does every task of the strip that finds the mark.  A repair launch that follows on the same
stream stores every part of a marked strip from the maxima, which are complete by then.  So a
call's codes never depend on the bound: they are the oracle's whether the wait completes or
not.  The first word of the columns pass's scratch counts the tasks that stopped waiting.

The shapes make one strip straddle the first wave of workgroups (one 1024-thread workgroup
per compute unit, 256 of them): columns of 49152 rows split into 48 tasks, so the first tasks
of the straddling strip arrive a whole task's time before the rest can start, and with the
limit at 1 they stop waiting.  The pass is repeated, up to ATTEMPTS times, until some task
has; every call must give the oracle's codes and scales exactly.
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


def _late_tasks(ws):
    """Tasks of the last columns pass on this scratch that stopped waiting (the scratch's
    first 32-bit word)."""
    return int(ws[:4].view(torch.int32).item())


@pytest.mark.parametrize("qt,io", [(O.I8, "bf16"), (O.E4M3, "bf16"), (O.I8, "f32")])
def test_columns_pass_exact_when_tasks_stop_waiting(qt, io):
    # 48 tasks per 64-column strip, 6 strips: tasks 240-287 (strip 5) straddle the first wave
    rows, cols, b = 49152, 384, 256
    rng = np.random.default_rng(808)
    g = synth.grads(rng, rows, cols)
    x_np = synth.bf16_bits(g) if io == "bf16" else g.astype(np.float32)
    ref_q, ref_s = O.fwht_quant(x_np, O.COLS, b, qt, precision=32)
    x = to_dev(x_np)
    ws = torch.empty(H.fwht_quant_workspace_bytes(rows, cols, H.COLS, b), dtype=torch.uint8,
                     device=x.device)
    assert ws.numel() > 0
    late = 0
    for attempt in range(ATTEMPTS):
        q, s = H.fwht_quant(x, axis=H.COLS, block=b, q_dtype=Q_TORCH[qt], workspace=ws,
                            exchange_polls=1)
        torch.cuda.synchronize()
        assert np.array_equal(codes_to_np(q), ref_q), f"call {attempt}: codes differ"
        assert np.array_equal(s.cpu().numpy().astype(np.float64), ref_s), \
            f"call {attempt}: scales differ"
        late = _late_tasks(ws)
        if late:
            break
    print(f"call {attempt}: {late} tasks stopped waiting", flush=True)
    assert late > 0, f"no task stopped waiting in {ATTEMPTS} calls with a limit of 1"

    # the default bound on the same scratch right after: complete exchanges, same result
    q, s = H.fwht_quant(x, axis=H.COLS, block=b, q_dtype=Q_TORCH[qt], workspace=ws)
    torch.cuda.synchronize()
    assert _late_tasks(ws) == 0
    assert np.array_equal(codes_to_np(q), ref_q)
    assert np.array_equal(s.cpu().numpy().astype(np.float64), ref_s)


def test_backward_exact_with_a_limit_of_one():
    # dW = dY^T X contracts over m = 49152 rows: its dY and X column passes exchange maxima,
    # 48 tasks per strip.  The launch runs W's columns (2 tasks), dY's (4 strips, 192 tasks),
    # then X's (8 strips): X's second strip, tasks 242-289, straddles the first wave.  Every
    # call with a limit of 1 poll gives the default call's dX and dW bit for bit.
    m, n, k, b = 49152, 256, 512, 256
    x_np, w_np, dy_np = synth.layer(m, n, k, seed=909, with_grad=True)
    x, w, dy = to_dev(x_np), to_dev(w_np), to_dev(dy_np)
    dx_ref, dw_ref = H.linear_bwd(dy, x, w, b)
    torch.cuda.synchronize()
    dx_ref, dw_ref = dx_ref.float().cpu().numpy(), dw_ref.float().cpu().numpy()
    assert np.isfinite(dw_ref).all()
    for attempt in range(4):
        dx, dw = H.linear_bwd(dy, x, w, b, exchange_polls=1)
        torch.cuda.synchronize()
        assert np.array_equal(dx.float().cpu().numpy(), dx_ref), f"call {attempt}: dX differs"
        assert np.array_equal(dw.float().cpu().numpy(), dw_ref), f"call {attempt}: dW differs"


def test_two_exchanging_passes_on_two_streams():
    # The case the bound is for: two such passes overlapping on two streams, whose partly
    # dispatched strips can together fill the compute units.  With 4096 polls (far above the
    # few that a strip straddling a wave needs, far below the default) any such stall ends in
    # milliseconds; every call must give the oracle's codes and scales.
    rows, cols, b = 49152, 384, 256
    rng = np.random.default_rng(1212)
    x_np = synth.bf16_bits(synth.grads(rng, rows, cols))
    ref_q, ref_s = O.fwht_quant(x_np, O.COLS, b, O.I8, precision=32)
    x = to_dev(x_np)
    nbytes = H.fwht_quant_workspace_bytes(rows, cols, H.COLS, b)
    ws = [torch.empty(nbytes, dtype=torch.uint8, device=x.device) for _ in range(2)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    late = 0
    for _ in range(8):
        res = []
        for i, st in enumerate(streams):
            with torch.cuda.stream(st):
                res.append(H.fwht_quant(x, axis=H.COLS, block=b, workspace=ws[i], stream=st,
                                        exchange_polls=4096))
        torch.cuda.synchronize()
        for i, (q, s) in enumerate(res):
            assert np.array_equal(codes_to_np(q), ref_q)
            assert np.array_equal(s.cpu().numpy().astype(np.float64), ref_s)
            late += _late_tasks(ws[i])
    print(f"{late} tasks stopped waiting over 16 overlapping passes", flush=True)
