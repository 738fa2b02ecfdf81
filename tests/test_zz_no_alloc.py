"""halo_fwht_quant_noalloc, the columns pass with the library's fixed scratch in place of a
caller workspace (for callers that cannot allocate), against halo_fwht_quant_ex with a
workspace: identical codes and scales, on two calls in a row (the second smaller, on the same
fixed scratch), both through the C ABI; plus the refusal of a pass that needs more scratch than
the fixed array holds, before anything is launched."""
import ctypes

import numpy as np
import pytest
import torch

import hadamard_rotated_precision_halo_amd as H
import oracle as O
import synth
from parity_util import DEV, check_fq_parity, codes_to_np, to_dev

pytestmark = pytest.mark.gpu


def _call(x, axis, block, q, s, workspace):
    L = H.lib()
    rows, cols = x.shape
    args = (H._ptr(x), H._code(x.dtype), rows, cols, H._ld(x), axis, block, H._code(q.dtype),
            H._ptr(q), H._ld(q), H._ptr(s), None)
    if workspace is None:
        return L.halo_fwht_quant_noalloc(*args, H._stream(None))
    return L.halo_fwht_quant_ex(*args, H._ptr(workspace), workspace.numel(), H._stream(None))


@pytest.mark.parametrize("qt", [torch.int8, torch.float8_e5m2])
def test_noalloc_matches_workspace_call(qt):
    shapes = [(12288, 520, 256), (8192, 136, 128)]  # the second call is smaller
    for i, (rows, cols, block) in enumerate(shapes):
        rng = np.random.default_rng(rows + cols)
        x_np = synth.bf16_bits(synth.grads(rng, rows, cols))
        x = to_dev(x_np)
        need = H.fwht_quant_workspace_bytes(rows, cols, H.COLS, block)
        assert 0 < need <= H.NOALLOC_SCRATCH_BYTES
        ws = torch.empty(need, dtype=torch.uint8, device=DEV)
        lp = H.padded_len(rows, block)
        q0 = torch.empty((cols, lp), dtype=qt, device=DEV)
        s0 = torch.empty(cols, dtype=torch.float32, device=DEV)
        q1, s1 = torch.empty_like(q0), torch.empty_like(s0)
        print(f"call {i}: columns {rows} x {cols}, block {block}, {qt}", flush=True)
        assert _call(x, H.COLS, block, q0, s0, ws) == 0
        assert _call(x, H.COLS, block, q1, s1, None) == 0
        torch.cuda.synchronize()
        assert torch.equal(q1.view(torch.uint8), q0.view(torch.uint8))
        assert torch.equal(s1, s0)
        oq = {torch.int8: O.I8, torch.float8_e5m2: O.E5M2}[qt]
        check_fq_parity(codes_to_np(q1), s1.cpu().numpy(), x_np, O.COLS, block, oq)


def test_noalloc_refuses_beyond_its_scratch():
    # columns of 8192 rows need 256 + strips * 4 (padded) + 4 per column of scratch; 300000
    # columns need more than the fixed 1 MiB: refused before any launch, outputs untouched
    rows, cols, block = 8192, 300000, 256
    assert H.fwht_quant_workspace_bytes(rows, cols, H.COLS, block) > H.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((8, 8), dtype=torch.bfloat16, device=DEV)  # never read
    L = H.lib()
    q = torch.full((64,), 7, dtype=torch.int8, device=DEV)
    s = torch.full((64,), 3.0, dtype=torch.float32, device=DEV)
    st = L.halo_fwht_quant_noalloc(H._ptr(x), H._code(x.dtype), rows, cols, cols, H.COLS, block,
                                   H._code(torch.int8), H._ptr(q), rows, H._ptr(s), None,
                                   H._stream(None))
    torch.cuda.synchronize()
    assert st == 6  # HALO_ERR_WORKSPACE
    assert (q == 7).all() and (s == 3.0).all()
