"""Race and bounds checks on the GPU: guard bands around every output, and bit-identical results
from two launch geometries of the same computation.

Guard bands: each output is a view into a larger buffer filled with a sentinel pattern (rows
before and after, columns past the row length where the leading dimension allows it, words
before and after the scale vectors, bytes past the end of the workspace); after the call every
sentinel byte must be unchanged and the view must hold the same values as a call on a dense
output.

Two geometries: the same values computed by launches whose grids, workgroup-to-tile and
task-to-XCD mappings differ (a product split into row or column slabs, a rotation pass over
slices of the vectors, the layer backward's batched launches against the standalone passes and
products) must agree bit for bit: each result element depends only on its own inputs.
"""
import numpy as np
import pytest
import torch

import hadamard_rotated_precision_halo_amd as H
import synth
from parity_util import DEV, padded_out, to_dev

pytestmark = pytest.mark.gpu

SENT = 0x5A


def _guarded(shape, dtype, pad_rows=2, pad_cols=0):
    """A view of `shape` inside a sentinel-filled buffer with pad_rows guard rows on each side
    and pad_cols guard columns at the end of each row; returns (buffer, view)."""
    rows, cols = shape
    buf = torch.empty((rows + 2 * pad_rows, cols + pad_cols), dtype=dtype, device=DEV)
    buf.view(torch.uint8).fill_(SENT)
    return buf, buf[pad_rows:pad_rows + rows, :cols]


def _guard_ok(buf, pad_rows, rows, cols):
    b = buf.view(torch.uint8).view(buf.shape[0], -1)
    es = buf.element_size()
    ok = (b[:pad_rows] == SENT).all() and (b[pad_rows + rows:] == SENT).all()
    ok = ok and (b[pad_rows:pad_rows + rows, cols * es:] == SENT).all()
    return bool(ok)


def _vec_guarded(n, dtype=torch.float32, pad=4):
    buf = torch.empty(n + 2 * pad, dtype=dtype, device=DEV)
    buf.view(torch.uint8).fill_(SENT)
    return buf, buf[pad:pad + n]


def _vec_guard_ok(buf, n, pad=4):
    b = buf.view(torch.uint8)
    es = buf.element_size()
    return bool((b[:pad * es] == SENT).all() and (b[(pad + n) * es:] == SENT).all())


def _bf16(rows, cols, seed, kind="act"):
    rng = np.random.default_rng(seed)
    a = {"act": synth.activations, "grad": synth.grads, "w": synth.weights}[kind](rng, rows, cols)
    return to_dev(synth.bf16_bits(a))


@pytest.mark.parametrize("axis,rows,cols,block,io", [(H.ROWS, 96, 4096, 256, "bf16"),
                                                     (H.ROWS, 40, 11008, 128, "bf16"),
                                                     (H.COLS, 4096, 200, 256, "bf16"),
                                                     (H.COLS, 8192, 136, 128, "bf16"),
                                                     (H.COLS, 4096, 200, 256, "f32"),
                                                     (H.COLS, 8192, 136, 128, "f32")])
def test_rotation_pass_guards(axis, rows, cols, block, io):
    if io == "bf16":
        x = _bf16(rows, cols, seed=rows + cols, kind="grad")
    else:
        x = to_dev(synth.grads(np.random.default_rng(rows + cols), rows, cols).astype(np.float32))
    nvec, L = (rows, cols) if axis == H.ROWS else (cols, rows)
    lp = H.padded_len(L, block)
    ref_q, ref_s = H.fwht_quant(x, axis=axis, block=block)
    need = H.fwht_quant_workspace_bytes(rows, cols, axis, block)
    ws_buf = torch.full((need + 4096,), SENT, dtype=torch.uint8, device=DEV)
    qbuf, q = _guarded((nvec, lp), torch.int8, pad_rows=3, pad_cols=32)
    sbuf, s = _vec_guarded(nvec)
    H.fwht_quant(x, axis=axis, block=block, q=q, scale=s,
                 workspace=ws_buf[:need] if need else False)
    torch.cuda.synchronize()
    assert _guard_ok(qbuf, 3, nvec, lp), "codes written outside their rows"
    assert _vec_guard_ok(sbuf, nvec), "scales written outside their vector"
    assert (ws_buf[need:] == SENT).all(), "scratch written past its size"
    assert torch.equal(q, ref_q) and torch.equal(s, ref_s)


@pytest.mark.parametrize("m,n,k,out", [(300, 520, 1024, torch.bfloat16),
                                       (4096, 4096, 4096, torch.int32),
                                       (513, 257, 4096, torch.float32)])
def test_gemm_guards(m, n, k, out):
    rng = np.random.default_rng(m + n)
    a = torch.from_numpy(rng.integers(-127, 128, (m, k), dtype=np.int8)).to(DEV)
    b = torch.from_numpy(rng.integers(-127, 128, (n, k), dtype=np.int8)).to(DEV)
    sa = torch.rand(m, device=DEV) * 1e-2
    sb = torch.rand(n, device=DEV) * 1e-2
    ref = H.gemm_i8(a, sa, b, sb, c=padded_out(m, n, out))
    es = torch.tensor([], dtype=out).element_size()
    ld_pad = 64 // es                       # guard columns: keeps rows 16-byte aligned
    cbuf, c = _guarded((m, n), out, pad_rows=2, pad_cols=ld_pad + (-n) % (16 // es))
    H.gemm_i8(a, sa, b, sb, c=c)
    torch.cuda.synchronize()
    assert _guard_ok(cbuf, 2, m, n), "product written outside its rows"
    assert torch.equal(c, ref)


def test_layer_guards():
    m, n, k, block = 320, 512, 1024, 256
    x, w, dy = _bf16(m, k, 1), _bf16(n, k, 2, "w"), _bf16(m, n, 3, "grad")
    ref_y = H.linear_fwd(x, w, block)
    ref_dx, ref_dw = H.linear_bwd(dy, x, w, block)
    ybuf, y = _guarded((m, n), torch.bfloat16)
    dxbuf, dx = _guarded((m, k), torch.bfloat16)
    dwbuf, dw = _guarded((n, k), torch.bfloat16)
    nf = H.linear_workspace_bytes(m, n, k, torch.int8, False)
    nb = H.linear_workspace_bytes(m, n, k, torch.int8, True)
    wsf = torch.full((nf + 4096,), SENT, dtype=torch.uint8, device=DEV)
    wsb = torch.full((nb + 4096,), SENT, dtype=torch.uint8, device=DEV)
    H.linear_fwd(x, w, block, y=y, workspace=wsf[:nf])
    H.linear_bwd(dy, x, w, block, dx=dx, dw=dw, workspace=wsb[:nb])
    torch.cuda.synchronize()
    for buf, rows, cols in ((ybuf, m, n), (dxbuf, m, k), (dwbuf, n, k)):
        assert _guard_ok(buf, 2, rows, cols), "layer output written outside its rows"
    assert (wsf[nf:] == SENT).all() and (wsb[nb:] == SENT).all(), "workspace overrun"
    assert torch.equal(y, ref_y) and torch.equal(dx, ref_dx) and torch.equal(dw, ref_dw)


def test_gemm_two_geometries():
    # 4096^3 int32 accumulators: one launch over the whole output, against row slabs and
    # column slabs launched separately (other tile counts, so other tile-to-XCD mappings)
    rng = np.random.default_rng(41)
    m = n = k = 4096
    a = torch.from_numpy(rng.integers(-127, 128, (m, k), dtype=np.int8)).to(DEV)
    b = torch.from_numpy(rng.integers(-127, 128, (n, k), dtype=np.int8)).to(DEV)
    full = H.gemm_i8(a, None, b, None, out_dtype=torch.int32)
    rows = torch.cat([H.gemm_i8(a[:2304], None, b, None, out_dtype=torch.int32),
                      H.gemm_i8(a[2304:], None, b, None, out_dtype=torch.int32)])
    cols = torch.cat([H.gemm_i8(a, None, b[:1536], None, out_dtype=torch.int32),
                      H.gemm_i8(a, None, b[1536:], None, out_dtype=torch.int32)], dim=1)
    torch.cuda.synchronize()
    assert torch.equal(full, rows) and torch.equal(full, cols)


def test_rotation_two_geometries():
    # rows pass over all rows against slices of them; columns pass over all columns against
    # slices that start inside a strip (other strip-to-XCD orders)
    x = _bf16(4096, 4096, seed=43, kind="grad")
    q, s = H.fwht_quant(x, axis=H.ROWS, block=256)
    q1, s1 = H.fwht_quant(x[:1000], axis=H.ROWS, block=256)
    q2, s2 = H.fwht_quant(x[1000:], axis=H.ROWS, block=256)
    torch.cuda.synchronize()
    assert torch.equal(q, torch.cat([q1, q2])) and torch.equal(s, torch.cat([s1, s2]))
    c, t = H.fwht_quant(x, axis=H.COLS, block=256)
    c1, t1 = H.fwht_quant(x[:, :200].contiguous(), axis=H.COLS, block=256)
    c2, t2 = H.fwht_quant(x[:, 200:].contiguous(), axis=H.COLS, block=256)
    torch.cuda.synchronize()
    assert torch.equal(c, torch.cat([c1, c2])) and torch.equal(t, torch.cat([t1, t2]))


@pytest.mark.parametrize("m", [4096, 8192])
def test_backward_batched_against_standalone(m):
    # the backward's batched rotation launch and paired products against the standalone
    # passes and products on the same inputs: bit-identical dX and dW (m = 8192: the columns
    # along m exchange partial maxima)
    n, k, block = 1024, 768, 256
    x, w, dy = _bf16(m, k, 5), _bf16(n, k, 6, "w"), _bf16(m, n, 7, "grad")
    dx, dw = H.linear_bwd(dy, x, w, block)
    qdy, sdy = H.fwht_quant(dy, axis=H.ROWS, block=block)
    qwt, swt = H.fwht_quant(w, axis=H.COLS, block=block)
    qdyt, sdyt = H.fwht_quant(dy, axis=H.COLS, block=block)
    qxt, sxt = H.fwht_quant(x, axis=H.COLS, block=block)
    dx2 = H.gemm_i8(qdy, sdy, qwt, swt, out_dtype=torch.bfloat16)
    dw2 = H.gemm_i8(qdyt, sdyt, qxt, sxt, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(dx, dx2) and torch.equal(dw, dw2)
