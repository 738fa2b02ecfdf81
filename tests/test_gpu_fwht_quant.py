"""GPU parity of halo_fwht_quant (rows and columns axes) against the CPU oracle.

Bars: codes and scales bit-identical to the oracle's fp32 decision (same butterfly order,
same fp32 quotient); rotated values (fp32 test mode) bit-identical to the oracle's fp32
butterflies and within 1e-5 relative L2 per vector of its fp64 transform; codes within the
+-1 / 0.01% budget of its fp64 decision and scales within 1e-5 of its fp64 scales.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import hadamard_rotated_precision_halo_amd as H
import oracle as O
import synth
from parity_util import (Q_TORCH, assert_codes_close_to_fp64, check_fq_parity, code_distance,
                         codes_to_np, scales_close_to_fp64, to_dev)

pytestmark = pytest.mark.gpu


def _input(rows, cols, io, seed, kind="act"):
    rng = np.random.default_rng(seed)
    if kind == "act":
        a = synth.activations(rng, rows, cols)
    elif kind == "grad":
        a = synth.grads(rng, rows, cols)
    else:
        a = synth.weights(rng, rows, cols)
    return synth.bf16_bits(a) if io == "bf16" else a


def _run(x_np, axis, block, qtype):
    x = to_dev(x_np)
    q, s = H.fwht_quant(x, axis=axis, block=block, q_dtype=Q_TORCH[qtype])
    torch.cuda.synchronize()
    return codes_to_np(q), s.cpu().numpy().astype(np.float64)


ROW_CASES = [
    # (io, block, rows, cols, qtype)
    ("bf16", 256, 37, 4096, O.I8),
    ("bf16", 128, 19, 11008, O.I8),        # 86 blocks: the last lane groups of a row idle
    ("f32", 1024, 9, 1024, O.I8),
    ("bf16", 512, 5, 14336, O.E5M2),
    ("bf16", 512, 33, 4096, O.E4M3),
    ("bf16", 1, 17, 64, O.I8),
    ("bf16", 2, 17, 64, O.I8),
    ("bf16", 4, 300, 16, O.I8),
    ("bf16", 8, 301, 16, O.E4M3),
    ("bf16", 16, 129, 48, O.I8),
    ("bf16", 32, 70, 96, O.E5M2),
    ("f32", 64, 65, 320, O.I8),
    ("bf16", 2048, 3, 4096, O.I8),
    ("bf16", 4096, 4, 8192, O.E4M3),
    ("bf16", 128, 2, 16384, O.I8),         # longest row the rows kernel takes at block 128
    ("bf16", 256, 1000, 256, O.I8),        # many short rows per workgroup
    ("bf16", 2048, 7, 2048, O.I8),         # two rows per wave, 32 lanes per block
    ("f32", 128, 13, 512, O.E4M3),         # eight rows per wave, a partial last wave
    ("bf16", 64, 50, 64, O.I8),            # one lane per row
    ("f32", 4096, 3, 12288, O.E5M2),       # three waves per row
    ("bf16", 256, 3, 28672, O.I8),         # seven waves per row (the dY rows of a wide layer)
    ("bf16", 4096, 2, 65536, O.E5M2),      # sixteen waves: the longest row
    ("f32", 512, 2, 20480, O.I8),          # fp32, five waves per row
    ("bf16", 128, 2, 16448, O.E4M3),       # padded to 16512: a partial last wave
    ("bf16", 4096, 64, 16, O.I8),          # 16 columns padded to one block of 4096
]


@pytest.mark.parametrize("io,block,rows,cols,qtype", ROW_CASES)
def test_rows_match_oracle(io, block, rows, cols, qtype):
    x = _input(rows, cols, io, seed=rows * 7 + cols)
    q, s = _run(x, H.ROWS, block, qtype)
    r32, s32 = O.fwht_quant(x, O.ROWS, block, qtype, precision=32)
    assert np.array_equal(q, r32), f"{int((q != r32).sum())} codes differ from the fp32 decision"
    assert np.array_equal(s, s32)
    r64, s64 = O.fwht_quant(x, O.ROWS, block, qtype, precision=64)
    assert_codes_close_to_fp64(q, r64, qtype, block, x=x, oaxis=O.ROWS)
    np.testing.assert_allclose(s, s64, rtol=1e-5)


COL_CASES = [
    ("bf16", 256, 4096, 64, O.I8),
    ("bf16", 128, 1024, 200, O.I8),       # 200 columns: a partial workgroup
    ("bf16", 512, 2048, 40, O.E5M2),
    ("bf16", 512, 1024, 56, O.E4M3),
    ("f32", 256, 512, 24, O.I8),
    ("bf16", 1, 64, 16, O.I8),
    ("bf16", 2, 64, 8, O.I8),
    ("bf16", 4, 48, 16, O.I8),
    ("bf16", 8, 64, 16, O.E4M3),
    ("bf16", 16, 96, 32, O.I8),
    ("bf16", 32, 64, 8, O.I8),
    ("bf16", 64, 192, 24, O.E5M2),
    ("bf16", 1024, 2048, 16, O.I8),
    ("bf16", 2048, 4096, 8, O.E4M3),
    ("bf16", 4096, 8192, 8, O.I8),
    ("bf16", 256, 4096, 520, O.I8),       # whole 4096-row columns, 16-column strips, partial last
    ("bf16", 128, 8192, 72, O.E4M3),      # 8 tasks per strip (1024-row parts)
    ("bf16", 512, 512, 136, O.E5M2),      # 512-row tiles of 128 columns
    ("bf16", 64, 256, 1032, O.I8),        # 256-row tiles, 5 strips
    ("bf16", 1024, 3072, 64, O.I8),       # 3 tasks per strip
    ("bf16", 256, 4096, 5120, O.I8),      # 320 tasks: more than one round of the persistent grid
    ("bf16", 256, 768, 64, O.I8),         # 256-row parts, 3 per strip
    ("bf16", 256, 2048, 96, O.E4M3),      # whole 2048-row columns, 32-column strips
    ("bf16", 128, 8192, 200, O.I8),       # 8 parts per strip, partial last strip
    # fp32 input: the same tiles through the LDS in two rounds (the rows whose offset bit
    # log2(max(block, 64)) - 1 is 0, then 1), every element read once
    ("f32", 256, 4096, 64, O.I8),         # whole 4096-row columns, 16-column strips
    ("f32", 256, 4096, 520, O.E4M3),      # partial last strip
    ("f32", 1, 64, 16, O.I8),             # 64-row tiles of 1024 columns
    ("f32", 8, 64, 16, O.E4M3),
    ("f32", 32, 128, 24, O.E5M2),
    ("f32", 64, 192, 24, O.E5M2),         # 64-row parts, 3 per strip
    ("f32", 1024, 2048, 16, O.I8),
    ("f32", 4096, 4096, 8, O.E4M3),       # one block per column
    ("f32", 4096, 8192, 8, O.I8),         # 2 parts per strip
    ("f32", 128, 8192, 72, O.E4M3),       # 8 parts per strip
    ("f32", 512, 512, 136, O.F64),        # the rotated values themselves
    ("f32", 256, 768, 64, O.I8),          # 256-row parts, 3 per strip
    # 16 rows padded to one block of 4096: 16 distinct rotated values per column, each 256
    # times, so one exact tie repeats across 256 codes
    ("bf16", 4096, 16, 128, O.I8),
]


@pytest.mark.parametrize("io,block,rows,cols,qtype", COL_CASES)
def test_cols_match_oracle(io, block, rows, cols, qtype):
    x = _input(rows, cols, io, seed=rows * 5 + cols, kind="grad")
    q, s = _run(x, H.COLS, block, qtype)
    assert q.shape == (cols, O.padded_len(rows, block))
    r32, s32 = O.fwht_quant(x, O.COLS, block, qtype, precision=32)
    assert np.array_equal(q, r32), f"{int((q != r32).sum())} codes differ from the fp32 decision"
    assert np.array_equal(s, s32)
    r64, s64 = O.fwht_quant(x, O.COLS, block, qtype, precision=64)
    assert_codes_close_to_fp64(q, r64, qtype, block, x=x, oaxis=O.COLS)
    np.testing.assert_allclose(s, s64, rtol=1e-5)


def test_cols_single_read_matches_two_read_path():
    # the same pass with and without scratch (one input read vs two), repeated on one scratch
    # buffer and on a second stream: identical codes and scales every time
    x = to_dev(_input(8192, 200, "bf16", seed=77, kind="grad"))
    ref_q, ref_s = H.fwht_quant(x, axis=H.COLS, block=256, workspace=False)
    ws = torch.empty(H.fwht_quant_workspace_bytes(8192, 200, H.COLS, 256), dtype=torch.uint8,
                     device="cuda")
    assert ws.numel() > 0
    for _ in range(3):
        q, s = H.fwht_quant(x, axis=H.COLS, block=256, workspace=ws)
        assert torch.equal(q, ref_q) and torch.equal(s, ref_s)
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        q, s = H.fwht_quant(x, axis=H.COLS, block=256, workspace=ws)
    st.synchronize()
    assert torch.equal(q, ref_q) and torch.equal(s, ref_s)


@pytest.mark.parametrize("axis,block,rows,cols", [(H.ROWS, 256, 24, 1024), (H.ROWS, 128, 6, 11008),
                                                  (H.COLS, 256, 1024, 64), (H.COLS, 512, 2048, 16),
                                                  (H.ROWS, 4096, 2, 4096), (H.COLS, 4096, 4096, 8)])
def test_rotated_values_fp32_mode(axis, block, rows, cols):
    x = _input(rows, cols, "bf16", seed=rows + cols)
    y, s = _run(x, axis, block, O.F64)
    oax = O.ROWS if axis == H.ROWS else O.COLS
    y32, s32 = O.fwht_quant(x, oax, block, O.F64, precision=32)
    assert np.array_equal(y.astype(np.float64), y32)       # bit-identical fp32 butterflies
    assert np.array_equal(s, s32)
    y64, _ = O.fwht_quant(x, oax, block, O.F64, precision=64)
    err = np.linalg.norm(y - y64, axis=1) / np.linalg.norm(y64, axis=1)
    assert err.max() <= 1e-5


def test_zero_vectors_and_constant_rows():
    x = _input(16, 512, "bf16", seed=3)
    x[3] = 0
    x[7] = synth.bf16_bits(np.full(512, 2.5, dtype=np.float32))
    for qt in (O.I8, O.E4M3, O.E5M2):
        q, s = _run(x, H.ROWS, 128, qt)
        check_fq_parity(q, s, x, O.ROWS, 128, qt)
        assert s[3] == 0 and not q[3].any()
    xc = _input(256, 16, "bf16", seed=4)
    xc[:, 5] = 0
    q, s = _run(xc, H.COLS, 64, O.I8)
    check_fq_parity(q, s, xc, O.COLS, 64, O.I8)
    assert s[5] == 0 and not q[5].any()


@pytest.mark.parametrize("axis,block,shape", [(H.ROWS, 1, (8, 4096)), (H.ROWS, 128, (8, 4096)),
                                               (H.ROWS, 32, (8, 96)), (H.COLS, 1, (256, 16)),
                                               (H.COLS, 64, (256, 16))])
def test_signed_zeros(axis, block, shape):
    # -0 inputs, -0 blocks and exact zeros inside rotated blocks: an exactly zero value takes
    # the +0 code whichever sign the arithmetic leaves on it, as in the oracle
    x = _input(*shape, "bf16", seed=9)
    x[:, ::3] = 0x8000                   # -0 in bf16
    x[1] = 0x8000
    x[2] = synth.bf16_bits(np.full(shape[1], -1.5, dtype=np.float32))
    if axis == H.COLS:
        x[:, 3] = 0x8000
    oax = O.ROWS if axis == H.ROWS else O.COLS
    for qt in (O.E4M3, O.E5M2, O.I8):
        q, s = _run(x, axis, block, qt)
        check_fq_parity(q, s, x, oax, block, qt)


def test_empty_inputs():
    x = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    q, s = H.fwht_quant(x, axis=H.ROWS, block=256)
    assert q.shape == (0, 256) and s.shape == (0,)
    x = torch.empty((256, 0), dtype=torch.bfloat16, device="cuda")
    q, s = H.fwht_quant(x, axis=H.COLS, block=256)
    assert q.shape == (0, 256)


def test_leading_dimensions_and_repeatability():
    # a strided view (ld > cols) for the input, and bit-identical repeated runs
    base = to_dev(_input(64, 1536, "bf16", seed=9))
    view = base[:, :1024]
    q1, s1 = H.fwht_quant(view, axis=H.ROWS, block=256)
    q2, s2 = H.fwht_quant(view.contiguous(), axis=H.ROWS, block=256)
    assert torch.equal(q1, q2) and torch.equal(s1, s2)
    c1, t1 = H.fwht_quant(view, axis=H.COLS, block=64)
    c2, t2 = H.fwht_quant(view.contiguous(), axis=H.COLS, block=64)
    assert torch.equal(c1, c2) and torch.equal(t1, t2)
    for _ in range(3):
        q3, s3 = H.fwht_quant(view, axis=H.ROWS, block=256)
        assert torch.equal(q1, q3) and torch.equal(s1, s3)


def test_invalid_call_leaves_outputs_untouched():
    # a block the library refuses (above 4096), outputs shaped as the call would need them:
    # the library's own validation rejects it before any launch
    x = to_dev(_input(8, 256, "bf16", seed=1))
    q = torch.full((8, 8192), 7, dtype=torch.int8, device="cuda")
    s = torch.full((8,), 3.0, device="cuda")
    with pytest.raises(H.HaloError):
        H.fwht_quant(x, axis=H.ROWS, block=8192, q=q, scale=s)
    torch.cuda.synchronize()
    assert (q == 7).all() and (s == 3.0).all()


# ---------------------------------------------------------------------------
# vectors of tiny values and gradual underflow
# ---------------------------------------------------------------------------

def _tiny_mix(nvec, L, io, seed):
    """[nvec x L] vectors of three kinds, cycling: tiny vectors (every element subnormal, so
    fp32 qmax / absmax overflows and the decision runs on the vector scaled by 2^64), vectors
    with subnormal elements among normal ones (the butterflies must keep gradual underflow),
    and ordinary vectors.  Returns the input (bf16 bits or fp32) and the same input times
    2^64 (exact)."""
    rng = np.random.default_rng(seed)
    g = rng.standard_normal((nvec, L))
    if io == "bf16":
        tiny = np.rint(np.clip(g, -3, 3)) * 2.0 ** -133       # bf16 subnormals
    else:
        tiny = np.rint(g * 2.0 ** 15) * 2.0 ** -149            # fp32 subnormals
    mixed = g * np.where(rng.random((nvec, L)) < 0.5, 2.0 ** -130, 1.0)
    kind = (np.arange(nvec) % 3)[:, None]
    x = np.where(kind == 0, tiny, np.where(kind == 1, mixed, g)).astype(np.float32)
    if io == "bf16":
        x = synth.bf16_bits(x)
        xf = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        big = synth.bf16_bits((xf * 2.0 ** 64).astype(np.float32))
        assert np.array_equal((big.astype(np.uint32) << 16).view(np.float32), xf * 2.0 ** 64)
    else:
        big = (x.astype(np.float64) * 2.0 ** 64).astype(np.float32)
        assert np.array_equal(big.astype(np.float64), x.astype(np.float64) * 2.0 ** 64)
    return x, big


def _exact_midpoint(y, a, qmax):
    """Whether y * qmax / a (exact rational arithmetic on the fp64 values) is an integer plus
    one half."""
    t = Fraction(float(y)) * qmax / Fraction(float(a))
    return t.denominator == 2


TINY_CASES = [
    # (axis, io, L): L = vector length; bf16 takes the wave kernels, fp32 the older ones
    (H.ROWS, "bf16", 512), (H.ROWS, "bf16", 4096), (H.ROWS, "f32", 512),
    (H.COLS, "bf16", 256), (H.COLS, "bf16", 4096), (H.COLS, "f32", 512),
]


@pytest.mark.parametrize("qtype", [O.I8, O.E4M3, O.E5M2])
@pytest.mark.parametrize("axis,io,L", TINY_CASES)
def test_tiny_and_subnormal_vectors(axis, io, L, qtype):
    nvec = 24
    x, big = _tiny_mix(nvec, L, io, seed=L + qtype)
    if axis == H.COLS:  # the vectors are the matrix's columns
        x, big = np.ascontiguousarray(x.T), np.ascontiguousarray(big.T)
    oax = O.ROWS if axis == H.ROWS else O.COLS
    q, s = _run(x, axis, 256, qtype)
    r32, s32 = O.fwht_quant(x, oax, 256, qtype, precision=32)
    assert np.array_equal(q, r32), f"{int((q != r32).sum())} codes differ from the fp32 decision"
    assert np.array_equal(s, s32)
    # the fp64 definition: the tiny vectors are small integers times 2^-133 (or 2^-149), so
    # their rotated values are exact integers and y * qmax / a lands exactly on a rounding
    # midpoint far more often than on rotated real data; at an exact midpoint both neighbours
    # are equally near, and the fp32 quotient (rounded) and the fp64 one (exact) may pick
    # either.  Flips at exact midpoints are therefore allowed; every other flip counts against
    # the 1e-4 bar.
    r64, s64 = O.fwht_quant(x, oax, 256, qtype, precision=64)
    d = code_distance(q, r64, qtype)
    assert d.max() <= 1, f"code off by {d.max()}"
    flips = np.argwhere(d == 1)
    if qtype == O.I8 and len(flips):
        y64, a64 = O.fwht_quant(x, oax, 256, O.F64, precision=64)
        flips = [(i, j) for i, j in flips if not _exact_midpoint(y64[i, j], a64[i], 127)]
    assert len(flips) <= max(2, 1e-4 * d.size), f"{len(flips)} of {d.size} codes off by one"
    scales_close_to_fp64(s, s64)
    # scale invariance on the GPU itself: the tiny vectors' codes are the scaled vectors' codes
    qb, _ = _run(big, axis, 256, qtype)
    tiny_rows = np.arange(nvec) % 3 == 0
    assert np.array_equal(q[tiny_rows], qb[tiny_rows])
    assert (q[tiny_rows] != 0).any()


@pytest.mark.parametrize("axis", [H.ROWS, H.COLS])
def test_tiny_vectors_stochastic(axis):
    x, _ = _tiny_mix(24, 4096, "bf16", seed=5)
    if axis == H.COLS:
        x = np.ascontiguousarray(x.T)
    q, s = H.fwht_quant(to_dev(x), axis=axis, block=256, q_dtype=Q_TORCH[O.E5M2],
                        rounding="stochastic", seed=(9 << 32) | 4, counter=(3 << 32) | 8)
    torch.cuda.synchronize()
    check_fq_parity(codes_to_np(q), s.cpu().numpy(), x, O.ROWS if axis == H.ROWS else O.COLS,
                    256, O.E5M2, rounding=O.STOCHASTIC, key=(4, 9), ctr_hi=(8, 3))


@pytest.mark.parametrize("rows,cols,block", [(263168, 16, 256), (525312, 8, 8)])
def test_very_long_columns(rows, cols, block):
    # Columns too long for all 1024-row parts of a strip to be resident at once (257 and 513
    # parts, on 256 compute units) take the two-sweep kernel even with a workspace; the
    # second shape also needs more than 65535 blocks of 8 rows, which that kernel
    # grid-strides over.
    x_np = _input(rows, cols, "bf16", seed=rows % 1000, kind="grad")
    print(f"columns {rows} x {cols}, block {block}", flush=True)
    assert H.fwht_quant_workspace_bytes(rows, cols, H.COLS, block) > 0
    q, s = _run(x_np, H.COLS, block, O.I8)
    check_fq_parity(q, s, x_np, O.COLS, block, O.I8)
