"""The binding's own argument checks (CPU, no launch): the C ABI takes plain pointers and sizes,
so it cannot see how large a caller's tensor is; the binding checks every tensor argument's
shape, strides, dtype and device against what the call will read and write, and raises
ValueError before the library is called."""
import pytest
import torch

import hadamard_rotated_precision_halo_amd as H


def _bf16(r, c):
    return torch.zeros((r, c), dtype=torch.bfloat16)


@pytest.mark.parametrize("axis,q_shape", [(H.ROWS, (8, 128)), (H.ROWS, (7, 256)),
                                          (H.COLS, (256, 8)), (H.COLS, (255, 256))])
def test_rotation_output_shape(axis, q_shape):
    # rows: q is [8 x 256]; columns: [256 x Lp], Lp = 8 padded to the block of 256
    x = _bf16(8, 256)
    with pytest.raises(ValueError, match="q has shape"):
        H.fwht_quant(x, axis=axis, block=256, q=torch.zeros(q_shape, dtype=torch.int8))


def test_rotation_scale_and_signs():
    x = _bf16(8, 300)  # rows padded to 512 positions: 16 sign words
    q = torch.zeros((8, 512), dtype=torch.int8)
    with pytest.raises(ValueError, match="scale"):
        H.fwht_quant(x, block=256, q=q, scale=torch.zeros(7))
    with pytest.raises(ValueError, match="scale"):
        H.fwht_quant(x, block=256, q=q, scale=torch.zeros(8, dtype=torch.float64))
    with pytest.raises(ValueError, match="signs"):
        H.fwht_quant(x, block=256, q=q, scale=torch.zeros(8),
                     signs=torch.zeros(10, dtype=torch.int32))  # covers 300, not 512
    with pytest.raises(ValueError, match="GPU"):  # shapes right, but host tensors
        H.fwht_quant(x, block=256, q=q, scale=torch.zeros(8),
                     signs=torch.zeros(16, dtype=torch.int32))


def test_rotation_output_strides():
    x = _bf16(8, 256)
    q = torch.zeros((256, 8), dtype=torch.int8).t()  # right shape, column-major
    with pytest.raises(ValueError, match="row-major"):
        H.fwht_quant(x, block=256, q=q)


def test_dual_outputs():
    x = _bf16(256, 512)
    with pytest.raises(ValueError, match="qc has shape"):
        H.fwht_quant_dual(x, block=256, qc=torch.zeros((512, 512), dtype=torch.int8))
    with pytest.raises(ValueError, match="qr has dtype"):
        H.fwht_quant_dual(x, block=256, qr=torch.zeros((256, 512), dtype=torch.float8_e4m3fn))


def test_noalloc_outputs():
    x = _bf16(4096, 64)
    with pytest.raises(ValueError, match="q has shape"):
        H.fwht_quant_noalloc(x, torch.zeros((64, 2048), dtype=torch.int8), torch.zeros(64),
                             axis=H.COLS)


def test_products():
    a = torch.zeros((64, 128), dtype=torch.int8)
    b = torch.zeros((32, 128), dtype=torch.int8)
    sa, sb = torch.zeros(64), torch.zeros(32)
    with pytest.raises(ValueError, match="b has shape"):
        H.gemm_i8(a, sa, torch.zeros((32, 96), dtype=torch.int8), sb)
    with pytest.raises(ValueError, match="c has shape"):
        H.gemm_i8(a, sa, b, sb, c=torch.zeros((64, 31), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="sb"):
        H.gemm_i8(a, sa, b, torch.zeros(31))
    with pytest.raises(ValueError, match="sa"):
        H.gemm_fp8(a.view(torch.float8_e4m3fn), torch.zeros(63), b.view(torch.float8_e4m3fn), sb)
    with pytest.raises(ValueError, match="GPU"):  # raw int32 output: no scales needed
        H.gemm_i8(a, None, b, None, c=torch.zeros((64, 32), dtype=torch.int32))


def test_layer_operands():
    m, n, k = 64, 32, 256
    x, w, dy = _bf16(m, k), _bf16(n, k), _bf16(m, n)
    with pytest.raises(ValueError, match="x must be contiguous"):
        H.linear_fwd(_bf16(k, m).t(), w, 256)
    with pytest.raises(ValueError, match="w has shape"):
        H.linear_fwd(x, _bf16(n, k + 32), 256)
    with pytest.raises(ValueError, match="w has dtype"):
        H.linear_fwd(x, w.float(), 256)
    with pytest.raises(ValueError, match="y has shape"):
        H.linear_fwd(x, w, 256, y=_bf16(m, n + 1))
    with pytest.raises(ValueError, match="signs_k"):  # k = 256 needs 8 words
        H.linear_fwd(x, w, 256, signs_k=torch.zeros(7, dtype=torch.int32))
    with pytest.raises(ValueError, match="dy has shape"):
        H.linear_bwd(_bf16(m, n + 1), x, w, 256)
    with pytest.raises(ValueError, match="dw has shape"):
        H.linear_bwd(dy, x, w, 256, dw=_bf16(n + 1, k))
    with pytest.raises(ValueError, match="signs_m"):  # m = 64 padded to 256: 8 words
        H.linear_bwd(dy, x, w, 256, signs_m=torch.zeros(2, dtype=torch.int32))
    with pytest.raises(ValueError, match="workspace"):
        H.linear_bwd(dy, x, w, 256, workspace=torch.zeros(16, dtype=torch.float32))
    with pytest.raises(ValueError, match="GPU"):
        H.linear_bwd(dy, x, w, 256)


def test_contraction_len():
    # the layer pads each contraction dimension to a multiple of the block and of 32
    assert H.contraction_len(4096, 256) == 4096
    assert H.contraction_len(11008, 128) == 11008
    assert H.contraction_len(100, 16) == 128
    assert H.contraction_len(300, 256) == 512
