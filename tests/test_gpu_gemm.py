"""GPU parity of halo_gemm_i8 / halo_gemm_fp8 against the oracle's integer and fp64 products,
given identical codes (the codes are the oracle's own, uploaded).

Bars: int32 accumulators bit-exact; the fp32 dequant within a few fp32 roundings; the bf16
dequant within one bf16 rounding of the exact value.  FP8: exact whenever every group sum of
the matrix cores is exact (integer products), otherwise within the measured accumulation bound
of the gfx950 FP8 matrix cores (parity_util.fp8_acc_bound: groups of 8 products summed in
~15-bit fixed point, groups accumulated in fp32).
"""
import numpy as np
import pytest
import torch

import hadamard_rotated_precision_halo_amd as H
import oracle as O
from parity_util import DEV, codes_to_dev, fp8_acc_bound, padded_out

pytestmark = pytest.mark.gpu


def _codes(rng, r, k):
    return rng.integers(-127, 128, (r, k), dtype=np.int8)


def _scales(rng, r):
    return rng.uniform(1e-4, 2e-2, r).astype(np.float32)


SHAPES = [(256, 256, 128), (300, 520, 1040), (1, 1, 16), (513, 257, 4096), (64, 1024, 48),
          (1024, 768, 11008 // 8), (256, 512, 16384)]


@pytest.mark.parametrize("m,n,k", SHAPES)
def test_gemm_i8_int32_bit_exact(m, n, k):
    rng = np.random.default_rng(m * 31 + n * 7 + k)
    a, b = _codes(rng, m, k), _codes(rng, n, k)
    ref = O.gemm_i8(a, b)
    c = H.gemm_i8(codes_to_dev(a, O.I8), None, codes_to_dev(b, O.I8), None,
                  c=padded_out(m, n, torch.int32))
    got = c.cpu().numpy().astype(np.int64)
    assert np.array_equal(got, ref), f"{int((got != ref).sum())} accumulators differ"


def test_gemm_i8_extreme_codes():
    # all +-127: the largest accumulators the method can produce at this k
    k = 16384
    a = np.full((32, k), 127, np.int8)
    b = np.full((40, k), -127, np.int8)
    b[::2] = 127
    c = H.gemm_i8(codes_to_dev(a, O.I8), None, codes_to_dev(b, O.I8), None, out_dtype=torch.int32)
    assert np.array_equal(c.cpu().numpy().astype(np.int64), O.gemm_i8(a, b))


@pytest.mark.parametrize("m,n,k", [(256, 256, 128), (300, 520, 1040), (513, 257, 4096)])
@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16])
def test_gemm_i8_dequant(m, n, k, out):
    rng = np.random.default_rng(k + m)
    a, b = _codes(rng, m, k), _codes(rng, n, k)
    sa, sb = _scales(rng, m), _scales(rng, n)
    exact = O.dequant(O.gemm_i8(a, b).astype(np.float64), sa, sb)
    c = H.gemm_i8(codes_to_dev(a, O.I8), torch.from_numpy(sa).to(DEV), codes_to_dev(b, O.I8),
                  torch.from_numpy(sb).to(DEV), c=padded_out(m, n, out))
    got = c.float().cpu().numpy().astype(np.float64)
    # int32 -> fp32 conversion plus two fp32 products: at most 3 roundings of 2^-24
    rel = 3.0 * 2.0 ** -24 if out == torch.float32 else 2.0 ** -8 + 3.0 * 2.0 ** -24
    assert (np.abs(got - exact) <= rel * np.abs(exact) + 1e-30).all()


@pytest.mark.parametrize("m,n,k", [(256, 256, 128), (300, 520, 1056), (64, 1024, 4096),
                                   (513, 257, 14336)])
@pytest.mark.parametrize("fa,fb", [(O.E4M3, O.E4M3), (O.E5M2, O.E4M3), (O.E4M3, O.E5M2),
                                   (O.E5M2, O.E5M2)])
def test_gemm_fp8_within_accumulation_bound(m, n, k, fa, fb):
    rng = np.random.default_rng(m + n + k + fa * 10 + fb)
    ta, tb = O.fp8_table(fa), O.fp8_table(fb)
    ca = rng.choice(np.nonzero(np.isfinite(ta))[0].astype(np.uint8), (m, k))
    cb = rng.choice(np.nonzero(np.isfinite(tb))[0].astype(np.uint8), (n, k))
    sa, sb = _scales(rng, m), _scales(rng, n)
    exact = O.gemm_fp8(ca, fa, cb, fb)
    absum = O.matmul_f64(np.abs(ta[ca]), np.abs(tb[cb]))
    c = H.gemm_fp8(codes_to_dev(ca, fa), torch.from_numpy(sa).to(DEV), codes_to_dev(cb, fb),
                   torch.from_numpy(sb).to(DEV), c=padded_out(m, n, torch.float32))
    got = c.cpu().numpy().astype(np.float64)
    u = 2.0 ** -24
    s = np.outer(sa.astype(np.float64), sb.astype(np.float64))
    bound = (fp8_acc_bound(absum, k) + 3 * u * np.abs(exact)) * s * (1 + 4 * u)
    err = np.abs(got - exact * s)
    assert (err <= bound + 1e-30).all(), f"max excess {np.max(err - bound)}"


@pytest.mark.parametrize("fa,fb", [(O.E4M3, O.E4M3), (O.E5M2, O.E4M3)])
@pytest.mark.parametrize("m,n,k", [(256, 256, 128), (300, 520, 4096)])
def test_gemm_fp8_exact_on_integer_products(m, n, k, fa, fb):
    # integers |v| <= 8 are exact in both formats; every product is an integer below 2^7 and
    # every partial sum stays far below 2^24, so each grouped fixed-point sum and each fp32
    # addition is exact: the accumulators must equal the exact sums bit for bit
    rng = np.random.default_rng(k + m)
    ints = np.arange(-8, 9, dtype=np.float64)
    ca = np.array([O.fp8_encode(v, fa) for v in rng.choice(ints, m * k)], np.uint8).reshape(m, k)
    cb = np.array([O.fp8_encode(v, fb) for v in rng.choice(ints, n * k)], np.uint8).reshape(n, k)
    exact = O.gemm_fp8(ca, fa, cb, fb)
    ones_m = torch.ones(m, device=DEV)
    ones_n = torch.ones(n, device=DEV)
    c = H.gemm_fp8(codes_to_dev(ca, fa), ones_m, codes_to_dev(cb, fb), ones_n,
                   c=padded_out(m, n, torch.float32))
    assert np.array_equal(c.cpu().numpy().astype(np.float64), exact)


def test_gemm_empty_and_degenerate():
    a = torch.empty((0, 128), dtype=torch.int8, device=DEV)
    b = torch.ones((64, 128), dtype=torch.int8, device=DEV)
    c = H.gemm_i8(a, None, b, None, out_dtype=torch.int32)
    assert c.shape == (0, 64)
    z = torch.zeros((40, 256), dtype=torch.int8, device=DEV)
    c = H.gemm_i8(z, None, z, None, out_dtype=torch.int32)
    assert (c == 0).all()


@pytest.mark.parametrize("big", ["a", "b"])
def test_gemm_i8_operand_spanning_almost_4gib(big):
    # The kernel loads each operand through a buffer resource with 32-bit byte offsets: an
    # operand of 2^20 - 1 rows of 4096 bytes spans 2^32 - 4096 bytes, the largest accepted, and
    # its last rows start just below 2^32 (rows past 2^31 / 4096 need the offsets unsigned).
    # Its rows repeat a seeded 4099-row pattern, so every accumulator is known from the
    # oracle's product of the pattern; every one is compared.
    rng = np.random.default_rng(41)
    rows, k, other = (1 << 20) - 1, 4096, 64
    pattern = _codes(rng, 4099, k)
    small = _codes(rng, other, k)
    idx = torch.arange(rows, device=DEV) % pattern.shape[0]
    big_dev = codes_to_dev(pattern, O.I8)[idx]          # torch gather: 4 GiB - 4 KiB of codes
    small_dev = codes_to_dev(small, O.I8)
    ref = O.gemm_i8(pattern, small)                      # [4099 x 64] int64
    print(f"operand {big}: {rows} x {k} codes", flush=True)
    if big == "a":
        acc = H.gemm_i8(big_dev, None, small_dev, None, out_dtype=torch.int32)
        want = torch.from_numpy(ref.astype(np.int32)).to(DEV)[idx]
    else:
        acc = padded_out(other, rows, torch.int32)
        H.gemm_i8(small_dev, None, big_dev, None, c=acc)
        want = torch.from_numpy(np.ascontiguousarray(ref.T).astype(np.int32)).to(DEV)[:, idx]
    torch.cuda.synchronize()
    assert np.abs(ref).max() < 2**31
    bad = int((acc != want).sum().item())
    assert bad == 0, f"{bad} accumulators differ"


def test_gemm_i8_strided_operands_and_output():
    rng = np.random.default_rng(5)
    a_full = _codes(rng, 200, 512)
    b_full = _codes(rng, 300, 512)
    a = codes_to_dev(a_full, O.I8)[:, :256]
    b = codes_to_dev(b_full, O.I8)[:, :256]
    cbig = torch.full((200, 320), -1, dtype=torch.int32, device=DEV)
    c = cbig[:, :300]
    H.gemm_i8(a, None, b, None, c=c)
    torch.cuda.synchronize()
    ref = O.gemm_i8(a_full[:, :256], b_full[:, :256])
    assert np.array_equal(c.cpu().numpy().astype(np.int64), ref)
    assert (cbig[:, 300:] == -1).all()  # nothing written past n
