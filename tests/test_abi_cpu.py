"""Host-side checks of the C ABI: the library loads without a GPU, exports every symbol the
header declares, and rejects every invalid call with its status code before any HIP call
(the fake device pointers below are never dereferenced)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "halo.h")

import hadamard_rotated_precision_halo_amd as H  # noqa: E402

OK, NULL, SHAPE, BLOCK, DTYPE, ALIGN, WORKSPACE, HIP, OPTION = range(9)
F32, BF16, I8, E4M3, E5M2, I32 = range(6)

P = ctypes.c_void_p(0x10000)    # 16-byte aligned fake device pointer
P2 = ctypes.c_void_p(0x20000)
P3 = ctypes.c_void_p(0x30000)
BAD = ctypes.c_void_p(0x10008)  # misaligned
NUL = None


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(H.LIB_PATH):
        import hadamard_rotated_precision_halo_amd.build as b
        b.build()
    return H.lib()


def declared_functions():
    text = open(HEADER, encoding="utf-8").read()
    return sorted(set(re.findall(r"^\s*(?:const char\*|halo_status|size_t)\s+(halo_\w+)\s*\(",
                                 text, re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for f in ("halo_fwht_quant", "halo_gemm_i8", "halo_gemm_fp8", "halo_linear_fwd",
              "halo_linear_bwd", "halo_linear_workspace_bytes", "halo_status_str"):
        assert f in names
    assert set(names) == set(H.EXPORTS)


def test_library_exports_every_declared_symbol(L):
    out = subprocess.run(["nm", "-D", "--defined-only", H.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s(halo_\w+)$", out, re.M))
    for f in declared_functions():
        assert f in exported, f
        getattr(L, f)  # resolvable through ctypes


def test_status_strings(L):
    for s in range(9):
        assert L.halo_status_str(s)
    assert L.halo_status_str(0) == b"ok"


def fq(L, x=P, xt=BF16, rows=64, cols=256, ldx=256, axis=0, block=256, qt=I8, q=P2, ldq=256,
       scale=P3, ws=None, wsb=0):
    return L.halo_fwht_quant(x, xt, rows, cols, ldx, axis, block, qt, q, ldq, scale, ws, wsb, None)


def test_fwht_quant_validation(L):
    assert fq(L, x=NUL) == NULL
    assert fq(L, q=NUL) == NULL
    assert fq(L, scale=NUL) == NULL
    assert fq(L, xt=I8) == DTYPE
    assert fq(L, qt=BF16) == DTYPE
    assert fq(L, qt=I32) == DTYPE
    assert fq(L, block=3) == BLOCK
    assert fq(L, block=0) == BLOCK
    assert fq(L, block=8192, cols=8192, ldx=8192, ldq=8192) == BLOCK
    assert fq(L, block=512) == SHAPE             # 256 padded to 512: codes need ldq >= 512
    assert fq(L, axis=1, block=128, ldq=64) == SHAPE  # 64 rows padded to 128 codes per column
    assert fq(L, rows=-1) == SHAPE
    assert fq(L, ldx=128) == SHAPE
    assert fq(L, ldq=128) == SHAPE
    assert fq(L, axis=7) == SHAPE
    assert fq(L, block=4, cols=12, ldx=16, ldq=16) == SHAPE          # length not a multiple of 8
    assert fq(L, axis=1, block=4, rows=12, ldq=16) == SHAPE  # padded length 12 not a multiple of 8
    assert fq(L, block=64, cols=200, ldx=200, ldq=200) == SHAPE      # 200 padded to 256 codes
    assert fq(L, axis=1, block=16, rows=64, cols=12, ldx=16, ldq=64) == SHAPE  # 12 columns
    big = 1 << 20
    assert fq(L, cols=big, ldx=big, ldq=big, block=256) == SHAPE     # beyond the rows kernel
    # rows of up to 65536 positions when a multiple of 64 (the wave kernel: a misaligned x
    # is the first error a call past the shape checks meets); else up to 16384
    w64 = 1 << 16
    assert fq(L, x=BAD, cols=w64, ldx=w64, ldq=w64) == ALIGN
    assert fq(L, x=BAD, cols=w64 + 256, ldx=w64 + 256, ldq=w64 + 256) == SHAPE
    assert fq(L, x=BAD, xt=F32, cols=28672, ldx=28672, ldq=28672) == ALIGN
    assert fq(L, x=BAD, block=32, cols=20000, ldx=20000, ldq=20000) == SHAPE   # not k * 64
    assert fq(L, x=BAD, block=32, cols=16352, ldx=16352, ldq=16352) == ALIGN   # older kernel
    assert fq(L, x=BAD) == ALIGN
    assert fq(L, q=BAD) == ALIGN
    assert fq(L, ldx=260, cols=256) == ALIGN  # 520 bytes per bf16 row
    assert fq(L, ldq=260) == ALIGN
    assert fq(L, ws=BAD, wsb=4096) == ALIGN


def fqx(L, opts, **kw):
    a = dict(x=P, xt=BF16, rows=64, cols=256, ldx=256, axis=0, block=256, qt=I8, q=P2, ldq=256,
             scale=P3)
    a.update(kw)
    return L.halo_fwht_quant_ex(a["x"], a["xt"], a["rows"], a["cols"], a["ldx"], a["axis"],
                                a["block"], a["qt"], a["q"], a["ldq"], a["scale"],
                                ctypes.byref(opts) if opts is not None else None, None, 0, None)


def test_fwht_quant_ex_validation(L):
    def opts(signs=None, rounding=0):
        return H.QuantOpts(signs, rounding, (ctypes.c_uint32 * 2)(1, 2), (ctypes.c_uint32 * 2)(3, 4))
    assert fqx(L, opts(rounding=2)) == OPTION
    assert fqx(L, opts(rounding=-1)) == OPTION
    assert fqx(L, opts(rounding=1), qt=F32, ldq=256) == OPTION   # values are not rounded
    assert fqx(L, opts(signs=BAD.value)) == ALIGN
    assert fqx(L, opts(), x=NUL) == NULL                           # the plain checks still run
    assert fqx(L, opts(rounding=1), block=3) == BLOCK
    # stochastic rounding of long fp32 rows: only the older kernel, up to 16384 positions
    assert fqx(L, opts(rounding=1), x=BAD, xt=F32, cols=20480, ldx=20480, ldq=20480) == SHAPE
    assert fqx(L, opts(rounding=1), x=BAD, cols=20480, ldx=20480, ldq=20480) == ALIGN


def test_fwht_quant_workspace_bytes(L):
    # single-read columns pass: the count of tasks that stopped waiting (256 bytes), per-strip
    # arrival counters (padded to 256 bytes) + one maximum per column, for columns longer
    # than one task (4096 rows: whole columns, no scratch)
    W = L.halo_fwht_quant_workspace_bytes
    assert W(4096, 4096, 1, 256, BF16) == 0      # whole 4096-row columns per task
    assert W(4000, 4096, 1, 256, BF16) == 0      # padded to 4096 rows: still whole columns
    assert W(8192, 4096, 1, 128, BF16) == 256 + 256 + 4096 * 4  # 64 strips of 64 columns, 8 parts
    assert W(16384, 14336, 1, 512, BF16) == 256 + 1024 + 14336 * 4
    assert W(8192, 4096, 1, 4096, BF16) == 256 + 1024 + 4096 * 4  # 16-column strips, 4096 rows
    assert W(1024, 4096, 1, 256, BF16) == 0      # one part per column: no exchange
    assert W(4096, 4096, 0, 256, BF16) == 0      # rows axis
    assert W(4096, 4096, 1, 256, F32) == 0       # fp32 input takes the two-read path
    assert W(4096, 4096, 1, 3, BF16) == 0
    assert W(-1, 4096, 1, 256, BF16) == 0


def gi8(L, a=P, lda=128, sa=P2, b=P3, ldb=128, sb=P2, m=64, n=64, k=128, c=P, ct=BF16, ldc=64):
    return L.halo_gemm_i8(a, lda, sa, b, ldb, sb, m, n, k, c, ct, ldc, None)


def test_gemm_i8_validation(L):
    assert gi8(L, a=NUL) == NULL
    assert gi8(L, c=NUL) == NULL
    assert gi8(L, sa=NUL) == NULL
    assert gi8(L, ct=I8) == DTYPE
    assert gi8(L, ct=E4M3) == DTYPE
    assert gi8(L, k=0) == SHAPE
    assert gi8(L, k=120, lda=128, ldb=128) == SHAPE
    assert gi8(L, m=-1) == SHAPE
    assert gi8(L, lda=64) == SHAPE
    assert gi8(L, ldc=32) == SHAPE
    assert gi8(L, a=BAD) == ALIGN
    assert gi8(L, lda=136, k=128) == ALIGN        # rows not 16-byte aligned
    assert gi8(L, ct=BF16, ldc=68) == ALIGN       # 136-byte output rows
    assert gi8(L, sa=BAD) == ALIGN
    # the kernel addresses each operand with 32-bit byte offsets: spans up to 4 GiB only
    big = (1 << 20) + 1                     # (big - 1) * 4096 + 4096 = 2^32 + 4096
    assert gi8(L, m=big, lda=4096, ldb=4096, k=4096) == SHAPE
    assert gi8(L, n=big, lda=4096, ldb=4096, k=4096) == SHAPE
    # a span of exactly 2^32 bytes is refused too: its last load would end past the
    # 2^32 - 1 bytes that the kernel's buffer resource covers
    assert gi8(L, m=1 << 20, lda=4096, ldb=4096, k=4096) == SHAPE
    assert gi8(L, n=1 << 20, lda=4096, ldb=4096, k=4096) == SHAPE


def gf8(L, a=P, at=E4M3, lda=128, sa=P2, b=P3, bt=E4M3, ldb=128, sb=P2, m=64, n=64, k=128, c=P,
        ct=BF16, ldc=64):
    return L.halo_gemm_fp8(a, at, lda, sa, b, bt, ldb, sb, m, n, k, c, ct, ldc, None)


def test_gemm_fp8_validation(L):
    assert gf8(L, at=I8) == DTYPE
    assert gf8(L, bt=BF16) == DTYPE
    assert gf8(L, ct=I32) == DTYPE
    assert gf8(L, k=112, lda=128, ldb=128) == SHAPE   # not a multiple of 32
    assert gf8(L, sb=NUL) == NULL
    assert gf8(L, b=BAD) == ALIGN


def test_workspace_bytes(L):
    r = lambda v: (v + 255) // 256 * 256  # noqa: E731
    pad = lambda d, b: -(-d // max(b, 32)) * max(b, 32)  # noqa: E731  contraction length
    m, n, k = 300, 520, 1024
    X = L.halo_linear_workspace_bytes_ex
    for b in (1, 64, 256):
        kq = pad(k, b)
        assert X(m, n, k, b, I8, 0) == r(m * kq) + r(4 * m) + r(n * kq) + r(4 * n)
    nq, mq = pad(n, 256), pad(m, 256)  # 768, 512
    want = (r(m * nq) + r(4 * m) + r(k * nq) + r(4 * k) + r(n * mq) + r(4 * n) + r(k * mq)
            + r(4 * k))
    # the W columns pass along n (768 rows) runs 256-row tasks in 3 parts: the count of tasks
    # that stopped waiting (256 bytes), 4 strips of 256 columns need arrival counters (256
    # bytes) and 1024 column maxima
    want += r(256 + r(4 * 4) + 4 * k)
    assert X(m, n, k, 256, E4M3, 1) == want
    # the block-free query covers every block: the largest padding (block 4096) decides here
    assert L.halo_linear_workspace_bytes(m, n, k, I8, 0) == X(m, n, k, 4096, I8, 0)
    assert L.halo_linear_workspace_bytes(m, n, k, I8, 0) == max(X(m, n, k, 1 << i, I8, 0)
                                                              for i in range(13))
    assert X(m, n, k, 3, I8, 0) == 0
    # 4096^3 backward: the code matrices only (4096-row columns go whole into one task, so the
    # columns passes need no scratch for any block)
    big = 4096
    codes = 4 * (r(big * big) + r(4 * big))
    assert L.halo_linear_workspace_bytes(big, big, big, I8, 1) == codes
    # 8192 tokens: the columns passes along m exchange partial maxima (dY: 4096 columns, X:
    # 4096 columns; block 4096 needs the most, 256 strips of 16 columns in 2 parts)
    m8 = 8192
    codes8 = (r(m8 * big) + r(4 * m8) + r(big * big) + r(4 * big) + r(big * m8) + r(4 * big)
              + r(big * m8) + r(4 * big))
    assert L.halo_linear_workspace_bytes(m8, big, big, I8, 1) == codes8 + 2 * r(256 + 1024 + 4096 * 4)
    assert L.halo_linear_workspace_bytes(-1, n, k, I8, 0) == 0
    assert L.halo_linear_workspace_bytes(m, n, k, BF16, 0) == 0


def fwd(L, x=P, w=P2, io=BF16, m=256, n=256, k=256, block=128, qt=I8, y=P3, yt=BF16, ws=P,
        wsb=None):
    if wsb is None:
        wsb = L.halo_linear_workspace_bytes(m, n, k, I8, 0)
    return L.halo_linear_fwd(x, w, io, m, n, k, block, qt, y, yt, ws, wsb, None)


def test_linear_fwd_validation(L):
    assert fwd(L, x=NUL) == NULL
    assert fwd(L, io=I8) == DTYPE
    assert fwd(L, qt=E5M2) == DTYPE
    assert fwd(L, yt=I32) == DTYPE
    assert fwd(L, k=244) == SHAPE              # not a multiple of 8
    assert fwd(L, k=70000) == SHAPE            # padded k beyond the rows kernels
    assert fwd(L, k=20000, block=32) == SHAPE  # padded k 20000: not k * 64, over 16384
    assert fwd(L, k=20000, y=BAD) == ALIGN     # padded to 20096 = 314 * 64: the wave kernel
    assert fwd(L, m=(1 << 20) + 1, k=4096, wsb=1 << 40) == SHAPE  # X codes span over 4 GiB
    assert fwd(L, block=6) == BLOCK
    assert fwd(L, ws=NUL) == WORKSPACE
    assert fwd(L, wsb=1000) == WORKSPACE
    assert fwd(L, y=BAD) == ALIGN


def bwd(L, dy=P, x=P2, w=P3, io=BF16, m=256, n=256, k=256, block=128, qt=I8, gqt=I8, dx=P,
        dw=P2, ws=P3, wsb=None):
    if wsb is None:
        wsb = L.halo_linear_workspace_bytes(m, n, k, I8, 1)
    return L.halo_linear_bwd(dy, x, w, io, m, n, k, block, qt, gqt, dx, dw, ws, wsb, None)


def test_linear_bwd_validation(L):
    assert bwd(L, dy=NUL) == NULL
    assert bwd(L, gqt=E5M2) == DTYPE          # INT8 operands need INT8 gradients
    assert bwd(L, qt=E4M3, gqt=I8) == DTYPE
    assert bwd(L, qt=E5M2, gqt=E5M2) == DTYPE
    assert bwd(L, n=244) == SHAPE              # not a multiple of 8
    assert bwd(L, n=70000) == SHAPE            # the dY rows beyond the rows kernels
    assert bwd(L, n=28672, dx=BAD) == ALIGN    # a 28672-wide layer's dX: the wave kernel
    assert bwd(L, k=244) == SHAPE
    assert bwd(L, m=0) == SHAPE
    assert bwd(L, block=6) == BLOCK
    # dW only (no rows-length limit): the W column codes [k x padded n] span over 4 GiB
    assert bwd(L, n=(1 << 20) + 8, k=4096, dx=NUL, wsb=1 << 40) == SHAPE
    assert bwd(L, wsb=10) == WORKSPACE
    assert bwd(L, dx=BAD) == ALIGN


def test_linear_ex_validation(L):
    def lopts(rounding=0, sk=None, sn=None, sm=None):
        return H.LinearOpts(sk, sn, sm, rounding, (ctypes.c_uint32 * 2)(1, 2),
                            (ctypes.c_uint32 * 2)(3, 4))
    m = n = k = 256
    wsf = L.halo_linear_workspace_bytes_ex(m, n, k, 128, I8, 0)
    wsb = L.halo_linear_workspace_bytes_ex(m, n, k, 128, I8, 1)
    f = lambda o: L.halo_linear_fwd_ex(P, P2, BF16, m, n, k, 128, I8, P3, BF16,  # noqa: E731
                                       ctypes.byref(o), P, wsf, None)
    b = lambda o: L.halo_linear_bwd_ex(P, P2, P3, BF16, m, n, k, 128, I8, I8, P, P2,  # noqa: E731
                                       ctypes.byref(o), P3, wsb, None)
    assert f(lopts(rounding=5)) == OPTION
    assert f(lopts(sk=BAD.value)) == ALIGN
    assert b(lopts(rounding=5)) == OPTION
    assert b(lopts(sn=BAD.value)) == ALIGN
    assert b(lopts(sm=BAD.value)) == ALIGN
    assert L.halo_linear_bwd_ex(P, P2, P3, BF16, m, n, k, 128, I8, I8, P, P2,
                                ctypes.byref(lopts()), P3, wsb - 256, None) == WORKSPACE


def test_mfma_rate_probe_validation(L):
    ops = ctypes.c_int64(-1)
    assert L.halo_mfma_rate_probe(0, 100, None, None) == NULL
    for kind, iters in ((-1, 100), (3, 100), (0, 1), (0, 0), (1, (1 << 20) + 1)):
        assert L.halo_mfma_rate_probe(kind, iters, ctypes.byref(ops), None) == SHAPE
    assert ops.value == -1  # refused before anything is written or launched


def test_fwht_quant_dual_validation(L):
    def dual(x=P, xt=BF16, rows=256, cols=256, ldx=256, block=128, qt=I8, qr=P2, ldqr=256,
             sr=P3, qc=P, ldqc=256, sc=P2, ws=None, wsb=0):
        return L.halo_fwht_quant_dual(x, xt, rows, cols, ldx, block, qt, qr, ldqr, sr, qc, ldqc,
                                      sc, None, None, ws, wsb, None)
    assert dual(qc=NUL) == NULL
    assert dual(sr=NUL) == NULL
    assert dual(xt=I8) == DTYPE
    assert dual(block=5) == BLOCK
    assert dual(ldqr=128) == SHAPE               # row codes need 256 per row
    assert dual(ldqc=128) == SHAPE               # column codes need 256 per column
    assert dual(qc=BAD) == ALIGN
    assert dual(ws=BAD, wsb=4096) == ALIGN
    W = L.halo_fwht_quant_dual_workspace_bytes
    # single read: late word (256 B), tile-column and tile-row counts (256 B each), maxima
    assert W(4096, 4096, 256, BF16) == 768 + 4 * 4096 + 4 * 4096
    assert W(8192, 8192, 256, BF16) == 768 + 4 * 8192 + 4 * 8192
    assert W(300, 512, 256, BF16) == 0           # no single read, and short columns need none
    assert W(8192, 520, 8, BF16) == L.halo_fwht_quant_workspace_bytes(8192, 520, 1, 8, BF16)
    assert W(4096, 4096, 256, F32) == 0
    assert W(4096, 4096, 512, BF16) == 0
    assert W(-1, 4096, 256, BF16) == 0
