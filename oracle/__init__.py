"""CPU oracle for the Hadamard-rotated low-precision linear layer.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` may import this package.  It shares no code with the GPU library and the
GPU library never calls it.  The arithmetic lives in ``halo_oracle.c`` (plain C, fp64 and
int64); this module only marshals numpy arrays into it.

Pages followed: "QWHA方法：基于Walsh-Hadamard变换的高效大模型微调技术" s2.1 (Sylvester
definition), s2.2 (butterfly, 1/sqrt(n), absmax quantiser), s3.1 (blockwise transform), s5
(zero padding, stochastic rounding); "HALO: Hadamard-Assisted Lower-Precision Optimization for
LLMs", abstract (rotations in both passes, every large product in low precision) and key
design 2 (INT8 or FP8); "企业官网建设流程全解析" s4.2 (one random seed for the Hadamard matrix on
every node: the randomised transform H D).  Stochastic rounding draws its uniforms from
Philox4x32-10 (Salmon et al., SC'11).
"""
import ctypes
import os

import numpy as np

from . import build as _build

F32, BF16, I8, E4M3, E5M2, F64 = 0, 1, 2, 3, 4, 5
ROWS, COLS = 0, 1
RNE, STOCHASTIC = 0, 1
QMAX = {I8: 127.0, E4M3: 448.0, E5M2: 57344.0}

_lib = None


def lib():
    """Load (building first if needed) the oracle shared library."""
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB) or (
                os.path.getmtime(_build.LIB) < os.path.getmtime(_build.SRC)):
            _build.build()
        L = ctypes.CDLL(_build.LIB)
        i64, vp, dp = ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p
        L.hor_fwht_quant.argtypes = [vp, ctypes.c_int, i64, i64, i64, ctypes.c_int, i64,
                                     ctypes.c_int, ctypes.c_int, vp, i64, vp, dp]
        L.hor_fwht_quant.restype = ctypes.c_int
        L.hor_fwht_quant_ex.argtypes = [vp, ctypes.c_int, i64, i64, i64, ctypes.c_int, i64,
                                        ctypes.c_int, ctypes.c_int, vp, i64, vp, ctypes.c_int, vp,
                                        vp, vp, dp]
        L.hor_fwht_quant_ex.restype = ctypes.c_int
        L.hor_philox4x32_10.argtypes = [vp, vp, vp]
        L.hor_philox4x32_10.restype = None
        L.hor_linear_fwd_ex.argtypes = [vp, vp, ctypes.c_int, i64, i64, i64, i64, ctypes.c_int,
                                        ctypes.c_int, vp, dp]
        L.hor_linear_fwd_ex.restype = ctypes.c_int
        L.hor_linear_bwd_ex.argtypes = [vp, vp, vp, ctypes.c_int, i64, i64, i64, i64,
                                        ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp,
                                        ctypes.c_int, vp, vp, dp, dp]
        L.hor_linear_bwd_ex.restype = ctypes.c_int
        L.hor_fwht_f64.argtypes = [dp, i64, i64]
        L.hor_fwht_f64.restype = ctypes.c_int
        L.hor_gemm_i8.argtypes = [vp, vp, i64, i64, i64, vp]
        L.hor_gemm_i8.restype = ctypes.c_int
        L.hor_gemm_fp8.argtypes = [vp, ctypes.c_int, vp, ctypes.c_int, i64, i64, i64, dp]
        L.hor_gemm_fp8.restype = ctypes.c_int
        L.hor_matmul_f64.argtypes = [dp, dp, i64, i64, i64, dp]
        L.hor_matmul_f64.restype = ctypes.c_int
        L.hor_dequant.argtypes = [dp, dp, dp, i64, i64, dp]
        L.hor_dequant.restype = None
        L.hor_linear_fwd.argtypes = [vp, vp, ctypes.c_int, i64, i64, i64, i64, ctypes.c_int,
                                     ctypes.c_int, dp]
        L.hor_linear_fwd.restype = ctypes.c_int
        L.hor_linear_bwd.argtypes = [vp, vp, vp, ctypes.c_int, i64, i64, i64, i64, ctypes.c_int,
                                     ctypes.c_int, ctypes.c_int, dp, dp]
        L.hor_linear_bwd.restype = ctypes.c_int
        L.hor_fp8_encode.argtypes = [ctypes.c_double, ctypes.c_int]
        L.hor_fp8_encode.restype = ctypes.c_uint8
        L.hor_fp8_decode.argtypes = [ctypes.c_uint8, ctypes.c_int]
        L.hor_fp8_decode.restype = ctypes.c_double
        L.hor_num_threads.argtypes = []
        L.hor_num_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def _xtype(x):
    if x.dtype == np.float32:
        return F32
    if x.dtype == np.uint16:  # bf16 bit patterns
        return BF16
    raise TypeError("oracle inputs are float32 arrays or uint16 arrays of bf16 bits")


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (status {rc})")


def num_threads() -> int:
    return lib().hor_num_threads()


def fwht(v, block):
    """Blockwise orthonormal Walsh-Hadamard transform (fp64) of the last axis of ``v``."""
    y = np.ascontiguousarray(np.array(v, dtype=np.float64))
    flat = y.reshape(-1, y.shape[-1]) if y.ndim else y.reshape(1, 1)
    for r in range(flat.shape[0]):
        row = np.ascontiguousarray(flat[r])
        _check(lib().hor_fwht_f64(_ptr(row), row.shape[0], int(block)), "fwht")
        flat[r] = row
    return flat.reshape(y.shape)


def padded_len(length, block):
    """Rotated length of a vector of ``length`` elements: rounded up to a multiple of block."""
    return -(-int(length) // int(block)) * int(block)


def _u32(a, n=None):
    if a is None:
        return None
    a = np.ascontiguousarray(np.asarray(a, dtype=np.uint32))
    if n is not None and a.shape[0] < n:
        raise ValueError(f"need at least {n} uint32 words, got {a.shape[0]}")
    return a


def philox4x32_10(ctr, key):
    """The four output words of Philox4x32-10 for a 4-word counter and a 2-word key."""
    c, k = _u32(ctr, 4), _u32(key, 2)
    out = np.empty(4, dtype=np.uint32)
    lib().hor_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def fwht_quant(x, axis, block, qtype, precision=64, vec_idx=None, signs=None, rounding=RNE,
               key=(0, 0), ctr_hi=(0, 0)):
    """Rotate and quantise the rows (axis ROWS) or columns (axis COLS) of ``x``.

    Each vector is padded with zeros to ``padded_len(L, block)``, multiplied by the signs
    (uint32 words, bit i set = element i negated; None = no signs), rotated and quantised with
    nearest-even (RNE) or stochastic (STOCHASTIC; Philox key ``key``, counter words 2-3
    ``ctr_hi``) rounding.

    Returns ``(codes, scales)``: codes is [nvec x Lp] (int8; uint8 fp8 bytes; or float64 rotated
    values when ``qtype`` is F64) with one vector per row, scales is float64 [nvec].
    """
    x = np.ascontiguousarray(x)
    rows, cols = x.shape
    L = cols if axis == ROWS else rows
    Lp = padded_len(L, block)
    total = rows if axis == ROWS else cols
    sg = _u32(signs, -(-Lp // 32))
    kk, ch = _u32(key, 2), _u32(ctr_hi, 2)
    idx = None
    if vec_idx is not None:
        idx = np.ascontiguousarray(np.asarray(vec_idx, dtype=np.int64))
        nvec = idx.shape[0]
    else:
        nvec = total
    dt = {I8: np.int8, E4M3: np.uint8, E5M2: np.uint8, F64: np.float64}[qtype]
    q = np.empty((nvec, Lp), dtype=dt)
    s = np.empty(nvec, dtype=np.float64)
    rc = lib().hor_fwht_quant_ex(_ptr(x), _xtype(x), rows, cols, cols, axis, int(block), qtype,
                                 int(precision), _ptr(idx), nvec, _ptr(sg), int(rounding),
                                 _ptr(kk), _ptr(ch), _ptr(q), _ptr(s))
    _check(rc, "fwht_quant")
    return q, s


def gemm_i8(a, b):
    """int64 accumulators of a[m x k] . b[n x k]^T."""
    a = np.ascontiguousarray(a, dtype=np.int8)
    b = np.ascontiguousarray(b, dtype=np.int8)
    m, k = a.shape
    n = b.shape[0]
    acc = np.empty((m, n), dtype=np.int64)
    _check(lib().hor_gemm_i8(_ptr(a), _ptr(b), m, n, k, _ptr(acc)), "gemm_i8")
    return acc


def gemm_fp8(a, afmt, b, bfmt):
    """fp64 sums of decoded fp8 codes a[m x k] . b[n x k]^T."""
    a = np.ascontiguousarray(a, dtype=np.uint8)
    b = np.ascontiguousarray(b, dtype=np.uint8)
    m, k = a.shape
    n = b.shape[0]
    out = np.empty((m, n), dtype=np.float64)
    _check(lib().hor_gemm_fp8(_ptr(a), afmt, _ptr(b), bfmt, m, n, k, _ptr(out)), "gemm_fp8")
    return out


def matmul_f64(a, b):
    """Exact fp64 product a[m x k] . b[n x k]^T (the unquantised reference)."""
    a = np.ascontiguousarray(a, dtype=np.float64)
    b = np.ascontiguousarray(b, dtype=np.float64)
    m, k = a.shape
    n = b.shape[0]
    out = np.empty((m, n), dtype=np.float64)
    _check(lib().hor_matmul_f64(_ptr(a), _ptr(b), m, n, k, _ptr(out)), "matmul_f64")
    return out


def dequant(acc, sa, sb):
    acc = np.ascontiguousarray(acc, dtype=np.float64)
    sa = np.ascontiguousarray(sa, dtype=np.float64)
    sb = np.ascontiguousarray(sb, dtype=np.float64)
    out = np.empty_like(acc)
    lib().hor_dequant(_ptr(acc), _ptr(sa), _ptr(sb), acc.shape[0], acc.shape[1], _ptr(out))
    return out


def fp8_encode(v, fmt):
    return lib().hor_fp8_encode(float(v), fmt)


def fp8_decode(c, fmt):
    return lib().hor_fp8_decode(int(c), fmt)


def fp8_table(fmt):
    """Decoded value of each of the 256 codes of ``fmt``."""
    return np.array([fp8_decode(c, fmt) for c in range(256)], dtype=np.float64)


def linear_fwd(x, w, block, qtype=I8, precision=64, signs_k=None):
    """Y = dequant(Q(X rotated along K) . Q(W rotated along K)^T), fp64 [m x n]; signs_k: the
    randomised transform's sign words along K (None: plain transform)."""
    x = np.ascontiguousarray(x)
    w = np.ascontiguousarray(w)
    assert x.dtype == w.dtype
    m, k = x.shape
    n = w.shape[0]
    y = np.empty((m, n), dtype=np.float64)
    sk = _u32(signs_k, -(-padded_len(k, block) // 32))
    rc = lib().hor_linear_fwd_ex(_ptr(x), _ptr(w), _xtype(x), m, n, k, int(block), qtype,
                                 int(precision), _ptr(sk), _ptr(y))
    _check(rc, "linear_fwd")
    return y


def linear_bwd(dy, x, w, block, qtype=I8, grad_qtype=I8, precision=64, want_dx=True,
               want_dw=True, signs_n=None, signs_m=None, grad_rounding=RNE, key=(0, 0),
               ctr_hi=(0, 0)):
    """dX = dY . W (rotated along N), dW = dY^T . X (rotated along M), fp64.

    signs_n / signs_m: the randomised transform's sign words along N / M.  grad_rounding:
    rounding of the dY codes (STOCHASTIC: Philox key ``key``; counter words 2-3 ``ctr_hi`` for
    the rows of dY and ``(ctr_hi[0], ctr_hi[1] ^ 2^31)`` for its columns)."""
    dy = np.ascontiguousarray(dy)
    x = np.ascontiguousarray(x)
    w = np.ascontiguousarray(w)
    assert dy.dtype == x.dtype == w.dtype
    m, k = x.shape
    n = w.shape[0]
    dx = np.empty((m, k), dtype=np.float64) if want_dx else None
    dw = np.empty((n, k), dtype=np.float64) if want_dw else None
    sn = _u32(signs_n, -(-padded_len(n, block) // 32))
    sm = _u32(signs_m, -(-padded_len(m, block) // 32))
    kk, ch = _u32(key, 2), _u32(ctr_hi, 2)
    rc = lib().hor_linear_bwd_ex(_ptr(dy), _ptr(x), _ptr(w), _xtype(x), m, n, k, int(block),
                                 qtype, grad_qtype, int(precision), _ptr(sn), _ptr(sm),
                                 int(grad_rounding), _ptr(kk), _ptr(ch), _ptr(dx), _ptr(dw))
    _check(rc, "linear_bwd")
    return dx, dw
