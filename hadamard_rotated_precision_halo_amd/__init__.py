"""Python binding of libhalo.so, the MI355X Hadamard-rotated low-precision linear layer.

Argument marshalling only: torch tensors supply device pointers and the current HIP stream;
every step of the computation runs in the library's gfx950 kernels.  The library must be
built (``python -m hadamard_rotated_precision_halo_amd.build``); importing the functions below
without it raises immediately -- there is no fallback path.

Method: "HALO: Hadamard-Assisted Lower-Precision Optimization for LLMs" (abstract: rotations
in the forward and backward pass, all large products in 8 bits; key design 2: INT8 or FP8),
with the orthonormal Walsh-Hadamard transform and absmax quantiser of
"QWHA方法：基于Walsh-Hadamard变换的高效大模型微调技术" s2.1-s2.2, applied blockwise (s3.1), with
the zero padding and stochastic rounding of its s5, and the seeded randomised transform H D of
"企业官网建设流程全解析" s4.2.
"""
import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libhalo.so")

# halo_dtype / halo_axis / halo_status values of include/halo.h
F32, BF16, I8, E4M3, E5M2, I32 = range(6)
ROWS, COLS = 0, 1
NEAREST, STOCHASTIC = 0, 1  # halo_rounding
NOALLOC_SCRATCH_BYTES = 1 << 20  # HALO_NOALLOC_SCRATCH_BYTES
STATUS = {0: "HALO_OK", 1: "HALO_ERR_NULL", 2: "HALO_ERR_SHAPE", 3: "HALO_ERR_BLOCK",
          4: "HALO_ERR_DTYPE", 5: "HALO_ERR_ALIGN", 6: "HALO_ERR_WORKSPACE", 7: "HALO_ERR_HIP",
          8: "HALO_ERR_OPTION"}

EXPORTS = ("halo_fwht_quant", "halo_fwht_quant_ex", "halo_fwht_quant_noalloc",
           "halo_fwht_quant_workspace_bytes",
           "halo_gemm_i8", "halo_gemm_fp8", "halo_linear_workspace_bytes",
           "halo_linear_workspace_bytes_ex", "halo_linear_fwd", "halo_linear_fwd_ex",
           "halo_linear_bwd", "halo_linear_bwd_ex", "halo_fwht_quant_dual",
           "halo_fwht_quant_dual_workspace_bytes", "halo_mfma_rate_probe", "halo_status_str")


class QuantOpts(ctypes.Structure):
    """halo_quant_opts of include/halo.h."""
    _fields_ = [("signs", ctypes.c_void_p), ("rounding", ctypes.c_int32),
                ("seed", ctypes.c_uint32 * 2), ("counter", ctypes.c_uint32 * 2),
                ("exchange_polls", ctypes.c_uint32)]


class LinearOpts(ctypes.Structure):
    """halo_linear_opts of include/halo.h."""
    _fields_ = [("signs_k", ctypes.c_void_p), ("signs_n", ctypes.c_void_p),
                ("signs_m", ctypes.c_void_p), ("grad_rounding", ctypes.c_int32),
                ("seed", ctypes.c_uint32 * 2), ("counter", ctypes.c_uint32 * 2),
                ("exchange_polls", ctypes.c_uint32)]

_TORCH_CODE = {torch.float32: F32, torch.bfloat16: BF16, torch.int8: I8,
               torch.float8_e4m3fn: E4M3, torch.float8_e5m2: E5M2, torch.int32: I32}


class HaloError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)} ({_status_str(status)})")


_lib = None


def lib():
    """The loaded libhalo.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run "
                              "`python -m hadamard_rotated_precision_halo_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        i64, vp, i32, sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        e = ctypes.c_int  # enums
        L.halo_fwht_quant.argtypes = [vp, e, i64, i64, i64, e, i32, e, vp, i64, vp, vp, sz, vp]
        L.halo_fwht_quant_workspace_bytes.argtypes = [i64, i64, e, i32, e]
        L.halo_fwht_quant_workspace_bytes.restype = sz
        L.halo_gemm_i8.argtypes = [vp, i64, vp, vp, i64, vp, i64, i64, i64, vp, e, i64, vp]
        L.halo_gemm_fp8.argtypes = [vp, e, i64, vp, vp, e, i64, vp, i64, i64, i64, vp, e, i64, vp]
        L.halo_linear_workspace_bytes.argtypes = [i64, i64, i64, e, ctypes.c_int]
        L.halo_linear_workspace_bytes.restype = sz
        L.halo_linear_fwd.argtypes = [vp, vp, e, i64, i64, i64, i32, e, vp, e, vp, sz, vp]
        L.halo_linear_bwd.argtypes = [vp, vp, vp, e, i64, i64, i64, i32, e, e, vp, vp, vp, sz, vp]
        qo, lo = ctypes.POINTER(QuantOpts), ctypes.POINTER(LinearOpts)
        L.halo_fwht_quant_ex.argtypes = [vp, e, i64, i64, i64, e, i32, e, vp, i64, vp, qo, vp, sz,
                                         vp]
        L.halo_fwht_quant_noalloc.argtypes = [vp, e, i64, i64, i64, e, i32, e, vp, i64, vp, qo,
                                              vp]
        L.halo_linear_workspace_bytes_ex.argtypes = [i64, i64, i64, i32, e, ctypes.c_int]
        L.halo_linear_workspace_bytes_ex.restype = sz
        L.halo_linear_fwd_ex.argtypes = [vp, vp, e, i64, i64, i64, i32, e, vp, e, lo, vp, sz, vp]
        L.halo_linear_bwd_ex.argtypes = [vp, vp, vp, e, i64, i64, i64, i32, e, e, vp, vp, lo, vp,
                                         sz, vp]
        L.halo_mfma_rate_probe.argtypes = [i32, i32, ctypes.POINTER(ctypes.c_int64), vp]
        L.halo_fwht_quant_dual_workspace_bytes.argtypes = [i64, i64, i32, e]
        L.halo_fwht_quant_dual_workspace_bytes.restype = sz
        L.halo_fwht_quant_dual.argtypes = [vp, e, i64, i64, i64, i32, e, vp, i64, vp, vp, i64, vp,
                                           qo, qo, vp, sz, vp]
        L.halo_status_str.argtypes = [e]
        L.halo_status_str.restype = ctypes.c_char_p
        for f in ("halo_fwht_quant", "halo_fwht_quant_ex", "halo_fwht_quant_noalloc",
                  "halo_gemm_i8", "halo_gemm_fp8",
                  "halo_linear_fwd", "halo_linear_fwd_ex", "halo_linear_bwd",
                  "halo_linear_bwd_ex", "halo_fwht_quant_dual", "halo_mfma_rate_probe"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def _status_str(s):
    try:
        return lib().halo_status_str(int(s)).decode()
    except Exception:  # pragma: no cover
        return "?"


def _code(dtype):
    try:
        return _TORCH_CODE[dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {dtype}") from None


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(status, what):
    if status != 0:
        raise HaloError(status, what)


def _ld(t):
    assert t.dim() == 2, "matrices are 2-D"
    if t.numel() == 0:  # an empty matrix has no meaningful stride; any aligned value works
        return max(t.shape[1], 16)
    assert t.stride(1) == 1, "matrices must be row-major with unit column stride"
    return t.stride(0)


def _require(cond, msg):
    if not cond:
        raise ValueError(msg)


def _matrix(t, name, shape, dtype=None, contiguous=False):
    """A 2-D matrix argument of exactly `shape` (and `dtype`): row-major with unit column stride
    and a row stride of at least its width, or contiguous for the layer calls, which take no
    leading dimension.  The kernels trust the shapes the call passes: a tensor smaller than
    that would be read or written past its end."""
    _require(isinstance(t, torch.Tensor) and t.dim() == 2, f"{name} must be a 2-D tensor")
    _require(tuple(t.shape) == tuple(shape),
             f"{name} has shape {tuple(t.shape)}, the call needs {tuple(shape)}")
    if dtype is not None:
        _require(t.dtype == dtype, f"{name} has dtype {t.dtype}, the call needs {dtype}")
    if contiguous:
        _require(t.is_contiguous(), f"{name} must be contiguous (row-major, no row padding)")
    elif t.numel() > 0:
        _require(t.stride(1) == 1 and t.stride(0) >= t.shape[1],
                 f"{name} must be row-major with unit column stride")


def _vector(t, name, n, dtype):
    """A contiguous 1-D argument of at least n entries of dtype."""
    _require(isinstance(t, torch.Tensor) and t.dim() == 1 and t.dtype == dtype
             and t.is_contiguous() and t.numel() >= n,
             f"{name} must be a contiguous 1-D {dtype} tensor of at least {n} entries")


def _bytes(t, name):
    """A workspace: a contiguous 1-D uint8 tensor (its size is checked by the library)."""
    _require(isinstance(t, torch.Tensor) and t.dim() == 1 and t.dtype == torch.uint8
             and t.is_contiguous(), f"{name} must be a contiguous 1-D uint8 tensor")


def _same_gpu(ref, **tensors):
    """The reference input on a GPU and every other tensor argument on the same device."""
    _require(isinstance(ref, torch.Tensor) and ref.is_cuda, "the inputs must be GPU tensors")
    for name, t in tensors.items():
        if t is not None:
            _require(t.device == ref.device, f"{name} is on {t.device}, the inputs on {ref.device}")


def _sign_words(length):
    return -(-int(length) // 32)


def contraction_len(dim, block):
    """Contraction length of a layer product: the dimension padded with zeros to a multiple of
    the block and of 32; a layer call's sign array covers this length."""
    step = max(int(block), 32)
    return -(-int(dim) // step) * step


def padded_len(length, block):
    """Rotated length of a vector of `length` elements: rounded up to a multiple of block
    (the zero padding)."""
    return -(-int(length) // int(block)) * int(block)


def hadamard_signs(length, seed, device=None):
    """Packed random signs of the randomised transform H D for vectors of `length` elements:
    ceil(length / 32) 32-bit words (bit i set = element i negated), drawn on the host from
    `seed`, so every process that uses the same seed gets the same transform.  Returned as an
    int32 tensor (the words' bit patterns) on `device`."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    words = torch.randint(-(2 ** 31), 2 ** 31, (-(-int(length) // 32),), dtype=torch.int32,
                          generator=g)
    return words.to(device) if device is not None else words


def _u32x2(v):
    v = int(v)
    return (ctypes.c_uint32 * 2)(v & 0xFFFFFFFF, (v >> 32) & 0xFFFFFFFF)


_ROUNDING = {"nearest": NEAREST, "stochastic": STOCHASTIC, NEAREST: NEAREST,
             STOCHASTIC: STOCHASTIC}


def _rounding(r):
    try:
        return _ROUNDING[r]
    except KeyError:
        raise ValueError(f"rounding must be 'nearest' or 'stochastic', not {r!r}") from None


def fwht_quant_workspace_bytes(rows, cols, axis, block, x_dtype=torch.bfloat16):
    return int(lib().halo_fwht_quant_workspace_bytes(rows, cols, axis, int(block),
                                                     _code(x_dtype)))


def fwht_quant(x, axis=ROWS, block=256, q_dtype=torch.int8, q=None, scale=None, workspace=None,
               stream=None, signs=None, rounding="nearest", seed=0, counter=0,
               exchange_polls=0):
    """Rotate + quantise the rows (axis ROWS) or columns (axis COLS) of x.

    Returns (q, scale): q is [rows x Lp] (ROWS) or [cols x Lp] (COLS) of q_dtype
    (torch.int8 / float8_e4m3fn / float8_e5m2, or torch.float32 for the rotated values
    themselves), Lp the vector length padded with zeros to a multiple of block; scale is
    float32 with one entry per vector.  `workspace` is the optional scratch of the single-read
    columns pass: a uint8 device tensor, allocated here when None and the shape can use one;
    pass False to run without it.  `signs`: the randomised transform's packed sign words (an
    int32 device tensor, see hadamard_signs) or None.  `rounding`: "nearest" or "stochastic"
    (Philox key `seed`, counter words 2-3 `counter`, each a 64-bit integer).
    `exchange_polls`: for columns longer than 4096 rows, the polls a waiting workgroup makes
    before it stops waiting (the strip is then stored by a follow-up launch, with the same
    codes); 0 = the library's default.
    """
    _require(isinstance(x, torch.Tensor) and x.dim() == 2, "x must be a 2-D tensor")
    rows, cols = x.shape
    nvec, L = (rows, cols) if axis == ROWS else (cols, rows)
    Lp = padded_len(L, block)
    if q is None:
        q = torch.empty((nvec, Lp), dtype=q_dtype, device=x.device)
    _matrix(q, "q", (nvec, Lp))
    if scale is None:
        scale = torch.empty(nvec, dtype=torch.float32, device=x.device)
    _vector(scale, "scale", nvec, torch.float32)
    if signs is not None:
        _vector(signs, "signs", _sign_words(Lp), torch.int32)
    if workspace is not None and workspace is not False:
        _bytes(workspace, "workspace")
    _same_gpu(x, q=q, scale=scale, signs=signs,
              workspace=workspace if workspace is not False else None)
    if workspace is False:
        ws_ptr, ws_bytes = None, 0
    else:
        need = fwht_quant_workspace_bytes(rows, cols, axis, block, x.dtype)
        if workspace is None and need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
        if workspace is None:
            ws_ptr, ws_bytes = None, 0
        else:
            ws_ptr, ws_bytes = _ptr(workspace), workspace.numel()
    opts = None
    rnd = _rounding(rounding)
    if signs is not None or rnd != NEAREST or exchange_polls:
        opts = QuantOpts(_ptr(signs), rnd, _u32x2(seed), _u32x2(counter), int(exchange_polls))
    st = lib().halo_fwht_quant_ex(_ptr(x), _code(x.dtype), rows, cols, _ld(x), axis, int(block),
                                  _code(q.dtype), _ptr(q), _ld(q), _ptr(scale),
                                  ctypes.byref(opts) if opts is not None else None, ws_ptr,
                                  ws_bytes, _stream(stream))
    _check(st, "halo_fwht_quant_ex")
    return q, scale


def fwht_quant_dual_workspace_bytes(rows, cols, block, x_dtype=torch.bfloat16):
    return int(lib().halo_fwht_quant_dual_workspace_bytes(int(rows), int(cols), int(block),
                                                          _code(x_dtype)))


def _quant_opts(signs, rounding, seed, counter, exchange_polls):
    rnd = _rounding(rounding)
    if signs is None and rnd == NEAREST and not exchange_polls:
        return None
    return QuantOpts(_ptr(signs), rnd, _u32x2(seed), _u32x2(counter), int(exchange_polls))


def fwht_quant_dual(x, block=256, q_dtype=torch.int8, qr=None, scale_r=None, qc=None,
                    scale_c=None, workspace=None, stream=None, row_signs=None, col_signs=None,
                    rounding="nearest", seed=0, row_counter=0, col_counter=0, exchange_polls=0):
    """Both passes of x from one read where the shape allows (halo_fwht_quant_dual): returns
    (qr, scale_r, qc, scale_c), the codes and scales of fwht_quant along the rows and along
    the columns.  `row_signs` / `col_signs`: each pass's sign words (along the columns of a row
    / the rows of a column); `rounding`, `seed`, the counters and `exchange_polls` as in
    fwht_quant (the counter of each pass its own).  `workspace`: the scratch, allocated here
    when None; False runs without it."""
    _require(isinstance(x, torch.Tensor) and x.dim() == 2, "x must be a 2-D tensor")
    rows, cols = x.shape
    if qr is None:
        qr = torch.empty((rows, padded_len(cols, block)), dtype=q_dtype, device=x.device)
    if scale_r is None:
        scale_r = torch.empty(rows, dtype=torch.float32, device=x.device)
    if qc is None:
        qc = torch.empty((cols, padded_len(rows, block)), dtype=q_dtype, device=x.device)
    if scale_c is None:
        scale_c = torch.empty(cols, dtype=torch.float32, device=x.device)
    _matrix(qr, "qr", (rows, padded_len(cols, block)), dtype=q_dtype)
    _matrix(qc, "qc", (cols, padded_len(rows, block)), dtype=q_dtype)
    _vector(scale_r, "scale_r", rows, torch.float32)
    _vector(scale_c, "scale_c", cols, torch.float32)
    if row_signs is not None:
        _vector(row_signs, "row_signs", _sign_words(padded_len(cols, block)), torch.int32)
    if col_signs is not None:
        _vector(col_signs, "col_signs", _sign_words(padded_len(rows, block)), torch.int32)
    if workspace is not None and workspace is not False:
        _bytes(workspace, "workspace")
    _same_gpu(x, qr=qr, qc=qc, scale_r=scale_r, scale_c=scale_c, row_signs=row_signs,
              col_signs=col_signs, workspace=workspace if workspace is not False else None)
    if workspace is False:
        ws_ptr, ws_bytes = None, 0
    else:
        need = fwht_quant_dual_workspace_bytes(rows, cols, block, x.dtype)
        if workspace is None and need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
        ws_ptr, ws_bytes = (None, 0) if workspace is None else (_ptr(workspace),
                                                                workspace.numel())
    ro = _quant_opts(row_signs, rounding, seed, row_counter, exchange_polls)
    co = _quant_opts(col_signs, rounding, seed, col_counter, exchange_polls)
    st = lib().halo_fwht_quant_dual(_ptr(x), _code(x.dtype), rows, cols, _ld(x), int(block),
                                    _code(q_dtype), _ptr(qr), _ld(qr), _ptr(scale_r), _ptr(qc),
                                    _ld(qc), _ptr(scale_c),
                                    ctypes.byref(ro) if ro is not None else None,
                                    ctypes.byref(co) if co is not None else None, ws_ptr,
                                    ws_bytes, _stream(stream))
    _check(st, "halo_fwht_quant_dual")
    return qr, scale_r, qc, scale_c


MFMA_PROBE_KINDS = {0: "v_mfma_i32_32x32x32_i8", 1: "v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3)",
                    2: "v_mfma_scale_f32_16x16x128_f8f6f4 (E4M3)"}


def mfma_rate_probe(kind, iters, stream=None):
    """One launch of the matrix-core rate probe (halo_mfma_rate_probe) on `stream`; returns the
    operations it performs.  A measurement aid: time it with events on the same stream."""
    ops = ctypes.c_int64(0)
    _check(lib().halo_mfma_rate_probe(int(kind), int(iters), ctypes.byref(ops), _stream(stream)),
           "halo_mfma_rate_probe")
    return ops.value


def fwht_quant_noalloc(x, q, scale, axis=ROWS, block=256, stream=None, signs=None,
                       rounding="nearest", seed=0, counter=0, exchange_polls=0):
    """fwht_quant into caller-provided q and scale with the library's fixed scratch in place of
    a workspace (halo_fwht_quant_noalloc): nothing is allocated.  Calls that may overlap on one
    device share that scratch and must be ordered by the caller."""
    _require(isinstance(x, torch.Tensor) and x.dim() == 2, "x must be a 2-D tensor")
    rows, cols = x.shape
    nvec, L = (rows, cols) if axis == ROWS else (cols, rows)
    Lp = padded_len(L, block)
    _matrix(q, "q", (nvec, Lp))
    _vector(scale, "scale", nvec, torch.float32)
    if signs is not None:
        _vector(signs, "signs", _sign_words(Lp), torch.int32)
    _same_gpu(x, q=q, scale=scale, signs=signs)
    opts = None
    rnd = _rounding(rounding)
    if signs is not None or rnd != NEAREST or exchange_polls:
        opts = QuantOpts(_ptr(signs), rnd, _u32x2(seed), _u32x2(counter), int(exchange_polls))
    st = lib().halo_fwht_quant_noalloc(_ptr(x), _code(x.dtype), rows, cols, _ld(x), axis,
                                       int(block), _code(q.dtype), _ptr(q), _ld(q), _ptr(scale),
                                       ctypes.byref(opts) if opts is not None else None,
                                       _stream(stream))
    _check(st, "halo_fwht_quant_noalloc")
    return q, scale


def gemm_i8(a, sa, b, sb, out_dtype=torch.bfloat16, c=None, stream=None):
    """c = (a . b^T) * sa[:, None] * sb[None, :] with int8 codes (int32 raw if out is int32)."""
    _require(isinstance(a, torch.Tensor) and a.dim() == 2 and isinstance(b, torch.Tensor)
             and b.dim() == 2, "a and b must be 2-D tensors")
    m, k = a.shape
    n = b.shape[0]
    _matrix(b, "b", (n, k))
    if c is None:
        c = torch.empty((m, n), dtype=out_dtype, device=a.device)
    _matrix(c, "c", (m, n))
    if c.dtype != torch.int32:  # the raw int32 output takes no scales
        _vector(sa, "sa", m, torch.float32)
        _vector(sb, "sb", n, torch.float32)
    _same_gpu(a, b=b, c=c, sa=sa, sb=sb)
    st = lib().halo_gemm_i8(_ptr(a), _ld(a), _ptr(sa), _ptr(b), _ld(b), _ptr(sb), m, n, k,
                            _ptr(c), _code(c.dtype), _ld(c), _stream(stream))
    _check(st, "halo_gemm_i8")
    return c


def gemm_fp8(a, sa, b, sb, out_dtype=torch.bfloat16, c=None, stream=None):
    """c = (dec(a) . dec(b)^T) * sa[:, None] * sb[None, :] with fp8 codes (E4M3 / E5M2)."""
    _require(isinstance(a, torch.Tensor) and a.dim() == 2 and isinstance(b, torch.Tensor)
             and b.dim() == 2, "a and b must be 2-D tensors")
    m, k = a.shape
    n = b.shape[0]
    _matrix(b, "b", (n, k))
    if c is None:
        c = torch.empty((m, n), dtype=out_dtype, device=a.device)
    _matrix(c, "c", (m, n))
    if c.dtype != torch.int32:  # the raw int32 output takes no scales
        _vector(sa, "sa", m, torch.float32)
        _vector(sb, "sb", n, torch.float32)
    _same_gpu(a, b=b, c=c, sa=sa, sb=sb)
    st = lib().halo_gemm_fp8(_ptr(a), _code(a.dtype), _ld(a), _ptr(sa), _ptr(b), _code(b.dtype),
                             _ld(b), _ptr(sb), m, n, k, _ptr(c), _code(c.dtype), _ld(c),
                             _stream(stream))
    _check(st, "halo_gemm_fp8")
    return c


def linear_workspace_bytes(m, n, k, q_dtype=torch.int8, backward=False, block=None):
    """Workspace bytes of the layer calls: for one block size, or for every block (None)."""
    if block is None:
        return int(lib().halo_linear_workspace_bytes(m, n, k, _code(q_dtype),
                                                     1 if backward else 0))
    return int(lib().halo_linear_workspace_bytes_ex(m, n, k, int(block), _code(q_dtype),
                                                    1 if backward else 0))


def _workspace(nbytes, device, ws):
    if ws is None:
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
    return ws


def linear_fwd(x, w, block, q_dtype=torch.int8, y=None, y_dtype=None, workspace=None,
               stream=None, signs_k=None):
    """Y = X W^T with both operands rotated and quantised along K (the layer's forward);
    signs_k: the randomised transform's sign words along K (see hadamard_signs) or None."""
    _require(isinstance(x, torch.Tensor) and x.dim() == 2 and isinstance(w, torch.Tensor)
             and w.dim() == 2, "x and w must be 2-D tensors")
    m, k = x.shape
    n = w.shape[0]
    _matrix(x, "x", (m, k), contiguous=True)
    _matrix(w, "w", (n, k), dtype=x.dtype, contiguous=True)
    if y is None:
        y = torch.empty((m, n), dtype=y_dtype or x.dtype, device=x.device)
    _matrix(y, "y", (m, n), contiguous=True)
    if signs_k is not None:
        _vector(signs_k, "signs_k", _sign_words(contraction_len(k, block)), torch.int32)
    if workspace is not None:
        _bytes(workspace, "workspace")
    _same_gpu(x, w=w, y=y, signs_k=signs_k, workspace=workspace)
    need = linear_workspace_bytes(m, n, k, q_dtype, False, block)
    ws = _workspace(need, x.device, workspace)
    opts = LinearOpts(_ptr(signs_k), None, None, NEAREST) if signs_k is not None else None
    st = lib().halo_linear_fwd_ex(_ptr(x), _ptr(w), _code(x.dtype), m, n, k, int(block),
                                  _code(q_dtype), _ptr(y), _code(y.dtype),
                                  ctypes.byref(opts) if opts is not None else None, _ptr(ws),
                                  ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "halo_linear_fwd_ex")
    return y


def linear_bwd(dy, x, w, block, q_dtype=torch.int8, grad_q_dtype=None, want_dx=True,
               want_dw=True, dx=None, dw=None, workspace=None, stream=None, signs_n=None,
               signs_m=None, grad_rounding="nearest", seed=0, counter=0, exchange_polls=0):
    """dX = dY W (rotated along N) and dW = dY^T X (rotated along M), 8-bit products.

    signs_n / signs_m: the randomised transform's sign words along N / M (or None).
    grad_rounding: "nearest" or "stochastic" rounding of the dY codes (Philox key `seed`,
    counter words 2-3 `counter`; the columns of dY draw with counter word 3 ^ 2^31).
    exchange_polls: as in fwht_quant, for the columns along m."""
    _require(all(isinstance(t, torch.Tensor) and t.dim() == 2 for t in (dy, x, w)),
             "dy, x and w must be 2-D tensors")
    m, k = x.shape
    n = w.shape[0]
    _matrix(x, "x", (m, k), contiguous=True)
    _matrix(w, "w", (n, k), dtype=x.dtype, contiguous=True)
    _matrix(dy, "dy", (m, n), dtype=x.dtype, contiguous=True)
    grad_q_dtype = grad_q_dtype or q_dtype
    if want_dx and dx is None:
        dx = torch.empty((m, k), dtype=x.dtype, device=x.device)
    if want_dw and dw is None:
        dw = torch.empty((n, k), dtype=x.dtype, device=x.device)
    if want_dx:
        _matrix(dx, "dx", (m, k), contiguous=True)
    if want_dw:
        _matrix(dw, "dw", (n, k), contiguous=True)
    if signs_n is not None:
        _vector(signs_n, "signs_n", _sign_words(contraction_len(n, block)), torch.int32)
    if signs_m is not None:
        _vector(signs_m, "signs_m", _sign_words(contraction_len(m, block)), torch.int32)
    if workspace is not None:
        _bytes(workspace, "workspace")
    _same_gpu(x, dy=dy, w=w, dx=dx if want_dx else None, dw=dw if want_dw else None,
              signs_n=signs_n, signs_m=signs_m, workspace=workspace)
    need = linear_workspace_bytes(m, n, k, q_dtype, True, block)
    ws = _workspace(need, x.device, workspace)
    rnd = _rounding(grad_rounding)
    opts = None
    if signs_n is not None or signs_m is not None or rnd != NEAREST or exchange_polls:
        opts = LinearOpts(None, _ptr(signs_n), _ptr(signs_m), rnd, _u32x2(seed),
                          _u32x2(counter), int(exchange_polls))
    st = lib().halo_linear_bwd_ex(_ptr(dy), _ptr(x), _ptr(w), _code(x.dtype), m, n, k,
                                  int(block), _code(q_dtype), _code(grad_q_dtype),
                                  _ptr(dx) if want_dx else None, _ptr(dw) if want_dw else None,
                                  ctypes.byref(opts) if opts is not None else None, _ptr(ws),
                                  ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "halo_linear_bwd_ex")
    return (dx if want_dx else None), (dw if want_dw else None)
