"""Helpers shared by the GPU parity tests: moving synthetic arrays to the device and back, and
the comparison bars (bit-exact codes against the oracle's fp32 decision, the +-1 budget against
its fp64 decision, relative Frobenius error of layer outputs)."""
import numpy as np
import torch

import oracle as O

DEV = "cuda:0"

Q_TORCH = {O.I8: torch.int8, O.E4M3: torch.float8_e4m3fn, O.E5M2: torch.float8_e5m2,
           O.F64: torch.float32}


def to_dev(a):
    """numpy float32 or uint16 (bf16 bits) -> device tensor of float32 or bfloat16."""
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def codes_to_np(q):
    if q.dtype == torch.int8:
        return q.cpu().numpy()
    if q.dtype in (torch.float8_e4m3fn, torch.float8_e5m2):
        return q.view(torch.uint8).cpu().numpy()
    return q.float().cpu().numpy()


def codes_to_dev(c, qtype):
    if qtype == O.I8:
        return torch.from_numpy(np.ascontiguousarray(c, dtype=np.int8)).to(DEV)
    t = torch.from_numpy(np.ascontiguousarray(c, dtype=np.uint8)).to(DEV)
    return t.view(Q_TORCH[qtype])


def fp8_ordinal(c):
    c = c.astype(np.int32)
    return np.where(c & 0x80, -(c & 0x7F), c & 0x7F)


def code_distance(a, b, qtype):
    if qtype == O.I8:
        return np.abs(a.astype(np.int32) - b.astype(np.int32))
    return np.abs(fp8_ordinal(a) - fp8_ordinal(b))


# FP8 grids: mantissa bits and the exponent of the smallest normal value.
FP8_GRID = {O.E4M3: (3, -6), O.E5M2: (2, -14)}


def fp8_step(t, qtype):
    """Spacing of the FP8 grid at magnitude |t| (in code units; the subnormal spacing below
    the smallest normal)."""
    mb, emin = FP8_GRID[qtype]
    e = np.floor(np.log2(np.maximum(np.abs(t), 2.0 ** emin)))
    return 2.0 ** (e - mb)


def fp32_rotation_code_bound(x, oaxis, block, qtype, opts=None, vec_idx=None):
    """Exact real code values t = y * qmax / a of the oracle's fp64 definition, and an a-priori
    bound e on how far the code value of an fp32 computation (fp32 butterflies, m = fl(qmax /
    a32), fl(y32 * m)) can lie from t.  Each fp32 butterfly output is within
    gamma_k * S of the exact sum (k = log2(block) stages, S = sum of |x| over its block); the
    absmax a32 inherits that error from its own block, which moves m by at most
    gamma_k * S_max / a + u; the product adds u.  Hence, per element,
        |c32 - t| <= gamma_k * S * qmax / a + |t| * (gamma_k * S_max / a + 2 u),
    with a the unnormalised absmax (the 1/sqrt(block) cancels).  vec_idx: only these vectors.
    Returns (t, e)."""
    opts = dict(opts or {})
    opts.pop("rounding", None)
    y, a = O.fwht_quant(x, oaxis, block, O.F64, precision=64, vec_idx=vec_idx, **opts)
    qmax = {O.I8: 127.0, O.E4M3: 448.0, O.E5M2: 57344.0}[qtype]
    xv = np.abs(np.asarray(x, dtype=np.float64))
    if x.dtype == np.uint16:
        import synth
        xv = np.abs(synth.bf16_to_f32(x).astype(np.float64))
    if oaxis == O.COLS:
        xv = xv.T
    if vec_idx is not None:
        xv = xv[np.asarray(vec_idx)]
    nvec, L = xv.shape
    Lp = y.shape[1]
    xp = np.zeros((nvec, Lp))
    xp[:, :L] = xv
    S = xp.reshape(nvec, Lp // block, block).sum(axis=2)               # [nvec, blocks]
    Smax = S.max(axis=1, initial=0.0)
    S_el = np.repeat(S, block, axis=1)                                  # per element
    au = a * np.sqrt(block)                                             # unnormalised absmax
    safe = np.where(au > 0, au, 1.0)
    t = np.where(a[:, None] > 0, y / np.where(a > 0, a, 1.0)[:, None] * qmax, 0.0)
    u = 2.0 ** -24
    k = max(1, int(np.log2(block)))
    g = k * u / (1 - k * u)
    e = (g * S_el * qmax / safe[:, None] + np.abs(t) * (g * Smax / safe + 2 * u)[:, None]) * 1.01
    return t, np.where(a[:, None] > 0, e, 0.0)


def assert_fp8_codes_close_to_exact(gpu_q, x, oaxis, block, qtype, stochastic=False, opts=None,
                                    vec_idx=None):
    """FP8 codes against the exact real code value t of the fp64 definition: the decoded code
    lies within half a grid step (a whole step for stochastic rounding) plus the fp32
    rotation's error bound of t.  This is the code bar read for FP8 codes: where the fp32
    butterflies' rounding (within the FWHT bar) spans more than a grid step -- near zero,
    where the E5M2 subnormal spacing is 2^-16 code units -- the fp32 and fp64 decisions
    legitimately differ by several steps.  The butterflies round for fp32 input, and for bf16
    input too once a block's sums need more than fp32's 24 bits (inputs spanning several
    binades, blocks of thousands)."""
    t, e = fp32_rotation_code_bound(x, oaxis, block, qtype, opts, vec_idx)
    g = fp8_table(qtype)[np.asarray(gpu_q)]
    step = fp8_step(np.abs(t) + e, qtype)
    lim = (step if stochastic else step / 2) + e
    bad = np.abs(g - t) > lim * (1 + 1e-12)
    assert not bad.any(), f"{int(bad.sum())} codes beyond the fp32 bound of the exact value"


def fp8_table(qtype):
    return O.fp8_table(qtype)


def undecidable_in_fp32(t, e, qtype):
    """Codes whose exact value t lies within the fp32 path's error bound e of a rounding
    midpoint (the midpoint between the two grid points around t; exact ties included): any
    fp32 computation within its rounding may round them either way."""
    if qtype == O.I8:
        mid = np.floor(t) + 0.5
    else:
        step = fp8_step(np.abs(t), qtype)
        mid = np.sign(t) * (np.floor(np.abs(t) / step) + 0.5) * step
    return np.abs(t - mid) <= e * (1 + 1e-9)


def assert_codes_close_to_fp64(gpu_q, ref_q, qtype, block, frac=1e-4, x=None, oaxis=None,
                               opts=None, vec_idx=None):
    """Code bar against the fp64 oracle: |dq| <= 1 everywhere and at most
    `frac` of the elements off by one (grid steps for FP8).  The fraction applies to rotated
    data (block >= 16); with block < 16 a bf16 input keeps its 8-bit mantissa, so values
    y * qmax / a that are exact ties in real arithmetic are common and the fp32 and fp64
    decisions legitimately split them -- there only the +-1 bound is checked.  Two flips are
    always allowed: on a few thousand codes one fp32-vs-fp64 split near a rounding midpoint is
    an ordinary event, not a sign of a wrong kernel (those are caught bit-exactly against the
    fp32-decision oracle).  With the input x given (axis oaxis, oracle options opts):
    - FP8 codes: each code is held to the exact value within half a grid step plus the fp32
      rotation's error bound (assert_fp8_codes_close_to_exact) instead of one grid step, for
      fp32 and bf16 input alike (the fp32 butterflies round once a block's sums need more
      than 24 bits, and near zero the FP8 grid is far finer than that rounding);
    - nearest rounding: the fraction counts only codes that fp32 arithmetic can decide, those
      whose exact value lies farther than the fp32 path's error bound from a rounding midpoint
      (undecidable_in_fp32; exact ties are the common case, and on padding-dominated vectors one
      tie repeats across many positions), at every block size."""
    if qtype == O.F64:  # the rotated values themselves: the FWHT bar, per vector
        got = np.asarray(gpu_q, dtype=np.float64)
        err = np.linalg.norm(got - ref_q, axis=1) / np.maximum(np.linalg.norm(ref_q, axis=1),
                                                                1e-300)
        assert err.max(initial=0) <= 1e-5, f"rotated values off by {err.max()} relative"
        return
    d = code_distance(gpu_q, ref_q, qtype)
    sr = bool(opts) and opts.get("rounding") == O.STOCHASTIC
    if x is not None and qtype in FP8_GRID:
        # FP8 codes: each code against the exact value and the fp32 rotation's error bound
        # instead of one grid step (see assert_fp8_codes_close_to_exact)
        assert_fp8_codes_close_to_exact(gpu_q, x, oaxis, block, qtype, sr, opts, vec_idx)
        d = np.minimum(d, 1)
    assert d.max(initial=0) <= 1, f"code off by {d.max()}"
    if x is not None and not sr:
        # with the input at hand, codes that fp32 arithmetic cannot decide (exact value within
        # the fp32 path's error bound of a rounding midpoint) do not count; at every block
        t, e = fp32_rotation_code_bound(x, oaxis, block, qtype, opts, vec_idx)
        n1 = int(((d == 1) & ~undecidable_in_fp32(t, e, qtype)).sum())
        assert n1 <= max(2.0, frac * d.size), f"{n1} of {d.size} decidable codes off by one"
    elif block >= 16:
        n1 = int((d == 1).sum())
        assert n1 <= max(2.0, frac * d.size), f"{n1} of {d.size} codes off by one"


def scales_close_to_fp64(gpu_s, ref_s, rtol=1e-5):
    """Scale bar against the fp64 oracle: within rtol relative, or within the fp32 subnormal
    quantum where the stored fp32 scale is itself subnormal."""
    gpu_s = np.asarray(gpu_s, dtype=np.float64)
    ok = np.abs(gpu_s - ref_s) <= rtol * np.abs(ref_s) + 2.0 ** -149
    assert ok.all(), f"{int((~ok).sum())} scales off the fp64 oracle by more than {rtol}"


def check_fq_parity(got_q, got_s, x, oaxis, block, qtype, vec_idx=None, **opts):
    """Both bars of a rotation pass against the oracle: codes and scales bit-exact to its
    fp32 decision, and within the code bar of its plain fp64 definition (|dq| <= 1 on
    at most 1e-4 of the codes, scales within 1e-5 relative).  opts: the oracle's signs /
    rounding / key / ctr_hi."""
    got_s = np.asarray(got_s, dtype=np.float64)
    r32, s32 = O.fwht_quant(x, oaxis, block, qtype, precision=32, vec_idx=vec_idx, **opts)
    assert np.array_equal(got_q, r32), \
        f"{int((got_q != r32).sum())} codes differ from the fp32 decision"
    assert np.array_equal(got_s, s32), f"{int((got_s != s32).sum())} scales differ"
    r64, s64 = O.fwht_quant(x, oaxis, block, qtype, precision=64, vec_idx=vec_idx, **opts)
    if qtype == O.F64:
        err = np.linalg.norm(got_q - r64, axis=1) / np.maximum(np.linalg.norm(r64, axis=1), 1e-300)
        assert err.max(initial=0) <= 1e-5
        scales_close_to_fp64(got_s, s64)
        return
    assert_codes_close_to_fp64(got_q, r64, qtype, block, x=x, oaxis=oaxis, opts=opts,
                               vec_idx=vec_idx)
    scales_close_to_fp64(got_s, s64)


# Accumulation of the gfx950 FP8 matrix cores (v_mfma_*_f8f6f4), measured with in-bounds
# probes: the products of 8 consecutive k are summed in fixed point aligned to the largest
# of them (about 15 bits below its leading bit are kept, lower bits dropped), and those group
# sums are accumulated in fp32 with round-to-nearest-even.  Hence, per output element,
#   |acc - exact| <= 2^-10 * sum_groups max|p| + gamma_{k/8+2} * sum |p|
#                 <= (2^-10 + gamma_{k/8+2}) * sum |p|,   gamma_n = n u / (1 - n u), u = 2^-24.
FP8_GROUP_REL = 2.0 ** -10


def fp8_acc_bound(absum, k):
    u = 2.0 ** -24
    n = k / 8 + 2
    return (FP8_GROUP_REL + n * u / (1 - n * u)) * absum


def padded_out(m, n, dtype, device=DEV):
    """An [m x n] output view whose rows start 16-byte aligned (leading dim padded)."""
    es = torch.tensor([], dtype=dtype).element_size()
    per = 16 // es
    ld = max(per, (n + per - 1) // per * per)
    return torch.empty((m, ld), dtype=dtype, device=device)[:, :n]


def rel_fro(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (den if den > 0 else 1.0)


# Philox key and counter words 2-3 of the stochastic-rounding tests, as the oracle takes them
# and as the binding's 64-bit seed / counter
KEY, CTR = (0x3C6EF372, 0xA54FF53A), (0x510E527F, 0x9B05688C)
SEED64 = KEY[0] | (KEY[1] << 32)
COUNTER64 = CTR[0] | (CTR[1] << 32)


def signs_dev(words):
    """Packed sign words (uint32) as the int32 device tensor the binding takes."""
    return torch.from_numpy(np.ascontiguousarray(words).view(np.int32)).to(DEV)


def fp8_extra(a, aax, at, b, bax, bt, block, aopt=None, bopt=None):
    """Accumulation bound of the FP8 matrix cores for the product of the oracle's codes of
    operand a (vectors along axis aax, options aopt) and operand b, in output units."""
    qa, sa = O.fwht_quant(a, aax, block, at, precision=32, **(aopt or {}))
    qb, sb = O.fwht_quant(b, bax, block, bt, precision=32, **(bopt or {}))
    absum = O.matmul_f64(np.abs(O.fp8_table(at)[qa]), np.abs(O.fp8_table(bt)[qb]))
    return fp8_acc_bound(absum, qa.shape[1]) * np.outer(sa, sb) * (1 + 1e-6)


def bound_ok(got, ref, rel, extra=0.0):
    """Elementwise |got - ref| <= rel |ref| (+ a floor of 1e-6 max |ref|) + extra; returns
    (all within, number outside)."""
    scale = np.abs(ref) + 1e-6 * np.abs(ref).max()
    bad = np.abs(got - ref) > rel * scale + extra
    return not bad.any(), int(bad.sum())


def to_np64(t):
    return t.float().cpu().numpy().astype(np.float64)


def random_rotation_case(case):
    """Seeded random rotation pass number `case`: random valid sizes, block, code type, input
    type, signs and rounding, all drawn from its own generator (the GPU random-shape test and
    the CPU bar tests replay the same cases).  Returns a dict with axis (0 rows, 1 columns),
    io, qt, block, rows, cols, sr, words (sign words or None) and x (bf16 bits or fp32)."""
    import synth
    rng = np.random.default_rng(5000 + case)
    axis = int(rng.integers(0, 2))
    io = synth.BF16 if rng.random() < 0.75 else synth.F32
    qt = (O.I8, O.E4M3, O.E5M2)[int(rng.integers(0, 3))]
    b = 1 << int(rng.integers(0, 13))
    # sizes the library takes: lengths and code rows in whole 16-byte units
    if axis == 0:
        rows, cols = int(rng.integers(1, 300)), 16 * int(rng.integers(1, 350))
    else:
        long_cols = rng.random() < 0.3  # columns longer than 4096: partial maxima exchanged
        rows = 16 * int(rng.integers(257, 560) if long_cols else rng.integers(1, 120))
        cols = 8 * int(rng.integers(1, 40 if long_cols else 120))
    signs, sr = rng.random() < 0.4, rng.random() < 0.3
    L = cols if axis == 0 else rows
    words = synth.sign_words(O.padded_len(L, b), seed=case) if signs else None
    a = synth.activations(rng, rows, cols)
    x = synth.bf16_bits(a) if io == synth.BF16 else a
    return dict(axis=axis, io=io, qt=qt, block=b, rows=rows, cols=cols, sr=sr, words=words, x=x)
