"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke check.

This module holds none of the method's arithmetic: it only draws random tensors (numpy
PCG64) with the shapes and value distributions of the layer workloads and rounds them to
bf16 bit patterns.  Both the CPU oracle and the GPU path consume exactly the arrays made
here.

Workloads (LLaMA-family linear layers; the fine-tuning tasks the HALO paper measures are
not named, so these stand in for real layer tensors):
  * activations X  ~ N(0, 1) with a few channels scaled x50, the outlier channels that
    motivate the rotation (HALO paper, abstract): round(0.1% of the K channels), at least one,
    unless a workload states its own count (the 256 x 1024 single forward has 4);
  * weights W      ~ 0.02 * N(0, 1);
  * output grads dY ~ 1e-3 * Student-t(nu = 4) (heavy tailed).
"""
import numpy as np

F32, BF16 = "f32", "bf16"


def bf16_bits(x):
    """Round float32 values to bf16 (nearest even) and return the uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    return r


def bf16_to_f32(bits):
    """Exact float32 values of uint16 bf16 bit patterns."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def outlier_channels(rng, k, frac=1e-3, count=None):
    """Distinct channel indices to scale: `count` of them, else round(frac * k) (at least 1)."""
    n = max(1, int(round(frac * k))) if count is None else int(count)
    return np.sort(rng.choice(k, size=n, replace=False))


def activations(rng, m, k, frac=1e-3, factor=50.0, count=None):
    x = rng.standard_normal((m, k), dtype=np.float32)
    ch = outlier_channels(rng, k, frac, count)
    x[:, ch] *= np.float32(factor)
    return x


def weights(rng, n, k):
    return (np.float32(0.02) * rng.standard_normal((n, k), dtype=np.float32)).astype(np.float32)


def grads(rng, m, n):
    return (1e-3 * rng.standard_t(4.0, size=(m, n))).astype(np.float32)


def sign_words(length, seed):
    """Packed random signs for the randomised transform H D: ceil(length / 32) uint32 words
    drawn from one seed (bit i set = element i negated).  Every party that draws with the same
    seed gets the same signs."""
    rng = np.random.default_rng(seed)
    return rng.integers(0, 2 ** 32, size=-(-int(length) // 32), dtype=np.uint32)


def _cast(a, io):
    return bf16_bits(a) if io == BF16 else np.ascontiguousarray(a, dtype=np.float32)


def layer(m, n, k, seed, io=BF16, with_grad=True, frac=1e-3, outliers=None):
    """X [m x k], W [n x k] and (optionally) dY [m x n], as bf16 bits or float32; `outliers`
    fixes the number of x50 channels of X (None: round(frac * k), at least one)."""
    rng = np.random.default_rng(seed)
    x = activations(rng, m, k, frac, count=outliers)
    w = weights(rng, n, k)
    dy = grads(rng, m, n) if with_grad else None
    return _cast(x, io), _cast(w, io), (_cast(dy, io) if dy is not None else None)


# The five layer workloads: (name, M tokens, N out features, K in features, block,
# io type, operand code type, gradient code type, passes; `outliers`: the stated number of
# x50 channels of X where a workload fixes one).
WORKLOADS = {
    "c1_fwd_256x1024x1024_f32_b1024_i8": dict(m=256, n=1024, k=1024, block=1024, io=F32,
                                              q="i8", gq="i8", fwd=True, bwd=False,
                                              outliers=4),
    "c2_fwd_4096x4096x4096_bf16_b256_i8": dict(m=4096, n=4096, k=4096, block=256, io=BF16,
                                               q="i8", gq="i8", fwd=True, bwd=False),
    "c3_bwd_4096x4096x4096_bf16_b256_i8": dict(m=4096, n=4096, k=4096, block=256, io=BF16,
                                               q="i8", gq="i8", fwd=False, bwd=True),
    "c4_fwdbwd_8192x4096x11008_bf16_b128_i8": dict(m=8192, n=4096, k=11008, block=128, io=BF16,
                                                   q="i8", gq="i8", fwd=True, bwd=True),
    "c5_fwdbwd_16384x14336x4096_bf16_b512_fp8": dict(m=16384, n=14336, k=4096, block=512,
                                                     io=BF16, q="e4m3", gq="e5m2", fwd=True,
                                                     bwd=True),
    # the 4096^3 backward again with one block over the whole 4096-long contraction
    "c3_bwd_4096x4096x4096_bf16_b4096_i8": dict(m=4096, n=4096, k=4096, block=4096, io=BF16,
                                                q="i8", gq="i8", fwd=False, bwd=True),
}
SEEDS = {name: 1000 + i for i, name in enumerate(WORKLOADS)}
SEEDS["c3_bwd_4096x4096x4096_bf16_b4096_i8"] = SEEDS["c3_bwd_4096x4096x4096_bf16_b256_i8"]


def workload(name, with_grad=None):
    cfg = WORKLOADS[name]
    g = cfg["bwd"] if with_grad is None else with_grad
    x, w, dy = layer(cfg["m"], cfg["n"], cfg["k"], SEEDS[name], cfg["io"], with_grad=g,
                     outliers=cfg.get("outliers"))
    return cfg, x, w, dy
