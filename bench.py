"""Benchmark of the Hadamard-rotated INT8 linear layer on one MI355X.

One step = halo_linear_fwd + halo_linear_bwd of a 4096 x 4096 layer over 4096 tokens (bf16
inputs, INT8 codes, rotation block 256): six rotation + quantisation passes (rows of X and W;
rows of dY and columns of W; columns of dY and of X) and three INT8 GEMMs (Y, dX, dW) --
every kernel of the hot path.  The headline value is the effective throughput: the three
8-bit GEMMs' algorithmic work (3 * 2 * 4096^3 operations) divided by the wall time of the
whole step, rotations included.

Inputs are synthetic (synth.layer: N(0,1) activations with 0.1% outlier channels x50, weights
0.02 * N(0,1), Student-t(4) * 1e-3 gradients), already resident in HBM.  Several input sets
rotate from step to step so that no operand stays in the 256 MB Infinity Cache.

Per-kernel figures are measured in the same run with HIP events on the launch stream: the
INT8 GEMM (the dominant kernel, MFMA-bound) and the rows / columns rotation passes
(HBM-bound).  The CPU baseline times the oracle on a bounded sample of the same step.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "HALO linear fwd+bwd effective TOP/s + FWHT-quant GB/s (% roofline), 4096x4096"
PEAK_INT8_TOPS = 5000.0   # MI355X dense INT8 MFMA, TOP/s
PEAK_HBM_GBS = 8000.0     # MI355X HBM3E, GB/s
M = N = K = 4096
BLOCK = 256
N_SETS = 6                # 6 x (X, W, dY) bf16 = 576 MB > 256 MB Infinity Cache
STEP_GOP = 3 * 2 * M * N * K / 1e9
KERNEL_SOURCES = ["hadamard_rotated_precision_halo_amd/csrc/gemm.hip",
                  "hadamard_rotated_precision_halo_amd/csrc/fwht_quant.hip",
                  "hadamard_rotated_precision_halo_amd/csrc/fwht_rows.hip",
                  "hadamard_rotated_precision_halo_amd/csrc/halo_device.h"]


def source_hash(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel_key):
    """Counter-derived HBM bytes per launch from a committed rocprofv3 summary, or None if the
    kernels changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic_4096.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("kernel_source_hash") != source_hash(KERNEL_SOURCES):
        return None
    return d.get("bytes_per_launch", {}).get(kernel_key)


def to_dev(a, torch):
    return torch.from_numpy(a.view(np.int16)).to("cuda:0").view(torch.bfloat16)


def time_events(fn, iters, torch):
    """Average duration (ms) of fn() over `iters` back-to-back launches on the current stream."""
    st = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for i in range(iters):
        fn(i)
    e1.record(st)
    e1.synchronize()
    return e0.elapsed_time(e1) / iters


def cpu_baseline():
    """The oracle (plain C, fp64/int64, OpenMP over vectors and rows) on a bounded sample of
    one step: all six rotation passes at full size, and each of the three products on a
    128-row slab of its output, scaled linearly to the full product."""
    import oracle as O
    import synth
    x, w, dy = synth.layer(M, N, K, seed=1001)
    slab = 128
    t_fq = t_gemm = 0.0
    t0 = time.perf_counter()
    # forward: rows of X and W along K
    a = time.perf_counter()
    qx, sx = O.fwht_quant(x, O.ROWS, BLOCK, O.I8)
    qw, sw = O.fwht_quant(w, O.ROWS, BLOCK, O.I8)
    b = time.perf_counter()
    acc = O.gemm_i8(qx[:slab], qw)
    O.dequant(acc.astype(np.float64), sx[:slab], sw)
    c = time.perf_counter()
    t_fq += b - a
    t_gemm += (c - b) * (M / slab)
    # dX: rows of dY along N, columns of W along N
    a = time.perf_counter()
    qd, sd = O.fwht_quant(dy, O.ROWS, BLOCK, O.I8)
    qwt, swt = O.fwht_quant(w, O.COLS, BLOCK, O.I8)
    b = time.perf_counter()
    acc = O.gemm_i8(qd[:slab], qwt)
    O.dequant(acc.astype(np.float64), sd[:slab], swt)
    c = time.perf_counter()
    t_fq += b - a
    t_gemm += (c - b) * (M / slab)
    # dW: columns of dY and of X along M
    a = time.perf_counter()
    qdt, sdt = O.fwht_quant(dy, O.COLS, BLOCK, O.I8)
    qxt, sxt = O.fwht_quant(x, O.COLS, BLOCK, O.I8)
    b = time.perf_counter()
    acc = O.gemm_i8(qdt[:slab], qxt)
    O.dequant(acc.astype(np.float64), sdt[:slab], sxt)
    c = time.perf_counter()
    t_fq += b - a
    t_gemm += (c - b) * (N / slab)
    wall = time.perf_counter() - t0
    est = t_fq + t_gemm
    return {"value": round(STEP_GOP / 1e3 / est, 6), "unit": "TOP/s",
            "cores": O.num_threads(), "kind": "oracle",
            "sample": (f"one fwd+bwd step of the 4096^3 layer: 6 rotation passes at full size "
                       f"({t_fq:.2f} s) + the 3 INT8 products on {slab}-row slabs, scaled "
                       f"linearly to full size ({t_gemm:.1f} s extrapolated); "
                       f"{wall:.1f} s of CPU work measured")}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--kernel-iters", type=int, default=60)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import hadamard_rotated_precision_halo_amd as H
    import synth

    torch.cuda.set_device(0)
    sets = []
    for s in range(N_SETS):
        x, w, dy = synth.layer(M, N, K, seed=1001 + 97 * s)
        sets.append((to_dev(x, torch), to_dev(w, torch), to_dev(dy, torch)))
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
    dx = torch.empty((M, K), dtype=torch.bfloat16, device="cuda:0")
    dw = torch.empty((N, K), dtype=torch.bfloat16, device="cuda:0")
    ws_f = torch.empty(H.linear_workspace_bytes(M, N, K, torch.int8, False), dtype=torch.uint8,
                       device="cuda:0")
    ws_b = torch.empty(H.linear_workspace_bytes(M, N, K, torch.int8, True), dtype=torch.uint8,
                       device="cuda:0")

    def step(i):
        X, W, DY = sets[i % N_SETS]
        H.linear_fwd(X, W, BLOCK, y=y, workspace=ws_f)
        H.linear_bwd(DY, X, W, BLOCK, dx=dx, dw=dw, workspace=ws_b)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_step = elapsed * 1e3 / args.steps
    value = STEP_GOP / (ms_step * 1e-3) / 1e3  # TOP/s

    # ---- per-kernel measurements (same kernels, same shapes, HIP events on the stream) ----
    codes = [H.fwht_quant(X, axis=H.ROWS, block=BLOCK) for (X, _, _) in sets[:2]]
    wcodes = [H.fwht_quant(W, axis=H.ROWS, block=BLOCK) for (_, W, _) in sets[:2]]
    it = args.kernel_iters
    for i in range(3):
        H.gemm_i8(codes[i % 2][0], codes[i % 2][1], wcodes[i % 2][0], wcodes[i % 2][1], c=y)
    t_gemm = time_events(lambda i: H.gemm_i8(codes[i % 2][0], codes[i % 2][1],
                                             wcodes[i % 2][0], wcodes[i % 2][1], c=y), it, torch)
    qbuf = torch.empty((M, K), dtype=torch.int8, device="cuda:0")
    sbuf = torch.empty(max(M, K), dtype=torch.float32, device="cuda:0")
    t_rows = time_events(lambda i: H.fwht_quant(sets[i % N_SETS][0], axis=H.ROWS, block=BLOCK,
                                                q=qbuf, scale=sbuf[:M]), it, torch)
    t_cols = time_events(lambda i: H.fwht_quant(sets[i % N_SETS][2], axis=H.COLS, block=BLOCK,
                                                q=qbuf, scale=sbuf[:N]), it, torch)
    gemm_tops = 2 * M * N * K / (t_gemm * 1e-3) / 1e12
    fq_bytes = M * K * (2 + 1) + 4 * M
    rows_gbs = fq_bytes / (t_rows * 1e-3) / 1e9
    cols_gbs = fq_bytes / (t_cols * 1e-3) / 1e9

    result = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic",
        "config": {"workload": "halo_linear_fwd+bwd, X[4096x4096] W[4096x4096] dY[4096x4096] "
                               "bf16, INT8 codes, FWHT block 256",
                   "m": M, "n": N, "k": K, "block": BLOCK, "io": "bf16", "codes": "int8",
                   "input_sets": N_SETS},
        "roofline": {"bound": "mfma", "achieved": round(gemm_tops, 2), "peak": PEAK_INT8_TOPS,
                     "unit": "TFLOP/s", "frac": round(gemm_tops / PEAK_INT8_TOPS, 4),
                     "traffic": load_traffic("gemm_i8_4096"),
                     "kernel": "gemm_kernel<INT8, bf16 out> 4096x4096x4096",
                     "ms_per_launch": round(t_gemm, 5)},
        "fwht_quant": {
            "rows": {"bound": "hbm", "achieved": round(rows_gbs, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(rows_gbs / PEAK_HBM_GBS, 4),
                     "traffic": load_traffic("fq_rows_4096"), "ms_per_launch": round(t_rows, 5),
                     "algorithmic_bytes": fq_bytes},
            "cols": {"bound": "hbm", "achieved": round(cols_gbs, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(cols_gbs / PEAK_HBM_GBS, 4),
                     "traffic": load_traffic("fq_cols_4096"), "ms_per_launch": round(t_cols, 5),
                     "algorithmic_bytes": fq_bytes},
        },
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
