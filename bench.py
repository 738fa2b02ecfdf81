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
(HBM-bound).  The CPU baseline times the oracle on one full step of the same layer.

Other modes:
  --kernels-only        launch each hot kernel --kernel-iters times next to a 64 MiB
                        elementwise read + write (the counter calibration); run under rocprofv3.
  --summarize-stats F   turn a rocprofv3 --stats kernel_stats.csv into a text summary.
  --summarize-pmc D1 D2 turn two rocprofv3 --pmc runs of --kernels-only (FETCH_SIZE in D1,
                        WRITE_SIZE in D2) into the per-launch HBM traffic of each kernel.
"""
import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "HALO linear fwd+bwd effective TOP/s + FWHT-quant GB/s (% roofline), 4096x4096"
PEAK_INT8_TOPS = 5000.0   # MI355X dense INT8 MFMA, TOP/s
PEAK_FP8_TFLOPS = 5000.0  # MI355X dense FP8 MFMA, TFLOP/s
PEAK_HBM_GBS = 8000.0     # MI355X HBM3E, GB/s
M = N = K = 4096
BLOCK = 256
N_SETS = 6                # 6 x (X, W, dY) bf16 = 576 MB > 256 MB Infinity Cache
STEP_GOP = 3 * 2 * M * N * K / 1e9
GEMM_OPS = 2 * M * N * K
FQ_BYTES = M * K * (2 + 1) + 4 * M          # bf16 in, one code byte out, one fp32 scale/vector
GEMM_BYTES = 2 * M * K + 2 * M * N + 4 * (M + N)  # both code operands, bf16 output, scales
COPY_BYTES = 64 << 20                       # calibration: 64 MiB read + 64 MiB written
KERNEL_SOURCES = ["hadamard_rotated_precision_halo_amd/csrc/gemm.hip",
                  "hadamard_rotated_precision_halo_amd/csrc/fwht_quant.hip",
                  "hadamard_rotated_precision_halo_amd/csrc/fwht_wave.h",
                  "hadamard_rotated_precision_halo_amd/csrc/fwht_wave.hip",
                  "hadamard_rotated_precision_halo_amd/csrc/fwht_wave_sr.hip",
                  "hadamard_rotated_precision_halo_amd/csrc/halo_device.h",
                  "hadamard_rotated_precision_halo_amd/csrc/halo_kernels.h"]
K_PAD = 4000                                # rows of 4000 elements, padded to 4096 codes
# algorithmic bytes of the rotation passes over a 16384 x 14336 bf16 gradient (codes + scales)
LARGE_BYTES = 16384 * 14336 * 3 + 4 * 16384
LARGE_COLS_BYTES = 16384 * 14336 * 3 + 4 * 14336
FQ_PAD_BYTES = M * K_PAD * 2 + M * K + 4 * M
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic_4096.json")

# kernel-name patterns of each measured pass (rocprofv3 Kernel_Name substrings); a pass may
# launch several kernels per call
PASSES = {
    "gemm_i8_4096": ["halo::gemm_kernel<0"],
    "fq_rows_4096": ["halo::fq_rows2_kernel<unsigned short, 256, 0, false>"],
    "fq_cols_4096": ["halo::fq_cols2_kernel<256, 0, false>"],
    "gemm_fp8_4096": ["halo::gemm_kernel<1"],
    "fq_rows_opt_4096": ["halo::fq_rows2_kernel<unsigned short, 256, 0, true>"],
    "fq_cols_opt_4096": ["halo::fq_cols2_kernel<256, 0, true>"],
    "copy_64MiB": ["neg_kernel"],
}


def code_text(src):
    """C++ source without its comments and with whitespace runs collapsed: what the compiler
    sees, so that a comment edit does not mark the kernels as changed."""
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return " ".join(src.split())


def source_hash(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), encoding="utf-8") as f:
            h.update(code_text(f.read()).encode())
    return h.hexdigest()[:16]


def load_traffic(pass_key):
    """Counter-derived HBM bytes per launch from the committed summary, or None if the kernels
    changed since the counters were taken."""
    if not os.path.exists(TRAFFIC_JSON):
        return None
    with open(TRAFFIC_JSON) as f:
        d = json.load(f)
    if d.get("kernel_source_hash") != source_hash(KERNEL_SOURCES):
        return None
    return d.get("bytes_per_launch", {}).get(pass_key)


def to_dev(a, torch):
    return torch.from_numpy(a.view(np.int16)).to("cuda:0").view(torch.bfloat16)


def time_events(fn, iters, torch):
    """Average duration (ms) of fn() over `iters` back-to-back launches on the current stream
    (the stream the binding launches on)."""
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
    """The oracle (plain C, int64 / fp64, OpenMP over vectors and output rows) on one full
    fwd+bwd step of the same 4096^3 layer: the six rotation + quantisation passes and the three
    INT8 products with their dequantisation, nothing extrapolated."""
    import oracle as O
    import synth
    x, w, dy = synth.layer(M, N, K, seed=1001)
    t = {"fq": 0.0, "gemm": 0.0}

    def fq(a, axis):
        t0 = time.perf_counter()
        r = O.fwht_quant(a, axis, BLOCK, O.I8)
        t["fq"] += time.perf_counter() - t0
        return r

    def product(qa, sa, qb, sb):
        t0 = time.perf_counter()
        O.dequant(O.gemm_i8(qa, qb).astype(np.float64), sa, sb)
        t["gemm"] += time.perf_counter() - t0

    t0 = time.perf_counter()
    steps = 0
    while steps < 5 and (steps == 0 or time.perf_counter() - t0 < 10.0):
        product(*fq(x, O.ROWS), *fq(w, O.ROWS))      # Y = X W^T, rotation along K
        product(*fq(dy, O.ROWS), *fq(w, O.COLS))     # dX = dY W, rotation along N
        product(*fq(dy, O.COLS), *fq(x, O.COLS))     # dW = dY^T X, rotation along M
        steps += 1
    wall = time.perf_counter() - t0
    return {"value": round(steps * STEP_GOP / 1e3 / wall, 6), "unit": "TOP/s",
            "cores": O.num_threads(), "kind": "oracle",
            "sample": (f"{steps} full fwd+bwd step(s) of the 4096^3 layer (seed 1001), repeated "
                       f"to at least 10 s: rotation passes {t['fq']:.2f} s + INT8 products with "
                       f"dequant {t['gemm']:.2f} s = {wall:.2f} s wall")}


def make_inputs(torch):
    import synth
    sets = []
    for s in range(N_SETS):
        x, w, dy = synth.layer(M, N, K, seed=1001 + 97 * s)
        sets.append((to_dev(x, torch), to_dev(w, torch), to_dev(dy, torch)))
    return sets


SEED64 = 0x0123456789ABCDEF  # Philox key of the stochastic-rounding legs


def _c_launcher(H, name, arg_sets):
    """Back-to-back launches through the C entry point `name` with argument lists marshalled
    once (the benchmark times the kernels, not the binding's per-call Python work)."""
    fn = getattr(H.lib(), name)

    def run(i):
        st = fn(*arg_sets[i % len(arg_sets)])
        if st != 0:
            raise RuntimeError(f"{name} failed with status {st}")
    return run


def measure_kernels(H, torch, sets, iters, with_copy=False):
    """Per-launch time (ms) of the dominant kernels, in the configuration the step launches
    them: INT8 GEMM 4096^3 -> bf16, rows pass of X, columns pass of dY (block 256); the FP8
    GEMM 4096^3 (E4M3 codes); and the option legs: the rows and columns passes of dY with the
    randomised transform's signs and stochastic rounding, and a rows pass over rows of 4000
    elements zero-padded to 4096.  The calls go straight to the C entry points with their
    arguments prepared beforehand."""
    import ctypes
    P, ld, code = H._ptr, H._ld, H._code
    st = H._stream(None)
    codes = [H.fwht_quant(X, axis=H.ROWS, block=BLOCK) for (X, _, _) in sets[:2]]
    wcodes = [H.fwht_quant(W, axis=H.ROWS, block=BLOCK) for (_, W, _) in sets[:2]]
    e4 = torch.float8_e4m3fn
    f8x = [H.fwht_quant(X, axis=H.ROWS, block=BLOCK, q_dtype=e4) for (X, _, _) in sets[:2]]
    f8w = [H.fwht_quant(W, axis=H.ROWS, block=BLOCK, q_dtype=e4) for (_, W, _) in sets[:2]]
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
    qbuf = torch.empty((M, K), dtype=torch.int8, device="cuda:0")
    sbuf = torch.empty(max(M, K), dtype=torch.float32, device="cuda:0")
    wsc = torch.empty(max(H.fwht_quant_workspace_bytes(M, N, H.COLS, BLOCK), 256),
                      dtype=torch.uint8, device="cuda:0")
    signs = H.hadamard_signs(K, seed=2024, device="cuda:0")
    padded = [X[:, :K_PAD].contiguous() for (X, _, _) in sets]
    keep = []  # option structs referenced by the prepared argument lists

    def gemm_args(a, b, kind_code):
        return (P(a[0]), ld(a[0]), P(a[1]), P(b[0]), ld(b[0]), P(b[1]), M, N, K, P(y),
                code(y.dtype), ld(y), st)

    gemm = _c_launcher(H, "halo_gemm_i8", [gemm_args(codes[i], wcodes[i], 0) for i in range(2)])
    gemm_fp8 = _c_launcher(H, "halo_gemm_fp8", [
        (P(f8x[i][0]), code(e4), ld(f8x[i][0]), P(f8x[i][1]), P(f8w[i][0]), code(e4),
         ld(f8w[i][0]), P(f8w[i][1]), M, N, K, P(y), code(y.dtype), ld(y), st) for i in range(2)])

    def fq_args(x, axis, opts=None, ws=None):
        rows_, cols_ = x.shape
        nvec = rows_ if axis == H.ROWS else cols_
        L = cols_ if axis == H.ROWS else rows_
        lp = H.padded_len(L, BLOCK)
        q = qbuf.view(-1)[:nvec * lp].view(nvec, lp)
        if opts is not None:
            keep.append(opts)
        return (P(x), code(x.dtype), rows_, cols_, ld(x), axis, BLOCK, code(torch.int8), P(q),
                ld(q), P(sbuf), ctypes.byref(opts) if opts is not None else None,
                P(ws) if ws is not None else None, ws.numel() if ws is not None else 0, st)

    def sr_opts(i):
        return H.QuantOpts(P(signs), H.STOCHASTIC, H._u32x2(SEED64), H._u32x2(i))

    fq = "halo_fwht_quant_ex"
    rows = _c_launcher(H, fq, [fq_args(X, H.ROWS) for (X, _, _) in sets])
    cols = _c_launcher(H, fq, [fq_args(DY, H.COLS, ws=wsc) for (_, _, DY) in sets])
    rows_opt = _c_launcher(H, fq, [fq_args(sets[i][2], H.ROWS, sr_opts(i))
                                   for i in range(N_SETS)])
    cols_opt = _c_launcher(H, fq, [fq_args(sets[i][2], H.COLS, sr_opts(i), wsc)
                                   for i in range(N_SETS)])
    rows_pad = _c_launcher(H, fq, [fq_args(Xp, H.ROWS) for Xp in padded])

    legs = {"gemm_i8_4096": gemm, "gemm_fp8_4096": gemm_fp8, "fq_rows_4096": rows,
            "fq_cols_4096": cols, "fq_rows_opt_4096": rows_opt, "fq_cols_opt_4096": cols_opt,
            "fq_rows_pad_4000": rows_pad}
    for f in legs.values():
        for i in range(3):
            f(i)
    # three rounds over all legs, the median per leg: the clock of a power-limited chip
    # still wanders in the first few hundred milliseconds of load
    runs = {k: [] for k in legs}
    for _ in range(3):
        for k, f in legs.items():
            runs[k].append(time_events(f, iters, torch))
    out = {k: float(np.median(v)) for k, v in runs.items()}
    if with_copy:
        src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0").normal_()
        dst = torch.empty_like(src)
        # the counter calibration: an elementwise kernel that reads and writes exactly 64 MiB,
        # with a name no other launch of the run shares
        out["copy_64MiB"] = time_events(lambda i: torch.neg(src, out=dst), iters, torch)
    return out


def summarize_stats(path, command, last=0):
    """rocprofv3 kernel_stats.csv -> text table (per-kernel average duration).  With `last`,
    the kernel_trace.csv beside it also gives each pass's average over its last `last`
    dispatches: the back-to-back launches the bench times with HIP events."""
    with open(path) as f:
        rows = list(csv.DictReader(f))
    lines = [f"command: {command}", "",
             f"{'calls':>6} {'avg us':>9} {'min us':>9} {'max us':>9} {'%':>6}  kernel"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        lines.append(f"{int(r['Calls']):>6} {float(r['AverageNs']) / 1e3:>9.2f} "
                     f"{float(r['MinNs']) / 1e3:>9.2f} {float(r['MaxNs']) / 1e3:>9.2f} "
                     f"{float(r['Percentage']):>6.2f}  {r['Name'][:150]}")
    trace = path.replace("kernel_stats.csv", "kernel_trace.csv")
    if last and os.path.exists(trace):
        with open(trace) as f:
            tr = sorted(csv.DictReader(f), key=lambda r: int(r["Start_Timestamp"]))
        lines += ["", f"per pass, last {last} calls (the event-timed measurement loop):"]
        for key, pats in PASSES.items():
            calls = {}
            for r in tr:
                if any(p in r["Kernel_Name"] for p in pats):
                    d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
                    calls.setdefault(r["Kernel_Name"], []).append(d)
            if calls:
                per = sum(float(np.mean(v[-last:])) for v in calls.values())
                lines.append(f"  {key:<14} {per:>9.2f} us per call ({len(calls)} kernel(s))")
    return "\n".join(lines) + "\n"


def _pmc_per_call(d, counter):
    """Average counter value (KiB) per call of each pass, from a counter_collection.csv."""
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    per_kernel = {}
    for fn in files:
        with open(fn) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                per_kernel.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    out = {}
    for key, pats in PASSES.items():
        tot = 0.0
        found = False
        for name, vals in per_kernel.items():
            if any(p in name for p in pats):
                tot += float(np.mean(vals))
                found = True
        out[key] = tot if found else None
    return out


def summarize_pmc(fetch_dir, write_dir, command):
    fetch = _pmc_per_call(fetch_dir, "FETCH_SIZE")
    write = _pmc_per_call(write_dir, "WRITE_SIZE")
    # calibration: the elementwise negation of COPY_BYTES reads and writes exactly COPY_BYTES
    f_scale = COPY_BYTES / (fetch["copy_64MiB"] * 1024.0)
    w_scale = COPY_BYTES / (write["copy_64MiB"] * 1024.0)
    algo = {"gemm_i8_4096": GEMM_BYTES, "gemm_fp8_4096": GEMM_BYTES, "fq_rows_4096": FQ_BYTES,
            "fq_cols_4096": FQ_BYTES, "fq_rows_opt_4096": FQ_BYTES, "fq_cols_opt_4096": FQ_BYTES}
    res = {"kernel_source_hash": source_hash(KERNEL_SOURCES), "command": command,
           "fetch_scale": f_scale, "write_scale": w_scale, "bytes_per_launch": {},
           "fetch_kib_raw": fetch, "write_kib_raw": write}
    lines = [f"command: {command}",
             f"calibration ({COPY_BYTES >> 20} MiB elementwise read + write): FETCH_SIZE x{f_scale:.3f}, "
             f"WRITE_SIZE x{w_scale:.3f} -> bytes", "",
             f"{'pass':<14} {'read MB':>9} {'write MB':>9} {'total MB':>9} {'algorithmic MB':>15}"]
    for key in algo:
        if fetch[key] is None or write[key] is None:
            continue
        rd = fetch[key] * 1024.0 * f_scale
        wr = write[key] * 1024.0 * w_scale
        res["bytes_per_launch"][key] = int(round(rd + wr))
        lines.append(f"{key:<14} {rd / 1e6:>9.2f} {wr / 1e6:>9.2f} {(rd + wr) / 1e6:>9.2f} "
                     f"{algo[key] / 1e6:>15.2f}")
    return res, "\n".join(lines) + "\n"


def measure_large_passes(H, torch, iters):
    """The rotation passes at the largest gradient shape (16384 x 14336 bf16, block 512, E5M2
    codes, as in the 16384-token MLP-up workload): per-launch time (ms) of the rows pass (along
    14336) and of the columns pass (along 16384 tokens, partial maxima exchanged), through the
    C entry point.  Inputs drawn on the GPU: a memory-bound pass's speed does not depend on
    the values."""
    P, ld, code = H._ptr, H._ld, H._code
    st = H._stream(None)
    rows_, cols_, blk = 16384, 14336, 512
    e5 = torch.float8_e5m2
    xs = [(torch.randn(rows_, cols_, device="cuda:0") * 1e-3).to(torch.bfloat16)
          for _ in range(2)]
    q = torch.empty(rows_ * cols_, dtype=torch.uint8, device="cuda:0")
    sc = torch.empty(max(rows_, cols_), dtype=torch.float32, device="cuda:0")
    ws = torch.empty(max(H.fwht_quant_workspace_bytes(rows_, cols_, H.COLS, blk), 256),
                     dtype=torch.uint8, device="cuda:0")

    def args(x, axis):
        nvec, lp = (rows_, cols_) if axis == H.ROWS else (cols_, rows_)
        return (P(x), code(x.dtype), rows_, cols_, ld(x), axis, blk, code(e5), P(q), lp,
                P(sc), None, P(ws), ws.numel(), st)

    out = {}
    for key, axis in (("rows", H.ROWS), ("cols", H.COLS)):
        f = _c_launcher(H, "halo_fwht_quant_ex", [args(x, axis) for x in xs])
        for i in range(3):
            f(i)
        out[key] = float(np.median([time_events(f, iters, torch) for _ in range(3)]))
    del xs, q
    return out


def bench_workload(name, args):
    """One named workload (fwd and / or bwd, as its configuration lists) on the inputs of the
    full-size parity tests (same seeded generator): one JSON line with times and rates.  These
    are the parity workloads, not the benchmark's headline line."""
    import torch
    import hadamard_rotated_precision_halo_amd as H
    import synth

    torch.cuda.set_device(0)
    print(f"{name}: generating the inputs", file=sys.stderr, flush=True)
    cfg, x, w, dy = synth.workload(name)
    print(f"{name}: inputs ready, timing", file=sys.stderr, flush=True)
    m, n, k, b = cfg["m"], cfg["n"], cfg["k"], cfg["block"]
    codes = {"i8": torch.int8, "e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}
    qd, gqd = codes[cfg["q"]], codes[cfg["gq"]]

    def dev(a):
        if a.dtype == np.uint16:
            return to_dev(a, torch)
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda:0")

    X, W = dev(x), dev(w)
    DY = dev(dy) if cfg["bwd"] else None
    del x, w, dy
    io = torch.float32 if cfg["io"] == synth.F32 else torch.bfloat16
    out = {"metric": "HALO linear effective TOP/s", "unit": "TOP/s", "workload": name,
           "m": m, "n": n, "k": k, "block": b, "codes": [cfg["q"], cfg["gq"]],
           "data": "synthetic", "steps": args.steps, "warmup": args.warmup}
    gop = 2.0 * m * n * k / 1e9
    total_ms, total_gop = 0.0, 0.0
    if cfg["fwd"]:
        y = torch.empty((m, n), dtype=io, device="cuda:0")
        ws_f = torch.empty(H.linear_workspace_bytes(m, n, k, qd, False, block=b),
                           dtype=torch.uint8, device="cuda:0")

        def fwd(i):
            H.linear_fwd(X, W, b, q_dtype=qd, y=y, workspace=ws_f)
        for i in range(args.warmup):
            fwd(i)
        ms = time_events(fwd, args.steps, torch)
        out["fwd_ms"], out["fwd_tops"] = round(ms, 4), round(gop / ms, 1)
        total_ms, total_gop = total_ms + ms, total_gop + gop
    if cfg["bwd"]:
        dx = torch.empty((m, k), dtype=io, device="cuda:0")
        dw = torch.empty((n, k), dtype=io, device="cuda:0")
        ws_b = torch.empty(H.linear_workspace_bytes(m, n, k, qd, True, block=b),
                           dtype=torch.uint8, device="cuda:0")

        def bwd(i):
            H.linear_bwd(DY, X, W, b, q_dtype=qd, grad_q_dtype=gqd, dx=dx, dw=dw,
                         workspace=ws_b)
        for i in range(args.warmup):
            bwd(i)
        ms = time_events(bwd, args.steps, torch)
        out["bwd_ms"], out["bwd_tops"] = round(ms, 4), round(2 * gop / ms, 1)
        total_ms, total_gop = total_ms + ms, total_gop + 2 * gop
    out["ms_per_step"] = round(total_ms, 4)
    out["value"] = round(total_gop / total_ms, 1)  # GOP per ms = TOP/s
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--kernel-iters", type=int, default=60)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kernels-only", action="store_true")
    ap.add_argument("--summarize-stats", metavar="CSV")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--command", default="", help="profiling command recorded in a summary")
    ap.add_argument("--out", help="summary file to write")
    ap.add_argument("--last", type=int, default=0, help="trace calls per pass to average")
    ap.add_argument("--workload", help="time one named parity workload instead (see synth)")
    args = ap.parse_args()

    if args.summarize_stats:
        text = summarize_stats(args.summarize_stats, args.command, args.last)
        if args.out:
            with open(args.out, "w") as f:
                f.write(text)
        print(text, end="")
        return
    if args.summarize_pmc:
        res, text = summarize_pmc(*args.summarize_pmc, args.command)
        with open(TRAFFIC_JSON, "w") as f:
            json.dump(res, f, indent=1)
        if args.out:
            with open(args.out, "w") as f:
                f.write(text)
        print(text, end="")
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    if args.workload:
        bench_workload(args.workload, args)
        return

    import torch
    import hadamard_rotated_precision_halo_amd as H

    torch.cuda.set_device(0)
    sets = make_inputs(torch)

    if args.kernels_only:
        t = measure_kernels(H, torch, sets, args.kernel_iters, with_copy=True)
        print(json.dumps({k: round(v * 1e3, 3) for k, v in t.items()} | {"unit": "us"}),
              flush=True)
        return

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
    st = torch.cuda.current_stream()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        evs[i].record(st)
        step(i)
    evs[-1].record(st)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_step = elapsed * 1e3 / args.steps
    value = STEP_GOP / (ms_step * 1e-3) / 1e3  # TOP/s
    per_step = np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)])

    # ---- the same step with the options: randomised transform on every contraction dim,
    # stochastic rounding of the dY codes (a fresh counter per step) ----
    sk = H.hadamard_signs(K, seed=11, device="cuda:0")
    sn = H.hadamard_signs(N, seed=12, device="cuda:0")
    sm = H.hadamard_signs(M, seed=13, device="cuda:0")

    def step_opt(i):
        X, W, DY = sets[i % N_SETS]
        H.linear_fwd(X, W, BLOCK, y=y, workspace=ws_f, signs_k=sk)
        H.linear_bwd(DY, X, W, BLOCK, dx=dx, dw=dw, workspace=ws_b, signs_n=sn, signs_m=sm,
                     grad_rounding="stochastic", seed=SEED64, counter=i)

    for i in range(3):
        step_opt(i)
    ms_opt = time_events(step_opt, args.steps, torch)

    # ---- the backward again with block 4096: one block over the whole contraction ----
    ws_b4 = torch.empty(H.linear_workspace_bytes(M, N, K, torch.int8, True, block=4096),
                        dtype=torch.uint8, device="cuda:0")

    def bwd_4096(i):
        X, W, DY = sets[i % N_SETS]
        H.linear_bwd(DY, X, W, 4096, dx=dx, dw=dw, workspace=ws_b4)

    def bwd_256(i):
        X, W, DY = sets[i % N_SETS]
        H.linear_bwd(DY, X, W, BLOCK, dx=dx, dw=dw, workspace=ws_b)

    for i in range(3):
        bwd_4096(i)
        bwd_256(i)
    ms_bwd4096 = time_events(bwd_4096, args.steps, torch)
    ms_bwd256 = time_events(bwd_256, args.steps, torch)

    # ---- per-kernel measurements (same kernels, same shapes, HIP events on the stream) ----
    t = measure_kernels(H, torch, sets, args.kernel_iters)
    t_large = measure_large_passes(H, torch, max(5, args.kernel_iters // 6))
    t_gemm, t_rows, t_cols = t["gemm_i8_4096"], t["fq_rows_4096"], t["fq_cols_4096"]
    gemm_tops = GEMM_OPS / (t_gemm * 1e-3) / 1e12
    rows_gbs = FQ_BYTES / (t_rows * 1e-3) / 1e9
    cols_gbs = FQ_BYTES / (t_cols * 1e-3) / 1e9

    def hbm(gbs, ms, key, nbytes=FQ_BYTES):
        return {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": load_traffic(key),
                "ms_per_launch": round(ms, 5), "algorithmic_bytes": nbytes}

    def hbm_pass(key, nbytes=FQ_BYTES):
        return hbm(nbytes / (t[key] * 1e-3) / 1e9, t[key], key, nbytes)

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
        "step_ms": {"p10": round(float(np.percentile(per_step, 10)), 4),
                    "p50": round(float(np.percentile(per_step, 50)), 4),
                    "p90": round(float(np.percentile(per_step, 90)), 4)},
        "roofline": {"bound": "mfma", "achieved": round(gemm_tops, 2), "peak": PEAK_INT8_TOPS,
                     "unit": "TFLOP/s", "frac": round(gemm_tops / PEAK_INT8_TOPS, 4),
                     "traffic": load_traffic("gemm_i8_4096"),
                     "kernel": "gemm_kernel<INT8, bf16 out> 4096x4096x4096",
                     "ms_per_launch": round(t_gemm, 5), "algorithmic_ops": GEMM_OPS},
        "fwht_quant": {"rows": hbm(rows_gbs, t_rows, "fq_rows_4096"),
                       "cols": hbm(cols_gbs, t_cols, "fq_cols_4096")},
        "gemm_fp8": {"bound": "mfma", "achieved": round(GEMM_OPS / (t["gemm_fp8_4096"] * 1e-3) / 1e12, 2),
                     "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(GEMM_OPS / (t["gemm_fp8_4096"] * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 4),
                     "traffic": load_traffic("gemm_fp8_4096"),
                     "kernel": "gemm_kernel<FP8 E4M3 x E4M3, bf16 out> 4096x4096x4096",
                     "ms_per_launch": round(t["gemm_fp8_4096"], 5), "algorithmic_ops": GEMM_OPS},
        "options": {
            "step": {"ms": round(ms_opt, 4),
                     "effective_tops": round(STEP_GOP / (ms_opt * 1e-3) / 1e3, 3),
                     "what": "the same fwd+bwd step with the randomised transform H D along "
                             "K, N and M and stochastic rounding of the dY codes"},
            "rows_signs_sr": hbm_pass("fq_rows_opt_4096"),
            "cols_signs_sr": hbm_pass("fq_cols_opt_4096"),
            "rows_padded_4000_to_4096": hbm_pass("fq_rows_pad_4000", FQ_PAD_BYTES),
        },
        "fwht_quant_16384x14336": {
            "what": "the rotation passes at the largest gradient shape: 16384 x 14336 bf16, "
                    "block 512, E5M2 codes; rows along 14336, columns along the 16384 tokens "
                    "(16 parts per column, partial maxima exchanged)",
            "rows": hbm(LARGE_BYTES / (t_large["rows"] * 1e-3) / 1e9, t_large["rows"],
                        "fq_rows_16384x14336", LARGE_BYTES),
            "cols": hbm(LARGE_COLS_BYTES / (t_large["cols"] * 1e-3) / 1e9, t_large["cols"],
                        "fq_cols_16384x14336", LARGE_COLS_BYTES),
        },
        "bwd_block_4096": {
            "ms": round(ms_bwd4096, 4),
            "effective_tops": round(2 * GEMM_OPS / (ms_bwd4096 * 1e-3) / 1e12, 3),
            "ms_block_256": round(ms_bwd256, 4),
            "what": "halo_linear_bwd alone (dX and dW) with block 4096 on N and M, beside the "
                    "same call with the step's block 256",
        },
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
