"""Benchmark of the Hadamard-rotated INT8 linear layer on one MI355X.

One step = halo_linear_fwd + halo_linear_bwd of a 4096 x 4096 layer over 4096 tokens (bf16
inputs, INT8 codes, rotation block 256): six rotation + quantisation passes (rows of X and W;
rows of dY and columns of W; columns of dY and of X) and three INT8 GEMMs (Y, dX, dW) --
every kernel of the hot path.  The headline value is the effective throughput: the three
8-bit GEMMs' algorithmic work (3 * 2 * 4096^3 operations) divided by the wall time of the
whole step, rotations included.

Inputs are synthetic (synth.layer: N(0,1) activations with 0.1% outlier channels x50, weights
0.02 * N(0,1), Student-t(4) * 1e-3 gradients), already resident in HBM.  Several input sets
rotate from step to step so that no operand stays in the 256 MB Infinity Cache.  Before the
counted warmup, steps run for --settle-s seconds: the chip's power management moves the clock
during the first second or so of load, and the timed steps should see the clock it sustains.
The shader clock and the board power are sampled from sysfs on a host thread while the steps
are timed, and reported beside the result.

Per-kernel figures are measured in the same run with HIP events on the launch stream: the
INT8 GEMM (the dominant kernel, MFMA-bound) and the rows / columns rotation passes
(HBM-bound), each cycling through more than 512 MB of distinct inputs so that no operand is
served from the Infinity Cache.  Beside the products, the library's matrix-core rate probe
measures what each product's MFMA instruction alone sustains on the whole device (with the
clock it runs at): the published peak assumes a 2.4 GHz clock the chip does not hold under a
sustained matrix load.  The CPU baseline times the oracle on full steps of the same
layer on all host threads, a one-thread sample of it, and each pass's oracle / GPU ratio.

Other modes:
  --kernels-only        launch each hot kernel --kernel-iters times next to a 64 MiB
                        elementwise read + write (the counter calibration); run under rocprofv3.
  --summarize-stats F   turn a rocprofv3 --stats kernel_stats.csv into a text summary.
  --summarize-pmc D1 D2 turn two rocprofv3 --pmc runs of --kernels-only (FETCH_SIZE in D1,
                        WRITE_SIZE in D2) into the per-launch HBM traffic of each kernel.
  --summarize-counters D...  any rocprofv3 --pmc runs of --kernels-only: each counter's mean
                        per call of each pass, and the products' matrix-core figures.
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
COPY_REF_BYTES = 512 << 20                  # streaming reference: 512 MiB read + 512 MiB written
KERNEL_SOURCES = ["hadamard_rotated_precision_halo_amd/csrc/gemm.hip",
                  "hadamard_rotated_precision_halo_amd/csrc/fwht_dual.hip",
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
DUAL_BYTES = M * N * 2 + 2 * M * N + 4 * (M + N)  # one bf16 read, two code matrices, scales
FQ_F32_BYTES = M * K * (4 + 1) + 4 * K       # fp32 columns in, one code byte out, scales
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic_4096.json")

# kernel-name patterns of each measured pass (rocprofv3 Kernel_Name substrings; a pass may
# launch several kernels per call) and, where one kernel serves launches of several sizes,
# the grid (work-items) of this pass's launches: the 4096^3 products run 256 workgroups of
# 512 work-items, the backward's paired products twice as many
GEMM_GRID = 256 * 512
PASSES = {
    "gemm_i8_4096": (["halo::gemm_kernel<0"], GEMM_GRID),
    "fq_rows_4096": (["halo::fq_rows2_kernel<unsigned short, 256, 0, false>"], None),
    "fq_cols_4096": (["halo::fq_cols2_kernel<256, 0, false, false, false>"], None),
    "gemm_fp8_4096": (["halo::gemm_kernel<1"], GEMM_GRID),
    "fq_rows_opt_4096": (["halo::fq_rows2_kernel<unsigned short, 256, 0, true>"], None),
    "fq_cols_opt_4096": (["halo::fq_cols2_kernel<256, 0, true, false, false>"], None),
    "copy_neg": (["neg_kernel"], None),  # 64 MiB calibration, or the 512 MiB copy reference
    "fq_batch_4096": (["halo::fq_batch_kernel<256, 0, 0, false, false>"], None),
    "gemm_i8_pair_4096": (["halo::gemm_kernel<0"], 2 * GEMM_GRID),
    "fq_dual_4096": (["fq_dual_kernel<256, 0, false, false>"], None),
    "fq_cols_f32_4096": (["halo::fq_cols2_kernel<256, 0, false, false, true>"], None),
}


def pass_match(key, name, grid):
    """Whether a dispatch of kernel `name` over `grid` work-items (None: not recorded) belongs
    to pass `key`."""
    pats, g = PASSES[key]
    return any(p in name for p in pats) and (g is None or grid is None or grid == g)


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


class ClockSampler:
    """Samples the GPU's current shader clock (sysfs pp_dpm_sclk: the level marked '*') and
    its board power (hwmon power1_input, microwatts) every `period` seconds on a host thread
    while active.  Either reading may be missing on a machine; its summary is then None."""

    def __init__(self, period=0.01):
        import threading
        self.period = period
        self.sclk_path = next(iter(sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))),
                              None)
        dev = os.path.dirname(self.sclk_path) if self.sclk_path else None
        self.power_path = next(iter(sorted(glob.glob(os.path.join(dev, "hwmon", "*",
                                                                  "power1_input")))), None) \
            if dev else None
        self.sclk, self.power = [], []
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    def _read(self):
        if self.sclk_path:
            try:
                with open(self.sclk_path) as f:
                    for line in f:
                        if "*" in line:
                            m = re.search(r"(\d+)\s*Mhz", line, re.I)
                            if m:
                                self.sclk.append(int(m.group(1)))
            except OSError:
                pass
        if self.power_path:
            try:
                with open(self.power_path) as f:
                    self.power.append(int(f.read().strip()) / 1e6)
            except (OSError, ValueError):
                pass

    def _run(self):
        # waiting on the stop event (not sleeping) lets __exit__ return at once, without an
        # idle gap on the GPU while the caller joins the thread
        self._read()
        while not self._stop.wait(self.period):
            self._read()

    def __enter__(self):
        self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        self._thread.join()

    @staticmethod
    def _stats(v, nd):
        if not v:
            return None
        a = np.array(v, dtype=np.float64)
        return {"median": round(float(np.median(a)), nd), "min": round(float(a.min()), nd),
                "max": round(float(a.max()), nd), "samples": int(a.size)}

    def summary(self):
        return {"sclk_mhz": self._stats(self.sclk, 0), "power_w": self._stats(self.power, 1),
                "source": self.sclk_path}


def settle(step, seconds, torch, sampler=None):
    """Run steps until `seconds` have passed (in groups of 10, synchronised): the clock-settle
    phase before the counted warmup.  With a ClockSampler, the shader clock and board power
    are sampled from 40 % to 80 % of the phase, the steady state of the same steps (sampling
    sysfs while steps run slows them by about 2 %, so the counted steps run unsampled); the
    phase's last fifth runs unsampled, so the steps that follow start from the same steady
    state.  Returns (steps run, seconds)."""
    t0 = time.perf_counter()
    n = 0
    state = 0  # 0: before sampling, 1: sampling, 2: done
    while time.perf_counter() - t0 < seconds:
        el = time.perf_counter() - t0
        if sampler is not None and state == 0 and el >= 0.4 * seconds:
            sampler.__enter__()
            state = 1
        elif state == 1 and el >= 0.8 * seconds:
            sampler.__exit__(None, None, None)
            state = 2
        for _ in range(10):
            step(n)
            n += 1
        torch.cuda.synchronize()
    if state == 1:
        sampler.__exit__(None, None, None)
    return n, time.perf_counter() - t0


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _one_thread_sample():
    """The oracle on one host thread (run in a child process with OMP_NUM_THREADS=1): the six
    rotation passes of a step at full size and one product on a 256-row slab of its A
    operand.  Returns the seconds of each part as JSON on stdout."""
    import oracle as O
    import synth
    x, w, dy = synth.layer(M, N, K, seed=1001)
    t0 = time.perf_counter()
    qx, sx = O.fwht_quant(x, O.ROWS, BLOCK, O.I8)
    qw, sw = O.fwht_quant(w, O.ROWS, BLOCK, O.I8)
    O.fwht_quant(dy, O.ROWS, BLOCK, O.I8)
    O.fwht_quant(w, O.COLS, BLOCK, O.I8)
    O.fwht_quant(dy, O.COLS, BLOCK, O.I8)
    O.fwht_quant(x, O.COLS, BLOCK, O.I8)
    t1 = time.perf_counter()
    O.dequant(O.gemm_i8(qx[:256], qw).astype(np.float64), sx[:256], sw)
    t2 = time.perf_counter()
    print(json.dumps({"threads": O.num_threads(), "fq_s": t1 - t0, "slab_s": t2 - t1}))


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
    out = {"value": round(steps * STEP_GOP / 1e3 / wall, 6), "unit": "TOP/s",
           "cores": O.num_threads(), "kind": "oracle",
           "sample": (f"{steps} full fwd+bwd step(s) of the 4096^3 layer (seed 1001), repeated "
                      f"to at least 10 s: rotation passes {t['fq']:.2f} s + INT8 products with "
                      f"dequant {t['gemm']:.2f} s = {wall:.2f} s wall"),
           "cpu_model": cpu_model(), "nproc": os.cpu_count(),
           "omp_num_threads": os.environ.get("OMP_NUM_THREADS"),
           "per_pass_ms": {"fq": round(t["fq"] * 1e3 / (6 * steps), 2),
                           "product": round(t["gemm"] * 1e3 / (3 * steps), 2)}}
    # one thread, in a child process (the thread count of OpenMP is fixed at its start)
    import subprocess
    env = dict(os.environ, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, os.path.abspath(__file__), "--one-thread-sample"],
                       capture_output=True, text=True, env=env, timeout=600)
    if r.returncode == 0 and r.stdout.strip():
        one = json.loads(r.stdout.strip().splitlines()[-1])
        step_s = one["fq_s"] + 3 * (M / 256) * one["slab_s"]
        out["one_thread"] = {
            "threads": one["threads"], "value": round(STEP_GOP / 1e3 / step_s, 6),
            "unit": "TOP/s", "fq_ms": round(one["fq_s"] * 1e3 / 6, 2),
            "product_ms": round(one["slab_s"] * (M / 256) * 1e3, 2),
            "sample": (f"the six rotation passes of a step at full size ({one['fq_s']:.2f} s) "
                       f"and one INT8 product on a 256-row slab ({one['slab_s']:.2f} s); the "
                       f"step's products extrapolated linearly by rows (x{M // 256})")}
    return out


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
    # every leg cycles through more than 512 MB of distinct inputs: the 18 bf16 matrices of
    # the input sets (604 MB) for the rotation passes, and 18 pairs of 16 MiB code matrices
    # (604 MB: rows and columns codes of those matrices) for the products
    mats = [t for st_ in sets for t in st_]
    e4 = torch.float8_e4m3fn
    c8 = [H.fwht_quant(t, axis=ax, block=BLOCK) for ax in (H.ROWS, H.COLS) for t in mats]
    f8 = [H.fwht_quant(t, axis=ax, block=BLOCK, q_dtype=e4) for ax in (H.ROWS, H.COLS)
          for t in mats]
    half = len(mats)
    codes, wcodes = c8[:half], c8[half:]
    f8x, f8w = f8[:half], f8[half:]
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
    qbuf = torch.empty((M, K), dtype=torch.int8, device="cuda:0")
    sbuf = torch.empty(max(M, K), dtype=torch.float32, device="cuda:0")
    wsc = torch.empty(max(H.fwht_quant_workspace_bytes(M, N, H.COLS, BLOCK), 256),
                      dtype=torch.uint8, device="cuda:0")
    signs = H.hadamard_signs(K, seed=2024, device="cuda:0")
    padded = [t[:, :K_PAD].contiguous() for t in mats]
    keep = []  # option structs referenced by the prepared argument lists

    def gemm_args(a, b, kind_code):
        return (P(a[0]), ld(a[0]), P(a[1]), P(b[0]), ld(b[0]), P(b[1]), M, N, K, P(y),
                code(y.dtype), ld(y), st)

    gemm = _c_launcher(H, "halo_gemm_i8", [gemm_args(codes[i], wcodes[i], 0)
                                            for i in range(half)])
    gemm_fp8 = _c_launcher(H, "halo_gemm_fp8", [
        (P(f8x[i][0]), code(e4), ld(f8x[i][0]), P(f8x[i][1]), P(f8w[i][0]), code(e4),
         ld(f8w[i][0]), P(f8w[i][1]), M, N, K, P(y), code(y.dtype), ld(y), st)
        for i in range(half)])

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
    rows = _c_launcher(H, fq, [fq_args(t, H.ROWS) for t in mats])
    cols = _c_launcher(H, fq, [fq_args(t, H.COLS, ws=wsc) for t in mats])
    rows_opt = _c_launcher(H, fq, [fq_args(t, H.ROWS, sr_opts(i)) for i, t in enumerate(mats)])
    cols_opt = _c_launcher(H, fq, [fq_args(t, H.COLS, sr_opts(i), wsc)
                                   for i, t in enumerate(mats)])
    rows_pad = _c_launcher(H, fq, [fq_args(Xp, H.ROWS) for Xp in padded])
    # the columns pass on fp32 input: 9 of the matrices in fp32 (604 MB cycled)
    mats32 = [t.float() for t in mats[:9]]
    cols_f32 = _c_launcher(H, fq, [fq_args(t, H.COLS, ws=wsc) for t in mats32])

    # both passes of a matrix from one read (halo_fwht_quant_dual), beside the rows and the
    # columns pass above on the same matrices
    qc_buf = torch.empty((N, M), dtype=torch.int8, device="cuda:0")
    sc_buf = torch.empty(N, dtype=torch.float32, device="cuda:0")
    wsd = torch.empty(max(H.fwht_quant_dual_workspace_bytes(M, N, BLOCK), 256),
                      dtype=torch.uint8, device="cuda:0")
    dual = _c_launcher(H, "halo_fwht_quant_dual", [
        (P(t), code(t.dtype), M, N, ld(t), BLOCK, code(torch.int8), P(qbuf), N, P(sbuf),
         P(qc_buf), M, P(sc_buf), None, None, P(wsd), wsd.numel(), st) for t in mats])

    # the INT8 product as the forward runs it: its codes written just before by the rows
    # passes of that step's X and W (so they sit where the rotation left them), events
    # around the product's launch alone
    qx = torch.empty((M, K), dtype=torch.int8, device="cuda:0")
    qw = torch.empty((N, K), dtype=torch.int8, device="cuda:0")
    sxw = torch.empty(M + N, dtype=torch.float32, device="cuda:0")
    rows_xw = _c_launcher(H, fq, [
        (P(t), code(t.dtype), t.shape[0], t.shape[1], ld(t), H.ROWS, BLOCK, code(torch.int8),
         P(q_), ld(q_), ctypes.c_void_p(sxw.data_ptr() + 4 * M * w_), None, None, 0, st)
        for st_ in sets for t, q_, w_ in ((st_[0], qx, 0), (st_[1], qw, 1))])
    gemm_xw = _c_launcher(H, "halo_gemm_i8", [
        (P(qx), ld(qx), P(sxw), P(qw), ld(qw), ctypes.c_void_p(sxw.data_ptr() + 4 * M),
         M, N, K, P(y), code(y.dtype), ld(y), st)])

    def gemm_in_path(iters_):
        stream = torch.cuda.current_stream()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(iters_)]
        for i in range(iters_):
            rows_xw(2 * i)
            rows_xw(2 * i + 1)
            ev[i][0].record(stream)
            gemm_xw(0)
            ev[i][1].record(stream)
        ev[-1][1].synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in ev]))

    # the layer backward, whose first launch runs its four rotation passes together (rows of
    # dY; columns of W, dY and X): its kernels are told apart by name in the traces
    dx = torch.empty((M, K), dtype=torch.bfloat16, device="cuda:0")
    dw = torch.empty((N, K), dtype=torch.bfloat16, device="cuda:0")
    wsb = torch.empty(H.linear_workspace_bytes(M, N, K, torch.int8, True, block=BLOCK),
                      dtype=torch.uint8, device="cuda:0")
    bwd = _c_launcher(H, "halo_linear_bwd_ex", [
        (P(DY), P(X), P(W), code(X.dtype), M, N, K, BLOCK, code(torch.int8), code(torch.int8),
         P(dx), P(dw), None, P(wsb), wsb.numel(), st) for (X, W, DY) in sets])

    legs = {"gemm_i8_4096": gemm, "gemm_fp8_4096": gemm_fp8, "fq_rows_4096": rows,
            "fq_cols_4096": cols, "fq_rows_opt_4096": rows_opt, "fq_cols_opt_4096": cols_opt,
            "fq_rows_pad_4000": rows_pad, "linear_bwd_4096": bwd, "fq_dual_4096": dual,
            "fq_cols_f32_4096": cols_f32}
    if with_copy:
        # the padded rows pass shares the rows kernel and its grid: kept out of the counter
        # runs, whose per-pass averages would mix its smaller reads in
        del legs["fq_rows_pad_4000"]
    for f in legs.values():
        for i in range(3):
            f(i)
    # three rounds over all legs, the median per leg: the clock of a power-limited chip
    # still wanders in the first few hundred milliseconds of load
    runs = {k: [] for k in legs}
    runs["gemm_i8_4096_in_path"] = []
    gemm_in_path(3)
    for _ in range(3):
        for k, f in legs.items():
            runs[k].append(time_events(f, iters, torch))
        runs["gemm_i8_4096_in_path"].append(gemm_in_path(iters))
    out = {k: float(np.median(v)) for k, v in runs.items()}
    if not with_copy:
        # the practical streaming rate of this HBM: torch's elementwise negation of 512 MiB
        # into another 512 MiB (1 GiB moved per launch, two pairs of buffers cycled: nothing
        # cache-resident).  Left out of the counter runs, whose calibration kernel is the same
        # negation on 64 MiB.
        big = [torch.empty(COPY_REF_BYTES // 4, dtype=torch.float32, device="cuda:0")
               for _ in range(4)]
        for b_ in big:
            b_.fill_(1.0)

        def copy_ref(i):
            torch.neg(big[(2 * i) % 4], out=big[(2 * i + 1) % 4])
        copy_ref(0)
        out["copy_ref_512MiB"] = float(np.median([time_events(copy_ref, 10, torch)
                                                  for _ in range(3)]))
        del big
    if with_copy:
        src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0").normal_()
        dst = torch.empty_like(src)
        # the counter calibration: an elementwise kernel that reads and writes exactly 64 MiB,
        # with a name no other launch of the run shares
        out["copy_64MiB"] = time_events(lambda i: torch.neg(src, out=dst), iters, torch)
    return out


def measure_mfma_sustained(H, torch, seconds=0.4):
    """Sustained whole-device rate (TOP/s) of each matrix-core instruction the products use,
    from the library's rate probe: launches back to back for about `seconds` after a short
    warm-up, HIP events on the stream, the shader clock and board power sampled meanwhile."""
    st = torch.cuda.current_stream()
    out = {}
    for kind, name in H.MFMA_PROBE_KINDS.items():
        iters = 2000
        H.mfma_rate_probe(kind, iters, st)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < 0.1:  # warm-up, and the launch count for `seconds`
            H.mfma_rate_probe(kind, iters, st)
            torch.cuda.synchronize()
        t0 = time.perf_counter()
        H.mfma_rate_probe(kind, iters, st)
        torch.cuda.synchronize()
        n = max(10, int(seconds / max(time.perf_counter() - t0, 1e-4)))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with ClockSampler() as clk:
            e0.record(st)
            ops = sum(H.mfma_rate_probe(kind, iters, st) for _ in range(n))
            e1.record(st)
            e1.synchronize()
        ms = e0.elapsed_time(e1)
        out[name] = {"tops": round(ops / (ms * 1e-3) / 1e12, 1), "launches": n,
                     "ms": round(ms, 2), "clock": clk.summary()}
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
    if os.path.exists(trace):
        # one kernel serves launches of different sizes (a product and the backward's paired
        # products, rotation passes of different shapes): split each kernel by launch grid
        with open(trace) as f:
            tr = sorted(csv.DictReader(f), key=lambda r: int(r["Start_Timestamp"]))
        by = {}
        for r in tr:
            grid = int(r["Grid_Size_X"]) if r.get("Grid_Size_X") else 0
            wg = int(r["Workgroup_Size_X"]) if r.get("Workgroup_Size_X") else 0
            d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
            by.setdefault((r["Kernel_Name"], grid, wg), []).append(d)
        lines += ["", "by kernel and launch grid (from the trace):",
                  f"{'calls':>6} {'avg us':>9} {'min us':>9} {'max us':>9} {'workgroups':>10}  kernel"]
        for (name, grid, wg), v in sorted(by.items(), key=lambda kv: -sum(kv[1])):
            lines.append(f"{len(v):>6} {float(np.mean(v)):>9.2f} {min(v):>9.2f} {max(v):>9.2f} "
                         f"{grid // wg if wg else 0:>10}  {name[:120]}")
    if last and os.path.exists(trace):
        lines += ["", f"per pass, last {last} calls (the event-timed measurement loop):"]
        for key in PASSES:
            calls = {}
            for r in tr:
                grid = int(r["Grid_Size_X"]) if r.get("Grid_Size_X") else None
                if pass_match(key, r["Kernel_Name"], grid):
                    d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
                    calls.setdefault(r["Kernel_Name"], []).append(d)
            if calls:
                per = sum(float(np.mean(v[-last:])) for v in calls.values())
                lines.append(f"  {key:<14} {per:>9.2f} us per call ({len(calls)} kernel(s))")
    return "\n".join(lines) + "\n"


def _counter_means(d):
    """{pass: {counter: mean value per call}} from the counter_collection.csv files under d
    (each pass's kernels summed, each kernel averaged over its dispatches)."""
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    per = {}
    for fn in files:
        with open(fn) as f:
            for r in csv.DictReader(f):
                grid = int(r["Grid_Size"]) if r.get("Grid_Size") else None
                per.setdefault((r["Kernel_Name"], grid, r["Counter_Name"]), []).append(
                    float(r["Counter_Value"]))
    out = {}
    for key in PASSES:
        for (name, grid, counter), vals in per.items():
            if pass_match(key, name, grid):
                c = out.setdefault(key, {})
                c[counter] = c.get(counter, 0.0) + float(np.mean(vals))
    return out


def summarize_counters(dirs, commands):
    """Text summary of rocprofv3 --pmc runs of --kernels-only (one directory per counter
    pass): each counter's mean per call of each pass, and for the products the matrix-core
    figures derived from them."""
    merged = {}
    for d in dirs:
        for key, cs in _counter_means(d).items():
            merged.setdefault(key, {}).update(cs)
    lines = [f"command (pass {i + 1}): {c}" for i, c in enumerate(commands)]
    lines += ["", "Average counter value per call (all XCDs summed):"]
    for key in PASSES:
        if key not in merged or key == "copy_neg":
            continue
        lines.append(f"  {key}")
        for counter in sorted(merged[key]):
            lines.append(f"    {counter:<32} {merged[key][counter]:>12.4g}")
    for key, mops in (("gemm_i8_4096", "SQ_INSTS_VALU_MFMA_MOPS_I8"),
                      ("gemm_fp8_4096", "SQ_INSTS_VALU_MFMA_MOPS_F8")):
        c = merged.get(key, {})
        lines += ["", f"Derived for {key}:"]
        if mops in c:
            lines.append(f"  MFMA ops = {mops} x 512 = {c[mops] * 512 / 1e9:.1f} G "
                         f"(2 x 4096^3 = {GEMM_OPS / 1e9:.1f} G)")
        if "SQ_VALU_MFMA_BUSY_CYCLES" in c and "GRBM_GUI_ACTIVE" in c:
            per_xcd = c["GRBM_GUI_ACTIVE"] / 8
            lines.append(f"  GRBM_GUI_ACTIVE / 8 XCDs = {per_xcd:.0f} cycles per call")
            lines.append(f"  MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x that) = "
                         f"{100 * c['SQ_VALU_MFMA_BUSY_CYCLES'] / (1024 * per_xcd):.1f} %")
        if "SQ_WAIT_INST_ANY" in c and "SQ_WAVE_CYCLES" in c:
            lines.append(f"  SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES = "
                         f"{100 * c['SQ_WAIT_INST_ANY'] / c['SQ_WAVE_CYCLES']:.1f} %")
        if "SQ_LDS_BANK_CONFLICT" in c:
            lines.append(f"  LDS bank conflicts: {c['SQ_LDS_BANK_CONFLICT']:.0f}")
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
                grid = int(r["Grid_Size"]) if r.get("Grid_Size") else None
                per_kernel.setdefault((r["Kernel_Name"], grid), []).append(
                    float(r["Counter_Value"]))
    out = {}
    for key in PASSES:
        tot = 0.0
        found = False
        for (name, grid), vals in per_kernel.items():
            if pass_match(key, name, grid):
                tot += float(np.mean(vals))
                found = True
        out[key] = tot if found else None
    return out


def summarize_pmc(fetch_dir, write_dir, command):
    fetch = _pmc_per_call(fetch_dir, "FETCH_SIZE")
    write = _pmc_per_call(write_dir, "WRITE_SIZE")
    # calibration: the elementwise negation of COPY_BYTES reads and writes exactly COPY_BYTES
    f_scale = COPY_BYTES / (fetch["copy_neg"] * 1024.0)
    w_scale = COPY_BYTES / (write["copy_neg"] * 1024.0)
    algo = {"gemm_i8_4096": GEMM_BYTES, "gemm_fp8_4096": GEMM_BYTES, "fq_rows_4096": FQ_BYTES,
            "fq_cols_4096": FQ_BYTES, "fq_rows_opt_4096": FQ_BYTES, "fq_cols_opt_4096": FQ_BYTES,
            "fq_batch_4096": 4 * FQ_BYTES, "gemm_i8_pair_4096": 2 * GEMM_BYTES,
            "fq_dual_4096": DUAL_BYTES, "fq_cols_f32_4096": FQ_F32_BYTES}
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


def workload_passes(cfg):
    """The rotation passes and products of one workload: rotation passes (name, source, axis,
    code key) and products (name, pass giving a, pass giving b)."""
    fq, products = [], []
    if cfg["fwd"]:
        fq += [("x_rows", "x", 0, "q"), ("w_rows", "w", 0, "q")]
        products += [("y", "x_rows", "w_rows")]
    if cfg["bwd"]:
        fq += [("dy_rows", "dy", 0, "gq"), ("w_cols", "w", 1, "q"), ("dy_cols", "dy", 1, "gq"),
               ("x_cols", "x", 1, "q")]
        products += [("dx", "dy_rows", "w_cols"), ("dw", "dy_cols", "x_cols")]
    return fq, products


def workload_per_pass(H, torch, cfg, host, dev_src, iters=20):
    """Each pass of a workload alone, on the GPU (HIP events over `iters` back-to-back calls
    through the binding, outputs preallocated) and by the oracle on the host cores: rotation
    passes at full size, products on the first 256 rows of their a operand with the oracle's
    own codes, scaled linearly by rows ("extrapolated").  Returns the cpu_baseline object."""
    import oracle as O
    b = cfg["block"]
    tq = {"i8": torch.int8, "e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}
    oq = {"i8": O.I8, "e4m3": O.E4M3, "e5m2": O.E5M2}
    fq, products = workload_passes(cfg)
    passes, gpu_codes, cpu_codes = {}, {}, {}
    for pname, src, axis, key in fq:
        x = dev_src[src]
        rows, cols = x.shape
        nvec, L = (rows, cols) if axis == 0 else (cols, rows)
        q = torch.empty((nvec, H.padded_len(L, b)), dtype=tq[cfg[key]], device="cuda:0")
        sc = torch.empty(nvec, dtype=torch.float32, device="cuda:0")
        need = H.fwht_quant_workspace_bytes(rows, cols, axis, b, x.dtype)
        ws = torch.empty(need, dtype=torch.uint8, device="cuda:0") if need else False

        def call(i, x=x, axis=axis, key=key, q=q, sc=sc, ws=ws):
            H.fwht_quant(x, axis=axis, block=b, q_dtype=tq[cfg[key]], q=q, scale=sc,
                         workspace=ws)
        for i in range(3):
            call(i)
        g_ms = time_events(call, iters, torch)
        gpu_codes[pname] = (q, sc, cfg[key])
        t0 = time.perf_counter()
        cpu_codes[pname] = O.fwht_quant(host[src], axis, b, oq[cfg[key]])
        c_ms = (time.perf_counter() - t0) * 1e3
        passes[pname] = {"gpu_ms": round(g_ms, 4), "cpu_ms": round(c_ms, 1),
                         "ratio": round(c_ms / g_ms, 1), "extrapolated": False}
    for pname, pa, pb in products:
        qa, sa, ka = gpu_codes[pa]
        qb, sb, kb = gpu_codes[pb]
        c = torch.empty((qa.shape[0], qb.shape[0]), dtype=torch.bfloat16, device="cuda:0")

        def call(i, qa=qa, sa=sa, qb=qb, sb=sb, c=c, ka=ka):
            if ka == "i8":
                H.gemm_i8(qa, sa, qb, sb, c=c)
            else:
                H.gemm_fp8(qa, sa, qb, sb, c=c)
        for i in range(3):
            call(i)
        g_ms = time_events(call, iters, torch)
        (ca, csa), (cb, csb) = cpu_codes[pa], cpu_codes[pb]
        rows = min(256, ca.shape[0])
        t0 = time.perf_counter()
        if ka == "i8":
            acc = O.gemm_i8(ca[:rows], cb).astype(np.float64)
        else:
            acc = O.gemm_fp8(ca[:rows], oq[ka], cb, oq[kb])
        O.dequant(acc, csa[:rows], csb)
        c_ms = (time.perf_counter() - t0) * 1e3 * ca.shape[0] / rows
        passes[pname] = {"gpu_ms": round(g_ms, 4), "cpu_ms": round(c_ms, 1),
                         "ratio": round(c_ms / g_ms, 1), "extrapolated": rows < ca.shape[0]}
    return {"kind": "oracle", "unit": "ms", "cores": O.num_threads(), "cpu_model": cpu_model(),
            "passes": passes,
            "sample": "each rotation pass at full size; each product on the first 256 rows of "
                      "its a operand (the oracle's own codes), scaled by rows where marked "
                      "extrapolated; GPU: the same pass alone, HIP events over back-to-back calls "
                      "on one input (operands under 256 MB may stay in the Infinity Cache, so "
                      "these are warm-cache GPU times, unlike the headline line's legs)"}


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
    host = {"x": x, "w": w, "dy": dy}
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
    if not args.no_cpu_baseline:
        print(f"{name}: each pass alone, GPU and oracle", file=sys.stderr, flush=True)
        out["cpu_baseline"] = workload_per_pass(H, torch, cfg, host,
                                                {"x": X, "w": W, "dy": DY})
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
    ap.add_argument("--summarize-counters", nargs="+", metavar="DIR",
                    help="rocprofv3 --pmc output directories, one per counter pass")
    ap.add_argument("--commands", nargs="+", default=[],
                    help="the profiling command of each --summarize-counters pass")
    ap.add_argument("--command", default="", help="profiling command recorded in a summary")
    ap.add_argument("--out", help="summary file to write")
    ap.add_argument("--last", type=int, default=0, help="trace calls per pass to average")
    ap.add_argument("--workload", help="time one named parity workload instead (see synth)")
    ap.add_argument("--settle-s", type=float, default=2.0,
                    help="seconds of steps before the counted warmup (clock settle)")
    ap.add_argument("--one-thread-sample", action="store_true", help=argparse.SUPPRESS)
    args = ap.parse_args()

    if args.one_thread_sample:
        _one_thread_sample()
        return

    if args.summarize_stats:
        text = summarize_stats(args.summarize_stats, args.command, args.last)
        if args.out:
            with open(args.out, "w") as f:
                f.write(text)
        print(text, end="")
        return
    if args.summarize_counters:
        text = summarize_counters(args.summarize_counters, args.commands)
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

    clk = ClockSampler()
    settle_steps, settle_s = settle(step, args.settle_s, torch, sampler=clk)
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
    with ClockSampler() as clk_k:
        t = measure_kernels(H, torch, sets, args.kernel_iters)
    t_large = measure_large_passes(H, torch, max(5, args.kernel_iters // 6))
    mfma = measure_mfma_sustained(H, torch)
    i8_sustained = mfma[H.MFMA_PROBE_KINDS[0]]["tops"]
    fp8_sustained = mfma[H.MFMA_PROBE_KINDS[1]]["tops"]
    t_gemm, t_rows, t_cols = t["gemm_i8_4096"], t["fq_rows_4096"], t["fq_cols_4096"]
    t_gemm_path = t["gemm_i8_4096_in_path"]
    gemm_tops = GEMM_OPS / (t_gemm * 1e-3) / 1e12
    rows_gbs = FQ_BYTES / (t_rows * 1e-3) / 1e9
    cols_gbs = FQ_BYTES / (t_cols * 1e-3) / 1e9

    copy_gbs = 2 * COPY_REF_BYTES / (t["copy_ref_512MiB"] * 1e-3) / 1e9

    def hbm(gbs, ms, key, nbytes=FQ_BYTES):
        return {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 4), "frac_of_copy": round(gbs / copy_gbs, 4),
                "traffic": load_traffic(key), "ms_per_launch": round(ms, 5),
                "algorithmic_bytes": nbytes}

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
        "settle": {"steps": settle_steps, "s": round(settle_s, 2),
                   "what": "steps run before the counted warmup, until the clock settles"},
        "clock": {"steps": clk.summary() | {
                      "what": "sampled every 10 ms from 40 % to 80 % of the clock-settle "
                              "phase: the same steps in steady state (the counted steps run "
                              "unsampled: sampling slows them by about 2 %)"},
                  "kernel_legs": clk_k.summary()},
        "roofline": {"bound": "mfma", "achieved": round(gemm_tops, 2), "peak": PEAK_INT8_TOPS,
                     "unit": "TFLOP/s", "frac": round(gemm_tops / PEAK_INT8_TOPS, 4),
                     "traffic": load_traffic("gemm_i8_4096"),
                     "kernel": "gemm_kernel<INT8, bf16 out> 4096x4096x4096",
                     "ms_per_launch": round(t_gemm, 5), "algorithmic_ops": GEMM_OPS,
                     "measured": "back-to-back launches cycling 18 pairs of 16 MiB code "
                                 "matrices (604 MB), none left in the Infinity Cache",
                     "instruction_sustained": {
                         "achieved": i8_sustained, "unit": "TFLOP/s",
                         "frac": round(gemm_tops / i8_sustained, 4),
                         "what": "v_mfma_i32_32x32x32_i8 alone on the whole device under a "
                                 "sustained load, on operands drawn like the product's codes, "
                                 "a different fragment pair for every MFMA "
                                 "(halo_mfma_rate_probe): the rate the chip's clock allows "
                                 "this instruction on such data; frac = the product's rate "
                                 "over it"},
                     "in_path": {"ms_per_launch": round(t_gemm_path, 5),
                                 "frac": round(GEMM_OPS / (t_gemm_path * 1e-3) / 1e12
                                               / PEAK_INT8_TOPS, 4),
                                 "what": "as the forward runs it: codes written just before by "
                                         "the rows passes of that step's X and W, events around "
                                         "the product alone"}},
        "fwht_quant": {"rows": hbm(rows_gbs, t_rows, "fq_rows_4096"),
                       "cols": hbm(cols_gbs, t_cols, "fq_cols_4096"),
                       "copy_reference": {
                           "achieved": round(copy_gbs, 1), "unit": "GB/s",
                           "frac": round(copy_gbs / PEAK_HBM_GBS, 4),
                           "what": "torch elementwise negation, 512 MiB read + 512 MiB written "
                                   "per launch: the streaming rate a plain copy reaches here; "
                                   "frac_of_copy of each pass is against it"},
                       "dual": hbm_pass("fq_dual_4096", DUAL_BYTES) | {
                           "two_passes_ms": round(t_rows + t_cols, 5),
                           "what": "halo_fwht_quant_dual: the rows and the columns codes of one "
                                   "4096 x 4096 bf16 matrix from a single read (algorithmic: "
                                   "one read, both code matrices and scales), beside the rows "
                                   "pass plus the columns pass"},
                       "cols_f32": hbm_pass("fq_cols_f32_4096", FQ_F32_BYTES) | {
                           "what": "the columns pass on fp32 input (4 B read + 1 B code per "
                                   "element): the same single-read tasks, the tile staged "
                                   "through the LDS in two rounds"}},
        "gemm_fp8": {"bound": "mfma", "achieved": round(GEMM_OPS / (t["gemm_fp8_4096"] * 1e-3) / 1e12, 2),
                     "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(GEMM_OPS / (t["gemm_fp8_4096"] * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 4),
                     "traffic": load_traffic("gemm_fp8_4096"),
                     "kernel": "gemm_kernel<FP8 E4M3 x E4M3, bf16 out> 4096x4096x4096",
                     "ms_per_launch": round(t["gemm_fp8_4096"], 5), "algorithmic_ops": GEMM_OPS,
                     "instruction_sustained": {
                         "achieved": fp8_sustained, "unit": "TFLOP/s",
                         "frac": round(GEMM_OPS / (t["gemm_fp8_4096"] * 1e-3) / 1e12
                                       / fp8_sustained, 4),
                         "what": "v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3) alone, as above"}},
        "mfma_sustained": mfma,
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
        cb = cpu_baseline()
        gpu_ms = {"fq": (t_rows + t_cols) / 2, "product": t_gemm}
        cb["oracle_over_gpu"] = {k: round(cb["per_pass_ms"][k] / gpu_ms[k], 1) for k in gpu_ms}
        result["cpu_baseline"] = cb
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
