"""Build libhalo.so (the gfx950 HIP kernels + the C ABI) in-tree with hipcc."""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libhalo.so")
SOURCES = ["halo_api.hip", "fwht_quant.hip", "fwht_wave.hip", "fwht_wave_sr.hip", "fwht_dual.hip",
           "gemm.hip", "mfma_probe.hip"]
HEADERS = ["halo_device.h", "halo_kernels.h", "fwht_wave.h"]

# -packed-fp32-ops off: hipcc -O3 would otherwise form v_pk_*_f32 from scalar float code.
HIPFLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I" + os.path.join(ROOT, "include")]


def _compile(src, verbose):
    obj = os.path.join(CSRC, os.path.splitext(src)[0] + ".o")
    cmd = ["hipcc", *HIPFLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip() and verbose:
        print(err, flush=True)
    return obj


def build(verbose: bool = False) -> str:
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    cmd = ["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", "-o", LIB + ".tmp", *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    for o in objs:
        os.remove(o)
    return LIB


def build_host_sanitized(out: str, verbose: bool = False) -> str:
    """The library with its host code built with AddressSanitizer and UndefinedBehaviorSanitizer
    (-Xarch_host: the device code is built as usual and never instrumented), for the CPU test
    that runs the C ABI's argument validation and size queries under them."""
    flags = ["--offload-arch=gfx950", "-O1", "-Xarch_host", "-g", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fsanitize=address",
             "-Xarch_host", "-fsanitize=undefined", "-Xarch_host",
             "-fno-sanitize-recover=undefined", "-I" + os.path.join(ROOT, "include")]
    tmp = os.path.dirname(os.path.abspath(out))

    def one(src):
        obj = os.path.join(tmp, os.path.splitext(src)[0] + ".san.o")
        cmd = ["hipcc", *flags, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc (sanitized host) failed on {src}:\n{r.stderr}")
        return obj

    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(one, SOURCES))
    cmd = ["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host",
           "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-shared-libasan",
           "-o", out, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True, capture_output=not verbose)
    for o in objs:
        os.remove(o)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
