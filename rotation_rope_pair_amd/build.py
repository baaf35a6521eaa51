"""Compile the HIP library (gfx950) in-tree: rotation_rope_pair_amd/librrp.so.

Each .hip translation unit is compiled to an object in parallel, then linked
into one shared library whose only exported symbols are the rrp_* entry points
of include/rrp.h.  Packed-fp32 instructions are disabled for the device code.
The benchmark's streaming-ceiling kernels (stream_probe.hip) go into a library
of their own, libstream_probe.so, which only bench.py loads.
"""
import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "librrp.so")
SOURCES = ["rrp_rotate.hip", "rrp_rotate_split.hip", "rrp_stats.hip", "rrp_sweep_bf16.hip", "rrp_sweep_f32.hip",
           "rrp_decode.hip", "rrp_calib.hip", "rrp_abi.hip"]
PROBE_LIB = os.path.join(HERE, "libstream_probe.so")
PROBE_SOURCES = ["stream_probe.hip"]
ARCH = os.environ.get("RRP_OFFLOAD_ARCH", "gfx950")


def hipcc():
    for cand in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"), shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: install ROCm or set ROCM_PATH")


def common_flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
        "-Wall", "-Wno-unused-function",
    ]


# Per-source flags.  The diagnostics kernels compare fp64 values with max / min
# (group absmax and range); K rows are finite by contract, and without NaN
# semantics those need no operand canonicalisation.
EXTRA_FLAGS = {s: ["-fno-honor-nans"] for s in ("rrp_stats.hip", "rrp_sweep_bf16.hip", "rrp_sweep_f32.hip")}


def _compile(src, verbose):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + common_flags() + EXTRA_FLAGS.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the device-only target feature: drop that warning
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    return obj


def _link(objs, lib, verbose):
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC"] + objs + ["-o", lib + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(lib + ".tmp", lib)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(7, os.cpu_count() or 1)) as ex:
        objs = dict(zip(srcs, ex.map(lambda s: _compile(s, verbose), srcs)))
    _link([objs[s] for s in SOURCES], LIB, verbose)
    _link([objs[s] for s in PROBE_SOURCES], PROBE_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
