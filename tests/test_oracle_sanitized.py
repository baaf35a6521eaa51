"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

oracle/rrp_oracle.c is built with gcc -fsanitize=address,undefined into a
temporary library, which the whole pin suite then loads through
RRP_ORACLE_LIB (the Python interpreter is not instrumented, so the ASan
runtime is preloaded).  Every out-of-bounds access, use after free or
undefined operation in the oracle aborts the run.  A copy with one planted
one-byte overflow (the nibble packer writing a byte past its row) must be
caught, which shows the sanitizers are live in this harness.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "rrp_oracle.c")
PINS = os.path.join(ROOT, "tests", "test_oracle_pins.py")

PLANTED_OVERFLOW = ("for (int i = 0; i < n / 2; ++i)\n        bytes[i]",
                    "for (int i = 0; i <= n / 2; ++i)\n        bytes[i]")


def _runtime(name):
    r = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


def _build(src_text, out_dir, name):
    csrc = os.path.join(out_dir, name + ".c")
    so = os.path.join(out_dir, name + ".so")
    with open(csrc, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", "-O1", "-g", "-std=gnu11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC",
                    "-shared", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", "-I", os.path.join(ROOT, "oracle"), csrc, "-o", so, "-lm"],
                   check=True)
    return so


def _run_pins(so, asan, log_dir, *extra):
    """Runs the pin suite on the sanitized library; returns (process, sanitizer reports).
    The reports go to files: pytest's own capture would swallow them on an abort."""
    log = os.path.join(log_dir, "san")
    env = dict(os.environ, RRP_ORACLE_LIB=so, LD_PRELOAD=asan, OMP_NUM_THREADS="2",
               ASAN_OPTIONS=f"detect_leaks=0:abort_on_error=1:log_path={log}",
               UBSAN_OPTIONS=f"halt_on_error=1:print_stacktrace=1:log_path={log}")
    r = subprocess.run([sys.executable, "-m", "pytest", PINS, "-x", "-q", "-p", "no:warnings",
                        "-p", "no:cacheprovider", *extra], env=env, cwd=ROOT, capture_output=True, text=True)
    reports = ""
    for name in sorted(os.listdir(log_dir)):
        if name.startswith("san."):
            with open(os.path.join(log_dir, name)) as f:
                reports += f.read()
    return r, reports


@pytest.fixture(scope="module")
def asan_runtime():
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    return asan


def test_pin_suite_is_clean_under_asan_and_ubsan(tmp_path, asan_runtime):
    so = _build(open(SRC).read(), str(tmp_path), "orc_san")
    r, reports = _run_pins(so, asan_runtime, str(tmp_path))
    assert r.returncode == 0 and not reports, (r.stdout[-3000:], reports[-3000:])
    assert "passed" in r.stdout


def test_planted_overflow_is_caught(tmp_path, asan_runtime):
    src = open(SRC).read()
    before, after = PLANTED_OVERFLOW
    assert before in src
    so = _build(src.replace(before, after, 1), str(tmp_path), "orc_san_overflow")
    r, reports = _run_pins(so, asan_runtime, str(tmp_path), "-k", "test_pack_roundtrip_with_numpy_unpack")
    assert r.returncode != 0
    assert "AddressSanitizer" in reports and "buffer-overflow" in reports, (r.stderr[-2000:], reports[-2000:])
