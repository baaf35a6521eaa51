"""Host-side logic of bench.py (no GPU): the one-GPU contract, the algorithmic
byte count behind roofline.achieved, and the rule that the committed traffic
counters are reported only for the kernel source they were taken on."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from rotation_rope_pair_amd import workloads as W  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_prefill_bytes_per_launch():
    """Q read and written back (bf16), K read (bf16), K codes (d/2 bytes per row),
    fp16 scales (d/g per row) and the int32 position, per token of the 128K
    prefill: 18 964 bytes, 2 485 649 408 per launch."""
    w = W.WORKLOADS[4]
    T, hq, hk, d, g = 131072, 32, 8, 128, 128
    assert (w.n_tokens, w.n_q_heads, w.n_kv_heads, w.head_dim) == (T, hq, hk, d)
    per_token = 2 * (hq * d * 2) + hk * d * 2 + hk * d // 2 + 2 * hk * (d // g) + 4
    assert per_token == 18964
    assert w.bytes_per_token(group=g, with_slot=False) == per_token
    assert w.bytes_per_token(group=g, with_slot=False) * T == 2485649408


def test_traffic_only_for_the_current_kernel_source(tmp_path, monkeypatch):
    f = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic() is None  # no summary
    f.write_text(json.dumps({"kernel_source_hash": "0" * 16, "hbm_bytes_per_launch": 123.0}))
    assert bench.measured_traffic() is None  # taken on another kernel source
    f.write_text(json.dumps({"kernel_source_hash": bench.kernel_source_hash(), "hbm_bytes_per_launch": 123.0}))
    assert bench.measured_traffic() == 123.0


def test_kernel_source_hash_covers_the_hot_kernel_files():
    for rel in bench.KERNEL_SOURCES:
        assert os.path.isfile(os.path.join(ROOT, rel)), rel
    assert any(rel.endswith("rrp_rotate_kernel.hpp") for rel in bench.KERNEL_SOURCES)
    assert len(bench.kernel_source_hash()) == 16


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
def test_bytes_per_token_counts_every_stream(n):
    """The V half adds exactly its read, codes and scales; a slot mapping adds 8 bytes."""
    w = W.WORKLOADS[n]
    d, hk, e, g = w.head_dim, w.n_kv_heads, w.elem_bytes, w.group
    base = w.bytes_per_token(with_slot=False)
    assert w.bytes_per_token(with_slot=True) == base + 8
    assert w.bytes_per_token(with_slot=False, with_v=True) == base + hk * d * e + hk * d // 2 + 2 * hk * (d // g)


def test_stream_probe_library_exports_and_rejects_bad_arguments():
    """The streaming-ceiling kernels' library loads and checks sizes and alignment
    on the host (nothing is launched on these calls)."""
    import ctypes
    if not os.path.exists(bench.PROBE_LIB):
        from rotation_rope_pair_amd import build
        build.build()
    L = ctypes.CDLL(bench.PROBE_LIB)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    L.stream_probe_copy.argtypes = [vp, vp, sz, vp]
    L.stream_probe_read.argtypes = [vp, sz, vp, vp]
    L.stream_probe_write.argtypes = [vp, sz, vp]
    p16, p8 = vp(1 << 20), vp((1 << 20) + 8)
    assert L.stream_probe_copy(None, p16, 64, None) == 1 and L.stream_probe_copy(p16, p8, 64, None) == 1
    assert L.stream_probe_copy(p16, p16, 40, None) == 1
    assert L.stream_probe_read(p16, 64, None, None) == 1 and L.stream_probe_read(p8, 64, p16, None) == 1
    assert L.stream_probe_write(p8, 64, None) == 1 and L.stream_probe_write(p16, 24, None) == 1


def test_per_config_rotated_sets_span_past_the_infinity_cache():
    """The per-workload timings rotate enough buffer sets to span 1 GiB (at least
    four, at most 256), so launches stream from HBM except where 256 sets of a tiny
    workload still fit the 256 MB cache, which the record then says."""
    assert bench.ROTATED_FOOTPRINT >= 4 * bench.INFINITY_CACHE_BYTES
    for n in (1, 2, 3, 5):
        w = W.WORKLOADS[n]
        T, d, hq, hk, g, e = w.n_tokens, w.head_dim, w.n_q_heads, w.n_kv_heads, w.group, w.elem_bytes
        set_bytes = 2 * T * hq * d * e + T * hk * d * e + 4 * T + T * hk * (d // 2 + 2 * (d // g))
        n_sets = int(min(256, max(4, -(-bench.ROTATED_FOOTPRINT // set_bytes))))
        assert n_sets >= 4
        assert n_sets * set_bytes >= bench.ROTATED_FOOTPRINT or n_sets == 256
