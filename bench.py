"""Benchmark of the Q/K rotate + INT4-quantise hot path on one MI355X.

A step is one rrp_rotate_quantize_qk launch over the whole 131072-token
Llama-3.1-8B-shaped prefill batch (32 Q / 8 KV heads, head_dim 128, RoPE theta
5e5, bf16, b = 128, group = 128, KV4 cache write): RoPE, the shared pair
rotation by the calibrated angles, the block Hadamard, the Q store and the K
group quantisation / nibble packing.  Inputs are resident in HBM before the
timed region.  Prints one JSON line.

    python bench.py [--gpus 1] [--steps 200] [--warmup 50] [--no-cpu-baseline] [--hot-path-only]

A step takes about half a millisecond.  After the --warmup launches, at
least 100 ms of untimed launches run back to back (the clocks settle; the
first few tens of launches of a process are slower) before the timed window,
whatever --warmup says; the JSON line records that settle time and its launch
count, and the per-launch median, min and max beside the mean.

--hot-path-only skips the supporting passes, the per-workload timings, the
decode timing and the CPU baseline (short runs under a profiler).  Every run
also times torch's device-to-device copy of the Q tensor (known size: 1 GiB
read + 1 GiB written; the reference kernel that scales the profiler's
FETCH_SIZE / WRITE_SIZE counters) and the streaming-ceiling kernels of
libstream_probe.so (copy, read-only and write-only at the same size).
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "Q/K rotate+INT4-quantise tokens/sec and achieved HBM GB/s (% of peak), 1 GPU"
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "rotate_quantize_prefill128k_traffic.json")
KERNEL_SOURCES = ["rotation_rope_pair_amd/csrc/rrp_device.hpp", "rotation_rope_pair_amd/csrc/rrp_rotate.hip",
                  "rotation_rope_pair_amd/csrc/rrp_rotate.hpp", "rotation_rope_pair_amd/csrc/rrp_rotate_kernel.hpp"]


def kernel_source_hash():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was
    taken on the current kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_baseline(w, inp, angles_np, budget_s=12.0):
    """The CPU oracle (untuned) on a bounded prefix of the same workload."""
    import oracle as O
    shp = O.shape(w.n_q_heads, w.n_kv_heads, w.head_dim, w.rope_theta)
    n = 256
    t0 = time.perf_counter()
    O.rotate_quantize_qk(shp, inp["q"][:n], inp["k"][:n], inp["pos"][:n], angles_np, 128, 128)
    per_tok = (time.perf_counter() - t0) / n
    n = int(min(w.n_tokens, max(256, budget_s / max(per_tok, 1e-9))))
    t0 = time.perf_counter()
    O.rotate_quantize_qk(shp, inp["q"][:n], inp["k"][:n], inp["pos"][:n], angles_np, 128, 128)
    dt = time.perf_counter() - t0
    threads = O.max_threads()
    # the same oracle on one thread, over a smaller prefix (about 3 s)
    n1 = int(min(w.n_tokens, max(64, 3.0 / max(per_tok * threads, 1e-9))))
    prev = O.set_threads(1)
    try:
        t0 = time.perf_counter()
        O.rotate_quantize_qk(shp, inp["q"][:n1], inp["k"][:n1], inp["pos"][:n1], angles_np, 128, 128)
        dt1 = time.perf_counter() - t0
    finally:
        O.set_threads(prev)
    return {"value": n / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"first {n} of {w.n_tokens} tokens, same inputs and angles, {dt:.1f} s",
            "single_thread": {"value": n1 / dt1, "unit": "tokens/s", "cores": 1,
                              "sample": f"first {n1} tokens, {dt1:.1f} s"}}


def to_device_bf16(a, dev):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)


def decode_latency_us(dev, stream, reps=200):
    """Per-launch time of the 256-token Mistral-shaped decode batch (slot scatter
    into a 256 x 32768-slot KV4 cache), three ways: launches through the Python
    binding (its argument checks cost more host time than the kernel takes), the
    binding's prepared call (checked and marshalled once, then re-issued), and
    back-to-back calls of the C entry point with the arguments marshalled once,
    which keeps the GPU busy and so times the kernel itself."""
    import torch
    import rotation_rope_pair_amd as rrp
    from rotation_rope_pair_amd import workloads as W
    w5 = W.WORKLOADS[5]
    inp5 = W.make_inputs(5)
    shape5 = rrp.layer_shape(w5.n_q_heads, w5.n_kv_heads, w5.head_dim, w5.rope_theta)
    q5, k5 = to_device_bf16(inp5["q"], dev), to_device_bf16(inp5["k"], dev)
    pos5 = torch.from_numpy(inp5["pos"]).to(dev)
    sm5 = torch.from_numpy(inp5["slot_mapping"]).to(dev)
    c5, s5 = rrp.new_kv4_cache(inp5["n_slots"], w5.n_kv_heads, w5.head_dim, w5.group, dev)
    q5o = torch.empty_like(q5)
    a5 = torch.zeros(w5.n_pairs, dtype=torch.float32, device=dev)

    def launch():
        rrp.rotate_quantize_qk(shape5, q5, k5, pos5, support_b=128, group=w5.group, k_codes=c5, k_scales=s5,
                               angles=a5, q_out=q5o, slot_mapping=sm5, n_slots=inp5["n_slots"])
    from rotation_rope_pair_amd import _abi, api
    L = _abi.load()
    args = api._rotate_args(shape5, q5, k5, None, pos5, 128, w5.group, c5, s5, None, None, a5, q5o, sm5,
                            inp5["n_slots"], None, None, None, None, None, None)

    def launch_c():
        _abi.check("rrp_rotate_quantize_qk", L.rrp_rotate_quantize_qk(*args))
    prepared = rrp.prepare_rotate_quantize_qk(shape5, q5, k5, pos5, support_b=128, group=w5.group, k_codes=c5,
                                              k_scales=s5, angles=a5, q_out=q5o, slot_mapping=sm5,
                                              n_slots=inp5["n_slots"])
    out = {}
    for key, fn in (("decode256_rotate_quantize_us", launch_c),
                    ("decode256_rotate_quantize_us_python_binding", launch),
                    ("decode256_rotate_quantize_us_prepared_call", prepared)):
        for _ in range(10):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        out[key] = e0.elapsed_time(e1) / reps * 1e3
    return out


SETTLE_MS = 100.0  # untimed back-to-back launches before the hot-path window


def settle(fn, ms_each, total_ms=25.0):
    """Untimed launches worth about total_ms, so the clocks settle before a
    supporting timing."""
    for _ in range(max(3, int(total_ms / max(ms_each, 1e-3)))):
        fn()


def settle_for(fn, stream, total_ms):
    """Untimed launches of fn until at least total_ms of GPU time has passed
    (measured with events on `stream`); returns the number of launches."""
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n, batch = 0, 8
    e0.record(stream)
    while True:
        for _ in range(batch):
            fn()
        n += batch
        e1.record(stream)
        e1.synchronize()
        spent = e0.elapsed_time(e1)
        if spent >= total_ms:
            return n
        # enqueue the rest in one go (no host wait between launches)
        batch = max(8, int((total_ms - spent) / max(spent / n, 1e-3)) + 1)


def qkv_timing(w, shape, q, k, pos, angles, q_out, codes, scales, dev, stream, b, g, reps=50):
    """The same prefill launch with the V half of the KV4 cache written too
    (one more read stream: V rows through the full-head Hadamard into INT4)."""
    import torch
    import rotation_rope_pair_amd as rrp
    from rotation_rope_pair_amd import workloads as W
    v = to_device_bf16(W.make_v(w.number), dev)
    vc, vs = rrp.new_kv4_cache(w.n_tokens, w.n_kv_heads, w.head_dim, g, dev)

    def launch():
        rrp.rotate_quantize_qkv(shape, q, k, v, pos, support_b=b, group=g, k_codes=codes, k_scales=scales,
                                v_codes=vc, v_scales=vs, angles=angles, q_out=q_out)
    settle(launch, 0.55)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        launch()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    nbytes = w.bytes_per_token(group=g, with_slot=False, with_v=True) * w.n_tokens
    return {"rotate_quantize_qkv_ms": ms, "qkv_bytes_per_launch": nbytes,
            "qkv_hbm_gbs": nbytes / (ms * 1e-3) / 1e9, "qkv_tokens_per_s": w.n_tokens / (ms * 1e-3)}


def per_head_timing(w, q, k, pos, q_out, codes, scales, dev, stream, b, g, reps=50):
    """The same prefill with one angle set per key head: per-set calibration, then
    the rotate launch reading each head's own set."""
    import torch
    import rotation_rope_pair_amd as rrp
    hk, d = w.n_kv_heads, w.head_dim
    shape = rrp.layer_shape(w.n_q_heads, hk, d, w.rope_theta, angle_heads=hk)
    moments = rrp.new_moments(d, dev, n_sets=hk)
    angles = torch.empty((hk, d // 2), dtype=torch.float32, device=dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]

    def calibrate():
        moments.zero_()
        rrp.calibrate_angles(shape, q, k, pos, moments=moments, estimator="default", angles_out=angles)
    settle(calibrate, 0.4)
    ev[0].record(stream)
    for _ in range(20):
        calibrate()
    ev[1].record(stream)

    def launch():
        rrp.rotate_quantize_qk(shape, q, k, pos, support_b=b, group=g, k_codes=codes, k_scales=scales,
                               angles=angles, q_out=q_out)
    settle(launch, 0.48)
    ev[2].record(stream)
    for _ in range(reps):
        launch()
    ev[3].record(stream)
    torch.cuda.synchronize()
    ms = ev[2].elapsed_time(ev[3]) / reps
    nbytes = w.bytes_per_token(group=g, with_slot=False) * w.n_tokens
    return {"per_head_calibrate_angles_ms": ev[0].elapsed_time(ev[1]) / 20,
            "per_head_rotate_quantize_ms": ms, "per_head_rotate_hbm_gbs": nbytes / (ms * 1e-3) / 1e9}


def decode_scores_timing(dev, stream, reps=40):
    """rrp_decode_scores over the 256-sequence decode batch (Mistral-shaped, 32 / 8
    heads, d 128, g 64) reading its 256 x 32768-slot KV4 cache: time per launch and
    algorithmic GB/s (cache rows read + logits written + queries read)."""
    import numpy as np
    import torch
    import rotation_rope_pair_amd as rrp
    from rotation_rope_pair_amd import workloads as W
    w = W.WORKLOADS[5]
    bt = W.make_decode_batch(5)
    shape = rrp.layer_shape(w.n_q_heads, w.n_kv_heads, w.head_dim, w.rope_theta)
    q = to_device_bf16(bt["q"], dev)
    codes = torch.from_numpy(bt["codes"]).to(dev)
    scales = torch.from_numpy(bt["scales"].view(np.int16)).to(dev)
    start = torch.from_numpy(bt["seq_start"]).to(dev)
    lens = torch.from_numpy(bt["seq_len"]).to(dev)
    out = torch.empty((len(bt["seq_len"]), w.n_q_heads, bt["max_len"]), dtype=torch.float32, device=dev)

    def launch():
        rrp.decode_scores(shape, q, codes, scales, group=bt["group"], seq_start=start, seq_len=lens,
                          max_len=bt["max_len"], scores=out)
    settle(launch, 0.6)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        launch()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    keys = int(np.minimum(bt["seq_len"], bt["max_len"]).sum())
    d, hq, hk, g = w.head_dim, w.n_q_heads, w.n_kv_heads, bt["group"]
    nbytes = keys * hk * (d // 2 + 2 * (d // g)) + keys * hq * 4 + len(bt["seq_len"]) * (hq * d * 2 + 12)
    return {"decode_scores_ms": ms, "decode_scores_keys": keys, "decode_scores_bytes": nbytes,
            "decode_scores_hbm_gbs": nbytes / (ms * 1e-3) / 1e9}


PROBE_LIB = os.path.join(ROOT, "rotation_rope_pair_amd", "libstream_probe.so")


def stream_ceiling(src, dst, stream, reps=20):
    """The GPU's practical streaming rates from plain kernels of known traffic
    (rotation_rope_pair_amd/csrc/stream_probe.hip: 16-byte non-temporal
    accesses, as in the rotate kernel): copy of the 1 GiB src into dst (1 GiB
    read + 1 GiB written), read-only of src, write-only of dst."""
    import ctypes
    import torch
    if not os.path.exists(PROBE_LIB):
        raise ImportError(f"{PROBE_LIB} is missing; run rotation_rope_pair_amd/build.py")
    L = ctypes.CDLL(PROBE_LIB)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    L.stream_probe_copy.argtypes = [vp, vp, sz, vp]
    L.stream_probe_read.argtypes = [vp, sz, vp, vp]
    L.stream_probe_write.argtypes = [vp, sz, vp]
    n = src.numel() * src.element_size()
    sink = torch.zeros(4, dtype=torch.int32, device=src.device)
    sp = vp(stream.cuda_stream)
    runs = {"copy": (lambda: L.stream_probe_copy(vp(src.data_ptr()), vp(dst.data_ptr()), n, sp), 2 * n),
            "read": (lambda: L.stream_probe_read(vp(src.data_ptr()), n, vp(sink.data_ptr()), sp), n),
            "write": (lambda: L.stream_probe_write(vp(dst.data_ptr()), n, sp), n)}
    out = {"kernels": "rotation_rope_pair_amd/csrc/stream_probe.hip", "bytes_per_buffer": n}
    for name, (fn, nbytes) in runs.items():
        if fn() != 0:
            raise RuntimeError(f"stream_probe_{name} failed")
        settle(fn, 0.3)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        out[f"{name}_ms"] = ms
        out[f"{name}_GBs"] = nbytes / (ms * 1e-3) / 1e9
    return out


INFINITY_CACHE_BYTES = 256 << 20  # MI355X last-level (Infinity) cache
ROTATED_FOOTPRINT = 1 << 30        # bytes the rotated buffer sets of one config span at least


def graph_us_per_launch(launches, stream, target_ms=50.0):
    """GPU time per launch of the closures in `launches`, captured once into a HIP
    graph (so no host launch cost sits between them) and replayed back to back
    for about target_ms after an untimed settle."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # first launches outside the capture
        for fn in launches:
            fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for fn in launches:
            fn()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    per_replay = max(e0.elapsed_time(e1), 1e-3)
    settle(graph.replay, per_replay, 25.0)
    replays = max(20, int(target_ms / per_replay))
    e0.record(stream)
    for _ in range(replays):
        graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (replays * len(launches))


def per_config_timing(dev, stream, with_oracle):
    """rotate_quantize_qk on each workload of the pages' shapes besides the 128K
    prefill (the tiny fp32 reference, the 1B and 3B layers, the 256-token decode
    batch): GPU time per launch over rotated buffer sets spanning at least 1 GiB
    (so successive launches do not find their inputs in the 256 MB Infinity
    Cache), through a HIP graph; tokens/s and algorithmic GB/s; and the CPU
    oracle on the same inputs (every token)."""
    import numpy as np
    import torch
    import rotation_rope_pair_amd as rrp
    from rotation_rope_pair_amd import workloads as W
    out = {}
    for n, b in ((1, 64), (2, 64), (3, 128), (5, 128)):
        w = W.WORKLOADS[n]
        g = w.group
        inp = W.make_inputs(n)
        T, d, hq, hk = w.n_tokens, w.head_dim, w.n_q_heads, w.n_kv_heads
        shape = rrp.layer_shape(hq, hk, d, w.rope_theta)
        conv = (lambda a: to_device_bf16(a, dev)) if w.dtype == "bf16" else \
            (lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev))
        q0, k0 = conv(inp["q"]), conv(inp["k"])
        pos0 = torch.from_numpy(inp["pos"]).to(dev)
        sm = None if inp["slot_mapping"] is None else torch.from_numpy(inp["slot_mapping"]).to(dev)
        n_slots = inp["n_slots"]
        src = inp["calib"] if inp["calib"] is not None else inp
        est = w.estimator
        cq = None if est == "k_only" else conv(src["q"])
        angles = torch.empty(w.n_pairs, dtype=torch.float32, device=dev)
        rrp.calibrate_angles(shape, cq, conv(src["k"]), torch.from_numpy(src["pos"]).to(dev),
                             moments=rrp.new_moments(d, dev), estimator=est, angles_out=angles)
        nbytes = w.bytes_per_token(group=g) * T
        # one set: inputs, Q output and (for the prefill shapes) the cache slots it writes
        set_bytes = 2 * q0.numel() * q0.element_size() + k0.numel() * k0.element_size() + 4 * T + \
            (T * hk * (d // 2 + 2 * (d // g)))
        n_sets = int(min(256, max(4, -(-ROTATED_FOOTPRINT // set_bytes))))
        sets = []
        shared_cache = None
        if sm is not None:  # the decode batch scatters into one 256 x 32768-slot cache, shared by every set
            shared_cache = rrp.new_kv4_cache(n_slots, hk, d, g, dev)
        for _ in range(n_sets):
            codes, scales = shared_cache if shared_cache is not None else rrp.new_kv4_cache(n_slots, hk, d, g, dev)
            sets.append((q0.clone(), k0.clone(), pos0.clone(), torch.empty_like(q0), codes, scales))

        def launcher(st):
            q, k, pos, q_out, codes, scales = st
            return lambda: rrp.rotate_quantize_qk(shape, q, k, pos, support_b=b, group=g, k_codes=codes,
                                                  k_scales=scales, angles=angles, q_out=q_out, slot_mapping=sm,
                                                  n_slots=n_slots)
        us = graph_us_per_launch([launcher(st) for st in sets], stream)
        footprint = n_sets * set_bytes
        rec = {"workload": w.name, "n_tokens": T, "heads": f"{hq}/{hk}", "head_dim": d, "dtype": w.dtype,
               "support_b": b, "group": g, "us_per_launch": us, "tokens_per_s": T / (us * 1e-6),
               "algorithmic_bytes": nbytes, "hbm_gbs": nbytes / (us * 1e-6) / 1e9,
               "frac_of_peak": nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS,
               "rotated_sets": n_sets, "footprint_bytes": footprint,
               "cache_resident": footprint < INFINITY_CACHE_BYTES,
               "timing": "HIP graph of one launch per set, replayed back to back"}
        del sets
        if with_oracle:
            import oracle as O
            shp = O.shape(hq, hk, d, w.rope_theta)
            ang = angles.cpu().numpy()
            t0 = time.perf_counter()
            O.rotate_quantize_qk(shp, inp["q"], inp["k"], inp["pos"], ang, b, g,
                                 slot_mapping=inp["slot_mapping"], n_slots=n_slots if sm is not None else None)
            dt = time.perf_counter() - t0
            rec["oracle"] = {"tokens_per_s": T / dt, "s": dt, "cores": O.max_threads(), "sample": "every token"}
        out[f"C{n}"] = rec
        torch.cuda.synchronize()
    return out


def kernels_once(w, shape, q, k, pos, angles, q_out, codes, scales, dev, b, g, launches=2):
    """Every kernel of the path and of its supporting passes, `launches` times
    each, on the benchmark's inputs, and nothing else: a short run for
    rocprofv3 counter passes (--pmc serialises every dispatch).  Prints the
    kernels it ran as one JSON line (not the benchmark's line)."""
    import numpy as np
    import torch
    import rotation_rope_pair_amd as rrp
    from rotation_rope_pair_amd import workloads as W
    hk, d = w.n_kv_heads, w.head_dim
    v = to_device_bf16(W.make_v(w.number), dev)
    vc, vs = rrp.new_kv4_cache(w.n_tokens, hk, d, g, dev)
    moments = rrp.new_moments(d, dev)
    shape_ph = rrp.layer_shape(w.n_q_heads, hk, d, w.rope_theta, angle_heads=hk)
    moments_ph = rrp.new_moments(d, dev, n_sets=hk)
    angles_ph = torch.empty((hk, d // 2), dtype=torch.float32, device=dev)
    stats = torch.empty(8, dtype=torch.float64, device=dev)
    sweep = torch.empty((len(rrp.sweep_supports(d)), 8), dtype=torch.float64, device=dev)
    w5 = W.WORKLOADS[5]
    bt = W.make_decode_batch(5)
    shape5 = rrp.layer_shape(w5.n_q_heads, w5.n_kv_heads, w5.head_dim, w5.rope_theta)
    q5 = to_device_bf16(bt["q"], dev)
    codes5 = torch.from_numpy(bt["codes"]).to(dev)
    scales5 = torch.from_numpy(bt["scales"].view(np.int16)).to(dev)
    start5 = torch.from_numpy(bt["seq_start"]).to(dev)
    lens5 = torch.from_numpy(bt["seq_len"]).to(dev)
    scores5 = torch.empty((len(bt["seq_len"]), w5.n_q_heads, bt["max_len"]), dtype=torch.float32, device=dev)
    runs = {
        "rotate_quantize_qk": lambda: rrp.rotate_quantize_qk(
            shape, q, k, pos, support_b=b, group=g, k_codes=codes, k_scales=scales, angles=angles, q_out=q_out),
        "rotate_quantize_qkv": lambda: rrp.rotate_quantize_qkv(
            shape, q, k, v, pos, support_b=b, group=g, k_codes=codes, k_scales=scales, v_codes=vc, v_scales=vs,
            angles=angles, q_out=q_out),
        "calibrate_angles": lambda: rrp.calibrate_angles(
            shape, q, k, pos, moments=moments.zero_(), estimator="default", angles_out=angles),
        "calibrate_angles_per_key_head": lambda: rrp.calibrate_angles(
            shape_ph, q, k, pos, moments=moments_ph.zero_(), estimator="default", angles_out=angles_ph),
        "rotate_quantize_qk_per_key_head": lambda: rrp.rotate_quantize_qk(
            shape_ph, q, k, pos, support_b=b, group=g, k_codes=codes, k_scales=scales, angles=angles_ph,
            q_out=q_out),
        "quant_error_stats": lambda: rrp.quant_error_stats(
            shape, k, pos, support_b=b, group=g, stats_out=stats, angles=angles),
        "quant_error_sweep": lambda: rrp.quant_error_sweep(
            shape, k, pos, group=g, stats_out=sweep, angles=angles),
        "decode_scores": lambda: rrp.decode_scores(
            shape5, q5, codes5, scales5, group=bt["group"], seq_start=start5, seq_len=lens5,
            max_len=bt["max_len"], scores=scores5),
    }
    for name, fn in runs.items():
        for _ in range(launches):
            fn()
        torch.cuda.synchronize()
    print(json.dumps({"kernels_once": list(runs), "launches": launches}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--hot-path-only", action="store_true")
    ap.add_argument("--kernels-once", action="store_true",
                    help="launch every kernel twice on the benchmark's inputs and exit (for counter passes)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the path shards over "
              "tokens or heads with no communication; only the one-GPU throughput is measured)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import rotation_rope_pair_amd as rrp
    from rotation_rope_pair_amd import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = W.WORKLOADS[4]
    inp = W.make_inputs(4)
    T, d, hq, hk, b, g = w.n_tokens, w.head_dim, w.n_q_heads, w.n_kv_heads, 128, 128
    shape = rrp.layer_shape(hq, hk, d, w.rope_theta)
    q, k = to_device_bf16(inp["q"], dev), to_device_bf16(inp["k"], dev)
    pos = torch.from_numpy(inp["pos"]).to(dev)
    q_out = torch.empty_like(q)
    codes, scales = rrp.new_kv4_cache(T, hk, d, g, dev)
    stream = torch.cuda.current_stream(dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(8)]

    # Supporting pass 1: calibrate the shared angles (default estimator) on this batch.
    moments = rrp.new_moments(d, dev)
    angles = torch.empty(d // 2, dtype=torch.float32, device=dev)
    rrp.calibrate_angles(shape, q, k, pos, moments=moments, estimator="default", angles_out=angles)
    if args.kernels_once:
        kernels_once(w, shape, q, k, pos, angles, q_out, codes, scales, dev, b, g)
        return
    supporting = {}
    if not args.hot_path_only:
        reps = 10

        def calibrate():
            moments.zero_()
            rrp.calibrate_angles(shape, q, k, pos, moments=moments, estimator="default", angles_out=angles)
        # the first GPU work of the run: settle as long as before the hot path
        settle_for(calibrate, stream, 100.0)
        torch.cuda.synchronize()
        ev[0].record(stream)
        for _ in range(2 * reps):
            calibrate()
        ev[1].record(stream)
        # Supporting pass 2: the K-range / quantisation-error diagnostic at b = 128.
        stats = torch.empty(8, dtype=torch.float64, device=dev)
        rrp.quant_error_stats(shape, k, pos, support_b=b, group=g, stats_out=stats, angles=angles)
        ev[2].record(stream)
        for _ in range(reps):
            rrp.quant_error_stats(shape, k, pos, support_b=b, group=g, stats_out=stats, angles=angles)
        ev[3].record(stream)
        torch.cuda.synchronize()
        st = stats.cpu().numpy()
        calib_bytes = (hq + hk) * d * 2 * T + 4 * T
        stats_bytes = hk * d * 2 * T + 4 * T
        cal_ms = ev[0].elapsed_time(ev[1]) / (2 * reps)
        st_ms = ev[2].elapsed_time(ev[3]) / reps
        # Supporting pass 3: the whole support sweep b = 1 .. 128 in one call.
        sweep = torch.empty((len(rrp.sweep_supports(d)), 8), dtype=torch.float64, device=dev)
        rrp.quant_error_sweep(shape, k, pos, group=g, stats_out=sweep, angles=angles)
        ev[2].record(stream)
        for _ in range(reps):
            rrp.quant_error_sweep(shape, k, pos, group=g, stats_out=sweep, angles=angles)
        ev[3].record(stream)
        torch.cuda.synchronize()
        sw_ms = ev[2].elapsed_time(ev[3]) / reps
        sw = sweep.cpu().numpy()
        supporting.update({"calibrate_angles_ms": cal_ms,
                           "calibrate_angles_hbm_gbs": calib_bytes / (cal_ms * 1e-3) / 1e9,
                           "quant_error_stats_ms": st_ms,
                           "quant_error_stats_hbm_gbs": stats_bytes / (st_ms * 1e-3) / 1e9,
                           "rel_quant_error_b128": float(np.sqrt(st[0] / st[1])),
                           "mean_k_range_b128": float(st[2] / st[5]),
                           "quant_error_sweep_ms": sw_ms,
                           "sweep_rel_quant_error": {str(int(r[7])): float(np.sqrt(r[0] / r[1])) for r in sw},
                           "sweep_mean_k_range": {str(int(r[7])): float(r[2] / r[5]) for r in sw}})
    torch.cuda.synchronize()

    def step():
        rrp.rotate_quantize_qk(shape, q, k, pos, support_b=b, group=g, k_codes=codes, k_scales=scales,
                               angles=angles, q_out=q_out)

    for _ in range(args.warmup):
        step()
    # Whatever --warmup says, the timed window starts only after at least
    # SETTLE_MS of back-to-back launches: the first tens of launches of a fresh
    # process run slower while the clocks settle.
    settle_launches = settle_for(step, stream, SETTLE_MS)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    marks[0].record(stream)
    for i in range(args.steps):
        step()
        marks[i + 1].record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms = marks[0].elapsed_time(marks[-1]) / args.steps
    per_launch = np.array([marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps)])

    bytes_per_launch = w.bytes_per_token(group=g, with_slot=False) * T
    achieved = bytes_per_launch / (ms * 1e-3) / 1e9

    # Reference streaming kernel of known size: device copy of the Q tensor.
    copy_bytes = 2 * q.numel() * q.element_size()
    for _ in range(3):
        q_out.copy_(q)
    ev[6].record(stream)
    for _ in range(10):
        q_out.copy_(q)
    ev[7].record(stream)
    torch.cuda.synchronize()
    copy_ms = ev[6].elapsed_time(ev[7]) / 10
    copy_ref = {"kernel": "torch device-to-device copy of Q (bf16)", "bytes_read_plus_written": copy_bytes,
                "ms": copy_ms, "GBs": copy_bytes / (copy_ms * 1e-3) / 1e9}
    ceiling = stream_ceiling(q, q_out, stream)
    ceiling["rotate_frac_of_copy"] = achieved / ceiling["copy_GBs"]
    per_config = None
    if not args.hot_path_only:
        per_config = per_config_timing(dev, stream, not args.no_cpu_baseline)
        supporting.update(decode_latency_us(dev, stream))
        supporting.update(qkv_timing(w, shape, q, k, pos, angles, q_out, codes, scales, dev, stream, b, g))
        supporting.update(per_head_timing(w, q, k, pos, q_out, codes, scales, dev, stream, b, g))
        supporting.update(decode_scores_timing(dev, stream))

    out = {
        "metric": METRIC,
        "value": T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "ms_per_step_median": float(np.median(per_launch)),
        "ms_per_step_min": float(per_launch.min()),
        "ms_per_step_max": float(per_launch.max()),
        "settle_ms": SETTLE_MS,
        "settle_launches": settle_launches,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded per-channel Gaussian + outlier pairs + Student-t(3) tail; shapes only)",
        "config": {"workload": w.name, "n_tokens": T, "n_q_heads": hq, "n_kv_heads": hk, "head_dim": d,
                   "rope_theta": w.rope_theta, "support_b": b, "group": g, "global_batch": 1, "seq_len": T,
                   "kv_cache": "int4 nibble-packed + fp16 group scales", "parallelism": "none (1 GPU)"},
        "hbm_gbs": achieved,
        "hbm_frac_of_peak": achieved / PEAK_HBM_GBS,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": measured_traffic(),
                     "algorithmic_bytes_per_launch": bytes_per_launch},
        "copy_reference": copy_ref,
        "stream_ceiling": ceiling,
        "per_config": per_config,
        "supporting": supporting,
        "wall_s_timed": t_wall,
    }
    if not (args.no_cpu_baseline or args.hot_path_only):
        out["cpu_baseline"] = cpu_baseline(w, inp, angles.cpu().numpy())
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
