"""GPU parity of the HIP path against the CPU oracle, through the C-ABI.

Inputs are the seeded synthetic workloads (rotation_rope_pair_amd/workloads.py);
the same bytes go to the GPU and to the oracle.  Small workloads are compared
element by element in full; the large ones run at their full size on the GPU
(in the launch configuration the benchmark times) and are compared on a
sample of tokens that the oracle evaluates one by one.  Tolerances: see
oracle/compare.py.
"""
import math
import os
import re

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle as O  # noqa: E402
from oracle import compare as C  # noqa: E402
import rotation_rope_pair_amd as rrp  # noqa: E402
from rotation_rope_pair_amd import workloads as W  # noqa: E402

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU-only container
    pytest.skip("no GPU", allow_module_level=True)

DEV = torch.device("cuda:0")


# ---------------------------------------------------------------------------
# helpers
# ---------------------------------------------------------------------------

def to_dev(a):
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def bits(t):
    """bf16 / fp16 device tensor -> uint16 numpy bit patterns."""
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def shape_of(w, layout=0, ah=0):
    return rrp.layer_shape(w.n_q_heads, w.n_kv_heads, w.head_dim, w.rope_theta, layout, angle_heads=ah)


def oshape_of(w, layout=0, hq=None, ah=0):
    return O.shape(w.n_q_heads if hq is None else hq, w.n_kv_heads, w.head_dim, w.rope_theta, layout,
                   angle_heads=ah)


def random_angles(P, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.uniform(-math.pi / 4, math.pi / 4, P).astype(np.float32)


def sample_tokens(T, n, seed=0):
    if T <= n:
        return np.arange(T)
    rng = np.random.Generator(np.random.PCG64(seed))
    head = np.arange(min(64, n // 4))
    tail = np.arange(T - min(64, n // 4), T)
    mid = rng.choice(np.arange(head.size, T - tail.size), n - head.size - tail.size, replace=False)
    return np.unique(np.concatenate([head, mid, tail]))


def run_rotate(w, inp, angles, b, g, *, debug=True, in_place=False, with_q=True, layout=0,
               q_dev=None, k_dev=None, pos_dev=None, ah=0):
    d, hq, hk = w.head_dim, w.n_q_heads, w.n_kv_heads
    q = q_dev if q_dev is not None else (to_dev(inp["q"]) if with_q else None)
    k = k_dev if k_dev is not None else to_dev(inp["k"])
    pos = pos_dev if pos_dev is not None else to_dev(inp["pos"])
    T = int(pos.numel())
    n_slots = inp.get("n_slots", T)
    codes, scales = rrp.new_kv4_cache(n_slots, hk, d, g, DEV)
    q_out = (q if in_place else torch.empty_like(q)) if with_q else None
    dbg = {}
    if debug:
        if with_q:
            dbg["q_rot_f32"] = torch.empty((T, hq, d), dtype=torch.float32, device=DEV)
        dbg["k_rot_f32"] = torch.empty((T, hk, d), dtype=torch.float32, device=DEV)
        dbg["k_scale_f32"] = torch.empty((T, hk, d // g), dtype=torch.float32, device=DEV)
    sm = to_dev(inp.get("slot_mapping"))
    rrp.rotate_quantize_qk(shape_of(w, layout, ah), q, k, pos, support_b=b, group=g, k_codes=codes, k_scales=scales,
                           angles=None if angles is None else to_dev(angles), q_out=q_out, slot_mapping=sm,
                           n_slots=n_slots, **dbg)
    torch.cuda.synchronize()
    return {"q_out": q_out, "codes": codes, "scales": scales, **dbg}


def check_rotate(w, inp, out, angles, b, g, idx, *, layout=0, with_q=True, ah=0):
    """Compare GPU outputs of the tokens `idx` with the oracle run on just those tokens."""
    d, hq, hk = w.head_dim, w.n_q_heads, w.n_kv_heads
    idx = np.asarray(idx)
    q = inp["q"][idx] if with_q else None
    ref = O.rotate_quantize_qk(oshape_of(w, layout, hq if with_q else 0, ah), q, inp["k"][idx], inp["pos"][idx],
                               angles, b, g)
    sm = inp.get("slot_mapping")
    slots = idx if sm is None else sm[idx]
    sl = torch.from_numpy(slots.astype(np.int64)).to(DEV)
    it = torch.from_numpy(idx.astype(np.int64)).to(DEV)
    fmt = "f32" if w.dtype == "f32" else "bf16"
    rep = {}
    if with_q and out["q_out"] is not None:
        qo = out["q_out"].index_select(0, it)
        qo = bits(qo) if fmt == "bf16" else qo.cpu().numpy()
        C.check_q_out(qo, ref["q_rot"], fmt)
        if "q_rot_f32" in out:
            rep["q_row_rel_err"] = C.row_rel_err(out["q_rot_f32"].index_select(0, it).cpu().numpy(), ref["q_rot"])
            assert rep["q_row_rel_err"] <= C.ROW_REL_TOL, rep
    codes = out["codes"].index_select(0, sl).cpu().numpy().reshape(-1, d // 2)
    scales = bits(out["scales"].index_select(0, sl)).reshape(-1, d // g)
    kw = {}
    if "k_rot_f32" in out:
        kw = dict(k_rot_gpu=out["k_rot_f32"].index_select(0, it).cpu().numpy().reshape(-1, d),
                  s32_gpu=out["k_scale_f32"].index_select(0, it).cpu().numpy().reshape(-1, d // g),
                  s32_ref=ref["k_scale32"].reshape(-1, d // g))
    rep.update(C.compare_k(codes, scales, ref["k_rot"].reshape(-1, d), ref["k_scales"].reshape(-1, d // g),
                           ref["k_codes"].reshape(-1, d // 2), g, **kw))
    return rep


_INPUTS = {}


def inputs(n):
    if n not in _INPUTS:
        _INPUTS[n] = W.make_inputs(n)
    return _INPUTS[n]


# ---------------------------------------------------------------------------
# rotate + quantise
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n,b", [(1, 1), (1, 2), (1, 64), (2, 1), (2, 2), (2, 4), (2, 8), (2, 16), (2, 32), (2, 64)])
def test_rotate_parity_small_workloads_in_full(n, b):
    w, inp = W.WORKLOADS[n], inputs(n)
    ang = random_angles(w.n_pairs, 100 + n)
    out = run_rotate(w, inp, ang, b, w.group)
    rep = check_rotate(w, inp, out, ang, b, w.group, np.arange(w.n_tokens))
    print(f"workload {n} b={b}: {rep}")


def test_rotate_parity_without_pair_angles():
    w, inp = W.WORKLOADS[2], inputs(2)
    out = run_rotate(w, inp, None, 64, 64)
    print(check_rotate(w, inp, out, None, 64, 64, np.arange(w.n_tokens)))


def test_rotate_parity_llama3b_layer_sampled():
    w, inp = W.WORKLOADS[3], inputs(3)
    ang = random_angles(w.n_pairs, 103)
    out = run_rotate(w, inp, ang, 128, 128)
    print(check_rotate(w, inp, out, ang, 128, 128, sample_tokens(w.n_tokens, 1024, 3)))


@pytest.mark.parametrize("b", [2, 128])
def test_rotate_parity_decode_slot_scatter(b):
    """Decode batch: 256 tokens at random positions scattered into a 256 x 32768-slot
    cache; only the mapped slots are written."""
    w, inp = W.WORKLOADS[5], inputs(5)
    ang = random_angles(w.n_pairs, 105)
    out = run_rotate(w, inp, ang, b, w.group)
    print(check_rotate(w, inp, out, ang, b, w.group, np.arange(w.n_tokens)))
    written = int(torch.count_nonzero(out["scales"]).item())
    sl = torch.from_numpy(inp["slot_mapping"]).to(DEV)
    assert written == int(torch.count_nonzero(out["scales"].index_select(0, sl)).item())
    nz_codes = int(torch.count_nonzero(out["codes"]).item())
    assert nz_codes == int(torch.count_nonzero(out["codes"].index_select(0, sl)).item())


def test_rotate_parity_prefill_128k_bench_launch():
    """Full 131072-token prefill in exactly the call the benchmark times (no debug
    outputs), checked on 2048 sampled tokens."""
    w, inp = W.WORKLOADS[4], inputs(4)
    ang = random_angles(w.n_pairs, 104)
    out = run_rotate(w, inp, ang, 128, 128, debug=False)
    rep = check_rotate(w, inp, out, ang, 128, 128, sample_tokens(w.n_tokens, 2048, 4))
    print(rep)


def test_rotate_parity_prefill_128k_every_token():
    """The same benchmark launch compared element by element on all 131072 tokens
    (Q output bits, K codes and fp16 scales), in chunks the oracle runs in about a
    second each."""
    w, inp = W.WORKLOADS[4], inputs(4)
    ang = random_angles(w.n_pairs, 114)
    out = run_rotate(w, inp, ang, 128, 128, debug=False)
    totals = {"rows": 0, "scale_mismatch": 0, "scale_band": 0, "code_mismatch": 0, "code_band": 0}
    chunk = 16384
    for t0 in range(0, w.n_tokens, chunk):
        rep = check_rotate(w, inp, out, ang, 128, 128, np.arange(t0, min(w.n_tokens, t0 + chunk)))
        for key in totals:
            totals[key] += rep[key]
    assert totals["rows"] == w.n_tokens * w.n_kv_heads
    print(totals)


@pytest.mark.parametrize("layout", [0, 1])
@pytest.mark.parametrize("n", [1, 2, 3])
def test_rotate_parity_rope_layouts(n, layout):
    w, inp = W.WORKLOADS[n], inputs(n)
    T = min(w.n_tokens, 512)
    sub = {k: (v[:T] if isinstance(v, np.ndarray) else v) for k, v in inp.items()}
    sub["n_slots"] = T
    ang = random_angles(w.n_pairs, 200 + n)
    b = w.head_dim
    out = run_rotate(w, sub, ang, b, w.group, layout=layout)
    print(check_rotate(w, sub, out, ang, b, w.group, np.arange(T), layout=layout))


@pytest.mark.parametrize("n,g", [(1, 2), (1, 4), (1, 8), (1, 32), (3, 2), (3, 4), (3, 8), (3, 16), (3, 32), (3, 64)])
def test_rotate_parity_group_sizes(n, g):
    w, inp = W.WORKLOADS[n], inputs(n)
    T = min(w.n_tokens, 256)
    sub = {k: (v[:T] if isinstance(v, np.ndarray) else v) for k, v in inp.items()}
    sub["n_slots"] = T
    ang = random_angles(w.n_pairs, 300 + g)
    for b in (2, w.head_dim):
        out = run_rotate(w, sub, ang, b, g)
        print(n, g, b, check_rotate(w, sub, out, ang, b, g, np.arange(T)))


@pytest.mark.parametrize("T", [1, 3, 5, 4097])
def test_rotate_ragged_token_counts(T):
    w = W.WORKLOADS[3]
    inp = W.make_inputs(3, n_tokens=T)
    ang = random_angles(w.n_pairs, 400)
    out = run_rotate(w, inp, ang, 128, 128)
    print(T, check_rotate(w, inp, out, ang, 128, 128, np.arange(T)))


def test_rotate_in_place_and_k_only():
    w, inp = W.WORKLOADS[2], inputs(2)
    ang = random_angles(w.n_pairs, 500)
    out = run_rotate(w, inp, ang, 16, 64, in_place=True)
    check_rotate(w, inp, out, ang, 16, 64, np.arange(w.n_tokens))
    out2 = run_rotate(w, inp, ang, 16, 64, with_q=False)
    check_rotate(w, inp, out2, ang, 16, 64, np.arange(w.n_tokens), with_q=False)
    assert torch.equal(out["codes"], out2["codes"]) and torch.equal(out["scales"], out2["scales"])


def test_rotate_degenerate_rows():
    """All-zero rows (scale 0, codes 0), rows so small the fp16 scale underflows,
    rows so large it saturates, and padding slots (-1, out of range)."""
    w = W.WORKLOADS[3]
    T = 16
    inp = W.make_inputs(3, n_tokens=T)
    k = inp["k"].copy()
    import torch as _t
    def bf(x):
        return _t.from_numpy(np.asarray(x, np.float32)).to(_t.bfloat16).view(_t.int16).numpy().view(np.uint16)
    k[0] = 0
    k[1] = bf(np.full((w.n_kv_heads, w.head_dim), 1e-9))
    k[2] = bf(np.full((w.n_kv_heads, w.head_dim), 3e5) * np.sign(np.arange(w.head_dim) - 63.5))
    k[3, 0] = bf(np.eye(w.head_dim)[5] * 100.0)
    inp["k"] = k
    slots = np.arange(T, dtype=np.int64)
    slots[4] = -1
    slots[5] = 10 ** 9
    inp["slot_mapping"] = slots
    inp["n_slots"] = T
    ang = random_angles(w.n_pairs, 600)
    for b in (1, 2, 128):
        out = run_rotate(w, inp, ang, b, 64)
        keep = np.array([t for t in range(T) if 0 <= slots[t] < T])
        print(b, check_rotate(w, inp, out, ang, b, 64, keep))
        assert not out["codes"][4].any() and not out["scales"][4].any()
        assert not out["codes"][0].any() and not out["scales"][0].any()


def test_rotate_is_deterministic():
    w, inp = W.WORKLOADS[3], inputs(3)
    ang = random_angles(w.n_pairs, 700)
    a = run_rotate(w, inp, ang, 128, 128)
    b = run_rotate(w, inp, ang, 128, 128)
    for key in ("q_out", "codes", "scales", "q_rot_f32", "k_rot_f32", "k_scale_f32"):
        assert torch.equal(a[key].view(torch.uint8) if a[key].dtype == torch.bfloat16 else a[key],
                           b[key].view(torch.uint8) if b[key].dtype == torch.bfloat16 else b[key]), key


# ---------------------------------------------------------------------------
# rotate + quantise with the V half of the cache
# ---------------------------------------------------------------------------

_VINPUTS = {}


def vinputs(n, T=None):
    key = (n, T)
    if key not in _VINPUTS:
        if T is None:  # reuse the full-size Q / K already drawn
            _VINPUTS[key] = dict(inputs(n), v=W.make_v(n))
        else:
            _VINPUTS[key] = W.make_inputs(n, n_tokens=T, want_v=True)
    return _VINPUTS[key]


def run_rotate_qkv(w, inp, angles, b, g, *, debug=True, ah=0):
    d, hq, hk = w.head_dim, w.n_q_heads, w.n_kv_heads
    q, k, v, pos = to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["v"]), to_dev(inp["pos"])
    T = int(pos.numel())
    n_slots = inp.get("n_slots", T)
    kc, ks = rrp.new_kv4_cache(n_slots, hk, d, g, DEV)
    vc, vs = rrp.new_kv4_cache(n_slots, hk, d, g, DEV)
    dbg = {}
    if debug:
        dbg = {"q_rot_f32": torch.empty((T, hq, d), dtype=torch.float32, device=DEV),
               "k_rot_f32": torch.empty((T, hk, d), dtype=torch.float32, device=DEV),
               "k_scale_f32": torch.empty((T, hk, d // g), dtype=torch.float32, device=DEV),
               "v_rot_f32": torch.empty((T, hk, d), dtype=torch.float32, device=DEV),
               "v_scale_f32": torch.empty((T, hk, d // g), dtype=torch.float32, device=DEV)}
    q_out = torch.empty_like(q)
    rrp.rotate_quantize_qkv(shape_of(w, 0, ah), q, k, v, pos, support_b=b, group=g, k_codes=kc, k_scales=ks,
                            v_codes=vc, v_scales=vs, angles=None if angles is None else to_dev(angles), q_out=q_out,
                            slot_mapping=to_dev(inp.get("slot_mapping")), n_slots=n_slots, **dbg)
    torch.cuda.synchronize()
    return {"q_out": q_out, "codes": kc, "scales": ks, "v_codes": vc, "v_scales": vs, **dbg}


def check_v(w, inp, out, g, idx):
    d, hk = w.head_dim, w.n_kv_heads
    idx = np.asarray(idx)
    ref = O.quantize_v(oshape_of(w), inp["v"][idx], g)
    sm = inp.get("slot_mapping")
    slots = idx if sm is None else sm[idx]
    sl = torch.from_numpy(slots.astype(np.int64)).to(DEV)
    it = torch.from_numpy(idx.astype(np.int64)).to(DEV)
    codes = out["v_codes"].index_select(0, sl).cpu().numpy().reshape(-1, d // 2)
    scales = bits(out["v_scales"].index_select(0, sl)).reshape(-1, d // g)
    kw = {}
    if "v_rot_f32" in out:
        kw = dict(k_rot_gpu=out["v_rot_f32"].index_select(0, it).cpu().numpy().reshape(-1, d),
                  s32_gpu=out["v_scale_f32"].index_select(0, it).cpu().numpy().reshape(-1, d // g),
                  s32_ref=ref["v_scale32"].reshape(-1, d // g))
    return C.compare_k(codes, scales, ref["v_rot"].reshape(-1, d), ref["v_scales"].reshape(-1, d // g),
                       ref["v_codes"].reshape(-1, d // 2), g, **kw)


@pytest.mark.parametrize("n,b,g", [(1, 2, 64), (1, 64, 4), (2, 16, 64), (2, 64, 8), (3, 128, 128), (3, 2, 2)])
def test_rotate_qkv_parity(n, b, g):
    """Q and K as the Q/K entry point (bit for bit), V against the oracle's V side."""
    w = W.WORKLOADS[n]
    T = min(w.n_tokens, 1024)
    inp = vinputs(n, T)
    ang = random_angles(w.n_pairs, 800 + n)
    out = run_rotate_qkv(w, inp, ang, b, g)
    rep_k = check_rotate(w, inp, out, ang, b, g, np.arange(T))
    rep_v = check_v(w, inp, out, g, np.arange(T))
    ref_qk = run_rotate(w, inp, ang, b, g)
    for key in ("q_out", "codes", "scales", "q_rot_f32", "k_rot_f32", "k_scale_f32"):
        a, c = out[key], ref_qk[key]
        if a.dtype == torch.bfloat16:
            a, c = a.view(torch.int16), c.view(torch.int16)
        assert torch.equal(a, c), key
    print(f"workload {n} b={b} g={g}: K {rep_k} V {rep_v}")


def test_rotate_qkv_decode_slot_scatter():
    w = W.WORKLOADS[5]
    inp = vinputs(5)
    ang = random_angles(w.n_pairs, 805)
    out = run_rotate_qkv(w, inp, ang, 128, w.group)
    print(check_v(w, inp, out, w.group, np.arange(w.n_tokens)))
    sl = torch.from_numpy(inp["slot_mapping"]).to(DEV)
    assert int(torch.count_nonzero(out["v_scales"]).item()) == \
        int(torch.count_nonzero(out["v_scales"].index_select(0, sl)).item())


def test_rotate_qkv_prefill_128k_sampled():
    """The 131072-token prefill with V, in the launch the benchmark times, checked
    on 2048 sampled tokens (V against the oracle, K and Q too)."""
    w = W.WORKLOADS[4]
    inp = vinputs(4)
    ang = random_angles(w.n_pairs, 804)
    out = run_rotate_qkv(w, inp, ang, 128, 128, debug=False)
    idx = sample_tokens(w.n_tokens, 2048, 14)
    print(check_rotate(w, inp, out, ang, 128, 128, idx), check_v(w, inp, out, 128, idx))


# ---------------------------------------------------------------------------
# calibration
# ---------------------------------------------------------------------------

def run_calib(w, q, k, pos, estimator, layout=0, moments=None, ah=0):
    d = w.head_dim
    A = ah if ah > 1 else 1
    mom = moments if moments is not None else rrp.new_moments(d, DEV, n_sets=A)
    ang = torch.empty((d // 2,) if A == 1 else (A, d // 2), dtype=torch.float32, device=DEV)
    rrp.calibrate_angles(shape_of(w, layout, ah), None if q is None else to_dev(q), to_dev(k), to_dev(pos),
                         moments=mom, estimator=estimator, angles_out=ang)
    torch.cuda.synchronize()
    return mom.cpu().numpy(), ang.cpu().numpy()


EST = {"default": O.EST_DEFAULT, "k_only": O.EST_K_ONLY, "stream_balanced": O.EST_STREAM_BALANCED}


@pytest.mark.parametrize("n,est", [(1, "default"), (2, "default"), (2, "k_only"), (2, "stream_balanced"),
                                   (3, "default"), (4, "default"), (5, "k_only")])
def test_calibration_parity(n, est):
    w = W.WORKLOADS[n]
    inp = inputs(n)
    src = inp["calib"] if inp["calib"] is not None else inp
    q = src["q"] if est != "k_only" else None
    mom_g, ang_g = run_calib(w, q, src["k"], src["pos"], est)
    shp = oshape_of(w)
    mom_r = O.calibrate_moments(shp, q, src["k"], src["pos"])
    phi64, phi32, abc = O.angles_from_moments(mom_r, EST[est])
    worst = C.compare_moments(mom_g, mom_r)
    rep = C.compare_angles(ang_g, phi64, abc)
    print(f"workload {n} {est}: moments {worst:.2e} {rep}")


@pytest.mark.parametrize("T", [1, 5, 127, 129, 383])
@pytest.mark.parametrize("est", ["default", "k_only"])
@pytest.mark.parametrize("ah", [0, 8])
def test_calibration_parity_small_batches(T, est, ah):
    """Batches from one token to a few blocks' worth, with ragged tails: the
    shared-set grid takes one block per 128 tokens, the per-set grid one per 32
    tokens and stream over the sets (at least one per stream and set)."""
    w = W.WORKLOADS[2]
    inp = inputs(2)
    q = inp["q"][:T] if est != "k_only" else None
    k, pos = inp["k"][:T], inp["pos"][:T]
    mom_g, ang_g = run_calib(w, q, k, pos, est, ah=ah)
    mom_r = O.calibrate_moments(oshape_of(w, ah=ah), q, k, pos)
    phi64, _, abc = O.angles_from_moments(mom_r, EST[est])
    C.compare_moments(mom_g, mom_r)
    C.compare_angles(ang_g.reshape(-1), phi64.reshape(-1), abc.reshape(-1, 3))


def test_calibration_accumulates_and_finalises_separately():
    w, inp = W.WORKLOADS[2], inputs(2)
    q, k, pos = inp["q"], inp["k"], inp["pos"]
    mom_all, ang_all = run_calib(w, q, k, pos, "default")
    mom = rrp.new_moments(w.head_dim, DEV)
    run_calib(w, q[:700], k[:700], pos[:700], "default", moments=mom)
    mom2, ang2 = run_calib(w, q[700:], k[700:], pos[700:], "default", moments=mom)
    C.compare_moments(mom2, mom_all, rel=1e-13)
    assert np.max(C.angle_diff(ang2, ang_all)) < 1e-6
    # finalise only (no tokens) with another estimator
    ang3 = torch.empty(w.n_pairs, dtype=torch.float32, device=DEV)
    e = torch.empty((0,), dtype=torch.bfloat16, device=DEV)
    rrp.calibrate_angles(shape_of(w), e, e, torch.empty((0,), dtype=torch.int32, device=DEV), moments=mom,
                         estimator="stream_balanced", angles_out=ang3)
    torch.cuda.synchronize()
    phi64, _, abc = O.angles_from_moments(mom2, O.EST_STREAM_BALANCED)
    C.compare_angles(ang3.cpu().numpy(), phi64, abc)
    assert np.array_equal(mom.cpu().numpy(), mom2)


def test_calibration_is_deterministic():
    w, inp = W.WORKLOADS[3], inputs(3)
    m1, a1 = run_calib(w, inp["q"], inp["k"], inp["pos"], "default")
    m2, a2 = run_calib(w, inp["q"], inp["k"], inp["pos"], "default")
    assert np.array_equal(m1, m2) and np.array_equal(a1, a2)


# ---------------------------------------------------------------------------
# diagnostics
# ---------------------------------------------------------------------------

# Both sides evaluate the K transform, the quantiser and the sums in fp64; only
# the summation order differs.
STAT_TOL = np.array([1e-9, 1e-11, 1e-11, 1e-13, 1e-11])


def run_stats(w, k, pos, angles, b, g, ah=0, layout=0):
    st = torch.empty(8, dtype=torch.float64, device=DEV)
    rrp.quant_error_stats(shape_of(w, layout, ah), to_dev(k), to_dev(pos), support_b=b, group=g, stats_out=st,
                          angles=None if angles is None else to_dev(angles))
    torch.cuda.synchronize()
    return st.cpu().numpy()


@pytest.mark.parametrize("n", [1, 2])
def test_quant_error_stats_parity_support_sweep(n):
    w, inp = W.WORKLOADS[n], inputs(n)
    _, phi32, _ = O.angles_from_moments(O.calibrate_moments(oshape_of(w), inp["q"], inp["k"], inp["pos"]),
                                        O.EST_DEFAULT)
    rows = []
    for b, ang in [(bb, None) for bb in (1, 2, 4, 8, 16, 32, 64)] + [(1, phi32), (64, phi32)]:
        g = run_stats(w, inp["k"], inp["pos"], ang, b, w.group)
        r = O.quant_error_stats(oshape_of(w), inp["k"], inp["pos"], ang, b, w.group)
        rel = np.abs(g[:5] - r[:5]) / np.maximum(np.abs(r[:5]), 1e-300)
        assert np.all(rel <= STAT_TOL), (b, g, r, rel)
        assert g[5] == r[5] and g[6] == r[6] and g[7] == 0
        rows.append((b, ang is not None, math.sqrt(g[0] / g[1]), g[2] / g[5], g[3]))
    print(f"workload {n}: (b, angles, rel_err, mean K range, max K range)")
    for row in rows:
        print("  ", row)


def test_quant_error_stats_is_deterministic():
    w, inp = W.WORKLOADS[3], inputs(3)
    a = run_stats(w, inp["k"], inp["pos"], None, 128, 128)
    b = run_stats(w, inp["k"], inp["pos"], None, 128, 128)
    assert np.array_equal(a, b)


def run_sweep(w, k, pos, angles, g, ah=0, layout=0):
    nb = len(rrp.sweep_supports(w.head_dim))
    st = torch.empty((nb, 8), dtype=torch.float64, device=DEV)
    rrp.quant_error_sweep(shape_of(w, layout, ah), to_dev(k), to_dev(pos), group=g, stats_out=st,
                          angles=None if angles is None else to_dev(angles))
    torch.cuda.synchronize()
    return st.cpu().numpy()


@pytest.mark.parametrize("n,g,with_angles", [(1, 64, True), (2, 64, True), (2, 64, False), (2, 4, True),
                                              (2, 2, True), (3, 128, True), (3, 16, False), (3, 8, True),
                                              (3, 2, False)])
def test_quant_error_sweep_every_support_matches_oracle(n, g, with_angles):
    """One launch for every support b = 1 .. head_dim: each row equals the oracle's
    diagnostic at that b, and the single-support kernel's, to the stated tolerance."""
    w = W.WORKLOADS[n]
    T = min(w.n_tokens, 1024)
    inp = W.make_inputs(n, n_tokens=T)
    ang = random_angles(w.n_pairs, 900 + n) if with_angles else None
    sw = run_sweep(w, inp["k"], inp["pos"], ang, g)
    supports = rrp.sweep_supports(w.head_dim)
    assert sw.shape[0] == len(supports)
    for j, b in enumerate(supports):
        r = O.quant_error_stats(oshape_of(w), inp["k"], inp["pos"], ang, b, g)
        one = run_stats(w, inp["k"], inp["pos"], ang, b, g)
        for ref in (r, one):
            rel = np.abs(sw[j, :5] - ref[:5]) / np.maximum(np.abs(ref[:5]), 1e-300)
            assert np.all(rel <= STAT_TOL), (b, sw[j], ref, rel)
        assert sw[j, 5] == r[5] and sw[j, 6] == r[6] and sw[j, 7] == b
    print(f"workload {n} g={g}: rel_err by b", [round(float(np.sqrt(x[0] / x[1])), 5) for x in sw])


def test_quant_error_sweep_prefill_128k_properties():
    """The full 131072-token prefill: every sweep row equals the single-support
    kernel at that b, and N (the energy) is the same at every b (orthogonality)."""
    w, inp = W.WORKLOADS[4], inputs(4)
    ang = random_angles(w.n_pairs, 904)
    k, pos = to_dev(inp["k"]), to_dev(inp["pos"])
    nb = len(rrp.sweep_supports(w.head_dim))
    st = torch.empty((nb, 8), dtype=torch.float64, device=DEV)
    rrp.quant_error_sweep(shape_of(w), k, pos, group=128, stats_out=st, angles=to_dev(ang))
    torch.cuda.synchronize()
    sw = st.cpu().numpy()
    one = torch.empty(8, dtype=torch.float64, device=DEV)
    for j, b in enumerate(rrp.sweep_supports(w.head_dim)):
        rrp.quant_error_stats(shape_of(w), k, pos, support_b=b, group=128, stats_out=one, angles=to_dev(ang))
        torch.cuda.synchronize()
        ref = one.cpu().numpy()
        rel = np.abs(sw[j, :5] - ref[:5]) / np.maximum(np.abs(ref[:5]), 1e-300)
        assert np.all(rel <= STAT_TOL), (b, sw[j], ref, rel)
        assert abs(sw[j, 1] - sw[0, 1]) <= 1e-11 * sw[0, 1]
        assert sw[j, 6] == w.n_tokens * w.n_kv_heads and sw[j, 7] == b
    print("rel_err by b", [round(float(np.sqrt(x[0] / x[1])), 5) for x in sw])


# ---------------------------------------------------------------------------
# per-key-head angle sets (one set of pair angles per key head; each query head
# uses its key head's set)
# ---------------------------------------------------------------------------

def random_angle_sets(w, seed):
    return np.stack([random_angles(w.n_pairs, seed + 17 * h) for h in range(w.n_kv_heads)])


@pytest.mark.parametrize("n,est", [(2, "default"), (2, "k_only"), (2, "stream_balanced"), (3, "default"),
                                   (4, "default"), (5, "k_only")])
def test_per_head_calibration_parity(n, est):
    w = W.WORKLOADS[n]
    inp = inputs(n)
    src = inp["calib"] if inp["calib"] is not None else inp
    q = src["q"] if est != "k_only" else None
    hk = w.n_kv_heads
    mom_g, ang_g = run_calib(w, q, src["k"], src["pos"], est, ah=hk)
    assert mom_g.shape == (hk, w.n_pairs, 2, 6) and ang_g.shape == (hk, w.n_pairs)
    mom_r = O.calibrate_moments(oshape_of(w, ah=hk), q, src["k"], src["pos"])
    phi64, _, abc = O.angles_from_moments(mom_r, EST[est])
    worst = C.compare_moments(mom_g, mom_r)
    rep = C.compare_angles(ang_g.reshape(-1), phi64.reshape(-1), abc.reshape(-1, 3))
    # the sets do differ from head to head, and from the shared angles
    _, ang_shared = run_calib(w, q, src["k"], src["pos"], est)
    assert np.max(C.angle_diff(ang_g, ang_shared[None, :])) > 1e-3
    print(f"workload {n} {est} per head: moments {worst:.2e} {rep}")


def test_per_head_calibration_accumulates_across_calls():
    w, inp = W.WORKLOADS[2], inputs(2)
    hk = w.n_kv_heads
    mom_all, ang_all = run_calib(w, inp["q"], inp["k"], inp["pos"], "default", ah=hk)
    mom = rrp.new_moments(w.head_dim, DEV, n_sets=hk)
    run_calib(w, inp["q"][:900], inp["k"][:900], inp["pos"][:900], "default", moments=mom, ah=hk)
    mom2, ang2 = run_calib(w, inp["q"][900:], inp["k"][900:], inp["pos"][900:], "default", moments=mom, ah=hk)
    C.compare_moments(mom2, mom_all, rel=1e-13)
    assert np.max(C.angle_diff(ang2, ang_all)) < 1e-6


@pytest.mark.parametrize("n,b", [(2, 2), (2, 16), (2, 64), (3, 2), (3, 128), (5, 128)])
def test_per_head_rotate_parity(n, b):
    w, inp = W.WORKLOADS[n], inputs(n)
    T = min(w.n_tokens, 2048)
    sub = {k: (v[:T] if isinstance(v, np.ndarray) and k != "slot_mapping" else v) for k, v in inp.items()}
    if inp.get("slot_mapping") is not None:
        sub["slot_mapping"] = inp["slot_mapping"][:T]
    else:
        sub["n_slots"] = T
    ang = random_angle_sets(w, 1000 + n)
    out = run_rotate(w, sub, ang, b, w.group, ah=w.n_kv_heads)
    print(f"workload {n} b={b} per head:", check_rotate(w, sub, out, ang, b, w.group, np.arange(T), ah=w.n_kv_heads))


def test_per_head_rotate_prefill_128k_sampled():
    """The 131072-token prefill with one angle set per key head, at full size (the
    benchmark's launch shape), checked on 2048 sampled tokens."""
    w, inp = W.WORKLOADS[4], inputs(4)
    ang = random_angle_sets(w, 1004)
    out = run_rotate(w, inp, ang, 128, 128, debug=False, ah=w.n_kv_heads)
    print(check_rotate(w, inp, out, ang, 128, 128, sample_tokens(w.n_tokens, 2048, 24), ah=w.n_kv_heads))


def test_per_head_identical_sets_equal_the_shared_path():
    """Every key head given the same set reproduces the shared-angle launch bit for bit."""
    w, inp = W.WORKLOADS[3], inputs(3)
    shared = random_angles(w.n_pairs, 1100)
    sets = np.tile(shared, (w.n_kv_heads, 1))
    for b in (2, 128):
        a = run_rotate(w, inp, shared, b, 128)
        c = run_rotate(w, inp, sets, b, 128, ah=w.n_kv_heads)
        for key in ("q_out", "codes", "scales", "q_rot_f32", "k_rot_f32", "k_scale_f32"):
            x, y = a[key], c[key]
            if x.dtype == torch.bfloat16:
                x, y = x.view(torch.int16), y.view(torch.int16)
            assert torch.equal(x, y), (b, key)
    for b, g in ((128, 128), (16, 16), (2, 128), (64, 8)):
        st_a = run_stats(w, inp["k"], inp["pos"], shared, b, g)
        st_c = run_stats(w, inp["k"], inp["pos"], sets, b, g, ah=w.n_kv_heads)
        assert np.array_equal(st_a, st_c), (b, g, st_a, st_c)
    for g in (128, 16):
        sw_a = run_sweep(w, inp["k"], inp["pos"], shared, g)
        sw_c = run_sweep(w, inp["k"], inp["pos"], sets, g, ah=w.n_kv_heads)
        assert np.array_equal(sw_a, sw_c), (g, sw_a, sw_c)


@pytest.mark.parametrize("n,b,g", [(2, 64, 64), (3, 128, 128), (3, 2, 16)])
def test_per_head_rotate_qkv_parity(n, b, g):
    w = W.WORKLOADS[n]
    T = min(w.n_tokens, 1024)
    inp = vinputs(n, T)
    ang = random_angle_sets(w, 1200 + n)
    hk = w.n_kv_heads
    out = run_rotate_qkv(w, inp, ang, b, g, ah=hk)
    rep_k = check_rotate(w, inp, out, ang, b, g, np.arange(T), ah=hk)
    rep_v = check_v(w, inp, out, g, np.arange(T))
    print(f"workload {n} b={b} g={g} per head: K {rep_k} V {rep_v}")


@pytest.mark.parametrize("n,g", [(2, 64), (3, 128), (3, 8)])
def test_per_head_stats_and_sweep_parity(n, g):
    w = W.WORKLOADS[n]
    T = min(w.n_tokens, 1024)
    inp = W.make_inputs(n, n_tokens=T)
    hk = w.n_kv_heads
    ang = random_angle_sets(w, 1300 + n)
    sw = run_sweep(w, inp["k"], inp["pos"], ang, g, ah=hk)
    for j, b in enumerate(rrp.sweep_supports(w.head_dim)):
        r = O.quant_error_stats(oshape_of(w, ah=hk), inp["k"], inp["pos"], ang, b, g)
        one = run_stats(w, inp["k"], inp["pos"], ang, b, g, ah=hk)
        for got in (sw[j], one):
            rel = np.abs(got[:5] - r[:5]) / np.maximum(np.abs(r[:5]), 1e-300)
            assert np.all(rel <= STAT_TOL), (b, got, r, rel)
            assert got[5] == r[5] and got[6] == r[6]
    print(f"workload {n} g={g} per head: rel_err by b", [round(float(np.sqrt(x[0] / x[1])), 5) for x in sw])


def _bf16_bits_to_f32(a):
    return (a.astype(np.uint32) << 16).view(np.float32)


@pytest.mark.parametrize("layout,b", [(0, 8), (1, 64), (1, 2)])
def test_per_head_fp32_inputs_and_layouts(layout, b):
    """Per-key-head sets with fp32 rows (the bf16 workload's values widened) under
    both RoPE pair layouts."""
    import dataclasses
    w = dataclasses.replace(W.WORKLOADS[2], dtype="f32")
    src = inputs(2)
    T = 1024
    sub = {"q": _bf16_bits_to_f32(src["q"][:T]), "k": _bf16_bits_to_f32(src["k"][:T]), "pos": src["pos"][:T],
           "n_slots": T}
    ang = random_angle_sets(w, 1400 + b)
    out = run_rotate(w, sub, ang, b, 16, layout=layout, ah=w.n_kv_heads)
    print(layout, b, check_rotate(w, sub, out, ang, b, 16, np.arange(T), layout=layout, ah=w.n_kv_heads))


def small_batch_waves():
    """The library's bound on the split-pass family (kSmallBatchWaves), read
    from the kernel source so the tests at the bound follow it."""
    src = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "rotation_rope_pair_amd", "csrc",
                       "rrp_rotate_kernel.hpp")
    with open(src) as f:
        return int(re.search(r"constexpr int kSmallBatchWaves = (\d+);", f.read()).group(1))


def split_bound(w, with_v=False, with_q=True):
    """Largest batch the split-pass kernel family takes: the library runs a
    batch there when its tokens x row passes per token are at most
    kSmallBatchWaves (one wave per pass), else one wave per token with a grid
    stride.  A pass is 2048 / (head_dim x element bytes) rows of one token."""
    rows = 2048 // (w.head_dim * (4 if w.dtype == "f32" else 2))
    npass = (-(-w.n_q_heads // rows) if with_q else 0) + (2 if with_v else 1) * -(-w.n_kv_heads // rows)
    return small_batch_waves() // npass


@pytest.mark.parametrize("ah,with_v", [(0, False), (0, True), (8, False)])
def test_small_batch_split_matches_grid_stride_kernel(ah, with_v):
    """Small batches run the split-pass kernel family, larger ones the
    grid-stride family: the same tokens give the same bits either way."""
    w = W.WORKLOADS[3]
    big = vinputs(3, 4096) if with_v else W.make_inputs(3, n_tokens=4096)
    T = split_bound(w, with_v)
    small = {k: (v[:T] if isinstance(v, np.ndarray) else v) for k, v in big.items()}
    small["n_slots"] = T
    ang = random_angle_sets(w, 1500) if ah else random_angles(w.n_pairs, 1500)
    run = (lambda inp: run_rotate_qkv(w, inp, ang, 128, 32, ah=ah)) if with_v else \
        (lambda inp: run_rotate(w, inp, ang, 128, 32, ah=ah))
    a, c = run(big), run(small)
    keys = ["q_out", "codes", "scales", "q_rot_f32", "k_rot_f32", "k_scale_f32"]
    if with_v:
        keys += ["v_codes", "v_scales", "v_rot_f32", "v_scale_f32"]
    for key in keys:
        x, y = a[key][:T], c[key]
        if x.dtype == torch.bfloat16:
            x, y = x.view(torch.int16), y.view(torch.int16)
        assert torch.equal(x, y), key


@pytest.mark.parametrize("n,b,g,ah,with_v", [(2, 16, 16, 0, False), (2, 64, 8, 0, True), (3, 128, 32, 0, False),
                                            (3, 2, 2, 8, False), (3, 64, 128, 0, True), (1, 64, 4, 0, False)])
def test_rotate_parity_at_the_kernel_family_bound(n, b, g, ah, with_v):
    """The last batch size the split-pass family takes and the first one the
    grid-stride family takes, every token against the oracle."""
    w = W.WORKLOADS[n]
    bound = split_bound(w, with_v)
    for T in (bound, bound + 1):
        inp = W.make_inputs(n, n_tokens=T, want_v=with_v)
        ang = random_angle_sets(w, 1900 + T) if ah else random_angles(w.n_pairs, 1900 + T)
        out = run_rotate_qkv(w, inp, ang, b, g, ah=ah) if with_v else run_rotate(w, inp, ang, b, g, ah=ah)
        rep = check_rotate(w, inp, out, ang, b, g, np.arange(T), ah=ah)
        if with_v:
            rep["v"] = check_v(w, inp, out, g, np.arange(T))
        print(f"workload {n} T={T} b={b} g={g} sets={max(ah, 1)} v={with_v}: {rep}")


def test_per_head_in_place_and_k_only():
    """Per-key-head sets with Q rotated in place, and with no Q at all."""
    w, inp = W.WORKLOADS[2], inputs(2)
    hk = w.n_kv_heads
    ang = random_angle_sets(w, 1600)
    out = run_rotate(w, inp, ang, 32, 64, in_place=True, ah=hk)
    check_rotate(w, inp, out, ang, 32, 64, np.arange(w.n_tokens), ah=hk)
    out2 = run_rotate(w, inp, ang, 32, 64, with_q=False, ah=hk)
    check_rotate(w, inp, out2, ang, 32, 64, np.arange(w.n_tokens), with_q=False, ah=hk)
    assert torch.equal(out["codes"], out2["codes"]) and torch.equal(out["scales"], out2["scales"])


@pytest.mark.parametrize("n,est,ah", [(1, "default", 0), (2, "default", 0), (2, "stream_balanced", 0),
                                      (2, "default", 8), (3, "k_only", 8)])
def test_calibration_parity_interleaved_pairs(n, est, ah):
    """Calibration with the interleaved RoPE pair layout (pairs (2k, 2k + 1))."""
    w = W.WORKLOADS[n]
    T = min(w.n_tokens, 2048)
    inp = W.make_inputs(n, n_tokens=T)
    q = inp["q"] if est != "k_only" else None
    mom_g, ang_g = run_calib(w, q, inp["k"], inp["pos"], est, layout=1, ah=ah)
    mom_r = O.calibrate_moments(oshape_of(w, 1, ah=ah), q, inp["k"], inp["pos"])
    phi64, _, abc = O.angles_from_moments(mom_r, EST[est])
    worst = C.compare_moments(mom_g, mom_r)
    rep = C.compare_angles(ang_g.reshape(-1), phi64.reshape(-1), abc.reshape(-1, 3))
    print(f"workload {n} {est} sets={max(ah, 1)} interleaved: moments {worst:.2e} {rep}")


@pytest.mark.parametrize("n,g,ah", [(1, 64, 0), (2, 8, 0), (3, 128, 8)])
def test_stats_and_sweep_parity_interleaved_pairs(n, g, ah):
    w = W.WORKLOADS[n]
    T = min(w.n_tokens, 512)
    inp = W.make_inputs(n, n_tokens=T)
    ang = random_angle_sets(w, 1700 + n) if ah else random_angles(w.n_pairs, 1700 + n)
    sw = run_sweep(w, inp["k"], inp["pos"], ang, g, ah=ah, layout=1)
    for j, b in enumerate(rrp.sweep_supports(w.head_dim)):
        r = O.quant_error_stats(oshape_of(w, 1, ah=ah), inp["k"], inp["pos"], ang, b, g)
        one = run_stats(w, inp["k"], inp["pos"], ang, b, g, ah=ah, layout=1)
        for got in (sw[j], one):
            rel = np.abs(got[:5] - r[:5]) / np.maximum(np.abs(r[:5]), 1e-300)
            assert np.all(rel <= STAT_TOL), (b, got, r, rel)
            assert got[5] == r[5] and got[6] == r[6]


# ---------------------------------------------------------------------------
# The large-batch kernel family (4096 tokens or more: one wave per token, waves
# walking the batch with a grid stride) against the oracle, for every
# compile-time variant a prefill can reach: runtime support b < d, groups
# smaller than a 16-byte chunk, interleaved pairs, fp32 rows, head_dim 64,
# per-key-head angle sets and the V half.  A grid-stride round is 32768 blocks
# x 4 waves = 131072 tokens for Q/K launches with shared angles (whose waves
# stage Q rows through LDS, reused token after token) and 8192 blocks x 4 waves
# = 32768 tokens with V rows or per-set angles.  Batches are longer than one
# round of their launch, and the sampled tokens include both ends of every
# round, the last one in particular.
# ---------------------------------------------------------------------------

GRID_STRIDE_TOKENS = 8192 * 4  # round of the launches with V rows or per-set angles
GRID_STRIDE_TOKENS_QK = 32768 * 4  # round of the Q/K launches with shared angles
T_TWO_ROUNDS = GRID_STRIDE_TOKENS_QK + 8192 + 77  # past one shared-angle round, ragged


def grid_sample(T, n, seed):
    """n sampled tokens of a T-token batch plus the first and last token of every
    grid-stride round of either launch shape."""
    assert T >= 4096
    edges = []
    for rnd in (GRID_STRIDE_TOKENS, GRID_STRIDE_TOKENS_QK):
        for r0 in range(0, T, rnd):
            edges += [r0, min(T, r0 + rnd) - 1]
    return np.unique(np.concatenate([sample_tokens(T, n, seed), np.array(edges)]))


def degenerate_k(w, T, seed, regime):
    """K rows of workload w's shape for one special case of the quantiser, so
    the diagnostics' sums are dominated by it:
    - "zero": all-zero rows and rows whose fp16 scale underflows to 0 (1e-9),
      among ordinary rows;
    - "saturated": +-1e6 rows and rows of ordinary values with a 1e6 outlier
      channel, whose fp16 scale saturates at 65504 (codes clamp at +-7);
    - "subnormal": rows of magnitude 10^U(-7, -6), whose fp16 scale is a coarse
      subnormal; about a fifth of the groups have codes past +-7.5 before
      clamping (the kernels' rare correction pass), some underflow to 0."""
    rng = np.random.default_rng(seed)
    hk, d = w.n_kv_heads, w.head_dim
    k = rng.normal(0.0, 1.0, (T, hk, d))
    if regime == "zero":
        k[0::3] = 0.0
        k[1::3] = 1e-9
    elif regime == "saturated":
        k[0::2] = 1e6 * np.sign(np.arange(d) - (d - 1) / 2.0) * rng.uniform(0.5, 2.0, (len(k[0::2]), hk, 1))
        k[1::2, :, 5] = 1e6
    else:
        k *= 10.0 ** rng.uniform(-7.0, -6.0, (T, hk, 1))
    k = k.astype(np.float32)
    if w.dtype == "bf16":
        return torch.from_numpy(k).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return k


@pytest.mark.parametrize("regime", ["zero", "saturated", "subnormal"])
@pytest.mark.parametrize("n", [1, 3])
def test_diagnostics_parity_degenerate_rows(n, regime):
    """Stats at several (b, g) and the sweep at several g on K rows of one
    special case of the quantiser (zero or underflowing scales, saturated
    scales, coarse subnormal scales: the latter two go through the rare
    clamped-code correction pass), against the oracle at the diagnostics
    tolerances."""
    w = W.WORKLOADS[n]
    T = 40
    inp = W.make_inputs(n, n_tokens=T)
    k = degenerate_k(w, T, 3100 + n, regime)
    pos = inp["pos"]
    ang = random_angles(w.n_pairs, 3200 + n)
    d = w.head_dim
    for b in (1, 2, 16, d):
        for g in (2, 16, d):
            got = run_stats(w, k, pos, ang, b, g)
            ref = O.quant_error_stats(oshape_of(w), k, pos, ang, b, g)
            rel = np.abs(got[:5] - ref[:5]) / np.maximum(np.abs(ref[:5]), 1e-300)
            assert np.all(rel <= STAT_TOL), (b, g, got, ref, rel)
    supports = rrp.sweep_supports(d)
    for g in (2, 8, d):
        sw = run_sweep(w, k, pos, ang, g)
        for j, b in enumerate(supports):
            ref = O.quant_error_stats(oshape_of(w), k, pos, ang, b, g)
            rel = np.abs(sw[j, :5] - ref[:5]) / np.maximum(np.abs(ref[:5]), 1e-300)
            assert np.all(rel <= STAT_TOL), (g, b, sw[j], ref, rel)


@pytest.mark.parametrize("ah", [0, 8])
def test_empty_batches_every_entry_point(ah):
    """No tokens (or no sequences, or only empty sequences): every entry point
    returns without error and writes only what its definition fixes for an
    empty batch.
    - rotate leaves the cache and the query outputs untouched;
    - calibration leaves the moments as they were and finalises the angles
      from them;
    - the diagnostics and the sweep equal the oracle's empty-batch statistics
      (zeros, and the sweep's support b in field 7);
    - decode writes no logit."""
    w = W.WORKLOADS[3]
    d, hq, hk, g = w.head_dim, w.n_q_heads, w.n_kv_heads, w.group
    shp = shape_of(w, ah=ah)
    e = torch.empty((0, hq, d), dtype=torch.bfloat16, device=DEV)
    ek = torch.empty((0, hk, d), dtype=torch.bfloat16, device=DEV)
    ep = torch.empty((0,), dtype=torch.int32, device=DEV)
    ang_np = random_angle_sets(w, 3300) if ah else random_angles(w.n_pairs, 3300)
    ang = to_dev(ang_np)
    codes, scales = rrp.new_kv4_cache(16, hk, d, g, DEV)
    codes.fill_(0x5A)
    scales.view(torch.int16).fill_(0x1234)
    rrp.rotate_quantize_qk(shp, e, ek, ep, support_b=d, group=g, k_codes=codes, k_scales=scales, angles=ang,
                           q_out=torch.empty_like(e), n_slots=16)
    torch.cuda.synchronize()
    assert bool((codes == 0x5A).all()) and bool((scales.view(torch.int16) == 0x1234).all())

    # calibration: moments carried in from an earlier batch stay; the angles follow from them
    inp = inputs(3)
    q0, k0, p0 = inp["q"][:64], inp["k"][:64], inp["pos"][:64]
    mom_prev, _ = run_calib(w, q0, k0, p0, "default", ah=ah)
    mom = torch.from_numpy(mom_prev).to(DEV)
    A = max(ah, 1)
    ang_out = torch.empty((d // 2,) if A == 1 else (A, d // 2), dtype=torch.float32, device=DEV)
    rrp.calibrate_angles(shp, e, ek, ep, moments=mom, estimator="default", angles_out=ang_out)
    torch.cuda.synchronize()
    assert np.array_equal(mom.cpu().numpy(), mom_prev)
    phi64, _, abc = O.angles_from_moments(mom_prev, O.EST_DEFAULT)
    C.compare_angles(ang_out.cpu().numpy().reshape(-1), phi64.reshape(-1), abc.reshape(-1, 3))

    oshp = oshape_of(w, ah=ah)
    empty_k = np.zeros((0, hk, d), np.uint16)
    empty_p = np.zeros((0,), np.int32)
    st = torch.full((8,), -1.0, dtype=torch.float64, device=DEV)
    rrp.quant_error_stats(shp, ek, ep, support_b=16, group=g, stats_out=st, angles=ang)
    sups = rrp.sweep_supports(d)
    sw = torch.full((len(sups), 8), -1.0, dtype=torch.float64, device=DEV)
    rrp.quant_error_sweep(shp, ek, ep, group=g, stats_out=sw, angles=ang)
    torch.cuda.synchronize()
    assert np.array_equal(st.cpu().numpy(), O.quant_error_stats(oshp, empty_k, empty_p, ang_np, 16, g))
    ref = np.stack([O.quant_error_stats(oshp, empty_k, empty_p, ang_np, b, g) for b in sups])
    ref[:, 7] = sups
    assert np.array_equal(sw.cpu().numpy(), ref)

    # decode: no sequences, then sequences that are all empty
    for lens in ([], [0, 0, 0]):
        B = len(lens)
        out = torch.full((B, hq, 8), float("-inf"), dtype=torch.float32, device=DEV)
        rrp.decode_scores(shape_of(w), torch.zeros((B, hq, d), dtype=torch.bfloat16, device=DEV), codes, scales,
                          group=g, seq_start=torch.zeros(B, dtype=torch.int64, device=DEV),
                          seq_len=torch.tensor(lens, dtype=torch.int32, device=DEV), max_len=8, scores=out)
        torch.cuda.synchronize()
        assert bool(torch.isneginf(out).all())


def long_inputs(n, T):
    key = ("long", n, T)
    if key not in _INPUTS:
        _INPUTS[key] = W.make_inputs(n, n_tokens=T)
    return _INPUTS[key]


@pytest.mark.parametrize("ah", [0, 8])
@pytest.mark.parametrize("b", [1, 2, 16, 64])
def test_grid_stride_prefill_128k_support_sweep(b, ah):
    """The 131072-token prefill at b < d, shared and per-key-head angles, in the
    benchmark's launch configuration (one round of the shared-angle launch, four
    of the per-set launch)."""
    w, inp = W.WORKLOADS[4], inputs(4)
    ang = random_angle_sets(w, 2000 + b) if ah else random_angles(w.n_pairs, 2000 + b)
    out = run_rotate(w, inp, ang, b, 128, debug=False, ah=ah)
    idx = grid_sample(w.n_tokens, 768, 2000 + b + ah)
    assert idx.max() == w.n_tokens - 1 and (idx >= 3 * GRID_STRIDE_TOKENS).sum() > 100
    print(b, ah, check_rotate(w, inp, out, ang, b, 128, idx, ah=ah))


@pytest.mark.parametrize("b", [2, 128])
@pytest.mark.parametrize("g", [2, 4, 16])
def test_grid_stride_prefill_128k_small_groups(g, b):
    """Groups of 2 and 4 channels (reduced inside a lane) and 16 (across two lanes)
    on the full prefill."""
    w, inp = W.WORKLOADS[4], inputs(4)
    ang = random_angles(w.n_pairs, 2100 + g)
    out = run_rotate(w, inp, ang, b, g, debug=False)
    print(g, b, check_rotate(w, inp, out, ang, b, g, grid_sample(w.n_tokens, 512, 2100 + g + b)))


@pytest.mark.parametrize("b,ah", [(128, 0), (16, 0), (2, 8)])
def test_grid_stride_prefill_128k_interleaved_pairs(b, ah):
    w, inp = W.WORKLOADS[4], inputs(4)
    ang = random_angle_sets(w, 2200 + b) if ah else random_angles(w.n_pairs, 2200 + b)
    out = run_rotate(w, inp, ang, b, 128, debug=False, layout=1, ah=ah)
    print(b, ah, check_rotate(w, inp, out, ang, b, 128, grid_sample(w.n_tokens, 512, 2200 + b), layout=1, ah=ah))


@pytest.mark.parametrize("b,g,layout", [(2, 64, 0), (64, 64, 0), (8, 2, 0), (32, 16, 1), (1, 64, 1)])
def test_grid_stride_fp32_rows_tiny_shape(b, g, layout):
    """fp32 rows of the tiny workload's shape (2 Q / 1 KV heads, d 64) over
    T_TWO_ROUNDS tokens (past one shared-angle round), with the fp32 debug
    copies."""
    w = W.WORKLOADS[1]
    T = T_TWO_ROUNDS
    inp = long_inputs(1, T)
    ang = random_angles(w.n_pairs, 2300 + b)
    out = run_rotate(w, inp, ang, b, g, layout=layout)
    print(b, g, layout, check_rotate(w, inp, out, ang, b, g, grid_sample(T, 2048, 2300 + b), layout=layout))


@pytest.mark.parametrize("b,g,ah", [(2, 64, 0), (16, 64, 0), (32, 4, 0), (64, 64, 8), (4, 16, 8)])
def test_grid_stride_head_dim_64(b, g, ah):
    """head_dim 64 (the 1B layer's 32 / 8 heads) over T_TWO_ROUNDS tokens (past
    one shared-angle round), with the fp32 debug copies."""
    w = W.WORKLOADS[2]
    T = T_TWO_ROUNDS
    inp = long_inputs(2, T)
    ang = random_angle_sets(w, 2400 + b) if ah else random_angles(w.n_pairs, 2400 + b)
    out = run_rotate(w, inp, ang, b, g, ah=ah)
    print(b, g, ah, check_rotate(w, inp, out, ang, b, g, grid_sample(T, 768, 2400 + b), ah=ah))


@pytest.mark.parametrize("b,g,layout", [(2, 4, 0), (16, 128, 1), (64, 16, 0), (128, 128, 0)])
def test_grid_stride_two_rounds_shared_angles(b, g, layout):
    """The 128K prefill's shape over T_TWO_ROUNDS tokens with shared angles: the
    waves of the first 8269 token slots walk a second token, reusing the LDS
    buffer their first token's Q rows were staged in."""
    w = W.WORKLOADS[4]
    T = T_TWO_ROUNDS
    inp = long_inputs(4, T)
    ang = random_angles(w.n_pairs, 2600 + b)
    out = run_rotate(w, inp, ang, b, g, debug=False, layout=layout)
    idx = grid_sample(T, 768, 2600 + b + g)
    assert (idx >= GRID_STRIDE_TOKENS_QK).sum() > 30
    print(b, g, layout, check_rotate(w, inp, out, ang, b, g, idx, layout=layout))


@pytest.mark.parametrize("hq,hk,b,g,ah", [(64, 8, 128, 128, 0), (64, 8, 16, 32, 0), (64, 8, 2, 8, 8),
                                          (12, 4, 128, 128, 0), (12, 4, 16, 4, 4)])
def test_grid_stride_many_query_heads(hq, hk, b, g, ah):
    """Head counts other than the workloads': 64 query heads over 8 key heads
    (eight Q passes per token: with shared angles the kernel stages Q passes 1-3
    through LDS and loads passes 4-7 one ahead into VGPRs), and 12 over 4 (the
    staged second Q pass and the K pass only half filled: the masked lanes
    neither load nor store).  A ragged batch past one grid-stride round of the
    shared-angle launch, against the oracle on sampled tokens."""
    import dataclasses
    w = dataclasses.replace(W.WORKLOADS[4], n_q_heads=hq, n_kv_heads=hk, n_tokens=T_TWO_ROUNDS)
    T = T_TWO_ROUNDS
    key = ("heads", hq, hk, T)
    if key not in _INPUTS:
        rng = np.random.Generator(np.random.PCG64(2700 + hq))
        scale = rng.lognormal(0.0, 0.7, w.head_dim).astype(np.float32)
        normal = lambda n: rng.standard_normal((T, n, w.head_dim), dtype=np.float32) * scale  # noqa: E731
        _INPUTS[key] = {"q": W._to_storage(normal(hq), "bf16"), "k": W._to_storage(normal(hk), "bf16"),
                        "pos": np.arange(T, dtype=np.int32)}
    inp = _INPUTS[key]
    ang = random_angle_sets(w, 2700 + b) if ah else random_angles(w.n_pairs, 2700 + b)
    out = run_rotate(w, inp, ang, b, g, debug=False, ah=ah)
    idx = grid_sample(T, 512, 2700 + b + g)
    print(b, g, ah, check_rotate(w, inp, out, ang, b, g, idx, ah=ah))


@pytest.mark.parametrize("b,g,ah", [(2, 4, 0), (16, 128, 8)])
def test_grid_stride_prefill_128k_with_v(b, g, ah):
    """The V half at b < d and a small group on the full prefill."""
    w = W.WORKLOADS[4]
    inp = vinputs(4)
    ang = random_angle_sets(w, 2500 + b) if ah else random_angles(w.n_pairs, 2500 + b)
    out = run_rotate_qkv(w, inp, ang, b, g, debug=False, ah=ah)
    idx = grid_sample(w.n_tokens, 512, 2500 + b)
    print(b, g, ah, check_rotate(w, inp, out, ang, b, g, idx, ah=ah), check_v(w, inp, out, g, idx))


# ---------------------------------------------------------------------------
# caller-owned workspace
# ---------------------------------------------------------------------------

def test_explicit_workspace_reused_across_calls():
    """One oversized workspace tensor passed to calibration, diagnostics and the
    sweep, call after call, gives the same results as the binding's own
    per-call workspace; a short one is rejected before any launch."""
    w, inp = W.WORKLOADS[3], inputs(3)
    shape = shape_of(w)
    q, k, pos = to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["pos"])
    T = w.n_tokens
    need = max(rrp.calibrate_workspace_bytes(shape, T), rrp.quant_error_stats_workspace_bytes(shape, T),
               rrp.quant_error_sweep_workspace_bytes(shape, T))
    ws = torch.full((need + 4096,), 0xA5, dtype=torch.uint8, device=DEV)  # stale contents must not matter
    nb = len(rrp.sweep_supports(w.head_dim))
    results = []
    for workspace in (ws, None, ws):
        mom = rrp.new_moments(w.head_dim, DEV)
        ang = torch.empty(w.n_pairs, dtype=torch.float32, device=DEV)
        rrp.calibrate_angles(shape, q, k, pos, moments=mom, angles_out=ang, workspace=workspace)
        st = torch.empty(8, dtype=torch.float64, device=DEV)
        rrp.quant_error_stats(shape, k, pos, support_b=16, group=32, stats_out=st, angles=ang, workspace=workspace)
        sw = torch.empty((nb, 8), dtype=torch.float64, device=DEV)
        rrp.quant_error_sweep(shape, k, pos, group=128, stats_out=sw, angles=ang, workspace=workspace)
        torch.cuda.synchronize()
        results.append([x.cpu().numpy() for x in (mom, ang, st, sw)])
    for a, b in zip(results[0], results[1]):
        assert np.array_equal(a, b)
    for a, b in zip(results[0], results[2]):
        assert np.array_equal(a, b)
    short = torch.empty(rrp.calibrate_workspace_bytes(shape, T) - 8, dtype=torch.uint8, device=DEV)
    with pytest.raises(ValueError, match="workspace"):
        rrp.calibrate_angles(shape, q, k, pos, moments=rrp.new_moments(w.head_dim, DEV), workspace=short)
