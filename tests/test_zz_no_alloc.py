"""rrp_calibrate_angles_noalloc (the calibration that allocates nothing, its
block partials in the library's static device scratch) against
rrp_calibrate_angles with a caller workspace, through the C-ABI: two calls in a
row on one GPU, the second with a smaller batch, each giving the same moments
and angles bit for bit (the same partials reduced in the same order), within
the oracle's bars too."""
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
EST = {"default": O.EST_DEFAULT, "k_only": O.EST_K_ONLY, "stream_balanced": O.EST_STREAM_BALANCED}


def to_dev(a):
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def both(w, q, k, pos, est, ah):
    """(moments, angles) of the no-allocation call and of the workspace call."""
    shape = rrp.layer_shape(w.n_q_heads, w.n_kv_heads, w.head_dim, w.rope_theta, angle_heads=ah)
    sets = rrp.angle_sets(shape)
    qd, kd, pd = to_dev(q), to_dev(k), to_dev(pos)
    out = []
    for fn in (rrp.calibrate_angles_noalloc, rrp.calibrate_angles):
        mom = rrp.new_moments(w.head_dim, DEV, n_sets=sets)
        ang = torch.empty((sets, w.head_dim // 2) if sets > 1 else (w.head_dim // 2,), dtype=torch.float32,
                          device=DEV)
        fn(shape, qd, kd, pd, moments=mom, estimator=est, angles_out=ang)
        torch.cuda.synchronize()
        out.append((mom.cpu().numpy(), ang.cpu().numpy()))
    return out


def check(w, q, k, pos, est, ah):
    (m0, a0), (m1, a1) = both(w, q, k, pos, est, ah)
    assert np.array_equal(m0, m1) and np.array_equal(a0, a1)
    shp = O.shape(w.n_q_heads, w.n_kv_heads, w.head_dim, w.rope_theta, angle_heads=ah)
    ref = O.calibrate_moments(shp, q, k, pos)
    phi64, _, abc = O.angles_from_moments(ref, EST[est])
    C.compare_moments(m0, ref)
    return C.compare_angles(a0.reshape(-1), phi64.reshape(-1), abc.reshape(-1, 3))


@pytest.mark.parametrize("est,ah", [("default", 0), ("k_only", 8)])
def test_noalloc_calibration_equals_workspace_call_twice(est, ah):
    w = W.WORKLOADS[3]
    inp = W.make_inputs(3, n_tokens=16384)
    q = inp["q"] if est != "k_only" else None
    print("first call:", check(w, q, inp["k"], inp["pos"], est, ah))
    T2 = 1000  # fewer blocks than the first call: the second reads only its own partials
    print("second call:", check(w, None if q is None else q[:T2], inp["k"][:T2], inp["pos"][:T2], est, ah))


def test_noalloc_calibration_accumulates_and_finalises():
    """Moments accumulate over two no-allocation calls as over two workspace calls,
    and a call with no tokens only finalises."""
    w = W.WORKLOADS[2]
    inp = W.make_inputs(2)
    shape = rrp.layer_shape(w.n_q_heads, w.n_kv_heads, w.head_dim, w.rope_theta)
    q, k, pos = to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["pos"])
    res = []
    for fn in (rrp.calibrate_angles_noalloc, rrp.calibrate_angles):
        mom = rrp.new_moments(w.head_dim, DEV)
        ang = torch.empty(w.n_pairs, dtype=torch.float32, device=DEV)
        fn(shape, q[:1500], k[:1500], pos[:1500], moments=mom)
        fn(shape, q[1500:], k[1500:], pos[1500:], moments=mom)
        e = torch.empty((0,), dtype=torch.bfloat16, device=DEV)
        fn(shape, e, e, torch.empty((0,), dtype=torch.int32, device=DEV), moments=mom, estimator="stream_balanced",
           angles_out=ang)
        torch.cuda.synchronize()
        res.append((mom.cpu().numpy(), ang.cpu().numpy()))
    assert np.array_equal(res[0][0], res[1][0]) and np.array_equal(res[0][1], res[1][1])
