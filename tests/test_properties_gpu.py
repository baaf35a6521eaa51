"""Properties of the HIP path at the full 131072-token prefill size, checked on
every token (the oracle is compared element by element elsewhere, on chunks and
samples of the same launch).

* The transform is orthogonal: each rotated row keeps the norm of its input row
  (the page on RoPE-aligned rotations, theoretical characterisation; the notes'
  section 2.1 on rotation equivalence).
* The pair rotation and the block Hadamard are shared by Q and K, so every
  query-key inner product equals the plain-RoPE one (the notes' section 3.2.1:
  the rotation cancels in Q K^T).  The plain-RoPE rows come from the same entry
  point with b = 1 and no pair angles.
* The group quantiser maps each group's absmax element to +-7, never uses -8,
  and leaves every element within half a scale step (the notes' section 1.2).

Tolerances follow from the fp32 rows the kernel exports (about 2^-24 per
operation over at most 2 * 7 + 2 roundings per value): 1e-5 relative.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import rotation_rope_pair_amd as rrp  # noqa: E402
from rotation_rope_pair_amd import workloads as W  # noqa: E402

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU-only container
    pytest.skip("no GPU", allow_module_level=True)

DEV = torch.device("cuda:0")
TOL = 1e-5

_STATE = {}


def bf16_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(torch.bfloat16)


def prefill():
    """The 128K prefill inputs on the device, and the rotated fp32 rows of two
    launches: b = 128 with random pair angles, and b = 1 with none (RoPE only)."""
    if "out" in _STATE:
        return _STATE["out"]
    w = W.WORKLOADS[4]
    inp = W.make_inputs(4)
    T, hq, hk, d, g = w.n_tokens, w.n_q_heads, w.n_kv_heads, w.head_dim, 128
    q, k = bf16_dev(inp["q"]), bf16_dev(inp["k"])
    pos = torch.from_numpy(inp["pos"]).to(DEV)
    shape = rrp.layer_shape(hq, hk, d, w.rope_theta)
    rng = np.random.Generator(np.random.PCG64(4242))
    ang = torch.from_numpy(rng.uniform(-np.pi / 4, np.pi / 4, d // 2).astype(np.float32)).to(DEV)
    runs = {}
    for name, b, angles in (("full", 128, ang), ("rope", 1, None)):
        codes, scales = rrp.new_kv4_cache(T, hk, d, g, DEV)
        qr = torch.empty((T, hq, d), dtype=torch.float32, device=DEV)
        kr = torch.empty((T, hk, d), dtype=torch.float32, device=DEV)
        s32 = torch.empty((T, hk, d // g), dtype=torch.float32, device=DEV)
        rrp.rotate_quantize_qk(shape, q, k, pos, support_b=b, group=g, k_codes=codes, k_scales=scales,
                               angles=angles, q_out=None, q_rot_f32=qr, k_rot_f32=kr, k_scale_f32=s32)
        runs[name] = {"q": qr, "k": kr, "codes": codes, "scales": scales, "s32": s32}
    torch.cuda.synchronize()
    _STATE["out"] = (w, q, k, runs)
    return _STATE["out"]


def test_prefill_128k_rows_keep_their_norm():
    w, q, k, runs = prefill()
    for name in ("full", "rope"):
        for x_in, x_out in ((q, runs[name]["q"]), (k, runs[name]["k"])):
            n_in = torch.linalg.vector_norm(x_in.double(), dim=-1)
            n_out = torch.linalg.vector_norm(x_out.double(), dim=-1)
            rel = ((n_out - n_in).abs() / n_in.clamp_min(1e-30)).max().item()
            assert rel <= TOL, (name, rel)


def test_prefill_128k_query_key_products_match_plain_rope():
    """<T q_h, T k_kv(h)> = <RoPE q_h, RoPE k_kv(h)> for every token and query head."""
    w, q, k, runs = prefill()
    gsz = w.n_q_heads // w.n_kv_heads
    worst = 0.0
    chunk = 16384
    for t0 in range(0, w.n_tokens, chunk):
        sl = slice(t0, min(w.n_tokens, t0 + chunk))
        dots = []
        norms = None
        for name in ("full", "rope"):
            qr = runs[name]["q"][sl].double()
            kr = runs[name]["k"][sl].double().repeat_interleave(gsz, dim=1)
            dots.append((qr * kr).sum(-1))
            if name == "rope":
                norms = torch.linalg.vector_norm(qr, dim=-1) * torch.linalg.vector_norm(kr, dim=-1)
        rel = ((dots[0] - dots[1]).abs() / norms.clamp_min(1e-30)).max().item()
        worst = max(worst, rel)
    assert worst <= 2 * TOL, worst
    print("max |<Tq,Tk> - <Rq,Rk>| / (|q||k|):", worst)


def test_prefill_128k_codes_follow_the_group_quantiser():
    """Every code of the 131072 x 8 K rows: in [-7, 7], +-7 at the group's absmax
    element, and within half a scale step of the fp32 row."""
    w, q, k, runs = prefill()
    d, g = w.head_dim, 128
    for name in ("full", "rope"):
        r = runs[name]
        by = r["codes"].to(torch.int16)
        lo = by & 0xF
        hi = (by >> 4) & 0xF
        codes = torch.stack((lo, hi), dim=-1).reshape(w.n_tokens, w.n_kv_heads, d)
        codes = torch.where(codes >= 8, codes - 16, codes)
        assert int(codes.min().item()) >= -7 and int(codes.max().item()) <= 7, name
        s_h = r["scales"].float().repeat_interleave(g, dim=-1)
        y = r["k"]
        groups = y.reshape(w.n_tokens, w.n_kv_heads, d // g, g)
        cg = codes.reshape(groups.shape)
        arg = groups.abs().argmax(dim=-1, keepdim=True)
        top = cg.gather(-1, arg).abs()
        nonzero = r["scales"].float() > 0
        assert bool((top.squeeze(-1)[nonzero] == 7).all()), name
        err = (codes.float() * s_h - y).abs()
        bound = 0.5 * s_h * (1 + TOL) + TOL * y.abs()
        assert bool((err <= bound).all()), (name, float((err - bound).max().item()))
