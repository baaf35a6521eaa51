"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks an oracle function against something other than itself: a
library routine (HF transformers' RoPE, scipy's Hadamard, numpy's float16 and
covariance, torch's bfloat16), a closed form, brute force on tiny inputs, an
invariant the pages state, or a worked example printed on a page
(tests/golden/).  Page references: [RAQK] = "When Local Variance Optimality Is
Not Enough: RoPE-Aligned Q/K Rotations for Dynamic 4-Bit Quantisation"
(abstract and technical summaries); [NOTES] = "LLM旋转量化笔记".
"""
import json
import math
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


# --------------------------------------------------------------------------
# RoPE: frequencies, layout, sign convention ([RAQK] problem statement).
# --------------------------------------------------------------------------

def _hf_inv_freq(theta, d):
    import torch
    from transformers import LlamaConfig
    from transformers.models.llama.modeling_llama import LlamaRotaryEmbedding
    cfg = LlamaConfig(hidden_size=d * 4, num_attention_heads=4, head_dim=d, rope_theta=theta,
                      max_position_embeddings=4096)
    emb = LlamaRotaryEmbedding(config=cfg, device=torch.device("cpu"))
    return emb.inv_freq.to(torch.float32).numpy()


@pytest.mark.parametrize("theta,d", [(5e5, 64), (5e5, 128), (1e6, 128), (1e4, 64)])
def test_inv_freq_matches_hf_default_rope(orc, theta, d):
    ours = orc.inv_freq(theta, d)
    hf = _hf_inv_freq(theta, d)
    # HF evaluates theta ** (2k/d) in fp32 and takes the reciprocal; ours rounds the
    # fp64 value once.  Both approximate theta^(-2k/d): allow a few fp32 ulps.
    ulp = np.spacing(np.abs(hf).astype(np.float32))
    assert np.all(np.abs(ours.astype(np.float64) - hf) <= 4 * ulp)
    # closed-form structure: w_0 = 1, a geometric progression of ratio theta^(-2/d),
    # extrapolating to 1/theta at k = d/2; all frequencies distinct.
    assert ours[0] == 1.0
    ratios = ours[1:].astype(np.float64) / ours[:-1]
    assert np.allclose(ratios, theta ** (-2.0 / d), rtol=2e-7)
    assert abs(ours[-1] * theta ** (-2.0 / d) * theta - 1) < 1e-6
    assert np.all(np.diff(ours) < 0)


def test_rope_angle_is_one_fp32_multiply(orc):
    for p, w in [(131071, 1.0), (131071, 0.8), (4095, 0.123456789), (32767, 3.1e-6), (0, 0.5)]:
        a = orc.rope_angle(p, np.float32(w))
        assert a == np.float32(np.float32(p) * np.float32(w))


def test_rope_matches_hf_apply_rotary_pos_emb(orc):
    import torch
    from transformers.models.llama.modeling_llama import apply_rotary_pos_emb
    d, theta = 64, 5e5
    inv = orc.inv_freq(theta, d)
    rng = _rng(1)
    x = rng.standard_normal((3, d))
    pos = [0, 17, 131071]
    # HF's half-split convention: cos/sin tables are cat(freqs, freqs).
    ang = np.array([[orc.rope_angle(p, w) for w in inv] for p in pos], np.float64)
    cos = torch.from_numpy(np.cos(np.concatenate([ang, ang], -1)))[None]
    sin = torch.from_numpy(np.sin(np.concatenate([ang, ang], -1)))[None]
    xt = torch.from_numpy(x)[None, None]  # [batch, heads, seq, d]
    qh, _ = apply_rotary_pos_emb(xt, xt, cos, sin)
    qh = qh[0, 0].numpy()
    for i, p in enumerate(pos):
        ours = orc.rope_row(x[i], orc.HALF_SPLIT, inv, p)
        assert np.allclose(ours, qh[i], rtol=0, atol=1e-13)


@pytest.mark.parametrize("layout", [0, 1])
def test_rope_complex_form(orc, layout):
    d = 16
    inv = orc.inv_freq(1e4, d)
    x = _rng(2).standard_normal(d)
    p = 1234
    out = orc.rope_row(x, layout, inv, p)
    for k in range(d // 2):
        lo, hi = (k, k + d // 2) if layout == 0 else (2 * k, 2 * k + 1)
        z = complex(x[lo], x[hi]) * np.exp(1j * float(orc.rope_angle(p, inv[k])))
        assert abs(out[lo] - z.real) < 1e-13 and abs(out[hi] - z.imag) < 1e-13


def test_rope_relative_position_property(orc):
    """<RoPE_p(a), RoPE_q(b)> depends only on p - q (up to the fp32 angle rounding)."""
    d = 64
    inv = orc.inv_freq(5e5, d)
    rng = _rng(3)
    a, b = rng.standard_normal(d), rng.standard_normal(d)
    ref = orc.rope_row(a, 0, inv, 40) @ orc.rope_row(b, 0, inv, 33)
    for s in (1, 7, 100):
        got = orc.rope_row(a, 0, inv, 40 + s) @ orc.rope_row(b, 0, inv, 33 + s)
        assert abs(got - ref) < 1e-4 * (np.linalg.norm(a) * np.linalg.norm(b))


def test_rope_at_position_zero_is_identity(orc):
    x = _rng(4).standard_normal(128)
    inv = orc.inv_freq(5e5, 128)
    for layout in (0, 1):
        assert np.array_equal(orc.rope_row(x, layout, inv, 0), x)


# --------------------------------------------------------------------------
# Block Hadamard ([RAQK] contributions: support b; [NOTES] 2.2, 6.1).
# --------------------------------------------------------------------------

@pytest.mark.parametrize("b", [1, 2, 4, 8, 16, 32, 64, 128])
def test_hadamard_matches_scipy_sylvester(orc, b):
    import scipy.linalg
    n = 256
    x = _rng(5).standard_normal(n)
    H = scipy.linalg.hadamard(b).astype(np.float64) / math.sqrt(b)
    ref = (x.reshape(-1, b) @ H.T).reshape(-1)
    assert np.allclose(orc.hadamard_blocks(x, b), ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("b", [2, 8, 64])
def test_hadamard_is_orthogonal(orc, b):
    M = np.stack([orc.hadamard_blocks(np.eye(b)[j], b) for j in range(b)], 1)
    assert np.allclose(M @ M.T, np.eye(b), atol=1e-13)
    # unnormalised entries are +-1 and the first row/column is all ones (Sylvester)
    assert np.allclose(np.abs(M) * math.sqrt(b), 1.0)
    assert np.allclose(M[0] * math.sqrt(b), 1.0) and np.allclose(M[:, 0] * math.sqrt(b), 1.0)


def test_hadamard_worked_example_outlier_spread(orc):
    g = json.load(open(os.path.join(GOLDEN, "hadamard_outlier_k4096.json")))
    K = g["input"]["K"]
    x = np.full(K, g["input"]["background_value"])
    x[g["input"]["outlier_index"]] = g["input"]["outlier_value"]
    y = orc.hadamard_blocks(x, K)
    share = g["page_values"]["outlier_share_per_channel"]
    # every output channel but the coherent first one carries ~ the page's share
    assert np.all(np.abs(np.abs(y[1:]) - share) / share < g["tolerance_vs_page"])
    # exact closed form with the background included
    bg, out = g["input"]["background_value"], g["input"]["outlier_value"]
    signs = np.array([(-1.0) ** bin(i).count("1") for i in range(1, K)])
    assert np.allclose(y[1:], signs * (out - bg) / math.sqrt(K), rtol=0, atol=1e-12)
    assert abs(y[0] - ((K - 1) * bg + out) / math.sqrt(K)) < 1e-11


@pytest.mark.parametrize("b", [1, 2, 4, 16, 128])
def test_one_hot_row_spreads_as_inverse_sqrt_b(orc, b):
    d, A, j = 128, 3.0, 37
    x = np.zeros(d)
    x[j] = A
    y = orc.hadamard_blocks(x, b)
    blk = slice((j // b) * b, (j // b + 1) * b)
    assert np.allclose(np.abs(y[blk]), A / math.sqrt(b), atol=1e-14)
    mask = np.ones(d, bool)
    mask[blk] = False
    assert np.all(y[mask] == 0)
    # through the whole transform at p = 0 without pair angles the same holds
    inv = orc.inv_freq(5e5, d)
    assert np.allclose(orc.transform_row(x, 0, inv, 0, None, b), y, atol=1e-14)


# --------------------------------------------------------------------------
# Pair rotation and the transform's invariants ([RAQK] theoretical
# characterisation; [NOTES] 2.2 norm preservation, 3.2.1 QK^T cancellation).
# --------------------------------------------------------------------------

def test_pair_rotation_complex_form_and_commutes_with_rope(orc):
    d = 32
    rng = _rng(6)
    x = rng.standard_normal(d)
    phi = rng.uniform(-math.pi / 4, math.pi / 4, d // 2).astype(np.float32)
    inv = orc.inv_freq(5e5, d)
    for layout in (0, 1):
        r = orc.pair_rotate_row(x, layout, phi)
        for k in range(d // 2):
            lo, hi = (k, k + d // 2) if layout == 0 else (2 * k, 2 * k + 1)
            z = complex(x[lo], x[hi]) * np.exp(1j * float(phi[k]))
            assert abs(r[lo] - z.real) < 1e-14 and abs(r[hi] - z.imag) < 1e-14
        for p in (1, 999, 70000):
            a = orc.pair_rotate_row(orc.rope_row(x, layout, inv, p), layout, phi)
            b = orc.rope_row(orc.pair_rotate_row(x, layout, phi), layout, inv, p)
            assert np.allclose(a, b, atol=1e-13)


def test_full_hadamard_does_not_commute_with_rope(orc):
    """Negative form of the converse result: a full-head Hadamard is not in the
    RoPE-commuting family, so H RoPE_p != RoPE_p H for p != 0."""
    d = 64
    x = _rng(7).standard_normal(d)
    inv = orc.inv_freq(5e5, d)
    for p in (1, 50):
        a = orc.hadamard_blocks(orc.rope_row(x, 0, inv, p), d)
        b = orc.rope_row(orc.hadamard_blocks(x, d), 0, inv, p)
        assert np.max(np.abs(a - b)) > 1e-3


@pytest.mark.parametrize("b", [1, 2, 16, 64])
def test_transform_preserves_qk_dot_products_and_norms(orc, b):
    d, hq, hk = 64, 4, 2
    rng = _rng(8 + b)
    q = rng.standard_normal((hq, d)) * rng.lognormal(0, 1, d)
    k = rng.standard_normal((hk, d)) * rng.lognormal(0, 1, d)
    phi = rng.uniform(-math.pi / 4, math.pi / 4, d // 2).astype(np.float32)
    inv = orc.inv_freq(5e5, d)
    pq, pk = 1000, 731
    for h in range(hq):
        kv = h * hk // hq
        tq = orc.transform_row(q[h], 0, inv, pq, phi, b)
        tk = orc.transform_row(k[kv], 0, inv, pk, phi, b)
        rq = orc.rope_row(q[h], 0, inv, pq)
        rk = orc.rope_row(k[kv], 0, inv, pk)
        assert abs(tq @ tk - rq @ rk) <= 1e-12 * np.linalg.norm(q[h]) * np.linalg.norm(k[kv])
        assert abs(np.linalg.norm(tq) - np.linalg.norm(q[h])) <= 1e-13 * np.linalg.norm(q[h])


# --------------------------------------------------------------------------
# Number formats.
# --------------------------------------------------------------------------

def test_f16_matches_numpy_float16(orc):
    rng = _rng(9)
    vals = np.concatenate([
        rng.uniform(-1, 1, 2000) * np.exp2(rng.integers(-26, 16, 2000)),
        np.float32(np.arange(1, 200)) * np.float32(2.0 ** -25),      # subnormal range incl. midpoints
        np.float32(1.0) + np.float32(2.0 ** -11) * np.arange(-8, 9),  # ties around 1
        [0.0, -0.0, 65504.0, 6.1035156e-05, 5.9604645e-08, 2.9802322e-08],
    ]).astype(np.float32)
    for v in vals:
        ref = np.float16(v)
        if not np.isfinite(ref):
            continue
        assert orc.f16_bits(v) == int(ref.view(np.uint16)), v
        assert orc.f16_value(orc.f16_bits(v)) == float(ref)


def test_f16_saturates_instead_of_overflowing(orc):
    for v in (65504.0, 65519.0, 65520.0, 1e6, 3.4e38):
        assert orc.f16_bits(np.float32(v)) == 0x7BFF
        assert orc.f16_bits(np.float32(-v)) == 0xFBFF


def test_bf16_matches_torch(orc):
    import torch
    rng = _rng(10)
    vals = np.concatenate([
        rng.standard_normal(3000).astype(np.float32) * np.exp2(rng.integers(-130, 120, 3000)).astype(np.float32),
        (np.float32(1.0) + np.float32(2.0 ** -8) * np.arange(-20, 21)).astype(np.float32),  # exact ties
    ]).astype(np.float32)
    vals = vals[np.isfinite(vals)]
    ref = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([orc.bf16_bits(float(v)) for v in vals], np.uint16)
    assert np.array_equal(got, ref)


# --------------------------------------------------------------------------
# Quantiser and packing ([NOTES] 1.2; [RAQK] contributions: tokenwise range).
# --------------------------------------------------------------------------

def test_quantiser_worked_example(orc):
    g = json.load(open(os.path.join(GOLDEN, "quantiser_outlier_group.json")))
    q, sh, s32 = orc.quantize_group(np.array(g["group"]))
    assert orc.f16_value(sh) == g["expected_scale"] and s32 == g["expected_scale"]
    assert list(q) == g["expected_codes"]


def test_quantiser_is_nearest_level_brute_force(orc):
    rng = _rng(11)
    for trial in range(300):
        g = int(rng.choice([2, 8, 64, 128]))
        y = rng.standard_normal(g) * np.exp(rng.uniform(-12, 8))
        if trial % 7 == 0:
            y[rng.integers(g)] *= 50.0
        q, sh, s32 = orc.quantize_group(y)
        m = np.max(np.abs(y))
        assert s32 == np.float32(m / 7.0)
        s = orc.f16_value(sh)
        assert s == float(np.float16(np.float32(m / 7.0)))
        levels = np.arange(-7, 8)
        for yi, qi in zip(y, q):
            err = np.abs(yi - levels * s)
            best = levels[np.argmin(err)]
            tie = np.sort(err)[1] - np.sort(err)[0] < 1e-12 * max(1.0, abs(yi))
            if not tie:
                assert qi == best
            if abs(yi) <= 7 * s:
                assert abs(yi - qi * s) <= s / 2 * (1 + 1e-12)
        assert abs(q[np.argmax(np.abs(y))]) == 7


def test_quantiser_degenerate_groups(orc):
    q, sh, s32 = orc.quantize_group(np.zeros(8))
    assert sh == 0 and not q.any()
    q, sh, s32 = orc.quantize_group(np.full(8, 1e-9))       # scale underflows fp16
    assert sh == 0 and not q.any()
    q, sh, s32 = orc.quantize_group(np.array([1e7, -1e7, 1.0, 0.0]))  # scale saturates
    assert sh == 0x7BFF and list(q) == [7, -7, 0, 0]


def test_pack_roundtrip_with_numpy_unpack(orc):
    q = _rng(12).integers(-7, 8, 256).astype(np.int8)
    packed = orc.pack_nibbles(q)
    lo = (packed & 0xF).astype(np.int8)
    hi = (packed >> 4).astype(np.int8)
    lo = np.where(lo > 7, lo - 16, lo)
    hi = np.where(hi > 7, hi - 16, hi)
    unpacked = np.stack([lo, hi], 1).reshape(-1)
    assert np.array_equal(unpacked, q)


# --------------------------------------------------------------------------
# The rotate + quantise operation, end to end on small inputs.
# --------------------------------------------------------------------------

def _unpack(codes):
    lo = (codes & 0xF).astype(np.int8)
    hi = (codes >> 4).astype(np.int8)
    lo = np.where(lo > 7, lo - 16, lo)
    hi = np.where(hi > 7, hi - 16, hi)
    return np.stack([lo, hi], -1).reshape(*codes.shape[:-1], -1)


def test_rotate_quantize_consistent_with_building_blocks(orc):
    import torch
    rng = _rng(13)
    T, hq, hk, d, b, g = 5, 4, 2, 64, 16, 32
    shp = orc.shape(hq, hk, d, 5e5)
    qf = (rng.standard_normal((T, hq, d)) * 3).astype(np.float32)
    kf = (rng.standard_normal((T, hk, d)) * 3).astype(np.float32)
    q = torch.from_numpy(qf).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    k = torch.from_numpy(kf).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    pos = np.array([0, 5, 100, 4095, 131071], np.int32)
    phi = rng.uniform(-0.7, 0.7, d // 2).astype(np.float32)
    slots = np.array([9, 2, -1, 4, 12], np.int64)
    out = orc.rotate_quantize_qk(shp, q, k, pos, phi, b, g, slot_mapping=slots, n_slots=11)
    inv = orc.inv_freq(5e5, d)
    qv = torch.from_numpy(q.view(np.int16)).view(torch.bfloat16).double().numpy()
    kv = torch.from_numpy(k.view(np.int16)).view(torch.bfloat16).double().numpy()
    written = np.zeros(11, bool)
    for t in range(T):
        for h in range(hq):
            y = orc.transform_row(qv[t, h], 0, inv, pos[t], phi, b)
            assert np.array_equal(out["q_rot"][t, h], y)
            assert [orc.bf16_bits(v) for v in y] == list(out["q_out"][t, h])
        for h in range(hk):
            y = orc.transform_row(kv[t, h], 0, inv, pos[t], phi, b)
            assert np.array_equal(out["k_rot"][t, h], y)
            for j in range(d // g):
                qq, sh, s32 = orc.quantize_group(y[j * g:(j + 1) * g])
                assert out["k_scale32"][t, h, j] == s32
                if 0 <= slots[t] < 11:
                    assert out["k_scales"][slots[t], h, j] == sh
                    assert np.array_equal(_unpack(out["k_codes"][slots[t], h])[j * g:(j + 1) * g], qq)
        if 0 <= slots[t] < 11:
            written[slots[t]] = True
    # slots -1 and 12 are outside the cache: nothing written there, others untouched
    assert not out["k_codes"][~written].any() and not out["k_scales"][~written].any()


def test_identity_configuration_is_plain_group_quantisation(orc):
    """p = 0, no pair angles and b = 1: the transform is the identity and the
    codes are plain group-absmax INT4 of the input."""
    rng = _rng(14)
    T, hk, d, g = 3, 2, 32, 8
    k = (rng.standard_normal((T, hk, d)) * 2).astype(np.float32)
    out = orc.rotate_quantize_qk(orc.shape(0, hk, d, 1e4), None, k, np.zeros(T, np.int32), None, 1, g)
    assert np.array_equal(out["k_rot"], k.astype(np.float64))
    codes = _unpack(out["k_codes"])
    for t in range(T):
        for h in range(hk):
            for j in range(d // g):
                y = k[t, h, j * g:(j + 1) * g].astype(np.float64)
                s = float(np.float16(np.float32(np.max(np.abs(y)) / 7)))
                ref = np.clip(np.round(y / s), -7, 7)  # numpy rounds half to even
                assert np.array_equal(codes[t, h, j * g:(j + 1) * g], ref)


# --------------------------------------------------------------------------
# Calibration ([RAQK] optimisation objective, estimator strategies).
# --------------------------------------------------------------------------

def _post_rope_samples(orc, shp, x, pos):
    """Post-RoPE pairs (u, v) per pair k: array [P][n_samples][2]."""
    inv = orc.inv_freq(shp.rope_theta, shp.head_dim)
    d, P = shp.head_dim, shp.head_dim // 2
    rows = []
    for t in range(x.shape[0]):
        for h in range(x.shape[1]):
            r = orc.rope_row(x[t, h].astype(np.float64), shp.rope_layout, inv, pos[t])
            rows.append(r)
    rows = np.array(rows)
    out = []
    for k in range(P):
        lo, hi = (k, k + P) if shp.rope_layout == 0 else (2 * k, 2 * k + 1)
        out.append(rows[:, [lo, hi]])
    return np.array(out)


def _small_calib(seed, hq=4, hk=2, d=16, T=12, layout=0):
    rng = _rng(seed)
    shp = type("S", (), {})()
    sig = rng.lognormal(0, 0.8, d)
    q = (rng.standard_normal((T, hq, d)) * sig + rng.normal(0, 1, d)).astype(np.float32)
    k = (rng.standard_normal((T, hk, d)) * sig[::-1] + rng.normal(0, 1, d)).astype(np.float32)
    pos = rng.integers(0, 50, T).astype(np.int32)
    return q, k, pos


@pytest.mark.parametrize("layout", [0, 1])
def test_calibration_moments_match_numpy_cov(orc, layout):
    q, k, pos = _small_calib(15, layout=layout)
    shp = orc.shape(4, 2, 16, 1e4, layout)
    mom = orc.calibrate_moments(shp, q, k, pos)
    sq = _post_rope_samples(orc, shp, q, pos)
    sk = _post_rope_samples(orc, shp, k, pos)
    for est, samples in [(orc.EST_DEFAULT, np.concatenate([sq, sk], 1)), (orc.EST_K_ONLY, sk)]:
        _, _, abc = orc.angles_from_moments(mom, est)
        for kk in range(8):
            C = np.cov(samples[kk].T, bias=True)
            assert np.allclose(abc[kk], [C[0, 0], C[1, 1], C[0, 1]], rtol=1e-10, atol=1e-12)
    # stream-balanced: equal weight to the per-stream normalised raw moments
    _, _, abc = orc.angles_from_moments(mom, orc.EST_STREAM_BALANCED)
    for kk in range(8):
        Eq = [sq[kk][:, 0].mean(), sq[kk][:, 1].mean(), (sq[kk][:, 0] ** 2).mean(),
              (sq[kk][:, 1] ** 2).mean(), (sq[kk][:, 0] * sq[kk][:, 1]).mean()]
        Ek = [sk[kk][:, 0].mean(), sk[kk][:, 1].mean(), (sk[kk][:, 0] ** 2).mean(),
              (sk[kk][:, 1] ** 2).mean(), (sk[kk][:, 0] * sk[kk][:, 1]).mean()]
        E = 0.5 * (np.array(Eq) + np.array(Ek))
        ref = [E[2] - E[0] ** 2, E[3] - E[1] ** 2, E[4] - E[0] * E[1]]
        assert np.allclose(abc[kk], ref, rtol=1e-10, atol=1e-12)


def _rotated_vars(s, phi):
    u = s[:, 0] * math.cos(phi) - s[:, 1] * math.sin(phi)
    v = s[:, 0] * math.sin(phi) + s[:, 1] * math.cos(phi)
    return np.var(u), np.var(v)


@pytest.mark.parametrize("est", [0, 1, 2])
def test_angle_attains_analytic_minimum_and_beats_brute_force(orc, est):
    """At phi*, both rotated variances equal (a+b)/2, the smallest possible value
    of the larger one (trace invariance); a brute-force search over
    (-pi/4, pi/4] agrees with phi* (P1, P5)."""
    q, k, pos = _small_calib(16 + est)
    shp = orc.shape(4, 2, 16, 1e4)
    mom = orc.calibrate_moments(shp, q, k, pos)
    phi64, phi32, abc = orc.angles_from_moments(mom, est)
    sq = _post_rope_samples(orc, shp, q, pos)
    sk = _post_rope_samples(orc, shp, k, pos)
    for kk in range(8):
        a, b, c = abc[kk]
        if est == orc.EST_STREAM_BALANCED:
            # the surrogate is the equal-weight mixture of the two streams' covariances
            def vmax(phi):
                vq, vk = _rotated_vars(sq[kk], phi), _rotated_vars(sk[kk], phi)
                mq, mk = sq[kk].mean(0), sk[kk].mean(0)
                mu = 0.5 * (mq + mk)
                cs, sn = math.cos(phi), math.sin(phi)
                R = np.array([[cs, -sn], [sn, cs]])
                out = []
                for i in range(2):
                    e2 = 0.5 * ((vq[i] + (R @ mq)[i] ** 2) + (vk[i] + (R @ mk)[i] ** 2))
                    out.append(e2 - (R @ mu)[i] ** 2)
                return out
        else:
            s = np.concatenate([sq[kk], sk[kk]]) if est == orc.EST_DEFAULT else sk[kk]

            def vmax(phi, s=s):
                return list(_rotated_vars(s, phi))
        v1, v2 = vmax(phi64[kk])
        assert abs(v1 - (a + b) / 2) <= 1e-10 * (a + b) and abs(v2 - (a + b) / 2) <= 1e-10 * (a + b)
        grid = np.linspace(-math.pi / 4, math.pi / 4, 20001)[1:]
        f = np.array([max(vmax(p)) for p in grid])
        i = int(np.argmin(f))
        lo, hi = grid[max(i - 1, 0)], grid[min(i + 1, len(grid) - 1)]
        gr = (math.sqrt(5) - 1) / 2
        for _ in range(80):  # golden-section refine of the V-shaped maximum
            m1, m2 = hi - gr * (hi - lo), lo + gr * (hi - lo)
            if max(vmax(m1)) < max(vmax(m2)):
                hi = m2
            else:
                lo = m1
        best = 0.5 * (lo + hi)
        r = math.hypot(a - b, 2 * c)
        if r > 1e-6 * (a + b):
            d_ang = abs(best - phi64[kk])
            d_ang = min(d_ang, abs(d_ang - math.pi / 2))
            assert d_ang < 1e-6, (kk, best, phi64[kk])
        assert max(vmax(phi64[kk])) <= f.min() + 1e-12 * (a + b)


def test_angle_closed_form_special_cases(orc):
    def mom_from_cov(a, b, c, n=10.0):
        m = np.zeros((1, 2, 6))
        m[0, 1] = [n, 0, 0, a * n, b * n, c * n]
        return m
    cases = [((2.0, 1.0, 0.0), math.pi / 4),      # tan 2phi = inf -> pi/4 (boundary kept)
             ((1.0, 2.0, 0.0), math.pi / 4),      # 2phi = -pi/2 -> wrapped to +pi/4
             ((1.0, 1.0, 0.5), 0.0),              # a == b, c > 0
             ((1.0, 1.0, -0.5), 0.0),             # a == b, c < 0: 2phi = pi -> wrapped to 0
             ((1.0, 1.0, 0.0), 0.0)]              # isotropic: degenerate
    for (a, b, c), want in cases:
        phi, _, _ = orc.angles_from_moments(mom_from_cov(a, b, c), orc.EST_K_ONLY)
        assert abs(phi[0] - want) < 1e-15, (a, b, c, phi[0])
    phi, _, _ = orc.angles_from_moments(np.zeros((3, 2, 6)), orc.EST_DEFAULT)
    assert not phi.any()
    # general position: phi* = atan2(a-b, 2c)/2 equalises the variances
    rng = _rng(17)
    for _ in range(200):
        L = rng.standard_normal((2, 2))
        C = L @ L.T
        a, b, c = C[0, 0], C[1, 1], C[0, 1]
        phi, _, _ = orc.angles_from_moments(mom_from_cov(a, b, c), orc.EST_K_ONLY)
        p = phi[0]
        assert -math.pi / 4 < p <= math.pi / 4
        cs, sn = math.cos(p), math.sin(p)
        R = np.array([[cs, -sn], [sn, cs]])
        V = R @ C @ R.T
        assert abs(V[0, 0] - V[1, 1]) < 1e-12 * np.trace(C)


def test_estimator_identities(orc):
    """H_q == H_kv: default (count-pooled) == stream-balanced; identical Q and K
    streams: all three estimators agree; K-only ignores Q (P10)."""
    q, k, pos = _small_calib(18, hq=2, hk=2)
    shp = orc.shape(2, 2, 16, 1e4)
    mom = orc.calibrate_moments(shp, q, k, pos)
    d_, _, _ = orc.angles_from_moments(mom, orc.EST_DEFAULT)
    sb, _, _ = orc.angles_from_moments(mom, orc.EST_STREAM_BALANCED)
    # equal counts make the pooled mean the average of the stream means
    assert np.allclose(d_, sb, atol=1e-12)
    mom2 = orc.calibrate_moments(shp, k, k, pos)
    e = [orc.angles_from_moments(mom2, est)[0] for est in (0, 1, 2)]
    assert np.allclose(e[0], e[1], atol=1e-13) and np.allclose(e[1], e[2], atol=1e-13)
    q2 = q * 3.0 + 1.0
    mom3 = orc.calibrate_moments(shp, q2, k, pos)
    assert np.array_equal(orc.angles_from_moments(mom3, 1)[0], orc.angles_from_moments(mom, 1)[0])


def test_calibration_accumulates_across_batches(orc):
    q, k, pos = _small_calib(19)
    shp = orc.shape(4, 2, 16, 1e4)
    whole = orc.calibrate_moments(shp, q, k, pos)
    part = orc.calibrate_moments(shp, q[:5], k[:5], pos[:5])
    part = orc.calibrate_moments(shp, q[5:], k[5:], pos[5:], moments=part)
    assert np.allclose(whole, part, rtol=1e-13)
    assert whole[0, 0, 0] == 12 * 4 and whole[0, 1, 0] == 12 * 2


# --------------------------------------------------------------------------
# Diagnostics ([RAQK] contributions/results: K range and relative error vs b).
# --------------------------------------------------------------------------

def test_quant_error_stats_against_rotate_outputs(orc):
    rng = _rng(20)
    T, hk, d, g = 6, 3, 64, 16
    k = (rng.standard_normal((T, hk, d)) * rng.lognormal(0, 1, d)).astype(np.float32)
    pos = rng.integers(0, 4096, T).astype(np.int32)
    phi = rng.uniform(-0.5, 0.5, d // 2).astype(np.float32)
    shp = orc.shape(0, hk, d, 5e5)
    for b in (1, 4, 64):
        st = orc.quant_error_stats(shp, k, pos, phi, b, g)
        out = orc.rotate_quantize_qk(shp, None, k, pos, phi, b, g)
        y = out["k_rot"].reshape(T, hk, d // g, g)
        s = np.vectorize(orc.f16_value)(out["k_scales"]).reshape(T, hk, d // g, 1)
        yhat = _unpack(out["k_codes"]).reshape(T, hk, d // g, g) * s
        assert np.isclose(st[0], ((yhat - y) ** 2).sum(), rtol=1e-12)
        # N is the energy of the raw input: the transform is orthogonal
        assert np.isclose(st[1], (k.astype(np.float64) ** 2).sum(), rtol=1e-12)
        assert np.isclose(st[2], np.abs(y).max(-1).sum(), rtol=1e-12)
        assert st[3] == np.abs(y).max()
        assert np.isclose(st[4], (y.max(-1) - y.min(-1)).sum(), rtol=1e-12)
        assert st[5] == T * hk * (d // g) and st[6] == T * hk and st[7] == 0


def test_k_range_of_one_hot_rows_scales_as_inverse_sqrt_b(orc):
    d, hk, T = 64, 1, 4
    k = np.zeros((T, hk, d), np.float32)
    for t in range(T):
        k[t, 0, 5 + 11 * t] = 8.0
    shp = orc.shape(0, hk, d, 5e5)
    for b in (1, 2, 8, 64):
        st = orc.quant_error_stats(shp, k, np.zeros(T, np.int32), None, b, d)
        assert np.isclose(st[3], 8.0 / math.sqrt(b), rtol=1e-14)
        assert np.isclose(st[2] / st[5], 8.0 / math.sqrt(b), rtol=1e-14)


def test_quantiser_rounds_exact_ties_to_even(orc):
    """Reading taken where the pages say only 'round to nearest': exact ties go to
    the even integer (IEEE default).  Ties are exact here because s = 7/7 = 1."""
    y = np.array([7.0, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 3.5])
    q, sh, _ = orc.quantize_group(y)
    assert orc.f16_value(sh) == 1.0
    assert list(q) == [7, 0, 2, 2, 0, -2, -2, 4]


@pytest.mark.parametrize("layout,b", [(0, 2), (0, 64), (1, 8), (1, 1)])
def test_transform_matches_complex_rotation_then_scipy_hadamard(orc, layout, b):
    """The full row transform, rebuilt independently: each pair as a complex number
    turned by alpha_k + phi_k (RoPE and the pair rotation are both plane rotations
    of the pair), then the Sylvester matrix of scipy applied block-wise (the
    composition order reading: Hadamard after the pair rotation)."""
    import scipy.linalg
    d = 64
    rng = _rng(30 + b)
    x = rng.standard_normal(d)
    phi = rng.uniform(-0.78, 0.78, d // 2).astype(np.float32)
    inv = orc.inv_freq(5e5, d)
    p = 77777
    r = np.empty(d)
    for k in range(d // 2):
        lo, hi = (k, k + d // 2) if layout == 0 else (2 * k, 2 * k + 1)
        z = complex(x[lo], x[hi]) * np.exp(1j * (float(orc.rope_angle(p, inv[k])) + float(phi[k])))
        r[lo], r[hi] = z.real, z.imag
    H = scipy.linalg.hadamard(b).astype(np.float64) / math.sqrt(b)
    ref = (r.reshape(-1, b) @ H.T).reshape(-1)
    assert np.allclose(orc.transform_row(x, layout, inv, p, phi, b), ref, rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# V side of the KV4 cache ([NOTES] section 3.2.2: V times the head-wise
# Hadamard online; the Hadamard left on the attention output folds into W_O).
# --------------------------------------------------------------------------

@pytest.mark.parametrize("d,g", [(64, 64), (128, 128), (128, 8), (64, 2)])
def test_v_transform_is_scipy_hadamard_and_codes_bound_the_error(orc, d, g):
    from scipy.linalg import hadamard
    rng = _rng(40 + d + g)
    T, hk = 5, 3
    v = (rng.standard_normal((T, hk, d)) * rng.lognormal(0, 1, d)).astype(np.float32)
    v[1, 2, 7] = 300.0                                   # an outlier channel
    out = orc.quantize_v(orc.shape(4, hk, d, 5e5), v, g)
    H = hadamard(d).astype(np.float64) / math.sqrt(d)
    ref = v.astype(np.float64) @ H.T
    assert np.max(np.abs(out["v_rot"] - ref)) <= 1e-12 * np.max(np.abs(ref))
    codes = _unpack(out["v_codes"]).astype(np.float64)
    s = out["v_scales"].view(np.float16).astype(np.float64)
    yhat = codes * np.repeat(s, g, axis=-1)
    y = out["v_rot"]
    assert np.all(np.abs(yhat - y) <= np.repeat(s, g, axis=-1) / 2 * (1 + 1e-9))
    grp = np.abs(codes.reshape(T, hk, d // g, g)).max(-1)
    assert np.all(grp == 7)                               # every group's absmax maps to +-7
    assert np.array_equal(out["v_scale32"], (np.abs(y.reshape(T, hk, d // g, g)).max(-1) / 7).astype(np.float32))


def test_v_rotation_folds_into_the_output_projection(orc):
    """A . V~ . H^T / sqrt(d) = A . V for attention weights A: the transform on V is
    undone by the Hadamard that the output projection absorbs."""
    from scipy.linalg import hadamard
    rng = _rng(50)
    T, hk, d = 24, 1, 64
    v = rng.standard_normal((T, hk, d)).astype(np.float32)
    out = orc.quantize_v(orc.shape(1, hk, d, 5e5), v, d)
    logits = rng.standard_normal((7, T))
    A = np.exp(logits) / np.exp(logits).sum(1, keepdims=True)
    H = hadamard(d).astype(np.float64) / math.sqrt(d)
    back = (A @ out["v_rot"][:, 0, :]) @ H
    assert np.max(np.abs(back - A @ v[:, 0, :].astype(np.float64))) < 1e-12


def test_v_one_hot_row_spreads_evenly(orc):
    d = 128
    v = np.zeros((1, 1, d), np.float32)
    v[0, 0, 37] = 8.0
    out = orc.quantize_v(orc.shape(1, 1, d, 5e5), v, 32)
    assert np.allclose(np.abs(out["v_rot"]), 8.0 / math.sqrt(d), rtol=0, atol=1e-15)
    assert np.all(np.abs(_unpack(out["v_codes"])) == 7)


def test_v_equals_k_path_at_position_zero_without_pair_angles(orc):
    """At p = 0 with no pair rotation and b = d the K transform reduces to H_d / sqrt(d):
    the V and K caches must then hold the same codes and scales."""
    rng = _rng(51)
    T, hk, d, g = 6, 2, 64, 16
    x = (rng.standard_normal((T, hk, d)) * 3).astype(np.float32)
    shp = orc.shape(0, hk, d, 5e5)
    kv = orc.rotate_quantize_qk(shp, None, x, np.zeros(T, np.int32), None, d, g)
    vv = orc.quantize_v(shp, x, g)
    assert np.array_equal(kv["k_codes"], vv["v_codes"]) and np.array_equal(kv["k_scales"], vv["v_scales"])
    assert np.max(np.abs(kv["k_rot"] - vv["v_rot"])) < 1e-13


def test_v_slot_mapping_and_padding(orc):
    rng = _rng(52)
    T, hk, d, g = 4, 2, 64, 64
    v = rng.standard_normal((T, hk, d)).astype(np.float32)
    slots = np.array([5, -1, 0, 9], np.int64)
    out = orc.quantize_v(orc.shape(2, hk, d, 5e5), v, g, slot_mapping=slots, n_slots=8)
    ident = orc.quantize_v(orc.shape(2, hk, d, 5e5), v, g)
    assert np.array_equal(out["v_codes"][5], ident["v_codes"][0])
    assert np.array_equal(out["v_codes"][0], ident["v_codes"][2])
    written = {0, 5}
    for sl in range(8):
        if sl not in written:
            assert not out["v_codes"][sl].any() and not out["v_scales"][sl].any()


# --------------------------------------------------------------------------
# Decode logits from the KV4 cache ([NOTES] section 3.2.1: the rotation cancels
# inside Q K^T; [QIFT] introduction: decode reads the KV cache).
# --------------------------------------------------------------------------

def _random_cache(rng, n_slots, hk, d, g):
    codes = rng.integers(0, 256, (n_slots, hk, d // 2), dtype=np.uint8)
    scales = np.exp2(rng.uniform(-8, 3, (n_slots, hk, d // g))).astype(np.float16).view(np.uint16)
    return codes, scales


@pytest.mark.parametrize("hq,hk,d,g", [(4, 2, 64, 64), (8, 2, 128, 16), (3, 3, 64, 2), (32, 8, 128, 128)])
def test_decode_scores_equal_numpy_dequant_matmul(orc, hq, hk, d, g):
    rng = _rng(60 + hq + g)
    n_slots, B, max_len = 300, 5, 70
    codes, scales = _random_cache(rng, n_slots, hk, d, g)
    q = rng.standard_normal((B, hq, d)).astype(np.float32)
    start = np.array([0, 50, 120, 230, 299], np.int64)
    lens = np.array([70, 1, 69, 70, 3], np.int32)          # the last runs past the cache: NaN
    out = orc.decode_scores(orc.shape(hq, hk, d, 5e5), q, codes, scales, g, start, lens, max_len)
    kdeq = _unpack(codes).astype(np.float64) * np.repeat(scales.view(np.float16).astype(np.float64), g, axis=-1)
    for b in range(B):
        for h in range(hq):
            kv = h * hk // hq                               # grouped-query head sharing
            for j in range(max_len):
                if j >= lens[b]:
                    assert out[b, h, j] == -np.inf          # not written
                    continue
                slot = start[b] + j
                if slot >= n_slots:
                    assert np.isnan(out[b, h, j])
                    continue
                ref = float(np.dot(q[b, h].astype(np.float64), kdeq[slot, kv]))
                tol = 1e-13 * float(np.dot(np.abs(q[b, h]), np.abs(kdeq[slot, kv])))
                assert abs(out[b, h, j] - ref) <= tol, (b, h, j)


def test_decode_scores_bf16_queries_read_as_bf16(orc):
    import torch
    rng = _rng(61)
    codes, scales = _random_cache(rng, 10, 1, 64, 64)
    qf = rng.standard_normal((1, 1, 64)).astype(np.float32)
    qb = torch.from_numpy(qf).to(torch.bfloat16)
    qbits = qb.view(torch.int16).numpy().view(np.uint16)
    a = orc.decode_scores(orc.shape(1, 1, 64, 5e5), qbits, codes, scales, 64, np.zeros(1, np.int64),
                          np.array([10], np.int32), 10)
    b = orc.decode_scores(orc.shape(1, 1, 64, 5e5), qb.float().numpy(), codes, scales, 64, np.zeros(1, np.int64),
                          np.array([10], np.int32), 10)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("b,g", [(128, 128), (2, 64), (128, 8)])
def test_decode_scores_approximate_exact_rope_logits(orc, b, g):
    """Cache written by the rotate path: the logit of the rotated query against
    the quantised rotated key is the plain RoPE logit (the rotation cancels) up
    to the quantisation error, |err| <= sum_c |q_c| s_h(c) / 2 (+ fp32 rounding of q)."""
    rng = _rng(62 + b + g)
    hq, hk, d, T = 4, 2, 128, 40
    shp = orc.shape(hq, hk, d, 1e6)
    q_new = (rng.standard_normal((1, hq, d)) * rng.lognormal(0, 1, d)).astype(np.float32)
    k = (rng.standard_normal((T, hk, d)) * rng.lognormal(0, 1, d)).astype(np.float32)
    ang = rng.uniform(-math.pi / 4, math.pi / 4, d // 2).astype(np.float32)
    pos = np.arange(T, dtype=np.int32)
    cache = orc.rotate_quantize_qk(orc.shape(0, hk, d, 1e6), None, k, pos, ang, b, g)
    qr = orc.rotate_quantize_qk(shp, q_new, np.zeros((1, hk, d), np.float32), np.array([T - 1], np.int32), ang, b, g)
    q_rot = qr["q_rot"].astype(np.float32)
    sc = orc.decode_scores(shp, q_rot, cache["k_codes"], cache["k_scales"], g, np.zeros(1, np.int64),
                           np.array([T], np.int32), T)
    inv = orc.inv_freq(1e6, d)
    s_h = cache["k_scales"].view(np.float16).astype(np.float64)
    for h in range(hq):
        kv = h * hk // hq
        qe = orc.rope_row(q_new[0, h].astype(np.float64), 0, inv, T - 1)
        for j in range(T):
            ke = orc.rope_row(k[j, kv].astype(np.float64), 0, inv, j)
            exact = float(np.dot(qe, ke))
            bound = float(np.sum(np.abs(q_rot[0, h]) * np.repeat(s_h[j, kv], g) / 2))
            bound += 2.0 ** -23 * float(np.dot(np.abs(qe), np.abs(ke))) * 8
            assert abs(sc[0, h, j] - exact) <= bound, (h, j, sc[0, h, j], exact, bound)


# --------------------------------------------------------------------------
# Per-head (non-shared) angles: one set per key head, query heads using their
# key head's set ([RAQK] optimisation objective: the head-shared set is the
# parameterisation the paper evaluates; this is the per-head one).
# --------------------------------------------------------------------------

def _ph_layer(seed, hq=8, hk=2, d=32, T=6):
    rng = _rng(seed)
    q = (rng.standard_normal((T, hq, d)) * rng.lognormal(0, 0.8, d)).astype(np.float32)
    k = (rng.standard_normal((T, hk, d)) * rng.lognormal(0, 0.8, d)).astype(np.float32)
    pos = rng.integers(0, 300, T).astype(np.int32)
    ang = rng.uniform(-math.pi / 4, math.pi / 4, (hk, d // 2)).astype(np.float32)
    return q, k, pos, ang


@pytest.mark.parametrize("b", [1, 4, 32])
def test_per_head_angles_keep_each_query_heads_logits(orc, b):
    """Query head h against its own key head keeps the RoPE inner product; against
    a key head of another group it does not (the sets differ)."""
    hq, hk, d = 8, 2, 32
    q, k, pos, ang = _ph_layer(70 + b, hq, hk, d)
    shp = orc.shape(hq, hk, d, 1e4, angle_heads=hk)
    out = orc.rotate_quantize_qk(shp, q, k, pos, ang, b, d)
    inv = orc.inv_freq(1e4, d)
    for t in range(len(pos)):
        for h in range(hq):
            qe = orc.rope_row(q[t, h].astype(np.float64), 0, inv, pos[t])
            for kh in range(hk):
                ke = orc.rope_row(k[t, kh].astype(np.float64), 0, inv, pos[t])
                got = float(np.dot(out["q_rot"][t, h], out["k_rot"][t, kh]))
                ref = float(np.dot(qe, ke))
                same = kh == h * hk // hq
                close = abs(got - ref) <= 1e-10 * float(np.linalg.norm(qe) * np.linalg.norm(ke))
                assert close == same, (t, h, kh, got, ref)


def test_per_head_with_identical_sets_is_the_shared_path(orc):
    hq, hk, d = 8, 4, 32
    q, k, pos, ang = _ph_layer(71, hq, hk, d)
    shared = ang[0]
    a = orc.rotate_quantize_qk(orc.shape(hq, hk, d, 1e4), q, k, pos, shared, 8, 16)
    b = orc.rotate_quantize_qk(orc.shape(hq, hk, d, 1e4, angle_heads=hk), q, k, pos, np.tile(shared, (hk, 1)), 8, 16)
    for key in ("q_rot", "k_rot", "k_codes", "k_scales"):
        assert np.array_equal(a[key], b[key]), key


def test_per_head_moments_are_each_groups_shared_moments(orc):
    """Group g's moments are the shared moments of the layer made of group g's
    query heads and key head g alone."""
    hq, hk, d = 8, 2, 32
    q, k, pos, _ = _ph_layer(72, hq, hk, d)
    mom = orc.calibrate_moments(orc.shape(hq, hk, d, 1e4, angle_heads=hk), q, k, pos)
    assert mom.shape == (hk, d // 2, 2, 6)
    G = hq // hk
    for g in range(hk):
        sub = orc.calibrate_moments(orc.shape(G, 1, d, 1e4), q[:, g * G:(g + 1) * G], k[:, g:g + 1], pos)
        assert np.array_equal(mom[g], sub)


@pytest.mark.parametrize("est", [0, 1, 2])
def test_per_head_angle_attains_each_groups_minimum(orc, est):
    hq, hk, d = 8, 2, 16
    q, k, pos, _ = _ph_layer(73 + est, hq, hk, d, T=40)
    shp = orc.shape(hq, hk, d, 1e4, angle_heads=hk)
    mom = orc.calibrate_moments(shp, q, k, pos)
    phi64, _, abc = orc.angles_from_moments(mom, est)
    assert phi64.shape == (hk, d // 2)
    for g in range(hk):
        a, b_, c = abc[g, :, 0], abc[g, :, 1], abc[g, :, 2]
        ph = phi64[g]
        va = (a + b_) / 2 + (a - b_) / 2 * np.cos(2 * ph) - c * np.sin(2 * ph)
        vb = (a + b_) / 2 - (a - b_) / 2 * np.cos(2 * ph) + c * np.sin(2 * ph)
        assert np.allclose(va, (a + b_) / 2, rtol=1e-12, atol=1e-12 * np.abs(a + b_).max())
        assert np.allclose(vb, (a + b_) / 2, rtol=1e-12, atol=1e-12 * np.abs(a + b_).max())
    # groups differ: the per-head sets are not all equal
    assert not np.allclose(phi64[0], phi64[1])


def test_per_head_stats_are_the_sum_of_each_groups_stats(orc):
    hq, hk, d, g = 8, 2, 32, 16
    q, k, pos, ang = _ph_layer(76, hq, hk, d, T=12)
    st = orc.quant_error_stats(orc.shape(hq, hk, d, 1e4, angle_heads=hk), k, pos, ang, 8, g)
    parts = [orc.quant_error_stats(orc.shape(1, 1, d, 1e4), np.ascontiguousarray(k[:, kh:kh + 1]), pos, ang[kh], 8, g)
             for kh in range(hk)]
    tot = np.sum(parts, axis=0)
    for i in (0, 1, 2, 4, 5, 6):
        assert abs(st[i] - tot[i]) <= 1e-12 * abs(tot[i])
    assert st[3] == max(p[3] for p in parts)
