"""GPU parity at sizes past the 32-bit offset limits, through the C-ABI.

A batch of 1 050 000 Llama-3.1-8B-shaped tokens (32 Q / 8 KV heads, d 128,
bf16) puts the query rows past 2^33 bytes and the key rows past 2^31 bytes.
To keep the oracle's work small, the batch is one 3000-token block of the
128K-prefill recipe (positions included), tiled 350 times on the device.
- Rotate outputs are compared element by element on sampled tokens. The
  sample includes the tokens on either side of every power-of-two byte offset
  the rows cross.
- Calibration moments and diagnostic sums are the oracle's block values times
  350, and maxima and angles equal the block's.

3000 does not divide 2^31 / 2048, 2^32 / 8192 or 2^33 / 8192.  A row read
through a wrapped 32-bit offset would therefore land on another token of the
block, and the comparison would see it.

The decode entry point is run with more sequences than one grid holds
(65535 along z), in both its grid forms, with sequences on both sides of
each launch boundary compared with the oracle.
"""
import math

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
BLOCK, REPS = 3000, 350
T_BIG = BLOCK * REPS
STAT_TOL = np.array([1e-9, 1e-11, 1e-11, 1e-13, 1e-11])


class Tiled:
    """Host view of the tiled batch: row t is row t mod BLOCK of the block."""

    def __init__(self, a):
        self.a = a

    def __getitem__(self, idx):
        return self.a[np.asarray(idx) % len(self.a)]


def dev_bits(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV)


@pytest.fixture(scope="module")
def big():
    w = W.WORKLOADS[4]
    blk = W.make_inputs(4, n_tokens=BLOCK)
    q = dev_bits(blk["q"]).repeat(REPS, 1, 1).view(torch.bfloat16)
    k = dev_bits(blk["k"]).repeat(REPS, 1, 1).view(torch.bfloat16)
    pos = torch.from_numpy(blk["pos"]).to(DEV).repeat(REPS)
    assert q.shape[0] == T_BIG and q.numel() * 2 > 2**33 and k.numel() * 2 > 2**31
    yield w, blk, q, k, pos
    del q, k, pos
    torch.cuda.empty_cache()


def angles_for(w, ah, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    n = max(ah, 1)
    a = rng.uniform(-math.pi / 4, math.pi / 4, (n, w.n_pairs)).astype(np.float32)
    return a[0] if ah == 0 else a


def sample_big(seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    edges = []
    for t_edge in (2**31 // 8192, 2**32 // 8192, 2**33 // 8192, 2**31 // 2048):
        edges += list(range(t_edge - 3, t_edge + 3))
    idx = np.concatenate([np.arange(64), np.arange(T_BIG - 64, T_BIG), np.array(edges),
                          rng.choice(T_BIG, 1500, replace=False)])
    return np.unique(idx[(idx >= 0) & (idx < T_BIG)])


@pytest.mark.parametrize("ah", [0, 8])
def test_rotate_past_32bit_offsets(big, ah):
    w, blk, q, k, pos = big
    d, hq, hk, g = w.head_dim, w.n_q_heads, w.n_kv_heads, 128
    ang = angles_for(w, ah, 1200 + ah)
    codes, scales = rrp.new_kv4_cache(T_BIG, hk, d, g, DEV)
    q_out = torch.empty_like(q)
    shp = rrp.layer_shape(hq, hk, d, w.rope_theta, angle_heads=ah)
    rrp.rotate_quantize_qk(shp, q, k, pos, support_b=128, group=g, k_codes=codes, k_scales=scales,
                           angles=torch.from_numpy(ang).to(DEV), q_out=q_out)
    torch.cuda.synchronize()
    idx = sample_big(1210 + ah)
    ref = O.rotate_quantize_qk(O.shape(hq, hk, d, w.rope_theta, angle_heads=ah), Tiled(blk["q"])[idx],
                               Tiled(blk["k"])[idx], Tiled(blk["pos"])[idx], ang, 128, g)
    it = torch.from_numpy(idx.astype(np.int64)).to(DEV)
    qo = q_out.index_select(0, it).view(torch.int16).cpu().numpy().view(np.uint16)
    C.check_q_out(qo, ref["q_rot"], "bf16")
    got_codes = codes.index_select(0, it).cpu().numpy().reshape(-1, d // 2)
    got_scales = scales.index_select(0, it).view(torch.int16).cpu().numpy().view(np.uint16).reshape(-1, d // g)
    rep = C.compare_k(got_codes, got_scales, ref["k_rot"].reshape(-1, d), ref["k_scales"].reshape(-1, d // g),
                      ref["k_codes"].reshape(-1, d // 2), g)
    print(f"{len(idx)} tokens up to {int(idx[-1])}: {rep}")


@pytest.mark.parametrize("ah,est", [(0, "default"), (8, "default"), (0, "k_only")])
def test_calibration_past_32bit_offsets(big, ah, est):
    w, blk, q, k, pos = big
    d = w.head_dim
    A = max(ah, 1)
    mom = rrp.new_moments(d, DEV, n_sets=A)
    ang = torch.empty((d // 2,) if A == 1 else (A, d // 2), dtype=torch.float32, device=DEV)
    rrp.calibrate_angles(rrp.layer_shape(w.n_q_heads, w.n_kv_heads, d, w.rope_theta, angle_heads=ah),
                         q if est != "k_only" else None, k, pos, moments=mom, estimator=est, angles_out=ang)
    torch.cuda.synchronize()
    oshp = O.shape(w.n_q_heads, w.n_kv_heads, d, w.rope_theta, angle_heads=ah)
    mom_r = O.calibrate_moments(oshp, blk["q"] if est != "k_only" else None, blk["k"], blk["pos"]) * REPS
    worst = C.compare_moments(mom.cpu().numpy(), mom_r)
    e = {"default": O.EST_DEFAULT, "k_only": O.EST_K_ONLY}[est]
    phi64, _, abc = O.angles_from_moments(mom_r, e)
    rep = C.compare_angles(ang.cpu().numpy().reshape(-1), phi64.reshape(-1), abc.reshape(-1, 3))
    print(f"moments {worst:.2e} {rep}")


def scaled_block_stats(r):
    """Statistics of REPS copies of the block: sums and counts scale, the maximum does not."""
    out = np.array(r, dtype=np.float64) * REPS
    out[..., 3] = r[..., 3]
    out[..., 7] = 0.0
    return out


def check_stats(g, r, last=0.0):
    """Sums within STAT_TOL, counts exact; field 7 is 0 (one support) or the row's b (sweep)."""
    rel = np.abs(g[..., :5] - r[..., :5]) / np.maximum(np.abs(r[..., :5]), 1e-300)
    assert np.all(rel <= STAT_TOL), (g, r, rel)
    assert np.array_equal(g[..., 5:7], r[..., 5:7]) and np.all(g[..., 7] == last)


@pytest.mark.parametrize("ah", [0, 8])
def test_diagnostics_past_32bit_offsets(big, ah):
    w, blk, q, k, pos = big
    d, g = w.head_dim, 128
    ang = angles_for(w, ah, 1220 + ah)
    shp = rrp.layer_shape(w.n_q_heads, w.n_kv_heads, d, w.rope_theta, angle_heads=ah)
    oshp = O.shape(w.n_q_heads, w.n_kv_heads, d, w.rope_theta, angle_heads=ah)
    st = torch.empty(8, dtype=torch.float64, device=DEV)
    rrp.quant_error_stats(shp, k, pos, support_b=128, group=g, stats_out=st, angles=torch.from_numpy(ang).to(DEV))
    torch.cuda.synchronize()
    check_stats(st.cpu().numpy(), scaled_block_stats(O.quant_error_stats(oshp, blk["k"], blk["pos"], ang, 128, g)))
    sups = rrp.sweep_supports(d)
    sw = torch.empty((len(sups), 8), dtype=torch.float64, device=DEV)
    rrp.quant_error_sweep(shp, k, pos, group=g, stats_out=sw, angles=torch.from_numpy(ang).to(DEV))
    torch.cuda.synchronize()
    ref = np.stack([O.quant_error_stats(oshp, blk["k"], blk["pos"], ang, b, g) for b in sups])
    check_stats(sw.cpu().numpy(), scaled_block_stats(ref), last=np.array(sups, dtype=np.float64))


# ---------------------------------------------------------------------------
# decode: more sequences than one grid holds
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("hq,hk", [(8, 4), (4, 2)])
def test_decode_more_sequences_than_one_grid(hq, hk):
    """70 000 sequences, so the batch goes out as two launches of 65535 and 4465
    sequences.  With 4 key heads the launches use the 3-D grid, with 2 the 1-D
    one.  The sequences share a small oracle-written cache: starts are drawn
    at random, a few run past its end (NaN logits), and some are empty."""
    d, g, B, max_len, n_slots = 64, 32, 70000, 40, 4096
    rng = np.random.Generator(np.random.PCG64(1300 + hk))
    k = (rng.standard_normal((n_slots, hk, d)) * rng.lognormal(0, 1, d)).astype(np.float32)
    k = W._to_storage(k, "bf16")
    ang = rng.uniform(-math.pi / 4, math.pi / 4, d // 2).astype(np.float32)
    cache = O.rotate_quantize_qk(O.shape(0, hk, d, 1e6), None, k, (np.arange(n_slots) % 997).astype(np.int32),
                                 ang, d, g)
    q = W._to_storage((rng.standard_normal((B, hq, d)) * rng.lognormal(0, 1, d)).astype(np.float32), "bf16")
    lens = rng.integers(0, max_len + 8, B).astype(np.int32)          # some above max_len: cut to it
    start = rng.integers(0, n_slots - max_len, B).astype(np.int64)
    start[rng.choice(B, 50, replace=False)] = n_slots - 10            # these run past the cache
    shp = rrp.layer_shape(hq, hk, d, 1e6)
    out = torch.full((B, hq, max_len), float("-inf"), dtype=torch.float32, device=DEV)
    rrp.decode_scores(shp, dev_bits(q).view(torch.bfloat16), torch.from_numpy(cache["k_codes"]).to(DEV),
                      dev_bits(cache["k_scales"]), group=g, seq_start=torch.from_numpy(start).to(DEV),
                      seq_len=torch.from_numpy(lens).to(DEV), max_len=max_len, scores=out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    n_written = int(np.minimum(lens, max_len).sum()) * hq
    assert int((~np.isneginf(got)).sum()) == n_written
    seqs = np.unique(np.concatenate([np.arange(8), np.arange(65530, 65541), np.arange(B - 8, B),
                                     np.flatnonzero(start == n_slots - 10)[:4], rng.choice(B, 200, replace=False)]))
    ref = O.decode_scores(O.shape(hq, hk, d, 1e6), q[seqs], cache["k_codes"], cache["k_scales"], g, start[seqs],
                          lens[seqs], max_len, n_slots=n_slots)
    qv = (q[seqs].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    worst = 0.0
    for i, b in enumerate(seqs):
        n = min(int(lens[b]), max_len)
        assert np.all(np.isneginf(got[b, :, n:]))
        sl = start[b] + np.arange(n)
        inside = sl < n_slots
        codes = cache["k_codes"][np.where(inside, sl, 0)]
        lo = (codes & 0xF).astype(np.int8)
        hi = (codes >> 4).astype(np.int8)
        cv = np.stack([np.where(lo > 7, lo - 16, lo), np.where(hi > 7, hi - 16, hi)], -1).reshape(n, hk, d)
        sc = np.repeat(cache["k_scales"][np.where(inside, sl, 0)].view(np.float16).astype(np.float64), g, axis=-1)
        mag = np.abs(cv * sc)
        for h in range(hq):
            r_ = ref[i, h, :n]
            g_ = got[b, h, :n].astype(np.float64)
            assert np.array_equal(np.isnan(g_), ~inside) and np.array_equal(np.isnan(r_), ~inside), (b, h)
            lim = 1e-5 * np.maximum(mag[:, h * hk // hq] @ np.abs(qv[i, h]), 1e-300)
            err = np.abs(g_ - r_)[inside]
            assert np.all(err <= lim[inside]), (b, h)
            if err.size:
                worst = max(worst, float((err / lim[inside]).max()))
    print(f"{len(seqs)} sequences compared, worst |err| / tolerance = {worst:.3f}")
