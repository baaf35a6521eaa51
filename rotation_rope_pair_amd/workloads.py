"""Seeded synthetic Q/K workloads (inputs only -- no step of the method lives here).

The pages evaluate real checkpoints on text; no weights or datasets are used
here.  Instead each workload reproduces the *shape* of one attention layer
(head counts, head_dim, RoPE theta, token count, positions) and fills Q and K
(pre-RoPE) with a per-channel Gaussian model with outlier channels:

    x[t, h, c] = mu[h, c] + sigma[h, c] * z,   z ~ N(0, 1)
    sigma ~ LogNormal(0, s_ln), mu ~ N(0, 0.1) (variance 0.1),
    outlier channels (or whole RoPE pairs) per head: sigma = s_out, mu = mu_out,
    optional heavy tail: + sigma[h, c] * t_3 on a fraction of channels.

Every random stream is numpy PCG64 seeded by a SeedSequence of
(1000 + workload number, stream id[, chunk index]): stream 0 draws the
per-(stream, head, channel) parameters (Q heads first, then K heads),
stream 1 the decode positions, streams 2 / 3 the Q / K samples of the
evaluated batch and 4 / 5 those of the calibration batch, stream 7 the V
parameters (K's recipe, own draw) and stream 6 the V samples, one generator per
chunk of 4096 tokens (so any token prefix draws identical bytes).  Values are
generated in fp32 and, for bf16 workloads, rounded to bf16 (nearest-even) by
torch; the same bytes feed the GPU path and the oracle.
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Tuple

import numpy as np

HALF_SPLIT = 0


@dataclasses.dataclass(frozen=True)
class Workload:
    number: int
    name: str
    n_tokens: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    rope_theta: float
    dtype: str                    # "f32" or "bf16"
    supports: Tuple[int, ...]     # block-Hadamard supports b exercised
    group: int
    sigma_lognormal: float        # s_ln
    outliers_per_head: int        # number of outlier channels (or pairs, see below)
    outliers_as_pairs: bool       # True: whole RoPE pairs (k, k + d/2)
    outlier_sigma: float
    outlier_mu: Optional[float]   # None: keep the base mu draw
    heavy_tail_frac: float = 0.0  # fraction of channels with an extra sigma * t_3 term
    seq_len: int = 0              # tokens per sequence (positions restart per sequence)
    decode_positions: int = 0     # >0: one token per sequence at a uniform position < this
    calib_tokens: int = 0         # >0: separate calibration batch of this many tokens
    estimator: str = "default"

    @property
    def n_pairs(self):
        return self.head_dim // 2

    @property
    def elem_bytes(self):
        return 4 if self.dtype == "f32" else 2

    def bytes_per_token(self, group=None, with_slot=None, with_v=False):
        """Algorithmic HBM bytes one rotate+quantise launch must move per token:
        Q read + K read + Q write + K codes + K fp16 scales + position (+ slot),
        plus V read + V codes + V scales when the V side is written too."""
        g = group or self.group
        e = self.elem_bytes
        d, hq, hk = self.head_dim, self.n_q_heads, self.n_kv_heads
        slot = self.decode_positions > 0 if with_slot is None else with_slot
        kv = hk * d * e + hk * d // 2 + 2 * hk * (d // g)
        return hq * d * e * 2 + kv * (2 if with_v else 1) + 4 + (8 if slot else 0)


WORKLOADS = {
    1: Workload(1, "tiny-ref-d64-fp32", 256, 2, 1, 64, 5e5, "f32", (2, 64), 64,
                0.5, 2, False, 20.0, 5.0, seq_len=256),
    2: Workload(2, "llama3.2-1b-layer-2k", 2048, 32, 8, 64, 5e5, "bf16", (2, 4, 8, 16, 32, 64), 64,
                0.5, 2, True, 20.0, 5.0, seq_len=2048),
    3: Workload(3, "llama3.2-3b-layer-4x4k", 4 * 4096, 24, 8, 128, 5e5, "bf16", (128,), 128,
                0.7, 6, True, 30.0, None, seq_len=4096),
    4: Workload(4, "llama3.1-8b-prefill-128k", 131072, 32, 8, 128, 5e5, "bf16", (128,), 128,
                0.5, 2, True, 20.0, 5.0, heavy_tail_frac=0.1, seq_len=131072),
    5: Workload(5, "mistral-7b-decode-256", 256, 32, 8, 128, 1e6, "bf16", (2, 128), 64,
                0.7, 6, True, 30.0, None, decode_positions=32768, calib_tokens=8192,
                estimator="k_only"),
}


def _draw_params(rng, w: Workload, n_heads: int):
    d = w.head_dim
    sigma = rng.lognormal(0.0, w.sigma_lognormal, size=(n_heads, d)).astype(np.float32)
    mu = rng.normal(0.0, np.sqrt(0.1), size=(n_heads, d)).astype(np.float32)
    heavy = np.zeros((n_heads, d), bool)
    for h in range(n_heads):
        if w.outliers_as_pairs:
            pairs = rng.choice(w.n_pairs, size=w.outliers_per_head, replace=False)
            chans = np.concatenate([pairs, pairs + w.n_pairs])
        else:
            chans = rng.choice(d, size=w.outliers_per_head, replace=False)
        sigma[h, chans] = w.outlier_sigma
        if w.outlier_mu is not None:
            mu[h, chans] = w.outlier_mu
        if w.heavy_tail_frac > 0:
            n_heavy = int(round(w.heavy_tail_frac * d))
            heavy[h, rng.choice(d, size=n_heavy, replace=False)] = True
    return sigma, mu, heavy


def _to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """fp32 -> stored format: fp32 values, or bf16 bit patterns (uint16) by nearest-even."""
    if dtype == "f32":
        return np.ascontiguousarray(x, np.float32)
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


CHUNK = 4096


def _rng(*key):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def _draw_samples(seed_key, w: Workload, params, n_tokens: int):
    sigma, mu, heavy = params
    n_heads, d = sigma.shape
    out = np.empty((n_tokens, n_heads, d), np.float32 if w.dtype == "f32" else np.uint16)
    heavy_idx = np.nonzero(heavy)
    for t0 in range(0, n_tokens, CHUNK):
        t1 = min(n_tokens, t0 + CHUNK)
        rng = _rng(*seed_key, t0 // CHUNK)
        z = rng.standard_normal(size=(t1 - t0, n_heads, d), dtype=np.float32)
        x = mu[None] + sigma[None] * z
        if heavy_idx[0].size:
            tt = rng.standard_t(3.0, size=(t1 - t0, heavy_idx[0].size)).astype(np.float32)
            x[:, heavy_idx[0], heavy_idx[1]] += sigma[heavy_idx][None] * tt
        out[t0:t1] = _to_storage(x, w.dtype)
    return out


def positions(w: Workload, n_tokens: int, rng=None) -> np.ndarray:
    if w.decode_positions:
        return rng.integers(0, w.decode_positions, size=n_tokens).astype(np.int32)
    L = w.seq_len or n_tokens
    return (np.arange(n_tokens, dtype=np.int64) % L).astype(np.int32)


def make_v(number: int, n_tokens: Optional[int] = None) -> np.ndarray:
    """V rows [T][Hkv][d] of workload `number` (K's recipe, streams 6 and 7)."""
    w = WORKLOADS[number]
    T = w.n_tokens if n_tokens is None else int(n_tokens)
    seed = 1000 + number
    return _draw_samples((seed, 6), w, _draw_params(_rng(seed, 7), w, w.n_kv_heads), T)


def make_inputs(number: int, n_tokens: Optional[int] = None, want_q: bool = True, want_v: bool = False):
    """Inputs of workload `number`: dict(q, k, v, pos, slot_mapping, n_slots, calib).

    q: [T][Hq][d], k and v: [T][Hkv][d] as fp32 or bf16 bits (v None unless
    want_v); pos: int32[T];
    slot_mapping: int64[T] or None (identity); calib: same dict for the
    separate calibration batch (decode workload) or None."""
    w = WORKLOADS[number]
    T = w.n_tokens if n_tokens is None else int(n_tokens)
    seed = 1000 + number
    rng = _rng(seed, 0)
    pq = _draw_params(rng, w, w.n_q_heads)
    pk = _draw_params(rng, w, w.n_kv_heads)
    res = {"workload": w}
    if w.decode_positions:
        pos = positions(w, T, _rng(seed, 1))
        res["slot_mapping"] = (np.arange(T, dtype=np.int64) * w.decode_positions + pos).astype(np.int64)
        res["n_slots"] = T * w.decode_positions
    else:
        pos = positions(w, T)
        res["slot_mapping"] = None
        res["n_slots"] = T
    res["pos"] = pos
    res["q"] = _draw_samples((seed, 2), w, pq, T) if want_q else None
    res["k"] = _draw_samples((seed, 3), w, pk, T)
    res["v"] = make_v(number, T) if want_v else None
    res["calib"] = None
    if w.calib_tokens:
        Tc = w.calib_tokens
        res["calib"] = {
            "pos": np.arange(Tc, dtype=np.int32),
            "q": _draw_samples((seed, 4), w, pq, Tc) if w.estimator != "k_only" else None,
            "k": _draw_samples((seed, 5), w, pk, Tc),
        }
    return res


def make_decode_batch(number: int = 5, group: Optional[int] = None):
    """Decode attention batch over a filled KV4 cache for the decode workload:
    one query token per sequence (the workload's Q rows stand in for the rotated
    queries), sequence b owning slots [b * C, (b + 1) * C) with C the position
    range, and its new token at position p_b attending to keys 0..p_b
    (seq_len = p_b + 1).  The cache holds seeded random code bytes (every nibble
    is a valid two's-complement INT4 code) and fp16 scales 2^U(-8, 3); streams 8
    and 9 of the workload seed.  Returns dict(q, codes, scales, seq_start,
    seq_len, n_slots, max_len, group)."""
    w = WORKLOADS[number]
    if not w.decode_positions:
        raise ValueError("workload has no decode batch")
    g = group or w.group
    inp = make_inputs(number)
    B, C, hk, d = w.n_tokens, w.decode_positions, w.n_kv_heads, w.head_dim
    n_slots = B * C
    seed = 1000 + number
    codes = _rng(seed, 8).integers(0, 256, size=(n_slots, hk, d // 2), dtype=np.uint8)
    expo = _rng(seed, 9).uniform(-8.0, 3.0, size=(n_slots, hk, d // g))
    scales = np.exp2(expo).astype(np.float16).view(np.uint16)
    return {"q": inp["q"], "codes": codes, "scales": scales,
            "seq_start": (np.arange(B, dtype=np.int64) * C), "seq_len": (inp["pos"].astype(np.int32) + 1),
            "n_slots": n_slots, "max_len": C, "group": g}
