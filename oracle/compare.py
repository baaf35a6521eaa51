"""Element-by-element comparison of GPU outputs with the oracle (TEST INFRASTRUCTURE ONLY).

Tolerances (fixed by the parity contract):
  rotated fp32 values   max over rows of max|gpu - ref| / max|ref| <= 1e-5 for Q rows
                        (fp32 arithmetic: RoPE, pair rotation and log2 b butterfly
                        roundings, amplified by at most sqrt(d) against the row
                        max), 2^-23 for K and V rows (fp64 values exported to fp32:
                        one rounding)
  Q output (bf16/fp32)  |out - ref| <= half an ulp of the output format at |ref|
                        + 1e-5 * max|ref row| (the fp32 allowance above)
  fp32 group scale s32  relative error <= 2^-23: both sides take the group absmax
                        m in fp64 and round m / 7 once to fp32, so they can differ by
                        at most that one rounding
  fp16 stored scale     bit-exact, except groups whose oracle s32 lies within
                        2^-23 (relative) of an fp16 rounding midpoint (counted)
  INT4 codes            bit-exact, except values whose oracle pre-round y / s_h lies
                        within 1e-9 of a half-integer, or whose group's fp16 scale
                        differs (counted); both sides evaluate y in fp64, where they
                        agree to about 1e-14
  angles                |dphi| <= min(2^-25 + 1e-11 / cond, 1e-6) rad: phi is
                        computed in fp64 and rounded once to fp32 (half an ulp,
                        <= 2^-25 for |phi| <= pi/4), and the moments differ by their
                        summation order (within the 1e-11 moment bar), which moves
                        atan2 by at most that over cond = sqrt((a - b)^2 + 4 c^2) /
                        (a + b); the bar never exceeds the 1e-6 rad angle tolerance.
                        Pairs whose centred covariance is isotropic to 1e-9 are
                        counted as ill-conditioned (the only pairs exempt)
"""
import math

import numpy as np

ROW_REL_TOL = 1e-5
KV_ROW_REL_TOL = 2.0 ** -23
SCALE_REL_TOL = 2.0 ** -23
CODE_BAND = 1e-9
ANGLE_HALF_ULP = 2.0 ** -25
ANGLE_TOL = 1e-6
MOMENT_REL_TOL = 1e-11
ILL_COND = 1e-9


class ParityError(AssertionError):
    pass


def unpack_codes(codes: np.ndarray) -> np.ndarray:
    """uint8 [..., d/2] -> int8 [..., d]: low nibble = even channel, two's complement."""
    lo = (codes & 0xF).astype(np.int8)
    hi = (codes >> 4).astype(np.int8)
    lo = np.where(lo > 7, lo - 16, lo).astype(np.int8)
    hi = np.where(hi > 7, hi - 16, hi).astype(np.int8)
    return np.stack([lo, hi], -1).reshape(*codes.shape[:-1], codes.shape[-1] * 2)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return bits.view(np.float16).astype(np.float64)


def _ulp(x: np.ndarray, mant_bits: int, emin: int) -> np.ndarray:
    ax = np.maximum(np.abs(x), np.ldexp(1.0, emin))
    e = np.floor(np.log2(ax))
    return np.ldexp(1.0, (e - mant_bits).astype(np.int64))


def row_rel_err(gpu: np.ndarray, ref: np.ndarray) -> float:
    """max over rows (last axis) of max|gpu - ref| / max|ref|."""
    g = gpu.reshape(-1, gpu.shape[-1]).astype(np.float64)
    r = ref.reshape(-1, ref.shape[-1]).astype(np.float64)
    num = np.abs(g - r).max(1)
    den = np.abs(r).max(1)
    bad_zero = (den == 0) & (num > 0)
    if bad_zero.any():
        return math.inf
    with np.errstate(invalid="ignore", divide="ignore"):
        rel = np.where(den > 0, num / np.where(den > 0, den, 1.0), 0.0)
    return float(rel.max(initial=0.0))


def check_q_out(q_out_gpu: np.ndarray, q_rot_ref: np.ndarray, fmt: str) -> float:
    """Q output within half an output ulp plus the fp32 row allowance."""
    r = q_rot_ref.reshape(-1, q_rot_ref.shape[-1])
    if fmt == "bf16":
        g = bf16_bits_to_f64(q_out_gpu.reshape(r.shape))
        half = 0.5 * _ulp(np.maximum(np.abs(r), np.abs(g)), 7, -126)
    else:
        g = q_out_gpu.reshape(r.shape).astype(np.float64)
        half = 0.5 * _ulp(np.maximum(np.abs(r), np.abs(g)), 23, -126)
    allow = half + ROW_REL_TOL * np.abs(r).max(1, keepdims=True)
    excess = np.abs(g - r) - allow * (1 + 1e-12)
    worst = float(excess.max(initial=-1.0))
    if worst > 0:
        i = np.unravel_index(np.argmax(excess), excess.shape)
        raise ParityError(f"Q output off by more than the allowance at row {i[0]} ch {i[1]}: "
                          f"gpu {g[i]!r} ref {r[i]!r} allow {allow[i]!r}")
    return worst


def f16_midpoint_band(s32: np.ndarray, rel: float = SCALE_REL_TOL) -> np.ndarray:
    """True where s32 lies within `rel` (relative) of the rounding midpoint between the
    two fp16 values that enclose it (values at or above the saturation bound excluded)."""
    s = np.abs(s32.astype(np.float64))
    with np.errstate(over="ignore", invalid="ignore"):
        h = np.minimum(s.astype(np.float16).astype(np.float64), 65504.0)  # nearest fp16
        below = np.where(h <= s, h, np.nextafter(h.astype(np.float16), np.float16(-np.inf)).astype(np.float64))
        above = np.nextafter(below.astype(np.float16), np.float16(np.inf)).astype(np.float64)
        mid = 0.5 * (below + above)
    near = np.abs(s - mid) <= rel * np.maximum(s, 1e-300)
    return near & (s < 65504.0)


def compare_k(codes_gpu, scales_gpu_bits, k_rot_ref, scales_ref_bits, codes_ref, group,
              s32_gpu=None, s32_ref=None, k_rot_gpu=None):
    """Compare the K side for rows given as [rows][d] (codes [rows][d/2], scales [rows][d/g]).
    Returns a report dict; raises ParityError on any mismatch outside the stated bands."""
    rows, d = k_rot_ref.shape[0], k_rot_ref.shape[-1]
    ng = d // group
    rep = {"rows": int(rows), "groups": int(rows * ng), "codes": int(rows * d)}
    if k_rot_gpu is not None:
        rep["k_row_rel_err"] = row_rel_err(k_rot_gpu, k_rot_ref)
        if not rep["k_row_rel_err"] <= KV_ROW_REL_TOL:
            raise ParityError(f"rotated K row error {rep['k_row_rel_err']:.3g} > {KV_ROW_REL_TOL}")
    if s32_gpu is not None:
        g, r = s32_gpu.astype(np.float64).ravel(), s32_ref.astype(np.float64).ravel()
        bad = (r == 0) & (g != 0)
        rel = np.where(r > 0, np.abs(g - r) / np.where(r > 0, r, 1.0), 0.0)
        rep["scale_rel_err"] = float(rel.max(initial=0.0))
        if bad.any() or rep["scale_rel_err"] > SCALE_REL_TOL:
            raise ParityError(f"fp32 group scale error {rep['scale_rel_err']:.3g} > {SCALE_REL_TOL}")
    sg = scales_gpu_bits.reshape(rows, ng)
    sr = scales_ref_bits.reshape(rows, ng)
    smis = sg != sr
    # band from the oracle's fp32 scale: recompute it from k_rot_ref if not given
    if s32_ref is None:
        m = np.abs(k_rot_ref.reshape(rows, ng, group)).max(-1)
        s32r = (m / 7.0).astype(np.float32)
    else:
        s32r = s32_ref.reshape(rows, ng)
    sband = f16_midpoint_band(s32r)
    rep["scale_mismatch"] = int(smis.sum())
    rep["scale_band"] = int(sband.sum())
    if (smis & ~sband).any():
        i = np.argwhere(smis & ~sband)[0]
        raise ParityError(f"fp16 scale mismatch outside the midpoint band at row {i[0]} group {i[1]}: "
                          f"gpu {sg[tuple(i)]:#06x} ref {sr[tuple(i)]:#06x} s32 {s32r[tuple(i)]!r}")
    cg = unpack_codes(codes_gpu.reshape(rows, d // 2))
    cr = unpack_codes(codes_ref.reshape(rows, d // 2))
    sh = f16_bits_to_f64(sr).reshape(rows, ng, 1)
    with np.errstate(invalid="ignore", divide="ignore"):
        v = np.where(sh > 0, k_rot_ref.reshape(rows, ng, group) / np.where(sh > 0, sh, 1.0), 0.0)
    frac = np.abs(v - np.floor(v) - 0.5)
    cband = (frac < CODE_BAND).reshape(rows, d) | np.repeat(smis, group, axis=1)
    cmis = cg != cr
    rep["code_mismatch"] = int(cmis.sum())
    rep["code_band"] = int(cband.sum())
    if (cmis & ~cband).any():
        i = np.argwhere(cmis & ~cband)[0]
        raise ParityError(f"INT4 code mismatch outside the rounding band at row {i[0]} ch {i[1]}: "
                          f"gpu {cg[tuple(i)]} ref {cr[tuple(i)]} v {v.reshape(rows, d)[tuple(i)]!r}")
    return rep


def angle_diff(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """|a - b| modulo the pi/2 period of the minimax solution set."""
    d = np.abs(a.astype(np.float64) - b.astype(np.float64)) % (math.pi / 2)
    return np.minimum(d, math.pi / 2 - d)


def compare_angles(phi_gpu, phi_ref64, abc_ref):
    a, b, c = abc_ref[:, 0], abc_ref[:, 1], abc_ref[:, 2]
    cond = np.hypot(a - b, 2 * c) / np.maximum(a + b, 1e-300)
    ill = cond < ILL_COND
    d = angle_diff(phi_gpu, phi_ref64)
    tol = np.minimum(ANGLE_HALF_ULP + MOMENT_REL_TOL / np.maximum(cond, 1e-300), ANGLE_TOL)
    rep = {"pairs": int(len(d)), "ill_conditioned": int(ill.sum()),
           "max_angle_err": float(d[~ill].max(initial=0.0)), "min_condition": float(cond.min(initial=1.0)),
           "max_err_over_tol": float((d / tol)[~ill].max(initial=0.0))}
    over = (d > tol) & ~ill
    if over.any():
        k = int(np.argmax(np.where(over, d - tol, -np.inf)))
        raise ParityError(f"angle of pair {k} off by {d[k]:.3g} rad > {tol[k]:.3g} (gpu {phi_gpu[k]!r}, "
                          f"ref {phi_ref64[k]!r}, condition {cond[k]:.3g})")
    return rep


def compare_moments(m_gpu, m_ref, rel=MOMENT_REL_TOL):
    """fp64 sums: n exact; first and second moments within rel of their natural scale."""
    g, r = m_gpu.reshape(-1, 2, 6), m_ref.reshape(-1, 2, 6)
    if not np.array_equal(g[..., 0], r[..., 0]):
        raise ParityError("sample counts differ")
    n = np.maximum(r[..., 0], 1.0)
    suu, svv = np.abs(r[..., 3]), np.abs(r[..., 4])
    scale = np.stack([np.sqrt(n * suu), np.sqrt(n * svv), suu, svv, np.sqrt(suu * svv)], -1)
    err = np.abs(g[..., 1:] - r[..., 1:]) / np.maximum(scale, 1e-300)
    worst = float(err.max(initial=0.0))
    if worst > rel:
        raise ParityError(f"calibration moment error {worst:.3g} > {rel}")
    return worst
