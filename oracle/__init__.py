"""NumPy front end of the CPU oracle (TEST INFRASTRUCTURE ONLY).

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library neither imports nor
links it.  Every array handed to the C oracle is host memory; inputs are the
exact same bytes the GPU path receives (fp32 values or bf16 bit patterns).
"""
import ctypes
import os

import numpy as np

from . import build as _build

F32, BF16 = 0, 1
HALF_SPLIT, INTERLEAVED = 0, 1
EST_DEFAULT, EST_K_ONLY, EST_STREAM_BALANCED = 0, 1, 2

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


class Shape(ctypes.Structure):
    _fields_ = [
        ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("rope_layout", ctypes.c_int32),
        ("rope_theta", ctypes.c_double),
        ("angle_heads", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


def lib():
    """Load liborc.so, building it with gcc first if it is not there."""
    global _LIB
    if _LIB is None:
        path = os.environ.get("RRP_ORACLE_LIB") or os.path.join(_HERE, "liborc.so")
        if not os.path.exists(path):
            _build.build()
        L = ctypes.CDLL(path)
        vp, i32, i64, dbl = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        L.orc_inv_freq.argtypes = [dbl, ctypes.c_int, vp]
        L.orc_rope_angle.argtypes = [i32, ctypes.c_float]
        L.orc_rope_angle.restype = ctypes.c_float
        L.orc_rope_row.argtypes = [vp, ctypes.c_int, ctypes.c_int, vp, i32, vp]
        L.orc_pair_rotate_row.argtypes = [vp, ctypes.c_int, ctypes.c_int, vp, vp]
        L.orc_hadamard_blocks.argtypes = [vp, ctypes.c_int, ctypes.c_int, vp]
        L.orc_transform_row.argtypes = [vp, ctypes.c_int, ctypes.c_int, vp, i32, vp, ctypes.c_int, vp]
        L.orc_f16_bits.argtypes = [ctypes.c_float]
        L.orc_f16_bits.restype = ctypes.c_uint16
        L.orc_f16_value.argtypes = [ctypes.c_uint16]
        L.orc_f16_value.restype = dbl
        L.orc_bf16_bits.argtypes = [dbl]
        L.orc_bf16_bits.restype = ctypes.c_uint16
        L.orc_quantize_group.argtypes = [vp, ctypes.c_int, vp, vp, vp]
        L.orc_pack_nibbles.argtypes = [vp, ctypes.c_int, vp]
        L.orc_rotate_quantize_qk.argtypes = [
            ctypes.POINTER(Shape), ctypes.c_int, vp, vp, vp, i64, vp, ctypes.c_int, ctypes.c_int,
            vp, vp, vp, vp, i64, vp, vp, vp]
        L.orc_calibrate_moments.argtypes = [ctypes.POINTER(Shape), ctypes.c_int, vp, vp, vp, i64, vp]
        L.orc_angles_from_moments.argtypes = [vp, ctypes.c_int, ctypes.c_int, vp, vp, vp]
        L.orc_quant_error_stats.argtypes = [
            ctypes.POINTER(Shape), ctypes.c_int, vp, vp, i64, vp, ctypes.c_int, ctypes.c_int, vp]
        L.orc_quantize_v.argtypes = [ctypes.POINTER(Shape), ctypes.c_int, vp, i64, ctypes.c_int, vp, vp, vp, i64,
                                     vp, vp]
        L.orc_quantize_v.restype = ctypes.c_int
        L.orc_decode_scores.argtypes = [ctypes.POINTER(Shape), ctypes.c_int, vp, i64, vp, vp, ctypes.c_int, i64,
                                        vp, vp, ctypes.c_int, vp]
        L.orc_decode_scores.restype = ctypes.c_int
        L.orc_max_threads.argtypes = []
        L.orc_max_threads.restype = ctypes.c_int
        L.orc_set_threads.argtypes = [ctypes.c_int]
        L.orc_set_threads.restype = ctypes.c_int
        for name in ("orc_rotate_quantize_qk", "orc_calibrate_moments",
                     "orc_angles_from_moments", "orc_quant_error_stats"):
            getattr(L, name).restype = ctypes.c_int
        _LIB = L
    return _LIB


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _in(x):
    """(array, dtype code) for an input stored as fp32 values or bf16 bits (uint16)."""
    if x is None:
        return None, F32
    x = np.ascontiguousarray(x)
    if x.dtype == np.float32:
        return x, F32
    if x.dtype == np.uint16:
        return x, BF16
    raise TypeError(f"oracle inputs are float32 values or bf16 bits (uint16), got {x.dtype}")


# ---- scalar building blocks ----------------------------------------------

def inv_freq(theta, head_dim):
    out = np.zeros(head_dim // 2, np.float32)
    lib().orc_inv_freq(float(theta), int(head_dim), _p(out))
    return out


def rope_angle(pos, inv_freq_k):
    return np.float32(lib().orc_rope_angle(int(pos), float(inv_freq_k)))


def rope_row(x, layout, inv_freq_tab, pos):
    x = _c(x, np.float64)
    out = np.empty_like(x)
    lib().orc_rope_row(_p(x), x.size, layout, _p(_c(inv_freq_tab, np.float32)), int(pos), _p(out))
    return out


def pair_rotate_row(x, layout, angles):
    x = _c(x, np.float64)
    out = np.empty_like(x)
    lib().orc_pair_rotate_row(_p(x), x.size, layout, _p(_c(angles, np.float32)), _p(out))
    return out


def hadamard_blocks(x, b):
    x = _c(x, np.float64)
    out = np.empty_like(x)
    lib().orc_hadamard_blocks(_p(x), x.size, int(b), _p(out))
    return out


def transform_row(x, layout, inv_freq_tab, pos, angles, b):
    x = _c(x, np.float64)
    out = np.empty_like(x)
    ang = None if angles is None else _c(angles, np.float32)
    lib().orc_transform_row(_p(x), x.size, layout, _p(_c(inv_freq_tab, np.float32)), int(pos),
                            _p(ang), int(b), _p(out))
    return out


def f16_bits(x):
    return int(lib().orc_f16_bits(float(np.float32(x))))


def f16_value(bits):
    return float(lib().orc_f16_value(int(bits)))


def bf16_bits(x):
    return int(lib().orc_bf16_bits(float(x)))


def quantize_group(y):
    y = _c(y, np.float64)
    q = np.zeros(y.size, np.int8)
    sh = np.zeros(1, np.uint16)
    s32 = np.zeros(1, np.float32)
    lib().orc_quantize_group(_p(y), y.size, _p(q), _p(sh), _p(s32))
    return q, int(sh[0]), np.float32(s32[0])


def pack_nibbles(q):
    q = _c(q, np.int8)
    out = np.zeros(q.size // 2, np.uint8)
    lib().orc_pack_nibbles(_p(q), q.size, _p(out))
    return out


# ---- operations ------------------------------------------------------------

def max_threads():
    """OpenMP threads the token-parallel oracle functions use."""
    return int(lib().orc_max_threads())


def set_threads(n):
    """Sets the OpenMP threads of later oracle calls; returns the previous count."""
    return int(lib().orc_set_threads(int(n)))


def shape(n_q_heads, n_kv_heads, head_dim, rope_theta, rope_layout=HALF_SPLIT, angle_heads=0):
    """angle_heads: 0 / 1 = one angle set shared by all heads; n_kv_heads = one per key head."""
    return Shape(int(n_q_heads), int(n_kv_heads), int(head_dim), int(rope_layout), float(rope_theta),
                 int(angle_heads), 0)


def angle_groups(shp):
    return shp.angle_heads if shp.angle_heads > 1 else 1


def rotate_quantize_qk(shp, q, k, pos, angles, support_b, group, slot_mapping=None,
                       n_slots=None, want_q_out=True):
    """Returns a dict with q_out (same format as q), q_rot / k_rot (fp64),
    k_codes (uint8 [n_slots][Hkv][d/2]), k_scales (fp16 bits), k_scale32 (fp32)."""
    qa, dt = _in(q)
    ka, dtk = _in(k)
    if qa is not None and dt != dtk:
        raise TypeError("q and k must have the same format")
    T = ka.shape[0]
    d, hq, hk = shp.head_dim, shp.n_q_heads, shp.n_kv_heads
    pos = _c(pos, np.int32)
    if n_slots is None:
        n_slots = T if slot_mapping is None else int(np.max(slot_mapping, initial=-1)) + 1
    sm = None if slot_mapping is None else _c(slot_mapping, np.int64)
    out = {
        "q_out": (np.zeros((T, hq, d), qa.dtype) if (qa is not None and want_q_out) else None),
        "q_rot": (np.zeros((T, hq, d), np.float64) if qa is not None else None),
        "k_rot": np.zeros((T, hk, d), np.float64),
        "k_codes": np.zeros((n_slots, hk, d // 2), np.uint8),
        "k_scales": np.zeros((n_slots, hk, d // group), np.uint16),
        "k_scale32": np.zeros((T, hk, d // group), np.float32),
    }
    ang = None if angles is None else _c(angles, np.float32)
    rc = lib().orc_rotate_quantize_qk(
        ctypes.byref(shp), dtk, _p(qa), _p(ka), _p(pos), T, _p(ang), int(support_b), int(group),
        _p(out["q_out"]), _p(out["k_codes"]), _p(out["k_scales"]), _p(sm), int(n_slots),
        _p(out["q_rot"]), _p(out["k_rot"]), _p(out["k_scale32"]))
    if rc != 0:
        raise ValueError("oracle rotate_quantize_qk rejected its arguments")
    return out


def quantize_v(shp, v, group, slot_mapping=None, n_slots=None):
    """V half of the KV4 cache.  Returns a dict with v_rot (fp64 [T][Hkv][d]),
    v_codes (uint8 [n_slots][Hkv][d/2]), v_scales (fp16 bits), v_scale32 (fp32)."""
    va, dt = _in(v)
    T = va.shape[0]
    d, hk = shp.head_dim, shp.n_kv_heads
    if n_slots is None:
        n_slots = T if slot_mapping is None else int(np.max(slot_mapping, initial=-1)) + 1
    sm = None if slot_mapping is None else _c(slot_mapping, np.int64)
    out = {
        "v_rot": np.zeros((T, hk, d), np.float64),
        "v_codes": np.zeros((n_slots, hk, d // 2), np.uint8),
        "v_scales": np.zeros((n_slots, hk, d // group), np.uint16),
        "v_scale32": np.zeros((T, hk, d // group), np.float32),
    }
    rc = lib().orc_quantize_v(ctypes.byref(shp), dt, _p(va), T, int(group), _p(out["v_codes"]),
                              _p(out["v_scales"]), _p(sm), int(n_slots), _p(out["v_rot"]), _p(out["v_scale32"]))
    if rc != 0:
        raise ValueError("oracle quantize_v rejected its arguments")
    return out


def decode_scores(shp, q, k_codes, k_scales, group, seq_start, seq_len, max_len, n_slots=None):
    """Decode logits fp64 [B][Hq][max_len] from the KV4 cache (entries past each
    sequence's length stay -inf here, NaN for slots outside the cache)."""
    qa, dt = _in(q)
    B = qa.shape[0]
    codes = _c(k_codes, np.uint8)
    scales = _c(k_scales, np.uint16)
    if n_slots is None:
        n_slots = codes.shape[0]
    out = np.full((B, shp.n_q_heads, int(max_len)), -np.inf, np.float64)
    rc = lib().orc_decode_scores(ctypes.byref(shp), dt, _p(qa), B, _p(codes), _p(scales), int(group), int(n_slots),
                                 _p(_c(seq_start, np.int64)), _p(_c(seq_len, np.int32)), int(max_len), _p(out))
    if rc != 0:
        raise ValueError("oracle decode_scores rejected its arguments")
    return out


def calibrate_moments(shp, q, k, pos, moments=None):
    qa, _ = _in(q)
    ka, dtk = _in(k)
    P = shp.head_dim // 2
    if moments is None:
        A = angle_groups(shp)
        moments = np.zeros((P, 2, 6) if A == 1 else (A, P, 2, 6), np.float64)
    rc = lib().orc_calibrate_moments(ctypes.byref(shp), dtk, _p(qa), _p(ka), _p(_c(pos, np.int32)),
                                     ka.shape[0], _p(moments))
    if rc != 0:
        raise ValueError("oracle calibrate_moments rejected its arguments")
    return moments


def angles_from_moments(moments, estimator):
    """moments [..., P, 2, 6] (one set per leading index) -> phi64, phi32 [..., P], abc [..., P, 3]."""
    moments = _c(moments, np.float64)
    lead = moments.shape[:-2]
    n = int(np.prod(lead))
    phi64 = np.zeros(n, np.float64)
    phi32 = np.zeros(n, np.float32)
    abc = np.zeros((n, 3), np.float64)
    rc = lib().orc_angles_from_moments(_p(moments), n, int(estimator), _p(phi64), _p(phi32), _p(abc))
    if rc != 0:
        raise ValueError("oracle angles_from_moments rejected its arguments")
    return phi64.reshape(lead), phi32.reshape(lead), abc.reshape(lead + (3,))


def quant_error_stats(shp, k, pos, angles, support_b, group):
    ka, dtk = _in(k)
    stats = np.zeros(8, np.float64)
    ang = None if angles is None else _c(angles, np.float32)
    rc = lib().orc_quant_error_stats(ctypes.byref(shp), dtk, _p(ka), _p(_c(pos, np.int32)),
                                     ka.shape[0], _p(ang), int(support_b), int(group), _p(stats))
    if rc != 0:
        raise ValueError("oracle quant_error_stats rejected its arguments")
    return stats
