"""ctypes declarations of the C-ABI in include/rrp.h (argument marshalling only).

The HIP library must have been built (``python rotation_rope_pair_amd/build.py``
or ``__graft_entry__.build()``); loading fails loudly otherwise -- there is no
fallback implementation.
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librrp.so")

RRP_OK, RRP_ERR_INVALID_ARG, RRP_ERR_MISALIGNED, RRP_ERR_UNSUPPORTED, RRP_ERR_HIP = range(5)
RRP_F32, RRP_BF16 = 0, 1
RRP_EST_DEFAULT, RRP_EST_K_ONLY, RRP_EST_STREAM_BALANCED = 0, 1, 2
RRP_ROPE_HALF_SPLIT, RRP_ROPE_INTERLEAVED = 0, 1

# Symbols declared in include/rrp.h.
EXPORTS = ("rrp_rotate_quantize_qk", "rrp_rotate_quantize_qkv", "rrp_calibrate_angles",
           "rrp_calibrate_angles_noalloc", "rrp_calibrate_angles_workspace_size", "rrp_quant_error_stats", "rrp_quant_error_stats_workspace_size",
           "rrp_quant_error_sweep", "rrp_quant_error_sweep_workspace_size", "rrp_decode_scores",
           "rrp_status_string", "rrp_version")


class RrpShape(ctypes.Structure):
    _fields_ = [
        ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("rope_layout", ctypes.c_int32),
        ("rope_theta", ctypes.c_double),
        ("angle_heads", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


class RrpError(RuntimeError):
    def __init__(self, func, status, msg):
        super().__init__(f"{func} failed: {msg} (status {status})")
        self.status = status


_LIB = None


def load():
    """Load librrp.so (once).  Raises if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"HIP library not built: {LIB_PATH} is missing; run rotation_rope_pair_amd/build.py")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    szp = ctypes.POINTER(ctypes.c_size_t)
    sp = ctypes.POINTER(RrpShape)
    L.rrp_rotate_quantize_qk.argtypes = [sp, i32, vp, vp, vp, i64, vp, i32, i32, vp, vp, vp, vp, i64,
                                         vp, vp, vp, vp]
    L.rrp_rotate_quantize_qkv.argtypes = [sp, i32, vp, vp, vp, vp, i64, vp, i32, i32, vp, vp, vp, vp, vp, vp,
                                          i64, vp, vp, vp, vp, vp, vp]
    L.rrp_calibrate_angles.argtypes = [sp, i32, vp, vp, vp, i64, i32, vp, vp, vp, sz, vp]
    L.rrp_calibrate_angles_workspace_size.argtypes = [sp, i64, i32, szp]
    L.rrp_calibrate_angles_noalloc.argtypes = [sp, i32, vp, vp, vp, i64, i32, vp, vp, vp]
    L.rrp_quant_error_sweep.argtypes = [sp, i32, vp, vp, i64, vp, i32, vp, vp, sz, vp]
    L.rrp_quant_error_sweep_workspace_size.argtypes = [sp, i64, szp]
    L.rrp_decode_scores.argtypes = [sp, i32, vp, i64, vp, vp, i32, i64, vp, vp, i32, vp, vp]
    L.rrp_quant_error_stats.argtypes = [sp, i32, vp, vp, i64, vp, i32, i32, vp, vp, sz, vp]
    L.rrp_quant_error_stats_workspace_size.argtypes = [sp, i64, szp]
    for f in EXPORTS:
        if f not in ("rrp_status_string", "rrp_version"):
            getattr(L, f).restype = ctypes.c_int
    L.rrp_status_string.argtypes = [ctypes.c_int]
    L.rrp_status_string.restype = ctypes.c_char_p
    L.rrp_version.argtypes = []
    L.rrp_version.restype = ctypes.c_int
    _LIB = L
    return L


def check(func, status):
    if status != RRP_OK:
        raise RrpError(func, status, load().rrp_status_string(status).decode())


def workspace_size(func, shape, *args) -> int:
    """Bytes of device workspace the entry point `func` needs (its
    <func>_workspace_size query, called with the shape and the trailing args)."""
    L = load()
    out = ctypes.c_size_t(0)
    check(func + "_workspace_size", getattr(L, func + "_workspace_size")(ctypes.byref(shape), *args,
                                                                          ctypes.byref(out)))
    return int(out.value)
