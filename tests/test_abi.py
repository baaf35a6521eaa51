"""The C-ABI library loads, exports every entry point include/rrp.h declares, and
rejects bad arguments on the host before touching the GPU (no GPU needed)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rrp.h")


@pytest.fixture(scope="module")
def lib():
    from rotation_rope_pair_amd import _abi
    if not os.path.exists(_abi.LIB_PATH):
        from rotation_rope_pair_amd import build
        build.build()
    return _abi.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rrp_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted(["rrp_calibrate_angles", "rrp_calibrate_angles_noalloc",
                                           "rrp_calibrate_angles_workspace_size",
                                           "rrp_quant_error_stats", "rrp_quant_error_stats_workspace_size",
                                           "rrp_rotate_quantize_qk", "rrp_rotate_quantize_qkv", "rrp_decode_scores",
                                           "rrp_quant_error_sweep", "rrp_quant_error_sweep_workspace_size",
                                           "rrp_status_string", "rrp_version"])


def test_library_exports_exactly_the_declared_symbols(lib):
    from rotation_rope_pair_amd import _abi
    out = subprocess.run(["nm", "-D", "--defined-only", _abi.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = sorted({l.split()[-1] for l in out.splitlines() if " T " in l and l.split()[-1].startswith("rrp_")})
    assert exported == declared_functions()
    for name in declared_functions():
        assert hasattr(lib, name)
    assert sorted(_abi.EXPORTS) == declared_functions()


def test_version_and_status_strings(lib):
    assert lib.rrp_version() == 10000
    assert lib.rrp_status_string(0) == b"ok"
    assert lib.rrp_status_string(2) == b"misaligned pointer"
    assert lib.rrp_status_string(99) == b"unknown status"


def _shape(hq=32, hk=8, d=128, layout=0, theta=5e5, ah=0):
    from rotation_rope_pair_amd._abi import RrpShape
    return RrpShape(hq, hk, d, layout, theta, ah, 0)


P16 = ctypes.c_void_p(1 << 20)       # a 16-byte aligned, never dereferenced address
P2 = ctypes.c_void_p((1 << 20) + 2)   # 2-byte aligned only


def rot(lib, shape=None, dtype=1, q=None, k=P16, pos=P16, T=4, angles=None, b=128, g=128, q_out=None,
        codes=P16, scales=P16, slots=None, n_slots=4, qd=None, kd=None, sd=None):
    return lib.rrp_rotate_quantize_qk(ctypes.byref(shape or _shape()), dtype, q, k, pos, T, angles, b, g, q_out,
                                      codes, scales, slots, n_slots, qd, kd, sd, None)


def test_rotate_validation(lib):
    assert rot(lib, T=0, n_slots=0) == 0                          # empty batch: no-op
    assert rot(lib, T=0, n_slots=0, k=None, pos=None, codes=None, scales=None) == 0  # empty arrays may be NULL
    assert rot(lib, T=0, b=3) == 1                                # but the call itself is still checked
    assert lib.rrp_rotate_quantize_qk(None, 1, None, P16, P16, 4, None, 128, 128, None, P16, P16, None, 4,
                                      None, None, None, None) == 1
    assert rot(lib, dtype=7) == 1
    assert rot(lib, shape=_shape(d=96)) == 3
    assert rot(lib, shape=_shape(d=65)) == 1
    assert rot(lib, shape=_shape(hk=0)) == 1
    assert rot(lib, shape=_shape(layout=5)) == 1
    assert rot(lib, shape=_shape(theta=-1.0)) == 1
    assert rot(lib, shape=_shape(theta=float("inf"))) == 1
    assert rot(lib, b=3) == 1 and rot(lib, b=256) == 1 and rot(lib, b=0) == 1
    assert rot(lib, g=1) == 1 and rot(lib, g=96) == 1 and rot(lib, g=256) == 1
    assert rot(lib, T=-1) == 1
    assert rot(lib, k=None) == 1 and rot(lib, pos=None) == 1
    assert rot(lib, codes=None) == 1 and rot(lib, scales=None) == 1
    assert rot(lib, q_out=P16) == 1                               # q_out needs q
    assert rot(lib, n_slots=3) == 1                               # identity slots need n_slots >= T
    assert rot(lib, k=P2) == 2 and rot(lib, q=P2, q_out=P16) == 2
    assert rot(lib, codes=P2) == 2 and rot(lib, kd=P2) == 2
    assert rot(lib, slots=ctypes.c_void_p((1 << 20) + 4)) == 2


def test_angle_heads_validation(lib):
    """angle_heads is 0 or 1 (one shared set) or n_kv_heads (one set per key head)."""
    assert rot(lib, shape=_shape(ah=-1)) == 1
    assert rot(lib, shape=_shape(ah=4)) == 1                      # neither shared nor n_kv_heads
    assert rot(lib, shape=_shape(hq=12, hk=8, ah=8)) == 1         # query heads must split evenly
    assert rot(lib, shape=_shape(hq=32, hk=16, ah=16)) == 3       # more sets than the LDS tables hold
    assert lib.rrp_calibrate_angles(ctypes.byref(_shape(ah=3)), 1, P16, P16, P16, 4, 0, P16, None, P16, 1 << 30,
                                    None) == 1
    assert lib.rrp_quant_error_stats(ctypes.byref(_shape(ah=2)), 1, P16, P16, 4, None, 128, 128, P16, P16,
                                     1 << 30, None) == 1
    from rotation_rope_pair_amd import api
    assert api.angle_sets(api.layer_shape(32, 8, 128, 5e5)) == 1
    assert api.angle_sets(api.layer_shape(32, 8, 128, 5e5, angle_heads=1)) == 1
    assert api.angle_sets(api.layer_shape(32, 8, 128, 5e5, angle_heads=8)) == 8


def test_rotate_qkv_validation(lib):
    def rqkv(v=P16, vc=P16, vs=P16, T=4, vd=None, vsd=None, k=P16):
        return lib.rrp_rotate_quantize_qkv(ctypes.byref(_shape()), 1, None, k, v, P16, T, None, 128, 128, None,
                                           P16, P16, vc, vs, None, 4, None, None, None, vd, vsd, None)
    assert rqkv(T=0) == 0
    assert rqkv(v=None) == 1 and rqkv(vc=None) == 1 and rqkv(vs=None) == 1 and rqkv(k=None) == 1
    assert rqkv(v=P2) == 2 and rqkv(vc=P2) == 2 and rqkv(vd=P2) == 2
    assert rqkv(vs=ctypes.c_void_p((1 << 20) + 1)) == 2


def test_decode_scores_validation(lib):
    def dec(shape=None, dtype=1, q=P16, B=4, codes=P16, scales=P16, g=64, n_slots=100, start=P16, lens=P16,
            max_len=64, out=P16):
        return lib.rrp_decode_scores(ctypes.byref(shape or _shape()), dtype, q, B, codes, scales, g, n_slots, start,
                                     lens, max_len, out, None)
    assert dec(B=0) == 0 and dec(max_len=0) == 0                  # nothing to do
    assert dec(shape=_shape(hq=12, hk=8)) == 1                    # query heads not a multiple of key heads
    assert dec(shape=_shape(hq=0)) == 1
    assert dec(shape=_shape(hq=32, hk=1)) == 3                    # more than 16 query heads per key head
    assert dec(shape=_shape(hq=1 << 17, hk=1 << 17)) == 3         # a 256-key band past 32-bit offsets
    assert dec(g=3) == 1 and dec(g=256) == 1 and dec(g=1) == 1
    assert dec(B=-1) == 1 and dec(n_slots=-1) == 1 and dec(max_len=-5) == 1 and dec(n_slots=0) == 1
    assert dec(q=None) == 1 and dec(codes=None) == 1 and dec(scales=None) == 1
    assert dec(start=None) == 1 and dec(lens=None) == 1 and dec(out=None) == 1
    assert dec(q=P2) == 2 and dec(codes=P2) == 2 and dec(start=ctypes.c_void_p((1 << 20) + 4)) == 2
    assert dec(codes=ctypes.c_void_p((1 << 20) + 8)) == 2                      # d = 128 rows: 16-byte loads
    assert dec(scales=ctypes.c_void_p((1 << 20) + 2), g=32) == 2   # 8-byte scale rows need 8-byte alignment
    assert dec(shape=_shape(d=96)) == 3
    assert dec(max_len=2**31 - 1) == 3 and dec(max_len=2**31 - 512) == 3   # key indices stay 32-bit
    # one sequence's waves (ceil(max_len / 128) * n_kv_heads) overfill a one-dimensional grid
    assert dec(shape=_shape(hq=9, hk=9), max_len=2**31 - 1024) == 3
    assert dec(shape=_shape(hq=12, hk=12), max_len=2**31 - 1024) == 3  # over 65535 chunks: no 3-D grid either


BIG = 1 << 30  # a workspace size above any requirement


def ws_size(lib, func, shape, *args):
    out = ctypes.c_size_t(0)
    rc = getattr(lib, func + "_workspace_size")(ctypes.byref(shape), *args, ctypes.byref(out))
    return rc, out.value


def test_calibrate_validation(lib):
    def cal(shape=None, dtype=1, q=P16, k=P16, pos=P16, T=4, est=0, mom=P16, ang=None, ws=P16, ws_bytes=BIG):
        return lib.rrp_calibrate_angles(ctypes.byref(shape or _shape()), dtype, q, k, pos, T, est, mom, ang, ws,
                                        ws_bytes, None)
    assert cal(est=3) == 1 and cal(est=-1) == 1
    assert cal(mom=None) == 1
    assert cal(q=None, est=0) == 1 and cal(q=None, est=2) == 1    # Q needed by these estimators
    assert cal(k=None) == 1 and cal(pos=None) == 1 and cal(T=-2) == 1
    assert cal(shape=_shape(d=256)) == 3
    assert cal(k=P2) == 2 and cal(mom=ctypes.c_void_p((1 << 20) + 4)) == 2
    assert cal(T=0, q=None, k=None, pos=None, ang=None, ws=None, ws_bytes=0) == 0  # nothing to do


def test_calibrate_workspace(lib):
    """The size query, and a missing, short or misaligned workspace rejected
    before anything is enqueued."""
    def cal(ws=P16, ws_bytes=BIG, q=P16, est=0, T=4096):
        return lib.rrp_calibrate_angles(ctypes.byref(_shape()), 1, q, P16, P16, T, est, P16, None, ws, ws_bytes,
                                        None)
    rc, need = ws_size(lib, "rrp_calibrate_angles", _shape(), 4096, 1)
    assert rc == 0 and need > 0 and need % (64 * 5 * 8) == 0      # [blocks][pairs][5 sums] doubles
    assert need <= 4096 * 64 * 5 * 8
    rc, need_k = ws_size(lib, "rrp_calibrate_angles", _shape(), 4096, 0)
    assert rc == 0 and 0 < need_k <= need                         # K stream only: no more blocks
    assert ws_size(lib, "rrp_calibrate_angles", _shape(), 0, 1) == (0, 0)
    _, big = ws_size(lib, "rrp_calibrate_angles", _shape(), 1 << 40, 1)
    assert big == 4096 * 64 * 5 * 8                               # capped partial columns
    _, sets = ws_size(lib, "rrp_calibrate_angles", _shape(ah=8), 1 << 40, 1)
    assert sets <= 4096 * 64 * 5 * 8
    assert ws_size(lib, "rrp_calibrate_angles", _shape(d=96), 16, 1)[0] == 3
    assert ws_size(lib, "rrp_calibrate_angles", _shape(), -1, 1)[0] == 1
    assert lib.rrp_calibrate_angles_workspace_size(ctypes.byref(_shape()), 16, 1, None) == 1
    assert cal(ws=None) == 1 and cal(ws_bytes=need - 8) == 1
    assert cal(q=None, est=1, ws_bytes=need_k - 8) == 1
    assert cal(ws=ctypes.c_void_p((1 << 20) + 4)) == 2


def test_calibrate_noalloc_validation(lib):
    """The no-allocation variant checks its arguments exactly as rrp_calibrate_angles
    does, before touching any device."""
    def cal(shape=None, dtype=1, q=P16, k=P16, pos=P16, T=4, est=0, mom=P16, ang=None):
        return lib.rrp_calibrate_angles_noalloc(ctypes.byref(shape or _shape()), dtype, q, k, pos, T, est, mom, ang,
                                                None)
    assert cal(est=3) == 1 and cal(mom=None) == 1 and cal(q=None, est=0) == 1 and cal(k=None) == 1
    assert cal(T=-1) == 1 and cal(shape=_shape(d=256)) == 3 and cal(shape=_shape(ah=3)) == 1
    assert cal(k=P2) == 2 and cal(mom=ctypes.c_void_p((1 << 20) + 4)) == 2


def test_stats_validation(lib):
    def stt(T=4, k=P16, pos=P16, b=128, g=128, out=P16, ws=P16, ws_bytes=BIG):
        return lib.rrp_quant_error_stats(ctypes.byref(_shape()), 1, k, pos, T, None, b, g, out, ws, ws_bytes, None)
    assert stt(out=None) == 1 and stt(k=None) == 1 and stt(b=5) == 1 and stt(g=3) == 1
    assert stt(out=ctypes.c_void_p((1 << 20) + 4)) == 2
    rc, need = ws_size(lib, "rrp_quant_error_stats", _shape(), 131072)
    assert rc == 0 and 0 < need <= 8192 * 5 * 8
    assert ws_size(lib, "rrp_quant_error_stats", _shape(), 0) == (0, 0)
    assert stt(T=131072, ws=None) == 1 and stt(T=131072, ws_bytes=need - 1) == 1
    assert stt(T=131072, ws=ctypes.c_void_p((1 << 20) + 4)) == 2


def test_sweep_validation(lib):
    def swp(T=4, k=P16, pos=P16, g=128, out=P16, shape=None, ws=P16, ws_bytes=BIG):
        return lib.rrp_quant_error_sweep(ctypes.byref(shape or _shape()), 1, k, pos, T, None, g, out, ws, ws_bytes,
                                         None)
    assert swp(out=None) == 1 and swp(k=None) == 1 and swp(g=3) == 1 and swp(g=256) == 1 and swp(T=-1) == 1
    assert swp(out=ctypes.c_void_p((1 << 20) + 4)) == 2 and swp(k=P2) == 2
    assert swp(shape=_shape(d=96)) == 3
    rc, need = ws_size(lib, "rrp_quant_error_sweep", _shape(), 131072)
    _, one = ws_size(lib, "rrp_quant_error_stats", _shape(), 131072)
    assert rc == 0 and need == 8 * 4096 * 5 * 8                   # b = 1, 2, ..., 128: eight supports
    _, need64 = ws_size(lib, "rrp_quant_error_sweep", _shape(d=64), 131072)
    assert need64 == 7 * 4096 * 5 * 8 and one == 8192 * 5 * 8
    assert swp(T=131072, ws_bytes=need - 8) == 1


def test_binding_rejects_host_tensors_before_any_launch():
    torch = pytest.importorskip("torch")
    import rotation_rope_pair_amd as rrp
    shape = rrp.layer_shape(2, 1, 64, 5e5)
    k = torch.zeros((4, 1, 64), dtype=torch.float32)
    pos = torch.zeros(4, dtype=torch.int32)
    codes = torch.zeros((4, 1, 32), dtype=torch.uint8)
    scales = torch.zeros((4, 1, 1), dtype=torch.float16)
    with pytest.raises(ValueError, match="device"):
        rrp.rotate_quantize_qk(shape, None, k, pos, support_b=64, group=64, k_codes=codes, k_scales=scales)


def test_prepared_call_checks_its_tensors_once_at_preparation():
    """prepare_* runs the binding's tensor checks when it is called (host logic:
    a host tensor is rejected before anything reaches the library)."""
    torch = pytest.importorskip("torch")
    import rotation_rope_pair_amd as rrp
    shape = rrp.layer_shape(4, 1, 64, 10000.0)
    x = torch.zeros(4 * 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="device"):
        rrp.prepare_rotate_quantize_qk(shape, x, x, torch.zeros(1, dtype=torch.int32), support_b=64, group=64,
                                       k_codes=torch.zeros((1, 1, 32), dtype=torch.uint8),
                                       k_scales=torch.zeros(1, dtype=torch.float16))
