"""Torch-facing binding of the C-ABI: passes device pointers, sizes and the
current HIP stream.  Every step of the path runs in the HIP kernels; this
module only checks that each tensor is a contiguous device tensor of the size
the kernels will touch, so no launch can read or write outside a buffer.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import torch

from . import _abi
from ._abi import (RRP_BF16, RRP_EST_DEFAULT, RRP_EST_K_ONLY, RRP_EST_STREAM_BALANCED, RRP_F32,
                   RRP_ROPE_HALF_SPLIT, RRP_ROPE_INTERLEAVED, RrpError, RrpShape)

ESTIMATORS = {"default": RRP_EST_DEFAULT, "k_only": RRP_EST_K_ONLY, "stream_balanced": RRP_EST_STREAM_BALANCED}


def layer_shape(n_q_heads: int, n_kv_heads: int, head_dim: int, rope_theta: float,
                rope_layout: int = RRP_ROPE_HALF_SPLIT, angle_heads: int = 0) -> RrpShape:
    """angle_heads: 0 (one angle set shared by all heads) or n_kv_heads (one set
    per key head, query heads using their key head's set)."""
    return RrpShape(int(n_q_heads), int(n_kv_heads), int(head_dim), int(rope_layout), float(rope_theta),
                    int(angle_heads), 0)


def angle_sets(shape: RrpShape) -> int:
    """Angle sets of a layer shape: 1 (shared) or n_kv_heads (per key head)."""
    return shape.angle_heads if shape.angle_heads > 1 else 1


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return RRP_F32
    if t.dtype == torch.bfloat16:
        return RRP_BF16
    raise TypeError(f"Q/K tensors must be float32 or bfloat16, got {t.dtype}")


def _dev(t: Optional[torch.Tensor], name: str, numel: Optional[int] = None, dtype=None, device=None):
    """Device pointer (an int; None for an absent tensor) of `t` after the
    binding's checks: a contiguous device tensor on device ordinal `device`
    with at least `numel` elements of `dtype` (one dtype or a tuple).  The
    checks read only the tensor's own fields, so they cost a few hundred ns."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a device (cuda) tensor")
    where = t.get_device()  # -1 for a host tensor
    if where < 0:
        raise ValueError(f"{name} must be a device (cuda) tensor")
    if device is not None and where != device:
        raise ValueError(f"{name} is on {t.device}, expected cuda:{device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None:
        dt = t.dtype
        if dt is not dtype and (type(dtype) is not tuple or dt not in dtype):
            raise TypeError(f"{name} must have dtype {dtype}, got {dt}")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, needs {numel}")
    return t.data_ptr()


def _device_of(t: torch.Tensor, name: str) -> int:
    """Device ordinal of the tensor that fixes a call's device; a host tensor
    is rejected here, before any workspace is taken."""
    where = t.get_device() if isinstance(t, torch.Tensor) else -1
    if where < 0:
        raise ValueError(f"{name} must be a device (cuda) tensor")
    return where


def _stream_ptr(stream, device: int):
    """Raw hipStream_t of `stream` (a torch stream or a raw handle), else of
    torch's current stream on `device`."""
    if stream is None:
        return torch._C._cuda_getCurrentRawStream(device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _workspace(func, nbytes, workspace, stream, device):
    """(pointer, size) of the device workspace of one call: the caller's
    `workspace` tensor if given (checked for size), else a fresh uint8 tensor
    from torch's caching allocator, tied to the stream the call runs on."""
    if workspace is not None:
        _dev(workspace, "workspace", device=device)
        have = workspace.numel() * workspace.element_size()
        if have < nbytes:
            raise ValueError(f"{func}: workspace holds {have} bytes, needs {nbytes}")
        return workspace.data_ptr(), have
    if nbytes == 0:
        return None, 0
    if stream is not None and not isinstance(stream, torch.cuda.Stream):
        raise ValueError(f"{func}: pass a workspace tensor when the stream is a raw handle")
    ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    if stream is not None and stream != torch.cuda.current_stream(device):
        ws.record_stream(stream)  # not reused by torch before the call's work on `stream` ends
    return ws.data_ptr(), nbytes


def calibrate_workspace_bytes(shape: RrpShape, n_tokens: int, with_q: bool = True) -> int:
    """Device workspace bytes of one calibrate_angles call (rrp_calibrate_angles_workspace_size)."""
    return _abi.workspace_size("rrp_calibrate_angles", shape, int(n_tokens), 1 if with_q else 0)


def quant_error_stats_workspace_bytes(shape: RrpShape, n_tokens: int) -> int:
    """Device workspace bytes of one quant_error_stats call."""
    return _abi.workspace_size("rrp_quant_error_stats", shape, int(n_tokens))


def quant_error_sweep_workspace_bytes(shape: RrpShape, n_tokens: int) -> int:
    """Device workspace bytes of one quant_error_sweep call."""
    return _abi.workspace_size("rrp_quant_error_sweep", shape, int(n_tokens))


def new_kv4_cache(n_slots: int, n_kv_heads: int, head_dim: int, group: int, device="cuda"):
    """Allocate one empty half (K or V) of a KV4 cache: packed codes uint8
    [n_slots][Hkv][d/2] and fp16 scales [n_slots][Hkv][d/group]."""
    codes = torch.zeros((n_slots, n_kv_heads, head_dim // 2), dtype=torch.uint8, device=device)
    scales = torch.zeros((n_slots, n_kv_heads, head_dim // group), dtype=torch.float16, device=device)
    return codes, scales


def new_moments(head_dim: int, device="cuda", n_sets: int = 1) -> torch.Tensor:
    """Zeroed calibration state double[head_dim/2][2][6] (double[n_sets][head_dim/2][2][6]
    for per-key-head angle sets)."""
    shape = (head_dim // 2, 2, 6) if n_sets == 1 else (n_sets, head_dim // 2, 2, 6)
    return torch.zeros(shape, dtype=torch.float64, device=device)


def _rotate_args(shape, q, k, v, pos, support_b, group, k_codes, k_scales, v_codes, v_scales, angles, q_out,
                 slot_mapping, n_slots, q_rot_f32, k_rot_f32, k_scale_f32, v_rot_f32, v_scale_f32, stream):
    d, hq, hk = shape.head_dim, shape.n_q_heads, shape.n_kv_heads
    T = int(pos.numel())
    dt = k.dtype
    dev = _device_of(k, "k")
    if n_slots is None:
        n_slots = int(k_codes.shape[0])
    ng = max(1, d // max(1, int(group)))
    for name, c in (("k_codes", k_codes), ("v_codes", v_codes)):
        if c is not None and n_slots * hk * (d // 2) > c.numel():
            raise ValueError(f"{name} is smaller than n_slots * n_kv_heads * head_dim / 2")
    head = [ctypes.byref(shape), _dtype_code(k),
            _dev(q, "q", T * hq * d, dt, dev), _dev(k, "k", T * hk * d, dt, dev)]
    if v is not None:
        head.append(_dev(v, "v", T * hk * d, dt, dev))
    mid = [_dev(pos, "pos", T, torch.int32, dev), T,
           _dev(angles, "angles", angle_sets(shape) * (d // 2), torch.float32, dev), int(support_b), int(group),
           _dev(q_out, "q_out", T * hq * d, dt, dev),
           _dev(k_codes, "k_codes", n_slots * hk * (d // 2), torch.uint8, dev),
           _dev(k_scales, "k_scales", n_slots * hk * ng, (torch.float16, torch.int16), dev)]
    if v is not None:
        mid += [_dev(v_codes, "v_codes", n_slots * hk * (d // 2), torch.uint8, dev),
                _dev(v_scales, "v_scales", n_slots * hk * ng, (torch.float16, torch.int16), dev)]
    tail = [_dev(slot_mapping, "slot_mapping", T, torch.int64, dev), int(n_slots),
            _dev(q_rot_f32, "q_rot_f32", T * hq * d, torch.float32, dev),
            _dev(k_rot_f32, "k_rot_f32", T * hk * d, torch.float32, dev),
            _dev(k_scale_f32, "k_scale_f32", T * hk * ng, torch.float32, dev)]
    if v is not None:
        tail += [_dev(v_rot_f32, "v_rot_f32", T * hk * d, torch.float32, dev),
                 _dev(v_scale_f32, "v_scale_f32", T * hk * ng, torch.float32, dev)]
    return head + mid + tail + [_stream_ptr(stream, dev)]


def rotate_quantize_qk(shape: RrpShape, q: Optional[torch.Tensor], k: torch.Tensor, pos: torch.Tensor, *,
                       support_b: int, group: int, k_codes: torch.Tensor, k_scales: torch.Tensor,
                       angles: Optional[torch.Tensor] = None, q_out: Optional[torch.Tensor] = None,
                       slot_mapping: Optional[torch.Tensor] = None, n_slots: Optional[int] = None,
                       q_rot_f32: Optional[torch.Tensor] = None, k_rot_f32: Optional[torch.Tensor] = None,
                       k_scale_f32: Optional[torch.Tensor] = None, stream=None) -> None:
    """Enqueue rrp_rotate_quantize_qk (see include/rrp.h)."""
    L = _abi.load()
    args = _rotate_args(shape, q, k, None, pos, support_b, group, k_codes, k_scales, None, None, angles, q_out,
                        slot_mapping, n_slots, q_rot_f32, k_rot_f32, k_scale_f32, None, None, stream)
    _abi.check("rrp_rotate_quantize_qk", L.rrp_rotate_quantize_qk(*args))


def rotate_quantize_qkv(shape: RrpShape, q: Optional[torch.Tensor], k: torch.Tensor, v: torch.Tensor,
                        pos: torch.Tensor, *, support_b: int, group: int, k_codes: torch.Tensor,
                        k_scales: torch.Tensor, v_codes: torch.Tensor, v_scales: torch.Tensor,
                        angles: Optional[torch.Tensor] = None, q_out: Optional[torch.Tensor] = None,
                        slot_mapping: Optional[torch.Tensor] = None, n_slots: Optional[int] = None,
                        q_rot_f32: Optional[torch.Tensor] = None, k_rot_f32: Optional[torch.Tensor] = None,
                        k_scale_f32: Optional[torch.Tensor] = None, v_rot_f32: Optional[torch.Tensor] = None,
                        v_scale_f32: Optional[torch.Tensor] = None, stream=None) -> None:
    """Enqueue rrp_rotate_quantize_qkv: the Q/K path plus the V half of the KV4
    cache in one launch (see include/rrp.h)."""
    L = _abi.load()
    if v is None or v_codes is None or v_scales is None:
        raise ValueError("rotate_quantize_qkv needs v, v_codes and v_scales")
    if v.dtype != k.dtype:
        raise TypeError("v must have the dtype of k")
    args = _rotate_args(shape, q, k, v, pos, support_b, group, k_codes, k_scales, v_codes, v_scales, angles, q_out,
                        slot_mapping, n_slots, q_rot_f32, k_rot_f32, k_scale_f32, v_rot_f32, v_scale_f32, stream)
    _abi.check("rrp_rotate_quantize_qkv", L.rrp_rotate_quantize_qkv(*args))


def calibrate_angles(shape: RrpShape, q: Optional[torch.Tensor], k: torch.Tensor, pos: torch.Tensor, *,
                     moments: torch.Tensor, estimator="default", angles_out: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """Enqueue rrp_calibrate_angles: accumulate pair moments into `moments` and,
    if angles_out is given, finalise the shared angles (see include/rrp.h).
    workspace: optional device tensor of at least calibrate_workspace_bytes()
    bytes; by default one is taken from torch's caching allocator."""
    L = _abi.load()
    est = ESTIMATORS[estimator] if isinstance(estimator, str) else int(estimator)
    d, hq, hk = shape.head_dim, shape.n_q_heads, shape.n_kv_heads
    T = int(pos.numel())
    dt, dev = k.dtype, _device_of(k, "k")
    ws, ws_bytes = _workspace("rrp_calibrate_angles", calibrate_workspace_bytes(shape, T, q is not None), workspace,
                              stream, dev)
    args = [
        ctypes.byref(shape), _dtype_code(k),
        _dev(q, "q", T * hq * d, dt, dev), _dev(k, "k", T * hk * d, dt, dev),
        _dev(pos, "pos", T, torch.int32, dev), T, est,
        _dev(moments, "moments", angle_sets(shape) * (d // 2) * 12, torch.float64, dev),
        _dev(angles_out, "angles_out", angle_sets(shape) * (d // 2), torch.float32, dev),
        ws, ws_bytes, _stream_ptr(stream, dev),
    ]
    _abi.check("rrp_calibrate_angles", L.rrp_calibrate_angles(*args))


def calibrate_angles_noalloc(shape: RrpShape, q: Optional[torch.Tensor], k: torch.Tensor, pos: torch.Tensor, *,
                             moments: torch.Tensor, estimator="default", angles_out: Optional[torch.Tensor] = None,
                             stream=None) -> None:
    """Enqueue rrp_calibrate_angles_noalloc: calibrate_angles with no device
    allocation at all (the library's static scratch holds the partials).  Calls
    that overlap on one GPU race (see include/rrp.h)."""
    L = _abi.load()
    est = ESTIMATORS[estimator] if isinstance(estimator, str) else int(estimator)
    d, hq, hk = shape.head_dim, shape.n_q_heads, shape.n_kv_heads
    T = int(pos.numel())
    dt, dev = k.dtype, _device_of(k, "k")
    args = [
        ctypes.byref(shape), _dtype_code(k),
        _dev(q, "q", T * hq * d, dt, dev), _dev(k, "k", T * hk * d, dt, dev),
        _dev(pos, "pos", T, torch.int32, dev), T, est,
        _dev(moments, "moments", angle_sets(shape) * (d // 2) * 12, torch.float64, dev),
        _dev(angles_out, "angles_out", angle_sets(shape) * (d // 2), torch.float32, dev),
        _stream_ptr(stream, dev),
    ]
    _abi.check("rrp_calibrate_angles_noalloc", L.rrp_calibrate_angles_noalloc(*args))


def quant_error_stats(shape: RrpShape, k: torch.Tensor, pos: torch.Tensor, *, support_b: int, group: int,
                      stats_out: torch.Tensor, angles: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """Enqueue rrp_quant_error_stats into stats_out (double[8], see include/rrp.h).
    workspace: as for calibrate_angles (quant_error_stats_workspace_bytes())."""
    L = _abi.load()
    d, hk = shape.head_dim, shape.n_kv_heads
    T = int(pos.numel())
    dt, dev = k.dtype, _device_of(k, "k")
    ws, ws_bytes = _workspace("rrp_quant_error_stats", quant_error_stats_workspace_bytes(shape, T), workspace,
                              stream, dev)
    args = [
        ctypes.byref(shape), _dtype_code(k), _dev(k, "k", T * hk * d, dt, dev),
        _dev(pos, "pos", T, torch.int32, dev), T,
        _dev(angles, "angles", angle_sets(shape) * (d // 2), torch.float32, dev), int(support_b), int(group),
        _dev(stats_out, "stats_out", 8, torch.float64, dev), ws, ws_bytes, _stream_ptr(stream, dev),
    ]
    _abi.check("rrp_quant_error_stats", L.rrp_quant_error_stats(*args))


def sweep_supports(head_dim: int):
    """The supports b = 1, 2, 4, ..., head_dim covered by quant_error_sweep (row order)."""
    out, b = [], 1
    while b <= head_dim:
        out.append(b)
        b <<= 1
    return out


def quant_error_sweep(shape: RrpShape, k: torch.Tensor, pos: torch.Tensor, *, group: int, stats_out: torch.Tensor,
                      angles: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                      stream=None) -> None:
    """Enqueue rrp_quant_error_sweep: the statistics of quant_error_stats for every
    support b = 1, 2, 4, ..., head_dim into stats_out double[len(supports)][8]
    (see include/rrp.h).  workspace: as for calibrate_angles
    (quant_error_sweep_workspace_bytes())."""
    L = _abi.load()
    d, hk = shape.head_dim, shape.n_kv_heads
    T = int(pos.numel())
    dt, dev = k.dtype, _device_of(k, "k")
    ws, ws_bytes = _workspace("rrp_quant_error_sweep", quant_error_sweep_workspace_bytes(shape, T), workspace,
                              stream, dev)
    args = [
        ctypes.byref(shape), _dtype_code(k), _dev(k, "k", T * hk * d, dt, dev),
        _dev(pos, "pos", T, torch.int32, dev), T,
        _dev(angles, "angles", angle_sets(shape) * (d // 2), torch.float32, dev), int(group),
        _dev(stats_out, "stats_out", 8 * len(sweep_supports(d)), torch.float64, dev), ws, ws_bytes,
        _stream_ptr(stream, dev),
    ]
    _abi.check("rrp_quant_error_sweep", L.rrp_quant_error_sweep(*args))


def _decode_args(shape, q, k_codes, k_scales, group, seq_start, seq_len, max_len, scores, n_slots, stream):
    d, hq, hk = shape.head_dim, shape.n_q_heads, shape.n_kv_heads
    B = int(seq_len.numel())
    dev = _device_of(q, "q")
    if n_slots is None:
        n_slots = int(k_codes.shape[0])
    ng = max(1, d // max(1, int(group)))
    args = [
        ctypes.byref(shape), _dtype_code(q), _dev(q, "q", B * hq * d, q.dtype, dev), B,
        _dev(k_codes, "k_codes", n_slots * hk * (d // 2), torch.uint8, dev),
        _dev(k_scales, "k_scales", n_slots * hk * ng, (torch.float16, torch.int16), dev), int(group), int(n_slots),
        _dev(seq_start, "seq_start", B, torch.int64, dev), _dev(seq_len, "seq_len", B, torch.int32, dev),
        int(max_len), _dev(scores, "scores", B * hq * int(max_len), torch.float32, dev), _stream_ptr(stream, dev),
    ]
    return args


def decode_scores(shape: RrpShape, q: torch.Tensor, k_codes: torch.Tensor, k_scales: torch.Tensor, *, group: int,
                  seq_start: torch.Tensor, seq_len: torch.Tensor, max_len: int, scores: torch.Tensor,
                  n_slots: Optional[int] = None, stream=None) -> None:
    """Enqueue rrp_decode_scores: decode logits of the rotated queries q
    [n_seqs][Hq][d] against the KV4 cache into scores fp32 [n_seqs][Hq][max_len]
    (see include/rrp.h)."""
    L = _abi.load()
    args = _decode_args(shape, q, k_codes, k_scales, group, seq_start, seq_len, max_len, scores, n_slots, stream)
    _abi.check("rrp_decode_scores", L.rrp_decode_scores(*args))


class PreparedCall:
    """One C-ABI call whose tensors were checked and whose arguments were
    marshalled once (by a prepare_* function): calling it enqueues the same
    launch again, on the same tensors and stream, with no per-call Python
    checks.  For loops that reuse fixed buffers (a decode step's queries,
    positions, slot mapping and cache), whose contents may change between
    calls.  The object holds references to the tensors and the shape, so their
    storage stays alive; a tensor that is resized or replaced needs a new
    prepared call.  The C entry point still validates its scalar arguments."""
    __slots__ = ("_name", "_fn", "_args", "_keep")

    def __init__(self, name, fn, args, keep):
        self._name, self._fn, self._args, self._keep = name, fn, tuple(args), keep

    def __call__(self) -> None:
        status = self._fn(*self._args)
        if status != _abi.RRP_OK:
            _abi.check(self._name, status)


def prepare_rotate_quantize_qk(shape: RrpShape, q: Optional[torch.Tensor], k: torch.Tensor, pos: torch.Tensor, *,
                               support_b: int, group: int, k_codes: torch.Tensor, k_scales: torch.Tensor,
                               angles: Optional[torch.Tensor] = None, q_out: Optional[torch.Tensor] = None,
                               slot_mapping: Optional[torch.Tensor] = None, n_slots: Optional[int] = None,
                               stream=None) -> PreparedCall:
    """rotate_quantize_qk checked and marshalled once (see PreparedCall); the
    stream is the one given, else the current stream at preparation."""
    L = _abi.load()
    args = _rotate_args(shape, q, k, None, pos, support_b, group, k_codes, k_scales, None, None, angles, q_out,
                        slot_mapping, n_slots, None, None, None, None, None, stream)
    keep = (shape, q, k, pos, angles, q_out, k_codes, k_scales, slot_mapping, stream)
    return PreparedCall("rrp_rotate_quantize_qk", L.rrp_rotate_quantize_qk, args, keep)


def prepare_decode_scores(shape: RrpShape, q: torch.Tensor, k_codes: torch.Tensor, k_scales: torch.Tensor, *,
                          group: int, seq_start: torch.Tensor, seq_len: torch.Tensor, max_len: int,
                          scores: torch.Tensor, n_slots: Optional[int] = None, stream=None) -> PreparedCall:
    """decode_scores checked and marshalled once (see PreparedCall)."""
    L = _abi.load()
    args = _decode_args(shape, q, k_codes, k_scales, group, seq_start, seq_len, max_len, scores, n_slots, stream)
    keep = (shape, q, k_codes, k_scales, seq_start, seq_len, scores, stream)
    return PreparedCall("rrp_decode_scores", L.rrp_decode_scores, args, keep)


__all__ = ["layer_shape", "angle_sets", "calibrate_angles_noalloc", "calibrate_workspace_bytes",
           "quant_error_stats_workspace_bytes", "PreparedCall", "prepare_rotate_quantize_qk", "prepare_decode_scores",
           "quant_error_sweep_workspace_bytes", "decode_scores", "quant_error_sweep", "sweep_supports",
           "rotate_quantize_qk", "rotate_quantize_qkv", "calibrate_angles", "quant_error_stats", "new_kv4_cache",
           "new_moments", "RrpError", "RrpShape", "ESTIMATORS", "RRP_F32", "RRP_BF16", "RRP_ROPE_HALF_SPLIT",
           "RRP_ROPE_INTERLEAVED"]
