"""GPU: the binding's argument checks on device tensors, and its stream handling.

A tensor of the wrong dtype, a non-contiguous view or a buffer too small for
the shape is refused with a Python error before anything is enqueued (the
outputs stay as they were).  A call on an explicit torch stream, or on a raw
stream handle, gives the same bits as the call on the current stream.
Workload: the 3B-layer shape (24 Q / 8 KV heads, d 128, bf16), 512 tokens."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import rotation_rope_pair_amd as rrp  # noqa: E402
from rotation_rope_pair_amd import workloads as W  # noqa: E402

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU-only container
    pytest.skip("no GPU", allow_module_level=True)

DEV = torch.device("cuda:0")
T = 512


def bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(torch.bfloat16)


@pytest.fixture(scope="module")
def case():
    w = W.WORKLOADS[3]
    inp = W.make_inputs(3, n_tokens=T)
    shape = rrp.layer_shape(w.n_q_heads, w.n_kv_heads, w.head_dim, w.rope_theta)
    ang = torch.from_numpy(np.random.default_rng(11).uniform(-0.7, 0.7, w.n_pairs).astype(np.float32)).to(DEV)
    return w, shape, bf16(inp["q"]), bf16(inp["k"]), torch.from_numpy(inp["pos"]).to(DEV), ang


def call(w, shape, q, k, pos, ang, stream=None, **over):
    codes, scales = rrp.new_kv4_cache(T, w.n_kv_heads, w.head_dim, 128, DEV)
    args = dict(support_b=128, group=128, k_codes=codes, k_scales=scales, angles=ang, q_out=torch.zeros_like(q))
    args.update(over)
    rrp.rotate_quantize_qk(shape, q, k, pos, stream=stream, **args)
    return args


def test_bad_device_tensors_are_refused_before_any_launch(case):
    w, shape, q, k, pos, ang = case
    codes, scales = rrp.new_kv4_cache(T, w.n_kv_heads, w.head_dim, 128, DEV)
    q_out = torch.zeros_like(q)
    base = dict(support_b=128, group=128, k_codes=codes, k_scales=scales, angles=ang, q_out=q_out)
    bad = [
        (TypeError, "float32 or bfloat16", dict(k=k.to(torch.float16))),
        (TypeError, "pos must have dtype", dict(pos=pos.to(torch.int64))),
        (TypeError, "angles must have dtype", dict(angles=ang.double())),
        (ValueError, "q must be contiguous", dict(q=q.transpose(0, 1).contiguous().transpose(0, 1))),
        (ValueError, "k_codes is smaller", dict(k_codes=codes[: T - 1], n_slots=T)),
        (ValueError, "k_scales holds", dict(k_scales=scales[: T - 1])),
        (ValueError, "q_out holds", dict(q_out=q_out[: T - 1])),
        (ValueError, "device", dict(angles=ang.cpu())),
    ]
    for exc, msg, over in bad:
        a = dict(base, q=q, k=k, pos=pos)
        a.update(over)
        qq, kk, pp = a.pop("q"), a.pop("k"), a.pop("pos")
        with pytest.raises(exc, match=msg):
            rrp.rotate_quantize_qk(shape, qq, kk, pp, **a)
    torch.cuda.synchronize()
    assert int(codes.count_nonzero()) == 0 and int(scales.count_nonzero()) == 0
    assert int(q_out.count_nonzero()) == 0


def test_explicit_and_raw_streams_give_the_same_bits(case):
    w, shape, q, k, pos, ang = case
    ref = call(w, shape, q, k, pos, ang)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    outs = []
    for stream in (side, side.cuda_stream):
        with torch.cuda.stream(side):  # the outputs are allocated on the stream the call uses
            codes, scales = rrp.new_kv4_cache(T, w.n_kv_heads, w.head_dim, 128, DEV)
            q_out = torch.zeros_like(q)
        rrp.rotate_quantize_qk(shape, q, k, pos, support_b=128, group=128, k_codes=codes, k_scales=scales,
                               angles=ang, q_out=q_out, stream=stream)
        outs.append((codes, scales, q_out))
    side.synchronize()
    for codes, scales, q_out in outs:
        assert torch.equal(codes, ref["k_codes"])
        assert torch.equal(scales.view(torch.int16), ref["k_scales"].view(torch.int16))
        assert torch.equal(q_out.view(torch.int16), ref["q_out"].view(torch.int16))
    assert int(ref["k_codes"].count_nonzero()) > 0


def test_int16_scale_views_are_accepted(case):
    """The scale buffer may be given as int16 (the fp16 bits), as the decode
    batch's cache is; the result is the same bits."""
    w, shape, q, k, pos, ang = case
    ref = call(w, shape, q, k, pos, ang)
    codes, scales = rrp.new_kv4_cache(T, w.n_kv_heads, w.head_dim, 128, DEV)
    s16 = scales.view(torch.int16)
    out = call(w, shape, q, k, pos, ang, k_codes=codes, k_scales=s16)
    torch.cuda.synchronize()
    assert torch.equal(out["k_codes"], ref["k_codes"])
    assert torch.equal(s16, ref["k_scales"].view(torch.int16))
