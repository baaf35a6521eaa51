"""GPU: the binding's prepared calls (arguments checked and marshalled once,
then re-issued) give bit-identical results to the plain binding calls, also
after the input tensors' contents change in place between calls.  Workload:
the 256-sequence decode batch (rotate + scatter into a 256 x 32768-slot KV4
cache, then decode logits over the full cache)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import rotation_rope_pair_amd as rrp  # noqa: E402
from rotation_rope_pair_amd import workloads as W  # noqa: E402

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU-only container
    pytest.skip("no GPU", allow_module_level=True)

DEV = torch.device("cuda:0")


def bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(torch.bfloat16)


def test_prepared_rotate_equals_plain_call_after_inputs_change():
    w = W.WORKLOADS[5]
    inp = W.make_inputs(5)
    shape = rrp.layer_shape(w.n_q_heads, w.n_kv_heads, w.head_dim, w.rope_theta)
    q, k = bf16(inp["q"]), bf16(inp["k"])
    pos = torch.from_numpy(inp["pos"]).to(DEV)
    sm = torch.from_numpy(inp["slot_mapping"]).to(DEV)
    n_slots = inp["n_slots"]
    ang = torch.from_numpy(np.random.default_rng(7).uniform(-0.7, 0.7, w.n_pairs).astype(np.float32)).to(DEV)

    def fresh():
        c, s = rrp.new_kv4_cache(n_slots, w.n_kv_heads, w.head_dim, w.group, DEV)
        return c, s, torch.empty_like(q)

    c0, s0, q0 = fresh()
    c1, s1, q1 = fresh()
    prep = rrp.prepare_rotate_quantize_qk(shape, q, k, pos, support_b=128, group=w.group, k_codes=c1, k_scales=s1,
                                          angles=ang, q_out=q1, slot_mapping=sm, n_slots=n_slots)
    for step in range(3):
        if step:  # new contents in the same tensors: the next decode step's tokens
            g = torch.Generator(device="cpu").manual_seed(100 + step)
            q.copy_(torch.randn(q.shape, generator=g).to(torch.bfloat16))
            k.copy_(torch.randn(k.shape, generator=g).to(torch.bfloat16))
            pos.add_(1)
            ang.mul_(-0.5)
        rrp.rotate_quantize_qk(shape, q, k, pos, support_b=128, group=w.group, k_codes=c0, k_scales=s0, angles=ang,
                               q_out=q0, slot_mapping=sm, n_slots=n_slots)
        prep()
        torch.cuda.synchronize()
        assert torch.equal(q0.view(torch.int16), q1.view(torch.int16)), step
        assert torch.equal(c0, c1) and torch.equal(s0, s1), step


def test_prepared_decode_scores_equals_plain_call():
    w = W.WORKLOADS[5]
    bt = W.make_decode_batch(5)
    shape = rrp.layer_shape(w.n_q_heads, w.n_kv_heads, w.head_dim, w.rope_theta)
    q = bf16(bt["q"])
    codes = torch.from_numpy(bt["codes"]).to(DEV)
    scales = torch.from_numpy(bt["scales"].view(np.int16)).to(DEV)
    start = torch.from_numpy(bt["seq_start"]).to(DEV)
    lens = torch.from_numpy(bt["seq_len"]).to(DEV)
    B, L = len(bt["seq_len"]), bt["max_len"]
    a = torch.full((B, w.n_q_heads, L), float("nan"), dtype=torch.float32, device=DEV)
    b = torch.full_like(a, float("nan"))
    prep = rrp.prepare_decode_scores(shape, q, codes, scales, group=bt["group"], seq_start=start, seq_len=lens,
                                     max_len=L, scores=b)
    for step in range(2):
        if step:
            lens.sub_(7).clamp_(min=0)
            q.mul_(-2.0)
        rrp.decode_scores(shape, q, codes, scales, group=bt["group"], seq_start=start, seq_len=lens, max_len=L,
                          scores=a)
        prep()
        torch.cuda.synchronize()
        assert torch.equal(torch.nan_to_num(a, nan=1e30), torch.nan_to_num(b, nan=1e30)), step
