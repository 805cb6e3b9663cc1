"""GPU parity of grouped-query / multi-query attention (fa2_fwd_gqa,
fa2_fwd_gqa_o32) against the oracle's definition of grouped K/V heads.
Every case prints its name before touching the GPU."""
import math
import sys

import pytest

import oracle
import parity
from exact_io_aware_24_amd import inputs as wl

pytestmark = pytest.mark.gpu


def say(msg):
    print("[case] " + msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def fa2():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests need an MI355X")
    import exact_io_aware_24_amd as m
    m.lib()
    return m


def run(fa2, q, k, v, causal, scale, out_dtype):
    import torch
    dev = torch.device("cuda:0")
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    o = torch.full(q.shape, float("nan"), dtype=out_dtype, device=dev)
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=dev)
    fa2.forward(qd, kd, vd, causal=causal, scale=scale, out_dtype=out_dtype,
                out=o, lse=lse)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


CASES = [
    # (B, H, H_kv, N, d, causal): groups of 2, 3, 8; MQA; ragged tails
    (1, 4, 2, 128, 128, True), (2, 6, 3, 200, 64, False),
    (1, 8, 1, 257, 128, True), (2, 4, 1, 64, 64, False),
    (1, 16, 2, 1000, 128, True), (3, 2, 1, 77, 128, False),
]


@pytest.mark.parametrize("B,H,Hk,N,d,causal", CASES,
                         ids=["B%dH%dkv%dN%dd%d%s" % (c[0], c[1], c[2], c[3], c[4],
                                                      "c" if c[5] else "")
                              for c in CASES])
def test_gqa_vs_oracle(fa2, B, H, Hk, N, d, causal):
    import torch
    q, k, v = wl.make_inputs(B, H, N, d, "bf16", seed=500 + N, H_kv=Hk)
    scale = 1.0 / math.sqrt(d)
    o_ref, l_ref, _ = oracle.attention_gqa(q, k, v, scale, causal)
    for odt, kind in ((torch.bfloat16, "bf16"), (torch.float32, "fp32")):
        say("gqa B=%d H=%d H_kv=%d N=%d d=%d causal=%s out=%s" % (B, H, Hk, N, d, causal, kind))
        o, lse = run(fa2, q, k, v, causal, scale, odt)
        res = parity.compare(parity.to_np(o), o_ref, parity.to_np(lse), l_ref, kind)
        assert res["ok"], parity.describe(res)


def test_gqa_equals_mha_on_repeated_heads(fa2):
    """The grouped call and the plain call on K/V heads repeated for their
    groups run the same arithmetic: bit-identical outputs."""
    import torch
    B, H, Hk, N, d = 2, 8, 2, 384, 128
    q, k, v = wl.make_inputs(B, H, N, d, "bf16", seed=61, H_kv=Hk)
    kx = k.repeat_interleave(H // Hk, dim=1)
    vx = v.repeat_interleave(H // Hk, dim=1)
    say("gqa vs repeated-head mha")
    a = run(fa2, q, k, v, True, 0.0884, torch.bfloat16)
    b = run(fa2, q, kx, vx, True, 0.0884, torch.bfloat16)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
