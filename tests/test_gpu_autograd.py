"""GPU check of the differentiable wrapper ``attention()``: torch autograd
through the library's forward and backward entry points.  The gradients
that ``loss.backward()`` leaves on q, k and v are compared with the fp64
gradient oracle for the same bf16 inputs and incoming gradient, and bit for
bit with an explicit ``forward`` + ``backward`` call (the wrapper only
marshals arguments); grouped K/V heads included.  Every case prints its
name first."""
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


CASES = [
    # (B, H, H_kv, N, d, causal)
    (1, 2, 2, 300, 128, True),
    (2, 2, 2, 200, 64, False),
    (1, 8, 2, 260, 128, True),
    (2, 8, 2, 100, 64, False),   # short unmasked grouped blocks: packed forward
]


@pytest.mark.parametrize("B,H,Hkv,N,d,causal", CASES,
                         ids=["B%dH%dkv%dN%dd%d%s" % (c[0], c[1], c[2], c[3], c[4],
                                                      "c" if c[5] else "") for c in CASES])
def test_autograd_grads(fa2, B, H, Hkv, N, d, causal):
    import torch
    dev = torch.device("cuda:0")
    q, k, v = wl.make_inputs(B, H, N, d, "bf16", seed=1300 + N, H_kv=Hkv)
    do = wl.make_dout(B, H, N, d, seed=1301 + N)
    scale = 1.0 / math.sqrt(d)
    say("autograd B=%d H=%d H_kv=%d N=%d d=%d causal=%s" % (B, H, Hkv, N, d, causal))
    qd, kd, vd = (t.to(dev).requires_grad_(True) for t in (q, k, v))
    dod = do.to(dev)
    o = fa2.attention(qd, kd, vd, causal=causal)
    # the gradient of sum(o * do) with respect to o is do itself
    (o.float() * dod.float()).sum().backward()
    torch.cuda.synchronize()
    got = [t.grad.cpu() for t in (qd, kd, vd)]
    assert all(g.dtype == torch.bfloat16 for g in got)

    # the same kernels called directly give the same bits
    o2, lse2 = fa2.forward(qd.detach(), kd.detach(), vd.detach(), causal=causal)
    direct = fa2.backward(qd.detach(), kd.detach(), vd.detach(), o2, dod, lse2, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o.detach(), o2)
    for a, b, name in zip(got, direct, ("dq", "dk", "dv")):
        assert torch.equal(a, b.cpu()), "%s differs from the direct call" % name

    if Hkv == H:
        ref = oracle.attention_bwd(q, k, v, do, scale, causal)
    else:
        ref = oracle.attention_bwd_gqa(q, k, v, do, scale, causal)
    for name, g, r in zip(("dq", "dk", "dv"), got, ref[:3]):
        res = parity.compare_grad(parity.to_np(g), r)
        assert res["ok"], "%s: %s" % (name, parity.describe(res))


def test_autograd_rejects_fp32(fa2):
    import torch
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in wl.make_inputs(1, 1, 64, 64, "fp32", seed=1310))
    say("autograd rejects fp32 inputs")
    with pytest.raises(ValueError):
        fa2.attention(q, k, v)
