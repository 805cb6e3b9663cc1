"""GPU parity on inputs built to drive the online softmax's rare paths: keys
along a ramp so that every 64-key tile raises the running maximum by more
than the lazy-rescale threshold (the reference and O~ are rescaled on every
tile), and the reverse ramp (the first tile holds the maximum, later tiles'
exponentials underflow towards zero).  The oracle sees the same bf16 values.
Every case prints its name first."""
import math
import sys

import numpy as np
import pytest

import oracle
import parity

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


def ramp_inputs(H, N, d, slope, seed):
    """q_i ~ 4u + noise, k_j = slope * j * u + noise, v random (u a unit
    vector): scores grow (slope > 0) or shrink (slope < 0) along the keys by
    about 4 * slope per key."""
    import torch
    g = torch.Generator(device="cpu").manual_seed(seed)
    u = torch.randn(d, generator=g)
    u = u / u.norm()
    q = 4.0 * u + 0.05 * torch.randn(1, H, N, d, generator=g)
    j = torch.arange(N, dtype=torch.float32).view(1, 1, N, 1)
    off = 0.0 if slope > 0 else -slope * (N - 1)  # keep |k| bounded for slope < 0
    k = (slope * j + off) * u + 0.05 * torch.randn(1, H, N, d, generator=g)
    v = torch.randn(1, H, N, d, generator=g)
    return tuple(t.to(torch.bfloat16) for t in (q, k, v))


CASES = [(0.5, True), (0.5, False), (-0.5, False), (-0.5, True)]


@pytest.mark.parametrize("slope,causal", CASES,
                         ids=["up_c", "up", "down", "down_c"])
def test_forward_ramp(fa2, slope, causal):
    import torch
    H, N, d = 2, 1000, 128
    q, k, v = ramp_inputs(H, N, d, slope, seed=61 if slope > 0 else 62)
    scale = 1.0 / math.sqrt(d)
    o_ref, l_ref, _ = oracle.attention(q, k, v, scale, causal)
    dev = torch.device("cuda:0")
    for odt, kind in ((torch.bfloat16, "bf16"), (torch.float32, "fp32")):
        say("ramp slope=%g causal=%s out=%s" % (slope, causal, kind))
        o, lse = fa2.forward(q.to(dev), k.to(dev), v.to(dev), causal=causal, scale=scale,
                             out_dtype=odt)
        torch.cuda.synchronize()
        res = parity.compare(parity.to_np(o.cpu()), o_ref, parity.to_np(lse.cpu()), l_ref, kind)
        assert res["ok"], parity.describe(res)


def test_ramp_drives_a_rescale_every_tile():
    """The inputs above really do what the tests rely on: on the rising ramp
    every 64-key tile's maximum logit (base 2) exceeds the previous tiles'
    by more than 8, for every query row (checked on the CPU)."""
    q, k, _ = ramp_inputs(2, 1000, 128, 0.5, seed=61)
    qd, kd = q.double().numpy(), k.double().numpy()
    c = (1.0 / math.sqrt(128)) * math.log2(math.e)
    s = np.einsum("hid,hjd->hij", qd[0], kd[0]) * c
    tiles = [s[:, :, t:t + 64].max(axis=2) for t in range(0, 1000, 64)]
    for a, b in zip(tiles[:-2], tiles[1:-1]):  # (the ragged last tile aside)
        assert np.all(b - a > 8.0)


def test_backward_ramp(fa2):
    """On the rising ramp P is nearly one-hot, so dS = P (dP - D) is a small
    difference of nearly equal terms, and dQ = scale dS K multiplies it by
    keys of norm up to ~150: the bf16 roundings every such backward makes
    (O, P, dS) cost dQ about 10 % on this input, as the CPU rounding model of
    the kernels shows.  Each gradient must be within the usual bound, or
    within 1.5 times the model's own error on the same input."""
    import torch
    from exact_io_aware_24_amd import inputs as wl
    from test_bwd_tolerance_model import model_grads
    H, N, d = 2, 300, 128
    q, k, v = ramp_inputs(H, N, d, 0.5, seed=63)
    do = wl.make_dout(1, H, N, d, seed=64)
    scale = 1.0 / math.sqrt(d)
    ref = oracle.attention_bwd(q, k, v, do, scale, True)
    model = model_grads(q, k, v, do, scale, True)
    dev = torch.device("cuda:0")
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    say("ramp backward N=%d" % N)
    o, lse = fa2.forward(qd, kd, vd, causal=True, scale=scale)
    grads = fa2.backward(qd, kd, vd, o, dod, lse, causal=True, scale=scale,
                         out_dtype=torch.float32)
    torch.cuda.synchronize()
    for name, g, r, m in zip(("dq", "dk", "dv"), grads, ref[:3], model):
        res = parity.compare_grad(parity.to_np(g.cpu()), r)
        mres = parity.compare_grad(np.asarray(m, dtype=np.float64), r)
        ok = res["finite"] and \
            res["rel_l2"] <= max(parity.GRAD_REL_L2, 1.5 * mres["rel_l2"]) and \
            res["max_rel"] <= max(parity.GRAD_MAX_REL, 1.5 * mres["max_rel"])
        assert ok, "%s: %s (model: %s)" % (name, parity.describe(res), parity.describe(mres))
