"""GPU parity of the backward pass (fa2_bwd, fa2_bwd_o32) against the fp64
gradient oracle.

The GPU forward produces O and lse, the GPU backward the gradients; the
oracle differentiates the exact definition from the same bf16 q, k, v and
dO.  Every case prints its name before touching the GPU; outputs start
NaN-poisoned so that an unwritten element fails.
"""
import math
import sys

import numpy as np
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


def run_bwd(fa2, q, k, v, do, causal, scale, out_dtype=None):
    """Forward then backward on the GPU; returns CPU (dq, dk, dv, delta)."""
    import torch
    dev = torch.device("cuda:0")
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    o, lse = fa2.forward(qd, kd, vd, causal=causal, scale=scale)
    odt = torch.bfloat16 if out_dtype is None else out_dtype
    grads = [torch.full(q.shape, float("nan"), dtype=odt, device=dev) for _ in range(3)]
    delta = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=dev)
    fa2.backward(qd, kd, vd, o, dod, lse, causal=causal, scale=scale,
                 out_dtype=out_dtype, dq=grads[0], dk=grads[1], dv=grads[2],
                 delta=delta)
    torch.cuda.synchronize()
    return [g.cpu() for g in grads] + [delta.cpu()]


def check(got, ref, heavy=False, what=""):
    for name, g, r in zip(("dq", "dk", "dv"), got[:3], ref[:3]):
        res = parity.compare_grad(parity.to_np(g), r, heavy=heavy)
        assert res["ok"], "%s %s: %s" % (what, name, parity.describe(res))


SMALL = [
    # (B, H, N, d, causal): a single row, below one tile, exact blocks,
    # ragged tails, several blocks
    (1, 1, 1, 64, True), (1, 1, 1, 128, False),
    (1, 2, 37, 64, True), (1, 2, 37, 128, False),
    (2, 2, 128, 128, True), (2, 2, 128, 64, False),
    (1, 2, 200, 128, True), (1, 2, 200, 64, False),
    (1, 3, 320, 64, True), (2, 1, 384, 128, False),
    (1, 1, 513, 128, True), (1, 2, 700, 64, True),
]


@pytest.mark.parametrize("B,H,N,d,causal", SMALL,
                         ids=["B%dH%dN%dd%d%s" % (c[0], c[1], c[2], c[3],
                                                  "c" if c[4] else "")
                              for c in SMALL])
def test_small_grads_vs_oracle(fa2, B, H, N, d, causal):
    import torch
    q, k, v = wl.make_inputs(B, H, N, d, "bf16", seed=300 + N + d)
    do = wl.make_dout(B, H, N, d, seed=301 + N + d)
    scale = 1.0 / math.sqrt(d)
    ref = oracle.attention_bwd(q, k, v, do, scale, causal)
    for odt, kind in ((torch.bfloat16, "bf16"), (torch.float32, "fp32")):
        say("bwd small B=%d H=%d N=%d d=%d causal=%s out=%s" % (B, H, N, d, causal, kind))
        got = run_bwd(fa2, q, k, v, do, causal, scale, out_dtype=odt)
        check(got, ref, what="B%dH%dN%dd%d %s" % (B, H, N, d, kind))
        # D_i = dO_i . O_i of the bf16 forward output: close to the exact D
        dl = parity.to_np(got[3])
        assert np.all(np.isfinite(dl))
        assert np.max(np.abs(dl - ref[3])) <= 2e-2 * max(1.0, np.abs(ref[3]).max())


@pytest.mark.parametrize("scale", [0.0, -0.09, 0.3])
def test_scale_values(fa2, scale):
    q, k, v = wl.make_inputs(1, 2, 190, 128, "bf16", seed=77)
    do = wl.make_dout(1, 2, 190, 128, seed=78)
    say("bwd scale=%g" % scale)
    ref = oracle.attention_bwd(q, k, v, do, scale, True)
    got = run_bwd(fa2, q, k, v, do, True, scale)
    if scale == 0.0:
        # dQ = dK = 0 exactly; dV is the closed form of uniform attention
        assert float(got[0].abs().max()) == 0.0 and float(got[1].abs().max()) == 0.0
        res = parity.compare_grad(parity.to_np(got[2]), ref[2])
        assert res["ok"], parity.describe(res)
    else:
        check(got, ref, what="scale %g" % scale)


FULL = ["train_b8h16_n2048_d64", "causal_b2h16_n8192_d128",
        "outlier_b4h32_n4096_d128"]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", FULL)
def test_full_size_workload(fa2, name):
    """The workload at its full size on the GPU; every gradient element of
    every head compared with the oracle's backward: rel-L2 and max-abs over
    the whole tensors, and the same bounds within each head."""
    import time
    w = wl.WORKLOADS[name]
    q, k, v = wl.workload_inputs(w)
    do = wl.make_dout(w.B, w.H, w.N, w.d)
    say("bwd full %s" % name)
    got = run_bwd(fa2, q, k, v, do, w.causal, w.scale)
    for g in got:
        assert bool(g.isfinite().all()), name
    say("bwd oracle %s (all heads)" % name)
    t0 = time.time()
    ref = oracle.attention_bwd(q, k, v, do, w.scale, w.causal)
    say("bwd oracle done in %.1f s" % (time.time() - t0))
    for gname, g, r in zip(("dq", "dk", "dv"), got[:3], ref[:3]):
        gn = parity.to_np(g)
        res = parity.compare_grad(gn, r, heavy=w.outliers)
        say("  %s whole tensor: %s" % (gname, parity.describe(res)))
        assert res["ok"], "%s %s: %s" % (name, gname, parity.describe(res))
        gh = gn.reshape(w.B * w.H, w.N, w.d)
        rh = r.reshape(w.B * w.H, w.N, w.d)
        worst = None
        for h in range(w.B * w.H):
            rs = parity.compare_grad(gh[h], rh[h], heavy=w.outliers)
            assert rs["ok"], "%s %s head %d: %s" % (name, gname, h, parity.describe(rs))
            if worst is None or rs["rel_l2"] > worst["rel_l2"]:
                worst = rs
        say("  %s worst head: %s" % (gname, parity.describe(worst)))


def test_deterministic(fa2):
    import torch
    q, k, v = wl.make_inputs(2, 4, 1024, 128, "bf16", seed=9)
    do = wl.make_dout(2, 4, 1024, 128, seed=10)
    say("bwd determinism")
    a = run_bwd(fa2, q, k, v, do, True, 0.0884)
    b = run_bwd(fa2, q, k, v, do, True, 0.0884)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
