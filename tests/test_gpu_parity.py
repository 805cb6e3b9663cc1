"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle.

Every case prints its name before touching the GPU.  Inputs come from the
seeded generator; the oracle sees exactly the values the GPU sees (bf16 or
fp32, widened to fp64).
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
    m.lib()  # raises if the library is missing: no fallback
    return m


def run(fa2, q, k, v, causal, scale=None, out_dtype=None):
    """Launch on GPU copies of CPU tensors; NaN-poisoned outputs catch any
    element the kernel fails to write.  Returns CPU tensors."""
    import torch
    dev = torch.device("cuda:0")
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    odt = torch.float32 if (q.dtype == torch.float32 or out_dtype == torch.float32) \
        else torch.bfloat16
    o = torch.full(q.shape, float("nan"), dtype=odt, device=dev)
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=dev)
    fa2.forward(qd, kd, vd, causal=causal, scale=scale, out_dtype=out_dtype,
                out=o, lse=lse)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


SMALL = [
    # (B, H, N, d, causal): single rows, below one block, exact blocks,
    # ragged tails, several blocks and tiles
    (1, 1, 1, 64, False), (1, 1, 1, 128, True),
    (1, 2, 37, 64, True), (1, 2, 37, 128, False),
    (2, 3, 128, 128, True), (2, 3, 128, 64, False),
    (1, 2, 200, 64, True), (1, 2, 200, 128, True),
    (2, 2, 300, 128, False), (2, 2, 300, 64, False),
    (1, 2, 513, 128, False), (1, 1, 257, 64, True),
    (1, 1, 1000, 128, True), (1, 1, 1000, 64, True),
    (1, 1, 1024, 128, False), (2, 1, 640, 64, False),
]


@pytest.mark.parametrize("B,H,N,d,causal", SMALL,
                         ids=["B%dH%dN%dd%d%s" % (c[0], c[1], c[2], c[3],
                                                  "c" if c[4] else "")
                              for c in SMALL])
def test_small_bf16_vs_oracle(fa2, B, H, N, d, causal):
    import torch
    q, k, v = wl.make_inputs(B, H, N, d, "bf16", seed=100 + N + d)
    scale = 1.0 / math.sqrt(d)
    o_ref, l_ref, _ = oracle.attention(q, k, v, scale, causal)
    for odt, kind in ((torch.bfloat16, "bf16"), (torch.float32, "fp32")):
        say("small B=%d H=%d N=%d d=%d causal=%s out=%s" % (B, H, N, d, causal, kind))
        o, lse = run(fa2, q, k, v, causal, out_dtype=odt)
        res = parity.compare(parity.to_np(o), o_ref, parity.to_np(lse), l_ref, kind)
        assert res["ok"], parity.describe(res)


@pytest.mark.parametrize("B,H,N,d,causal", [
    (1, 1, 128, 64, False), (1, 1, 128, 128, True), (2, 2, 77, 64, True),
    (1, 3, 300, 128, False), (1, 1, 1, 64, False)])
def test_small_fp32_vs_oracle(fa2, B, H, N, d, causal):
    q, k, v = wl.make_inputs(B, H, N, d, "fp32", seed=7 + N)
    scale = 1.0 / math.sqrt(d)
    say("fp32 B=%d H=%d N=%d d=%d causal=%s" % (B, H, N, d, causal))
    o_ref, l_ref, _ = oracle.attention(q, k, v, scale, causal)
    o, lse = run(fa2, q, k, v, causal)
    res = parity.compare(parity.to_np(o), o_ref, parity.to_np(lse), l_ref, "fp32in")
    assert res["ok"], parity.describe(res)


def test_tiny_exact_workload(fa2):
    """The tiny float32 workload (B=1, H=1, N=128, d=64), every element."""
    w = wl.WORKLOADS["tiny_fp32_n128_d64"]
    q, k, v = wl.workload_inputs(w)
    say("workload " + w.describe())
    o_ref, l_ref, _ = oracle.attention(q, k, v, w.scale, w.causal)
    o, lse = run(fa2, q, k, v, w.causal)
    res = parity.compare(parity.to_np(o), o_ref, parity.to_np(lse), l_ref, "fp32in")
    assert res["ok"], parity.describe(res)


@pytest.mark.parametrize("scale", [0.0, -0.09, 0.5, 3.0])
def test_scale_values(fa2, scale):
    """scale = 0 (uniform attention), negative scales (handled exactly by
    negating q) and large scales, both masks."""
    import torch
    q, k, v = wl.make_inputs(1, 2, 190, 128, "bf16", seed=31)
    for causal in (False, True):
        say("scale=%g causal=%s" % (scale, causal))
        o_ref, l_ref, _ = oracle.attention(q, k, v, scale, causal)
        o, lse = run(fa2, q, k, v, causal, scale=scale, out_dtype=torch.float32)
        res = parity.compare(parity.to_np(o), o_ref, parity.to_np(lse), l_ref, "fp32")
        assert res["ok"], parity.describe(res)


BIG = [n for n, w in wl.WORKLOADS.items()
       if w.dtype == "bf16" and w.q_rows == w.N]


def full_oracle(w, q, k, v):
    """The fp64 oracle over every head of a workload (grouped K/V heads
    expanded by their definition)."""
    if w.kv_heads != w.H:
        return oracle.attention_gqa(q, k, v, w.scale, w.causal)[:2]
    return oracle.attention(q, k, v, w.scale, w.causal)[:2]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", BIG)
def test_full_size_workload(fa2, name):
    """Each bf16 workload at its full size, in the launch configuration the
    benchmark uses, compared with the fp64 oracle element by element over
    the whole output (every head, every row), for both output types;
    rel-L2 is taken over the whole tensor.  A bf16 output is held to the
    literal max-abs 1e-2 except on the x20 outlier workload, whose outputs
    exceed 4 in magnitude, where half a bf16 spacing of the stored value
    alone can exceed it (bound max(1e-2, ulp_bf16(O_ref)))."""
    import time

    import torch
    w = wl.WORKLOADS[name]
    q, k, v = wl.workload_inputs(w)
    say("oracle %s (all heads)" % w.describe())
    t0 = time.time()
    o_ref, l_ref = full_oracle(w, q, k, v)
    say("oracle done in %.1f s" % (time.time() - t0))
    for odt, kind in ((torch.bfloat16, "bf16"), (torch.float32, "fp32")):
        say("workload %s out=%s" % (w.describe(), kind))
        o, lse = run(fa2, q, k, v, w.causal, out_dtype=odt)
        res = parity.compare(parity.to_np(o), o_ref, parity.to_np(lse), l_ref,
                             kind, literal=not w.outliers)
        say("  " + parity.describe(res))
        assert res["ok"], parity.describe(res)
        del o, lse


def test_deterministic(fa2):
    """Repeated launches give bit-identical results (no atomics)."""
    import torch
    w = wl.WORKLOADS[wl.HEADLINE]
    q, k, v = (t.to("cuda:0") for t in wl.workload_inputs(w))
    say("determinism " + w.describe())
    o1, l1 = fa2.forward(q, k, v, causal=True)
    o1, l1 = o1.clone(), l1.clone()
    for _ in range(5):
        o2, l2 = fa2.forward(q, k, v, causal=True)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_causal_last_row_equals_full(fa2):
    """The causal mask hides nothing from the last query row."""
    import torch
    q, k, v = wl.make_inputs(2, 2, 700, 128, "bf16", seed=17)
    say("causal vs full last row")
    oc, lc = run(fa2, q, k, v, True, out_dtype=torch.float32)
    on, ln = run(fa2, q, k, v, False, out_dtype=torch.float32)
    assert torch.allclose(oc[:, :, -1], on[:, :, -1], atol=1e-6, rtol=0)
    assert torch.allclose(lc[:, :, -1], ln[:, :, -1], atol=1e-5, rtol=0)


def test_lse_optional_and_stream(fa2):
    """lse may be omitted; work is enqueued on torch's current stream."""
    import torch
    q, k, v = (t.to("cuda:0") for t in wl.make_inputs(1, 2, 256, 64, "bf16", seed=3))
    say("no lse, side stream")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o, lse = fa2.forward(q, k, v, causal=True, return_lse=False)
    s.synchronize()
    assert lse is None
    o_ref, _ = fa2.forward(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref)
