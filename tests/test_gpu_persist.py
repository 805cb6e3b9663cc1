"""GPU checks of the forward's persistent mode (d = 128, causal, at most 64
query blocks per head, equal query and key lengths, whole key tiles, more
work items than two per compute unit): the
grid walks the items and issues each item's first loads during the last
tile of the item before.  Every item is computed exactly as when a
workgroup takes it alone, so a call that walks must agree bit for bit with
calls on single heads (few items: one workgroup each); a few heads are also
compared with the fp64 oracle.  Every case prints its name first."""
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


def heads_for(n, extra):
    """Query heads that give more than two items per compute unit."""
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    blocks = (n + 127) // 128
    return (2 * cus) // blocks + 1 + extra


CASES = [
    # (N, causal, scale, group, extra heads): last block of 64 rows and an
    # odd tile count (the next item's V issued after the last tile), whole
    # blocks with an even count (V issued during it), a negative scale,
    # grouped K/V heads, items just above the grid, and two launches that
    # do not walk (no mask; 65 query blocks per head)
    (1600, True, None, 1, 7),
    (1664, True, None, 1, 0),
    (1088, True, -0.1, 1, 3),
    (1088, True, None, 4, 5),
    (2048, False, None, 2, 1),
    (8320, True, None, 1, 0),
]


@pytest.mark.parametrize("N,causal,scale,group,extra", CASES,
                         ids=["N%d%s%sg%d" % (c[0], "c" if c[1] else "",
                                              "neg" if c[2] else "", c[3]) for c in CASES])
def test_walk_equals_single_heads(fa2, N, causal, scale, group, extra):
    import torch
    d = 128
    H = -(-heads_for(N, extra) // group) * group  # a multiple of the group
    Hk = H // group
    sc = 1.0 / math.sqrt(d) if scale is None else scale
    q, k, v = wl.make_inputs(1, H, N, d, "bf16", seed=880 + N + group, H_kv=Hk)
    dev = torch.device("cuda:0")
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    say("persistent walk N=%d H=%d H_kv=%d causal=%s scale=%g" % (N, H, Hk, causal, sc))
    for odt in (torch.bfloat16, torch.float32):
        o = torch.full(qd.shape, float("nan"), dtype=odt, device=dev)
        lse = torch.full(qd.shape[:3], float("nan"), dtype=torch.float32, device=dev)
        fa2.forward(qd, kd, vd, causal=causal, scale=sc, out_dtype=odt, out=o, lse=lse)
        torch.cuda.synchronize()
        for h in range(H):
            o1, l1 = fa2.forward(qd[:, h:h + 1].contiguous(),
                                 kd[:, h // group:h // group + 1].contiguous(),
                                 vd[:, h // group:h // group + 1].contiguous(),
                                 causal=causal, scale=sc, out_dtype=odt)
            torch.cuda.synchronize()
            assert torch.equal(o[:, h:h + 1], o1) and torch.equal(lse[:, h:h + 1], l1), \
                "head %d differs from its single-head call (%s)" % (h, odt)
    # absolute check of three heads against the oracle
    kind = "fp32"
    for h in (0, H // 2, H - 1):
        o_ref, l_ref, _ = oracle.attention(q[0, h], k[0, h // group], v[0, h // group], sc, causal)
        res = parity.compare(parity.to_np(o[0, h].cpu()), o_ref,
                             parity.to_np(lse[0, h].cpu()), l_ref, kind)
        assert res["ok"], "head %d: %s" % (h, parity.describe(res))


def test_walk_repeatable(fa2):
    """Two calls of a walking launch give identical bits."""
    import torch
    N = 1024
    H = heads_for(N, 9)
    q, k, v = wl.make_inputs(1, H, N, 128, "bf16", seed=881)
    dev = torch.device("cuda:0")
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    say("persistent walk repeatable H=%d N=%d" % (H, N))
    a = fa2.forward(qd, kd, vd, causal=True)
    b = fa2.forward(qd, kd, vd, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    assert bool(np.isfinite(a[1].cpu().numpy()).all())
