"""GPU check of causal tile skipping.  With FA2_DEBUG_NO_SKIP=1 in the
environment the bf16 forward kernels run every key tile for causal query
blocks, the tiles past a block's diagonal through the masked path, where
every score is hidden: their probabilities are exactly zero and add nothing
to l, to the rounded normaliser or to O~.  Skipping those tiles (the normal
path) must therefore give the same bits.  Cases cover the persistent walk,
a ragged key end, d = 64, grouped K/V heads and split key ranges with fewer
queries than keys; one case is also held against the fp64 oracle.  Every
case prints its name first."""
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
    # (name, B, H, H_kv, Nq, Nk, d, n_splits): n_splits None = fa2.forward
    ("walk", 1, 40, 40, 2048, 2048, 128, None),  # 640 items: the grid walks
    ("ragged", 1, 3, 3, 1000, 1000, 128, None),
    ("d64", 2, 3, 3, 777, 777, 64, None),
    ("gqa", 1, 8, 2, 1100, 1100, 128, None),
    ("splitkv", 1, 4, 2, 300, 1500, 128, 3),
    ("splitkv_d64", 1, 2, 2, 129, 700, 64, 4),
]


def run(fa2, qd, kd, vd, n_splits, odt):
    import torch
    if n_splits is None:
        o, lse = fa2.forward(qd, kd, vd, causal=True, out_dtype=odt)
    else:
        o, lse = fa2.forward_splitkv(qd, kd, vd, causal=True, n_splits=n_splits,
                                     out_dtype=odt)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("name,B,H,Hkv,Nq,Nk,d,n_splits", CASES, ids=[c[0] for c in CASES])
def test_no_skip_same_bits(fa2, monkeypatch, name, B, H, Hkv, Nq, Nk, d, n_splits):
    import torch
    q, k, v = wl.make_inputs(B, H, Nk, d, "bf16", seed=930 + Nq + d, H_kv=Hkv, Nq=Nq)
    dev = torch.device("cuda:0")
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    for odt in (torch.bfloat16, torch.float32):
        say("no-skip %s B=%d H=%d H_kv=%d Nq=%d Nk=%d d=%d splits=%s out=%s"
            % (name, B, H, Hkv, Nq, Nk, d, n_splits, odt))
        monkeypatch.delenv("FA2_DEBUG_NO_SKIP", raising=False)
        o1, l1 = run(fa2, qd, kd, vd, n_splits, odt)
        monkeypatch.setenv("FA2_DEBUG_NO_SKIP", "1")
        o2, l2 = run(fa2, qd, kd, vd, n_splits, odt)
        monkeypatch.delenv("FA2_DEBUG_NO_SKIP")
        assert torch.equal(o1, o2), "O differs with tile skipping off (%s)" % odt
        assert torch.equal(l1, l2), "lse differs with tile skipping off (%s)" % odt


def test_no_skip_matches_oracle(fa2, monkeypatch):
    """The unskipped path on its own, against the fp64 oracle (two heads)."""
    import torch
    B, H, N, d = 1, 2, 700, 128
    q, k, v = wl.make_inputs(B, H, N, d, "bf16", seed=939)
    dev = torch.device("cuda:0")
    monkeypatch.setenv("FA2_DEBUG_NO_SKIP", "1")
    say("no-skip against the oracle N=%d d=%d" % (N, d))
    o, lse = fa2.forward(q.to(dev), k.to(dev), v.to(dev), causal=True,
                         out_dtype=torch.float32)
    torch.cuda.synchronize()
    scale = 1.0 / math.sqrt(d)
    for h in range(H):
        o_ref, l_ref, _ = oracle.attention(q[0, h], k[0, h], v[0, h], scale, True)
        res = parity.compare(parity.to_np(o[0, h].cpu()), o_ref,
                             parity.to_np(lse[0, h].cpu()), l_ref, "fp32")
        assert res["ok"], "head %d: %s" % (h, parity.describe(res))
