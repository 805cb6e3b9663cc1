"""GPU parity at the largest sizes: a million keys per head, near the top of
the range the kernels' 32-bit per-head offsets cover (N*d*2 bytes < 2^31).
Rows are compared one by one against the fp64 oracle (first, last, tile and
block boundaries, random), and every output must be finite.  Every case
prints its name first."""
import math
import sys

import numpy as np
import pytest

import oracle
import parity
from exact_io_aware_24_amd import inputs as wl

pytestmark = pytest.mark.gpu

N_BIG = 1 << 20


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


def rows_to_check(n, seed):
    rng = np.random.default_rng(seed)
    rows = set(range(4)) | set(range(n - 4, n))
    for b in (63, 64, 127, 128, n // 2, n // 2 + 1):
        rows.add(b)
    rows |= set(int(x) for x in rng.choice(n, size=8, replace=False))
    return np.array(sorted(rows), dtype=np.int64)


@pytest.mark.parametrize("causal", [True, False])
def test_forward_million_keys(fa2, causal):
    import torch
    d = 128
    q, k, v = wl.make_inputs(1, 1, N_BIG, d, "bf16", seed=4242)
    scale = 1.0 / math.sqrt(d)
    dev = torch.device("cuda:0")
    say("forward B=1 H=1 N=%d d=%d causal=%s" % (N_BIG, d, causal))
    o, lse = fa2.forward(q.to(dev), k.to(dev), v.to(dev), causal=causal, scale=scale,
                         out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
    rows = rows_to_check(N_BIG, 7)
    o_ref, l_ref, _ = oracle.attention_rows(q[0, 0][rows], rows, k[0, 0], v[0, 0], scale, causal)
    res = parity.compare(parity.to_np(o[0, 0][rows].cpu()), o_ref,
                         parity.to_np(lse[0, 0][rows].cpu()), l_ref, "fp32")
    assert res["ok"], parity.describe(res)


def test_decode_million_keys(fa2):
    """One query per head against a million keys shared by four query heads
    (multi-query), the key range split with the default count."""
    import torch
    d, H = 128, 4
    q, k, v = wl.make_inputs(1, H, N_BIG, d, "bf16", seed=4343, H_kv=1, Nq=1)
    scale = 1.0 / math.sqrt(d)
    dev = torch.device("cuda:0")
    say("decode B=1 H=%d H_kv=1 Nq=1 Nk=%d d=%d" % (H, N_BIG, d))
    o, lse = fa2.forward_splitkv(q.to(dev), k.to(dev), v.to(dev), causal=True, scale=scale,
                                 out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
    row = np.array([N_BIG - 1], dtype=np.int64)  # the query sits after every key
    for h in range(H):
        o_ref, l_ref, _ = oracle.attention_rows(q[0, h], row, k[0, 0], v[0, 0], scale, True)
        res = parity.compare(parity.to_np(o[0, h].cpu()), o_ref,
                             parity.to_np(lse[0, h].cpu()), l_ref, "fp32")
        assert res["ok"], "head %d: %s" % (h, parity.describe(res))


def test_decode_at_the_key_limit(fa2):
    """The most keys a K/V head may hold at d = 128 (N*d <= 2^30 - 2^16, so
    the last tile's byte offset sits just under 2^31): one query per head
    for two query heads sharing the K/V head, against the oracle."""
    import torch
    d, H = 128, 2
    nk = ((1 << 30) - (1 << 16)) // d  # 8388096 keys, 2 GiB each of K and V
    g = torch.Generator(device="cpu").manual_seed(4444)
    q = torch.randn(1, H, 1, d, generator=g).to(torch.bfloat16)
    k = torch.empty(1, 1, nk, d, dtype=torch.bfloat16)
    v = torch.empty(1, 1, nk, d, dtype=torch.bfloat16)
    step = 1 << 20
    for t in (k, v):  # drawn in chunks to bound the fp32 temporaries
        for a in range(0, nk, step):
            b = min(nk, a + step)
            t[0, 0, a:b] = torch.randn(b - a, d, generator=g).to(torch.bfloat16)
    scale = 1.0 / math.sqrt(d)
    dev = torch.device("cuda:0")
    say("decode at the key limit: B=1 H=%d H_kv=1 Nq=1 Nk=%d d=%d" % (H, nk, d))
    o, lse = fa2.forward_splitkv(q.to(dev), k.to(dev), v.to(dev), causal=False, scale=scale,
                                 out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
    row = np.array([0], dtype=np.int64)
    for h in range(H):
        o_ref, l_ref, _ = oracle.attention_rows(q[0, h], row, k[0, 0], v[0, 0], scale, False)
        res = parity.compare(parity.to_np(o[0, h].cpu()), o_ref,
                             parity.to_np(lse[0, h].cpu()), l_ref, "fp32")
        assert res["ok"], "head %d: %s" % (h, parity.describe(res))


@pytest.mark.parametrize("entry", ["forward", "splitkv"])
def test_grouped_heads_at_the_packing_limit(fa2, entry):
    """One K/V head shared by tens of thousands of query heads of 127 rows.
    Short grouped query blocks run as one block of (H / H_kv) * Nq rows per
    K/V head while that packed head fits the per-head offset range (N*d <=
    2^30 - 2^16): 66048 query heads pack to exactly 2^30 - 2^16 elements,
    66052 heads would exceed it and run unpacked.  Sampled heads of both are
    compared with the oracle."""
    import torch
    d, nq = 128, 127
    nk = nq if entry == "forward" else 300
    h_big = 66052
    g = torch.Generator(device="cpu").manual_seed(4545)
    q = torch.empty(1, h_big, nq, d, dtype=torch.bfloat16)
    step = 4096
    for a in range(0, h_big, step):  # drawn in chunks to bound the fp32 temporaries
        b = min(h_big, a + step)
        q[0, a:b] = torch.randn(b - a, nq, d, generator=g).to(torch.bfloat16)
    k = torch.randn(1, 1, nk, d, generator=g).to(torch.bfloat16)
    v = torch.randn(1, 1, nk, d, generator=g).to(torch.bfloat16)
    scale = 1.0 / math.sqrt(d)
    dev = torch.device("cuda:0")
    qd_all, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    rows = np.arange(nq, dtype=np.int64)
    for H in (66048, h_big):
        qd = qd_all[:, :H]
        say("%s grouped heads B=1 H=%d H_kv=1 Nq=%d Nk=%d d=%d (packed rows %d)"
            % (entry, H, nq, nk, d, H * nq))
        if entry == "forward":
            o, lse = fa2.forward(qd, kd, vd, causal=False, scale=scale, out_dtype=torch.float32)
        else:
            o, lse = fa2.forward_splitkv(qd, kd, vd, causal=False, scale=scale, n_splits=2,
                                         out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert bool(torch.isfinite(lse).all())
        for h in (0, 1, H // 2, H - 2, H - 1):
            o_ref, l_ref, _ = oracle.attention_rows(q[0, h], rows, k[0, 0], v[0, 0], scale, False)
            res = parity.compare(parity.to_np(o[0, h].cpu()), o_ref,
                                 parity.to_np(lse[0, h].cpu()), l_ref, "fp32")
            assert res["ok"], "H=%d head %d: %s" % (H, h, parity.describe(res))
        del o, lse
        torch.cuda.empty_cache()
