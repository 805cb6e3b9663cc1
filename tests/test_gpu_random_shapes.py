"""Seeded sweep of random shapes through every bf16 entry point, each
checked against the fp64 oracle: batch, heads,
shared K/V heads, sequence lengths (ragged, below a tile, a few blocks),
head dimension, mask, scale (sign and size), output dtype, key-range
counts, query-head ranges of the grouped backward.  A few draws are large
enough for the forward's persistent walk.  Forward outputs are held to the
stated tolerance at every scale (sharp softmaxes included); gradients as
described in the backward test.
Every case prints its name first; the draws are fixed by the seed."""
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


def draws(kind, n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        d = int(rng.choice([64, 128]))
        Hk = int(rng.integers(1, 4))
        H = Hk * int(rng.choice([1, 1, 2, 3, 4]))
        B = int(rng.integers(1, 3))
        N = int(rng.choice([int(rng.integers(1, 64)), int(rng.integers(64, 700)),
                            int(rng.integers(700, 2100))]))
        causal = bool(rng.integers(0, 2))
        scale = float(rng.choice([1.0 / math.sqrt(d), rng.uniform(-0.3, 0.3),
                                  rng.uniform(0.3, 1.0)]))
        out.append((kind, i, B, H, Hk, N, d, causal, scale, int(rng.integers(0, 1 << 30))))
    return out


def kv_ref(k, v, H):
    if k.shape[1] == H:
        return k, v
    return oracle.expand_kv_heads(k, H), oracle.expand_kv_heads(v, H)


FWD = draws("fwd", 96, 2026)


@pytest.mark.parametrize("case", FWD, ids=["fwd%d" % c[1] for c in FWD])
def test_forward_random(fa2, case):
    import torch
    _, i, B, H, Hk, N, d, causal, scale, seed = case
    q, k, v = wl.make_inputs(B, H, N, d, "bf16", seed=seed, H_kv=Hk)
    kx, vx = kv_ref(k, v, H)
    o_ref, l_ref, _ = oracle.attention(q, kx, vx, scale, causal)
    dev = torch.device("cuda:0")
    odt = torch.float32 if i % 2 else torch.bfloat16
    kind = "fp32" if i % 2 else "bf16"
    say("fwd B=%d H=%d H_kv=%d N=%d d=%d causal=%s scale=%.4f out=%s"
        % (B, H, Hk, N, d, causal, scale, kind))
    o, lse = fa2.forward(q.to(dev), k.to(dev), v.to(dev), causal=causal, scale=scale,
                         out_dtype=odt)
    torch.cuda.synchronize()
    res = parity.compare(parity.to_np(o.cpu()), o_ref, parity.to_np(lse.cpu()), l_ref, kind)
    assert res["ok"], parity.describe(res)


SPLIT = draws("split", 48, 2027)


@pytest.mark.parametrize("case", SPLIT, ids=["split%d" % c[1] for c in SPLIT])
def test_splitkv_random(fa2, case):
    import torch
    _, i, B, H, Hk, N, d, causal, scale, seed = case
    rng = np.random.default_rng(seed)
    nq = int(rng.integers(1, max(2, min(N, 300))))
    S = int(rng.choice([1, 2, 3, 7, 16]))
    q, k, v = wl.make_inputs(B, H, N, d, "bf16", seed=seed, H_kv=Hk, Nq=nq)
    kx, vx = kv_ref(k, v, H)
    o_ref, l_ref, _ = oracle.attention_offset(q, kx, vx, scale, causal)
    dev = torch.device("cuda:0")
    say("splitkv B=%d H=%d H_kv=%d Nq=%d Nk=%d d=%d causal=%s scale=%.4f splits=%d"
        % (B, H, Hk, nq, N, d, causal, scale, S))
    o, lse = fa2.forward_splitkv(q.to(dev), k.to(dev), v.to(dev), causal=causal,
                                 scale=scale, n_splits=S, out_dtype=torch.float32)
    torch.cuda.synchronize()
    o_np, l_np = parity.to_np(o.cpu()), parity.to_np(lse.cpu())
    empty = np.isneginf(l_ref)
    if empty.any():  # rows that see no key: O = 0, lse = -inf exactly
        assert np.all(np.isneginf(l_np[empty])) and np.all(o_np[empty] == 0)
        o_np, l_np, o_ref, l_ref = o_np[~empty], l_np[~empty], o_ref[~empty], l_ref[~empty]
    res = parity.compare(o_np, o_ref, l_np, l_ref, "fp32")
    assert res["ok"], parity.describe(res)


BWD = [c for c in draws("bwd", 32, 2028)]


@pytest.mark.parametrize("case", BWD, ids=["bwd%d" % c[1] for c in BWD])
def test_backward_random(fa2, case):
    """Gradients against the oracle.  The draws include scales well above
    1/sqrt(d), where the softmax is sharp and the bf16 roundings weigh more
    than on the inputs the standard bounds were derived for; each case is
    therefore held to max(standard bound, 1.5 x the error of the rounding
    model evaluated on the same inputs)."""
    import torch
    from test_bwd_tolerance_model import model_grads
    _, i, B, H, Hk, N, d, causal, scale, seed = case
    N = min(N, 900)  # the gradient oracle is O(N^2 d) per head
    q, k, v = wl.make_inputs(B, H, N, d, "bf16", seed=seed, H_kv=Hk)
    do = wl.make_dout(B, H, N, d, seed=seed + 1)
    ref = oracle.attention_bwd_gqa(q, k, v, do, scale, causal)
    kx, vx = (torch.from_numpy(oracle.expand_kv_heads(t, H)) for t in (k, v))
    mq, mk, mv = model_grads(q, kx, vx, do, scale, causal)
    model = (mq, oracle.sum_kv_groups(mk, Hk), oracle.sum_kv_groups(mv, Hk))
    dev = torch.device("cuda:0")
    odt = torch.float32 if i % 2 else torch.bfloat16
    ns = None if H == Hk else int(np.random.default_rng(seed).integers(1, H // Hk + 1))
    say("bwd B=%d H=%d H_kv=%d N=%d d=%d causal=%s scale=%.4f out=%s ranges=%s"
        % (B, H, Hk, N, d, causal, scale, odt, ns))
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    o, lse = fa2.forward(qd, kd, vd, causal=causal, scale=scale)
    grads = fa2.backward(qd, kd, vd, o, dod, lse, causal=causal, scale=scale,
                         out_dtype=odt, n_gsplits=ns)
    torch.cuda.synchronize()
    for name, g, r, m in zip(("dq", "dk", "dv"), grads, ref[:3], model):
        res = parity.compare_grad(parity.to_np(g.cpu()), r)
        mres = parity.compare_grad(m, r)
        ok = res["finite"] and \
            res["rel_l2"] <= max(parity.GRAD_REL_L2, 1.5 * mres["rel_l2"]) and \
            res["max_rel"] <= max(parity.GRAD_MAX_REL, 1.5 * mres["max_rel"])
        assert ok, "%s: %s (model: %s)" % (name, parity.describe(res), parity.describe(mres))


def test_random_walking_launches(fa2):
    """Causal d = 128 launches with more query blocks than two per compute
    unit and lengths that are multiples of the 64-key tile (the forward's
    persistent walk), random lengths and heads, sampled rows of the first
    and last head against the oracle."""
    import torch
    rng = np.random.default_rng(2029)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    dev = torch.device("cuda:0")
    for _ in range(3):
        N = 64 * int(rng.integers(10, 27))
        blocks = (N + 127) // 128
        Hk = int(rng.integers(1, 3))
        H = Hk * (-(-(2 * cus + 1) // (blocks * Hk)) + int(rng.integers(0, 3)))
        q, k, v = wl.make_inputs(1, H, N, 128, "bf16", seed=int(rng.integers(0, 1 << 30)), H_kv=Hk)
        say("walking launch H=%d H_kv=%d N=%d (%d blocks)" % (H, Hk, N, H * blocks))
        o, lse = fa2.forward(q.to(dev), k.to(dev), v.to(dev), causal=True,
                             out_dtype=torch.float32)
        torch.cuda.synchronize()
        rows = np.unique(np.concatenate([np.arange(4), np.arange(N - 4, N),
                                         rng.choice(N, 12, replace=False)])).astype(np.int64)
        for h in (0, H - 1):
            hk = h // (H // Hk)
            o_ref, l_ref, _ = oracle.attention_rows(q[0, h][rows], rows, k[0, hk], v[0, hk],
                                                    1.0 / math.sqrt(128), True)
            res = parity.compare(parity.to_np(o[0, h][rows].cpu()), o_ref,
                                 parity.to_np(lse[0, h][rows].cpu()), l_ref, "fp32")
            assert res["ok"], "head %d: %s" % (h, parity.describe(res))
