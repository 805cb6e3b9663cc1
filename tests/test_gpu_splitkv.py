"""GPU parity of the general forward (fa2_fwd_splitkv[_o32]): separate query
and key lengths, grouped K/V heads, and key ranges computed by separate
workgroups then merged.  Every case prints its name before touching the GPU."""
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


def run(fa2, q, k, v, causal, scale, n_splits, out_dtype):
    import torch
    dev = torch.device("cuda:0")
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    o = torch.full(q.shape, float("nan"), dtype=out_dtype, device=dev)
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=dev)
    fa2.forward_splitkv(qd, kd, vd, causal=causal, scale=scale, n_splits=n_splits,
                        out_dtype=out_dtype, out=o, lse=lse)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def reference(q, k, v, scale, causal):
    h = q.shape[1]
    kx = oracle.expand_kv_heads(k, h) if k.shape[1] != h else k
    vx = oracle.expand_kv_heads(v, h) if v.shape[1] != h else v
    return oracle.attention_offset(q, kx, vx, scale, causal)


CASES = [
    # (B, H, H_kv, Nq, Nk, d, causal, n_splits)
    (2, 4, 4, 1, 1000, 128, False, 1),     # one decode step
    (2, 4, 4, 1, 1000, 128, False, 3),
    (2, 4, 4, 1, 1000, 128, True, 8),
    (1, 8, 2, 16, 2048, 128, True, 4),     # a few new tokens, grouped heads
    (1, 8, 1, 3, 777, 64, True, 5),        # MQA, d = 64, ragged keys
    (1, 2, 2, 200, 513, 64, True, 5),      # chunked prefill, ragged
    (1, 2, 2, 130, 4096, 128, False, 64),  # more ranges than ... kept busy
    (1, 1, 1, 2, 100, 128, False, 16),     # more ranges than key tiles
    (1, 2, 2, 300, 100, 128, True, 2),     # more queries than keys
    (2, 2, 2, 256, 256, 128, True, 3),     # square, split
    # shared K/V heads with few queries: a group's rows run as one matrix
    (2, 8, 2, 1, 1000, 128, True, 3),      # grouped decode (one query sees all keys)
    (1, 8, 1, 1, 700, 64, False, 1),       # multi-query decode, one range, d = 64
    (2, 8, 2, 5, 900, 128, False, 2),      # a few queries per head, no mask
    (1, 16, 2, 100, 600, 128, False, 1),   # 800 rows per group: blocks span heads
    (1, 32, 4, 1, 4096, 128, True, 16),    # eight query heads per K/V head
]


@pytest.mark.parametrize("B,H,Hk,Nq,Nk,d,causal,S", CASES,
                         ids=["B%dH%dkv%dq%dk%dd%d%ss%d" % (c[0], c[1], c[2], c[3], c[4], c[5],
                                                          "c" if c[6] else "", c[7])
                              for c in CASES])
def test_splitkv_vs_oracle(fa2, B, H, Hk, Nq, Nk, d, causal, S):
    import torch
    q, k, v = wl.make_inputs(B, H, Nk, d, "bf16", seed=700 + Nq + Nk, H_kv=Hk, Nq=Nq)
    scale = 1.0 / math.sqrt(d)
    o_ref, l_ref, _ = reference(q, k, v, scale, causal)
    for odt, kind in ((torch.bfloat16, "bf16"), (torch.float32, "fp32")):
        say("splitkv B=%d H=%d H_kv=%d Nq=%d Nk=%d d=%d causal=%s splits=%d out=%s"
            % (B, H, Hk, Nq, Nk, d, causal, S, kind))
        o, lse = run(fa2, q, k, v, causal, scale, S, odt)
        o_np, l_np = parity.to_np(o), parity.to_np(lse)
        empty = np.isneginf(l_ref)
        if empty.any():  # rows that see no key: O = 0, lse = -inf exactly
            assert np.all(np.isneginf(l_np[empty])) and np.all(o_np[empty] == 0)
            o_np, l_np = o_np[~empty], l_np[~empty]
            o_r, l_r = o_ref[~empty], l_ref[~empty]
        else:
            o_r, l_r = o_ref, l_ref
        res = parity.compare(o_np, o_r, l_np, l_r, kind)
        assert res["ok"], parity.describe(res)


@pytest.mark.parametrize("N,causal", [(1, True), (40, False), (130, False)])
def test_grouped_short_sequences(fa2, N, causal):
    """fa2_fwd_gqa with fewer than 128 rows per head and every row seeing
    the same keys runs each group's rows together; against the oracle."""
    import torch
    q, k, v = wl.make_inputs(2, 8, N, 128, "bf16", seed=760 + N, H_kv=2)
    scale = 1.0 / math.sqrt(128)
    o_ref, l_ref, _ = reference(q, k, v, scale, causal)
    dev = torch.device("cuda:0")
    say("grouped forward N=%d causal=%s" % (N, causal))
    o, lse = fa2.forward(q.to(dev), k.to(dev), v.to(dev), causal=causal, scale=scale,
                         out_dtype=torch.float32)
    torch.cuda.synchronize()
    res = parity.compare(parity.to_np(o), o_ref, parity.to_np(lse), l_ref, "fp32")
    assert res["ok"], parity.describe(res)


def test_one_range_equals_fa2_fwd(fa2):
    """With equal lengths and one key range the general entry point runs the
    same kernel as fa2_fwd: bit-identical outputs."""
    import torch
    q, k, v = wl.make_inputs(2, 3, 700, 128, "bf16", seed=71)
    say("splitkv n_splits=1 vs fa2_fwd")
    a = run(fa2, q, k, v, True, 0.0884, 1, torch.bfloat16)
    dev = torch.device("cuda:0")
    o, lse = fa2.forward(q.to(dev), k.to(dev), v.to(dev), causal=True, scale=0.0884)
    torch.cuda.synchronize()
    assert torch.equal(a[0], o.cpu()) and torch.equal(a[1], lse.cpu())


@pytest.mark.parametrize("name", ["decode_b8h32_nq1_nk16384_d128",
                                  "decode_gqa_b8h32kv8_nq1_nk16384_d128"])
def test_decode_workload_full_size(fa2, name):
    """The decode workloads at full size with the default range count: every
    row against the oracle (one query row per head; with grouped K/V heads a
    group's rows run together)."""
    import torch
    w = wl.WORKLOADS[name]
    q, k, v = wl.workload_inputs(w)
    say("decode workload %s" % w.describe())
    dev = torch.device("cuda:0")
    o, lse = fa2.forward_splitkv(q.to(dev), k.to(dev), v.to(dev), causal=w.causal,
                                 scale=w.scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref, l_ref, _ = reference(q, k, v, w.scale, w.causal)
    res = parity.compare(parity.to_np(o), o_ref, parity.to_np(lse), l_ref, "fp32")
    assert res["ok"], parity.describe(res)
