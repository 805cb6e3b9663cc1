"""GPU check of the kernels' synchronisation under a different occupancy.
With FA2_DEBUG_ONE_WG_PER_CU=1 in the environment every attention kernel is
launched with extra dynamic LDS that it never touches, so that at most one
workgroup runs per compute unit instead of two to four.  The timing of the
waves, the co-resident workgroups and the order in which the hardware hands
out workgroups all change; a missing barrier or a buffer reused too early
would then show as different output bits.  Every path is run both ways and
compared bit for bit: the d = 128 forward with and without the persistent
walk, d = 64, grouped heads, split key ranges with their merge, the fp32
path, FP8, and the backward (plain, grouped with paired blocks, d = 64).
One timing check shows that the switch takes effect.  Every case prints
its name first."""
import sys
import time

import pytest

from exact_io_aware_24_amd import inputs as wl

pytestmark = pytest.mark.gpu
ENV = "FA2_DEBUG_ONE_WG_PER_CU"


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


def both(monkeypatch, fn):
    """fn() with the switch off and on; returns the two output tuples."""
    import torch
    monkeypatch.delenv(ENV, raising=False)
    a = fn()
    torch.cuda.synchronize()
    monkeypatch.setenv(ENV, "1")
    b = fn()
    torch.cuda.synchronize()
    monkeypatch.delenv(ENV)
    return a, b


def same(a, b, what):
    import torch
    for i, (x, y) in enumerate(zip(a, b)):
        assert torch.equal(x, y), "%s: output %d differs at one workgroup per CU" % (what, i)


FWD = [
    # (name, B, H, H_kv, N, d, causal)
    ("walk", 1, 40, 40, 2048, 128, True),      # 640 items: the persistent walk
    ("ragged", 1, 3, 3, 1000, 128, False),
    ("causal_ragged", 2, 3, 3, 777, 128, True),
    ("d64", 2, 3, 3, 777, 64, True),
    ("d64_noncausal", 1, 4, 4, 1030, 64, False),
    ("gqa", 1, 8, 2, 1100, 128, True),
]


@pytest.mark.parametrize("name,B,H,Hkv,N,d,causal", FWD, ids=[c[0] for c in FWD])
def test_forward_same_bits(fa2, monkeypatch, name, B, H, Hkv, N, d, causal):
    import torch
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in wl.make_inputs(B, H, N, d, "bf16", seed=990 + N, H_kv=Hkv))
    for odt in (torch.bfloat16, torch.float32):
        say("one wg/CU forward %s B=%d H=%d H_kv=%d N=%d d=%d causal=%s out=%s"
            % (name, B, H, Hkv, N, d, causal, odt))
        a, b = both(monkeypatch, lambda: fa2.forward(q, k, v, causal=causal, out_dtype=odt))
        same(a, b, name)


def test_splitkv_same_bits(fa2, monkeypatch):
    import torch
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in wl.make_inputs(1, 4, 1500, 128, "bf16", seed=993, H_kv=2,
                                                  Nq=300))
    say("one wg/CU split-KV Nq=300 Nk=1500 splits=3")
    a, b = both(monkeypatch,
                lambda: fa2.forward_splitkv(q, k, v, causal=True, n_splits=3))
    same(a, b, "splitkv")


def test_fp32_same_bits(fa2, monkeypatch):
    import torch
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in wl.make_inputs(1, 2, 300, 64, "fp32", seed=994))
    say("one wg/CU fp32 path N=300 d=64 causal")
    a, b = both(monkeypatch, lambda: fa2.forward(q, k, v, causal=True))
    same(a, b, "fp32")


def test_fp8_same_bits(fa2, monkeypatch):
    import torch
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in wl.make_inputs(1, 3, 1000, 128, "bf16", seed=995))
    signs = wl.make_signs(128).to(dev)
    say("one wg/CU FP8 N=1000 d=128 causal rotated")
    a, b = both(monkeypatch,
                lambda: fa2.attention_fp8(q, k, v, causal=True, signs=signs))
    same(a, b, "fp8")


BWD = [
    # (name, B, H, H_kv, N, d, causal)
    ("plain", 1, 4, 4, 600, 128, True),
    ("noncausal", 1, 2, 2, 530, 128, False),
    ("gqa_pairs", 1, 8, 2, 700, 128, True),
    ("d64", 2, 2, 2, 450, 64, True),
]


@pytest.mark.parametrize("name,B,H,Hkv,N,d,causal", BWD, ids=[c[0] for c in BWD])
def test_backward_same_bits(fa2, monkeypatch, name, B, H, Hkv, N, d, causal):
    import torch
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in wl.make_inputs(B, H, N, d, "bf16", seed=996 + N, H_kv=Hkv))
    g = torch.Generator().manual_seed(997 + N)
    do = torch.randn(q.shape, generator=g).to(torch.bfloat16).to(dev)
    o, lse = fa2.forward(q, k, v, causal=causal)
    torch.cuda.synchronize()
    say("one wg/CU backward %s B=%d H=%d H_kv=%d N=%d d=%d causal=%s"
        % (name, B, H, Hkv, N, d, causal))
    a, b = both(monkeypatch, lambda: fa2.backward(q, k, v, o, do, lse, causal=causal))
    same(a, b, name)


def test_switch_takes_effect(fa2, monkeypatch):
    """The d = 64 kernel runs four workgroups per compute unit; with one it
    takes measurably longer (about 1.4x on the training-sized shape)."""
    import torch
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in wl.make_inputs(8, 16, 2048, 64, "bf16", seed=998))
    o = torch.empty_like(q)

    def best_ms():
        for _ in range(3):
            fa2.forward(q, k, v, out=o, return_lse=False)
        torch.cuda.synchronize()
        ts = []
        for _ in range(5):
            t0 = time.perf_counter()
            for _ in range(10):
                fa2.forward(q, k, v, out=o, return_lse=False)
            torch.cuda.synchronize()
            ts.append((time.perf_counter() - t0) / 10)
        return min(ts)

    say("one wg/CU timing check d=64 B=8 H=16 N=2048")
    monkeypatch.delenv(ENV, raising=False)
    t_normal = best_ms()
    monkeypatch.setenv(ENV, "1")
    t_one = best_ms()
    monkeypatch.delenv(ENV)
    print("normal %.3f ms, one workgroup per CU %.3f ms" % (t_normal * 1e3, t_one * 1e3))
    assert t_one > 1.15 * t_normal
