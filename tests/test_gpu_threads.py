"""GPU check that calls from several host threads, each on its own stream,
give the same bits as the same calls made one at a time.  The header states
that calls are thread-safe: the library's host side (argument checks, the
cached compute-unit count, the launch) keeps no per-call state, and each
call enqueues only on the stream it is given.  Four threads run the
forward (d = 128 causal with the persistent walk, d = 64, grouped heads),
split key ranges and the backward concurrently, several times each, and
every result is compared with a single-threaded reference.  (The
allocation-free split-KV entry point shares one workspace per GPU and is
documented as racing when calls overlap, so it is not used here.)  Every
case prints its name first."""
import sys
import threading

import pytest

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


def jobs(fa2, torch, dev):
    """(name, callable returning a tuple of tensors) for each thread."""
    out = []
    q, k, v = (t.to(dev) for t in wl.make_inputs(1, 40, 2048, 128, "bf16", seed=1201))
    out.append(("walk", lambda: fa2.forward(q, k, v, causal=True)))
    q2, k2, v2 = (t.to(dev) for t in wl.make_inputs(2, 4, 1000, 64, "bf16", seed=1202))
    out.append(("d64", lambda: fa2.forward(q2, k2, v2, causal=False, out_dtype=torch.float32)))
    q3, k3, v3 = (t.to(dev) for t in wl.make_inputs(1, 8, 1500, 128, "bf16", seed=1203, H_kv=2,
                                                   Nq=300))
    out.append(("splitkv", lambda: fa2.forward_splitkv(q3, k3, v3, causal=True, n_splits=3)))
    q4, k4, v4 = (t.to(dev) for t in wl.make_inputs(1, 8, 700, 128, "bf16", seed=1204, H_kv=2))
    g = torch.Generator().manual_seed(1205)
    do4 = torch.randn(q4.shape, generator=g).to(torch.bfloat16).to(dev)
    o4, l4 = fa2.forward(q4, k4, v4, causal=True)
    out.append(("bwd_gqa", lambda: fa2.backward(q4, k4, v4, o4, do4, l4, causal=True)))
    return out


def test_threads_same_bits(fa2):
    import torch
    dev = torch.device("cuda:0")
    work = jobs(fa2, torch, dev)
    torch.cuda.synchronize()
    say("threads: single-threaded references")
    refs = {}
    for name, fn in work:
        refs[name] = tuple(t.clone() for t in fn() if t is not None)
    torch.cuda.synchronize()

    errors = []
    results = {}

    def worker(name, fn):
        try:
            s = torch.cuda.Stream(device=dev)
            got = []
            with torch.cuda.stream(s):
                for _ in range(5):
                    got.append(tuple(t.clone() for t in fn() if t is not None))
            s.synchronize()
            results[name] = got
        except Exception as e:  # reported in the main thread
            errors.append("%s: %r" % (name, e))

    say("threads: %d threads, 5 calls each, own streams" % len(work))
    threads = [threading.Thread(target=worker, args=(n, f)) for n, f in work]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    torch.cuda.synchronize()
    assert not any(t.is_alive() for t in threads), "a thread did not finish"
    assert not errors, errors
    for name, _ in work:
        for i, got in enumerate(results[name]):
            for j, (a, b) in enumerate(zip(got, refs[name])):
                assert torch.equal(a, b), "%s call %d output %d differs" % (name, i, j)
