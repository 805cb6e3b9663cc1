"""The allocation-free split-KV entry point (fa2_fwd_splitkv_noalloc) against
fa2_fwd_splitkv with caller-allocated workspaces: the same kernels on the
same inputs, so the outputs must be bit-identical.  Two calls in a row, the
second one smaller, so that the second runs on a workspace that still holds
the first call's partials."""
import ctypes
import sys

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


CASES = [
    # (B, H, H_kv, Nq, Nk, d, causal, n_splits): decode against a long cache
    # with grouped heads, then a smaller ragged chunked prefill
    (2, 8, 2, 1, 5000, 128, False, 4),
    (1, 4, 4, 130, 700, 64, True, 3),
]


def one_call(fa2, B, H, H_kv, Nq, Nk, d, causal, n_splits, seed):
    import torch
    dev = torch.device("cuda:0")
    q, k, v = wl.make_inputs(B, H, Nk, d, "bf16", seed=seed, H_kv=H_kv, Nq=Nq)
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    scale = d ** -0.5
    o_ref = torch.full((B, H, Nq, d), float("nan"), dtype=torch.bfloat16, device=dev)
    l_ref = torch.full((B, H, Nq), float("nan"), dtype=torch.float32, device=dev)
    fa2.forward_splitkv(qd, kd, vd, causal=causal, scale=scale, n_splits=n_splits,
                        out=o_ref, lse=l_ref)
    o = torch.full_like(o_ref, float("nan"))
    lse = torch.full_like(l_ref, float("nan"))
    stream = torch.cuda.current_stream(dev).cuda_stream
    rc = fa2.lib().fa2_fwd_splitkv_noalloc(
        qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), lse.data_ptr(),
        B, H, H_kv, Nq, Nk, d, ctypes.c_float(scale), int(causal), n_splits, stream)
    assert rc == 0, fa2.strerror(rc)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
    assert torch.equal(o, o_ref), float((o.float() - o_ref.float()).abs().max())
    assert torch.equal(lse, l_ref), float((lse - l_ref).abs().max())


def test_noalloc_matches_caller_workspace(fa2):
    for i, case in enumerate(CASES):
        say("noalloc call %d: B,H,H_kv,Nq,Nk,d,causal,splits = %s" % (i + 1, case))
        one_call(fa2, *case, seed=600 + i)


def test_noalloc_rejects_oversize(fa2):
    import torch
    dev = torch.device("cuda:0")
    say("noalloc oversize request")
    B, H, Nq, Nk, d = 1, 1, 1 << 15, 256, 128
    q = torch.zeros((B, H, Nq, d), dtype=torch.bfloat16, device=dev)
    k = torch.zeros((B, H, Nk, d), dtype=torch.bfloat16, device=dev)
    o = torch.empty_like(q)
    stream = torch.cuda.current_stream(dev).cuda_stream
    rc = fa2.lib().fa2_fwd_splitkv_noalloc(
        q.data_ptr(), k.data_ptr(), k.data_ptr(), o.data_ptr(), None, B, H, H, Nq,
        Nk, d, ctypes.c_float(0.1), 0, 4, stream)
    assert rc == fa2.FA2_ERR_WORKSPACE
