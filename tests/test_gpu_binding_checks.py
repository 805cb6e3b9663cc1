"""GPU check of the Python binding's buffer validation.  Caller-supplied
outputs and workspaces (out, lse, o_part, lse_part, codes, exps, the FP8
block exponents, the sign vector) must have the shape, dtype, layout and
device the kernels write or read; the C ABI takes bare pointers and cannot
see their sizes, so the binding rejects a wrong buffer with ValueError
before anything is enqueued, and out-of-range key-range or query-head-range
counts before a workspace is sized from them.  The rejected calls launch
nothing; one test runs a valid call with oversized workspaces and compares
it with the call that allocates its own.  Every case prints its name first."""
import sys

import pytest

from exact_io_aware_24_amd import inputs as wl

pytestmark = pytest.mark.gpu


def say(msg):
    print("[case] " + msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests need an MI355X")
    import exact_io_aware_24_amd as m
    m.lib()
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in wl.make_inputs(1, 2, 200, 64, "bf16", seed=4242))
    return m, torch, dev, q, k, v


def rejects(fn, *args, **kw):
    with pytest.raises(ValueError):
        fn(*args, **kw)


def test_forward_outputs(env):
    m, torch, dev, q, k, v = env
    B, H, N, d = q.shape
    say("forward: wrong out / lse buffers")
    rejects(m.forward, q, k, v, out=torch.empty(B, H, N - 1, d, dtype=torch.bfloat16, device=dev))
    rejects(m.forward, q, k, v, out=torch.empty(B, H, N, d, dtype=torch.float32, device=dev))
    rejects(m.forward, q, k, v,
            out=torch.empty(B, H, d, N, dtype=torch.bfloat16, device=dev).transpose(2, 3))
    rejects(m.forward, q, k, v, out=torch.empty(B, H, N, d, dtype=torch.bfloat16))
    rejects(m.forward, q, k, v, lse=torch.empty(B, H, N - 1, device=dev))
    rejects(m.forward, q, k, v, lse=torch.empty(B, H, N, dtype=torch.float64, device=dev))


def test_splitkv_buffers(env):
    m, torch, dev, q, k, v = env
    B, H, N, d = q.shape
    say("forward_splitkv: workspaces smaller than n_splits x the output")
    f32 = dict(dtype=torch.float32, device=dev)
    rejects(m.forward_splitkv, q, k, v, n_splits=2, o_part=torch.empty(1, B, H, N, d, **f32))
    rejects(m.forward_splitkv, q, k, v, n_splits=2, lse_part=torch.empty(2, B, H, N - 1, **f32))
    rejects(m.forward_splitkv, q, k, v, n_splits=2,
            o_part=torch.empty(2, B, H, N, d, dtype=torch.bfloat16, device=dev))
    rejects(m.forward_splitkv, q, k, v, n_splits=2,
            out=torch.empty(B, H, N, d + 1, dtype=torch.bfloat16, device=dev))
    say("forward_splitkv[_noalloc]: key-range counts out of range, rejected before any "
        "workspace is sized from them")
    for ns in (0, -1, m.MAX_SPLITS + 1, 1 << 40):
        rejects(m.forward_splitkv, q, k, v, n_splits=ns)
        rejects(m.forward_splitkv_noalloc, q, k, v, n_splits=ns)
    say("forward_splitkv_noalloc: wrong out / lse buffers")
    rejects(m.forward_splitkv_noalloc, q, k, v, n_splits=2,
            out=torch.empty(B, H, N, d, **f32))
    rejects(m.forward_splitkv_noalloc, q, k, v, n_splits=2,
            lse=torch.empty(B, H, N + 1, **f32))


def test_fp8_buffers(env):
    m, torch, dev, q, k, v = env
    B, H, N, d = q.shape
    signs = wl.make_signs(d).to(dev)
    say("quantize_fp8: wrong codes / exps / signs / block_rows")
    rejects(m.quantize_fp8, q, 64, codes=torch.empty(B, H, N, d - 1, dtype=torch.uint8, device=dev))
    rejects(m.quantize_fp8, q, 64, exps=torch.empty(B, H, 4, dtype=torch.int64, device=dev))
    rejects(m.quantize_fp8, q, 64, exps=torch.empty(B, H, 3, dtype=torch.int32, device=dev))
    rejects(m.quantize_fp8, q, 64, signs=signs[: d // 2])
    rejects(m.quantize_fp8, q, 64, signs=torch.stack([signs, signs], 1)[:, 0])
    rejects(m.quantize_fp8, q, 64, signs=signs.cpu())
    rejects(m.quantize_fp8, q, 32)
    say("forward_fp8: wrong block exponents / out")
    q8, qe = m.quantize_fp8(q, 128, signs)
    k8, ke = m.quantize_fp8(k, 64, signs)
    v8, ve = m.quantize_fp8(v, 64, None)
    torch.cuda.synchronize()
    rejects(m.forward_fp8, q8, ke, k8, ke, v8, ve, rotated=True)  # 64-row exponents as Q's
    rejects(m.forward_fp8, q8, qe, k8, ke.long(), v8, ve, rotated=True)
    rejects(m.forward_fp8, q8, qe, k8, ke, v8, ve[..., :-1].contiguous(), rotated=True)
    rejects(m.forward_fp8, q8, qe, k8, ke, v8, ve, rotated=True,
            out=torch.empty(B, H, N, d, dtype=torch.float32, device=dev))
    rejects(m.forward_fp8, q8, qe, k8, ke, v8, ve, rotated=True,
            lse=torch.empty(B, H, N - 1, device=dev))


def test_oversized_workspaces_work(env):
    m, torch, dev, q, k, v = env
    B, H, N, d = q.shape
    say("forward_splitkv with oversized flat workspaces, against self-allocated ones")
    o_part = torch.full((2 * B * H * N * d + 17,), float("nan"), device=dev)
    lse_part = torch.full((2 * B * H * N + 5,), float("nan"), device=dev)
    o1, l1 = m.forward_splitkv(q, k, v, causal=True, n_splits=2, o_part=o_part,
                               lse_part=lse_part)
    o2, l2 = m.forward_splitkv(q, k, v, causal=True, n_splits=2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_backward_range_count(env):
    m, torch, dev, q, k, v = env
    B, H, N, d = q.shape
    kv = k[:, :1].contiguous(), v[:, :1].contiguous()
    o, lse = m.forward(q, *kv)
    say("backward: query-head range counts outside 1..H/H_kv rejected before the "
        "workspace is sized from them")
    for ns in (0, -3, H + 1, 1 << 40):
        rejects(m.backward, q, *kv, o, o, lse, n_gsplits=ns)
