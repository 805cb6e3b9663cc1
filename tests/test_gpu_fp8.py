"""GPU checks of the FP8 path: the quantiser's codes and exponents bit for
bit against the oracle's, the FP8 attention against the exact attention of
the (oracle-)dequantised inputs, and the end-to-end error against the exact
attention of the original inputs.  Every case prints its name first."""
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


def outlier_channels(x, chans, factor=20.0):
    import torch
    y = x.float()
    for ch in chans:
        y[..., ch] *= factor
    return y.to(torch.bfloat16)


QCASES = [(1, 2, 100, 64), (2, 1, 300, 128), (1, 1, 1, 128), (1, 2, 64, 64),
          (1, 1, 1000, 128)]


@pytest.mark.parametrize("B,H,N,d", QCASES)
def test_quantize_bit_exact(fa2, B, H, N, d):
    import torch
    dev = torch.device("cuda:0")
    x = wl.make_inputs(B, H, N, d, "bf16", seed=900 + N, outliers=True)[0]
    x = outlier_channels(x, (1, d // 2))
    signs = wl.make_signs(d)
    for rows in (64, 128):
        for sg in (None, signs):
            say("quantize B=%d H=%d N=%d d=%d rows=%d rotate=%s" % (B, H, N, d, rows, sg is not None))
            codes, exps = fa2.quantize_fp8(x.to(dev), rows, sg.to(dev) if sg is not None else None)
            torch.cuda.synchronize()
            c_ref, e_ref = oracle.quantize_fp8(x, rows, sg.numpy() if sg is not None else None)
            assert np.array_equal(exps.cpu().numpy(), e_ref)
            assert np.array_equal(codes.cpu().numpy(), c_ref)


ACASES = [(1, 2, 256, 128, True), (2, 2, 300, 64, False), (1, 1, 1000, 128, True),
          (1, 3, 129, 64, True), (1, 1, 1, 128, False)]


def run_fp8(fa2, q, k, v, causal, signs, out_dtype=None, scale=None):
    import torch
    dev = torch.device("cuda:0")
    o, lse = fa2.attention_fp8(q.to(dev), k.to(dev), v.to(dev), causal=causal,
                               scale=scale,
                               signs=signs.to(dev) if signs is not None else None,
                               out_dtype=out_dtype)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


@pytest.mark.parametrize("B,H,N,d,causal", ACASES)
def test_fp8_attention_vs_dequantised(fa2, B, H, N, d, causal):
    import torch
    q, k, v = wl.make_inputs(B, H, N, d, "bf16", seed=950 + N)
    scale = 1.0 / math.sqrt(d) if N != 129 else -0.2  # one negative scale
    for sg in (None, wl.make_signs(d)):
        o_ref, l_ref, _ = oracle.attention_fp8_reference(
            q, k, v, scale, causal, sg.numpy() if sg is not None else None)
        for odt in (torch.bfloat16, torch.float32):
            say("fp8 attention B=%d H=%d N=%d d=%d causal=%s rotate=%s out=%s"
                % (B, H, N, d, causal, sg is not None, odt))
            o, lse = run_fp8(fa2, q, k, v, causal, sg, odt, scale)
            res = parity.compare_fp8(parity.to_np(o), o_ref)
            assert res["finite"] and res["rel_l2"] <= parity.FP8_REL_L2 \
                and res["max_rel"] <= parity.FP8_MAX_REL, res
            # lse: exact scores of the dequantised inputs up to the MFMA's
            # fp8 dot-product rounding; P' sums are fp32
            assert np.max(np.abs(parity.to_np(lse) - l_ref)) <= 1e-2


@pytest.mark.parametrize("N,d", [(200, 128), (77, 64)])
def test_fp8_zero_scale(fa2, N, d):
    """scale = 0: every visible key has weight one (the causal mask keeps
    the prefix), so O is the running mean of the dequantised V rows; the
    masked scores meet a zero scale on the diagonal tiles."""
    import torch
    q, k, v = wl.make_inputs(1, 2, N, d, "bf16", seed=970 + N)
    for sg in (None, wl.make_signs(d)):
        say("fp8 attention scale=0 N=%d d=%d causal rotate=%s" % (N, d, sg is not None))
        o_ref, l_ref, _ = oracle.attention_fp8_reference(
            q, k, v, 0.0, True, sg.numpy() if sg is not None else None)
        o, lse = run_fp8(fa2, q, k, v, True, sg, torch.float32, 0.0)
        res = parity.compare_fp8(parity.to_np(o), o_ref)
        assert res["finite"] and res["rel_l2"] <= parity.FP8_REL_L2 \
            and res["max_rel"] <= parity.FP8_MAX_REL, res
        assert np.max(np.abs(parity.to_np(lse) - l_ref)) <= 1e-2


def test_fp8_end_to_end(fa2):
    """Against the exact attention of the original bf16 inputs: within the
    bound on standard normal inputs; with outlier channels the rotation
    keeps the error low and beats the unrotated path several times."""
    d = 128
    q, k, v = wl.make_inputs(1, 4, 1024, d, "bf16", seed=77)
    o_ex, _, _ = oracle.attention(q, k, v, 1 / math.sqrt(d), True)
    say("fp8 end-to-end standard inputs")
    o, _ = run_fp8(fa2, q, k, v, True, wl.make_signs(d))
    res = parity.compare_fp8(parity.to_np(o), o_ex)
    assert res["rel_l2"] <= parity.FP8_E2E_REL_L2, res
    qo, ko = outlier_channels(q, (3, 17, d - 5)), outlier_channels(k, (3, 17, d - 5))
    o_ex, _, _ = oracle.attention(qo, ko, v, 1 / math.sqrt(d), True)
    say("fp8 end-to-end outlier channels")
    rot = parity.compare_fp8(parity.to_np(run_fp8(fa2, qo, ko, v, True, wl.make_signs(d))[0]), o_ex)
    plain = parity.compare_fp8(parity.to_np(run_fp8(fa2, qo, ko, v, True, None)[0]), o_ex)
    assert rot["rel_l2"] <= parity.FP8_E2E_ROT_OUTLIER_REL_L2, rot
    assert plain["rel_l2"] > 2.0 * rot["rel_l2"], (plain, rot)


@pytest.mark.timeout(600)
def test_fp8_full_size_headline(fa2):
    """The headline shape (B=2, H=16, N=8192, d=128, causal) with rotation:
    every element of every head against the exact attention of the
    dequantised inputs (rel-L2 and max-abs relative to the largest
    reference value, over the whole tensor and within each head), every
    output finite."""
    import time

    import torch  # noqa: F811
    w = wl.WORKLOADS[wl.HEADLINE]
    q, k, v = wl.workload_inputs(w)
    signs = wl.make_signs(w.d)
    say("fp8 full size %s" % w.describe())
    o, lse = run_fp8(fa2, q, k, v, True, signs)
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
    say("fp8 oracle (all heads)")
    t0 = time.time()
    o_ref, _, _ = oracle.attention_fp8_reference(q, k, v, w.scale, True,
                                                 signs=signs.numpy())
    say("fp8 oracle done in %.1f s" % (time.time() - t0))
    on = parity.to_np(o)
    res = parity.compare_fp8(on, o_ref)
    say("  whole tensor: " + parity.describe(res))
    assert res["rel_l2"] <= parity.FP8_REL_L2 and res["max_rel"] <= parity.FP8_MAX_REL, res
    oh = on.reshape(w.B * w.H, w.N, w.d)
    rh = o_ref.reshape(w.B * w.H, w.N, w.d)
    for h in range(w.B * w.H):
        rs = parity.compare_fp8(oh[h], rh[h])
        assert rs["rel_l2"] <= parity.FP8_REL_L2 and rs["max_rel"] <= parity.FP8_MAX_REL, (h, rs)


def fp8_draws(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        d = int(rng.choice([64, 128]))
        N = int(rng.choice([int(rng.integers(1, 64)), int(rng.integers(64, 700)),
                            int(rng.integers(700, 1600))]))
        out.append((i, int(rng.integers(1, 3)), int(rng.integers(1, 4)), N, d,
                    bool(rng.integers(0, 2)),
                    float(rng.choice([1.0 / math.sqrt(d), rng.uniform(-0.2, 0.2)])),
                    bool(rng.integers(0, 2)), int(rng.choice([64, 128])),
                    int(rng.integers(0, 1 << 30))))
    return out


FP8_RANDOM = fp8_draws(32, 2030)


@pytest.mark.parametrize("case", FP8_RANDOM, ids=["fp8r%d" % c[0] for c in FP8_RANDOM])
def test_fp8_random(fa2, case):
    """Seeded random shapes, masks, scales, rotations and quantiser block
    heights: codes and exponents bit for bit, attention against the
    dequantised oracle as above."""
    import torch
    i, B, H, N, d, causal, scale, rot, rows, seed = case
    q, k, v = wl.make_inputs(B, H, N, d, "bf16", seed=seed)
    sg = wl.make_signs(d) if rot else None
    dev = torch.device("cuda:0")
    say("fp8 random B=%d H=%d N=%d d=%d causal=%s scale=%.4f rotate=%s rows=%d"
        % (B, H, N, d, causal, scale, rot, rows))
    codes, exps = fa2.quantize_fp8(q.to(dev), rows, sg.to(dev) if sg is not None else None)
    torch.cuda.synchronize()
    c_ref, e_ref = oracle.quantize_fp8(q, rows, sg.numpy() if sg is not None else None)
    assert np.array_equal(exps.cpu().numpy(), e_ref)
    assert np.array_equal(codes.cpu().numpy(), c_ref)
    o_ref, l_ref, _ = oracle.attention_fp8_reference(
        q, k, v, scale, causal, sg.numpy() if sg is not None else None)
    odt = torch.float32 if i % 2 else torch.bfloat16
    o, lse = run_fp8(fa2, q, k, v, causal, sg, odt, scale)
    res = parity.compare_fp8(parity.to_np(o), o_ref)
    assert res["finite"] and res["rel_l2"] <= parity.FP8_REL_L2 \
        and res["max_rel"] <= parity.FP8_MAX_REL, res
    assert np.max(np.abs(parity.to_np(lse) - l_ref)) <= 1e-2
