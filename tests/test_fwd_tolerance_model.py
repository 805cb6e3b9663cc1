"""The forward's stated element-wise bound at every scale, checked against
a rounding model of the bf16 forward kernel (CPU only; no GPU code
involved).

The model follows the kernel's arithmetic where it rounds: waves of 32
query rows, key tiles of 64 in ascending order, the base-2 reference m
raised for the whole wave only when some row's tile maximum exceeds it by
more than 8 (the lazy rescale), P~ = 2^(s log2(e) scale - m) rounded to
bf16 for P~.V, and O~ divided by the sum of those ROUNDED P~.  With a sharp
softmax (a large scale) most of the weight sits on one P~, which under the
lazy rescale lies anywhere in (1, 2^8] rather than at exactly 1; dividing by
the sum of the unrounded values would leave that P~'s bf16 rounding in O
undiluted and exceed the stated tolerance, which the model shows too.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import parity
from exact_io_aware_24_amd import inputs as wl

LOG2E = 1.0 / math.log(2.0)


def bf(x):
    return x.to(torch.bfloat16).to(torch.float64)


def lazy_model(q, k, v, scale, causal, plant=None, rounded_l=True, threshold=8.0):
    """O of the bf16 forward's rounding model; ``q`` ``[..., N, d]``, ``k``,
    ``v`` ``[..., N, d]`` with the same leading shape.  ``plant`` names a
    mistake to build in: "no_o_rescale" (l follows a raised reference but
    O~ does not) or "drop_last_tile".  ``rounded_l`` False divides by the
    sum of the unrounded P~ instead of the rounded ones.  ``threshold`` is
    the lazy rescale's margin in base-2 units (the kernel's 8; 0 raises the
    reference to the running maximum whenever some row's maximum grows)."""
    q64, k64, v64 = (torch.as_tensor(np.asarray(x, dtype=np.float64))
                     if not torch.is_tensor(x) else x.to(torch.float64)
                     for x in (q, k, v))
    n, nk = q64.shape[-2], k64.shape[-2]
    s = (q64 @ k64.transpose(-1, -2)) * (scale * LOG2E)
    if causal:
        s = s.masked_fill(torch.triu(torch.ones(n, nk, dtype=torch.bool), 1), -math.inf)
    lead = s.shape[:-2]
    s = s.reshape(-1, n, nk)
    vv = v64.reshape(-1, nk, v64.shape[-1])
    out = torch.zeros(s.shape[0], n, vv.shape[-1], dtype=torch.float64)
    tiles = list(range(0, nk, 64))
    if plant == "drop_last_tile":
        tiles = tiles[:-1]
    for r0 in range(0, n, 32):
        st = s[:, r0:r0 + 32]
        m = torch.full(st.shape[:2], -math.inf, dtype=torch.float64)
        l = torch.zeros_like(m)
        o = torch.zeros(st.shape[0], st.shape[1], vv.shape[-1], dtype=torch.float64)
        for j0 in tiles:
            t = st[:, :, j0:j0 + 64]
            mt = t.amax(-1)
            raise_ = (mt > m + threshold).any(-1, keepdim=True)
            m_new = torch.where(raise_, torch.maximum(m, mt), m)
            alpha = torch.where(raise_ & torch.isfinite(m), torch.exp2(m - m_new),
                                torch.ones_like(m))
            m = m_new
            l = l * alpha
            if plant != "no_o_rescale":
                o = o * alpha.unsqueeze(-1)
            p = torch.exp2(t - m.unsqueeze(-1)).to(torch.float32).to(torch.float64)
            l = l + (bf(p).sum(-1) if rounded_l else p.sum(-1))
            o = o + bf(p) @ vv[:, j0:j0 + 64]
        out[:, r0:r0 + 32] = o / l.unsqueeze(-1)
    return out.reshape(lead + (n, vv.shape[-1])).numpy()


def check(o, o_ref, kind):
    o = np.asarray(o, dtype=np.float64)
    if kind == "bf16":
        o = bf(torch.from_numpy(o)).numpy()
    return parity.compare(o, o_ref, None, None, kind)


# (B, H, N, d, causal, scale / (1/sqrt(d)), seed): sharp softmaxes, one of
# them the shape and scale of a GPU case that exceeded the stated bound when
# the kernel divided by the sum of the unrounded P~
SHARP = [(2, 4, 571, 128, False, 0.268091874587789 * math.sqrt(128), 638938142),
         (1, 2, 803, 128, True, 9.82, 11),
         (2, 2, 305, 64, False, 7.77, 12),
         (1, 3, 599, 64, True, 4.69, 13)]


def sharp_case(B, H, N, d, causal, rel, seed):
    q, k, v = wl.make_inputs(B, H, N, d, "bf16", seed=seed)
    scale = rel / math.sqrt(d)
    o_ref, _, _ = oracle.attention(q, k, v, scale, causal)
    return q, k, v, scale, o_ref


def test_model_within_stated_bound_at_the_stated_scale():
    for causal, N, d in ((True, 1024, 128), (False, 700, 64)):
        q, k, v = wl.make_inputs(1, 2, N, d, "bf16", seed=21)
        scale = 1 / math.sqrt(d)
        o_ref, _, _ = oracle.attention(q, k, v, scale, causal)
        o = lazy_model(q, k, v, scale, causal)
        for kind in ("bf16", "fp32"):
            res = check(o, o_ref, kind)
            assert res["ok"] and res["worst_over_bound"] < 0.75, parity.describe(res)


def test_model_within_stated_bound_at_sharp_scales():
    for case in SHARP:
        q, k, v, scale, o_ref = sharp_case(*case)
        o = lazy_model(q, k, v, scale, case[4])
        for kind in ("bf16", "fp32"):
            res = check(o, o_ref, kind)
            assert res["ok"] and res["worst_over_bound"] < 0.75, (case, kind, parity.describe(res))


def test_unrounded_normaliser_exceeds_the_bound():
    """Why O~ is divided by the sum of the rounded P~: with the unrounded
    sum the same arithmetic leaves the stated bound at sharp scales."""
    exceeded = 0
    for case in SHARP:
        q, k, v, scale, o_ref = sharp_case(*case)
        o = lazy_model(q, k, v, scale, case[4], rounded_l=False)
        for kind in ("bf16", "fp32"):
            exceeded += not check(o, o_ref, kind)["ok"]
    assert exceeded >= 3


@pytest.mark.parametrize("plant", ["no_o_rescale", "drop_last_tile"])
def test_stated_bound_rejects_planted_mistakes(plant):
    rejected = 0
    for case in SHARP:
        q, k, v, scale, o_ref = sharp_case(*case)
        o = lazy_model(q, k, v, scale, case[4], plant=plant)
        rejected += not check(o, o_ref, "fp32")["ok"]
    assert rejected == len(SHARP)


# Two forward draws of a one-off GPU run of the random-shape checks (seeds
# other than the committed ones) whose bf16 outputs exceeded the element
# bound, both at scales about seven times 1/sqrt(d):
# (B, H, H_kv, N, d, causal, scale, seed, b, h, GPU worst / bound), where
# (b, h) is the head that holds the worst element.
SHARPEST = [(2, 6, 2, 382, 64, True, 0.8472718645335111, 948904470, 0, 5, 1.196),
            (2, 12, 3, 566, 128, False, 0.8935182584416261, 259570758, 1, 2, 1.010)]


@pytest.mark.parametrize("case", SHARPEST, ids=["d64_causal", "d128"])
def test_lazy_reference_at_very_sharp_scales(case):
    """A limit of the lazy rescale, pinned: when two keys of similar weight
    dominate a row and the later one exceeds the wave's reference by less
    than the threshold, neither P~ is exactly 1, both are rounded to bf16,
    and the rounding of the weights plus that of the bf16 output can pass
    the element bound.  The model reproduces the GPU's figure for both
    draws (to the printed digits); with the reference kept at the running
    maximum (threshold 0) the dominant P~ is exactly 1 and the same heads
    stay well inside the bound."""
    B, H, Hk, N, d, causal, scale, seed, b, h, gpu_worst = case
    q, k, v = wl.make_inputs(B, H, N, d, "bf16", seed=seed, H_kv=Hk)
    kx = oracle.expand_kv_heads(k, H)[b:b + 1, h:h + 1]
    vx = oracle.expand_kv_heads(v, H)[b:b + 1, h:h + 1]
    qs = q[b:b + 1, h:h + 1]
    o_ref, _, _ = oracle.attention(qs, kx, vx, scale, causal)
    lazy = check(lazy_model(qs, kx, vx, scale, causal), o_ref, "bf16")
    assert abs(lazy["worst_over_bound"] - gpu_worst) < 1e-3, parity.describe(lazy)
    assert lazy["worst_over_bound"] > 1.0
    exact = check(lazy_model(qs, kx, vx, scale, causal, threshold=0.0), o_ref, "bf16")
    assert exact["ok"] and exact["worst_over_bound"] < 0.75, parity.describe(exact)
