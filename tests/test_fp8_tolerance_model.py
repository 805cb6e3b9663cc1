"""The FP8 tolerances of parity.py, checked against a rounding model of the
FP8 kernel (CPU only).  The model takes the oracle's block-quantised
inputs, computes the scores exactly, rounds the probabilities (relative to
the row maximum) to e4m3 before P.V and the output to bf16.  It also shows
the point of incoherent processing: with outlier channels the rotation cuts
the end-to-end error several times."""
import math

import numpy as np
import pytest
import torch

import oracle
import parity
from exact_io_aware_24_amd import inputs as wl


def model(q, k, v, scale, causal, signs):
    o_ref, _, codes = oracle.attention_fp8_reference(q, k, v, scale, causal, signs)
    (q8, qe), (k8, ke), (v8, ve) = codes
    d = q.shape[-1]
    qd = oracle.dequantize_fp8(q8, qe, 128)
    kd = oracle.dequantize_fp8(k8, ke, 64)
    vd = oracle.dequantize_fp8(v8, ve, 64)
    s = np.einsum("bhqd,bhkd->bhqk", qd, kd) * (scale / d if signs is not None else scale)
    n = s.shape[-1]
    if causal:
        s = np.where(np.triu(np.ones((n, n), bool), 1), -np.inf, s)
    p = np.exp(s - s.max(-1, keepdims=True))
    pq = oracle.e4m3_values(oracle.to_e4m3_codes(p.astype(np.float32)))
    o = np.einsum("bhqk,bhkd->bhqd", pq, vd) / p.sum(-1, keepdims=True)
    o = torch.from_numpy(o).to(torch.bfloat16).double().numpy()
    o_exact, _, _ = oracle.attention(q, k, v, scale, causal)
    return parity.compare_fp8(o, o_ref), parity.compare_fp8(o, o_exact)


@pytest.mark.parametrize("N,d,causal", [(512, 128, False), (512, 128, True), (384, 64, True)])
def test_model_within_half_the_bounds(N, d, causal):
    q, k, v = wl.make_inputs(1, 2, N, d, "bf16")
    signs = wl.make_signs(d).numpy()
    for sg in (None, signs):
        par, e2e = model(q, k, v, 1 / math.sqrt(d), causal, sg)
        assert par["rel_l2"] <= parity.FP8_REL_L2 / 2, par
        assert par["max_rel"] <= parity.FP8_MAX_REL / 2, par
        assert e2e["rel_l2"] <= parity.FP8_E2E_REL_L2 / 2, e2e


def channel_outliers(d, chans=(3, 17), factor=20.0):
    q, k, v = wl.make_inputs(1, 2, 512, d, "bf16")
    q, k = q.float(), k.float()
    for ch in chans + (d - 5,):
        q[..., ch] *= factor
        k[..., ch] *= factor
    return q.to(torch.bfloat16), k.to(torch.bfloat16), v


@pytest.mark.parametrize("d", [64, 128])
def test_rotation_helps_with_outlier_channels(d):
    q, k, v = channel_outliers(d)
    plain = model(q, k, v, 1 / math.sqrt(d), True, None)[1]
    rot = model(q, k, v, 1 / math.sqrt(d), True, wl.make_signs(d).numpy())[1]
    assert rot["rel_l2"] <= parity.FP8_E2E_ROT_OUTLIER_REL_L2 / 1.5, rot
    assert plain["rel_l2"] > 2.5 * rot["rel_l2"], (plain, rot)
