"""The fp64 oracle against what the pages and the mathematics fix."""
import numpy as np
import pytest

import oracle
import oracle_pins
from oracle_pins import ALL_PINS


@pytest.fixture(scope="module")
def orc():
    return oracle._default()


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)


def test_thread_count_does_not_change_bits(orc):
    """Rows are independent: 1 thread and many threads give identical bits."""
    r = np.random.default_rng(11)
    q = r.standard_normal((3, 40, 16))
    k = r.standard_normal((3, 40, 16))
    v = r.standard_normal((3, 40, 16))
    o1, l1, t1 = orc.attention(q, k, v, 0.25, True, nthreads=1)
    o8, l8, t8 = orc.attention(q, k, v, 0.25, True, nthreads=8)
    assert t1 == 1 and t8 >= 1
    assert np.array_equal(o1, o8) and np.array_equal(l1, l8)


def test_bwd_threads_repeatable(orc):
    """The gradient oracle gives the same bits whatever the thread count: no
    sum is split between threads."""
    r = np.random.default_rng(5)
    q, k, v, g = (r.standard_normal((2, 77, 16)) for _ in range(4))
    a = orc.attention_bwd(q, k, v, g, 0.3, True, nthreads=3)
    b = orc.attention_bwd(q, k, v, g, 0.3, True, nthreads=3)
    c = orc.attention_bwd(q, k, v, g, 0.3, True, nthreads=1)
    for i in range(4):
        assert np.array_equal(a[i], b[i])
        assert np.array_equal(a[i], c[i])
    assert a[4] == 3 and c[4] == 1


def test_gqa_pin_rejects_an_interleaved_head_map(orc, monkeypatch):
    """A plausible mistake in the grouped-head map -- query head h using K/V
    head h % H_kv instead of h // (H / H_kv) -- fails the head-map pin."""
    import oracle as orc_mod
    from oracle_pins import pin_gqa_head_map

    def interleaved(kv, heads):
        kv = np.asarray(kv, dtype=np.float64)
        return np.tile(kv, (1,) * (kv.ndim - 3) + (heads // kv.shape[-3], 1, 1))

    monkeypatch.setattr(orc_mod, "expand_kv_heads", interleaved)
    with pytest.raises(AssertionError):
        pin_gqa_head_map(orc)


def test_gqa_bwd_pin_rejects_interleaved_group_sums(orc, monkeypatch):
    """A plausible mistake in the gradient of shared K/V heads -- summing
    query heads h, h + H_kv, ... (an interleaved group) instead of the
    consecutive group h // (H / H_kv) -- fails the finite-difference pin."""
    import oracle as orc_mod
    from oracle_pins import pin_gqa_bwd_finite_differences

    def interleaved(x, heads_kv):
        x = np.asarray(x, dtype=np.float64)
        h = x.shape[-3]
        shape = x.shape[:-3] + (h // heads_kv, heads_kv) + x.shape[-2:]
        return x.reshape(shape).sum(axis=-4)

    monkeypatch.setattr(orc_mod, "sum_kv_groups", interleaved)
    with pytest.raises(AssertionError):
        pin_gqa_bwd_finite_differences(orc)


def test_merge_reading_o2_unnormalised(orc):
    """The online-softmax section's O update weights the new block by
    e^(m2-m)/l without an l2 factor; that is only consistent if the new
    block's O2 is the unnormalised sum P~2 V.  Reading O2 as the normalised
    block output instead does not reproduce the full softmax."""
    r = np.random.default_rng(12)
    n, d = 32, 8
    q = r.standard_normal((n, d)) * 2
    k = r.standard_normal((n, d)) * 2
    v = r.standard_normal((n, d))
    o_full, _, _ = orc.attention(q[None], k[None], v[None], 0.5, False)
    o_ok, _ = oracle_pins.merge_blocks(orc, q, k, v, 0.5, [0, 13, n])
    assert np.max(np.abs(o_ok - o_full[0])) < 1e-12
    # the other reading: O2 normalised
    o1, _, _ = orc.attention(q[None], k[None, :13], v[None, :13], 0.5, False)
    o2, _, _ = orc.attention(q[None], k[None, 13:], v[None, 13:], 0.5, False)
    _, m1, l1 = orc.probs(q, k[:13], 0.5, False)
    _, m2, l2 = orc.probs(q, k[13:], 0.5, False)
    m = np.maximum(m1, m2)
    ln = l1 * np.exp(m1 - m) + l2 * np.exp(m2 - m)
    o_bad = o1[0] * (l1 * np.exp(m1 - m) / ln)[:, None] + \
        o2[0] * (np.exp(m2 - m) / ln)[:, None]
    assert np.max(np.abs(o_bad - o_full[0])) > 1e-3


def test_single_block_update_without_old_l_is_wrong_past_one_block(orc):
    """The simplified code on the unite.ai page keeps O normalised and
    updates it as (alpha*O + P~V)/l_new.  That equals the definition when the
    keys fit one block and drifts once a second block arrives (the old
    normaliser l is missing from the first term); the kernels therefore keep
    O unnormalised and divide once at the end."""
    r = np.random.default_rng(13)
    n, d, bs = 64, 8, 32
    q = r.standard_normal((n, d))
    k = r.standard_normal((n, d))
    v = r.standard_normal((n, d))
    s = 0.35 * (q @ k.T)

    def stale(nkeys):
        m = np.full(n, -np.inf)
        l = np.zeros(n)
        o = np.zeros((n, d))
        for j0 in range(0, nkeys, bs):
            sb = s[:, j0:j0 + bs]
            m_new = np.maximum(m, sb.max(axis=1))
            e = np.exp(sb - m_new[:, None])
            a = np.exp(m - m_new)
            l_new = a * l + e.sum(axis=1)
            o = (a[:, None] * o + e @ v[j0:j0 + bs]) / l_new[:, None]
            m, l = m_new, l_new
        return o

    one, _, _ = orc.attention(q[None], k[None, :bs], v[None, :bs], 0.35, False)
    two, _, _ = orc.attention(q[None], k[None], v[None], 0.35, False)
    assert np.max(np.abs(stale(bs) - one[0])) < 1e-12
    assert np.max(np.abs(stale(n) - two[0])) > 1e-2
