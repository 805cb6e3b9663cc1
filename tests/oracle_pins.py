"""Pins for the fp64 attention oracle.

Each ``pin_*`` function takes an oracle object (``oracle.OracleLib``) and
raises ``AssertionError`` when the oracle disagrees with something fixed
outside the oracle itself: a closed form, an invariant of softmax attention,
the two-block merge rule printed on the pages, or a brute-force evaluation
written differently (no max subtraction, ``math.fsum``) on tiny inputs.

The same functions run against the real oracle (``test_oracle_pins.py``) and
against deliberately broken copies of it (``test_oracle_mutants.py``), which
shows that each plausible mistake is caught by at least one pin.
"""
from __future__ import annotations

import math

import numpy as np

TOL = 1e-12


def _rng(seed):
    return np.random.default_rng(seed)


def _close(a, b, tol=TOL, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    assert np.all(np.isfinite(a)) and np.all(np.isfinite(b)), what
    err = np.max(np.abs(a - b)) if a.size else 0.0
    scale = max(1.0, float(np.max(np.abs(b))) if b.size else 1.0)
    assert err <= tol * scale, "%s: max |diff| %.3e" % (what, err)


# ---------------------------------------------------------------------------
# softmax step


def pin_rows_sum_to_one(orc):
    """Every probability row is non-negative and sums to 1; masked entries
    (causal, key after query) are exactly 0."""
    r = _rng(1)
    for causal in (False, True):
        q = r.standard_normal((37, 16))
        k = r.standard_normal((37, 16)) * 3
        p, m, l = orc.probs(q, k, 0.25, causal)
        assert np.all(p >= 0)
        _close(p.sum(axis=1), np.ones(37), what="row sums")
        if causal:
            assert np.all(np.triu(p, 1) == 0.0), "masked entries non-zero"
            assert np.all(np.diag(p) > 0), "diagonal masked"


def pin_probs_closed_form_two_keys(orc):
    """Two keys: p = logistic(s1 - s2), the textbook closed form; the row
    maximum and l = 1 + exp(-|s1 - s2|) follow as well."""
    q = np.array([[1.5, -0.5, 2.0]])
    k = np.array([[0.3, 1.0, -0.7], [-1.2, 0.4, 0.9]])
    scale = 0.7
    s = [scale * float(np.dot(q[0], k[j])) for j in range(2)]
    p, m, l = orc.probs(q, k, scale, False)
    p0 = 1.0 / (1.0 + math.exp(s[1] - s[0]))
    _close(p[0], [p0, 1.0 - p0], what="two-key probabilities")
    _close(m, [max(s)], what="row max")
    _close(l, [1.0 + math.exp(-abs(s[0] - s[1]))], what="row l")


# ---------------------------------------------------------------------------
# whole pipeline: closed forms


def pin_zero_query_is_mean_of_v(orc):
    """Q = 0 makes every score 0: attention is uniform over the visible keys,
    so O is the mean of V (causal: the mean of rows 0..i) and lse = ln(count).
    scale = 0 with any Q gives the same."""
    r = _rng(2)
    n, d = 23, 8
    v = r.standard_normal((1, n, d))
    k = r.standard_normal((1, n, d))
    for q, scale in ((np.zeros((1, n, d)), 0.37),
                     (r.standard_normal((1, n, d)), 0.0)):
        o, lse, _ = orc.attention(q, k, v, scale, False)
        _close(o[0], np.broadcast_to(v[0].mean(axis=0), (n, d)), what="mean V")
        _close(lse[0], np.full(n, math.log(n)), what="ln N")
        o, lse, _ = orc.attention(q, k, v, scale, True)
        prefix = np.cumsum(v[0], axis=0) / np.arange(1, n + 1)[:, None]
        _close(o[0], prefix, what="prefix mean V")
        _close(lse[0], np.log(np.arange(1, n + 1)), what="ln(i+1)")


def pin_constant_v_column(orc):
    """A V column that is the same constant for every key comes out
    unchanged in every output row (the weights sum to 1)."""
    r = _rng(3)
    n, d = 31, 6
    q = r.standard_normal((2, n, d)) * 2
    k = r.standard_normal((2, n, d)) * 2
    v = r.standard_normal((2, n, d))
    v[:, :, 2] = -3.25
    v[:, :, 5] = 7.0
    for causal in (False, True):
        o, _, _ = orc.attention(q, k, v, 0.5, causal)
        _close(o[:, :, 2], np.full((2, n), -3.25), what="const col 2")
        _close(o[:, :, 5], np.full((2, n), 7.0), what="const col 5")


def pin_single_key(orc):
    """With one key the only weight is 1: O = v_0 and lse = scale*q.k_0."""
    r = _rng(4)
    d = 5
    q = r.standard_normal((3, 1, d))
    k = r.standard_normal((3, 1, d))
    v = r.standard_normal((3, 1, d))
    o, lse, _ = orc.attention(q, k, v, 1.3, False)
    _close(o, v, what="O = V")
    _close(lse[:, 0], 1.3 * np.einsum("hd,hd->h", q[:, 0], k[:, 0]),
           what="lse = scale q.k")


def pin_dominant_key(orc):
    """When one key's score exceeds all others by > 750 every other weight
    underflows to exactly 0 in double precision: O is that key's V row and
    lse is its score (no overflow even for scores near 1e4)."""
    d, n = 4, 9
    k = np.zeros((1, n, d))
    for j in range(n):
        k[0, j, 0] = float(j)  # key j has first component j
    q = np.zeros((1, 1, d))
    q[0, 0, 0] = 1000.0
    v = np.arange(n * d, dtype=np.float64).reshape(1, n, d)
    o, lse, _ = orc.attention(q, k, v, 1.0, False)
    _close(o[0, 0], v[0, n - 1], what="dominant key O")
    _close(lse[0], [1000.0 * (n - 1)], what="dominant key lse")


# ---------------------------------------------------------------------------
# invariants


def pin_key_shift(orc):
    """Adding one vector u to every key adds scale*q_i.u to every score of
    row i: O is unchanged and lse moves by exactly that amount."""
    r = _rng(5)
    n, d = 19, 7
    q = r.standard_normal((1, n, d))
    k = r.standard_normal((1, n, d))
    v = r.standard_normal((1, n, d))
    u = r.standard_normal(d) * 2
    for causal in (False, True):
        o1, l1, _ = orc.attention(q, k, v, 0.6, causal)
        o2, l2, _ = orc.attention(q, k + u, v, 0.6, causal)
        _close(o2, o1, tol=1e-11, what="shift O")
        _close(l2[0] - l1[0], 0.6 * (q[0] @ u), tol=1e-11, what="shift lse")


def pin_key_permutation(orc):
    """Without a mask attention is a sum over keys: permuting the K and V
    rows together leaves O and lse unchanged."""
    r = _rng(6)
    n, d = 29, 8
    q = r.standard_normal((2, n, d))
    k = r.standard_normal((2, n, d))
    v = r.standard_normal((2, n, d))
    perm = r.permutation(n)
    o1, l1, _ = orc.attention(q, k, v, 0.4, False)
    o2, l2, _ = orc.attention(q, k[:, perm], v[:, perm], 0.4, False)
    _close(o2, o1, what="perm O")
    _close(l2, l1, what="perm lse")


def pin_causal_consistency(orc):
    """The causal mask hides nothing from the last row and everything but
    key 0 from row 0."""
    r = _rng(7)
    n, d = 17, 6
    q = r.standard_normal((1, n, d))
    k = r.standard_normal((1, n, d))
    v = r.standard_normal((1, n, d))
    oc, lc, _ = orc.attention(q, k, v, 0.8, True)
    on, ln, _ = orc.attention(q, k, v, 0.8, False)
    _close(oc[0, n - 1], on[0, n - 1], what="last row")
    _close(lc[0, n - 1], ln[0, n - 1], what="last row lse")
    _close(oc[0, 0], v[0, 0], what="row 0 = v0")
    _close(lc[0, 0], 0.8 * (q[0, 0] @ k[0, 0]), what="row 0 lse")
    # causal row i equals non-causal attention over the prefix 0..i
    for i in (3, 9):
        op, lp, _ = orc.attention(q[:, i:i + 1], k[:, :i + 1], v[:, :i + 1],
                                  0.8, False)
        _close(oc[0, i], op[0, 0], what="prefix row %d" % i)
        _close(lc[0, i], lp[0, 0], what="prefix lse %d" % i)


# ---------------------------------------------------------------------------
# the online-softmax merge printed on the pages


def merge_blocks(orc, q, k, v, scale, bounds):
    """Fold per-block results with the two-block merge rule of the online
    softmax section: m = max(m1, m2), l = l1 e^(m1-m) + l2 e^(m2-m),
    O = O1 (l1 e^(m1-m) / l) + O2 (e^(m2-m) / l), where O1 is the normalised
    output so far and O2 the new block's unnormalised sum P~2 V."""
    m_acc = l_acc = o_acc = None
    for lo, hi in zip(bounds[:-1], bounds[1:]):
        kb, vb = k[lo:hi], v[lo:hi]
        ob, _, _ = orc.attention(q[None], kb[None], vb[None], scale, False)
        _, mb, lb = orc.probs(q, kb, scale, False)
        ob = ob[0] * lb[:, None]  # unnormalised block output P~ V
        if m_acc is None:
            m_acc, l_acc, o_acc = mb, lb, ob / lb[:, None]
            continue
        m_new = np.maximum(m_acc, mb)
        a1 = np.exp(m_acc - m_new)
        a2 = np.exp(mb - m_new)
        l_new = l_acc * a1 + lb * a2
        o_acc = o_acc * (l_acc * a1 / l_new)[:, None] + ob * (a2 / l_new)[:, None]
        m_acc, l_acc = m_new, l_new
    return o_acc, m_acc + np.log(l_acc)


def pin_online_merge(orc):
    """Splitting each row's keys into 2..8 blocks at random points and
    folding the blocks with the printed merge rule gives the full result."""
    r = _rng(8)
    n, d = 64, 12
    q = r.standard_normal((n, d)) * 2
    k = r.standard_normal((n, d)) * 2
    v = r.standard_normal((n, d))
    o_full, l_full, _ = orc.attention(q[None], k[None], v[None], 0.5, False)
    for nblocks in (2, 3, 5, 8):
        cuts = np.sort(r.choice(np.arange(1, n), nblocks - 1, replace=False))
        bounds = [0] + list(cuts) + [n]
        o_m, l_m = merge_blocks(orc, q, k, v, 0.5, bounds)
        _close(o_m, o_full[0], what="merge O (%d blocks)" % nblocks)
        _close(l_m, l_full[0], what="merge lse (%d blocks)" % nblocks)


# ---------------------------------------------------------------------------
# brute force


def brute_force(q, k, v, scale, causal):
    """sum_j e^(s_ij) v_j / sum_j e^(s_ij), summed with math.fsum, with no
    maximum subtracted (inputs are kept small so nothing overflows)."""
    nq, d = q.shape
    nk = k.shape[0]
    o = np.zeros((nq, d))
    lse = np.zeros(nq)
    for i in range(nq):
        w = []
        for j in range(nk):
            if causal and j > i:
                continue
            s = scale * math.fsum(float(q[i, c]) * float(k[j, c]) for c in range(d))
            w.append((j, math.exp(s)))
        z = math.fsum(x for _, x in w)
        for c in range(d):
            o[i, c] = math.fsum(x * float(v[j, c]) for j, x in w) / z
        lse[i] = math.log(z)
    return o, lse


def pin_brute_force(orc):
    """Tiny shapes, including Nq != Nk and d != N, against the brute force."""
    r = _rng(9)
    for (nq, nk, d, causal) in ((1, 1, 1, False), (5, 5, 3, True),
                                (7, 11, 4, False), (16, 16, 8, True),
                                (16, 16, 8, False), (9, 4, 2, False)):
        q = r.standard_normal((nq, d))
        k = r.standard_normal((nk, d))
        v = r.standard_normal((nk, d))
        if causal and nq > nk:
            continue
        o, lse, _ = orc.attention(q[None], k[None], v[None], 0.45, causal)
        ob, lb = brute_force(q, k, v, 0.45, causal)
        _close(o[0], ob, what="brute O %s" % ((nq, nk, d, causal),))
        _close(lse[0], lb, what="brute lse %s" % ((nq, nk, d, causal),))


def pin_rows_match_full(orc):
    """The selected-rows entry point gives the same rows as the full one."""
    r = _rng(10)
    n, d = 50, 8
    q = r.standard_normal((n, d))
    k = r.standard_normal((n, d))
    v = r.standard_normal((n, d))
    rows = np.array([0, 1, 13, 48, 49, 7])
    for causal in (False, True):
        o, lse, _ = orc.attention(q[None], k[None], v[None], 0.3, causal)
        orow, lrow, _ = orc.attention_rows(q[rows], rows, k, v, 0.3, causal)
        _close(orow, o[0, rows], tol=0, what="rows O")
        _close(lrow, lse[0, rows], tol=0, what="rows lse")


def pin_gqa_head_map(orc):
    """Grouped K/V heads: with every value row of K/V head g equal to the
    constant g + 1, the output of query head h is exactly h // (H / H_kv) + 1
    (a constant V passes through the softmax), which fixes the head map; with
    H_kv = H the grouped call is the plain one."""
    import oracle as orc_mod
    r = _rng(30)
    B, H, Hk, N, d = 2, 6, 2, 9, 4
    q = r.standard_normal((B, H, N, d))
    k = r.standard_normal((B, Hk, N, d))
    v = np.empty((B, Hk, N, d))
    for g in range(Hk):
        v[:, g] = g + 1.0
    kx = orc_mod.expand_kv_heads(k, H)
    vx = orc_mod.expand_kv_heads(v, H)
    o, _, _ = orc.attention(q, kx, vx, 0.5, True)
    for h in range(H):
        _close(o[:, h], np.full((B, N, d), h // (H // Hk) + 1.0), what="gqa head %d" % h)
    k2 = r.standard_normal((B, H, N, d))
    assert np.array_equal(orc_mod.expand_kv_heads(k2, H), k2)


def pin_offset_causal(orc):
    """Causal mask with more keys than queries (query i at key position
    i + Nk - Nq): with Nq = Nk it is the plain causal mask; the last query
    sees every key (equals the unmasked row); rows before the first key
    position see nothing (O = 0, lse = -inf); and each row equals the
    brute-force softmax over its visible keys."""
    import oracle as orc_mod
    r = _rng(31)
    q = r.standard_normal((2, 7, 5))
    k = r.standard_normal((2, 11, 5))
    v = r.standard_normal((2, 11, 5))
    o, lse, _ = orc_mod.attention_offset(q, k, v, 0.6, True)
    ou, lu, _ = orc.attention(q, k, v, 0.6, False)
    _close(o[:, -1], ou[:, -1], what="last row")
    _close(lse[:, -1], lu[:, -1], what="last lse")
    for h in range(2):
        for i in range(7):
            vis = 11 - 7 + i + 1
            s = 0.6 * k[h, :vis] @ q[h, i]
            w = np.exp(s - s.max())
            _close(o[h, i], (w / w.sum()) @ v[h, :vis], what="row %d" % i)
    sq, _, _ = orc_mod.attention_offset(q, k[:, :7], v[:, :7], 0.6, True)
    sq2, _, _ = orc.attention(q, k[:, :7], v[:, :7], 0.6, True)
    _close(sq, sq2, tol=0, what="square")
    o3, l3, _ = orc_mod.attention_offset(k, q, q, 0.6, True)  # 11 queries, 7 keys
    assert np.all(o3[:, :4] == 0) and np.all(np.isneginf(l3[:, :4]))


def pin_fwht_is_hadamard(orc):
    """The fast transform equals multiplication by the Sylvester Hadamard
    matrix (built with Kronecker products) on small integers, where float32
    is exact; applying it twice gives d times the input."""
    import oracle as orc_mod
    r = _rng(40)
    for d in (8, 64, 128):
        H = np.array([[1.0]])
        while H.shape[0] < d:
            H = np.kron(H, np.array([[1.0, 1.0], [1.0, -1.0]]))
        x = r.integers(-50, 50, (5, d)).astype(np.float32)
        y = orc_mod.fwht_f32(x)
        assert np.array_equal(y.astype(np.float64), x.astype(np.float64) @ H), d
        assert np.array_equal(orc_mod.fwht_f32(y), x * d), d


def pin_e4m3_codes(orc):
    """e4m3 (OCP FP8: bias 7, 3 mantissa bits, no infinities, max 448) by
    its definition: the codes of 1, 2, 448, the smallest normal 2^-6 and the
    smallest subnormal 2^-9; round to nearest even at ties (1 + 1/16 -> 1,
    1 + 3/16 -> 1 + 1/4); values past 448 but below the next rounding
    boundary 464 -> 448."""
    import oracle as orc_mod
    vals = np.array([1.0, 2.0, 448.0, 2.0 ** -6, 2.0 ** -9, -1.0, 0.0,
                     1.0625, 1.1875, 450.0, 3.0 * 2.0 ** -9], dtype=np.float32)
    want = [0x38, 0x40, 0x7E, 0x08, 0x01, 0xB8, 0x00, 0x38, 0x3A, 0x7E, 0x03]
    assert orc_mod.to_e4m3_codes(vals).tolist() == want
    assert np.array_equal(orc_mod.e4m3_values(np.array(want, dtype=np.uint8)),
                          np.array([1, 2, 448, 2.0 ** -6, 2.0 ** -9, -1, 0, 1,
                                    1.25, 448, 3.0 * 2.0 ** -9]))


def pin_block_exponent(orc):
    """The block scale exponent is the smallest e with amax <= 448 * 2^e."""
    import oracle as orc_mod
    a = np.array([448.0, 448.5, 224.0, 224.25, 1.0, 0.875, 0.0, 3.5e-5, 7e4])
    e = orc_mod.block_exponent(a)
    assert e.tolist() == [0, 1, -1, 0, -8, -9, 0, -23, 8], e.tolist()
    for ai, ei in zip(a[a > 0], e[a > 0]):
        assert ai <= 448 * 2.0 ** ei and ai > 448 * 2.0 ** (ei - 1)


def pin_fp8_quantize_error(orc):
    """Block quantisation error: each dequantised value is within half an
    e4m3 step of its (rotated) input -- 2^-4 relative for normals, 2^-10
    times the block scale below them -- and every block uses the top of the
    e4m3 range; with the rotation, inner products of rows are those of the
    unrotated rows times d (the transform is d^(1/2) times orthogonal)."""
    import oracle as orc_mod
    r = _rng(41)
    x = r.standard_normal((3, 200, 64)).astype(np.float32)
    x[:, 7] *= 30.0
    signs = r.choice([-1.0, 1.0], 64)
    for sg in (None, signs):
        c, e = orc_mod.quantize_fp8(x, 64, sg)
        y = orc_mod.fwht_f32(x * sg) if sg is not None else x
        dq = orc_mod.dequantize_fp8(c, e, 64)
        scale = np.exp2(np.repeat(e, 64, axis=-1)[..., :200])[..., None]
        tol = np.maximum(np.abs(y) * 2.0 ** -4, scale * 2.0 ** -10)
        assert np.all(np.abs(dq - y) <= tol + 1e-30)
        amax_codes = np.abs(orc_mod.e4m3_values(c)).reshape(3, -1)
        assert np.all(amax_codes.max(axis=1) >= 224)
    yq = orc_mod.fwht_f32(x[0] * signs).astype(np.float64)
    _close(yq @ yq.T, 64.0 * (x[0].astype(np.float64) @ x[0].T.astype(np.float64)),
           tol=1e-6, what="rotation inner products")


def pin_fp8_block_grouping(orc):
    """Which rows share a scale.  Blocks are runs of ``block_rows``
    consecutive rows of one head, the last one possibly short.  A value
    planted in row r of one head, far above every other magnitude, must move
    exactly block r // R of that head, to the closed-form exponent of the
    planted value (1000: 448 * 2^1 < 1000 <= 448 * 2^2, so e = 2), and leave
    every other block of every head with its codes and exponent unchanged --
    with and without the rotation (which spreads the value over its row, so
    the block maximum stays within 1000 +- 0.64 here).  And every block uses
    the top of the e4m3 range: its largest code magnitude is at least 224
    (the block maximum scaled into (224, 448], then rounded)."""
    import oracle as orc_mod
    r = _rng(43)
    n, d = 200, 64
    x = (r.uniform(-0.01, 0.01, (2, 3, n, d))).astype(np.float32)
    signs = r.choice([-1.0, 1.0], d)
    for sg in (None, signs):
        for R in (64, 128):
            nb = -(-n // R)
            c0, e0 = orc_mod.quantize_fp8(x, R, sg)
            assert e0.shape == (2, 3, nb), e0.shape
            vals = np.abs(orc_mod.e4m3_values(c0))
            for b in range(nb):
                top = vals[..., b * R:min(n, (b + 1) * R), :].max(axis=(-2, -1))
                assert np.all(top >= 224), (R, b, top)
            for (bi, hi, row) in ((0, 0, 0), (1, 2, R - 1), (0, 1, R),
                                  (1, 0, n - 1), (0, 2, 131)):
                xp = x.copy()
                xp[bi, hi, row, 5] = 1000.0
                c1, e1 = orc_mod.quantize_fp8(xp, R, sg)
                blk = row // R
                assert e1[bi, hi, blk] == 2, (R, row, e1[bi, hi, blk])
                moved = np.argwhere(e1 != e0)
                assert [tuple(m) for m in moved] == [(bi, hi, blk)], (R, row, moved)
                same = np.ones(c0.shape, dtype=bool)
                same[bi, hi, blk * R:min(n, (blk + 1) * R)] = False
                assert np.array_equal(c1[same], c0[same]), (R, row)


# ---------------------------------------------------------------------------
# gradients


def _loss(orc, q, k, v, g, scale, causal):
    """L = sum(O * g): its gradient with respect to O is g."""
    o, _, _ = orc.attention(q, k, v, scale, causal)
    return float(np.sum(o * g))


def pin_bwd_finite_differences(orc):
    """Every gradient entry matches the central difference of the forward
    oracle's loss sum(O * dO): d/dx is read off the forward definition by
    perturbing x, independently of how the gradient formula is written."""
    r = _rng(20)
    h = 1e-5
    for nh, nq, nk, d, scale, causal in ((1, 5, 5, 3, 0.8, False),
                                         (2, 4, 4, 3, -1.1, True),
                                         (1, 3, 6, 2, 0.5, False),
                                         (1, 1, 1, 2, 0.9, False),
                                         (1, 6, 6, 4, 1.3, True)):
        q = r.standard_normal((nh, nq, d))
        k = r.standard_normal((nh, nk, d))
        v = r.standard_normal((nh, nk, d))
        g = r.standard_normal((nh, nq, d))
        dq, dk, dv, _, _ = orc.attention_bwd(q, k, v, g, scale, causal)
        for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
            num = np.empty_like(x)
            for idx in np.ndindex(x.shape):
                x0 = x[idx]
                x[idx] = x0 + h
                lp = _loss(orc, q, k, v, g, scale, causal)
                x[idx] = x0 - h
                lm = _loss(orc, q, k, v, g, scale, causal)
                x[idx] = x0
                num[idx] = (lp - lm) / (2 * h)
            _close(grad, num, tol=1e-7, what="d%s finite differences %s"
                   % (name, (nh, nq, nk, d, scale, causal)))


def pin_gqa_bwd_finite_differences(orc):
    """Grouped K/V heads: every entry of dQ, dK, dV matches the central
    difference of the grouped forward's loss sum(O * dO), so the shared K/V
    gradients carry the contributions of exactly the query heads that read
    them (grouped-query and multi-query cases, causal and not)."""
    import oracle as orc_mod
    r = _rng(22)
    h = 1e-5
    for B, H, Hk, n, d, scale, causal in ((1, 4, 2, 4, 3, 0.7, True),
                                          (2, 3, 1, 3, 2, -0.9, False),
                                          (1, 6, 3, 3, 2, 1.1, True)):
        q = r.standard_normal((B, H, n, d))
        k = r.standard_normal((B, Hk, n, d))
        v = r.standard_normal((B, Hk, n, d))
        g = r.standard_normal((B, H, n, d))
        dq, dk, dv, _, _ = orc_mod.attention_bwd_gqa(q, k, v, g, scale, causal)

        def loss():
            o, _, _ = orc_mod.attention_gqa(q, k, v, scale, causal)
            return float(np.sum(o * g))

        for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
            num = np.empty_like(x)
            for idx in np.ndindex(x.shape):
                x0 = x[idx]
                x[idx] = x0 + h
                lp = loss()
                x[idx] = x0 - h
                lm = loss()
                x[idx] = x0
                num[idx] = (lp - lm) / (2 * h)
            _close(grad, num, tol=1e-7, what="gqa d%s finite differences %s"
                   % (name, (B, H, Hk, n, d, scale, causal)))


def pin_bwd_sums(orc):
    """Rows of P sum to one, so sum_j dV_j = sum_i dO_i; the softmax is
    unchanged by a common shift of a row's logits, so sum_j dS_ij = 0 and
    sum_j dK_j = 0."""
    r = _rng(21)
    for causal in (False, True):
        q = r.standard_normal((2, 40, 8))
        k = r.standard_normal((2, 40, 8)) * 2
        v = r.standard_normal((2, 40, 8))
        g = r.standard_normal((2, 40, 8))
        _, dk, dv, _, _ = orc.attention_bwd(q, k, v, g, 0.6, causal)
        _close(dv.sum(axis=1), g.sum(axis=1), what="sum dV")
        _close(dk.sum(axis=1), np.zeros((2, 8)), what="sum dK")


def pin_bwd_constant_v(orc):
    """All value rows equal: O does not depend on Q or K, so dQ = dK = 0."""
    r = _rng(22)
    for causal in (False, True):
        q = r.standard_normal((1, 30, 6))
        k = r.standard_normal((1, 30, 6))
        v = np.tile(r.standard_normal((1, 1, 6)), (1, 30, 1))
        g = r.standard_normal((1, 30, 6))
        dq, dk, _, _, _ = orc.attention_bwd(q, k, v, g, 0.9, causal)
        _close(dq, np.zeros_like(dq), what="dQ constant V")
        _close(dk, np.zeros_like(dk), what="dK constant V")


def pin_bwd_zero_scale(orc):
    """scale = 0: uniform attention over the visible keys; dQ = dK = 0 and
    dV_j = sum over the rows i that see key j of dO_i / (number of keys row
    i sees) -- 1/N for every row without a mask, 1/(i+1) with it."""
    r = _rng(23)
    n, d = 12, 5
    q = r.standard_normal((1, n, d))
    k = r.standard_normal((1, n, d))
    v = r.standard_normal((1, n, d))
    g = r.standard_normal((1, n, d))
    for causal in (False, True):
        dq, dk, dv, _, _ = orc.attention_bwd(q, k, v, g, 0.0, causal)
        _close(dq, np.zeros_like(dq), what="dQ scale 0")
        _close(dk, np.zeros_like(dk), what="dK scale 0")
        want = np.zeros((n, d))
        for j in range(n):
            for i in range(n):
                if causal and j > i:
                    continue
                want[j] += g[0, i] / ((i + 1) if causal else n)
        _close(dv[0], want, what="dV scale 0")


def pin_bwd_delta_is_dout_dot_o(orc):
    """D_i = sum_j P_ij dP_ij equals dO_i . O_i because O_i = sum_j P_ij V_j
    (the identity a tiled backward uses to get D without P)."""
    r = _rng(24)
    for causal in (False, True):
        q = r.standard_normal((2, 25, 7))
        k = r.standard_normal((2, 25, 7))
        v = r.standard_normal((2, 25, 7))
        g = r.standard_normal((2, 25, 7))
        o, _, _ = orc.attention(q, k, v, 0.4, causal)
        _, _, _, delta, _ = orc.attention_bwd(q, k, v, g, 0.4, causal)
        _close(delta, np.sum(g * o, axis=-1), what="delta")


def pin_bwd_causal_first_row_and_single_key(orc):
    """Causal row 0 sees one key, so its P is the constant 1 and dQ_0 = 0;
    with a single key everywhere, dV_0 = sum_i dO_i and dQ = dK = 0."""
    r = _rng(25)
    q = r.standard_normal((1, 9, 4))
    k = r.standard_normal((1, 9, 4))
    v = r.standard_normal((1, 9, 4))
    g = r.standard_normal((1, 9, 4))
    dq, _, _, _, _ = orc.attention_bwd(q, k, v, g, 0.7, True)
    _close(dq[0, 0], np.zeros(4), what="causal dQ row 0")
    dq, dk, dv, _, _ = orc.attention_bwd(q, k[:, :1], v[:, :1], g, 0.7, False)
    _close(dv[0, 0], g[0].sum(axis=0), what="single key dV")
    _close(dq, np.zeros_like(dq), what="single key dQ")
    _close(dk, np.zeros_like(dk), what="single key dK")


def pin_bwd_linear_in_dout(orc):
    """The gradients are linear in the incoming gradient dO."""
    r = _rng(26)
    q = r.standard_normal((1, 20, 6))
    k = r.standard_normal((1, 20, 6))
    v = r.standard_normal((1, 20, 6))
    g1 = r.standard_normal((1, 20, 6))
    g2 = r.standard_normal((1, 20, 6))
    a = orc.attention_bwd(q, k, v, g1, 0.5, True)
    b = orc.attention_bwd(q, k, v, g2, 0.5, True)
    c = orc.attention_bwd(q, k, v, g1 + 2 * g2, 0.5, True)
    for i, name in enumerate(("dq", "dk", "dv")):
        _close(c[i], a[i] + 2 * b[i], what="linearity " + name)


ALL_PINS = [
    pin_rows_sum_to_one,
    pin_probs_closed_form_two_keys,
    pin_zero_query_is_mean_of_v,
    pin_constant_v_column,
    pin_single_key,
    pin_dominant_key,
    pin_key_shift,
    pin_key_permutation,
    pin_causal_consistency,
    pin_online_merge,
    pin_brute_force,
    pin_rows_match_full,
    pin_gqa_head_map,
    pin_offset_causal,
    pin_fwht_is_hadamard,
    pin_e4m3_codes,
    pin_block_exponent,
    pin_fp8_quantize_error,
    pin_fp8_block_grouping,
    pin_bwd_finite_differences,
    pin_gqa_bwd_finite_differences,
    pin_bwd_sums,
    pin_bwd_constant_v,
    pin_bwd_zero_scale,
    pin_bwd_delta_is_dout_dot_o,
    pin_bwd_causal_first_row_and_single_key,
    pin_bwd_linear_in_dout,
]
