"""Pins of the CPU oracle against what the pages and the mathematics fix.

Every check here compares the oracle with something other than itself: a
count or example the RAM-Net pages print (tests/golden/), a closed form, an
invariant the pages state, a special case that reduces to a library routine,
or brute force on tiny inputs.  "Project page" is the RAM-Net project page
(muoncat.github.io/ramnet_web); paragraph names follow its topics.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- Product Softmax

@pytest.mark.parametrize("d_p,U", [(2, 1), (2, 6), (3, 4), (4, 5), (5, 3), (4, 2)])
def test_weights_sum_to_one(orc, d_p, U):
    """Project page, 'Product Softmax': the slot distribution is a product of
    U digit distributions, so it sums to one over all M slots."""
    r = rng(1)
    for _ in range(5):
        lg = (r.standard_normal(U * d_p) * 3).astype(np.float32)
        W = orc.slot_weights(lg, U, d_p)
        assert W.shape == (d_p ** U,)
        assert abs(W.sum() - 1.0) < 1e-12
        assert (W > 0).all()


def test_two_value_digit_is_logistic(orc):
    """d_p = 2: a softmax over two logits is the logistic function of their
    difference (closed form)."""
    r = rng(2)
    for _ in range(20):
        lg = (r.standard_normal(6) * 4).astype(np.float32)
        probs, _ = orc.digit_probs(lg, 3, 2)
        for u in range(3):
            a, b = float(lg[2 * u]), float(lg[2 * u + 1])
            p1 = 1.0 / (1.0 + math.exp(a - b))
            assert abs(probs[u, 1] - p1) < 1e-15
            assert abs(probs[u, 0] - (1 - p1)) < 1e-15


def test_scores_per_address_golden(orc):
    """Project page, 'Product Softmax': M = 1024 = 4^5 is addressed with 20
    scores.  The oracle reads exactly U*d_p = 20 logits, evaluates 20
    exponentials, and each of the 20 logits matters."""
    g = golden("product_softmax_counts.json")
    d_p, U, M, n = g["d_p"], g["U"], g["M"], g["scores"]
    assert d_p ** U == M and U * d_p == n
    lg = rng(3).standard_normal(n).astype(np.float32)
    _, _, _, n_exp, _ = orc.decode_one(lg, U, d_p, 8)
    assert n_exp == n
    W0 = orc.slot_weights(lg, U, d_p)
    assert W0.size == M
    for j in range(n):
        lg2 = lg.copy()
        lg2[j] += 1.0
        assert not np.array_equal(orc.slot_weights(lg2, U, d_p), W0)


def test_place_value_one_hot_digits(orc):
    """Project page, 'Soft Radix Address' / 'Waveform Modulation': block u is
    digit u, the most significant first.  Near one-hot digit distributions
    select slot sum_u a_u * d_p^(U-1-u) with weight ~1."""
    r = rng(4)
    for d_p, U in [(4, 5), (3, 4), (2, 7), (5, 3)]:
        for _ in range(10):
            digits = r.integers(0, d_p, size=U)
            lg = np.zeros(U * d_p, np.float32)
            for u, a in enumerate(digits):
                lg[u * d_p + a] = 40.0
            expect = 0
            for a in digits:
                expect = expect * d_p + int(a)
            idx, wt, _, _, _ = orc.decode_one(lg, U, d_p, 1)
            assert idx[0] == expect
            assert abs(wt[0] - 1.0) < 1e-12


def test_waveform_periods(orc):
    """Project page, 'Waveform Modulation': read along the slot index, the
    lowest digit's distribution repeats with period d_p, the highest digit
    holds each value over runs of d_p^(U-1) slots."""
    d_p, U = 4, 4
    r = rng(5)
    lg = np.zeros(U * d_p, np.float32)
    lg[(U - 1) * d_p:] = r.standard_normal(d_p)
    W = orc.slot_weights(lg, U, d_p)
    assert np.allclose(W, np.tile(W[:d_p], d_p ** (U - 1)), rtol=0, atol=1e-15)
    assert len(set(np.round(W[:d_p], 12))) == d_p
    lg = np.zeros(U * d_p, np.float32)
    lg[:d_p] = r.standard_normal(d_p)
    W = orc.slot_weights(lg, U, d_p)
    runs = W.reshape(d_p, -1)
    assert np.allclose(runs, runs[:, :1], rtol=0, atol=1e-15)


def test_regroupings_are_rank_one(orc):
    """Project page, 'Regroupable Address': splitting the digits into two
    groups arranges the weights as an outer product, e.g. 64 x 4 and 4 x 64
    at U = d_p = 4 (golden), and likewise at every split point."""
    g = golden("regroupings.json")
    d_p, U = g["d_p"], g["U"]
    r = rng(6)
    for _ in range(5):
        lg = (r.standard_normal(U * d_p) * 2).astype(np.float32)
        W = orc.slot_weights(lg, U, d_p)
        shapes = [tuple(s) for s in g["groupings"]]
        shapes += [(d_p ** a, d_p ** (U - a)) for a in range(1, U)]
        for rows, cols in shapes:
            s = np.linalg.svd(W.reshape(rows, cols), compute_uv=False)
            assert s[1] / s[0] < 1e-12
    # The figure's 64 x 4 and 4 x 64 views are different arrangements of
    # the same weights.
    assert W.reshape(64, 4).T.shape == (4, 64)


def test_u1_is_softmax_and_sort(orc):
    """U = 1 reduces Product Softmax to one softmax and Top-K to a sort of
    the logits (library routines)."""
    r = rng(7)
    for d_p in (2, 5, 16, 64):
        lg = r.standard_normal(d_p).astype(np.float32)
        e = np.exp(lg.astype(np.float64) - lg.max())
        p = e / e.sum()
        W = orc.slot_weights(lg, 1, d_p)
        assert np.allclose(W, p, rtol=1e-14, atol=0)
        for K in (1, d_p // 2, d_p):
            idx, wt, _, _, _ = orc.decode_one(lg, 1, d_p, max(K, 1))
            order = np.argsort(-p, kind="stable")[:max(K, 1)]
            assert np.array_equal(idx, order)


# ---------------------------------------------------------------- Top-K

def _lexsort_topk(W, K):
    order = np.lexsort((np.arange(W.size), -W))  # weight desc, index asc
    return order[:K]


@pytest.mark.parametrize("d_p,U", [(2, 1), (2, 3), (2, 6), (3, 2), (3, 4),
                                   (4, 2), (4, 3), (4, 5), (5, 3)])
def test_brute_topk_matches_sort(orc, d_p, U):
    """The plain Top-K is the first K slots of a full sort by (weight desc,
    index asc) of the oracle's slot weights (numpy lexsort)."""
    M = d_p ** U
    r = rng(8)
    for trial in range(3):
        lg = (r.standard_normal(U * d_p) * 2).astype(np.float32)
        W = orc.slot_weights(lg, U, d_p)
        for K in sorted({1, 2, min(8, M), M // 2 or 1, M}):
            idx, wt, gap, _, _ = orc.decode_one(lg, U, d_p, K)
            ref = _lexsort_topk(W, K)
            assert np.array_equal(idx, ref)
            assert np.array_equal(wt, W[ref])
            if K < M:
                Ws = W[_lexsort_topk(W, K + 1)]
                assert gap == pytest.approx((Ws[K - 1] - Ws[K]) / Ws[K - 1],
                                            rel=0, abs=1e-15)
            else:
                assert gap == math.inf


def _tie_logits(r, U, d_p, kind):
    if kind == "zeros":
        return np.zeros(U * d_p, np.float32)
    if kind == "repeat":
        base = r.standard_normal(d_p).astype(np.float32)
        return np.tile(base, U)
    if kind == "pairs":
        lg = r.standard_normal(U * d_p).astype(np.float32)
        lg[1::2] = lg[0::2][: lg[1::2].size]
        return lg
    if kind == "extreme":
        return (r.choice([-30.0, 0.0, 30.0], size=U * d_p)).astype(np.float32)
    return (r.standard_normal(U * d_p) * 2).astype(np.float32)


def _assert_valid_topk(W, idx, wt, K, rel=1e-12):
    """Where mathematically equal weights round differently (repeated digit
    distributions), any of the near-equal slots at the K-th place is a
    correct answer: the set must hold every slot clearly above the K-th
    weight and only slots within `rel` of it or above."""
    WK = np.sort(W)[::-1][K - 1]
    assert len(set(idx.tolist())) == K
    assert np.array_equal(wt, W[idx])
    must = np.nonzero(W > WK * (1 + rel))[0]
    assert set(must.tolist()) <= set(idx.tolist())
    assert (W[idx] >= WK * (1 - rel)).all()


@pytest.mark.parametrize("d_p,U", [(2, 1), (2, 4), (2, 8), (3, 3), (3, 5),
                                   (4, 2), (4, 3), (4, 4), (4, 5), (5, 2),
                                   (5, 3), (5, 4)])
def test_tree_equals_brute_exhaustive(orc, d_p, U):
    """Project page, exact Top-K paragraph: keeping the K best partial
    addresses per level returns exactly the Top-K of all M slots.  Checked
    for every K and for random and tied logits."""
    M = d_p ** U
    r = rng(9 + d_p * 10 + U)
    Ks = range(1, M + 1) if M <= 64 else sorted(
        {1, 2, 3, 4, 7, 8, 16, 31, 32, 33, 64, M // 2, M - 1, M})
    for kind in ("random", "zeros", "repeat", "pairs", "extreme"):
        lg = _tie_logits(r, U, d_p, kind)
        for K in Ks:
            bi, bw, gap, _, _ = orc.decode_one(lg, U, d_p, K, mode=orc.TOPK_BRUTE)
            ti, tw, _, _, cand = orc.decode_one(lg, U, d_p, K, mode=orc.TOPK_TREE)
            if kind in ("random", "zeros") or gap > 1e-12:
                assert np.array_equal(bi, ti), (kind, K)
                assert np.array_equal(bw, tw), (kind, K)
            else:
                _assert_valid_topk(orc.slot_weights(lg, U, d_p), ti, tw, K)


def test_all_ties_pick_lowest_indices(orc):
    """Equal weights rank by slot index: uniform digits select slots 0..K-1."""
    for d_p, U, K in [(4, 5, 8), (4, 5, 32), (2, 6, 5), (3, 3, 27)]:
        lg = np.zeros(U * d_p, np.float32)
        for mode in (orc.TOPK_BRUTE, orc.TOPK_TREE):
            idx, wt, gap, _, _ = orc.decode_one(lg, U, d_p, K, mode=mode)
            assert np.array_equal(idx, np.arange(K))
            assert np.allclose(wt, float(d_p) ** -U, rtol=1e-15)
            if mode == orc.TOPK_BRUTE and K < d_p ** U:
                assert gap == 0.0


@pytest.mark.parametrize("d_p,U,K", [(4, 5, 8), (4, 5, 16), (4, 5, 32),
                                     (4, 8, 32), (3, 6, 10), (2, 10, 64)])
def test_candidates_per_level(orc, d_p, U, K):
    """Project page, exact Top-K paragraph: the search scores at most K*d_p
    candidates per level instead of all M slots."""
    lg = rng(10).standard_normal(U * d_p).astype(np.float32)
    _, _, _, _, cand = orc.decode_one(lg, U, d_p, K, mode=orc.TOPK_TREE)
    for u in range(U):
        assert cand[u] == min(K, d_p ** u) * d_p
        assert cand[u] <= K * d_p
    assert cand.sum() < d_p ** U or d_p ** U <= K * d_p * U


def test_tree_equals_brute_large_random(orc):
    """Tree = brute force at the large-state shape (M = 4^8, K = 32)."""
    r = rng(11)
    for _ in range(20):
        lg = (r.standard_normal(32) * 2).astype(np.float32)
        bi, bw, _, _, _ = orc.decode_one(lg, 8, 4, 32, mode=orc.TOPK_BRUTE)
        ti, tw, _, _, _ = orc.decode_one(lg, 8, 4, 32, mode=orc.TOPK_TREE)
        assert np.array_equal(bi, ti) and np.array_equal(bw, tw)


# ---------------------------------------------------------------- CAPE

def test_cape_hand_worked_cases(orc):
    g = golden("cape_small.json")
    for c in g["cases"]:
        a0, a1 = c["digits"]
        assert c["slot"] == a0 * g["d_p"] + a1
        out = orc.cape(np.array([c["slot"]], np.int32), c["P"], g["U"], g["d_p"])
        assert out[0] == c["moved"], c


def test_cape_shift_zero_is_identity(orc):
    """No shift at positions that are multiples of d_p."""
    idx = np.arange(1024, dtype=np.int32)
    for P in (0, 4, 8, 4096):
        assert np.array_equal(orc.cape(idx, P, 5, 4), idx)


def test_cape_is_a_permutation(orc):
    """Project page, CAPE: the shift only permutes slot indices."""
    for d_p, U in [(4, 5), (3, 4), (5, 2), (4, 8)]:
        M = d_p ** U
        idx = np.arange(M, dtype=np.int32)
        for P in range(2 * d_p + 1):
            out = orc.cape(idx, P, U, d_p)
            assert np.array_equal(np.sort(out), idx)
            # composition: moving by P then by Q equals moving by P + Q
            out2 = orc.cape(out, 3, U, d_p)
            assert np.array_equal(out2, orc.cape(idx, P + 3, U, d_p))


def test_cape_keeps_weights_and_distinctness(orc):
    r = rng(12)
    for P in range(8):
        lg = (r.standard_normal(20) * 1.5).astype(np.float32)
        i0, w0, _, _, _ = orc.decode_one(lg, 5, 4, 16, cape=0)
        i1, w1, _, _, _ = orc.decode_one(lg, 5, 4, 16, cape=1, pos=P)
        assert np.array_equal(w0, w1)
        assert len(set(i1.tolist())) == 16
        assert np.array_equal(i1, orc.cape(i0, P, 5, 4))


# CAPE readings B (digit-wise shift by the position's own digits, no carry)
# and C (rotation of the whole slot array by the position): project page,
# CAPE, where the exact shift is left open.

def test_cape_forms_b_c_are_permutations(orc):
    for d_p, U in [(4, 5), (3, 4), (5, 2), (2, 7)]:
        M = d_p ** U
        idx = np.arange(M, dtype=np.int32)
        for form in (2, 3):
            for P in (1, 2, d_p, d_p + 1, M - 1, M + 3, 12345):
                out = orc.cape(idx, P, U, d_p, form)
                assert np.array_equal(np.sort(out), idx), (form, P)


def test_cape_form_c_rotates_the_slot_array(orc):
    for d_p, U in [(4, 5), (3, 3)]:
        M = d_p ** U
        idx = np.arange(M, dtype=np.int32)
        one = orc.cape(idx, 1, U, d_p, 3)
        assert one[M - 1] == 0 and np.array_equal(one[:-1], idx[1:])  # wraps once
        assert np.array_equal(orc.cape(idx, M, U, d_p, 3), idx)       # full turn
        assert np.array_equal(orc.cape(idx, 2 * M + 5, U, d_p, 3), orc.cape(idx, 5, U, d_p, 3))
        for P, Q in [(1, 1), (7, M - 3), (M - 1, M - 1)]:
            assert np.array_equal(orc.cape(orc.cape(idx, P, U, d_p, 3), Q, U, d_p, 3),
                                  orc.cape(idx, P + Q, U, d_p, 3))


def test_cape_form_b_moves_each_digit_by_its_own_position_digit(orc):
    d_p, U = 4, 5
    M = d_p ** U
    idx = np.arange(M, dtype=np.int32)
    # a position below d_p moves only the last (least significant) digit
    for P in range(1, d_p):
        out = orc.cape(idx, P, U, d_p, 2)
        assert np.array_equal(out // d_p, idx // d_p)
        assert np.array_equal(out % d_p, (idx % d_p + P) % d_p)
    # a position a * d_p^(U-1) moves only the first digit, and such moves add
    top = d_p ** (U - 1)
    for a in range(1, d_p):
        out = orc.cape(idx, a * top, U, d_p, 2)
        assert np.array_equal(out % top, idx % top)
        assert np.array_equal(out // top, (idx // top + a) % d_p)
        for b in range(d_p):
            assert np.array_equal(orc.cape(out, b * top, U, d_p, 2),
                                  orc.cape(idx, ((a + b) % d_p) * top, U, d_p, 2))
    # all position digits equal to s: every digit moves by s, which is form A
    # at a position congruent to s
    rep1 = sum(d_p ** u for u in range(U))
    for s_ in range(d_p):
        assert np.array_equal(orc.cape(idx, s_ * rep1, U, d_p, 2), orc.cape(idx, s_, U, d_p, 1))


def test_cape_forms_agree_with_one_digit(orc):
    """U = 1: every reading is the same cyclic shift of d_p slots."""
    for d_p in (2, 5, 8):
        idx = np.arange(d_p, dtype=np.int32)
        for P in range(3 * d_p):
            a = orc.cape(idx, P, 1, d_p, 1)
            assert np.array_equal(a, (idx + P) % d_p)
            assert np.array_equal(orc.cape(idx, P, 1, d_p, 2), a)
            assert np.array_equal(orc.cape(idx, P, 1, d_p, 3), a)


# ---------------------------------------------------------------- layer helpers

def _small_inputs(seed, B, T, H, U, d_p, d_v, sigma=1.5, bf16=False):
    r = rng(seed)
    L = U * d_p
    f = lambda *s: r.standard_normal(s).astype(np.float32)
    x = dict(q=f(B, T, H, L) * sigma, k=f(B, T, H, L) * sigma, v=f(B, T, H, d_v),
             gamma=f(B, T, H), g=f(B, T, H, d_v))
    if bf16:
        import oracle as o
        for n in x:
            x[n] = np.vectorize(o.round_bf16)(x[n]).astype(np.float32)
    return x


def _run(orc, x, S, m, **kw):
    return orc.layer(x["q"], x["k"], x["v"], x["gamma"], x["g"], S, m, **kw)


# ---------------------------------------------------------------- GSU

def _given(B, T, H, K, idx_w, wt_w, idx_r, wt_r):
    shp = (B, T, H, K)
    return (np.broadcast_to(np.asarray(idx_w, np.int32), shp).copy(),
            np.broadcast_to(np.asarray(wt_w, np.float64), shp).copy(),
            np.broadcast_to(np.asarray(idx_r, np.int32), shp).copy(),
            np.broadcast_to(np.asarray(wt_r, np.float64), shp).copy())


def test_untouched_rows_bit_unchanged(orc):
    """Project page, GSU: slots outside the write addresses keep their
    content and mass exactly (w = 0 gives alpha = 1, lambda = 0)."""
    B, T, H, U, d_p, K, d_v = 2, 40, 2, 5, 4, 8, 32
    M = d_p ** U
    x = _small_inputs(13, B, T, H, U, d_p, d_v)
    r = rng(14)
    for bf16 in (False, True):
        S0 = r.standard_normal((B, H, M, d_v)).astype(np.float32)
        if bf16:
            S0 = np.vectorize(orc.round_bf16)(S0).astype(np.float32)
        m0 = r.random((B, H, M)).astype(np.float32)
        S, m = S0.copy(), m0.copy()
        res = _run(orc, x, S, m, d_p=d_p, U=U, K=K, state_bf16=bf16)
        for b in range(B):
            for h in range(H):
                written = set(res["w_idx"][b, :, h].ravel().tolist())
                untouched = np.array(sorted(set(range(M)) - written))
                assert untouched.size > 0
                assert np.array_equal(S[b, h, untouched].view(np.uint32),
                                      S0[b, h, untouched].view(np.uint32))
                assert np.array_equal(m[b, h, untouched].view(np.uint32),
                                      m0[b, h, untouched].view(np.uint32))
                wl = np.array(sorted(written))
                assert not np.array_equal(S[b, h, wl], S0[b, h, wl])


def test_zero_weight_write_changes_nothing(orc):
    """Project page, GSU: w = 0 gives alpha = 1 and lambda = 0, also at the
    extreme gates (no inf * 0)."""
    B, T, H, K, d_v = 1, 5, 1, 2, 16
    r = rng(15)
    S0 = r.standard_normal((1, 1, 16, d_v)).astype(np.float32)
    m0 = r.random((1, 1, 16)).astype(np.float32)
    gi = _given(B, T, H, K, [3, 7], [0.0, 0.0], [3, 7], [0.6, 0.4])
    for gm in (-1000.0, 0.0, 1000.0):
        S, m = S0.copy(), m0.copy()
        v = r.standard_normal((B, T, H, d_v)).astype(np.float32)
        out = orc.scan_given(*gi, v, np.full((B, T, H), gm, np.float32),
                             np.zeros((B, T, H, d_v), np.float32), S, m,
                             d_p=4, U=2, state_bf16=False)
        assert np.array_equal(S, S0) and np.array_equal(m, m0)
        assert np.isfinite(out).all()


def test_first_write_from_empty_slot(orc):
    """From mass 0 the retained mass is 0, so m = w and lambda = w/(w+eps):
    the slot becomes lambda * v (closed form of GSU steps 2-4)."""
    d_v, eps = 8, 1e-3
    r = rng(16)
    v = r.standard_normal((1, 1, 1, d_v)).astype(np.float32)
    for w in (0.05, 0.5, 0.999):
        S = np.zeros((1, 1, 16, d_v), np.float32)
        m = np.zeros((1, 1, 16), np.float32)
        gi = _given(1, 1, 1, 1, [6], [w], [6], [1.0])
        orc.scan_given(*gi, v, np.zeros((1, 1, 1), np.float32),
                       np.zeros((1, 1, 1, d_v), np.float32), S, m, d_p=4, U=2,
                       state_bf16=False, eps_gsu=eps)
        assert m[0, 0, 6] == np.float32(w)
        lam = float(np.float32(w)) / (float(np.float32(w)) + eps)
        assert np.allclose(S[0, 0, 6], lam * v[0, 0, 0].astype(np.float64),
                           rtol=1e-7, atol=0)


def test_gamma_to_minus_inf_averages_all_writes(orc):
    """Project page, GSU: as gamma -> -inf the slot averages all past writes;
    with eps = 0 it is the write-weighted mean sum w_s v_s / sum w_s."""
    T, d_v = 50, 16
    r = rng(17)
    w = r.uniform(0.05, 0.9, size=T)
    v = r.standard_normal((1, T, 1, d_v)).astype(np.float32)
    S = np.zeros((1, 1, 16, d_v), np.float32)
    m = np.zeros((1, 1, 16), np.float32)
    wi = np.full((1, T, 1, 1), 9, np.int32)
    ww = w.reshape(1, T, 1, 1)
    orc.scan_given(wi, ww, wi.copy(), np.ones_like(ww), v,
                   np.full((1, T, 1), -1000.0, np.float32),
                   np.zeros((1, T, 1, d_v), np.float32), S, m, d_p=4, U=2,
                   state_bf16=False, eps_gsu=0.0)
    ref = (w[:, None] * v[0, :, 0].astype(np.float64)).sum(0) / w.sum()
    assert np.allclose(S[0, 0, 9], ref, rtol=2e-5, atol=2e-6)
    assert m[0, 0, 9] == pytest.approx(w.sum(), rel=1e-6)


def test_gamma_to_plus_inf_overwrites(orc):
    """Project page, GSU: as gamma -> +inf the newest value overwrites the
    slot (lambda = 1 with eps = 0)."""
    T, d_v = 20, 16
    r = rng(18)
    # fp32-representable weights: the stored mass then equals w exactly
    w = r.uniform(0.05, 0.9, size=T).astype(np.float32).astype(np.float64)
    v = r.standard_normal((1, T, 1, d_v)).astype(np.float32)
    S = r.standard_normal((1, 1, 16, d_v)).astype(np.float32)
    m = np.ones((1, 1, 16), np.float32)
    wi = np.full((1, T, 1, 1), 2, np.int32)
    ww = w.reshape(1, T, 1, 1)
    orc.scan_given(wi, ww, wi.copy(), np.ones_like(ww), v,
                   np.full((1, T, 1), 1000.0, np.float32),
                   np.zeros((1, T, 1, d_v), np.float32), S, m, d_p=4, U=2,
                   state_bf16=False, eps_gsu=0.0)
    assert np.array_equal(S[0, 0, 2], v[0, -1, 0])
    assert m[0, 0, 2] == np.float32(w[-1])


def test_retention_direction(orc):
    """Project page, GSU step 1: a stronger write or a larger gamma keeps less
    of the previous mass.  Measured as the retained part m2 - w2 after a
    second write onto a slot of mass m1."""
    def retained(w2, gm):
        S = np.zeros((1, 1, 16, 4), np.float32)
        m = np.full((1, 1, 16), 2.0, np.float32)
        gi = _given(1, 1, 1, 1, [1], [w2], [1], [1.0])
        orc.scan_given(*gi, np.ones((1, 1, 1, 4), np.float32),
                       np.full((1, 1, 1), gm, np.float32),
                       np.zeros((1, 1, 1, 4), np.float32), S, m, d_p=4, U=2,
                       state_bf16=False)
        return float(m[0, 0, 1]) - float(np.float32(w2))
    gms = [-3.0, -1.0, 0.0, 1.0, 2.0]
    ws = [0.01, 0.1, 0.3, 0.6, 0.9]
    for w2 in ws:
        vals = [retained(w2, g) for g in gms]
        assert all(a > b for a, b in zip(vals, vals[1:])), (w2, vals)
    for gm in gms:
        vals = [retained(w2, gm) for w2 in ws]
        assert all(a > b for a, b in zip(vals, vals[1:])), (gm, vals)
    assert 0.0 < retained(0.3, 0.0) < 2.0
    assert retained(1.0, 0.0) == 0.0


def test_bounded_averages_and_nonnegative_mass(orc):
    """Project page, GSU step 4 and the summary's 'bounded averages': each
    content update is a convex step toward v, so every stored element stays
    within the range of its initial value and the values written to it."""
    B, T, H, U, d_p, K, d_v = 1, 200, 2, 3, 4, 8, 16
    M = d_p ** U
    x = _small_inputs(19, B, T, H, U, d_p, d_v, sigma=1.0)
    S0 = rng(20).standard_normal((B, H, M, d_v)).astype(np.float32)
    S, m = S0.copy(), np.zeros((B, H, M), np.float32)
    res = _run(orc, x, S, m, d_p=d_p, U=U, K=K, state_bf16=False)
    for h in range(H):
        lo, hi = S0[0, h].copy(), S0[0, h].copy()
        for t in range(T):
            for i in res["w_idx"][0, t, h]:
                lo[i] = np.minimum(lo[i], x["v"][0, t, h])
                hi[i] = np.maximum(hi[i], x["v"][0, t, h])
        assert (S[0, h] >= lo).all() and (S[0, h] <= hi).all()
    assert (m >= 0).all()


# ---------------------------------------------------------------- read, norm, gate

def test_read_sees_this_tokens_write_and_hash_table_limit(orc):
    """Project page, three stages: the value is written, then the read slots
    are combined, normalized and gated.  K = 1 and gamma -> +inf make the
    layer a hash table: a query addressing the slot a key wrote returns that
    value, RMS-normalized and gated by sigmoid(g)."""
    d_p, U, d_v = 4, 3, 16
    L = U * d_p
    r = rng(21)
    slot_digits = [2, 0, 3]
    lg = np.full(L, -20.0, np.float32)
    for u, a in enumerate(slot_digits):
        lg[u * d_p + a] = 20.0
    v = r.standard_normal((1, 1, 1, d_v)).astype(np.float32)
    g = r.standard_normal((1, 1, 1, d_v)).astype(np.float32)
    x = dict(q=lg.reshape(1, 1, 1, L), k=lg.reshape(1, 1, 1, L), v=v,
             gamma=np.full((1, 1, 1), 1000.0, np.float32), g=g)
    S = np.zeros((1, 1, d_p ** U, d_v), np.float32)
    m = np.zeros((1, 1, d_p ** U), np.float32)
    res = _run(orc, x, S, m, d_p=d_p, U=U, K=1, state_bf16=False, cape=0,
               eps_gsu=0.0, eps_norm=0.0)
    slot = 2 * 16 + 0 * 4 + 3
    assert res["w_idx"][0, 0, 0, 0] == slot == res["r_idx"][0, 0, 0, 0]
    assert np.array_equal(S[0, 0, slot], v[0, 0, 0])
    vv = v[0, 0, 0].astype(np.float64)
    sig = 1 / (1 + np.exp(-g[0, 0, 0].astype(np.float64)))
    expect = vv / np.sqrt(np.mean(vv ** 2)) * sig
    assert np.allclose(res["out"][0, 0, 0], expect, rtol=1e-6, atol=1e-7)


def test_output_rms_is_one_before_gate(orc):
    """RMSNorm: dividing the output by omega * sigmoid(g) leaves a vector of
    unit RMS (eps_norm = 0 here; the read weights are products of digit
    probabilities, so mean(r^2) is small and eps_norm would show)."""
    B, T, H, U, d_p, K, d_v = 1, 64, 2, 5, 4, 8, 64
    M = d_p ** U
    x = _small_inputs(22, B, T, H, U, d_p, d_v)
    S = rng(23).standard_normal((B, H, M, d_v)).astype(np.float32)
    m = np.ones((B, H, M), np.float32)
    omega = rng(24).uniform(0.5, 2.0, size=d_v).astype(np.float32)
    res = _run(orc, x, S, m, d_p=d_p, U=U, K=K, state_bf16=False, norm_w=omega,
               eps_norm=0.0)
    sig = 1 / (1 + np.exp(-x["g"].astype(np.float64)))
    z = res["out"] / (omega.astype(np.float64) * sig)
    rms = np.sqrt((z ** 2).mean(-1))
    assert np.allclose(rms, 1.0, rtol=1e-5)


# ---------------------------------------------------------------- CAPE in the layer

def test_cape_relative_positions_only(orc):
    """Project page, CAPE: overlap depends on content and the distance t - s,
    not on absolute position.  From an empty state, shifting every position
    by c leaves all outputs bit-identical and permutes the final state by the
    constant digit shift."""
    B, T, H, U, d_p, K, d_v = 2, 60, 2, 5, 4, 8, 32
    M = d_p ** U
    x = _small_inputs(25, B, T, H, U, d_p, d_v)
    S_a = np.zeros((B, H, M, d_v), np.float32)
    m_a = np.zeros((B, H, M), np.float32)
    ra = _run(orc, x, S_a, m_a, d_p=d_p, U=U, K=K, state_bf16=False,
              pos0=np.zeros(B, np.int32))
    for c in (1, 2, 3, 5):
        S_b = np.zeros_like(S_a)
        m_b = np.zeros_like(m_a)
        rb = _run(orc, x, S_b, m_b, d_p=d_p, U=U, K=K, state_bf16=False,
                  pos0=np.full(B, c, np.int32))
        assert np.array_equal(ra["out"], rb["out"])
        perm = orc.cape(np.arange(M, dtype=np.int32), c, U, d_p)
        assert np.array_equal(S_b[:, :, perm], S_a)
        assert np.array_equal(m_b[:, :, perm], m_a)
    # CAPE does change which slots see which writes in general.
    S_c = np.zeros_like(S_a)
    m_c = np.zeros_like(m_a)
    rc = _run(orc, x, S_c, m_c, d_p=d_p, U=U, K=K, state_bf16=False, cape=0)
    assert not np.array_equal(rc["out"], ra["out"])


def test_cape_off_equals_positions_multiple_of_dp(orc):
    """Shift 0 everywhere: with cape on and only one token per sequence at
    position 0 mod d_p, the result equals content-only addressing."""
    B, T, H, U, d_p, K, d_v = 3, 1, 2, 5, 4, 8, 16
    M = d_p ** U
    x = _small_inputs(26, B, T, H, U, d_p, d_v)
    S1 = rng(27).standard_normal((B, H, M, d_v)).astype(np.float32)
    m1 = np.ones((B, H, M), np.float32)
    S2, m2 = S1.copy(), m1.copy()
    r1 = _run(orc, x, S1, m1, d_p=d_p, U=U, K=K, state_bf16=False, cape=0)
    r2 = _run(orc, x, S2, m2, d_p=d_p, U=U, K=K, state_bf16=False, cape=1,
              pos0=np.array([0, 4, 400], np.int32))
    assert np.array_equal(r1["out"], r2["out"]) and np.array_equal(S1, S2)


def test_cape_form_c_relative_positions_only(orc):
    """Form C is a rotation by the position, so as for form A, shifting every
    position by c leaves the outputs bit-identical and rotates the final
    state by c."""
    B, T, H, U, d_p, K, d_v = 1, 40, 2, 4, 3, 5, 16
    M = d_p ** U
    x = _small_inputs(31, B, T, H, U, d_p, d_v)
    S_a = np.zeros((B, H, M, d_v), np.float32)
    m_a = np.zeros((B, H, M), np.float32)
    ra = _run(orc, x, S_a, m_a, d_p=d_p, U=U, K=K, state_bf16=False, cape=3,
              pos0=np.zeros(B, np.int32))
    for c in (1, 7, M + 2):
        S_b, m_b = np.zeros_like(S_a), np.zeros_like(m_a)
        rb = _run(orc, x, S_b, m_b, d_p=d_p, U=U, K=K, state_bf16=False, cape=3,
                  pos0=np.full(B, c, np.int32))
        assert np.array_equal(ra["out"], rb["out"])
        perm = orc.cape(np.arange(M, dtype=np.int32), c, U, d_p, 3)
        assert np.array_equal(S_b[:, :, perm], S_a)


def test_content_heads_mask_selects_per_head(orc):
    """Project page, CAPE: some heads use CAPE, others content-only
    addresses.  A head whose bit is set behaves exactly as with CAPE off; the
    others exactly as with CAPE on (heads are independent units)."""
    B, T, H, U, d_p, K, d_v = 2, 24, 3, 5, 4, 8, 16
    M = d_p ** U
    x = _small_inputs(32, B, T, H, U, d_p, d_v)
    pos0 = np.array([5, 2], np.int32)
    runs = {}
    for name, cape, mask in [("off", 0, 0), ("on", 2, 0), ("mixed", 2, 0b101)]:
        S = np.zeros((B, H, M, d_v), np.float32)
        m = np.zeros((B, H, M), np.float32)
        runs[name] = (_run(orc, x, S, m, d_p=d_p, U=U, K=K, state_bf16=False,
                           cape=cape, content_heads=mask, pos0=pos0), S)
    for h in range(H):
        ref = "off" if (0b101 >> h) & 1 else "on"
        assert np.array_equal(runs["mixed"][0]["out"][:, :, h], runs[ref][0]["out"][:, :, h])
        assert np.array_equal(runs["mixed"][0]["w_idx"][:, :, h], runs[ref][0]["w_idx"][:, :, h])
        assert np.array_equal(runs["mixed"][1][:, h], runs[ref][1][:, h])
    assert not np.array_equal(runs["off"][0]["out"], runs["on"][0]["out"])
    # the decoder alone follows the same mask
    idx, _, _ = orc.decode_all(x["k"], U, d_p, K, cape=2, pos0=pos0, content_heads=0b101)
    assert np.array_equal(idx, runs["mixed"][0]["w_idx"])


# ---------------------------------------------------------------- resume

@pytest.mark.parametrize("bf16", [False, True])
def test_resume_split_equals_whole(orc, bf16):
    """The state (S, m) is the whole carry of the recurrence: a prefill split
    at T1 and resumed at position pos0 + T1 is bit-identical to the whole
    prefill, and T one-token calls equal one T-token call."""
    B, T, H, U, d_p, K, d_v = 2, 48, 2, 5, 4, 8, 32
    M = d_p ** U
    x = _small_inputs(28, B, T, H, U, d_p, d_v, bf16=bf16)
    pos0 = np.array([3, 10], np.int32)
    S_w = np.zeros((B, H, M, d_v), np.float32)
    m_w = np.zeros((B, H, M), np.float32)
    rw = _run(orc, x, S_w, m_w, d_p=d_p, U=U, K=K, state_bf16=bf16, pos0=pos0)
    S_s = np.zeros_like(S_w)
    m_s = np.zeros_like(m_w)
    T1 = 17
    sl = lambda a, s: np.ascontiguousarray(a[:, s])
    ra = _run(orc, {n: sl(a, slice(0, T1)) for n, a in x.items()}, S_s, m_s,
              d_p=d_p, U=U, K=K, state_bf16=bf16, pos0=pos0)
    rb = _run(orc, {n: sl(a, slice(T1, T)) for n, a in x.items()}, S_s, m_s,
              d_p=d_p, U=U, K=K, state_bf16=bf16, pos0=pos0 + T1)
    assert np.array_equal(np.concatenate([ra["out"], rb["out"]], 1), rw["out"])
    assert np.array_equal(S_s, S_w) and np.array_equal(m_s, m_w)
    S_d = np.zeros_like(S_w)
    m_d = np.zeros_like(m_w)
    outs = []
    for t in range(T):
        rd = _run(orc, {n: sl(a, slice(t, t + 1)) for n, a in x.items()}, S_d,
                  m_d, d_p=d_p, U=U, K=K, state_bf16=bf16, pos0=pos0 + t)
        outs.append(rd["out"])
    assert np.array_equal(np.concatenate(outs, 1), rw["out"])
    assert np.array_equal(S_d, S_w)


def test_tree_mode_layer_equals_brute_mode(orc):
    B, T, H, U, d_p, K, d_v = 1, 64, 2, 5, 4, 16, 16
    M = d_p ** U
    x = _small_inputs(29, B, T, H, U, d_p, d_v)
    outs = []
    for mode in (orc.TOPK_BRUTE, orc.TOPK_TREE):
        S = np.zeros((B, H, M, d_v), np.float32)
        m = np.zeros((B, H, M), np.float32)
        outs.append((_run(orc, x, S, m, d_p=d_p, U=U, K=K, state_bf16=False,
                          mode=mode)["out"], S))
    assert np.array_equal(outs[0][0], outs[1][0])
    assert np.array_equal(outs[0][1], outs[1][1])


# ---------------------------------------------------------------- storage

def test_bf16_rounding_cases(orc):
    """Nearest-even rounding to bf16 (8 significant bits), worked by hand,
    plus agreement with torch's float32 -> bfloat16 conversion."""
    cases = [
        (1.0, 1.0),
        (1.0 + 2 ** -8, 1.0),                    # tie, even is 1.0
        (1.0 + 3 * 2 ** -8, 1.0 + 2 ** -6),      # tie, even is 1 + 2^-6
        (1.0 + 2 ** -8 + 2 ** -20, 1.0 + 2 ** -7),
        (-2.5 - 2 ** -7, -2.5),                  # below half spacing
        (3.0e38, 226 * 2.0 ** 120),              # spacing 2^120 near 2^127
        (3.5e38, math.inf),
        (2 ** -133, 2 ** -133),                  # smallest subnormal
        (2 ** -134, 0.0),                        # tie to even (zero)
        (1.5 * 2 ** -133, 2 ** -132),            # tie, even is 2 * 2^-133
    ]
    for x, y in cases:
        got = orc.round_bf16(x)
        if math.isinf(y):
            assert math.isinf(got)
        else:
            assert got == y, (x, got, y)
    torch = pytest.importorskip("torch")
    xs = rng(30).standard_normal(2000).astype(np.float32) * 10
    ref = torch.from_numpy(xs).to(torch.bfloat16).to(torch.float32).numpy()
    got = np.array([orc.round_bf16(float(v)) for v in xs], np.float32)
    assert np.array_equal(ref, got)


def test_bf16_state_is_stored_rounded(orc):
    B, T, H, U, d_p, K, d_v = 1, 30, 1, 5, 4, 8, 16
    M = d_p ** U
    x = _small_inputs(31, B, T, H, U, d_p, d_v, bf16=True)
    S = np.zeros((B, H, M, d_v), np.float32)
    m = np.zeros((B, H, M), np.float32)
    res = _run(orc, x, S, m, d_p=d_p, U=U, K=K, state_bf16=True)
    for a in (S, res["out"]):
        bits = a.view(np.uint32)
        assert (bits & 0xFFFF == 0).all()


# ---------------------------------------------------------------- access accounting

def test_state_access_accounting_golden(orc):
    """Project page, state-access paragraph: a token accesses K write slots
    and K read slots of d_v elements each, 2*K/M of the state.  With M = 1024
    that fraction reproduces the printed counts."""
    g = golden("state_access.json")
    M = g["M"]
    # The oracle touches exactly K distinct rows per write and per read.
    B, T, H, U, d_p, d_v = 1, 1, 1, 5, 4, 8
    for K in (8, 16):
        x = _small_inputs(32 + K, B, T, H, U, d_p, d_v)
        S = np.zeros((B, H, M, d_v), np.float32)
        m = np.zeros((B, H, M), np.float32)
        res = _run(orc, x, S, m, d_p=d_p, U=U, K=K, state_bf16=False)
        assert len(set(res["w_idx"].ravel())) == K
        assert len(set(res["r_idx"].ravel())) == K
        assert int((m != 0).sum()) == K
    for c in g["cases"]:
        frac = 2 * c["K"] / M
        assert round(c["total_M_elems"] * frac, 1) == c["active_M_elems"]
        if "percent" in c:
            assert 100 * frac == pytest.approx(c["percent"], abs=0.1)  # "about"
    top8 = g["cases"][0]
    ratio = g["mamba2_340M_active_M_elems"] / (top8["total_M_elems"] * 16 / M)
    assert round(ratio) == g["ratio_to_mamba2_340M_top8"]


def test_zero_read_with_zero_eps_is_zero(orc):
    """A token whose read slots are all still empty reads r = 0; with
    eps_norm = 0 the RMSNorm is 0/0 and the output is taken as 0, the value
    any eps_norm > 0 gives for a zero read."""
    d_v = 8
    S = np.zeros((1, 1, 16, d_v), np.float32)
    m = np.zeros((1, 1, 16), np.float32)
    gi = _given(1, 1, 1, 1, [3], [0.5], [9], [0.7])   # read an unwritten slot
    g = rng(40).standard_normal((1, 1, 1, d_v)).astype(np.float32)
    for eps in (0.0, 1e-6):
        out = orc.scan_given(*gi, np.ones((1, 1, 1, d_v), np.float32),
                             np.zeros((1, 1, 1), np.float32), g, S.copy(),
                             m.copy(), d_p=4, U=2, state_bf16=False,
                             eps_norm=eps)
        assert np.array_equal(out, np.zeros_like(out))
