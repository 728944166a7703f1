"""Pins of the projection oracle (the dense steps either side of the layer)
against things other than itself: a library's bf16 conversion, exact
rational rounding, a hand-summed dot product, the closed form of a softmax
at doubled temperature, and the already pinned layer oracle reached through
selection matrices."""
import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import projections as P

torch = pytest.importorskip("torch")


def rng(seed):
    return np.random.default_rng(seed)


def bf16_exact(v: float) -> float:
    """Nearest 8-significant-bit value, ties to even, by rational arithmetic."""
    if v == 0:
        return 0.0
    f = Fraction(v)
    e = math.floor(math.log2(abs(f)))
    while abs(f) >= Fraction(2) ** (e + 1):
        e += 1
    while abs(f) < Fraction(2) ** e:
        e -= 1
    ulp = Fraction(2) ** (e - 7)
    n = f / ulp
    lo = math.floor(n)
    rem = n - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    return float(lo * ulp)


def test_bf16_rounding_matches_library_conversion():
    """fp32 inputs: identical to torch's float32 -> bfloat16 conversion."""
    x = (rng(1).standard_normal(200000) * np.exp(rng(2).uniform(-20, 20, 200000)))
    x = x.astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    assert np.array_equal(P.to_bf16(x), ref)


def test_bf16_rounding_of_wide_values_is_single_and_exact():
    """fp64 inputs with more bits than fp32 (as the exact product of a bf16
    weight and an fp32 temperature has): rounded once, ties to even."""
    r = rng(3)
    vals = list(r.standard_normal(3000) * 10)
    one = 1.0
    vals += [one + 2 ** -8, one + 3 * 2 ** -8, one + 2 ** -8 + 2 ** -40,
             -(one + 2 ** -8 - 2 ** -40), 3 * 2 ** -9 + 2 ** -35]
    got = P.to_bf16(np.array(vals))
    for v, g in zip(vals, got):
        assert float(g) == bf16_exact(v), v
    # a tie only after rounding to fp32 first: single rounding goes up
    v = one + 2 ** -8 + 2 ** -30
    assert float(P.to_bf16(v)) == one + 2 ** -7
    assert float(P.to_bf16(np.float32(v))) == one


def test_projection_equals_hand_summed_dot_products():
    """Each output is the bf16 rounding of the exact dot product (inputs on
    a dyadic grid, so the fp64 sums are exact)."""
    r = rng(4)
    x = r.integers(-8, 9, (3, 5, 48)) / 8.0
    W = r.integers(-8, 9, (48, 7)) / 64.0
    y = P.project(x, W)
    for b, t, j in np.ndindex(3, 5, 7):
        s = math.fsum(x[b, t, i] * W[i, j] for i in range(48))
        assert float(y[b, t, j]) == bf16_exact(s)


def test_temperature_of_ln2_doubles_the_address_logits(orc):
    """Paper digest, re-parameterisation W = e^alpha W': alpha = ln 2 doubles
    the weights exactly, and a digit softmax of doubled logits is p^2 / sum p^2
    (temperature one half)."""
    H, L, D = 3, 20, 16
    Wp = P.to_bf16(rng(5).standard_normal((D, H * L)))
    alpha = np.array([0.0, math.log(2), -math.log(2)], np.float32)
    t = P.temperatures(alpha, H)
    assert list(t) == [1.0, 2.0, 0.5]
    W = P.address_weights(Wp, alpha, H, L)
    assert np.array_equal(W, Wp * np.repeat(t, L)[None, :])
    lg = P.to_bf16(rng(6).standard_normal(L) * 1.5)
    p1, _ = orc.digit_probs(lg, 5, 4)
    p2, _ = orc.digit_probs(lg * 2, 5, 4)
    ref = p1 ** 2 / (p1 ** 2).sum(axis=1, keepdims=True)
    assert np.allclose(p2, ref, rtol=1e-12, atol=0)


def test_temperature_rounds_the_scaled_weight_once():
    """A general alpha: W = bf16(t * W') from the exact product, t = fp32(e^alpha)."""
    H, L, D = 2, 3, 40
    Wp = P.to_bf16(rng(7).standard_normal((D, H * L)))
    alpha = np.array([0.3, -1.7], np.float32)
    W = P.address_weights(Wp, alpha, H, L)
    for h in range(H):
        t = float(np.float32(math.exp(float(alpha[h]))))
        for i in range(D):
            for j in range(L):
                assert float(W[i, h * L + j]) == bf16_exact(float(Wp[i, h * L + j]) * t)


def _selection_setup(seed, B, T, H, U, d_p, d_v):
    """x whose columns hold bf16 q, k, v, g, gamma, and one-hot weights that
    pick them out again."""
    L = U * d_p
    r = rng(seed)
    blocks = {"q": (H * L, 1.5), "k": (H * L, 1.5), "v": (H * d_v, 1.0),
              "g": (H * d_v, 1.0), "gamma": (H, 1.0)}
    D = sum(n for n, _ in blocks.values()) + 3          # three unused columns
    x = P.to_bf16(r.standard_normal((B, T, D)))
    W, c = {}, 0
    for name, (n, sigma) in blocks.items():
        x[..., c:c + n] = P.to_bf16(r.standard_normal((B, T, n)) * sigma)
        Wn = np.zeros((D, n), np.float32)
        Wn[c + np.arange(n), np.arange(n)] = 1.0
        W[name] = Wn
        c += n
    return x, W, D


def test_selection_projections_reduce_to_the_layer(orc):
    """With one-hot weights the projections return columns of x unchanged,
    the layer forward equals the (pinned) layer oracle on them, and an
    identity-like output projection returns bf16 of the layer output."""
    B, T, H, U, d_p, K, d_v = 2, 30, 3, 5, 4, 8, 16
    M, L = d_p ** U, U * d_p
    x, W, D = _selection_setup(8, B, T, H, U, d_p, d_v)
    Wo = np.zeros((H * d_v, D), np.float32)
    Wo[np.arange(H * d_v), 5 + np.arange(H * d_v)] = 1.0
    pos0 = np.array([3, 11], np.int32)
    S1 = np.zeros((B, H, M, d_v), np.float32)
    m1 = np.zeros((B, H, M), np.float32)
    y, res = P.layer_forward(x, W["q"], W["k"], W["v"], W["g"], W["gamma"], Wo,
                             None, S1, m1, H=H, d_p=d_p, U=U, K=K,
                             state_bf16=False, pos0=pos0)
    inp = res["inputs"]
    assert np.array_equal(inp["q"].reshape(B, T, -1), x[..., :H * L])
    assert np.array_equal(inp["gamma"].reshape(B, T, -1), x[..., -H - 3:-3])
    S2, m2 = np.zeros_like(S1), np.zeros_like(m1)
    ref = orc.layer(inp["q"], inp["k"], inp["v"], inp["gamma"], inp["g"], S2, m2,
                    d_p=d_p, U=U, K=K, state_bf16=False, pos0=pos0)
    assert np.array_equal(S1, S2) and np.array_equal(m1, m2)
    out = P.to_bf16(ref["out"]).reshape(B, T, H * d_v)
    assert np.array_equal(y[..., 5:5 + H * d_v], out)
    assert not y[..., :5].any() and not y[..., 5 + H * d_v:].any()


def test_head_temperature_applies_to_its_own_columns(orc):
    """alpha of head h scales only head h's key and query logits: with one
    head at alpha = ln 2 the layer equals the layer oracle on that head's
    doubled logits."""
    B, T, H, U, d_p, K, d_v = 1, 20, 2, 5, 4, 8, 16
    M, L = d_p ** U, U * d_p
    x, W, D = _selection_setup(9, B, T, H, U, d_p, d_v)
    Wo = np.eye(H * d_v, D, dtype=np.float32)
    alpha = np.array([0.0, math.log(2)], np.float32)
    S1 = np.zeros((B, H, M, d_v), np.float32)
    m1 = np.zeros((B, H, M), np.float32)
    _, res = P.layer_forward(x, W["q"], W["k"], W["v"], W["g"], W["gamma"], Wo,
                             alpha, S1, m1, H=H, d_p=d_p, U=U, K=K,
                             state_bf16=False)
    q = x[..., :H * L].reshape(B, T, H, L).copy()
    k = x[..., H * L:2 * H * L].reshape(B, T, H, L).copy()
    q[:, :, 1] *= 2
    k[:, :, 1] *= 2
    S2, m2 = np.zeros_like(S1), np.zeros_like(m1)
    ref = orc.layer(q, k, res["inputs"]["v"], res["inputs"]["gamma"],
                    res["inputs"]["g"], S2, m2, d_p=d_p, U=U, K=K, state_bf16=False)
    assert np.array_equal(res["out"], ref["out"]) and np.array_equal(S1, S2)
    assert np.array_equal(res["w_idx"], ref["w_idx"])
