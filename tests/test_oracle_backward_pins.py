"""Pins of the backward-pass oracle (oracle/backward.py, torch fp64
autograd through the recurrence): its forward against the pinned C oracle,
its gradients against central finite differences, and the gradient of
untouched slots passing through unchanged."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import backward as BW  # noqa: E402


def rng(seed):
    return np.random.default_rng(seed)


def inputs(seed, B, T, H, U, d_p, d_v, sigma=1.5, state=True):
    r = rng(seed)
    L, M = U * d_p, d_p ** U
    f = lambda *s: r.standard_normal(s)
    x = dict(q=f(B, T, H, L) * sigma, k=f(B, T, H, L) * sigma, v=f(B, T, H, d_v),
             gamma=f(B, T, H), g=f(B, T, H, d_v))
    x["S0"] = f(B, H, M, d_v) * 0.3 if state else np.zeros((B, H, M, d_v))
    x["m0"] = r.uniform(0.2, 1.5, (B, H, M)) if state else np.zeros((B, H, M))
    x["dout"] = f(B, T, H, d_v)
    x["dS_final"] = f(B, H, M, d_v)
    x["dm_final"] = f(B, H, M)
    x["norm_w"] = 1.0 + 0.3 * f(d_v)
    x["pos0"] = r.integers(0, 50, B)
    # fp32-representable values so that the C oracle sees the same inputs
    for n in x:
        if n != "pos0":
            x[n] = np.asarray(x[n], np.float32).astype(np.float64)
    return x


def run(x, **kw):
    return BW.layer_grads(x["q"], x["k"], x["v"], x["gamma"], x["g"], x["S0"], x["m0"],
                          x["dout"], pos0=x["pos0"], norm_w=x["norm_w"],
                          dS_final=x["dS_final"], dm_final=x["dm_final"], **kw)


def test_forward_matches_c_oracle(orc):
    """The torch forward equals the pinned C oracle's layer (which stores the
    state in fp32 after every write, hence the tolerance)."""
    B, T, H, U, d_p, K, d_v = 1, 40, 2, 3, 4, 4, 8
    x = inputs(1, B, T, H, U, d_p, d_v)
    res = run(x, d_p=d_p, U=U, K=K)
    S = x["S0"].astype(np.float32).copy()
    m = x["m0"].astype(np.float32).copy()
    ref = orc.layer(x["q"], x["k"], x["v"], x["gamma"], x["g"], S, m, d_p=d_p, U=U, K=K,
                    state_bf16=False, pos0=x["pos0"].astype(np.int32),
                    norm_w=x["norm_w"].astype(np.float32))
    assert np.array_equal(res["w_idx"], ref["w_idx"]) and np.array_equal(res["r_idx"], ref["r_idx"])
    np.testing.assert_allclose(res["out"], ref["out"], rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(res["S"], S, rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(res["mass"], m, rtol=1e-5, atol=1e-6)


@pytest.mark.parametrize("bf16", [False, True])
def test_rounded_forward_equals_c_oracle_exactly(orc, bf16):
    """With the storage rounding the torch forward takes the C oracle's
    steps in the same order and precision, so the state, mass and outputs
    agree to the bit (outputs stored in the state dtype)."""
    B, T, H, U, d_p, K, d_v = 1, 30, 2, 3, 4, 4, 8
    x = inputs(4, B, T, H, U, d_p, d_v)
    if bf16:
        x["S0"] = BW._round_bf16(x["S0"])
    res = run(x, d_p=d_p, U=U, K=K, round_storage=True, state_bf16=bf16)
    S = x["S0"].astype(np.float32).copy()
    m = x["m0"].astype(np.float32).copy()
    ref = orc.layer(x["q"], x["k"], x["v"], x["gamma"], x["g"], S, m, d_p=d_p, U=U, K=K,
                    state_bf16=bf16, pos0=x["pos0"].astype(np.int32),
                    norm_w=x["norm_w"].astype(np.float32))
    assert np.array_equal(res["S"], S.astype(np.float64))
    assert np.array_equal(res["mass"], m.astype(np.float64))
    if bf16:  # rounded from fp64 values that may differ in their last bits
        np.testing.assert_allclose(BW._round_bf16(res["out"]), ref["out"], rtol=2 ** -7, atol=0)
    else:
        np.testing.assert_allclose(res["out"].astype(np.float32), ref["out"], rtol=1e-7, atol=0)


@pytest.mark.parametrize("cape,state", [(1, True), (0, False), (3, True)])
def test_gradients_match_finite_differences(cape, state):
    """Every gradient against central differences of the loss along a random
    direction (the Top-K sets do not change under the perturbation)."""
    B, T, H, U, d_p, K, d_v = 1, 6, 2, 4, 2, 3, 4
    x = inputs(2 + cape, B, T, H, U, d_p, d_v, state=state)
    base = run(x, d_p=d_p, U=U, K=K, cape=cape)
    r = rng(10 + cape)
    eps = 1e-6
    names = {"q": "dq", "k": "dk", "v": "dv", "gamma": "dgamma", "g": "dg",
             "S0": "dS0", "m0": "dm0", "norm_w": "dnorm_w"}
    for n, gname in names.items():
        d = r.standard_normal(x[n].shape)
        if n == "m0" and not state:
            d = np.abs(d)   # the mass stays >= 0
        lp, lm = dict(x), dict(x)
        lp[n] = x[n] + eps * d
        lm[n] = x[n] - eps * d
        rp = run(lp, d_p=d_p, U=U, K=K, cape=cape)
        rm = run(lm, d_p=d_p, U=U, K=K, cape=cape)
        for a in ("w_idx", "r_idx"):
            assert np.array_equal(rp[a], base[a]) and np.array_equal(rm[a], base[a]), n
        fd = (rp["loss"] - rm["loss"]) / (2 * eps)
        an = float((base[gname] * d).sum())
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (n, fd, an)


def test_untouched_slots_pass_gradient_through():
    """A slot no token writes or reads keeps dS0 = dS_final and dm0 =
    dm_final exactly; a slot only read keeps dm0 = dm_final."""
    B, T, H, U, d_p, K, d_v = 1, 5, 1, 3, 4, 2, 4
    x = inputs(7, B, T, H, U, d_p, d_v)
    res = run(x, d_p=d_p, U=U, K=K)
    written = set(res["w_idx"][0, :, 0].ravel().tolist())
    read = set(res["r_idx"][0, :, 0].ravel().tolist())
    M = d_p ** U
    untouched = [s for s in range(M) if s not in written and s not in read]
    assert untouched
    for s in untouched:
        assert np.array_equal(res["dS0"][0, 0, s], x["dS_final"][0, 0, s])
        assert res["dm0"][0, 0, s] == x["dm_final"][0, 0, s]
    for s in read - written:
        assert res["dm0"][0, 0, s] == x["dm_final"][0, 0, s]
