"""GPU parity of the whole layer (projections, recurrence, output projection)
through the C ABI against the projection oracle.

Grid inputs (synth.make_layer_weights, kind "grid") make every projection an
exact sum, so the projected q, k, v, g, gamma must match the oracle bit for
bit and the layer's comparisons follow the recurrence rules of parity.py.
Gaussian inputs check the fp32-accumulated products within one bf16 ulp.
"""
import os
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from sparse_slot_recurrent_amd import synth  # noqa: E402

sys.path.insert(0, os.path.dirname(__file__))
from parity import assert_close, bf16_ulp, compare_address_sets, to_np  # noqa: E402


@pytest.fixture(scope="module")
def rn():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_slot_recurrent_amd import ramnet
    ramnet.load_library()
    return ramnet


@pytest.fixture(scope="module")
def P():
    import oracle
    oracle.load()
    from oracle import projections
    return projections


def bf(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).cuda()


def gpu_weights(rn, d):
    """The library takes weights as [out, in]; the generator and the oracle
    write them as [in, out] (x W)."""
    alpha = None
    if "alpha" in d:
        alpha = torch.from_numpy(d["alpha"]).cuda()
    t = lambda a: bf(np.ascontiguousarray(np.asarray(a).T))
    return rn.LayerWeights(t(d["w_q"]), t(d["w_k"]), t(d["w_v"]), t(d["w_g"]),
                           t(d["w_gamma"]), t(d["w_o"]), alpha)


def oracle_weights(d):
    return (d["w_q"], d["w_k"], d["w_v"], d["w_g"], d["w_gamma"], d["w_o"], d.get("alpha"))


def y_bound(out_ref, Wo, y_ref, state_bf16):
    """Largest |y_gpu - y_oracle| the arithmetic allows: each layer output
    may differ by its tolerance plus one bf16 ulp (both sides round it), the
    fp32 accumulation of the product adds at most 2^-16 of the absolute sum
    here, and y itself is rounded to bf16 on both sides (one more ulp)."""
    o = np.abs(np.asarray(out_ref, np.float64))
    if state_bf16:
        rms = np.sqrt((o ** 2).mean(-1, keepdims=True))
        e = 2e-2 * np.maximum(o, rms)
    else:
        e = 1e-6 + 1e-5 * o
    e = (e + bf16_ulp(o)).reshape(*o.shape[:-2], -1)
    a = np.abs(np.asarray(Wo, np.float64))
    o2 = o.reshape(*o.shape[:-2], -1)
    return e @ a + 2.0 ** -16 * (o2 @ a) + bf16_ulp(np.abs(y_ref))


# Cuts that keep the oracle within seconds; d_model 256.
CASES = {
    "top8": ("prefill_top8", dict(B=2, T=333, H=8)),
    "top32": ("prefill_top32", dict(B=1, T=300, H=8)),
    "short": ("prefill_top8", dict(B=3, T=17, H=4)),          # serial path, fp32 out copy
    "large_state": ("large_state", dict(B=1, T=70, H=3)),
}
D_MODEL = 256


@pytest.mark.parametrize("alpha", [None, "general"])
def test_address_weights_are_tempered_exactly(rn, P, alpha):
    """x = identity rows: q and k are the rows of W = bf16(e^alpha W')
    (one-term sums), so they show the tempered weights bit for bit."""
    w = synth.WORKLOADS["prefill_top8"]
    H, D = 8, 64
    d = synth.make_layer_weights(w, D, B=1, T=D, H=H, kind="gauss", alpha=alpha)
    d["x"] = np.eye(D, dtype=np.float32)[None]
    gw = gpu_weights(rn, d)
    plan = rn.LayerPlan(1, D, H, w.d_p, w.U, w.K, w.d_v, D, torch.float32)
    got = plan.project_inputs(gw, bf(d["x"]))
    torch.cuda.synchronize()
    for nm, W in (("q", d["w_q"]), ("k", d["w_k"])):
        ref = P.address_weights(W, d.get("alpha"), H, w.L)
        assert np.array_equal(to_np(got[nm]).reshape(D, -1), ref), nm
    assert np.array_equal(to_np(got["v"]).reshape(D, -1), d["w_v"])
    assert np.array_equal(to_np(got["gamma"]).reshape(D, -1), d["w_gamma"])


@pytest.mark.parametrize("case", ["top8", "large_state"])
def test_projections_exact_on_grid(rn, P, case):
    name, cut = CASES[case]
    w = synth.WORKLOADS[name]
    d = synth.make_layer_weights(w, D_MODEL, **cut)
    B, T, H = cut["B"], cut["T"], cut["H"]
    plan = rn.LayerPlan(B, T, H, w.d_p, w.U, w.K, w.d_v, D_MODEL, torch.float32)
    got = plan.project_inputs(gpu_weights(rn, d), bf(d["x"]))
    torch.cuda.synchronize()
    ref = P.project_inputs(d["x"], *oracle_weights(d)[:5], d["alpha"], H=H, L=w.L, d_v=w.d_v)
    for nm in ("q", "k", "v", "g", "gamma"):
        assert np.array_equal(to_np(got[nm]), ref[nm]), nm


@pytest.mark.parametrize("B,T", [(2, 200), (1, 200), (3, 1)])
def test_projections_gaussian_within_accumulation_bound(rn, P, B, T):
    """Arbitrary bf16 inputs: an fp32 sum of D terms in any order is within
    D * 2^-24 * sum|x_i W_i| of the exact one, and rounding that to bf16 adds
    at most one bf16 ulp of the result; most results agree exactly.  The
    row counts cover prefill-sized and decoding-sized GEMMs (different
    library kernels)."""
    w = synth.WORKLOADS["prefill_top8"]
    H, D = 8, 512
    d = synth.make_layer_weights(w, D, B=B, T=T, H=H, kind="gauss", alpha="general")
    plan = rn.LayerPlan(B, T, H, w.d_p, w.U, w.K, w.d_v, D, torch.float32)
    got = plan.project_inputs(gpu_weights(rn, d), bf(d["x"]))
    torch.cuda.synchronize()
    ref = P.project_inputs(d["x"], *oracle_weights(d)[:5], d["alpha"], H=H, L=w.L, d_v=w.d_v)
    Wmap = {"q": P.address_weights(d["w_q"], d["alpha"], H, w.L),
            "k": P.address_weights(d["w_k"], d["alpha"], H, w.L),
            "v": d["w_v"], "g": d["w_g"], "gamma": d["w_gamma"]}
    ax = np.abs(d["x"].reshape(B * T, D).astype(np.float64))
    for nm in ("q", "k", "v", "g", "gamma"):
        g = to_np(got[nm]).astype(np.float64).reshape(B * T, -1)
        r = ref[nm].astype(np.float64).reshape(B * T, -1)
        bound = bf16_ulp(r) + D * 2.0 ** -24 * (ax @ np.abs(Wmap[nm].astype(np.float64)))
        diff = np.abs(g - r)
        bad = diff > bound
        assert not bad.any(), (nm, int(bad.sum()), np.argwhere(bad)[:3].tolist())
        frac = float((diff > 0).mean())
        assert frac < 0.01 or diff.size < 200, (nm, frac)


def run_forward(rn, P, case, cape=1, content_heads=0, alpha="pow2", norm=False):
    name, cut = CASES[case]
    w = synth.WORKLOADS[name].replace(pos0_max=5000, cape=cape)
    B, T, H = cut["B"], cut["T"], cut["H"]
    d = synth.make_layer_weights(w, D_MODEL, alpha=alpha, **cut)
    st = synth.make_inputs(w, B=B, T=T, H=H)
    sbf = w.state_dtype == "bf16"
    norm_w = (1.0 + 0.25 * np.sin(np.arange(w.d_v))).astype(np.float32) if norm else None
    # oracle
    S_ref, m_ref = st["S0"].copy(), st["m0"].copy()
    y_ref, res = P.layer_forward(d["x"], *oracle_weights(d), S_ref, m_ref, H=H, d_p=w.d_p,
                                 U=w.U, K=w.K, state_bf16=sbf, cape=cape, pos0=st["pos0"],
                                 norm_w=norm_w, content_heads=content_heads)
    # GPU
    sdt = torch.bfloat16 if sbf else torch.float32
    S = torch.from_numpy(st["S0"]).to(sdt).cuda()
    mass = torch.from_numpy(st["m0"]).cuda()
    pos0 = torch.from_numpy(st["pos0"]).cuda()
    nw = torch.from_numpy(norm_w).cuda() if norm else None
    y, addr = rn.layer_forward(gpu_weights(rn, d), bf(d["x"]), S, mass, d_p=w.d_p, U=w.U,
                               K=w.K, cape=cape, pos0=pos0, norm_w=nw,
                               export_addresses=True, content_heads=content_heads)
    torch.cuda.synchronize()
    return w, d, st, (y, addr, S, mass), (y_ref, res, S_ref, m_ref)


def weights_of(orc, w, logits, pos0, T, H, cape, content_heads):
    lg = logits.reshape(-1, w.L)
    M = w.M

    def f(flat, slots):
        b, t, h = flat // (T * H), (flat // H) % T, flat % H
        form = 0 if (content_heads >> min(h, 63)) & 1 else cape
        slots = np.asarray(slots, np.int64)
        if form:
            perm = orc.cape(np.arange(M, dtype=np.int32), int(pos0[b]) + t, w.U, w.d_p, form)
            inv = np.empty(M, np.int64)
            inv[perm] = np.arange(M)
            slots = inv[slots]
        return orc.slot_weights(lg[flat], w.U, w.d_p)[slots]
    return f


def check_forward(w, d, st, gpu, ref, cape=1, content_heads=0):
    import oracle as orc
    y, addr, S, mass = gpu
    y_ref, res, S_ref, m_ref = ref
    B, T, H = res["w_idx"].shape[:3]
    sbf = w.state_dtype == "bf16"
    inp = res["inputs"]
    g_wi, g_ww, g_ri, g_rw = (to_np(a) for a in addr)
    dw = compare_address_sets(g_wi, g_ww, res["w_idx"], res["w_wt"], res["w_gap"],
                              weights_of(orc, w, inp["k"], st["pos0"], T, H, cape, content_heads))
    dr = compare_address_sets(g_ri, g_rw, res["r_idx"], res["r_wt"], res["r_gap"],
                              weights_of(orc, w, inp["q"], st["pos0"], T, H, cape, content_heads))
    div = (dw | dr).any(2)                                     # [B,T]: any head
    first = np.where(div.any(1), div.argmax(1), T)             # [B]
    tmask = np.arange(T)[None, :] < first[:, None]             # [B,T]
    bound = y_bound(res["out"], d["w_o"], y_ref, sbf)
    gy = to_np(y).astype(np.float64)
    bad = (np.abs(gy - y_ref) > bound) & tmask[..., None]
    assert not bad.any(), (int(bad.sum()), np.argwhere(bad)[:3])
    clean = first == T
    gS, gm = to_np(S), to_np(mass)
    assert_close(gS[clean], S_ref[clean], sbf, "S", slot_state=True)
    assert_close(gm[clean], m_ref[clean], False, "mass")
    for b in range(B):
        for h in range(H):
            written = np.union1d(res["w_idx"][b, :, h].ravel(), g_wi[b, :, h].ravel())
            keep = np.ones(w.M, bool)
            keep[written] = False
            assert np.array_equal(gS[b, h][keep], st["S0"][b, h][keep])
            assert np.array_equal(gm[b, h][keep].view(np.uint32),
                                  st["m0"][b, h][keep].view(np.uint32))
    return int((~clean).sum())


@pytest.mark.parametrize("case", list(CASES))
def test_layer_forward_matches_oracle(rn, P, case):
    w, d, st, gpu, ref = run_forward(rn, P, case)
    check_forward(w, d, st, gpu, ref)


@pytest.mark.parametrize("cape,mask", [(2, 0b0101), (3, 0)])
def test_layer_forward_cape_forms_and_norm(rn, P, cape, mask):
    w, d, st, gpu, ref = run_forward(rn, P, "top8", cape=cape, content_heads=mask, norm=True,
                                     alpha=None)
    check_forward(w, d, st, gpu, ref, cape=cape, content_heads=mask)


def test_layer_step_matches_oracle(rn, P):
    """Decode steps of the whole layer from a pre-filled state; a sequence
    whose addresses legitimately differ at a near-tie is compared only up to
    that step."""
    import oracle as orc
    w = synth.WORKLOADS["decode"]
    B, H, steps, D = 24, 4, 6, D_MODEL
    st = synth.make_inputs(w, B=B, T=1, H=H)
    S_ref, m_ref = st["S0"].copy(), st["m0"].copy()
    S = torch.from_numpy(st["S0"]).to(torch.bfloat16).cuda()
    mass = torch.from_numpy(st["m0"]).cuda()
    plan = rn.LayerPlan(B, 1, H, w.d_p, w.U, w.K, w.d_v, D, torch.bfloat16, step=True)
    alive = np.ones(B, bool)
    for s in range(steps):
        d = synth.make_layer_weights(w, D, seed=100 + s, B=B, T=1, H=H)
        pos = st["pos0"] + s
        y_ref, res = P.layer_forward(d["x"], *oracle_weights(d), S_ref, m_ref, H=H, d_p=w.d_p,
                                     U=w.U, K=w.K, state_bf16=True, pos0=pos)
        y = torch.empty((B, D), dtype=torch.bfloat16, device="cuda")
        ao = rn.new_addresses((B, H, w.K), "cuda")
        plan(gpu_weights(rn, d), bf(d["x"][:, 0]), S, mass, y,
             pos=torch.from_numpy(pos).cuda(), addr_out=ao)
        torch.cuda.synchronize()
        inp = res["inputs"]
        g_wi, g_ww, g_ri, g_rw = (to_np(a)[:, None] for a in ao)
        dw = compare_address_sets(g_wi, g_ww, res["w_idx"], res["w_wt"], res["w_gap"],
                                  weights_of(orc, w, inp["k"], pos, 1, H, 1, 0))
        dr = compare_address_sets(g_ri, g_rw, res["r_idx"], res["r_wt"], res["r_gap"],
                                  weights_of(orc, w, inp["q"], pos, 1, H, 1, 0))
        alive &= ~(dw | dr)[:, 0].any(1)
        bound = y_bound(res["out"], d["w_o"], y_ref, True)[:, 0]
        ok = np.abs(to_np(y) - y_ref[:, 0]) <= bound
        assert ok[alive].all(), s
    gS, gm = to_np(S), to_np(mass)
    assert_close(gS[alive], S_ref[alive], True, "S", slot_state=True)
    assert_close(gm[alive], m_ref[alive], False, "mass")
    assert alive.sum() >= B // 2


def test_packed_weights_give_the_same_layer(rn, P):
    """Packing once (ramnet_pack_weights) and passing the packed matrix gives
    bit-identical results to packing inside every call."""
    w = synth.WORKLOADS["prefill_top8"].replace(pos0_max=100)
    B, T, H = 2, 96, 8
    d = synth.make_layer_weights(w, D_MODEL, B=B, T=T, H=H, kind="gauss", alpha="general")
    st = synth.make_inputs(w, B=B, T=T, H=H)
    W = gpu_weights(rn, d)
    plan = rn.LayerPlan(B, T, H, w.d_p, w.U, w.K, w.d_v, D_MODEL, torch.float32)
    Wp = rn.pack_weights(plan.p, W)
    x = bf(d["x"])
    pos0 = torch.from_numpy(st["pos0"]).cuda()
    res = []
    for weights in (W, Wp):
        S = torch.from_numpy(st["S0"]).cuda()
        mass = torch.from_numpy(st["m0"]).cuda()
        y = torch.empty_like(x)
        plan(weights, x, S, mass, y, pos=pos0)
        torch.cuda.synchronize()
        res.append((to_np(y), to_np(S), to_np(mass)))
    for a, b in zip(*res):
        assert np.array_equal(a, b)
