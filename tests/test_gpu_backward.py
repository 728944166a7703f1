"""GPU parity of the backward pass (ramnet_scan_backward) against the torch
fp64 autograd oracle (oracle/backward.py).

The GPU replays its own forward (fp32 state) and walks back in fp32; the
oracle differentiates an fp64 forward.  A unit whose GPU addresses
legitimately differ from the oracle's at a near-tie follows another valid
trajectory, and since gradients flow back over the whole sequence, such a
unit is left out of the comparison entirely.
"""
import os
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from sparse_slot_recurrent_amd import synth  # noqa: E402

sys.path.insert(0, os.path.dirname(__file__))
from parity import compare_address_sets, to_np  # noqa: E402

# |gpu - oracle| <= GRAD_TOL * (|oracle| + rms of the oracle tensor): fp32
# replay and adjoint against fp64 over a few hundred dependent steps (the
# worst case seen on these cuts is 1.3e-6, on the logit gradients)
GRAD_TOL = 1e-5
# bf16 state: both sides round every stored row to 8 significant bits, the
# GPU from an fp32 value and the oracle from an fp64 one; where the two
# roundings part (rarely), the trajectories differ by one bf16 ulp (2^-8);
# the worst case seen on the Top-32 cut is 1.6e-4
GRAD_TOL_BF16 = 2e-3


@pytest.fixture(scope="module")
def rn():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_slot_recurrent_amd import ramnet
    ramnet.load_library()
    return ramnet


@pytest.fixture(scope="module")
def BWo():
    import oracle
    oracle.load()
    from oracle import backward
    return backward


def dev(a, bf16=False):
    t = torch.from_numpy(np.ascontiguousarray(a, np.float32))
    return (t.to(torch.bfloat16) if bf16 else t).cuda()


CASES = {
    "tiny": ("tiny", dict(B=1, T=256, H=1), {}),
    "top32_bf16_state": ("prefill_top32", dict(B=1, T=64, H=2), {}),
    "top8": ("prefill_top8", dict(B=1, T=96, H=2), {}),
    "cape3_mask_norm": ("prefill_top8", dict(B=2, T=64, H=2), dict(cape=3, content_heads=0b10, norm=True)),
    "dp2": ("tiny", dict(B=1, T=80, H=2), dict(d_p=2, U=8, K=5)),
    # the largest K (8-bit base, 512 slots; three chunks at 32 tokens)
    "kmax": ("tiny", dict(B=1, T=70, H=1), dict(d_p=8, U=3, K=64)),
    # K = 1 (64 slots; two chunks at 64 tokens).  With one read per token
    # the RMSNorm leaves the output independent of the read weight except
    # through eps_norm, so d rho = <dr, S_j> is what remains after the 64
    # fp32 terms cancel (dr is orthogonal to r = rho S_j up to eps): dq is
    # compared to 1e-3 (worst seen 2.5e-4); dk, from the writes, keeps the
    # standard tolerance.
    "k1": ("tiny", dict(B=1, T=90, H=2), dict(d_p=4, U=3, K=1, dq_tol=1e-3)),
    # shapes of the per-token walk (state in HBM): d_v 128 with a bf16 state
    # (the decoding workload's layer), d_v 192 and 256, 4096 slots, and the
    # 4^8-slot workload itself (K = 32, bf16 state)
    "walk_dv128_bf16_state": ("decode", dict(B=1, T=48, H=2), dict(wl=dict(steps=0))),
    "walk_dv192": ("prefill_top8", dict(B=1, T=40, H=2), dict(wl=dict(d_v=192))),
    "walk_dv256_m4096": ("tiny", dict(B=1, T=40, H=2), dict(wl=dict(d_v=256, U=6, K=16))),
    "walk_large_state": ("large_state", dict(B=1, T=40, H=2), dict(wl=dict(steps=0))),
    # the walk with CAPE form B, a content-only head and a norm weight
    "walk_dv128_cape2_mask_norm": ("decode", dict(B=2, T=32, H=2),
                                   dict(wl=dict(steps=0), cape=2, content_heads=0b01, norm=True)),
}


def weights_of(orc, w, logits, pos0, T, H, cape, content_heads, U, d_p):
    lg = logits.reshape(-1, U * d_p)
    M = d_p ** U

    def f(flat, slots):
        b, t, h = flat // (T * H), (flat // H) % T, flat % H
        form = 0 if (content_heads >> min(h, 63)) & 1 else cape
        slots = np.asarray(slots, np.int64)
        if form:
            perm = orc.cape(np.arange(M, dtype=np.int32), int(pos0[b]) + t, U, d_p, form)
            inv = np.empty(M, np.int64)
            inv[perm] = np.arange(M)
            slots = inv[slots]
        return orc.slot_weights(lg[flat], U, d_p)[slots]
    return f


def close(name, got, ref, mask=None, tol=None):
    tol = GRAD_TOL if tol is None else tol
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if mask is not None:
        got, ref = got[mask], ref[mask]
    rms = np.sqrt((ref ** 2).mean()) if ref.size else 0.0
    err = np.abs(got - ref)
    worst = float((err / (np.abs(ref) + rms + 1e-30)).max()) if ref.size else 0.0
    assert np.isfinite(got).all(), name
    assert (err <= tol * (np.abs(ref) + rms)).all(), (name, worst)
    return worst


@pytest.mark.parametrize("case", list(CASES))
def test_backward_matches_oracle(rn, BWo, case):
    import oracle as orc
    name, cut, opt = CASES[case]
    w = synth.WORKLOADS[name].replace(s0_sigma=0.3, m0_uniform=(0.2, 1.5), pos0_max=3000,
                                      cape=opt.get("cape", 1))
    if "d_p" in opt:
        w = w.replace(d_p=opt["d_p"], U=opt["U"], K=opt["K"])
    if "wl" in opt:
        w = w.replace(**opt["wl"])
    B, T, H = cut["B"], cut["T"], cut["H"]
    x = synth.make_inputs(w, B=B, T=T, H=H)
    r = np.random.default_rng(99)
    dout = r.standard_normal((B, T, H, w.d_v)).astype(np.float32)
    dSf = r.standard_normal(x["S0"].shape).astype(np.float32)
    dmf = r.standard_normal(x["m0"].shape).astype(np.float32)
    norm_w = (1.0 + 0.25 * np.sin(np.arange(w.d_v))).astype(np.float32) if opt.get("norm") else None
    mask = opt.get("content_heads", 0)
    sbf = w.state_dtype == "bf16"
    ref = BWo.layer_grads(x["q"], x["k"], x["v"], x["gamma"], x["g"], x["S0"], x["m0"], dout,
                          d_p=w.d_p, U=w.U, K=w.K, cape=w.cape, pos0=x["pos0"], norm_w=norm_w,
                          content_heads=mask, dS_final=dSf, dm_final=dmf, round_storage=True,
                          state_bf16=sbf)
    bf = w.in_dtype == "bf16"
    d = {n: dev(x[n], bf) for n in ("q", "k", "v", "gamma", "g")}
    S0, m0 = dev(x["S0"], sbf), dev(x["m0"])
    S, m = S0.clone(), m0.clone()
    pos0 = torch.from_numpy(x["pos0"]).cuda()
    nw = dev(norm_w) if norm_w is not None else None
    _, addr = rn.scan_prefill(d["q"], d["k"], d["v"], d["gamma"], d["g"], S, m, d_p=w.d_p,
                              U=w.U, K=w.K, cape=w.cape, pos0=pos0, norm_w=nw,
                              export_addresses=True, content_heads=mask)
    got = rn.scan_backward(d["q"], d["k"], d["v"], d["gamma"], d["g"], S0, m0, addr, dev(dout),
                           d_p=w.d_p, U=w.U, K=w.K, cape=w.cape, norm_w=nw, pos0=pos0,
                           content_heads=mask, dS_final=dev(dSf), dmass_final=dev(dmf))
    torch.cuda.synchronize()
    g_wi, g_ww, g_ri, g_rw = (to_np(a) for a in addr)
    # the oracle's weights, for the tie-aware comparison of the sets
    _, o_ww, _ = orc.decode_all(x["k"], w.U, w.d_p, w.K, cape=w.cape, pos0=x["pos0"], content_heads=mask)
    _, o_rw, _ = orc.decode_all(x["q"], w.U, w.d_p, w.K, cape=w.cape, pos0=x["pos0"], content_heads=mask)
    dw = compare_address_sets(g_wi, g_ww, ref["w_idx"], o_ww, ref["w_gap"],
                              weights_of(orc, w, x["k"], x["pos0"], T, H, w.cape, mask, w.U, w.d_p))
    dr = compare_address_sets(g_ri, g_rw, ref["r_idx"], o_rw, ref["r_gap"],
                              weights_of(orc, w, x["q"], x["pos0"], T, H, w.cape, mask, w.U, w.d_p))
    clean = ~(dw | dr).any(1)            # [B, H]: units with the oracle's sets throughout
    assert clean.mean() >= 0.5
    tok = np.broadcast_to(clean[:, None, :], (B, T, H))
    tol = GRAD_TOL_BF16 if sbf else GRAD_TOL
    worst = {}
    for n, m_ in (("dv", tok), ("dg", tok), ("dgamma", tok), ("dq", tok), ("dk", tok)):
        worst[n] = close(n, to_np(got[n]), ref[n], m_, opt.get("dq_tol", tol) if n == "dq" else tol)
    worst["dS0"] = close("dS0", to_np(got["dS0"]), ref["dS0"], clean, tol)
    worst["dm0"] = close("dm0", to_np(got["dmass0"]), ref["dm0"], clean, tol)
    if clean.all():
        worst["dnorm_w"] = close("dnorm_w", to_np(got["dnorm_w"]), ref["dnorm_w"], None, tol)
    print(case, {k: f"{v:.2e}" for k, v in worst.items()}, "clean units", int(clean.sum()), "of", clean.size)


def test_backward_repeatable(rn):
    """Two calls on the same inputs give the same bits."""
    w = synth.WORKLOADS["prefill_top8"].replace(s0_sigma=0.3, m0_uniform=(0.2, 1.5))
    B, T, H = 2, 64, 3
    x = synth.make_inputs(w, B=B, T=T, H=H)
    d = {n: dev(x[n], True) for n in ("q", "k", "v", "gamma", "g")}
    S0, m0 = dev(x["S0"]), dev(x["m0"])
    S, m = S0.clone(), m0.clone()
    _, addr = rn.scan_prefill(d["q"], d["k"], d["v"], d["gamma"], d["g"], S, m, d_p=w.d_p,
                              U=w.U, K=w.K, export_addresses=True)
    dout = dev(np.random.default_rng(5).standard_normal((B, T, H, w.d_v)))
    runs = [rn.scan_backward(d["q"], d["k"], d["v"], d["gamma"], d["g"], S0, m0, addr, dout,
                             d_p=w.d_p, U=w.U, K=w.K) for _ in range(2)]
    torch.cuda.synchronize()
    for n in runs[0]:
        if runs[0][n] is not None:
            assert torch.equal(runs[0][n], runs[1][n]), n


def test_full_size_directional_derivatives(rn):
    """At the Top-8 benchmark's full size (B 8, T 4096, H 8), the gradients of
    v, gamma, g, S0 and m0 against central differences of the GPU forward's
    loss along random directions.  Those inputs do not move the addresses,
    so the loss is smooth along them.  Tolerance: the forward is fp32, so
    the difference quotient carries about 1e-7 * |L| / eps of rounding; the
    worst error seen is 4.5e-6 of sum |grad| |direction| (gamma)."""
    w = synth.WORKLOADS["prefill_top8"].replace(s0_sigma=0.3, m0_uniform=(0.2, 1.5))
    B, T, H = w.B, w.T, w.H
    x = synth.make_inputs(w)
    d = {n: dev(x[n], True) for n in ("q", "k", "v", "gamma", "g")}
    base = {n: dev(x[n]) for n in ("v", "gamma", "g")}  # fp32 copies to perturb
    S0, m0 = dev(x["S0"]), dev(x["m0"])
    pos0 = torch.from_numpy(x["pos0"]).cuda()
    gen = torch.Generator(device="cuda")
    gen.manual_seed(7)
    dout = torch.randn(B, T, H, w.d_v, generator=gen, device="cuda")
    plan = rn.PrefillPlan(B, T, H, w.d_p, w.U, w.K, w.d_v, rn.F32, rn.F32, cape=w.cape)
    out = torch.empty(B, T, H, w.d_v, device="cuda")
    addr = rn.new_addresses((B, T, H, w.K), "cuda")
    q32, k32 = dev(x["q"]), dev(x["k"])

    def loss(v, gamma, g, S, m):
        S, m = S.clone(), m.clone()
        plan(q32, k32, v, gamma, g, S, m, out, pos0=pos0)
        return float((out.double() * dout.double()).sum())

    S, m = S0.clone(), m0.clone()
    plan(q32, k32, base["v"], base["gamma"], base["g"], S, m, out, pos0=pos0, addr_out=addr)
    gr = rn.scan_backward(q32, k32, base["v"], base["gamma"], base["g"], S0, m0, addr, dout,
                          d_p=w.d_p, U=w.U, K=w.K, cape=w.cape, pos0=pos0, want_logits=False)
    args = {"v": base["v"], "gamma": base["gamma"], "g": base["g"], "S": S0, "m": m0}
    grads = {"v": gr["dv"], "gamma": gr["dgamma"], "g": gr["dg"], "S": gr["dS0"], "m": gr["dmass0"]}
    for n, eps in (("v", 1e-3), ("gamma", 1e-3), ("g", 1e-3), ("S", 1e-3), ("m", 1e-3)):
        dirn = torch.randn(args[n].shape, generator=gen, device="cuda")
        if n == "m":
            dirn = dirn.abs()  # the mass stays positive
        ap, am = dict(args), dict(args)
        ap[n] = args[n] + eps * dirn
        am[n] = args[n] - eps * dirn
        fd = (loss(**ap) - loss(**am)) / (2 * eps)
        an = float((grads[n].double() * dirn.double()).sum())
        scale = float((grads[n].double().abs() * dirn.double().abs()).sum())
        print(f"{n}: difference quotient {fd:.6g}, gradient {an:.6g}, |error| / scale "
              f"{abs(fd - an) / scale:.2e}")
        assert abs(fd - an) <= 1e-4 * scale, (n, fd, an, scale)


@pytest.mark.parametrize("case", ["slot_owner_top8", "walk_dv128"])
def test_backward_given_addresses_with_repeats(rn, BWo, case):
    """Caller-given addresses in which a token writes one slot twice, reads
    one slot twice and reads a slot it writes: the writes to one slot apply
    in address order and a read sees the token's last write, as in the
    forward.  Both sides take the same addresses, so every unit is compared.
    Their weights are the Product Softmax weights of the slots' content
    digits, as the oracle differentiates them."""
    import oracle as orc
    name = {"slot_owner_top8": "prefill_top8", "walk_dv128": "decode"}[case]
    w = synth.WORKLOADS[name].replace(s0_sigma=0.3, m0_uniform=(0.2, 1.5), pos0_max=3000, steps=0)
    B, T, H = 1, 40, 2
    x = synth.make_inputs(w, B=B, T=T, H=H)
    wi, _, _ = orc.decode_all(x["k"], w.U, w.d_p, w.K, cape=w.cape, pos0=x["pos0"])
    ri, _, _ = orc.decode_all(x["q"], w.U, w.d_p, w.K, cape=w.cape, pos0=x["pos0"])
    wi, ri = wi.copy(), ri.copy()
    wi[:, ::3, :, 1] = wi[:, ::3, :, 0]      # one slot written twice
    ri[:, ::3, :, 2] = ri[:, ::3, :, 0]      # one slot read twice
    ri[:, 1::3, :, 3] = wi[:, 1::3, :, 0]    # a read of a slot the token writes
    fk = weights_of(orc, w, x["k"], x["pos0"], T, H, w.cape, 0, w.U, w.d_p)
    fq = weights_of(orc, w, x["q"], x["pos0"], T, H, w.cape, 0, w.U, w.d_p)
    ww = np.stack([fk(f, wi.reshape(-1, w.K)[f]) for f in range(B * T * H)]).reshape(wi.shape)
    rw = np.stack([fq(f, ri.reshape(-1, w.K)[f]) for f in range(B * T * H)]).reshape(ri.shape)
    r = np.random.default_rng(3)
    dout = r.standard_normal((B, T, H, w.d_v)).astype(np.float32)
    dSf = r.standard_normal(x["S0"].shape).astype(np.float32)
    dmf = r.standard_normal(x["m0"].shape).astype(np.float32)
    sbf = w.state_dtype == "bf16"
    ref = BWo.layer_grads(x["q"], x["k"], x["v"], x["gamma"], x["g"], x["S0"], x["m0"], dout,
                          d_p=w.d_p, U=w.U, K=w.K, cape=w.cape, pos0=x["pos0"], dS_final=dSf,
                          dm_final=dmf, round_storage=True, state_bf16=sbf, addresses=(wi, ri))
    bf = w.in_dtype == "bf16"
    d = {n: dev(x[n], bf) for n in ("q", "k", "v", "gamma", "g")}
    ti = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).cuda()
    addr = rn.Addresses(ti(wi), dev(ww), ti(ri), dev(rw))
    got = rn.scan_backward(d["q"], d["k"], d["v"], d["gamma"], d["g"], dev(x["S0"], sbf), dev(x["m0"]),
                           addr, dev(dout), d_p=w.d_p, U=w.U, K=w.K, cape=w.cape,
                           pos0=torch.from_numpy(x["pos0"]).cuda(), dS_final=dev(dSf), dmass_final=dev(dmf))
    torch.cuda.synchronize()
    tol = GRAD_TOL_BF16 if sbf else GRAD_TOL
    worst = {n: close(n, to_np(got[n]), ref[n], None, tol) for n in ("dv", "dg", "dgamma", "dq", "dk")}
    worst["dS0"] = close("dS0", to_np(got["dS0"]), ref["dS0"], None, tol)
    worst["dm0"] = close("dm0", to_np(got["dmass0"]), ref["dm0"], None, tol)
    print(case, {k: f"{v:.2e}" for k, v in worst.items()})


def test_full_size_large_state_directional_derivatives(rn):
    """The 4^8-slot workload at full size (B 2, T 32768, H 16, K 32), with an
    fp32 state so that the loss is smooth at the step sizes used: the
    gradients of v, gamma, g, S0 and m0 against central differences of the
    GPU forward's loss along random directions (those inputs do not move the
    addresses).  Same tolerance as the Top-8 case."""
    w = synth.WORKLOADS["large_state"].replace(s0_sigma=0.3, m0_uniform=(0.2, 1.5), state_dtype="f32")
    B, T, H = w.B, w.T, w.H
    x = synth.make_inputs(w)
    base = {n: dev(x[n]) for n in ("v", "gamma", "g")}
    S0, m0 = dev(x["S0"]), dev(x["m0"])
    pos0 = torch.from_numpy(x["pos0"]).cuda()
    q32, k32 = dev(x["q"]), dev(x["k"])
    del x
    gen = torch.Generator(device="cuda")
    gen.manual_seed(11)
    dout = torch.randn(B, T, H, w.d_v, generator=gen, device="cuda")
    plan = rn.PrefillPlan(B, T, H, w.d_p, w.U, w.K, w.d_v, rn.F32, rn.F32, cape=w.cape)
    out = torch.empty(B, T, H, w.d_v, device="cuda")
    addr = rn.new_addresses((B, T, H, w.K), "cuda")

    def loss(v, gamma, g, S, m):
        S, m = S.clone(), m.clone()
        plan(q32, k32, v, gamma, g, S, m, out, pos0=pos0)
        return float((out.double() * dout.double()).sum())

    S, m = S0.clone(), m0.clone()
    plan(q32, k32, base["v"], base["gamma"], base["g"], S, m, out, pos0=pos0, addr_out=addr)
    del S, m
    gr = rn.scan_backward(q32, k32, base["v"], base["gamma"], base["g"], S0, m0, addr, dout,
                          d_p=w.d_p, U=w.U, K=w.K, cape=w.cape, pos0=pos0, want_logits=False)
    torch.cuda.synchronize()
    args = {"v": base["v"], "gamma": base["gamma"], "g": base["g"], "S": S0, "m": m0}
    grads = {"v": gr["dv"], "gamma": gr["dgamma"], "g": gr["dg"], "S": gr["dS0"], "m": gr["dmass0"]}
    for n, eps in (("v", 1e-3), ("gamma", 1e-3), ("g", 1e-3), ("S", 1e-3), ("m", 1e-3)):
        dirn = torch.randn(args[n].shape, generator=gen, device="cuda")
        if n == "m":
            dirn = dirn.abs()  # the mass stays positive
        ap, am = dict(args), dict(args)
        ap[n] = args[n] + eps * dirn
        am[n] = args[n] - eps * dirn
        fd = (loss(**ap) - loss(**am)) / (2 * eps)
        an = float((grads[n].double() * dirn.double()).sum())
        scale = float((grads[n].double().abs() * dirn.double().abs()).sum())
        print(f"{n}: difference quotient {fd:.6g}, gradient {an:.6g}, |error| / scale "
              f"{abs(fd - an) / scale:.2e}", flush=True)
        assert abs(fd - an) <= 1e-4 * scale, (n, fd, an, scale)
