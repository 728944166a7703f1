"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Inputs come from the seeded generator with each workload's shapes and value
distributions, cut to sizes the oracle finishes in seconds (several tiles
and a ragged tail), and at full size with the oracle run on sampled
(batch, head) units over the whole sequence.
"""
import os
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from sparse_slot_recurrent_amd import synth  # noqa: E402

sys.path.insert(0, os.path.dirname(__file__))
from parity import adopt, assert_close, compare_address_sets, to_np  # noqa: E402


@pytest.fixture(scope="module")
def rn():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_slot_recurrent_amd import ramnet
    ramnet.load_library()
    return ramnet


@pytest.fixture(scope="module")
def orc():
    import oracle
    oracle.load()
    return oracle


def dev(a, dtype):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    return t.cuda()


def tdt(name):
    return torch.bfloat16 if name == "bf16" else torch.float32


# Cuts that keep the oracle (brute-force Top-K) within seconds.
CUTS = {
    "tiny": dict(B=1, T=256, H=1),
    "prefill_top8": dict(B=2, T=333, H=8),
    "prefill_top32": dict(B=1, T=300, H=8),
    "large_state": dict(B=1, T=70, H=3),
}


def gpu_inputs(w, x):
    d = {n: dev(x[n], w.in_dtype) for n in ("q", "k", "v", "gamma", "g")}
    d["S"] = dev(x["S0"], w.state_dtype)
    d["mass"] = dev(x["m0"], "f32")
    d["pos0"] = torch.from_numpy(x["pos0"]).cuda()
    return d


def run_gpu(rn, w, x, addr_in=None, export=True, norm_w=None):
    d = gpu_inputs(w, x)
    res = rn.scan_prefill(d["q"], d["k"], d["v"], d["gamma"], d["g"], d["S"],
                          d["mass"], d_p=w.d_p, U=w.U, K=w.K, cape=w.cape,
                          pos0=d["pos0"], eps_gsu=w.eps_gsu,
                          eps_norm=w.eps_norm, addr_in=addr_in,
                          export_addresses=export, norm_w=norm_w)
    torch.cuda.synchronize()
    out, addr = res if export else (res, None)
    return out, addr, d


def run_oracle(orc, w, x, mode=0, norm_w=None):
    S = x["S0"].copy()
    m = x["m0"].copy()
    res = orc.layer(x["q"], x["k"], x["v"], x["gamma"], x["g"], S, m,
                    d_p=w.d_p, U=w.U, K=w.K, state_bf16=w.state_dtype == "bf16",
                    cape=w.cape, eps_gsu=w.eps_gsu, eps_norm=w.eps_norm,
                    pos0=x["pos0"], mode=mode, norm_w=norm_w)
    return res, S, m


def weights_fn(orc, w, x, logits_name, pos, content_heads=0):
    """Oracle fp64 weight of given post-CAPE slots of flat address f."""
    lg = x[logits_name].reshape(-1, w.L)
    B, T, H = x["gamma"].shape
    M = w.d_p ** w.U

    def f(flat, slots):
        b = flat // (T * H)
        t = (flat // H) % T
        h = flat % H
        P = int(pos[b]) + t
        form = 0 if (content_heads >> min(h, 63)) & 1 else w.cape
        slots = np.asarray(slots, np.int64)
        if form:
            perm = orc.cape(np.arange(M, dtype=np.int32), P, w.U, w.d_p, form)
            inv = np.empty(M, np.int64)
            inv[perm] = np.arange(M)
            slots = inv[slots]
        W = orc.slot_weights(lg[flat], w.U, w.d_p)
        return W[slots]
    return f


def check_layer(orc, w, x, out, addr, S, mass, ref, content_heads=0, norm_w=None):
    """Tie-aware address check; then the oracle's recurrence on the adopted
    addresses (its own, or the GPU's where a near-tie made both correct),
    compared with every output, the final state and the mass of every unit
    over the whole sequence; rows never written bit-exact.  Returns the
    number of units that adopted at least one GPU set."""
    bf = w.state_dtype == "bf16"
    g_wi, g_ww, g_ri, g_rw = (to_np(a) for a in addr)
    wf_k = weights_fn(orc, w, x, "k", x["pos0"], content_heads)
    wf_q = weights_fn(orc, w, x, "q", x["pos0"], content_heads)
    dw = compare_address_sets(g_wi, g_ww, ref["w_idx"], ref["w_wt"], ref["w_gap"], wf_k)
    dr = compare_address_sets(g_ri, g_rw, ref["r_idx"], ref["r_wt"], ref["r_gap"], wf_q)
    wi, ww = adopt(g_wi, ref["w_idx"], ref["w_wt"], dw, wf_k)
    ri, rw = adopt(g_ri, ref["r_idx"], ref["r_wt"], dr, wf_q)
    S_a, m_a = x["S0"].copy(), x["m0"].copy()
    out_a = orc.scan_given(wi, ww, ri, rw, x["v"], x["gamma"], x["g"], S_a, m_a,
                           d_p=w.d_p, U=w.U, state_bf16=bf, eps_gsu=w.eps_gsu,
                           eps_norm=w.eps_norm, norm_w=norm_w)
    B, T, H = x["gamma"].shape
    adopted = (dw | dr).any(1)                                   # [B,H]
    if "out" in ref:
        # where nothing was adopted, the recurrence on given addresses is the
        # oracle's own layer, bit for bit
        keep = ~adopted[:, None, :]
        assert np.array_equal(out_a[np.broadcast_to(keep, (B, T, H))],
                              ref["out"][np.broadcast_to(keep, (B, T, H))])
    got = to_np(out)
    assert got.shape[1] == out_a.shape[1] == T, "every token compared"
    assert_close(got, out_a, bf, "out")
    gS, gm = to_np(S), to_np(mass)
    assert_close(gS, S_a, bf, "S", slot_state=True)
    assert_close(gm, m_a, False, "mass")
    # rows never written: bit-exact
    for b in range(B):
        for h in range(H):
            written = np.union1d(wi[b, :, h].ravel(), g_wi[b, :, h].ravel())
            keep = np.ones(w.M, bool)
            keep[written] = False
            assert np.array_equal(gS[b, h][keep], x["S0"][b, h][keep])
            assert np.array_equal(gm[b, h][keep].view(np.uint32),
                                  x["m0"][b, h][keep].view(np.uint32))
    return int(adopted.sum())


@pytest.mark.parametrize("logits", ["plain", "ties", "spread"])
@pytest.mark.parametrize("name", ["prefill_top8", "prefill_top32", "large_state"])
def test_prefill_decoder_sets_equal_fp64_search(rn, orc, name, logits):
    """The prefill decodes bf16 logits in fixed point (exact integer drops;
    rounded drops with a per-cut margin where the logits span more than 30
    binary orders, the rest left to fp64); the standalone decoder searches
    in fp64.  Both rank by exact weight, ties by the smaller prefix, so the
    slot sets agree bit for bit.  "ties": logits on a coarse grid, most cuts
    exact ties.  "spread": a quarter of the logits scaled by 2^-40, so most
    addresses take the rounded drops."""
    w = synth.WORKLOADS[name]
    x = synth.make_inputs(w, **CUTS[name])
    if logits == "ties":
        for n in ("q", "k"):
            x[n] = (np.round(x[n] * 2) / 2).astype(x[n].dtype)
    elif logits == "spread":
        rng = np.random.default_rng(9)
        for n in ("q", "k"):
            small = rng.random(x[n].shape) < 0.25
            x[n] = np.where(small, x[n] * np.float32(2.0 ** -40), x[n]).astype(x[n].dtype)
    out, paddr, d = run_gpu(rn, w, x)
    addr = rn.decode_addresses(d["q"], d["k"], d_p=w.d_p, U=w.U, K=w.K,
                               cape=w.cape, pos0=d["pos0"])
    torch.cuda.synchronize()
    for lg, (pi, pw), (fi, fw) in (("k", paddr[:2], (addr.w_idx, addr.w_wt)),
                                   ("q", paddr[2:], (addr.r_idx, addr.r_wt))):
        pi, pw, fi, fw = to_np(pi), to_np(pw), to_np(fi), to_np(fw)
        assert np.array_equal(np.sort(pi, -1), np.sort(fi, -1)), lg
        po = np.take_along_axis(pw, np.argsort(pi, -1), -1)
        fo = np.take_along_axis(fw, np.argsort(fi, -1), -1)
        assert (np.abs(po - fo) <= 1e-5 * np.abs(fo)).all(), lg
        assert (np.diff(pw, axis=-1) <= 0).all(), lg
        oi, ow, og = orc.decode_all(x[lg], w.U, w.d_p, w.K, cape=w.cape, pos0=x["pos0"])
        compare_address_sets(pi, pw, oi, ow, og, weights_fn(orc, w, x, lg, x["pos0"]))
        near = float((og <= 2.0 ** -16).mean())
        print(f"{name} {logits} {lg}: {pi.shape[:-1]} addresses, "
              f"cuts within 2^-16: {near:.3f}")
        if logits == "ties":
            assert near > 0.1


@pytest.mark.parametrize("name", list(CUTS))
def test_decode_addresses(rn, orc, name):
    w = synth.WORKLOADS[name]
    x = synth.make_inputs(w, **CUTS[name])
    d = gpu_inputs(w, x)
    addr = rn.decode_addresses(d["q"], d["k"], d_p=w.d_p, U=w.U, K=w.K,
                               cape=w.cape, pos0=d["pos0"])
    torch.cuda.synchronize()
    for lg, (gi, gw), nm in (("k", (addr.w_idx, addr.w_wt), "write"),
                             ("q", (addr.r_idx, addr.r_wt), "read")):
        oi, ow, og = orc.decode_all(x[lg], w.U, w.d_p, w.K, cape=w.cape,
                                    pos0=x["pos0"])
        gi, gw = to_np(gi), to_np(gw)
        differ = compare_address_sets(gi, gw, oi, ow, og,
                                      weights_fn(orc, w, x, lg, x["pos0"]))
        # heaviest first within every address
        assert (np.diff(gw, axis=-1) <= 0).all(), nm
        print(f"{name} {nm}: {gi.shape[:-1]} addresses, near-ties "
              f"{int((og <= 1e-6).sum())}, differing sets {int(differ.sum())}")


@pytest.mark.parametrize("name", list(CUTS))
def test_prefill_matches_oracle(rn, orc, name):
    w = synth.WORKLOADS[name]
    x = synth.make_inputs(w, **CUTS[name])
    out, addr, d = run_gpu(rn, w, x)
    ref, _, _ = run_oracle(orc, w, x)
    n_div = check_layer(orc, w, x, out, addr, d["S"], d["mass"], ref)
    print(f"{name}: units with an adopted near-tie set: {n_div}")


@pytest.mark.parametrize("name", list(CUTS))
def test_prefill_with_oracle_addresses(rn, orc, name):
    """The recurrence alone: the oracle's addresses drive the GPU scan."""
    w = synth.WORKLOADS[name]
    x = synth.make_inputs(w, **CUTS[name])
    ref, S_ref, m_ref = run_oracle(orc, w, x)
    ai = rn.Addresses(torch.from_numpy(ref["w_idx"]).cuda(),
                      torch.from_numpy(ref["w_wt"].astype(np.float32)).cuda(),
                      torch.from_numpy(ref["r_idx"]).cuda(),
                      torch.from_numpy(ref["r_wt"].astype(np.float32)).cuda())
    out, addr, d = run_gpu(rn, w, x, addr_in=ai)
    bf = w.state_dtype == "bf16"
    assert_close(to_np(out), ref["out"], bf, "out")
    assert_close(to_np(d["S"]), S_ref, bf, "S", slot_state=True)
    assert_close(to_np(d["mass"]), m_ref, False, "mass")
    assert np.array_equal(to_np(addr.w_idx), ref["w_idx"])


@pytest.mark.parametrize("d_p,U,K,d_v,st_dt,T,pool,B,H", [
    # slot rows in registers, 8-channel slices; ~8 writes per slot and
    # token-chunk, busiest slots handed to helpers (two lanes per fp32 row)
    (4, 5, 16, 64, "f32", 300, 40, 1, 2),
    (4, 6, 8, 64, "bf16", 700, 300, 1, 2),    # 4096 slots: rows in HBM, slot-indexed plan table
    (4, 8, 16, 64, "bf16", 300, 5000, 1, 2),  # 65536 slots: rows in HBM, hashed plan table
    # rows in HBM at wider rows: fp32 partials and 32-lane norm groups
    # (d_v 128), 64-lane groups and an odd number of units (d_v 256)
    (4, 6, 8, 128, "f32", 300, 300, 1, 2),
    (2, 12, 16, 256, "bf16", 200, 500, 1, 3),
    # 64 units: 16-channel slices, hand-off with four lanes per fp32 row
    # (256 slots) and two lanes per bf16 row (1024 slots)
    (4, 4, 8, 64, "f32", 300, 60, 8, 8),
    (4, 5, 16, 64, "bf16", 300, 200, 8, 8),
])
def test_chunked_given_addresses_edge_cases(rn, orc, d_p, U, K, d_v, st_dt, T, pool, B, H):
    """Caller-given addresses through the slot-grouped path: two chunks with
    a ragged tail, slots drawn from a small pool (long per-slot write lists
    within a chunk), slots outside [0, M) and zero weights, which the ABI
    skips.  The oracle gets a skipped entry as slot 0 with weight 0, which
    changes nothing and reads nothing (project page, Gated Sparse Update:
    w = 0 gives alpha = 1 and lambda = 0)."""
    w = synth.Workload("given", B=B, T=T, H=H, d_p=d_p, U=U, K=K, d_v=d_v,
                       in_dtype="f32", state_dtype=st_dt, logit_sigma=1.0,
                       seed=21, s0_sigma=0.5, m0_uniform=(0.0, 2.0))
    x = synth.make_inputs(w)
    M = d_p ** U
    rng = np.random.default_rng(77)
    slots = rng.choice(M, size=pool, replace=False)

    def addresses():
        n = B * T * H
        idx = np.stack([rng.choice(slots, size=K, replace=False) for _ in range(n)])
        idx = idx.reshape(B, T, H, K).astype(np.int32)
        wt = rng.uniform(0.0, 1.0, idx.shape).astype(np.float32)
        wt[rng.random(idx.shape) < 0.05] = 0.0
        bad = rng.random(idx.shape) < 0.05
        nb = int(bad.sum())
        idx_g = idx.copy()
        idx_g[bad] = np.where(rng.random(nb) < 0.5, -1 - rng.integers(0, 3, nb),
                              M + rng.integers(0, 3, nb))
        idx_o, wt_o = idx.copy(), wt.copy()
        idx_o[bad] = 0
        wt_o[bad] = 0.0
        return idx_g, wt, idx_o, wt_o

    wi_g, ww_g, wi_o, ww_o = addresses()
    ri_g, rw_g, ri_o, rw_o = addresses()
    S_ref, m_ref = x["S0"].copy(), x["m0"].copy()
    ref = orc.scan_given(wi_o, ww_o, ri_o, rw_o, x["v"], x["gamma"], x["g"],
                         S_ref, m_ref, d_p=d_p, U=U, state_bf16=st_dt == "bf16")
    ai = rn.Addresses(*(torch.from_numpy(a).cuda() for a in (wi_g, ww_g, ri_g, rw_g)))
    out, _, d = run_gpu(rn, w, x, addr_in=ai, export=False)
    bf = st_dt == "bf16"
    assert_close(to_np(out), ref, bf, "out")
    assert_close(to_np(d["S"]), S_ref, bf, "S", slot_state=True)
    assert_close(to_np(d["mass"]), m_ref, False, "mass")
    # rows no valid write touched are bit-unchanged
    touched = np.zeros((B, H, M), bool)
    valid = (wi_g >= 0) & (wi_g < M) & (ww_g > 0)
    for b in range(B):
        for h in range(H):
            touched[b, h, wi_g[b, :, h][valid[b, :, h]]] = True
    S0 = x["S0"]
    S_gpu = to_np(d["S"])
    if bf:
        S0 = synth.round_bf16(S0)
    assert np.array_equal(S_gpu[~touched], S0[~touched])


def test_norm_weight_and_cape_off(rn, orc):
    w = synth.WORKLOADS["prefill_top8"].replace(cape=0)
    x = synth.make_inputs(w, B=1, T=100, H=4)
    nw = np.random.default_rng(5).uniform(0.5, 1.5, w.d_v).astype(np.float32)
    out, addr, d = run_gpu(rn, w, x, norm_w=torch.from_numpy(nw).cuda())
    ref, _, _ = run_oracle(orc, w, x, norm_w=nw)
    check_layer(orc, w, x, out, addr, d["S"], d["mass"], ref, norm_w=nw)


@pytest.mark.parametrize("cape,mask", [(2, 0), (3, 0), (2, 0b0101), (3, 0b1000)])
def test_cape_forms_and_content_heads(rn, orc, cape, mask):
    """CAPE readings B (2) and C (3) and per-head content-only addresses:
    the decoder alone and the whole prefill against the oracle."""
    w = synth.WORKLOADS["prefill_top8"].replace(cape=cape)
    x = synth.make_inputs(w, B=2, T=150, H=4)
    d = gpu_inputs(w, x)
    addr = rn.decode_addresses(d["q"], d["k"], d_p=w.d_p, U=w.U, K=w.K,
                               cape=cape, pos0=d["pos0"], content_heads=mask)
    torch.cuda.synchronize()
    for lg, gi, gw in (("k", addr.w_idx, addr.w_wt), ("q", addr.r_idx, addr.r_wt)):
        oi, ow, og = orc.decode_all(x[lg], w.U, w.d_p, w.K, cape=cape,
                                    pos0=x["pos0"], content_heads=mask)
        compare_address_sets(to_np(gi), to_np(gw), oi, ow, og,
                             weights_fn(orc, w, x, lg, x["pos0"], mask))
    res = rn.scan_prefill(d["q"], d["k"], d["v"], d["gamma"], d["g"], d["S"],
                          d["mass"], d_p=w.d_p, U=w.U, K=w.K, cape=cape,
                          pos0=d["pos0"], export_addresses=True, content_heads=mask)
    torch.cuda.synchronize()
    out, gaddr = res
    S_ref, m_ref = x["S0"].copy(), x["m0"].copy()
    ref = orc.layer(x["q"], x["k"], x["v"], x["gamma"], x["g"], S_ref, m_ref,
                    d_p=w.d_p, U=w.U, K=w.K, state_bf16=False, cape=cape,
                    pos0=x["pos0"], content_heads=mask)
    check_layer(orc, w, x, out, gaddr, d["S"], d["mass"], ref, content_heads=mask)


@pytest.mark.parametrize("cape,mask", [(2, 0b0011), (3, 0)])
def test_step_decode_cape_forms(rn, orc, cape, mask):
    """The fused decode step with CAPE readings B and C and mixed heads:
    8 sequences x 16 heads, 3 steps, every unit compared."""
    w = synth.WORKLOADS["decode"].replace(cape=cape)
    n_div, n_u, n_steps = decode_steps_check(rn, orc, w, 8, 3, content_heads=mask)
    assert n_steps == 3


@pytest.mark.parametrize("d_p,U,K,d_v,in_dt,st_dt", [
    (2, 3, 8, 64, "f32", "f32"),      # K = M
    (2, 10, 1, 64, "f32", "f32"),     # K = 1, deep tree
    (3, 4, 5, 128, "bf16", "bf16"),   # odd base, K not a power of two
    (5, 3, 7, 192, "f32", "bf16"),
    (8, 3, 64, 256, "bf16", "f32"),   # K = KMAX
    (4, 5, 32, 64, "f32", "bf16"),
])
def test_shapes_and_edge_parameters(rn, orc, d_p, U, K, d_v, in_dt, st_dt):
    w = synth.Workload("edge", B=2, T=37, H=3, d_p=d_p, U=U, K=K, d_v=d_v,
                       in_dtype=in_dt, state_dtype=st_dt, logit_sigma=1.5,
                       seed=11, s0_sigma=0.5, m0_uniform=(0.0, 2.0),
                       pos0_max=9)
    x = synth.make_inputs(w)
    out, addr, d = run_gpu(rn, w, x)
    ref, _, _ = run_oracle(orc, w, x)
    check_layer(orc, w, x, out, addr, d["S"], d["mass"], ref)


def test_extreme_gates_and_zero_eps(rn, orc):
    """gamma = -1000 (average all writes) and +1000 (overwrite) with
    eps_gsu = 0 and eps_norm = 0."""
    w = synth.WORKLOADS["tiny"].replace(eps_gsu=0.0, eps_norm=0.0)
    x = synth.make_inputs(w, T=64)
    x["gamma"][0, :32] = -1000.0
    x["gamma"][0, 32:] = 1000.0
    out, addr, d = run_gpu(rn, w, x)
    ref, _, _ = run_oracle(orc, w, x)
    check_layer(orc, w, x, out, addr, d["S"], d["mass"], ref)


def test_empty_calls_leave_state_untouched(rn):
    w = synth.WORKLOADS["tiny"]
    x = synth.make_inputs(w, T=4)
    d = gpu_inputs(w, x)
    S0 = d["S"].clone()
    for T in (0,):
        e = lambda a: a[:, :T].contiguous()
        out = rn.scan_prefill(e(d["q"]), e(d["k"]), e(d["v"]), e(d["gamma"]),
                              e(d["g"]), d["S"], d["mass"], d_p=w.d_p, U=w.U,
                              K=w.K)
        torch.cuda.synchronize()
        assert out.numel() == 0
    assert torch.equal(d["S"], S0)


@pytest.mark.parametrize("name", ["prefill_top8", "prefill_top32"])
def test_resume_and_steps(rn, name):
    """Split prefill = whole prefill, and one-token steps = prefill (GPU vs
    GPU).  Addresses agree bit for bit; values to the fp32 / bf16 tolerance,
    since the long-sequence path accumulates reads in arrival order and the
    two sides may take different paths."""
    w = synth.WORKLOADS[name]
    x = synth.make_inputs(w, B=2, T=40, H=4)
    bf = w.state_dtype == "bf16"
    out_w, addr_w, dw = run_gpu(rn, w, x)
    d = gpu_inputs(w, x)
    T1 = 13
    outs, addrs = [], []
    for sl, p0 in ((slice(0, T1), d["pos0"]), (slice(T1, 40), d["pos0"] + T1)):
        c = lambda a: a[:, sl].contiguous()
        o, ad = rn.scan_prefill(c(d["q"]), c(d["k"]), c(d["v"]), c(d["gamma"]),
                                c(d["g"]), d["S"], d["mass"], d_p=w.d_p, U=w.U,
                                K=w.K, pos0=p0, export_addresses=True)
        outs.append(o)
        addrs.append(ad)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([a.w_idx for a in addrs], 1), addr_w.w_idx)
    assert torch.equal(torch.cat([a.r_idx for a in addrs], 1), addr_w.r_idx)
    assert_close(to_np(torch.cat(outs, 1)), to_np(out_w), bf, "split out")
    assert_close(to_np(d["S"]), to_np(dw["S"]), bf, "split S", slot_state=True)
    assert_close(to_np(d["mass"]), to_np(dw["mass"]), False, "split mass")
    d2 = gpu_inputs(w, x)
    for t in range(40):
        o = rn.step_decode(d2["q"][:, t].contiguous(), d2["k"][:, t].contiguous(),
                           d2["v"][:, t].contiguous(), d2["gamma"][:, t].contiguous(),
                           d2["g"][:, t].contiguous(), d2["pos0"] + t, d2["S"],
                           d2["mass"], d_p=w.d_p, U=w.U, K=w.K)
        assert_close(to_np(o), to_np(out_w[:, t]), bf, f"step {t}")
    assert_close(to_np(d2["S"]), to_np(dw["S"]), bf, "steps S", slot_state=True)


def decode_steps_check(rn, orc, w, B, n_steps, seqs=None, content_heads=0, tier_lines=None,
                       rebalance_every=4):
    """Runs n_steps decode steps for all B x H units on the GPU and, for the
    sequences `seqs` (None = all; every head of each), in the oracle.  Each
    step: addresses tie-aware against the oracle's; then the oracle's GSU,
    read, norm and gate on the adopted addresses (its own, or the GPU's where
    a near-tie made both correct), so every step of every sampled unit is
    compared, and the state and mass at the end.  With tier_lines, the GPU
    runs the tiered step (rows in pinned host memory, tier_lines cached per
    unit, a rebalance every rebalance_every steps) and its state is flushed
    to host memory at the end.  Returns (units that adopted a GPU set, units
    compared, steps compared)."""
    H = w.H
    init = synth.make_inputs(w, B=B, T=1)
    S_d = dev(init["S0"], "bf16")
    m_d = dev(init["m0"], "f32")
    if tier_lines:
        tp = rn.make_params(B, 1, H, w.d_p, w.U, w.K, w.d_v, rn.BF16, rn.BF16, cape=w.cape,
                            content_heads=content_heads)
        ts = rn.TieredState(S_d, tier_lines)
        rn.tier_reset(tp, ts)
        del S_d
    seqs = np.arange(B) if seqs is None else np.asarray(seqs)
    # the oracle holds the sampled sequences (all heads) as a batch
    S_o = np.ascontiguousarray(init["S0"][seqs])
    m_o = np.ascontiguousarray(init["m0"][seqs])
    pos = init["pos0"].copy()
    adopted = np.zeros((len(seqs), H), bool)
    plan = rn.StepPlan(B, H, w.d_p, w.U, w.K, w.d_v, rn.BF16, rn.BF16,
                       cape=w.cape, device="cuda", content_heads=content_heads)
    out = torch.empty((B, H, w.d_v), dtype=torch.bfloat16, device="cuda")
    ao = rn.new_addresses((B, H, w.K), "cuda")
    done = 0
    for step in range(n_steps):
        s = synth.make_decode_step(w, step, B=B)
        if tier_lines:
            rn.step_decode_tiered(tp, dev(s["q"], "bf16"), dev(s["k"], "bf16"), dev(s["v"], "bf16"),
                                  dev(s["gamma"], "bf16"), dev(s["g"], "bf16"),
                                  torch.from_numpy(pos).cuda(), ts, m_d, out, addr_out=ao)
            if (step + 1) % rebalance_every == 0:
                rn.tier_rebalance(tp, ts)
        else:
            plan(dev(s["q"], "bf16"), dev(s["k"], "bf16"), dev(s["v"], "bf16"),
                 dev(s["gamma"], "bf16"), dev(s["g"], "bf16"),
                 torch.from_numpy(pos).cuda(), S_d, m_d, out, addr_out=ao)
        torch.cuda.synchronize()
        x = {n: np.ascontiguousarray(s[n][seqs][:, None]) for n in s}  # [b,1,H,*]
        p_u = np.ascontiguousarray(pos[seqs])
        xs = dict(x, pos0=p_u)
        sel = lambda a: np.ascontiguousarray(to_np(a)[seqs][:, None])
        g_wi, g_ww, g_ri, g_rw = (sel(a) for a in ao)
        res = {}
        for nm, lg in (("w", "k"), ("r", "q")):
            oi, ow, og = orc.decode_all(x[lg], w.U, w.d_p, w.K, cape=w.cape, pos0=p_u,
                                        content_heads=content_heads)
            gi, gw = (g_wi, g_ww) if nm == "w" else (g_ri, g_rw)
            wf = weights_fn(orc, w, xs, lg, p_u, content_heads)
            d = compare_address_sets(gi, gw, oi, ow, og, wf)
            res[nm] = adopt(gi, oi, ow, d, wf)
            adopted |= d[:, 0]
        ref = orc.scan_given(*res["w"], *res["r"], x["v"], x["gamma"], x["g"], S_o, m_o,
                             d_p=w.d_p, U=w.U, state_bf16=True, eps_gsu=w.eps_gsu,
                             eps_norm=w.eps_norm)
        assert_close(to_np(out)[seqs], ref[:, 0], True, f"out step {step}")
        pos = pos + 1
        done += 1
    if tier_lines:
        rn.tier_flush(tp, ts)
        torch.cuda.synchronize()
        S_d = ts.S_host
    assert_close(to_np(S_d)[seqs], S_o, True, "S", slot_state=True)
    assert_close(to_np(m_d)[seqs], m_o, False, "mass")
    return int(adopted.sum()), adopted.size, done


def test_decode_steps_match_oracle(rn, orc):
    """Batched decode from a pre-filled random state: 6 steps, 64 sequences x
    16 heads, d_v = 128, K = 16, bf16 state; all units checked."""
    n_div, n_u, n_steps = decode_steps_check(rn, orc, synth.WORKLOADS["decode"], 64, 6)
    assert n_steps == 6
    print(f"decode cut: {n_div} of {n_u} units adopted a near-tie set")


def test_full_size_decode_sampled(rn, orc):
    """The decode workload in full: 256 sequences x 16 heads for all 1024
    steps on the GPU, with the oracle on two sampled sequences (32 units)
    for every step."""
    w = synth.WORKLOADS["decode"]
    seqs = np.random.default_rng(99).choice(w.B, size=2, replace=False)
    n_div, n_u, n_steps = decode_steps_check(rn, orc, w, w.B, w.steps, seqs=seqs)
    assert n_steps == w.steps == 1024
    print(f"decode full size: {n_steps} steps, {n_div} of {n_u} sampled units "
          f"adopted a near-tie set")


@pytest.mark.parametrize("name", ["prefill_top8", "prefill_top32"])
def test_full_size_prefill(rn, orc, name):
    """The benchmark's prefill shape in full, every unit.  (1) The oracle's
    addresses drive the GPU recurrence (given addresses, token-major): every
    output and the whole final state.  (2) The GPU's own call (decoder, then
    the recurrence on its head-major addresses) against the oracle on the
    adopted addresses: every token, state and mass."""
    w = synth.WORKLOADS[name]
    x = synth.make_inputs(w)
    ref, S_ref, m_ref = run_oracle(orc, w, x)
    ai = rn.Addresses(torch.from_numpy(ref["w_idx"]).cuda(),
                      torch.from_numpy(ref["w_wt"].astype(np.float32)).cuda(),
                      torch.from_numpy(ref["r_idx"]).cuda(),
                      torch.from_numpy(ref["r_wt"].astype(np.float32)).cuda())
    out, _, d = run_gpu(rn, w, x, addr_in=ai)
    bf = w.state_dtype == "bf16"
    assert_close(to_np(out), ref["out"], bf, "out")
    assert_close(to_np(d["S"]), S_ref, bf, "S", slot_state=True)
    assert_close(to_np(d["mass"]), m_ref, False, "mass")
    del out, d, ai, S_ref, m_ref
    out, addr, d = run_gpu(rn, w, x)
    n_adopt = check_layer(orc, w, x, out, addr, d["S"], d["mass"], ref)
    print(f"{name} full size: {x['gamma'].size} token-heads, "
          f"{n_adopt} units adopted a near-tie set")


def _large_state_unit_check(orc, w, x, b, h, out, addr, S, mass):
    """One (b, h) unit of the full-size 4^8-slot run against the oracle over
    the whole sequence: tree-search addresses (pinned equal to brute force),
    with brute-force margins where the GPU's set differs; the adopted
    recurrence; every output, the unit's state and mass."""
    xu = {n: np.ascontiguousarray(x[n][b:b + 1, :, h:h + 1])
          for n in ("q", "k", "v", "gamma", "g")}
    xu["S0"] = np.ascontiguousarray(x["S0"][b:b + 1, h:h + 1])
    xu["m0"] = np.ascontiguousarray(x["m0"][b:b + 1, h:h + 1])
    xu["pos0"] = x["pos0"][b:b + 1].copy()
    ref = {}
    for nm, lg in (("w", "k"), ("r", "q")):
        oi, ow, _ = orc.decode_all(xu[lg], w.U, w.d_p, w.K, cape=w.cape,
                                   pos0=xu["pos0"], mode=orc.TOPK_TREE)
        gap = np.full(oi.shape[:-1], np.inf)
        gi = to_np(getattr(addr, nm + "_idx")[b:b + 1, :, h:h + 1])
        diff = ~(np.sort(gi, -1) == np.sort(oi, -1)).all(-1)
        for f in np.nonzero(diff.reshape(-1))[0]:
            _, _, gp, _, _ = orc.decode_one(xu[lg].reshape(-1, w.L)[f], w.U, w.d_p, w.K,
                                            cape=w.cape, pos=int(xu["pos0"][0]) + int(f))
            gap.reshape(-1)[f] = gp
        ref[nm + "_idx"], ref[nm + "_wt"], ref[nm + "_gap"] = oi, ow, gap
    au = type(addr)(*[a[b:b + 1, :, h:h + 1].contiguous() for a in addr])
    return check_layer(orc, w, xu, out[b:b + 1, :, h:h + 1].contiguous(), au,
                       S[b:b + 1, h:h + 1].contiguous(),
                       mass[b:b + 1, h:h + 1].contiguous(), ref)


@pytest.fixture(scope="module")
def large_state_inputs():
    return synth.make_inputs(synth.WORKLOADS["large_state"])


def test_full_size_large_state_sampled(rn, orc, large_state_inputs):
    """The 4^8-slot prefill at full size (B 2, T 32768, H 16) in the
    benchmark's launch configuration: the GPU's own call in full, and two
    sampled units compared with the oracle over all 32768 tokens (addresses
    tie-aware, then the adopted recurrence: every output, state, mass)."""
    w = synth.WORKLOADS["large_state"]
    x = large_state_inputs
    out, addr, d = run_gpu(rn, w, x)
    for b, h in ((0, 0), (1, 11)):
        n = _large_state_unit_check(orc, w, x, b, h, out, addr, d["S"], d["mass"])
        print(f"large_state unit ({b},{h}): all {w.T} tokens compared, adopted "
              f"near-tie sets: {bool(n)}")


def test_large_state_given_addresses_full_length(rn, orc, large_state_inputs):
    """The 4^8-slot, K = 32, bf16-row scan driven by the oracle's
    tree-search addresses over the whole sequence (B 1, H 2, T 32768): every
    output, the whole final state and mass, with no tie exemption."""
    w = synth.WORKLOADS["large_state"]
    x = {n: np.ascontiguousarray(large_state_inputs[n][:1, :, :2])
         for n in ("q", "k", "v", "gamma", "g")}
    x["S0"] = np.ascontiguousarray(large_state_inputs["S0"][:1, :2])
    x["m0"] = np.ascontiguousarray(large_state_inputs["m0"][:1, :2])
    x["pos0"] = large_state_inputs["pos0"][:1].copy()
    wi, ww, _ = orc.decode_all(x["k"], w.U, w.d_p, w.K, cape=w.cape, pos0=x["pos0"],
                               mode=orc.TOPK_TREE)
    ri, rw, _ = orc.decode_all(x["q"], w.U, w.d_p, w.K, cape=w.cape, pos0=x["pos0"],
                               mode=orc.TOPK_TREE)
    S_ref, m_ref = x["S0"].copy(), x["m0"].copy()
    ref = orc.scan_given(wi, ww, ri, rw, x["v"], x["gamma"], x["g"], S_ref, m_ref,
                         d_p=w.d_p, U=w.U, state_bf16=True)
    ai = rn.Addresses(*(torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in
                        (wi, ww.astype(np.float32), ri, rw.astype(np.float32))))
    out, _, d = run_gpu(rn, w, x, addr_in=ai, export=False)
    assert out.shape[1] == w.T
    assert_close(to_np(out), ref, True, "out")
    assert_close(to_np(d["S"]), S_ref, True, "S", slot_state=True)
    assert_close(to_np(d["mass"]), m_ref, False, "mass")


@pytest.mark.parametrize("name", ["prefill_top8", "prefill_top32"])
def test_prefill_bitwise_repeatable(rn, name):
    """The slot-grouped prefill is deterministic: every sum runs in a fixed
    order, and the helpers that take over the busiest slots (whose
    assignment varies from run to run) apply each slot's writes with the
    same arithmetic.  Two runs over several chunks give identical bits in
    the outputs, the state, the mass and the addresses."""
    w = synth.WORKLOADS[name]
    x = synth.make_inputs(w, B=1, T=600, H=8)
    o1, a1, d1 = run_gpu(rn, w, x)
    o2, a2, d2 = run_gpu(rn, w, x)
    for f in ("w_idx", "w_wt", "r_idx", "r_wt"):
        assert torch.equal(getattr(a1, f), getattr(a2, f)), f
    assert torch.equal(o1, o2)
    assert torch.equal(d1["S"], d2["S"])
    assert torch.equal(d1["mass"], d2["mass"])


def test_repeatability(rn):
    """Two runs on the same inputs: addresses identical; values equal to the
    fp32 rounding of the read accumulation order."""
    w = synth.WORKLOADS["prefill_top32"]
    x = synth.make_inputs(w, B=1, T=200, H=8)
    o1, a1, d1 = run_gpu(rn, w, x)
    o2, a2, d2 = run_gpu(rn, w, x)
    assert torch.equal(a1.w_idx, a2.w_idx) and torch.equal(a1.r_wt, a2.r_wt)
    assert_close(to_np(o2), to_np(o1), True, "out")
    assert_close(to_np(d2["S"]), to_np(d1["S"]), True, "S", slot_state=True)


def test_binding_checks_shapes_and_dtypes(rn):
    """Tensors whose shape or dtype disagree with the parameters are refused
    by the binding before anything is enqueued (the C ABI derives every
    extent from the parameters)."""
    w = synth.WORKLOADS["tiny"]
    x = synth.make_inputs(w, T=40)
    d = gpu_inputs(w, x)
    plan = rn.PrefillPlan(1, 40, 1, w.d_p, w.U, w.K, w.d_v, rn.F32, rn.F32)
    out = torch.empty((1, 40, 1, w.d_v), device="cuda")
    S0, m0 = d["S"].clone(), d["mass"].clone()
    args = [d[n] for n in ("q", "k", "v", "gamma", "g")]
    bad = [("S", d["S"][:, :, :512].contiguous()), ("mass", d["mass"].to(torch.bfloat16)),
           ("out", out.double())]
    for name, t in bad:
        kw = {"S": d["S"], "mass": d["mass"], "out": out}
        kw[name] = t
        with pytest.raises(ValueError, match=name):
            plan(*args, kw["S"], kw["mass"], kw["out"])
    with pytest.raises(ValueError, match="pos0"):
        plan(*args, d["S"], d["mass"], out, pos0=d["pos0"].long())
    a = rn.new_addresses((1, 40, 1, w.K), "cuda")
    with pytest.raises(ValueError, match="addr_in.w_wt"):
        plan(*args, d["S"], d["mass"], out,
             addr_in=a._replace(w_wt=a.w_wt.double()))
    torch.cuda.synchronize()
    assert torch.equal(d["S"], S0) and torch.equal(d["mass"], m0)
