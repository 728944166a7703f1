"""The prefill entry point that allocates nothing (static device scratch)
against ramnet_scan_prefill with a caller's workspace: the same kernels on
the same inputs give the same bits.  Two calls in a row, the second smaller
(the scratch keeps the first call's contents), on the slot-grouped path with
rows in registers (Top-8 and Top-32 cuts, the latter with the hand-off),
with rows in HBM (4^8 slots), and on the short-prefill path; a prefill too
large for the scratch is refused before anything is enqueued."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from sparse_slot_recurrent_amd import synth  # noqa: E402


@pytest.fixture(scope="module")
def rn():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_slot_recurrent_amd import ramnet
    ramnet.load_library()
    return ramnet


def dev(a, dtype):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    return t.cuda()


def both(rn, w, x, export):
    """Runs the workspace entry point and the no-alloc one on copies of the
    same state; returns both results."""
    res = []
    for noalloc in (False, True):
        d = {n: dev(x[n], w.in_dtype) for n in ("q", "k", "v", "gamma", "g")}
        S, m = dev(x["S0"], w.state_dtype), dev(x["m0"], "f32")
        pos0 = torch.from_numpy(x["pos0"]).cuda()
        B, T, H = x["gamma"].shape
        sdt = torch.bfloat16 if w.state_dtype == "bf16" else torch.float32
        out = torch.full((B, T, H, w.d_v), float("nan"), dtype=sdt, device="cuda")
        ao = rn.new_addresses((B, T, H, w.K), "cuda") if export else None
        if noalloc:
            rn.scan_prefill_noalloc(d["q"], d["k"], d["v"], d["gamma"], d["g"], S, m, out,
                                    d_p=w.d_p, U=w.U, K=w.K, cape=w.cape, pos0=pos0,
                                    addr_out=ao)
        else:
            plan = rn.PrefillPlan(B, T, H, w.d_p, w.U, w.K, w.d_v,
                                  rn.BF16 if w.in_dtype == "bf16" else rn.F32,
                                  rn.BF16 if w.state_dtype == "bf16" else rn.F32, cape=w.cape)
            plan(d["q"], d["k"], d["v"], d["gamma"], d["g"], S, m, out, pos0=pos0, addr_out=ao)
        torch.cuda.synchronize()
        res.append((out, S, m, ao))
    return res


def assert_same(a, b, what):
    (o1, S1, m1, a1), (o2, S2, m2, a2) = a, b
    assert torch.equal(o1, o2), f"{what}: out"
    assert torch.equal(S1, S2), f"{what}: S"
    assert torch.equal(m1.view(torch.int32), m2.view(torch.int32)), f"{what}: mass"
    if a1 is not None:
        for f in ("w_idx", "w_wt", "r_idx", "r_wt"):
            assert torch.equal(getattr(a1, f), getattr(a2, f)), f"{what}: {f}"


@pytest.mark.parametrize("name,first,second,export", [
    ("prefill_top8", dict(B=2, T=700, H=8), dict(B=1, T=300, H=4), False),
    ("prefill_top32", dict(B=1, T=600, H=8), dict(B=1, T=200, H=2), True),
    ("large_state", dict(B=1, T=400, H=2), dict(B=1, T=150, H=1), False),
    ("tiny", dict(T=256), dict(T=20), True),
])
def test_noalloc_matches_workspace_entry(rn, name, first, second, export):
    w = synth.WORKLOADS[name]
    for i, cut in enumerate((first, second)):
        x = synth.make_inputs(w, **cut)
        a, b = both(rn, w, x, export)
        assert_same(a, b, f"{name} call {i + 1} {cut}")


def test_noalloc_refuses_a_prefill_too_large(rn):
    w = synth.WORKLOADS["prefill_top8"]
    B, T, H = w.B, w.T, w.H
    p = rn.make_params(B, T, H, w.d_p, w.U, w.K, w.d_v, rn.BF16, rn.F32)
    assert rn.workspace_bytes(p, rn.OP_PREFILL) > rn.NOALLOC_SCRATCH_BYTES
    x = synth.make_inputs(w, T=64)
    d = {n: dev(np.broadcast_to(x[n][:, :1], (B, T) + x[n].shape[2:]), "bf16")
         for n in ("q", "k", "v", "gamma", "g")}
    S, m = dev(np.zeros((B, H, w.M, w.d_v), np.float32), "f32"), dev(
        np.zeros((B, H, w.M), np.float32), "f32")
    out = torch.zeros((B, T, H, w.d_v), device="cuda")
    with pytest.raises(rn.RamnetError, match="static scratch"):
        rn.scan_prefill_noalloc(d["q"], d["k"], d["v"], d["gamma"], d["g"], S, m, out,
                                d_p=w.d_p, U=w.U, K=w.K)
    torch.cuda.synchronize()
    assert not S.any() and not out.any()
