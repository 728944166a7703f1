"""GPU tests of the tiered decoding state (ramnet_step_decode_tiered and the
cache upkeep calls): rows in pinned host memory, the most accessed ones of
each unit cached in device memory.

* Against the oracle: the decoding check of test_gpu_parity run on the
  tiered state (every step of every unit, the state flushed to host memory
  at the end).
* Against the all-in-HBM step: bit-identical outputs, addresses, masses and
  final state over many steps with rebalances in between (only where a row
  lives differs).
* The rebalance's choice of cached slots against the rule stated in
  include/ramnet.h, computed here on the host from the counts it started
  from.
"""
import os
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from sparse_slot_recurrent_amd import synth  # noqa: E402

sys.path.insert(0, os.path.dirname(__file__))
from parity import to_np  # noqa: E402


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
    t = torch.from_numpy(np.ascontiguousarray(a, np.float32))
    return (t.to(torch.bfloat16) if dtype == "bf16" else t).cuda()


def test_tiered_decode_steps_match_oracle(rn, orc):
    """16 sequences x 16 heads of the decoding workload (M 1024, K 16, d_v
    128, bf16 state), 12 steps, 128 of 1024 rows per unit cached, a
    rebalance every 3 steps: every unit against the oracle."""
    from test_gpu_parity import decode_steps_check
    n_div, n_u, n_steps = decode_steps_check(rn, orc, synth.WORKLOADS["decode"], 16, 12,
                                             tier_lines=128, rebalance_every=3)
    assert n_steps == 12
    print(f"tiered decode: {n_div} of {n_u} units adopted a near-tie set")


CASES = {
    # the decoding workload's layer, an eighth of the rows cached
    "decode_bf16": (dict(), 64, 128, 16, 3),
    # fp32 state, 4096 slots, d_v 64, K 8, every unit rebalanced each step
    "m4096_f32": (dict(U=6, K=8, d_v=64, state_dtype="f32", in_dtype="f32"), 24, 512, 10, 1),
    # a cache of one line
    "one_line": (dict(K=4), 8, 1, 8, 2),
    # CAPE form C, d_v 256, K 32
    "cape3_dv256_k32": (dict(cape=3, d_v=256, K=32), 8, 64, 6, 2),
}


@pytest.mark.parametrize("case", list(CASES))
def test_tiered_step_bitwise_equals_plain(rn, case):
    repl, B, lines, n_steps, every = CASES[case]
    w = synth.WORKLOADS["decode"].replace(**repl)
    H = w.H
    bf = w.state_dtype == "bf16"
    sd = rn.BF16 if bf else rn.F32
    ind = rn.BF16 if w.in_dtype == "bf16" else rn.F32
    init = synth.make_inputs(w, B=B, T=1)
    S = dev(init["S0"], w.state_dtype)
    m_plain = dev(init["m0"], "f32")
    m_tier = m_plain.clone()
    p = rn.make_params(B, 1, H, w.d_p, w.U, w.K, w.d_v, ind, sd, cape=w.cape)
    ts = rn.TieredState(S, lines)
    rn.tier_reset(p, ts)
    plan = rn.StepPlan(B, H, w.d_p, w.U, w.K, w.d_v, ind, sd, cape=w.cape, device="cuda")
    odt = torch.bfloat16 if bf else torch.float32
    o1 = torch.empty((B, H, w.d_v), dtype=odt, device="cuda")
    o2 = torch.empty_like(o1)
    a1 = rn.new_addresses((B, H, w.K), "cuda")
    a2 = rn.new_addresses((B, H, w.K), "cuda")
    pos = torch.from_numpy(init["pos0"]).cuda()
    for step in range(n_steps):
        s = synth.make_decode_step(w, step, B=B)
        x = [dev(s[n], w.in_dtype) for n in ("q", "k", "v", "gamma", "g")]
        plan(*x, pos, S, m_plain, o1, addr_out=a1)
        rn.step_decode_tiered(p, *x, pos, ts, m_tier, o2, addr_out=a2)
        if (step + 1) % every == 0:
            rn.tier_rebalance(p, ts)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2), f"out, step {step}"
        for i in range(4):
            assert torch.equal(a1[i], a2[i]), f"addresses {i}, step {step}"
        assert torch.equal(m_plain, m_tier), f"mass, step {step}"
        pos += 1
    # the cache holds rows: at most `lines` slots per unit, maps consistent
    ls, sl = to_np(ts.line_slot), to_np(ts.slot_line)
    assert (ls >= 0).any()
    for u in np.ndindex(B, H):
        held = ls[u][ls[u] >= 0]
        assert len(set(held.tolist())) == len(held)
        assert (sl[u][held] == np.nonzero(ls[u] >= 0)[0]).all()
        assert (sl[u] >= 0).sum() == len(held)
    cached_rows = to_np(ts.cache)
    rn.tier_flush(p, ts)
    torch.cuda.synchronize()
    assert torch.equal(ts.S_host, S.cpu()), "final state"
    # a cached line equals its slot's row
    for u in list(np.ndindex(B, H))[:8]:
        for ln in np.nonzero(ls[u] >= 0)[0]:
            assert np.array_equal(cached_rows[u][ln], to_np(S[u][int(ls[u][ln])]))


def expected_cache(hits, cached, C):
    """The rule of ramnet_tier_rebalance, for one unit: key = 2 hits +
    cached, capped at 255; the C largest keys, ties to the smaller slot; key
    0 never."""
    key = np.minimum(2 * np.minimum(hits.astype(np.int64), 1 << 20) + cached, 255)
    order = np.lexsort((np.arange(len(key)), -key))   # key desc, slot asc
    chosen = [int(s) for s in order[:C] if key[s] > 0]
    return set(chosen)


def test_rebalance_policy(rn):
    """After a few steps with no rebalance, then after a second round: the
    cached set is the rule's choice on the counts it started from, slots that
    stay keep their line, entering slots take the free lines in line order
    (in slot order), the counts are halved."""
    w = synth.WORKLOADS["decode"].replace(K=16, U=4)      # 256 slots: many repeats
    B, H, lines = 4, w.H, 40
    init = synth.make_inputs(w, B=B, T=1)
    S = dev(init["S0"], "bf16")
    m = dev(init["m0"], "f32")
    p = rn.make_params(B, 1, H, w.d_p, w.U, w.K, w.d_v, rn.BF16, rn.BF16, cape=w.cape)
    ts = rn.TieredState(S, lines)
    rn.tier_reset(p, ts)
    out = torch.empty((B, H, w.d_v), dtype=torch.bfloat16, device="cuda")
    pos = torch.from_numpy(init["pos0"]).cuda()
    step = 0
    for rnd in range(3):
        for _ in range(5):
            s = synth.make_decode_step(w, step, B=B)
            rn.step_decode_tiered(p, *[dev(s[n], "bf16") for n in ("q", "k", "v", "gamma", "g")],
                                  pos, ts, m, out)
            pos += 1
            step += 1
        torch.cuda.synchronize()
        hits = to_np(ts.hits).astype(np.int64)
        sl0, ls0 = to_np(ts.slot_line).copy(), to_np(ts.line_slot).copy()
        rn.tier_rebalance(p, ts)
        torch.cuda.synchronize()
        sl1, ls1 = to_np(ts.slot_line), to_np(ts.line_slot)
        for u in np.ndindex(B, H):
            want = expected_cache(hits[u], (sl0[u] >= 0).astype(np.int64), lines)
            got = set(int(x) for x in ls1[u] if x >= 0)
            assert got == want, (rnd, u)
            # staying slots keep their line
            for sl in want & set(int(x) for x in ls0[u] if x >= 0):
                assert sl1[u][sl] == sl0[u][sl]
            # entering slots, in slot order, take the free lines in line order
            entering = sorted(want - set(int(x) for x in ls0[u] if x >= 0))
            free = [ln for ln in range(lines) if ls0[u][ln] < 0 or int(ls0[u][ln]) not in want]
            assert [int(sl1[u][s_]) for s_ in entering] == free[:len(entering)]
        assert (to_np(ts.hits).astype(np.int64) == hits // 2).all()
