"""C ABI checks that run without a GPU: the library loads, exports every
entry point include/ramnet.h declares, and rejects bad arguments on the host
before anything is enqueued (no call here reaches the HIP runtime)."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ramnet.h")


@pytest.fixture(scope="module")
def rn():
    from sparse_slot_recurrent_amd import ramnet
    if not os.path.exists(ramnet.LIB_PATH):
        from sparse_slot_recurrent_amd import build
        build.build()
    ramnet.load_library()
    return ramnet


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ramnet_[a-z_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("ramnet_decode_addresses", "ramnet_scan_prefill",
              "ramnet_step_decode", "ramnet_workspace_bytes"):
        assert n in names


def test_library_exports_every_declared_symbol(rn):
    lib = rn.load_library()
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} not exported"
    assert set(declared_functions()) == set(rn.EXPORTED)


def test_version_and_status_strings(rn):
    lib = rn.load_library()
    assert lib.ramnet_version() == 6
    for code in (0, -1, -2, -3, -4):
        assert lib.ramnet_status_str(code).decode() != "unknown status"


def good(rn, **kw):
    base = dict(B=2, T=8, H=2, d_p=4, U=5, K=8, d_v=64, in_dtype=rn.BF16,
                state_dtype=rn.F32, cape=1)
    base.update(kw)
    return rn.make_params(**base)


FAKE = 1 << 40  # aligned, never dereferenced: validation fails first


def call_prefill(rn, p, q=FAKE, k=FAKE + (1 << 32), v=FAKE + (2 << 32),
                 gamma=FAKE + (3 << 32), g=FAKE + (4 << 32), S=FAKE + (5 << 32),
                 mass=FAKE + (6 << 32), out=FAKE + (7 << 32), ws=None,
                 ws_bytes=0, addr_in=None, norm_w=None, pos0=None):
    lib = rn.load_library()
    P = lambda x: None if x is None else C.c_void_p(x)
    st = lib.ramnet_scan_prefill(C.byref(p), P(q), P(k), P(v), P(gamma), P(g),
                                 P(norm_w), P(pos0), P(S), P(mass), P(out),
                                 addr_in, None, P(ws), ws_bytes, None)
    return st, lib.ramnet_last_error().decode()


@pytest.mark.parametrize("field,value,code,msg", [
    ("M", 1000, -1, "d_p^U"),
    ("K", 0, -1, "K"),
    ("K", 2000, -1, "K"),
    ("d_p", 1, -1, "d_p"),
    ("U", 0, -1, "U"),
    ("B", -1, -1, ">= 0"),
    ("in_dtype", 7, -1, "in_dtype"),
    ("state_dtype", 3, -1, "state_dtype"),
    ("cape", 4, -1, "cape"),
    ("cape", -1, -1, "cape"),
    ("eps_gsu", -1.0, -1, "eps"),
    ("eps_norm", float("nan"), -1, "eps"),
    ("d_v", 96, -2, "d_v"),
    ("d_v", 512, -2, "d_v"),
])
def test_bad_params_rejected(rn, field, value, code, msg):
    p = good(rn)
    setattr(p, field, value)
    st, err = call_prefill(rn, p)
    assert st == code, err
    assert msg in err


def test_unsupported_k_and_dp(rn):
    p = good(rn, d_p=2, U=10, K=65)
    st, err = call_prefill(rn, p)
    assert st == -2 and "KMAX" in err
    p = good(rn, d_p=16, U=2, K=8)
    st, err = call_prefill(rn, p)
    assert st == -2 and "d_p" in err


def test_slot_count_limit(rn):
    p = good(rn, d_p=2, U=31, K=8)
    st, err = call_prefill(rn, p)
    assert st == -1 and "2^30" in err


def test_null_and_misaligned_pointers(rn):
    p = good(rn)
    st, err = call_prefill(rn, p, v=None)
    assert st == -1 and "v is NULL" in err
    st, err = call_prefill(rn, p, S=FAKE + (5 << 32) + 4)
    assert st == -1 and "S is not 16-byte aligned" in err


def test_workspace_required_and_sized(rn):
    p = good(rn)
    need = rn.workspace_bytes(p, rn.OP_PREFILL)
    n = 2 * 8 * 2
    assert need >= 4 * n * 8 * 4
    st, err = call_prefill(rn, p)
    assert st == -3 and "workspace" in err
    st, err = call_prefill(rn, p, ws=FAKE + (9 << 32), ws_bytes=need - 1)
    assert st == -3
    assert rn.workspace_bytes(p, rn.OP_DECODE) == 0
    bad = good(rn, K=0)
    assert rn.workspace_bytes(bad, rn.OP_PREFILL) == 0


def test_overlapping_output_rejected(rn):
    p = good(rn)
    need = rn.workspace_bytes(p, rn.OP_PREFILL)
    st, err = call_prefill(rn, p, out=FAKE + (5 << 32) + 4096,
                           ws=FAKE + (9 << 32), ws_bytes=need)
    assert st == -1 and "overlaps" in err
    st, err = call_prefill(rn, p, mass=FAKE, ws=FAKE + (9 << 32), ws_bytes=need)
    assert st == -1 and "overlaps" in err


def test_empty_inputs_are_a_no_op(rn):
    for kw in (dict(T=0), dict(B=0), dict(H=0)):
        p = good(rn, **kw)
        st, err = call_prefill(rn, p, q=None, k=None, v=None, gamma=None,
                               g=None, S=None, mass=None, out=None)
        assert st == 0, err
    lib = rn.load_library()
    p = good(rn, T=0)
    out = rn.Addr(None, None, None, None)
    assert lib.ramnet_decode_addresses(C.byref(p), None, None, None,
                                       C.byref(out), None) == 0


def test_step_requires_t1_and_pos(rn):
    lib = rn.load_library()
    p = good(rn, T=2)
    P = C.c_void_p
    st = lib.ramnet_step_decode(C.byref(p), *[P(FAKE + (i << 32)) for i in range(5)],
                                None, None, *[P(FAKE + ((5 + i) << 32)) for i in range(3)],
                                None, None, 0, None)
    assert st == -1 and "T == 1" in lib.ramnet_last_error().decode()
    p = good(rn, T=1)
    st = lib.ramnet_step_decode(C.byref(p), *[P(FAKE + (i << 32)) for i in range(5)],
                                None, None, *[P(FAKE + ((5 + i) << 32)) for i in range(3)],
                                None, None, 0, None)
    assert st == -1 and "pos is required" in lib.ramnet_last_error().decode()


def test_product_path_has_no_cpu_fallback():
    """The binding must not import or load the oracle, and must raise when
    the HIP library is missing."""
    src = open(os.path.join(ROOT, "sparse_slot_recurrent_amd", "ramnet.py")).read()
    assert "oracle" not in src
    import importlib
    from sparse_slot_recurrent_amd import ramnet
    mod = importlib.reload(ramnet)
    with pytest.raises(RuntimeError, match="missing"):
        mod._lib = None
        mod.load_library(os.path.join(ROOT, "does_not_exist.so"))


def call_forward(rn, p, d_model=256, ws_bytes=None, **kw):
    lib = rn.load_library()
    w = rn.Proj(d_model, *[FAKE + ((20 + i) << 32) for i in range(6)], None, None)
    for k, v in kw.items():
        setattr(w, k, v)
    need = rn.layer_workspace_bytes(p, d_model)
    ws = FAKE + (40 << 32)
    st = lib.ramnet_layer_forward(C.byref(p), C.byref(w), C.c_void_p(FAKE),
                                  None, None, C.c_void_p(FAKE + (5 << 32)),
                                  C.c_void_p(FAKE + (6 << 32)),
                                  C.c_void_p(FAKE + (7 << 32)), None,
                                  C.c_void_p(ws), need if ws_bytes is None else ws_bytes,
                                  None)
    return st, lib.ramnet_last_error().decode()


def test_layer_workspace_query(rn):
    p = good(rn)
    big = rn.layer_workspace_bytes(p, 1024)
    assert big > rn.layer_workspace_bytes(p, 256) > rn.workspace_bytes(p, rn.OP_PREFILL)
    assert rn.layer_workspace_bytes(p, 12) == 0           # not a multiple of 8
    assert rn.layer_workspace_bytes(good(rn, in_dtype=rn.F32), 256) == 0
    step = good(rn, T=1)
    assert rn.layer_workspace_bytes(step, 256) > 0


@pytest.mark.parametrize("kw,code,msg", [
    (dict(d_model=12), -1, "d_model"),
    (dict(d_model=0), -1, "d_model"),
    (dict(w_o=None), -1, "w_o is NULL"),
    (dict(w_q=FAKE + 8), -1, "w_q is not 16-byte aligned"),
    (dict(ws_bytes=1000), -3, "workspace"),
])
def test_layer_forward_bad_arguments(rn, kw, code, msg):
    p = good(rn)
    st, err = call_forward(rn, p, **kw)
    assert st == code, err
    assert msg in err


def test_layer_forward_needs_bf16_inputs(rn):
    st, err = call_forward(rn, good(rn, in_dtype=rn.F32))
    assert st == -2 and "in_dtype" in err


def test_layer_forward_rejects_overlaps(rn):
    p = good(rn)
    # y on top of a weight
    lib = rn.load_library()
    w = rn.Proj(256, *[FAKE + ((20 + i) << 32) for i in range(6)], None, None)
    need = rn.layer_workspace_bytes(p, 256)
    st = lib.ramnet_layer_forward(C.byref(p), C.byref(w), C.c_void_p(FAKE), None, None,
                                  C.c_void_p(FAKE + (5 << 32)), C.c_void_p(FAKE + (6 << 32)),
                                  C.c_void_p(FAKE + (21 << 32) + 256), None,
                                  C.c_void_p(FAKE + (40 << 32)), need, None)
    assert st == -1 and "overlaps" in lib.ramnet_last_error().decode()


def test_packed_weights_size(rn):
    # H = 2, U*d_p = 20, d_v = 64: q at 0, k at 40, v at 80, g at 208,
    # gamma at 336, N = 344 (blocks start at multiples of 8 columns)
    p = good(rn)
    lib = rn.load_library()
    assert lib.ramnet_packed_weights_bytes(C.byref(p), 256) == 256 * 344 * 2
    assert lib.ramnet_packed_weights_bytes(C.byref(p), 100) == 0


def test_pack_rejects_short_buffer(rn):
    p = good(rn)
    lib = rn.load_library()
    w = rn.Proj(256, *[FAKE + ((20 + i) << 32) for i in range(6)], None, None)
    st = lib.ramnet_pack_weights(C.byref(p), C.byref(w), C.c_void_p(FAKE + (40 << 32)),
                                 1000, None)
    assert st == -1 and "packed needs" in lib.ramnet_last_error().decode()


def call_backward(rn, p, **kw):
    lib = rn.load_library()
    ptrs = {n: C.c_void_p(FAKE + ((50 + i) << 32)) for i, n in enumerate(
        ["q", "k", "v", "gamma", "g", "S0", "mass0", "dout", "dv", "dgamma", "dg",
         "dS0", "dmass0", "ws"])}
    for n, v in kw.items():
        ptrs[n] = None if v is None else C.c_void_p(v)
    a = rn.Addr(*[FAKE + ((80 + i) << 32) for i in range(4)])
    need = rn.workspace_bytes(p, rn.OP_BACKWARD)
    st = lib.ramnet_scan_backward(C.byref(p), ptrs["q"], ptrs["k"], ptrs["v"], ptrs["gamma"],
                                  ptrs["g"], None, None, ptrs["S0"], ptrs["mass0"], C.byref(a),
                                  ptrs["dout"], None, None, None, None, ptrs["dv"],
                                  ptrs["dgamma"], ptrs["dg"], None, ptrs["dS0"], ptrs["dmass0"],
                                  ptrs["ws"], kw.get("ws_bytes", need), None)
    return st, lib.ramnet_last_error().decode()


def test_backward_scope_and_arguments(rn):
    p = good(rn, d_v=64, state_dtype=rn.F32)
    assert rn.workspace_bytes(p, rn.OP_BACKWARD) > 0
    assert rn.workspace_bytes(good(rn, state_dtype=rn.BF16), rn.OP_BACKWARD) > 0
    # any d_v and M: d_v 64 with M <= 1024 keeps the state on chip, other
    # shapes walk the tokens with a copy of the state in the workspace
    dv128 = rn.workspace_bytes(good(rn, d_v=128, state_dtype=rn.BF16), rn.OP_BACKWARD)
    p4k = good(rn, d_p=4, U=6, state_dtype=rn.BF16)   # M = 4096
    walk = rn.workspace_bytes(p4k, rn.OP_BACKWARD)
    assert dv128 > 0 and walk > 0
    units = p4k.B * p4k.H
    base = rn.workspace_bytes(good(rn, state_dtype=rn.BF16), rn.OP_BACKWARD)
    assert walk >= base + units * 4096 * (p4k.d_v * 2 + 4)   # state and mass copies
    st, err = call_backward(rn, good(rn, d_p=6, U=11))   # U * d_p = 66 logits
    assert st == -2 and "U*d_p <= 64" in err
    st, err = call_backward(rn, p, dout=None)
    assert st == -1 and "dout is NULL" in err
    st, err = call_backward(rn, p, ws_bytes=16)
    assert st == -3 and "workspace" in err
    st, err = call_backward(rn, p, dv=FAKE + ((50 + 7) << 32))   # dv on dout
    assert st == -1 and "overlaps" in err


def test_binding_rejects_host_tensors(rn):
    """The binding checks every tensor before a pointer reaches the C ABI:
    a host tensor is refused (with a GPU, shapes and dtypes are checked too;
    see the GPU parity tests)."""
    import torch
    with pytest.raises(ValueError, match="must live on the GPU"):
        rn._arg(torch.zeros(4), "x", (4,), torch.float32)
    with pytest.raises(ValueError, match="is required"):
        rn._arg(None, "x", (4,), torch.float32)
    assert rn._arg(None, "x", (4,), torch.float32, required=False) is None


def test_tiered_state_arguments(rn):
    """Host-side checks of the tiered-state calls: the cache size, NULL
    buffers, overlaps and the fused step's shapes (nothing is launched)."""
    lib = rn.load_library()
    p = good(rn, T=1, K=16, d_v=128, state_dtype=rn.BF16)
    M = p.M
    units = p.B * p.H

    def ts(**kw):
        base = dict(S_host=FAKE, cache=FAKE + (1 << 32), line_slot=FAKE + (2 << 32),
                    slot_line=FAKE + (3 << 32), hits=FAKE + (4 << 32), C=64)
        base.update(kw)
        return rn.TieredStateC(**base)

    for C_ in (0, -1, M + 1):
        st = lib.ramnet_tier_rebalance(C.byref(p), C.byref(ts(C=C_)), None)
        assert st == -1 and "outside" in lib.ramnet_last_error().decode()
    assert lib.ramnet_tier_flush(C.byref(p), C.byref(ts(hits=None)), None) == -1
    assert "ts->hits is NULL" in lib.ramnet_last_error().decode()
    assert lib.ramnet_tier_reset(C.byref(p), None, None) == -1
    # the cache on top of the host rows
    st = lib.ramnet_tier_reset(C.byref(p), C.byref(ts(cache=FAKE + units * M * 64)), None)
    assert st == -1 and "overlaps" in lib.ramnet_last_error().decode()
    x = [C.c_void_p(FAKE + ((10 + i) << 32)) for i in range(10)]
    st = lib.ramnet_step_decode_tiered(C.byref(good(rn, T=1, K=40)), *x[:7], C.byref(ts()),
                                       x[7], x[8], None, None)
    assert st == -2 and "fused step" in lib.ramnet_last_error().decode()
    st = lib.ramnet_step_decode_tiered(C.byref(p), *x[:7], C.byref(ts()), x[7], None, None, None)
    assert st == -1 and "out is NULL" in lib.ramnet_last_error().decode()
    # a zero-size host allocation is refused by nothing; NULL out pointer is
    assert lib.ramnet_host_alloc(16, None) == -1
