"""ctypes wrapper over liboracle.so (plain C, fp64).  TEST INFRASTRUCTURE ONLY.

Each function marshals numpy arrays into the C entry points of
ramnet_oracle.c and back; no arithmetic of the method lives here.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "ramnet_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

TOPK_BRUTE = 0
TOPK_TREE = 1

_lib = None


def build(verbose: bool = False) -> str:
    """Compile ramnet_oracle.c into liboracle.so (gcc, OpenMP)."""
    cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-Wno-unused-parameter",
           "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        build()
    lib = C.CDLL(LIB)
    P = C.c_void_p
    i32, i64, f64, u64 = C.c_int, C.c_long, C.c_double, C.c_uint64
    lib.oracle_slot_weights.argtypes = [P, i32, i32, P]
    lib.oracle_digit_probs.argtypes = [P, i32, i32, P, P]
    lib.oracle_decode_one.argtypes = [P, i32, i32, i32, i32, i32, i64, P, P,
                                      P, P, P]
    lib.oracle_decode_all.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32,
                                      u64, P, P, P, P, P, i32]
    lib.oracle_cape.argtypes = [P, i64, i64, i32, i32, i32, P]
    lib.oracle_layer.argtypes = ([i32] * 7 + [i32, i32, u64, f64, f64, i32]
                                 + [P] * 16 + [i32])
    lib.oracle_scan_given.argtypes = ([i32] * 7 + [i32, f64, f64]
                                      + [P] * 11 + [i32])
    lib.oracle_round_bf16.argtypes = [f64]
    lib.oracle_round_bf16.restype = f64
    lib.oracle_max_threads.restype = i32
    _lib = lib
    return lib


def _p(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(C.c_void_p)


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what} failed with code {rc}")


def max_threads() -> int:
    return load().oracle_max_threads()


def round_bf16(x: float) -> float:
    return load().oracle_round_bf16(float(x))


def slot_weights(logits: np.ndarray, U: int, d_p: int) -> np.ndarray:
    """All M = d_p^U slot weights of one address."""
    lg = _f32(logits).reshape(-1)
    assert lg.size == U * d_p
    W = np.empty(d_p ** U, np.float64)
    _check(load().oracle_slot_weights(_p(lg), U, d_p, _p(W)), "slot_weights")
    return W


def digit_probs(logits: np.ndarray, U: int, d_p: int):
    lg = _f32(logits).reshape(-1)
    probs = np.empty(U * d_p, np.float64)
    n_exp = C.c_long(0)
    _check(load().oracle_digit_probs(_p(lg), U, d_p, _p(probs), C.byref(n_exp)),
           "digit_probs")
    return probs.reshape(U, d_p), n_exp.value


def decode_one(logits: np.ndarray, U: int, d_p: int, K: int,
               mode: int = TOPK_BRUTE, cape: int = 0, pos: int = 0):
    """One address: (idx int32[K], wt f64[K], gap, n_exp, cand_per_level)."""
    lg = _f32(logits).reshape(-1)
    idx = np.empty(K, np.int32)
    wt = np.empty(K, np.float64)
    gap = np.empty(1, np.float64)
    n_exp = C.c_long(0)
    cand = np.zeros(U, np.int64)
    _check(load().oracle_decode_one(_p(lg), U, d_p, K, mode, cape, pos,
                                    _p(idx), _p(wt), _p(gap), C.byref(n_exp),
                                    _p(cand)), "decode_one")
    return idx, wt, float(gap[0]), n_exp.value, cand


def decode_all(logits: np.ndarray, U: int, d_p: int, K: int, cape: int = 1,
               pos0: Optional[np.ndarray] = None, mode: int = TOPK_BRUTE,
               nthreads: int = 0, content_heads: int = 0):
    """Addresses of a [B,T,H,U*d_p] logit tensor: idx, wt [B,T,H,K], gap.
    cape: 0 content-only, 1/2/3 CAPE form A/B/C; heads whose bit is set in
    content_heads (bit 63 for heads >= 63) are content-only."""
    lg = _f32(logits)
    B, T, H, L = lg.shape
    assert L == U * d_p
    idx = np.empty((B, T, H, K), np.int32)
    wt = np.empty((B, T, H, K), np.float64)
    gap = np.empty((B, T, H), np.float64)
    p0 = None if pos0 is None else np.ascontiguousarray(pos0, dtype=np.int32)
    _check(load().oracle_decode_all(B, T, H, U, d_p, K, mode, cape,
                                    int(content_heads), _p(p0),
                                    _p(lg), _p(idx), _p(wt), _p(gap),
                                    nthreads), "decode_all")
    return idx, wt, gap


def cape(idx: np.ndarray, pos: int, U: int, d_p: int, form: int = 1) -> np.ndarray:
    """Slots moved by CAPE form 1 (A), 2 (B) or 3 (C) at position pos."""
    a = np.ascontiguousarray(idx, dtype=np.int32)
    out = np.empty_like(a)
    _check(load().oracle_cape(_p(a), a.size, int(pos), U, d_p, form, _p(out)), "cape")
    return out


def layer(q, k, v, gamma, g, S, mass, *, d_p: int, U: int, K: int,
          state_bf16: bool, cape: int = 1, eps_gsu: float = 1e-6,
          eps_norm: float = 1e-6, norm_w=None, pos0=None,
          mode: int = TOPK_BRUTE, want_addresses: bool = True,
          nthreads: int = 0, content_heads: int = 0):
    """Runs the layer over [B,T,H].  S [B,H,M,d_v] and mass [B,H,M] are
    float32 arrays updated IN PLACE (their values must be representable in
    the storage dtype).  Returns dict(out, w_idx, w_wt, r_idx, r_wt, w_gap,
    r_gap)."""
    q, k, v, gamma, g = (_f32(x) for x in (q, k, v, gamma, g))
    B, T, H, L = q.shape
    d_v = v.shape[-1]
    assert L == U * d_p and k.shape == q.shape
    assert v.shape == (B, T, H, d_v) and g.shape == v.shape
    assert gamma.shape == (B, T, H)
    M = d_p ** U
    assert S.shape == (B, H, M, d_v) and S.dtype == np.float32
    assert mass.shape == (B, H, M) and mass.dtype == np.float32
    assert S.flags["C_CONTIGUOUS"] and mass.flags["C_CONTIGUOUS"]
    out = np.empty((B, T, H, d_v), np.float32)
    res = {"out": out}
    if want_addresses:
        for n, dt in (("w_idx", np.int32), ("w_wt", np.float64),
                      ("r_idx", np.int32), ("r_wt", np.float64)):
            res[n] = np.empty((B, T, H, K), dt)
        res["w_gap"] = np.empty((B, T, H), np.float64)
        res["r_gap"] = np.empty((B, T, H), np.float64)
    nw = None if norm_w is None else _f32(norm_w)
    p0 = None if pos0 is None else np.ascontiguousarray(pos0, dtype=np.int32)
    rc = load().oracle_layer(
        B, T, H, d_p, U, K, d_v, int(state_bf16), int(cape), int(content_heads), eps_gsu,
        eps_norm, mode, _p(q), _p(k), _p(v), _p(gamma), _p(g), _p(nw), _p(p0),
        _p(S), _p(mass), _p(out), _p(res.get("w_idx")), _p(res.get("w_wt")),
        _p(res.get("r_idx")), _p(res.get("r_wt")), _p(res.get("w_gap")),
        _p(res.get("r_gap")), nthreads)
    _check(rc, "layer")
    return res


def scan_given(w_idx, w_wt, r_idx, r_wt, v, gamma, g, S, mass, *, d_p: int,
               U: int, state_bf16: bool, eps_gsu: float = 1e-6,
               eps_norm: float = 1e-6, norm_w=None, nthreads: int = 0):
    """The recurrence with given post-CAPE addresses; S, mass in place."""
    v, gamma, g = (_f32(x) for x in (v, gamma, g))
    w_idx = np.ascontiguousarray(w_idx, dtype=np.int32)
    r_idx = np.ascontiguousarray(r_idx, dtype=np.int32)
    w_wt = np.ascontiguousarray(w_wt, dtype=np.float64)
    r_wt = np.ascontiguousarray(r_wt, dtype=np.float64)
    B, T, H, K = w_idx.shape
    d_v = v.shape[-1]
    M = d_p ** U
    assert S.shape == (B, H, M, d_v) and mass.shape == (B, H, M)
    out = np.empty((B, T, H, d_v), np.float32)
    nw = None if norm_w is None else _f32(norm_w)
    rc = load().oracle_scan_given(
        B, T, H, d_p, U, K, d_v, int(state_bf16), eps_gsu, eps_norm,
        _p(w_idx), _p(w_wt), _p(r_idx), _p(r_wt), _p(v), _p(gamma), _p(g),
        _p(nw), _p(S), _p(mass), _p(out), nthreads)
    _check(rc, "scan_given")
    return out
