"""Comparison rules between the HIP path and the CPU oracle.

Top-K sets (tie-aware): where the oracle's relative margin between the K-th
and (K+1)-th weight exceeds 1e-6, the GPU's slot set must equal the oracle's
and matched weights agree within 1e-5 relative.  Where the margin is smaller,
more than one set is correct: the GPU's set must hold every slot clearly
heavier than the K-th weight and only slots within 1e-6 of it or heavier.
Where the GPU's set legitimately differs (a near-tie), the oracle's
recurrence adopts the GPU's set: it runs on the GPU's slots with its own fp64
weights of those slots, everywhere else on its own addresses.  Outputs, the
final state and the mass are then compared for every token of every unit
(project page, exact Top-K paragraph: at a tie more than one set is the Top-K;
Gated Sparse Update: the recurrence depends on the addresses only through
the chosen slots and their weights).

Values: fp32 state |d| <= 1e-6 + 1e-5 |ref| elementwise; bf16 state
|d| <= 2e-2 * max(|ref|, rms of the reference row).  For the bf16 slot state
itself (not the layer output) a difference of up to 4 bf16 ulps of the
reference is also accepted: every update is rounded to 8 significant bits,
the GPU rounds an fp32 value and the oracle an fp64 one, and once the two
differ by an ulp, later updates smaller than half an ulp leave the
difference in place.
"""
from __future__ import annotations

import numpy as np

TIE_REL = 1e-6
WT_REL = 1e-5


def to_np(t):
    import torch
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy()
    return t.cpu().numpy()


def compare_address_sets(gpu_idx, gpu_wt, ora_idx, ora_wt, ora_gap,
                         weights_of=None):
    """Compares [..., K] address tensors.  Returns a boolean [...] array that
    is True where the GPU's set differs from the oracle's (only allowed at
    near-ties).  `weights_of(flat_index, slots)` must return the oracle's
    fp64 weights of the given post-CAPE slots for address `flat_index`; it is
    needed only when a near-tie set differs."""
    gi = np.sort(gpu_idx, axis=-1)
    oi = np.sort(ora_idx, axis=-1)
    same = (gi == oi).all(-1)
    K = gpu_idx.shape[-1]
    # distinct slots per address
    assert (np.diff(gi, axis=-1) > 0).all(), "GPU address has repeated slots"
    clear = ora_gap > TIE_REL
    bad = clear & ~same
    if bad.any():
        loc = np.argwhere(bad)[:5]
        raise AssertionError(
            f"{int(bad.sum())} addresses with margin > {TIE_REL} differ from "
            f"the oracle's Top-K set, e.g. at {loc.tolist()}")
    # weights of matched sets
    m = same
    go = np.take_along_axis(gpu_wt, np.argsort(gpu_idx, -1), -1)
    oo = np.take_along_axis(ora_wt, np.argsort(ora_idx, -1), -1)
    err = np.abs(go[m] - oo[m]) / np.maximum(np.abs(oo[m]), 1e-300)
    assert err.size == 0 or err.max() <= WT_REL, f"weight rel err {err.max()}"
    differ = ~same
    if differ.any():
        assert weights_of is not None, "near-tie sets differ; need weights_of"
        flat_g = gpu_idx.reshape(-1, K)
        flat_o = ora_idx.reshape(-1, K)
        flat_ow = ora_wt.reshape(-1, K)
        for f in np.nonzero(differ.reshape(-1))[0]:
            wk = flat_ow[f].min()
            w_gpu = weights_of(int(f), flat_g[f])
            assert (w_gpu >= wk * (1 - TIE_REL)).all(), "GPU took a light slot"
            # every slot of the oracle's set that is clearly heavier than the
            # K-th weight must be in the GPU's set
            must = flat_o[f][flat_ow[f] > wk * (1 + TIE_REL)]
            assert set(must.tolist()) <= set(flat_g[f].tolist())
    return differ


def adopt(gpu_idx, ora_idx, ora_wt, differ, weights_of):
    """Oracle addresses [..., K] with the GPU's set adopted where `differ`
    (from compare_address_sets) marks a legitimate near-tie difference: those
    addresses take the GPU's slots, in the GPU's order, with the oracle's fp64
    weights of those slots (`weights_of(flat_index, slots)`).  Returns int32
    slots and fp64 weights."""
    K = ora_idx.shape[-1]
    idx = np.array(ora_idx, np.int32, copy=True)
    wt = np.array(ora_wt, np.float64, copy=True)
    fi, fw = idx.reshape(-1, K), wt.reshape(-1, K)
    fg = np.asarray(gpu_idx).reshape(-1, K)
    for f in np.nonzero(np.asarray(differ).reshape(-1))[0]:
        fi[f] = fg[f]
        fw[f] = weights_of(int(f), fg[f])
    return idx, wt


def bf16_ulp(x):
    """Spacing of bf16 numbers at |x| (8 significant bits)."""
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -126)))
    return 2.0 ** (e - 7)


def assert_close(got, ref, state_bf16: bool, what: str, mask=None,
                 slot_state: bool = False):
    """Elementwise tolerance check over the last axis as the 'row'."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite GPU values"
    if state_bf16:
        rms = np.sqrt((ref ** 2).mean(-1, keepdims=True))
        tol = 2e-2 * np.maximum(np.abs(ref), rms)
        if slot_state:
            tol = np.maximum(tol, 4 * bf16_ulp(ref))
    else:
        tol = 1e-6 + 1e-5 * np.abs(ref)
    bad = np.abs(got - ref) > tol
    if mask is not None:
        bad &= mask
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {bad.size} elements out of tolerance;"
            f" first at {i}: gpu {got[i]!r} oracle {ref[i]!r}")


def rel_err_stats(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    d = np.abs(got - ref)
    return float(d.max()), float((d / np.maximum(np.abs(ref), 1e-30)).max())
