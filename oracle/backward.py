"""Gradients of the RAM-Net layer recurrence, for the backward-pass tests.
TEST INFRASTRUCTURE ONLY: plain PyTorch on the CPU in fp64, with autograd
through a token-by-token loop (no blocking, fusion or reordering).

The forward steps are the same as the C oracle's (project page, Product
Softmax and exact Top-K for the weights, CAPE on indices, Gated Sparse Update
in write order, read after the writes, RMSNorm and sigmoid gate), written
again here in torch so that autograd can differentiate them:

  w_k   = prod_u softmax(l_u)[a_u(k)]        the content slot's digits a_u(k)
  alpha = (1 - w)^(e^gamma)                  (0 when w >= 1)
  m_i  <- alpha m_i + w,   lam = w / (m_i + eps_gsu)
  S_i  <- S_i + lam (v - S_i)
  r     = sum_k rho_k S_{j_k}
  out   = r / sqrt(mean(r^2) + eps_norm) * omega * sigmoid(g)

Readings fixed here (the pages do not define the backward pass):
  * the Top-K selection is held fixed (it is piecewise constant in the
    logits); gradients reach the logits only through the selected weights;
  * the power-decay retention is differentiated exactly.  The AI Radio page
    mentions a proxy gradient for it but does not give one ("parity
    unpinned" for that proxy, which is not implemented);
  * with round_storage, each stored state row is rounded to its storage
    dtype (bf16 or fp32) and each mass to fp32 after every write, as the C
    oracle's forward does, and a rounding step passes its gradient through
    unchanged; without it the forward is plain fp64 (smooth, for finite
    differences).

The loss whose gradients are returned is
  sum(out * dout) + sum(S_final * dS_final) + sum(m_final * dm_final).
"""
from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from . import oracle as _o


def content_indices(post_idx, pos, U: int, d_p: int, form: int) -> np.ndarray:
    """Pre-CAPE (content) slots of post-CAPE slots at position pos."""
    if form == 0:
        return np.asarray(post_idx, np.int64)
    M = d_p ** U
    perm = _o.cape(np.arange(M, dtype=np.int32), int(pos), U, d_p, form)
    inv = np.empty(M, np.int64)
    inv[perm] = np.arange(M)
    return inv[np.asarray(post_idx, np.int64)]


def slot_weights(logits, content, U: int, d_p: int):
    """Product Softmax weights of the given content slots (differentiable):
    logits [U*d_p], content int [K] -> [K]."""
    p = torch.softmax(logits.view(U, d_p), dim=-1)
    w = torch.ones(len(content), dtype=logits.dtype)
    for u in range(U):
        digit = torch.as_tensor((np.asarray(content) // d_p ** (U - 1 - u)) % d_p)
        w = w * p[u, digit]
    return w


def _round_bf16(x: np.ndarray) -> np.ndarray:
    m, e = np.frexp(x)
    return np.ldexp(np.rint(m * 256.0) / 256.0, e)


def stored(x, bf16: bool):
    """x rounded to bf16 or fp32 in the forward, gradient passed through."""
    v = x.detach().numpy()
    r = _round_bf16(v) if bf16 else v.astype(np.float32).astype(np.float64)
    return x + torch.as_tensor(r - v)


def retention(w, e):
    """(1 - w)^e, 0 for w >= 1 (where the factor reaches 0)."""
    if float(w.detach()) >= 1.0:
        return torch.zeros((), dtype=w.dtype)
    return torch.exp(e * torch.log1p(-w))


def layer_grads(q, k, v, gamma, g, S0, m0, dout, *, d_p: int, U: int, K: int,
                cape: int = 1, pos0=None, norm_w=None, eps_gsu: float = 1e-6,
                eps_norm: float = 1e-6, content_heads: int = 0, dS_final=None,
                dm_final=None, round_storage: bool = False, state_bf16: bool = False,
                addresses=None):
    """Inputs as for oracle.layer (q, k [B,T,H,U*d_p], v, g [B,T,H,d_v],
    gamma [B,T,H], S0 [B,H,M,d_v], m0 [B,H,M]) plus dout [B,T,H,d_v].
    Returns a dict of fp64 numpy arrays: out, S, mass (the forward), the
    addresses used (w_idx, r_idx post-CAPE, and the oracle's gaps), and the
    gradients dq, dk, dv, dgamma, dg, dS0, dm0, dnorm_w.

    addresses: None (the exact Top-K of the logits), or given post-CAPE write
    and read slots (w_idx, r_idx), [B,T,H,K] each, as the backward entry
    point takes them; their weights are still the Product Softmax weights of
    the slots' content digits, and the gaps returned are then +inf."""
    q, k, v, gamma, g = (np.asarray(x, np.float64) for x in (q, k, v, gamma, g))
    B, T, H, L = q.shape
    d_v = v.shape[-1]
    M = d_p ** U
    pos0 = np.zeros(B, np.int64) if pos0 is None else np.asarray(pos0, np.int64)
    # The addresses: the C oracle's exact Top-K, post-CAPE
    w_idx, _, w_gap = _o.decode_all(k.astype(np.float32), U, d_p, K, cape=cape,
                                    pos0=pos0.astype(np.int32), content_heads=content_heads)
    r_idx, _, r_gap = _o.decode_all(q.astype(np.float32), U, d_p, K, cape=cape,
                                    pos0=pos0.astype(np.int32), content_heads=content_heads)
    if addresses is not None:
        w_idx, r_idx = (np.asarray(a, np.int32) for a in addresses)
        w_gap = np.full(w_idx.shape[:3], np.inf)
        r_gap = np.full(r_idx.shape[:3], np.inf)

    leaf = lambda a: torch.tensor(np.asarray(a, np.float64), requires_grad=True)
    tq, tk, tv, tgam, tg = leaf(q), leaf(k), leaf(v), leaf(gamma), leaf(g)
    tS0, tm0 = leaf(S0), leaf(m0)
    tom = leaf(np.ones(d_v) if norm_w is None else norm_w)
    outs = []
    S_fin = []
    m_fin = []
    for b in range(B):
        for h in range(H):
            form = 0 if (content_heads >> min(h, 63)) & 1 else cape
            # the rows and masses the unit has written so far, by slot; every
            # other slot still holds its starting value
            base_rows, base_mass = tS0[b, h].unbind(0), tm0[b, h].unbind(0)
            rows, mass = {}, {}
            row_of = lambda i: rows[i] if i in rows else base_rows[i]
            mass_of = lambda i: mass[i] if i in mass else base_mass[i]
            unit_out = []
            for t in range(T):
                P = int(pos0[b]) + t
                wi = w_idx[b, t, h]
                ri = r_idx[b, t, h]
                ww = slot_weights(tk[b, t, h], content_indices(wi, P, U, d_p, form), U, d_p)
                rw = slot_weights(tq[b, t, h], content_indices(ri, P, U, d_p, form), U, d_p)
                e = torch.exp(tgam[b, t, h])
                for j in range(K):
                    w = ww[j]
                    if not float(w.detach()) > 0.0:
                        continue
                    i = int(wi[j])
                    mass[i] = retention(w, e) * mass_of(i) + w
                    if round_storage:
                        mass[i] = stored(mass[i], False)
                    lam = w / (mass[i] + eps_gsu)
                    rows[i] = row_of(i) + lam * (tv[b, t, h] - row_of(i))
                    if round_storage:
                        rows[i] = stored(rows[i], state_bf16)
                r = sum(rw[j] * row_of(int(ri[j])) for j in range(K))
                inv = torch.rsqrt(torch.mean(r * r) + eps_norm)
                unit_out.append(r * inv * tom * torch.sigmoid(tg[b, t, h]))
            outs.append(torch.stack(unit_out))
            # the final state: the starting one with the written slots replaced
            ws = sorted(rows)
            if ws:
                sel = torch.as_tensor(ws, dtype=torch.int64)
                S_fin.append(tS0[b, h].index_put((sel,), torch.stack([rows[i] for i in ws])))
                m_fin.append(tm0[b, h].index_put((sel,), torch.stack([mass[i] for i in ws])))
            else:
                S_fin.append(tS0[b, h] * 1.0)
                m_fin.append(tm0[b, h] * 1.0)
    out = torch.stack(outs).view(B, H, T, d_v).permute(0, 2, 1, 3)
    S_f = torch.stack(S_fin).view(B, H, M, d_v)
    m_f = torch.stack(m_fin).view(B, H, M)
    loss = (out * torch.as_tensor(np.asarray(dout, np.float64))).sum()
    if dS_final is not None:
        loss = loss + (S_f * torch.as_tensor(np.asarray(dS_final, np.float64))).sum()
    if dm_final is not None:
        loss = loss + (m_f * torch.as_tensor(np.asarray(dm_final, np.float64))).sum()
    loss.backward()
    z = lambda t: np.zeros(t.shape) if t.grad is None else t.grad.numpy()
    return {
        "out": out.detach().numpy(), "S": S_f.detach().numpy(), "mass": m_f.detach().numpy(),
        "loss": float(loss.detach()), "w_idx": w_idx, "r_idx": r_idx, "w_gap": w_gap, "r_gap": r_gap,
        "dq": z(tq), "dk": z(tk), "dv": z(tv), "dgamma": z(tgam), "dg": z(tg),
        "dS0": z(tS0), "dm0": z(tm0), "dnorm_w": z(tom),
    }
