"""Dense steps either side of the RAM-Net layer, for the layer-forward tests.
TEST INFRASTRUCTURE ONLY: plain numpy in fp64, no blocking or fusion.

Follows two passages: the project page's outline of a layer (the token is
projected to key, query and value; the GSU's gamma comes "from the current
token by a learned projection" in its Gated Sparse Update section; the gated
read is projected out), and the AI Radio page's remark that the address weights
are re-parameterised as W = e^alpha * W' with one learned alpha per head,
which sets the temperature of the Product Softmax.

Readings fixed here (the pages give no formulas for these steps):
  * the five input projections are plain products x W with row-major
    [d_model, n] bf16 weights, each result rounded to bf16 (the layer's
    input dtype); the column order of q and k is (head, block, digit), of v
    and g (head, channel), of gamma (head);
  * the re-parameterisation applies to the key and query weights: the
    columns of head h are W = bf16(t_h * W') with t_h = fp32(e^alpha_h),
    rounded once from the exact product;
  * the layer output is rounded to bf16 and projected with W_o
    [H*d_v, d_model], the product rounded to bf16.
"""
from __future__ import annotations

import math

import numpy as np

from . import oracle as _o


def to_bf16(x) -> np.ndarray:
    """Nearest bf16 (8 significant bits, ties to even) of finite fp64 values
    in the normal range, returned as float32."""
    x = np.asarray(x, np.float64)
    m, e = np.frexp(x)                       # x = m * 2^e, 0.5 <= |m| < 1
    return np.ldexp(np.rint(m * 256.0) / 256.0, e).astype(np.float32)


def temperatures(alpha, H: int) -> np.ndarray:
    """t_h = e^alpha_h as fp32 (alpha None: all ones)."""
    if alpha is None:
        return np.ones(H, np.float32)
    a = np.asarray(alpha, np.float32).reshape(H)
    return np.array([math.exp(float(v)) for v in a], np.float64).astype(np.float32)


def address_weights(Wp, alpha, H: int, L: int) -> np.ndarray:
    """W = bf16(t_h * W') for the q or k weights [d_model, H*L]."""
    Wp = np.asarray(Wp, np.float64)
    t = temperatures(alpha, H).astype(np.float64)
    return to_bf16(Wp * np.repeat(t, L)[None, :])


def project(x, W) -> np.ndarray:
    """bf16(x W) for x [..., d_model]."""
    x = np.asarray(x, np.float64)
    return to_bf16(x @ np.asarray(W, np.float64))


def project_inputs(x, Wq, Wk, Wv, Wg, Wgamma, alpha, *, H: int, L: int, d_v: int):
    """x [B,T,D] -> dict q, k [B,T,H,L], v, g [B,T,H,d_v], gamma [B,T,H]."""
    B, T, _ = np.shape(x)
    q = project(x, address_weights(Wq, alpha, H, L)).reshape(B, T, H, L)
    k = project(x, address_weights(Wk, alpha, H, L)).reshape(B, T, H, L)
    v = project(x, Wv).reshape(B, T, H, d_v)
    g = project(x, Wg).reshape(B, T, H, d_v)
    gamma = project(x, Wgamma).reshape(B, T, H)
    return {"q": q, "k": k, "v": v, "g": g, "gamma": gamma}


def layer_forward(x, Wq, Wk, Wv, Wg, Wgamma, Wo, alpha, S, mass, *, H: int,
                  d_p: int, U: int, K: int, state_bf16: bool, cape: int = 1,
                  pos0=None, norm_w=None, eps_gsu=1e-6, eps_norm=1e-6,
                  content_heads: int = 0):
    """x [B,T,D] -> y [B,T,D]; S [B,H,M,d_v] and mass [B,H,M] updated in
    place.  Returns (y, res): res is the oracle layer's result (addresses,
    gaps, out) plus the projected inputs under res["inputs"]."""
    B, T, _ = np.shape(x)
    d_v = np.shape(Wv)[1] // H
    inp = project_inputs(x, Wq, Wk, Wv, Wg, Wgamma, alpha, H=H, L=U * d_p, d_v=d_v)
    res = _o.layer(inp["q"], inp["k"], inp["v"], inp["gamma"], inp["g"], S,
                   mass, d_p=d_p, U=U, K=K, state_bf16=state_bf16, cape=cape,
                   eps_gsu=eps_gsu, eps_norm=eps_norm, norm_w=norm_w,
                   pos0=pos0, content_heads=content_heads)
    out = to_bf16(res["out"]).reshape(B, T, H * d_v)
    res["inputs"] = inp
    return project(out, Wo), res
