"""fp64 oracle of the attention sub-block, x + attn(rmsnorm(x)), forward and backward.

TEST INFRASTRUCTURE ONLY (like the rest of ``oracle/``): only ``tests/`` and ``bench.py``'s
``cpu_baseline`` leg may use it.  It shares no code with the HIP library.

What is computed follows the NanoEuler README translations, section "Architecture": each block
adds attn(rmsnorm(x)) to x; RMSNorm is a pre-normalisation without bias; RoPE applies to
queries and keys; query heads share a smaller set of key/value heads.  The pages fix neither
the RMSNorm epsilon nor the packing of the QKV projection; the readings here are eps as an
argument (1e-5 in the tests) and the projection's columns ordered [q heads | k heads | v heads],
D columns per head.  The attention step is ``oracle.attn_fwd`` / ``attn_bwd`` (causal).

Shapes: x, y [B, T, C] with C = Hq D; gamma [C]; w_qkv [C, (Hq + 2 Hkv) D]; w_o [Hq D, C].
The backward is the chain rule written out step by step (matrix products from numpy).
"""
from __future__ import annotations

import numpy as np

from . import attn_bwd, attn_fwd


def _split(qkv, B, T, Hq, Hkv, D):
    """[B, T, (Hq + 2 Hkv) D] -> q [B, Hq, T, D], k, v [B, Hkv, T, D]."""
    h = qkv.reshape(B, T, Hq + 2 * Hkv, D).transpose(0, 2, 1, 3)
    return h[:, :Hq], h[:, Hq:Hq + Hkv], h[:, Hq + Hkv:]


def _merge(o):
    """[B, H, T, D] -> [B, T, H D]."""
    B, H, T, D = o.shape
    return o.transpose(0, 2, 1, 3).reshape(B, T, H * D)


def block_fwd(x, gamma, w_qkv, w_o, Hq, Hkv, D, eps=1e-5, rope_base=0.0):
    """Returns y and the saved state (xn, rstd, q, k, v, o) of the forward, float64."""
    x, gamma, w_qkv, w_o = (np.asarray(a, dtype=np.float64) for a in (x, gamma, w_qkv, w_o))
    B, T, C = x.shape
    rstd = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)   # RMSNorm
    xn = x * rstd * gamma
    q, k, v = (np.ascontiguousarray(a) for a in _split(xn @ w_qkv, B, T, Hq, Hkv, D))
    o, _ = attn_fwd(q, k, v, causal=True, rope_base=rope_base)
    y = x + _merge(o) @ w_o                                               # residual branch
    return y, dict(xn=xn, rstd=rstd, q=q, k=k, v=v, o=o)


def block_bwd(x, gamma, w_qkv, w_o, dy, Hq, Hkv, D, eps=1e-5, rope_base=0.0):
    """Returns (dx, dgamma, dw_qkv, dw_o): the gradient of sum(dy * y), float64."""
    x, gamma, w_qkv, w_o, dy = (np.asarray(a, dtype=np.float64)
                                for a in (x, gamma, w_qkv, w_o, dy))
    B, T, C = x.shape
    _, st = block_fwd(x, gamma, w_qkv, w_o, Hq, Hkv, D, eps, rope_base)
    om = _merge(st["o"])
    # y = x + om w_o
    dw_o = om.reshape(-1, om.shape[-1]).T @ dy.reshape(-1, C)
    dom = dy @ w_o.T
    do = np.ascontiguousarray(dom.reshape(B, T, Hq, D).transpose(0, 2, 1, 3))
    dq, dk, dv = attn_bwd(st["q"], st["k"], st["v"], do, causal=True, rope_base=rope_base)
    dqkv = np.concatenate([_merge(dq), _merge(dk), _merge(dv)], axis=-1)
    # qkv = xn w_qkv
    dw_qkv = st["xn"].reshape(-1, C).T @ dqkv.reshape(-1, dqkv.shape[-1])
    dxn = dqkv @ w_qkv.T
    # xn = x r gamma with r = (mean x^2 + eps)^(-1/2):  dr/dx = -x r^3 / C
    r = st["rstd"]
    dgamma = np.sum(dxn * x * r, axis=(0, 1))
    g = dxn * gamma
    dx = dy + g * r - x * (r ** 3) * np.sum(g * x, axis=-1, keepdims=True) / C
    return dx, dgamma, dw_qkv, dw_o
