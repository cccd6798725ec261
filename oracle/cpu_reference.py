"""A full-size CPU reference of the layer forward: NumPy float32, sorted dispatch, one
matrix product per expert.

TEST INFRASTRUCTURE, like moe_oracle: only ``tests/`` and the ``cpu_baseline`` leg of
``bench.py`` import it, and it imports nothing from the GPU package. It exists to put a
full-N CPU throughput beside the GPU's (the per-token float64 oracle takes hours at the
large shapes); tests/test_cpu_reference.py pins it to the oracle within float32 rounding.

It computes what moe_oracle.forward_sorted computes, in float32 and vectorised over tokens:
  * z = x W_g^T (+ logit offset), p = softmax(z) with the row maximum subtracted
    ("Mixture of Experts: routing, sorted dispatch, Switch aux loss, aux-free bias" (L7.8)
    §2 symbol table);
  * the top-k of the selection score (z, or sigmoid(z) + b for the sigmoid router), largest
    first, ties to the lowest id, and the gates of the L7.8 §2.1 routers table times
    routed_scaling;
  * a stable sort of the assignments by expert ([L7.8] §2.2), each expert's FFN once on its
    contiguous slice (GELU with optional biases, or SwiGLU), and the combine through the
    inverse permutation, j ascending;
  * plus the shared expert with weight 1 when present.
"""
from __future__ import annotations

import math
from typing import Any, Mapping, Optional

import numpy as np

f32 = np.float32

try:
    from scipy.special import erf as _erf
except Exception:  # pragma: no cover
    _erf = np.vectorize(math.erf, otypes=[np.float64])


def _sigmoid(z):
    e = np.exp(-np.abs(z))  # no overflow for either sign
    return np.where(z >= 0, 1.0 / (1.0 + e), e / (1.0 + e)).astype(f32)


def route_f32(x, w_g, n_experts: int, top_k: int, router: str = "softmax_topk", norm_topk: bool = True,
              routed_scaling: float = 1.0, logit_bias=None, sel_bias=None):
    """ids [N,k] (int64, largest first, ties to the lowest id) and gates [N,k] float32."""
    z = np.asarray(x, f32) @ np.asarray(w_g, f32).T
    if logit_bias is not None:
        z = z + np.asarray(logit_bias, f32)[None, :]
    s = _sigmoid(z) if router == "sigmoid" else z
    if sel_bias is not None:
        s = s + np.asarray(sel_bias, f32)[None, :]
    # a stable sort of -s keeps equal scores in id order: ties go to the lowest id
    ids = np.argsort(-s, axis=1, kind="stable")[:, :top_k]
    zt = np.take_along_axis(z, ids, axis=1)
    if router == "topk_softmax" or (router == "softmax_topk" and norm_topk):
        e = np.exp(zt - zt.max(axis=1, keepdims=True))     # p_T / sum p_T = softmax over z_T
        w = e / e.sum(axis=1, keepdims=True)
    elif router == "softmax_topk":
        m = z.max(axis=1, keepdims=True)
        w = np.exp(zt - m) / np.exp(z - m).sum(axis=1, keepdims=True)
    else:
        u = _sigmoid(zt)
        w = u / u.sum(axis=1, keepdims=True) if norm_topk else u
    return ids, (w * f32(routed_scaling)).astype(f32)


def _ffn(xr, act, w1, w2, w3=None, b1=None, b2=None):
    if act == "gelu":
        u = xr @ w1.T
        if b1 is not None:
            u = u + b1[None, :]
        h = (0.5 * u * (1.0 + _erf(u * f32(1.0 / math.sqrt(2.0))))).astype(f32)
        y = h @ w2.T
        return y + b2[None, :] if b2 is not None else y
    g = xr @ w1.T
    return ((g * _sigmoid(g)) * (xr @ w3.T)) @ w2.T


def forward_f32(x, params: Mapping[str, Any], n_experts: int, top_k: int, act: str, router: str = "softmax_topk",
                norm_topk: bool = True, routed_scaling: float = 1.0, logit_bias=None, sel_bias=None):
    """The layer forward in float32. params as for moe_oracle.forward_loop, each per-expert
    entry indexable by expert (a list of float32 arrays or a stacked array). Returns (y, ids)."""
    x = np.asarray(x, f32)
    n, d = x.shape
    ids, w = route_f32(x, params["w_g"], n_experts, top_k, router, norm_topk, routed_scaling, logit_bias, sel_bias)
    expert_of = ids.reshape(-1)
    perm = np.argsort(expert_of, kind="stable")
    offsets = np.concatenate([[0], np.cumsum(np.bincount(expert_of, minlength=n_experts))])
    x_sorted = x[perm // top_k]
    y_sorted = np.empty((perm.size, d), f32)
    get = lambda name, e: None if params.get(name) is None else params[name][e]
    for e in range(n_experts):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi > lo:
            y_sorted[lo:hi] = _ffn(x_sorted[lo:hi], act, get("w1", e), get("w2", e), get("w3", e), get("b1", e),
                                   get("b2", e))
    inv = np.empty_like(perm)
    inv[perm] = np.arange(perm.size)
    y = np.zeros((n, d), f32)
    for j in range(top_k):
        y += w[:, j:j + 1] * y_sorted[inv[np.arange(n) * top_k + j]]
    if params.get("s_w1") is not None:
        y += _ffn(x, act, params["s_w1"], params["s_w2"], params.get("s_w3"), params.get("s_b1"), params.get("s_b2"))
    return y, ids
