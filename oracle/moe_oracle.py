"""Plain CPU oracle for the forward pass of a dropless top-k mixture-of-experts FFN layer.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` may import this module. The GPU path never imports, links or calls it,
and this module imports nothing from the GPU package: the two share no code.

Everything here is NumPy float64, evaluated per token, on exactly the values the GPU sees
(bf16 inputs are widened to float64 exactly; there is no intermediate rounding here).

Pages cited (by title, section / table / figure):
  [L7.8]   "Mixture of Experts: routing, sorted dispatch, Switch aux loss, aux-free bias"
           (openlearn course module L7.8): §2 symbol table, §2.1 routers table and output
           equation, §2.2 sorted dispatch, §2.3 load-balancing loss, §2.5 aux-free bias,
           §3 worked example, §4 interface and "Your graded tests" (the oracle recipe:
           a per-token loop in float64, top-k sorted with an explicit (score, id) key).
  [RB-15]  "15. Mixture of Experts" (RustingBrain tutorial): §15.2 routing and renormalised
           gates, "Dropless", §15.3 the z-loss, §15.4 the shared expert (shared_output).
  [GPT2-MoE] "Extending Raschka's GPT-2: an MoE trained from scratch on an RTX 3090":
           the router walk-through (Diagram 4, all experts active; Diagrams 10-12, top-k of
           one context vector), the per-expert masked loop (Diagrams 13-19), and the
           router-loss function.
  [nanoMoE] "nanoMoE: Mixture-of-Experts (MoE) LLMs from Scratch in PyTorch": the MLP and
           MLPExperts listings (nn.GELU, optional biases), "Expert Capacity" and "Computing
           the expert capacity" (capacity_dispatch), the z-loss.

Readings taken where the pages are silent or ambiguous:
  * selection for the softmax routers uses the logits z (softmax is monotone, so the chosen
    set equals "top k of p"); ties go to the lowest expert id; the k chosen experts are
    stored largest first.
  * GELU is the exact erf form (nn.GELU's default in [nanoMoE]'s listings).
  * SwiGLU is h = silu(x Wg^T) * (x Wu^T), y = h W2^T, no biases.  PARITY UNPINNED: the
    pages name SwiGLU / GatedMLP but print no formula.
  * P_e always averages p = softmax(z), with any logit offset included and without the
    sigmoid router's selection bias ([L7.8] §2 symbol table).

Pins (tests/test_oracle_pins.py): the [L7.8] §3 worked example in exact rationals, the
[GPT2-MoE] router printouts, the [RB-15] §15.2 gate example, textbook normal-CDF values for
GELU, brute-force top-k over all subsets, the L = k balance construction, collapse, counting
identities, sorted dispatch == per-token loop == [GPT2-MoE] masked loop, k = E dense mixture,
shared-weight and zero-W2 reductions, and a mutation self-check that plants each [L7.8] §5
pitfall here and requires a pin to fail.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Any, Mapping, Optional

import numpy as np

try:  # scipy's erf is a vectorised library routine; math.erf is the fallback
    from scipy.special import erf as _erf
except Exception:  # pragma: no cover
    _erf = np.vectorize(math.erf, otypes=[np.float64])

ROUTERS = ("softmax_topk", "topk_softmax", "sigmoid")
ACTS = ("gelu", "swiglu")

f64 = np.float64


@dataclass
class Spec:
    """Layer hyper-parameters, named as in [L7.8] §4 (the MoE constructor)."""

    n_experts: int
    top_k: int
    router: str = "softmax_topk"
    norm_topk: bool = True
    routed_scaling: float = 1.0
    act: str = "swiglu"

    def __post_init__(self):
        # [L7.8] §4 "What the tests check": bad top_k / router fail loudly.
        if self.router not in ROUTERS:
            raise ValueError(f"unknown router {self.router!r}")
        if self.act not in ACTS:
            raise ValueError(f"unknown act {self.act!r}")
        if not (1 <= self.top_k <= self.n_experts):
            raise ValueError(f"top_k={self.top_k} must be in [1, n_experts={self.n_experts}]")


@dataclass
class Route:
    """Routing of N tokens: ids [N,k] largest first, weights [N,k], probs p [N,E]."""

    z: np.ndarray
    p: np.ndarray
    scores: np.ndarray
    ids: np.ndarray
    w: np.ndarray
    gap: np.ndarray = field(default=None)        # s_(k) - s_(k+1), +inf when k == E
    intra_gap: np.ndarray = field(default=None)  # smallest adjacent gap inside the top k


# ----------------------------------------------------------------------------------------
# Router: [L7.8] §2 symbol table (z_n = W_g x_n, p_n = softmax(z_n)), §2.1 routers table.
# ----------------------------------------------------------------------------------------

def router_logits(x, w_g, logit_bias=None) -> np.ndarray:
    """z = x W_g^T (+ a per-expert logit offset). [L7.8] §2; [RB-15] §15.2 (bias-free
    d_model -> n_experts projection). The offset, when given, is part of the logits."""
    z = np.asarray(x, f64) @ np.asarray(w_g, f64).T
    if logit_bias is not None:
        z = z + np.asarray(logit_bias, f64)[None, :]
    return z


def softmax(z) -> np.ndarray:
    """Row softmax with the row maximum subtracted first. [L7.8] §2; [GPT2-MoE] Diagram 4."""
    z = np.asarray(z, f64)
    e = np.exp(z - z.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def sigmoid(z) -> np.ndarray:
    """Logistic function, evaluated without overflow for either sign."""
    z = np.asarray(z, f64)
    out = np.empty_like(z)
    pos = z >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-z[pos]))
    ez = np.exp(z[~pos])
    out[~pos] = ez / (1.0 + ez)
    return out


def selection_scores(z, router: str, sel_bias=None) -> np.ndarray:
    """The score the top-k is taken over ([L7.8] §2.1 "chooses by" column).

    softmax_topk / topk_softmax: the logits z (same order as p, since softmax is monotone).
    sigmoid: sigma(z) + b, where b is the aux-free bias of [L7.8] §2.5 (selection only).
    A selection bias on the softmax routers is added to z, again for selection only.
    """
    z = np.asarray(z, f64)
    s = sigmoid(z) if router == "sigmoid" else z.copy()
    if sel_bias is not None:
        s = s + np.asarray(sel_bias, f64)[None, :]
    return s


def topk_ids(scores, k: int) -> np.ndarray:
    """[N,k] ids, largest score first, ties to the lowest id ([L7.8] §2.1 and §4).

    Per token, the experts are sorted by the explicit key (-score, id), as the [L7.8] §4
    oracle recipe asks, and the first k are kept.
    """
    s = np.asarray(scores, f64)
    n, e = s.shape
    if not (1 <= k <= e):
        raise ValueError(f"top_k={k} must be in [1, {e}]")
    out = np.empty((n, k), dtype=np.int64)
    for t in range(n):
        row = s[t]
        order = sorted(range(e), key=lambda i: (-row[i], i))
        out[t] = order[:k]
    return out


def topk_gaps(scores, ids):
    """gap_n = s_(k) - s_(k+1) (+inf when k == E) and the smallest adjacent gap within the
    chosen k. They mark tokens whose choice or order a rounding difference could flip."""
    s = np.asarray(scores, f64)
    n, e = s.shape
    k = ids.shape[1]
    gap = np.full(n, np.inf)
    intra = np.full(n, np.inf)
    for t in range(n):
        chosen = s[t, ids[t]]
        if k < e:
            rest = np.delete(s[t], ids[t])
            gap[t] = chosen[-1] - rest.max()
        if k > 1:
            intra[t] = np.min(chosen[:-1] - chosen[1:])
    return gap, intra


def gate_weights(z, ids, spec: Spec) -> np.ndarray:
    """w_{n,j} for the chosen ids, by the [L7.8] §2.1 "weights" column, then x routed_scaling.

    softmax_topk: p_{n,e} over the chosen set, divided by their sum when norm_topk
                  ([RB-15] §15.2 "renormalized to sum to one").
    topk_softmax: a softmax over the chosen logits only.
    sigmoid:      sigma(z_{n,e}) of the UNBIASED logit, divided by their sum when norm_topk.
    """
    z = np.asarray(z, f64)
    n, k = ids.shape
    w = np.empty((n, k), f64)
    for t in range(n):
        zt = z[t, ids[t]]
        if spec.router == "softmax_topk":
            p = softmax(z[t][None, :])[0]
            u = p[ids[t]]
            w[t] = u / u.sum() if spec.norm_topk else u
        elif spec.router == "topk_softmax":
            w[t] = softmax(zt[None, :])[0]
        else:
            u = sigmoid(zt)
            w[t] = u / u.sum() if spec.norm_topk else u
    return w * f64(spec.routed_scaling)


def route(x, w_g, spec: Spec, logit_bias=None, sel_bias=None) -> Route:
    """Routing of every token: logits, probabilities, choice, gates and tie margins."""
    z = router_logits(x, w_g, logit_bias)
    p = softmax(z)
    s = selection_scores(z, spec.router, sel_bias)
    ids = topk_ids(s, spec.top_k)
    w = gate_weights(z, ids, spec)
    gap, intra = topk_gaps(s, ids)
    return Route(z=z, p=p, scores=s, ids=ids, w=w, gap=gap, intra_gap=intra)


# ----------------------------------------------------------------------------------------
# Experts: GELU MLP ([nanoMoE] MLP / MLPExperts listings) and SwiGLU (named in [L7.8] §4).
# ----------------------------------------------------------------------------------------

def gelu_erf(u) -> np.ndarray:
    """GELU(u) = u * Phi(u) = 0.5 u (1 + erf(u / sqrt 2)), the exact (erf) form."""
    u = np.asarray(u, f64)
    return 0.5 * u * (1.0 + _erf(u / math.sqrt(2.0)))


def silu(u) -> np.ndarray:
    """silu(u) = u * sigma(u)."""
    u = np.asarray(u, f64)
    return u * sigmoid(u)


def expert_ffn(xr, act: str, w1, w2, w3=None, b1=None, b2=None) -> np.ndarray:
    """One expert applied to rows xr [m, d]; weights in [out, in] (nn.Linear) layout.

    gelu:   y = gelu(xr W1^T + b1) W2^T + b2          (biases optional)
    swiglu: y = (silu(xr W1^T) * (xr W3^T)) W2^T       (W1 = gate, W3 = up; no biases)
    """
    xr = np.asarray(xr, f64)
    if act == "gelu":
        u = xr @ np.asarray(w1, f64).T
        if b1 is not None:
            u = u + np.asarray(b1, f64)[None, :]
        h = gelu_erf(u)
        y = h @ np.asarray(w2, f64).T
        if b2 is not None:
            y = y + np.asarray(b2, f64)[None, :]
        return y
    if act == "swiglu":
        g = xr @ np.asarray(w1, f64).T
        u = xr @ np.asarray(w3, f64).T
        return (silu(g) * u) @ np.asarray(w2, f64).T
    raise ValueError(f"unknown act {act!r}")


def _expert(params: Mapping[str, Any], e: int):
    """Expert e's weights from a params mapping whose per-expert tensors support [e]."""
    get = lambda name: None if params.get(name) is None else params[name][e]
    return dict(w1=get("w1"), w2=get("w2"), w3=get("w3"), b1=get("b1"), b2=get("b2"))


def shared_output(x, params: Mapping[str, Any], act: str):
    """Shared(x) of the [L7.8] §2.1 output equation: the shared expert(s) every token passes
    through with weight 1 ([RB-15] §15.4). S shared experts of width f are one MLP of width
    S f ([L7.8] §2.1), so params hold a single MLP: s_w1 [S f, d], s_w3 [S f, d] (swiglu),
    s_w2 [d, S f], s_b1 / s_b2 (gelu, optional). Returns 0 when there is no shared expert."""
    if params.get("s_w1") is None:
        return 0.0
    return expert_ffn(x, act, params["s_w1"], params["s_w2"], params.get("s_w3"), params.get("s_b1"),
                      params.get("s_b2"))


# ----------------------------------------------------------------------------------------
# The oracle proper: y_n = sum_{e in T_n} w_{n,e} Expert_e(x_n) + Shared(x_n)
# ([L7.8] §2.1 equation).
# ----------------------------------------------------------------------------------------

def with_choice(r: Route, ids, spec: Spec) -> Route:
    """The routing r with the chosen experts replaced by a given choice ids [N,k] (for
    instance the device's, on a token whose k-th and (k+1)-th scores are within rounding of
    each other): the gates are recomputed for that choice by the [L7.8] §2.1 routers table,
    from the same logits. z, p, the scores and the tie margins (which describe the scores,
    not a choice) are kept."""
    ids = np.asarray(ids).astype(np.int64)
    if ids.shape != r.ids.shape:
        raise ValueError(f"choice shape {ids.shape} != {r.ids.shape}")
    if ids.size and (ids.min() < 0 or ids.max() >= spec.n_experts):
        raise ValueError("expert id out of range")
    return Route(z=r.z, p=r.p, scores=r.scores, ids=ids, w=gate_weights(r.z, ids, spec), gap=r.gap,
                 intra_gap=r.intra_gap)


def forward_loop(x, params: Mapping[str, Any], spec: Spec, logit_bias=None, sel_bias=None, ids=None):
    """Per-token loop over the chosen experts, j ascending ([L7.8] §4 oracle recipe).

    params: w_g [E,d]; w1 [E,d_ff,d]; w3 [E,d_ff,d] (swiglu); w2 [E,d,d_ff];
            b1 [E,d_ff], b2 [E,d] (optional, gelu only); the shared expert's s_w1, s_w3,
            s_w2, s_b1, s_b2 (optional, see shared_output).
    ids:    None (the oracle's own top-k), or a given choice [N,k] whose gates follow the
            routers table (with_choice): y_n = sum_j w_{n,j} FFN_{ids[n,j]}(x_n) + Shared(x_n),
            the [L7.8] §2.1 output equation for that choice.
    Returns (y [N,d], Route); the Route carries the choice used.
    """
    x = np.asarray(x, f64)
    r = route(x, params["w_g"], spec, logit_bias, sel_bias)
    if ids is not None:
        r = with_choice(r, ids, spec)
    n, d = x.shape
    y = np.zeros((n, d), f64)
    for t in range(n):
        for j in range(spec.top_k):
            e = int(r.ids[t, j])
            y[t] += r.w[t, j] * expert_ffn(x[t][None, :], spec.act, **_expert(params, e))[0]
        y[t] += shared_output(x[t][None, :], params, spec.act)[0] if params.get("s_w1") is not None else 0.0
    return y, r


# ----------------------------------------------------------------------------------------
# Sorted dispatch and combine: [L7.8] §2.2, §3 (worked example), §4 interface.
# ----------------------------------------------------------------------------------------

def dispatch(ids, n_experts: int):
    """Dispatch arrays for ids [N,k]: assignment a = n k + j is stably sorted by expert.

    Returns perm [A] (sorted position -> assignment), inv_perm [A] (inv_perm[perm[i]] = i),
    counts [E] and offsets [E+1] (offsets[e] is the START of expert e's slice, offsets[E]
    = A). The token of sorted row i is perm[i] // k.
    """
    ids = np.asarray(ids)
    n, k = ids.shape
    expert_of = ids.reshape(-1).astype(np.int64)
    if expert_of.size and (expert_of.min() < 0 or expert_of.max() >= n_experts):
        raise ValueError("expert id out of range")  # [L7.8] §4: bad expert ids fail loudly
    perm = np.argsort(expert_of, kind="stable")
    counts = np.bincount(expert_of, minlength=n_experts)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    inv_perm = np.empty_like(perm)
    inv_perm[perm] = np.arange(perm.size)
    return perm, inv_perm, counts, offsets


def combine(y_sorted, w, inv_perm) -> np.ndarray:
    """y_n = sum_j w_{n,j} y_sorted[inv_perm[n k + j]], j ascending ([L7.8] §2.2)."""
    y_sorted = np.asarray(y_sorted, f64)
    w = np.asarray(w, f64)
    n, k = w.shape
    out = np.zeros((n,) + y_sorted.shape[1:], f64)
    for j in range(k):
        out += w[:, j].reshape((n,) + (1,) * (y_sorted.ndim - 1)) * y_sorted[inv_perm[np.arange(n) * k + j]]
    return out


def forward_sorted(x, params: Mapping[str, Any], spec: Spec, logit_bias=None, sel_bias=None):
    """The same output by sorted dispatch: each expert runs once on its contiguous slice
    ([L7.8] §2.2), then combine. Pinned equal to forward_loop."""
    x = np.asarray(x, f64)
    r = route(x, params["w_g"], spec, logit_bias, sel_bias)
    y = expert_output_sorted(x, r.ids, r.w, params, spec) + shared_output(x, params, spec.act)
    return y, r


def expert_output_sorted(x, ids, w, params, spec: Spec) -> np.ndarray:
    """sum_j w_{n,j} FFN_{ids[n,j]}(x_n) computed via dispatch -> per-slice FFN -> combine."""
    x = np.asarray(x, f64)
    k = ids.shape[1]
    perm, inv_perm, counts, offsets = dispatch(ids, spec.n_experts)
    x_sorted = x[perm // k]
    y_sorted = np.zeros((perm.size, x.shape[1]), f64)
    for e in range(spec.n_experts):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi > lo:  # an idle expert runs nothing and its weights are never read
            y_sorted[lo:hi] = expert_ffn(x_sorted[lo:hi], spec.act, **_expert(params, e))
    return combine(y_sorted, w, inv_perm)


def forward_masked_loop(x, params: Mapping[str, Any], spec: Spec, logit_bias=None, sel_bias=None):
    """[GPT2-MoE] Diagrams 13-19 form: a dense [N,E] weight matrix that is zero off the
    chosen set; for each expert, the rows with a non-zero weight are gathered, run through
    the expert, scaled by their weight and accumulated. Pinned equal to forward_loop."""
    x = np.asarray(x, f64)
    r = route(x, params["w_g"], spec, logit_bias, sel_bias)
    n = x.shape[0]
    dense_w = np.zeros((n, spec.n_experts), f64)
    for t in range(n):
        dense_w[t, r.ids[t]] = r.w[t]
    y = np.zeros_like(x)
    for e in range(spec.n_experts):
        mask = dense_w[:, e] > 0
        if mask.any():
            y[mask] += expert_ffn(x[mask], spec.act, **_expert(params, e)) * dense_w[mask, e][:, None]
    return y + shared_output(x, params, spec.act), r


# ----------------------------------------------------------------------------------------
# Capacity-factor (token-dropping) dispatch: [nanoMoE] "Expert Capacity", "Computing the
# expert capacity" and the capacity router listing's ranking.
# ----------------------------------------------------------------------------------------

def expert_capacity(top_k: int, capacity_factor: float, n_tokens: int, n_experts: int) -> int:
    """floor(k * cf * N / E), raised by one when odd so that the capacity is even."""
    cap = math.floor(f64(top_k) * f64(capacity_factor) * f64(n_tokens) / f64(n_experts))
    return int(cap + cap % 2)


def capacity_dispatch(ids, n_experts: int, cap: int):
    """Token-dropping dispatch. Within each expert the assignments are ranked in k-major order:
    every token's first choice before any token's second choice, tokens ascending within a
    choice level, so top choices win the capacity. Ranks >= cap are dropped (no computation,
    no contribution). The kept assignments of expert e form one contiguous slice in rank
    order (a ragged batch of at most cap rows; the pages pad it to cap rows).
    Returns slot [N*k] (row of assignment a = n*k + j in the kept slices, -1 if dropped),
    kept [E] and offsets [E+1]."""
    ids = np.asarray(ids)
    n, k = ids.shape
    rank = np.zeros((n, k), np.int64)
    seen = np.zeros(n_experts, np.int64)
    for j in range(k):
        for t in range(n):
            e = int(ids[t, j])
            rank[t, j] = seen[e]
            seen[e] += 1
    kept = np.minimum(seen, cap)
    offsets = np.concatenate([[0], np.cumsum(kept)]).astype(np.int64)
    slot = np.where(rank < cap, offsets[ids] + rank, -1).reshape(-1)
    return slot, kept, offsets


def forward_capacity(x, params: Mapping[str, Any], spec: Spec, capacity_factor: float, logit_bias=None,
                     sel_bias=None, ids=None):
    """The layer with capacity-factor dispatch: dropped assignments contribute nothing, kept
    ones keep their router weight (no renormalisation over the survivors), plus Shared(x).
    ids: None, or a given choice [N,k] (see forward_loop); the ranking and the drops then
    follow that choice. Returns (y, Route, slot, kept)."""
    x = np.asarray(x, f64)
    r = route(x, params["w_g"], spec, logit_bias, sel_bias)
    if ids is not None:
        r = with_choice(r, ids, spec)
    n, d = x.shape
    cap = expert_capacity(spec.top_k, capacity_factor, n, spec.n_experts)
    slot, kept, _ = capacity_dispatch(r.ids, spec.n_experts, cap)
    y = np.zeros((n, d), f64)
    for t in range(n):
        for j in range(spec.top_k):
            if slot[t * spec.top_k + j] >= 0:
                e = int(r.ids[t, j])
                y[t] += r.w[t, j] * expert_ffn(x[t][None, :], spec.act, **_expert(params, e))[0]
    return y + shared_output(x, params, spec.act), r, slot, kept


# ----------------------------------------------------------------------------------------
# Backward: gradients of  J = <dy, y> + aux_coef * L + z_coef * z_loss  with respect to x and
# every weight, by the chain rule through the same steps as forward_loop (selection and f_e
# are piecewise constant and carry no gradient; [L7.8] §2.3 and §2.5: the selection bias
# never weighs, so it gets none either).
# ----------------------------------------------------------------------------------------

def _phi(u):
    return np.exp(-0.5 * u * u) / math.sqrt(2.0 * math.pi)


def expert_ffn_backward(xr, act: str, do, w1, w2, w3=None, b1=None, b2=None, weights: bool = True):
    """One expert on rows xr [m, d] with upstream do [m, d_out]: returns (dx, grads) where
    grads holds dw1, dw2 (and dw3 for swiglu, db1 / db2 when the biases are given);
    weights=False skips the weight gradients (grads is then empty)."""
    xr, do = np.asarray(xr, f64), np.asarray(do, f64)
    w1, w2 = np.asarray(w1, f64), np.asarray(w2, f64)
    g = {}
    if act == "gelu":
        a = xr @ w1.T + (0.0 if b1 is None else np.asarray(b1, f64)[None, :])
        dh = do @ w2
        da = dh * (0.5 * (1.0 + _erf(a / math.sqrt(2.0))) + a * _phi(a))
        if weights:
            g["dw2"] = do.T @ gelu_erf(a)
            if b2 is not None:
                g["db2"] = do.sum(axis=0)
            g["dw1"] = da.T @ xr
            if b1 is not None:
                g["db1"] = da.sum(axis=0)
        return da @ w1, g
    w3 = np.asarray(w3, f64)
    gt = xr @ w1.T
    ut = xr @ w3.T
    sg = sigmoid(gt)
    dh = do @ w2
    du = dh * gt * sg
    dg = dh * ut * sg * (1.0 + gt * (1.0 - sg))
    if weights:
        g["dw2"] = do.T @ (gt * sg * ut)
        g["dw1"] = dg.T @ xr
        g["dw3"] = du.T @ xr
    return dg @ w1 + du @ w3, g


def gate_weights_backward(z_row, ids_row, dw, spec: Spec) -> np.ndarray:
    """dJ/dz_n [E] from dJ/dw_{n,j} through the routers table's weights ([L7.8] §2.1)."""
    z_row = np.asarray(z_row, f64)
    dw = np.asarray(dw, f64)
    sc = f64(spec.routed_scaling)
    dz = np.zeros_like(z_row)
    zt = z_row[ids_row]
    if spec.router == "topk_softmax" or (spec.router == "softmax_topk" and spec.norm_topk):
        wt = softmax(zt[None, :])[0]  # p_T / sum p_T = softmax over the chosen logits
        dz[ids_row] = sc * wt * (dw - np.dot(wt, dw))
    elif spec.router == "softmax_topk":
        p = softmax(z_row[None, :])[0]
        gp = np.zeros_like(z_row)
        gp[ids_row] = sc * dw
        dz = p * (gp - np.dot(p, gp))
    else:
        sg = sigmoid(zt)
        if spec.norm_topk:
            S = sg.sum()
            wt = sg / S
            dsg = sc / S * (dw - np.dot(wt, dw))
        else:
            dsg = sc * dw
        dz[ids_row] = dsg * sg * (1.0 - sg)
    return dz


def backward(x, params: Mapping[str, Any], spec: Spec, dy, aux_coef: float = 0.0, z_coef: float = 0.0,
             logit_bias=None, sel_bias=None, tokens=None):
    """Gradients of J = <dy, y> + aux_coef L + z_coef z_loss, y and L as in forward_loop /
    load_balance, z_loss as in z_loss. Returns a dict: dx, dw_g, dw1 / dw3 / dw2 / db1 / db2
    (per expert, like params; zero for idle experts), the shared expert's ds_w1 ... when
    present, dgate [N, k] (dJ/dw) and dz [N, E].

    tokens: None, or a list of token indices: then only dx, dz and dgate of those tokens are
    returned (rows in the list's order); routing, f, P and the z-loss still cover all N
    tokens, so the rows equal the full result's."""
    x, dy = np.asarray(x, f64), np.asarray(dy, f64)
    r = route(x, params["w_g"], spec, logit_bias, sel_bias)
    n, d = x.shape
    E, k = spec.n_experts, spec.top_k
    rows = list(range(n)) if tokens is None else [int(t) for t in tokens]
    full = tokens is None
    m = len(rows)
    out = {"dx": np.zeros((m, d), f64), "dz": np.zeros((m, E), f64), "dgate": np.zeros((m, k), f64)}
    if full:
        for name in ("w1", "w3", "w2", "b1", "b2"):
            if params.get(name) is not None:
                out["d" + name] = np.zeros((E,) + np.shape(params[name][0]), f64)
    for i, t in enumerate(rows):
        for j in range(k):
            e = int(r.ids[t, j])
            pe = _expert(params, e)
            o = expert_ffn(x[t][None, :], spec.act, **pe)[0]
            out["dgate"][i, j] = np.dot(dy[t], o)
            dxt, g = expert_ffn_backward(x[t][None, :], spec.act, r.w[t, j] * dy[t][None, :], **pe, weights=full)
            out["dx"][i] += dxt[0]
            if full:
                for name, v in g.items():
                    out[name][e] += v
        out["dz"][i] = gate_weights_backward(r.z[t], r.ids[t], out["dgate"][i], spec)
    if params.get("s_w1") is not None:
        dxs, g = expert_ffn_backward(x[rows], spec.act, dy[rows], params["s_w1"], params["s_w2"], params.get("s_w3"),
                                     params.get("s_b1"), params.get("s_b2"), weights=full)
        out["dx"] += dxs
        if full:
            for name, v in g.items():
                out["ds_" + name[1:]] = v
    # aux losses through p = softmax(z): L = E sum_e f_e P_e with f constant, and z_loss
    f, _, _ = load_balance(r.p, r.ids, E)
    p = r.p[rows]
    if aux_coef:
        gp = (E / n) * f[None, :]
        out["dz"] += f64(aux_coef) * p * (gp - (p * gp).sum(axis=1, keepdims=True))
    if z_coef:
        z = r.z[rows]
        mx = z.max(axis=1)
        lse = mx + np.log(np.exp(z - mx[:, None]).sum(axis=1))
        out["dz"] += f64(z_coef) * (2.0 * lse / n)[:, None] * p
    w_g = np.asarray(params["w_g"], f64)
    out["dx"] += out["dz"] @ w_g
    if full:
        out["dw_g"] = out["dz"].T @ x
    return out


# ----------------------------------------------------------------------------------------
# Switch load-balance statistics: [L7.8] §2.3; [GPT2-MoE] router-loss function.
# ----------------------------------------------------------------------------------------

def load_balance(p, ids, n_experts: int):
    """f_e = (assignments to e) / N, P_e = mean_n p_{n,e}, L = E sum_e f_e P_e.

    f counts assignments (never probabilities); sum_e f_e = k, so L = k at perfect balance.
    """
    p = np.asarray(p, f64)
    n = p.shape[0]
    counts = np.bincount(np.asarray(ids).reshape(-1), minlength=n_experts)
    f = counts.astype(f64) / n
    P = p.mean(axis=0)
    L = n_experts * float(np.dot(f, P))
    return f, P, L


def z_loss(z) -> float:
    """Router z-loss: mean_n (logsumexp_e z_{n,e})^2 ([RB-15] §15.3; [nanoMoE] z-loss)."""
    z = np.asarray(z, f64)
    m = z.max(axis=-1)
    lse = m + np.log(np.exp(z - m[:, None]).sum(axis=-1))
    return float(np.mean(lse ** 2))


def update_bias(b, load, rate: float) -> np.ndarray:
    """Aux-free balancing step b_e <- b_e + gamma sign(mean(load) - load_e) ([L7.8] §2.5)."""
    load = np.asarray(load, f64)
    return np.asarray(b, f64) + f64(rate) * np.sign(load.mean() - load)
