"""Test-side helpers for GPU-vs-oracle parity: host copies of device inputs in float64 and
the comparison protocol (near-tie exclusion, tolerances). Imports the oracle and the
binding, but neither of those imports this, nor each other."""
from __future__ import annotations

import numpy as np
import torch

from oracle import moe_oracle as O

NEAR_TIE = 1e-4          # tokens whose score margin is below this are excluded from id checks
TOL = {"f32": 1e-4, "bf16": 2e-2}   # max |err| <= TOL * max |y|


def f64(t):
    """Exact float64 copy of a device tensor (bf16 and f32 widen exactly)."""
    if t is None:
        return None
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def spec_of(cfg) -> O.Spec:
    return O.Spec(n_experts=cfg.n_experts, top_k=cfg.top_k, router=cfg.router, norm_topk=cfg.norm_topk,
                  routed_scaling=cfg.routed_scaling, act=cfg.act)


class LazyExperts:
    """Per-expert float64 host copies of a stacked [E, ...] device weight, fetched on use."""

    def __init__(self, t):
        self.t = t
        self.cache = {}

    def __getitem__(self, e):
        if e not in self.cache:
            if len(self.cache) > 4:
                self.cache.clear()
            self.cache[e] = f64(self.t[e])
        return self.cache[e]


def oracle_params(inp, lazy=False):
    conv = (lambda t: None if t is None else LazyExperts(t)) if lazy else f64
    p = {"w_g": f64(inp["w_router"]), "w1": conv(inp["w1"]), "w3": conv(inp["w3"]),
         "w2": conv(inp["w2"]), "b1": conv(inp["b1"]), "b2": conv(inp["b2"])}
    for name, t in (inp.get("shared") or {}).items():
        p[name] = f64(t)
    return p


def tie_masks(route: O.Route):
    """near: the k-th / (k+1)-th margin is below NEAR_TIE (choice may flip);
    intra: an adjacent margin inside the top k is below NEAR_TIE (order may flip)."""
    near = route.gap < NEAR_TIE
    intra = (~near) & (route.intra_gap < NEAR_TIE)
    return near, intra


def compare_ids(gpu_ids: np.ndarray, route: O.Route, k: int):
    """Bit-exact ids on clean tokens, same set on intra-near-tie tokens; near-tie tokens
    must still hold k distinct valid ids whose oracle scores are within NEAR_TIE of the
    oracle's k-th score. Returns (near, intra, agree) boolean masks."""
    near, intra = tie_masks(route)
    clean = ~(near | intra)
    bad = np.nonzero((gpu_ids != route.ids).any(axis=1) & clean)[0]
    assert bad.size == 0, (f"{bad.size} clean tokens route differently, e.g. token {bad[0]}: "
                           f"gpu {gpu_ids[bad[0]]} oracle {route.ids[bad[0]]} gap {route.gap[bad[0]]:.3e}")
    for t in np.nonzero(intra)[0]:
        assert sorted(gpu_ids[t]) == sorted(route.ids[t]), f"intra-tie token {t} chose another set"
    E = route.scores.shape[1]
    for t in np.nonzero(near)[0]:
        g = gpu_ids[t]
        assert len(set(g.tolist())) == k and g.min() >= 0 and g.max() < E
        kth = route.scores[t, route.ids[t, -1]]
        assert route.scores[t, g].min() >= kth - NEAR_TIE, f"near-tie token {t} chose an expert far below the k-th"
    agree = (gpu_ids == route.ids).all(axis=1)
    return near, intra, agree


def check_dispatch_valid(ids, perm, inv_perm, counts, offsets, E):
    """Properties of a correct stable dispatch of these ids (valid for any ids)."""
    ids = np.asarray(ids).reshape(-1)
    A = ids.size
    assert np.array_equal(np.sort(perm), np.arange(A)), "perm is not a permutation"
    assert np.array_equal(inv_perm[perm], np.arange(A)), "inv_perm is not perm's inverse"
    assert np.array_equal(counts, np.bincount(ids, minlength=E))
    assert offsets[0] == 0 and np.array_equal(np.diff(offsets), counts)
    for e in range(E):
        sl = perm[offsets[e]:offsets[e + 1]]
        assert (ids[sl] == e).all() and (np.diff(sl) > 0).all()


def assert_close_rel(got, want, tol, what, rows=None):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    scale = np.max(np.abs(want)) if want.size else 0.0
    err = np.max(np.abs(got - want)) if want.size else 0.0
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    assert err <= tol * max(scale, 1e-30), f"{what}: max|err| {err:.3e} > {tol:.0e} * max|y| {scale:.3e}"
    return err, scale


def check_forward_dispatch(out, gpu_ids, E):
    """moe_forward's own dispatch arrays (want_dispatch=True) against the oracle's stable sort
    of the device's ids ([L7.8] §2.2): perm, inv_perm, counts and offsets bit-exact, always
    (an integer-only stage: a near-tie choice changes the ids, never how they are sorted)."""
    perm, inv, counts, offsets = O.dispatch(np.asarray(gpu_ids), E)
    assert np.array_equal(out["perm"].cpu().numpy(), perm), "moe_forward's perm differs from the stable sort"
    assert np.array_equal(out["inv_perm"].cpu().numpy(), inv), "moe_forward's inv_perm differs"
    assert np.array_equal(out["offsets"].cpu().numpy(), offsets), "moe_forward's offsets differ"
    assert np.array_equal(out["counts"].cpu().numpy(), counts), "moe_forward's counts differ"
    return perm, inv, counts, offsets


def reference_on_device_choice(x64, params, spec, route, gpu_ids, y_own, logit_bias=None, sel_bias=None):
    """The oracle output on the device's choice: rows where the device chose as the oracle did
    keep the oracle's own output y_own; the others (a legitimate near-tie choice) are
    recomputed by the oracle for the device's ids, with the routers table's gates for that
    choice (forward_loop(ids=...)). Returns (y_ref, w_ref) for every token."""
    gpu_ids = np.asarray(gpu_ids)
    agree = (gpu_ids == route.ids).all(axis=1)
    y_ref, w_ref = np.array(y_own, copy=True), np.array(route.w, copy=True)
    rows = np.nonzero(~agree)[0]
    if rows.size:
        lb = None if logit_bias is None else logit_bias
        y_r, r_r = O.forward_loop(x64[rows], params, spec, lb, sel_bias, ids=gpu_ids[rows])
        y_ref[rows] = y_r
        w_ref[rows] = r_r.w
    return y_ref, w_ref
