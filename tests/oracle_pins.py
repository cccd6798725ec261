"""Pins for the CPU oracle: checks against what the pages print and what the mathematics
fixes, written so that a plausible mistake in the oracle (a dropped term, a wrong sign or
index, a transposed operand, a wrong tie rule) fails at least one of them.

Each pin takes the oracle module as its argument, so that tests/test_oracle_mutations.py
can run the same pins against copies of the oracle with one planted mistake each.
This file is a helper (pytest does not collect it); tests/test_oracle_pins.py runs it.
"""
from __future__ import annotations

import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as fh:
        return json.load(fh)


def _q(v):
    """Rational strings (nested lists) -> float64 array."""
    if isinstance(v, list):
        return np.array([_q(u) for u in v], dtype=np.float64)
    return float(Fraction(v))


def _close(a, b, tol, what):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} != {b.shape}"
    err = np.max(np.abs(a - b)) if a.size else 0.0
    assert err <= tol, f"{what}: max |diff| {err:.3e} > {tol:.1e}\n got {a}\n want {b}"


def _rand_params(rng, E, d, d_ff, act, bias=False):
    p = {
        "w_g": rng.normal(0, 0.5, (E, d)),
        "w1": rng.normal(0, 0.3, (E, d_ff, d)),
        "w2": rng.normal(0, 0.3, (E, d, d_ff)),
    }
    if act == "swiglu":
        p["w3"] = rng.normal(0, 0.3, (E, d_ff, d))
    if bias:
        p["b1"] = rng.normal(0, 0.3, (E, d_ff))
        p["b2"] = rng.normal(0, 0.3, (E, d))
    return p


# ---------------------------------------------------------------------------------------
# L7.8 §3 worked example (exact rationals)
# ---------------------------------------------------------------------------------------

def _worked_route(O, norm=True):
    g = _load("worked_example.json")
    z = np.log(_q(g["exp_z"]))
    spec = O.Spec(n_experts=g["n_experts"], top_k=g["top_k"], router="softmax_topk", norm_topk=norm)
    # x = z and W_g = I, so the router projection returns the page's logits unchanged
    r = O.route(z, np.eye(g["n_experts"]), spec)
    return g, r


def pin_worked_example_routing(O):
    g, r = _worked_route(O)
    _close(r.p, _q(g["p"]), 1e-15, "softmax probs")
    assert r.ids.tolist() == g["ids"], f"ids {r.ids.tolist()} != {g['ids']} (tie must go to the lowest id)"
    _close(r.w, _q(g["w"]), 1e-15, "renormalised gates")
    _, r2 = _worked_route(O, norm=False)
    _close(r2.w, _q(g["raw_w"]), 1e-15, "gates with norm_topk off")


def pin_worked_example_dispatch(O):
    g = _load("worked_example.json")
    ids = np.array(g["ids"])
    perm, inv_perm, counts, offsets = O.dispatch(ids, g["n_experts"])
    assert ids.reshape(-1).tolist() == g["expert_of"]
    assert perm.tolist() == g["perm"], f"perm {perm.tolist()}"
    assert (perm // g["top_k"]).tolist() == g["token_of_sorted"]
    assert counts.tolist() == g["counts"], f"counts {counts.tolist()}"
    assert offsets.tolist() == g["offsets"], f"offsets {offsets.tolist()}"
    assert inv_perm.tolist() == g["inv_perm"], f"inv_perm {inv_perm.tolist()}"


def pin_worked_example_combine(O):
    g = _load("worked_example.json")
    y_sorted = _q(g["y_sorted"])[:, None]
    inv_perm = np.array(g["inv_perm"])
    _close(y_sorted[inv_perm, 0], _q(g["y_assignment_order"]), 0, "y back in assignment order")
    y = O.combine(y_sorted, _q(g["w"]), inv_perm)
    _close(y[:, 0], _q(g["y"]), 1e-13, "combined outputs 70/3, 30")


def pin_worked_example_loss(O):
    g, r = _worked_route(O)
    f, P, L = O.load_balance(r.p, r.ids, g["n_experts"])
    _close(f, _q(g["f"]), 1e-15, "f")
    _close(P, _q(g["P"]), 1e-15, "P")
    _close(L, _q(g["L"]), 1e-14, "L = 161/72")


def pin_worked_example_constant_experts(O):
    """W2 = 0 and b2_e = c_e make expert e output the constant c_e, so the layer returns
    sum_j w_{n,j} c_{T_j}: with c = (10,20,30,40) that is 50/3 and 20 for the two tokens."""
    g = _load("worked_example.json")
    E, d, d_ff = 4, 4, 3
    z = np.log(_q(g["exp_z"]))
    c = np.array([10.0, 20.0, 30.0, 40.0])
    rng = np.random.default_rng(5)
    params = {
        "w_g": np.eye(E), "w1": rng.normal(size=(E, d_ff, d)), "b1": rng.normal(size=(E, d_ff)),
        "w2": np.zeros((E, d, d_ff)), "b2": np.repeat(c[:, None], d, axis=1),
    }
    spec = O.Spec(n_experts=E, top_k=2, router="softmax_topk", act="gelu")
    for fwd in (O.forward_loop, O.forward_sorted, O.forward_masked_loop):
        y, _ = fwd(z, params, spec)
        _close(y, np.array([[50 / 3] * d, [20.0] * d]), 1e-12, fwd.__name__)


def pin_worked_example_gaps(O):
    """The tie margins on the [L7.8] §3 worked example (selection on z = ln of the page's
    exp_z). Token 0 picks ln 4, ln 2 over 0, 0: both margins are ln 2. Token 1 picks ln 3, ln 3
    (the exact tie) over ln 2: the margin inside the top k is 0, the k-th / (k+1)-th one
    ln 3 - ln 2."""
    _, r = _worked_route(O)
    gap, intra = O.topk_gaps(r.scores, r.ids)
    _close(gap, [math.log(2), math.log(3) - math.log(2)], 1e-15, "k-th / (k+1)-th margins")
    _close(intra, [math.log(2), 0.0], 1e-15, "smallest margin inside the top k")
    _close(r.gap, gap, 0, "route() carries the margins")


def pin_gpt2_moe_gaps(O):
    """Margins on [GPT2-MoE]'s printed logits. The four-logit top-2 example keeps 0.5106 and
    0.4254 over 0.1342: gap 0.4254 - 0.1342, intra 0.5106 - 0.4254. The six-logit walk-through
    at k = 3 keeps 0.5106, 0.4254, 0.1342 over 0.0418: gap 0.1342 - 0.0418 and intra the
    smaller of 0.0852 and 0.2912; k = 6 has no (k+1)-th score (gap +inf) and k = 1 no pair
    inside the top k (intra +inf)."""
    g = _load("gpt2_moe_router_printout.json")
    s4 = np.array([g["topk_example_logits"]])
    ids = O.topk_ids(s4, 2)
    gap, intra = O.topk_gaps(s4, ids)
    _close(gap, [0.4254 - 0.1342], 1e-15, "top-2 margin")
    _close(intra, [0.5106 - 0.4254], 1e-15, "top-2 intra margin")
    s6 = np.array([g["logits"]])
    gap, intra = O.topk_gaps(s6, O.topk_ids(s6, 3))
    _close(gap, [0.1342 - 0.0418], 1e-15, "top-3 margin")
    _close(intra, [0.5106 - 0.4254], 1e-15, "top-3 intra margin (the smallest pair)")
    gap, intra = O.topk_gaps(s6, O.topk_ids(s6, 6))
    assert np.isinf(gap[0]) and gap[0] > 0, "k = E: no (k+1)-th score"
    gap, intra = O.topk_gaps(s6, O.topk_ids(s6, 1))
    assert np.isinf(intra[0]) and intra[0] > 0, "k = 1: no pair inside the top k"
    _close(gap, [0.5106 - 0.4254], 1e-15, "top-1 margin")


def pin_given_choice(O):
    """The output for a given choice follows the [L7.8] §2.1 output equation with the routers
    table's gates for THAT choice. Worked example logits, constant experts c = (10, 20, 30, 40)
    (W2 = 0, b2_e = c_e): forcing token 0 onto experts (1, 3) renormalises p = (1/4, 1/2, 1/8,
    1/8) over them to (4/5, 1/5), so y_0 = 4/5 20 + 1/5 40 = 24; forcing token 1's exact tie
    the other way round, (2, 0), keeps the gates (1/2, 1/2) and y_1 = 20. With the oracle's own
    choice given back, the result is the plain forward."""
    g = _load("worked_example.json")
    E, d, d_ff = 4, 4, 3
    z = np.log(_q(g["exp_z"]))
    c = np.array([10.0, 20.0, 30.0, 40.0])
    rng = np.random.default_rng(6)
    params = {"w_g": np.eye(E), "w1": rng.normal(size=(E, d_ff, d)), "b1": rng.normal(size=(E, d_ff)),
              "w2": np.zeros((E, d, d_ff)), "b2": np.repeat(c[:, None], d, axis=1)}
    spec = O.Spec(n_experts=E, top_k=2, router="softmax_topk", act="gelu")
    y, r = O.forward_loop(z, params, spec, ids=np.array([[1, 3], [2, 0]]))
    _close(r.w, [[4 / 5, 1 / 5], [1 / 2, 1 / 2]], 1e-15, "gates of the given choice")
    _close(y, np.array([[24.0] * d, [20.0] * d]), 1e-12, "output of the given choice")
    y_own, r_own = O.forward_loop(z, params, spec)
    y_back, _ = O.forward_loop(z, params, spec, ids=r_own.ids)
    _close(y_back, y_own, 0, "own choice given back")


# ---------------------------------------------------------------------------------------
# Printed router values on the other pages
# ---------------------------------------------------------------------------------------

def pin_gpt2_moe_printout(O):
    g = _load("gpt2_moe_router_printout.json")
    z = np.array([g["logits"]])
    _close(O.softmax(z)[0], g["softmax"], 1e-4, "softmax of six logits")
    for k, key in ((2, "top2_masked_softmax"), (1, "top1_masked_softmax")):
        for router in ("topk_softmax", "softmax_topk"):
            spec = O.Spec(n_experts=6, top_k=k, router=router)
            r = O.route(z, np.eye(6), spec)
            dense = np.zeros(6)
            dense[r.ids[0]] = r.w[0]
            _close(dense, g[key], 1e-4, f"{key} via {router}")
    s = np.array([g["topk_example_logits"]])
    ids = O.topk_ids(s, g["topk_example_k"])
    assert ids[0].tolist() == g["topk_example_ids"], f"top-k ids {ids[0].tolist()}"
    _close(s[0, ids[0]], g["topk_example_values"], 0, "top-k values, largest first")


def pin_rustingbrain_gates(O):
    g = _load("rustingbrain_gates.json")
    z = np.log(np.array([g["probs"]]))
    spec = O.Spec(n_experts=len(g["probs"]), top_k=g["top_k"], router="softmax_topk")
    r = O.route(z, np.eye(len(g["probs"])), spec)
    assert r.ids[0].tolist() == g["ids"]
    _close(r.w[0], g["gates"], 5e-3, "renormalised gates 0.69 / 0.31")


# ---------------------------------------------------------------------------------------
# Textbook values and library routines
# ---------------------------------------------------------------------------------------

def pin_gelu_textbook(O):
    """GELU(u) = u Phi(u) with Phi the standard normal CDF (textbook table values)."""
    phi = {0.5: 0.6914624612740131, 1.0: 0.8413447460685429, -1.0: 0.15865525393145707,
           2.0: 0.9772498680518208, -2.0: 0.022750131948179195}
    u = np.array(list(phi))
    _close(O.gelu_erf(u), u * np.array(list(phi.values())), 1e-15, "gelu = u Phi(u)")
    _close(O.gelu_erf(np.array([0.0])), [0.0], 0, "gelu(0)")


def pin_logistic_textbook(O):
    _close(O.sigmoid(np.array([0.0, 1.0, -1.0])), [0.5, 0.7310585786300049, 0.2689414213699951],
           1e-16, "sigma")
    big = O.sigmoid(np.array([40.0, -40.0, 800.0, -800.0]))
    assert np.all(np.isfinite(big)) and abs(big[0] - 1) < 1e-15 and 0 <= big[1] < 1e-17
    _close(O.silu(np.array([1.0, -1.0, 0.0])), [0.7310585786300049, -0.2689414213699951, 0.0],
           1e-16, "silu = u sigma(u)")


def pin_expert_ffn_torch(O):
    """The expert FFN against torch.nn.functional on the CPU in float64: linear layers in
    nn.Linear's [out, in] convention, exact GELU, silu. Non-square shapes catch transposes."""
    import torch
    import torch.nn.functional as F
    rng = np.random.default_rng(11)
    m, d, d_ff = 5, 6, 9
    xr = rng.normal(size=(m, d))
    w1, w3, w2 = rng.normal(size=(d_ff, d)), rng.normal(size=(d_ff, d)), rng.normal(size=(d, d_ff))
    b1, b2 = rng.normal(size=d_ff), rng.normal(size=d)
    t = lambda a: torch.from_numpy(a)
    ref_gelu = F.linear(F.gelu(F.linear(t(xr), t(w1), t(b1)), approximate="none"), t(w2), t(b2)).numpy()
    _close(O.expert_ffn(xr, "gelu", w1, w2, b1=b1, b2=b2), ref_gelu, 1e-12, "gelu MLP vs torch")
    ref_nb = F.linear(F.gelu(F.linear(t(xr), t(w1))), t(w2)).numpy()
    _close(O.expert_ffn(xr, "gelu", w1, w2), ref_nb, 1e-12, "gelu MLP, no bias, vs torch")
    ref_swi = F.linear(F.silu(F.linear(t(xr), t(w1))) * F.linear(t(xr), t(w3)), t(w2)).numpy()
    _close(O.expert_ffn(xr, "swiglu", w1, w2, w3=w3), ref_swi, 1e-12, "swiglu vs torch")


# ---------------------------------------------------------------------------------------
# Brute force, invariants and reductions
# ---------------------------------------------------------------------------------------

def pin_topk_bruteforce(O):
    """All C(E,k) subsets: the chosen set maximises the sorted (score desc, id asc) key.
    Integer scores make ties frequent."""
    rng = np.random.default_rng(3)
    for _ in range(300):
        E = int(rng.integers(1, 7))
        k = int(rng.integers(1, E + 1))
        s = rng.integers(-2, 3, size=(1, E)).astype(np.float64)
        best = None
        for sub in itertools.combinations(range(E), k):
            key = sorted(((-s[0, e], e) for e in sub))
            if best is None or key < best:
                best = key
        want = [e for _, e in best]
        got = O.topk_ids(s, k)[0].tolist()
        assert got == want, f"scores {s[0]} k={k}: got {got}, want {want}"


def pin_balance_equals_k(O):
    """Cyclic construction: token n puts logit c on experts n..n+k-1 (mod E) and 0 elsewhere.
    By symmetry P_e = 1/E and f_e = k/E, so L = k exactly ([L7.8] §2.3)."""
    for E, k, c in ((4, 2, 1.7), (6, 2, 0.3), (8, 3, 2.0), (5, 1, 1.0), (7, 7, 0.5)):
        z = np.zeros((E, E))
        for n in range(E):
            for j in range(k):
                z[n, (n + j) % E] = c
        spec = O.Spec(n_experts=E, top_k=k)
        r = O.route(z, np.eye(E), spec)
        f, P, L = O.load_balance(r.p, r.ids, E)
        _close(f, np.full(E, k / E), 1e-15, "f at balance")
        _close(P, np.full(E, 1 / E), 1e-15, "P at balance")
        _close(L, k, 1e-13, f"L = k at balance (E={E}, k={k})")


def pin_collapse(O):
    """Identical tokens all take the same k experts; L = E sum_{e in T} p_e >= k, with
    equality only for uniform p ([RB-15] §15.7 collapsed routing)."""
    rng = np.random.default_rng(4)
    E, k, n = 8, 2, 64
    z = np.repeat(rng.normal(size=(1, E)), n, axis=0)
    r = O.route(z, np.eye(E), O.Spec(n_experts=E, top_k=k))
    assert (r.ids == r.ids[0]).all()
    f, P, L = O.load_balance(r.p, r.ids, E)
    _close(L, E * r.p[0, r.ids[0]].sum(), 1e-13, "collapsed L")
    assert L > k + 1e-3
    ru = O.route(np.zeros((n, E)), np.eye(E), O.Spec(n_experts=E, top_k=k))
    _close(O.load_balance(ru.p, ru.ids, E)[2], k, 1e-13, "collapsed but uniform p gives L = k")


def pin_counting_identities(O):
    rng = np.random.default_rng(6)
    for (N, E, k) in ((37, 5, 2), (64, 8, 3), (9, 3, 3), (1, 4, 1)):
        z = rng.normal(size=(N, E))
        r = O.route(z, np.eye(E), O.Spec(n_experts=E, top_k=k))
        perm, inv_perm, counts, offsets = O.dispatch(r.ids, E)
        A = N * k
        assert counts.sum() == A and offsets[-1] == A and offsets[0] == 0
        assert sorted(perm.tolist()) == list(range(A))
        assert (inv_perm[perm] == np.arange(A)).all() and (perm[inv_perm] == np.arange(A)).all()
        eo = r.ids.reshape(-1)
        for e in range(E):
            sl = perm[offsets[e]:offsets[e + 1]]
            assert (eo[sl] == e).all(), "slice holds another expert's assignments"
            assert (np.diff(sl) > 0).all(), "slice not in ascending assignment order (unstable)"
        f, P, L = O.load_balance(r.p, r.ids, E)
        _close(f.sum(), k, 1e-12, "sum f = k")
        _close(P.sum(), 1.0, 1e-12, "sum P = 1")
        _close(r.w.sum(axis=1), np.ones(N), 1e-12, "sum of gates = 1")


def pin_sorted_equals_loop(O):
    """Sorted dispatch equals the per-token loop ([L7.8] §2.2), and so does the masked
    per-expert loop, for every router and both activations."""
    rng = np.random.default_rng(7)
    for router in ("softmax_topk", "topk_softmax", "sigmoid"):
        for act, bias in (("gelu", True), ("gelu", False), ("swiglu", False)):
            N, d, d_ff, E, k = 23, 6, 10, 5, 2
            params = _rand_params(rng, E, d, d_ff, act, bias)
            x = rng.normal(size=(N, d))
            sel = rng.uniform(-0.1, 0.1, size=E) if router == "sigmoid" else None
            spec = O.Spec(n_experts=E, top_k=k, router=router, act=act)
            y0, r0 = O.forward_loop(x, params, spec, sel_bias=sel)
            y1, r1 = O.forward_sorted(x, params, spec, sel_bias=sel)
            y2, r2 = O.forward_masked_loop(x, params, spec, sel_bias=sel)
            assert (r0.ids == r1.ids).all() and (r0.ids == r2.ids).all()
            _close(y1, y0, 1e-12, f"sorted vs loop ({router}, {act})")
            _close(y2, y0, 1e-12, f"masked loop vs loop ({router}, {act})")
            # the token of sorted row i is perm[i] // k: each slice runs its own expert
            perm, _, _, offsets = O.dispatch(r0.ids, E)
            for e in range(E):
                rows = perm[offsets[e]:offsets[e + 1]] // k
                assert all(e in r0.ids[t] for t in rows)


def pin_dense_mixture(O):
    """k = E with softmax renormalisation is the dense mixture sum_e p_e FFN_e(x)
    ([GPT2-MoE] Diagram 4, all experts active)."""
    rng = np.random.default_rng(8)
    N, d, d_ff, E = 7, 5, 8, 4
    params = _rand_params(rng, E, d, d_ff, "gelu", True)
    x = rng.normal(size=(N, d))
    y, r = O.forward_loop(x, params, O.Spec(n_experts=E, top_k=E, act="gelu"))
    p = r.p
    want = sum(p[:, e:e + 1] * O.expert_ffn(x, "gelu", params["w1"][e], params["w2"][e],
                                            b1=params["b1"][e], b2=params["b2"][e]) for e in range(E))
    _close(y, want, 1e-12, "k = E dense mixture")


def pin_single_expert(O):
    """E = 1, k = 1: the gate is 1 for every router with renormalisation and the layer is
    the expert itself."""
    rng = np.random.default_rng(9)
    params = _rand_params(rng, 1, 4, 6, "swiglu")
    x = rng.normal(size=(5, 4))
    for router in ("softmax_topk", "topk_softmax", "sigmoid"):
        y, r = O.forward_sorted(x, params, O.Spec(n_experts=1, top_k=1, router=router))
        _close(r.w, np.ones((5, 1)), 1e-15, "single gate")
        _close(y, O.expert_ffn(x, "swiglu", params["w1"][0], params["w2"][0], w3=params["w3"][0]),
               1e-12, "E = 1 is the dense MLP")


def pin_shared_weights(O):
    """All experts with the same weights: any routing returns FFN(x) when the gates sum to 1
    (independent of routing; checks dispatch and combine)."""
    rng = np.random.default_rng(10)
    N, d, d_ff, E = 19, 6, 7, 6
    one = _rand_params(rng, 1, d, d_ff, "swiglu")
    params = {k: (np.repeat(v, E, axis=0) if k != "w_g" else rng.normal(size=(E, d))) for k, v in one.items()}
    x = rng.normal(size=(N, d))
    want = O.expert_ffn(x, "swiglu", one["w1"][0], one["w2"][0], w3=one["w3"][0])
    for router in ("softmax_topk", "topk_softmax", "sigmoid"):
        for k in (1, 2, 4):
            y, _ = O.forward_sorted(x, params, O.Spec(n_experts=E, top_k=k, router=router))
            _close(y, want, 1e-12, f"shared weights ({router}, k={k})")


def _with_shared(rng, params, S, d, f, act, bias=False):
    p = dict(params)
    p["s_w1"] = rng.normal(0, 0.3, (S * f, d))
    p["s_w2"] = rng.normal(0, 0.3, (d, S * f))
    if act == "swiglu":
        p["s_w3"] = rng.normal(0, 0.3, (S * f, d))
    if bias:
        p["s_b1"] = rng.normal(0, 0.3, (S * f,))
        p["s_b2"] = rng.normal(0, 0.3, (d,))
    return p


def pin_shared_expert_sees_every_token(O):
    """With every routed expert's output zero (W2 = 0, no b2) the layer is the shared MLP
    alone, for every token ([L7.8] §2.1: Shared(x_n) with weight 1; [RB-15] §15.4), and the
    shared term is exactly additive on top of the routed sum."""
    rng = np.random.default_rng(21)
    N, d, f, E, k = 13, 6, 5, 4, 2
    for act, bias in (("swiglu", False), ("gelu", True)):
        routed = _rand_params(rng, E, d, f, act, bias)
        params = _with_shared(rng, routed, 1, d, f, act, bias)
        x = rng.normal(size=(N, d))
        zero = dict(params, w2=np.zeros_like(params["w2"]))
        if bias:
            zero["b2"] = np.zeros_like(params["b2"])
        y0, _ = O.forward_loop(x, zero, O.Spec(n_experts=E, top_k=k, act=act))
        want = O.expert_ffn(x, act, params["s_w1"], params["s_w2"], params.get("s_w3"), params.get("s_b1"),
                            params.get("s_b2"))
        _close(y0, want, 1e-12, f"routed outputs zero: y = shared MLP ({act})")
        y_routed, _ = O.forward_loop(x, routed, O.Spec(n_experts=E, top_k=k, act=act))
        y_all, _ = O.forward_loop(x, params, O.Spec(n_experts=E, top_k=k, act=act))
        _close(y_all - y_routed, want, 1e-12, f"shared term is additive ({act})")
        y_sorted, _ = O.forward_sorted(x, params, O.Spec(n_experts=E, top_k=k, act=act))
        y_masked, _ = O.forward_masked_loop(x, params, O.Spec(n_experts=E, top_k=k, act=act))
        _close(y_sorted, y_all, 1e-12, f"sorted with shared ({act})")
        _close(y_masked, y_all, 1e-12, f"masked loop with shared ({act})")


def pin_shared_experts_concatenate(O):
    """S shared experts of width f are one gated MLP of width S f ([L7.8] §2.1): the sum of
    two separate shared experts equals one MLP whose hidden units are both sets."""
    rng = np.random.default_rng(22)
    N, d, f = 9, 7, 4
    x = rng.normal(size=(N, d))
    a = _with_shared(rng, {}, 1, d, f, "swiglu")
    b = _with_shared(rng, {}, 1, d, f, "swiglu")
    both = {"s_w1": np.concatenate([a["s_w1"], b["s_w1"]]), "s_w3": np.concatenate([a["s_w3"], b["s_w3"]]),
            "s_w2": np.concatenate([a["s_w2"], b["s_w2"]], axis=1)}
    _close(O.shared_output(x, both, "swiglu"),
           O.shared_output(x, a, "swiglu") + O.shared_output(x, b, "swiglu"), 1e-12, "S = 2 shared experts")


def pin_capacity_formula(O):
    """[nanoMoE] "Computing the expert capacity": floor(k cf N / E), odd values raised by one."""
    assert O.expert_capacity(2, 1.25, 8, 4) == 6       # floor(5) = 5 -> 6
    assert O.expert_capacity(1, 1.0, 10, 4) == 2       # floor(2.5) = 2
    assert O.expert_capacity(2, 1.0, 16, 4) == 8       # exactly 8
    assert O.expert_capacity(8, 1.0, 100, 128) == 6    # floor(6.25) = 6
    assert O.expert_capacity(1, 1.0, 3, 4) == 0        # floor(0.75) = 0: everything dropped


def pin_capacity_worked_example(O):
    """A small case ranked by hand in k-major order (all first choices, then all second
    choices, tokens ascending), capacity 2:
      first choices:  t0 e0 #0, t1 e0 #1, t2 e1 #0, t3 e0 #2 (dropped), t4 e2 #0
      second choices: t0 e1 #1, t1 e2 #1, t2 e0 #3 (dropped), t3 e1 #2 (dropped), t4 e0 #4 (dropped)
    kept = (2, 2, 2), offsets (0, 2, 4, 6); slot of a = n k + j is offsets[e] + rank."""
    ids = np.array([[0, 1], [0, 2], [1, 0], [0, 1], [2, 0]])
    slot, kept, offsets = O.capacity_dispatch(ids, 3, 2)
    assert list(kept) == [2, 2, 2] and list(offsets) == [0, 2, 4, 6]
    assert list(slot) == [0, 3, 1, 5, 2, -1, -1, -1, 4, -1]


def pin_capacity_top_choices_win(O):
    """Over capacity, an expert keeps all of its top-1 assignments before any top-2 one, and
    the kept slices hold each kept assignment once; with a capacity at least every expert's
    load, nothing is dropped and the layer equals the dropless one."""
    rng = np.random.default_rng(23)
    N, d, f, E, k = 40, 5, 6, 6, 3
    params = _rand_params(rng, E, d, f, "swiglu")
    x = rng.normal(size=(N, d))
    spec = O.Spec(n_experts=E, top_k=k, act="swiglu")
    r = O.route(x, params["w_g"], spec)
    for cap in (2, 6, 10):
        slot, kept, offsets = O.capacity_dispatch(r.ids, E, cap)
        s2 = slot.reshape(N, k)
        for e in range(E):
            first_dropped = (s2[:, 0] < 0) & (r.ids[:, 0] == e)
            later_kept = (s2[:, 1:] >= 0) & (r.ids[:, 1:] == e)
            assert not (first_dropped.any() and later_kept.any()), (cap, e)
        used = np.sort(slot[slot >= 0])
        assert np.array_equal(used, np.arange(offsets[-1])) and (kept <= cap).all()
    y_cap, _, slot, _ = O.forward_capacity(x, params, spec, capacity_factor=float(E))
    y_ref, _ = O.forward_loop(x, params, spec)
    assert (slot >= 0).all()
    _close(y_cap, y_ref, 1e-12, "capacity >= load is dropless")


def pin_capacity_drops(O):
    """Dropped assignments contribute nothing and kept ones keep their gate ([nanoMoE] "Expert
    Capacity"). The hand-ranked case of pin_capacity_worked_example (capacity 2: k cf N / E
    = 2 * 0.6 * 5 / 3 = 2) with zero router logits (uniform p, so every kept gate is 1/2) and
    constant experts c = (10, 20, 30): token 0 keeps both (10 + 20) / 2 = 15, token 1 both
    (10 + 30) / 2 = 20, token 2 only its first choice 20 / 2 = 10, token 3 nothing, token 4
    its first choice 30 / 2 = 15."""
    ids = np.array([[0, 1], [0, 2], [1, 0], [0, 1], [2, 0]])
    N, E, d, d_ff = 5, 3, 4, 3
    c = np.array([10.0, 20.0, 30.0])
    rng = np.random.default_rng(7)
    params = {"w_g": np.zeros((E, d)), "w1": rng.normal(size=(E, d_ff, d)), "b1": rng.normal(size=(E, d_ff)),
              "w2": np.zeros((E, d, d_ff)), "b2": np.repeat(c[:, None], d, axis=1)}
    spec = O.Spec(n_experts=E, top_k=2, router="softmax_topk", act="gelu")
    assert O.expert_capacity(2, 0.6, N, E) == 2
    y, r, slot, kept = O.forward_capacity(rng.normal(size=(N, d)), params, spec, 0.6, ids=ids)
    assert list(slot) == [0, 3, 1, 5, 2, -1, -1, -1, 4, -1] and list(kept) == [2, 2, 2]
    _close(r.w, np.full((N, 2), 0.5), 1e-15, "kept gates are not renormalised over survivors")
    _close(y, np.repeat([[15.0], [20.0], [10.0], [0.0], [15.0]], d, axis=1), 1e-12, "dropped rows add nothing")


def _objective(O, x, params, spec, dy, aux, zc):
    y, r = O.forward_loop(x, params, spec)
    _, _, L = O.load_balance(r.p, r.ids, spec.n_experts)
    return float(np.sum(dy * y)) + aux * L + zc * O.z_loss(r.z)


def pin_backward_matches_finite_differences(O):
    """Every gradient of J = <dy, y> + a L + b z_loss against central finite differences of
    the forward oracle itself (no shared code with the backward), for every router, both
    activations, biases and a shared expert; 8 random coordinates per tensor."""
    rng = np.random.default_rng(24)
    N, d, f, E, k = 6, 4, 3, 4, 2
    eps = 1e-6
    for router, norm, act, bias, shared, scale in (
            ("softmax_topk", True, "swiglu", False, True, 1.0), ("softmax_topk", False, "gelu", True, False, 2.5),
            ("topk_softmax", True, "gelu", False, True, 1.0), ("sigmoid", True, "swiglu", False, False, 2.5),
            ("sigmoid", False, "gelu", True, True, 1.0)):
        spec = O.Spec(n_experts=E, top_k=k, router=router, norm_topk=norm, routed_scaling=scale, act=act)
        params = _rand_params(rng, E, d, f, act, bias)
        if shared:
            params = _with_shared(rng, params, 1, d, 5, act, bias)
        x = rng.normal(size=(N, d))
        dy = rng.normal(size=(N, d))
        aux, zc = 0.3, 0.2
        g = O.backward(x, params, spec, dy, aux, zc)
        J = lambda xx, pp: _objective(O, xx, pp, spec, dy, aux, zc)
        checks = [("x", None, "dx")] + [(nm, nm, "d" + nm) for nm in ("w1", "w3", "w2", "b1", "b2", "w_g")
                                        if params.get(nm) is not None]
        checks[-1] = ("w_g", "w_g", "dw_g")
        checks += [(nm, nm, "ds_" + nm[2:]) for nm in ("s_w1", "s_w3", "s_w2", "s_b1", "s_b2") if params.get(nm) is not None]
        for label, name, gname in checks:
            base = x if name is None else np.asarray(params[name])
            for _ in range(8):
                idx = tuple(rng.integers(0, s) for s in base.shape)
                plus, minus = base.copy(), base.copy()
                plus[idx] += eps
                minus[idx] -= eps
                if name is None:
                    num = (J(plus, params) - J(minus, params)) / (2 * eps)
                else:
                    num = (J(x, dict(params, **{name: plus})) - J(x, dict(params, **{name: minus}))) / (2 * eps)
                got = g[gname][idx]
                assert abs(got - num) <= 1e-6 * max(1.0, abs(num)), (router, norm, act, label, idx, got, num)


def pin_routed_scaling(O):
    rng = np.random.default_rng(12)
    z = rng.normal(size=(11, 6))
    for router in ("softmax_topk", "topk_softmax", "sigmoid"):
        r1 = O.route(z, np.eye(6), O.Spec(n_experts=6, top_k=3, router=router))
        r2 = O.route(z, np.eye(6), O.Spec(n_experts=6, top_k=3, router=router, routed_scaling=2.5))
        assert (r1.ids == r2.ids).all()
        _close(r2.w, 2.5 * r1.w, 1e-15, f"routed_scaling multiplies every weight ({router})")
        _close(r1.w.sum(axis=1), np.ones(11), 1e-12, f"gates sum to 1 ({router})")


def pin_bias_chooses_never_weighs(O):
    """[L7.8] §2.5: the selection bias changes which experts are chosen but never their
    weights. A bias equal for every expert changes nothing; a bias that forces an expert
    in gives it its own unbiased sigma(z) share."""
    rng = np.random.default_rng(13)
    z = rng.normal(size=(16, 6))
    spec = O.Spec(n_experts=6, top_k=2, router="sigmoid")
    r0 = O.route(z, np.eye(6), spec)
    r1 = O.route(z, np.eye(6), spec, sel_bias=np.full(6, 0.37))
    assert (r0.ids == r1.ids).all()
    _close(r1.w, r0.w, 1e-15, "a uniform bias leaves the weights alone")
    b = np.zeros(6)
    b[5] = 10.0
    r2 = O.route(z, np.eye(6), spec, sel_bias=b)
    assert (r2.ids[:, 0] == 5).all(), "a large bias must choose expert 5 first"
    s = O.sigmoid(z)
    for t in range(16):
        u = s[t, r2.ids[t]]
        _close(r2.w[t], u / u.sum(), 1e-15, "weights from unbiased sigma(z)")
    # P ignores the selection bias: it is the mean softmax of the logits
    _close(O.load_balance(r2.p, r2.ids, 6)[1], O.softmax(z).mean(axis=0), 1e-15, "P without bias")


def pin_update_bias(O):
    """[L7.8] §2.5 sign rule by hand, then a skewed router spread by repeated updates."""
    got = O.update_bias(np.array([0.5, 0.0, -0.25]), np.array([3.0, 1.0, 2.0]), 0.1)
    _close(got, [0.4, 0.1, -0.25], 1e-15, "b + gamma sign(mean - load)")
    rng = np.random.default_rng(14)
    E, k, n = 4, 1, 64
    z = rng.normal(0, 0.1, size=(n, E))
    z[:, 0] += 2.0  # skewed: nearly every token prefers expert 0
    spec = O.Spec(n_experts=E, top_k=k, router="sigmoid")
    b = np.zeros(E)
    load0 = np.bincount(O.route(z, np.eye(E), spec, sel_bias=b).ids.reshape(-1), minlength=E)
    for _ in range(60):
        load = np.bincount(O.route(z, np.eye(E), spec, sel_bias=b).ids.reshape(-1), minlength=E)
        b = O.update_bias(b, load, 0.01)
    load = np.bincount(O.route(z, np.eye(E), spec, sel_bias=b).ids.reshape(-1), minlength=E)
    assert load0.max() >= 60, f"not skewed to start with: {load0}"
    assert load.max() <= 32 and load.min() >= 4, f"60 updates did not spread the load: {load}"


def pin_z_loss(O):
    """mean_n (logsumexp z_n)^2: zero logits give (ln E)^2; a constant shift c gives (c + ln E)^2."""
    _close(O.z_loss(np.zeros((3, 8))), math.log(8) ** 2, 1e-14, "z-loss of zeros")
    _close(O.z_loss(np.full((2, 4), 1.5)), (1.5 + math.log(4)) ** 2, 1e-14, "z-loss of a constant")
    z = np.array([[0.0, math.log(3.0)], [math.log(2.0), math.log(2.0)]])
    _close(O.z_loss(z), (math.log(4.0) ** 2 + math.log(4.0) ** 2) / 2, 1e-14, "z-loss by hand")


def pin_logit_bias_is_an_input_column(O):
    """A per-expert logit offset equals one more input feature fixed at 1 whose router
    weights are the offsets; it moves the choice, the gates and P alike."""
    rng = np.random.default_rng(15)
    N, d, E = 13, 5, 6
    x = rng.normal(size=(N, d))
    w_g = rng.normal(size=(E, d))
    b = rng.normal(0, 2.0, size=E)
    spec = O.Spec(n_experts=E, top_k=2)
    r = O.route(x, w_g, spec, logit_bias=b)
    ra = O.route(np.hstack([x, np.ones((N, 1))]), np.hstack([w_g, b[:, None]]), spec)
    assert (r.ids == ra.ids).all()
    _close(r.z, ra.z, 1e-13, "logits with offset")
    _close(r.w, ra.w, 1e-13, "gates with offset")
    _close(O.load_balance(r.p, r.ids, E)[1], O.load_balance(ra.p, ra.ids, E)[1], 1e-13, "P with offset")


def pin_validation(O):
    """[L7.8] §4: config bugs fail loudly."""
    import pytest
    with pytest.raises(ValueError):
        O.Spec(n_experts=4, top_k=0)
    with pytest.raises(ValueError):
        O.Spec(n_experts=4, top_k=5)
    with pytest.raises(ValueError):
        O.Spec(n_experts=4, top_k=2, router="argmax")
    with pytest.raises(ValueError):
        O.Spec(n_experts=4, top_k=2, act="relu")
    with pytest.raises(ValueError):
        O.dispatch(np.array([[0, 4]]), 4)
    with pytest.raises(ValueError):
        O.dispatch(np.array([[-1, 0]]), 4)


def pin_backward_token_subset_equals_full(O):
    """backward(tokens=...) returns exactly the full result's rows (routing, f, P and the
    z-loss over all tokens)."""
    rng = np.random.default_rng(11)
    n, d, E, k, f = 12, 6, 5, 2, 7
    x = rng.standard_normal((n, d))
    params = {"w_g": rng.standard_normal((E, d)),
              "w1": rng.standard_normal((E, f, d)) * 0.3, "w3": rng.standard_normal((E, f, d)) * 0.3,
              "w2": rng.standard_normal((E, d, f)) * 0.3}
    spec = O.Spec(n_experts=E, top_k=k, router="softmax_topk", norm_topk=True, act="swiglu")
    dy = rng.standard_normal((n, d))
    full = O.backward(x, params, spec, dy, 0.3, 0.2)
    sub = [7, 2, 11]
    part = O.backward(x, params, spec, dy, 0.3, 0.2, tokens=sub)
    assert set(part) == {"dx", "dz", "dgate"}
    for key in ("dx", "dz", "dgate"):
        np.testing.assert_allclose(part[key], full[key][sub], rtol=1e-13, atol=1e-13)


PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]

