"""Mutation self-check of the pins: each mutant plants one plausible mistake in a copy of
the oracle (the pitfalls of the L7.8 module's section 5 table, plus slips of our own:
transposes, dropped terms, wrong signs), and at least one pin must fail on it."""
import importlib.util
import os
import sys

import numpy as np
import pytest

import oracle_pins

ORACLE_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "moe_oracle.py")


def fresh_oracle():
    spec = importlib.util.spec_from_file_location("moe_oracle_mutant", ORACLE_PATH)
    mod = importlib.util.module_from_spec(spec)
    sys.modules[spec.name] = mod  # dataclasses resolve annotations through sys.modules
    spec.loader.exec_module(mod)
    return mod


def m_renorm_always(O):  # pitfall 1: renormalising although norm_topk is off
    orig = O.gate_weights
    def gw(z, ids, spec):
        s2 = O.Spec(spec.n_experts, spec.top_k, spec.router, True, spec.routed_scaling, spec.act)
        return orig(z, ids, s2)
    O.gate_weights = gw


def m_weigh_by_biased_score(O):  # pitfall 2: the bias leaks into the weights
    orig_route = O.route
    def route(x, w_g, spec, logit_bias=None, sel_bias=None):
        r = orig_route(x, w_g, spec, logit_bias, sel_bias)
        if spec.router == "sigmoid":
            u = np.take_along_axis(r.scores, r.ids, axis=1)
            r.w = (u / u.sum(axis=1, keepdims=True) if spec.norm_topk else u) * spec.routed_scaling
        return r
    O.route = route


def m_combine_with_perm(O):  # pitfall 3: scattering back with perm instead of its inverse
    orig = O.combine
    def combine(y_sorted, w, inv_perm):
        return orig(y_sorted, w, np.argsort(inv_perm))
    O.combine = combine


def m_token_order(O):  # pitfall 4: reading tokens in token order, not grouped by expert
    def eos(x, ids, w, params, spec):
        x = np.asarray(x, np.float64)
        k = ids.shape[1]
        perm, inv_perm, counts, offsets = O.dispatch(ids, spec.n_experts)
        x_sorted = x[np.arange(perm.size) // k]
        y_sorted = np.zeros((perm.size, x.shape[1]))
        for e in range(spec.n_experts):
            lo, hi = int(offsets[e]), int(offsets[e + 1])
            if hi > lo:
                y_sorted[lo:hi] = O.expert_ffn(x_sorted[lo:hi], spec.act, **O._expert(params, e))
        return O.combine(y_sorted, w, inv_perm)
    O.expert_output_sorted = eos


def m_f_from_probs(O):  # pitfall 5: f counted from probabilities
    def lb(p, ids, E):
        p = np.asarray(p, np.float64)
        f = p.sum(axis=0) * ids.shape[1] / p.shape[0]
        P = p.mean(axis=0)
        return f, P, E * float(np.dot(f, P))
    O.load_balance = lb


def m_bias_sign_flipped(O):  # pitfall 6
    O.update_bias = lambda b, load, rate: np.asarray(b, float) - rate * np.sign(np.mean(load) - np.asarray(load, float))


def m_ties_to_highest(O):  # pitfall 7
    def topk(scores, k):
        s = np.asarray(scores, np.float64)
        return np.array([sorted(range(s.shape[1]), key=lambda i: (-row[i], -i))[:k] for row in s], dtype=np.int64)
    O.topk_ids = topk


def m_scaling_ignored(O):  # pitfall 9
    orig = O.gate_weights
    def gw(z, ids, spec):
        s2 = O.Spec(spec.n_experts, spec.top_k, spec.router, spec.norm_topk, 1.0, spec.act)
        return orig(z, ids, s2)
    O.gate_weights = gw


def m_offsets_hold_end(O):  # pitfall 11
    orig = O.dispatch
    def dispatch(ids, E):
        perm, inv_perm, counts, offsets = orig(ids, E)
        return perm, inv_perm, counts, np.concatenate([np.cumsum(counts), [perm.size]])
    O.dispatch = dispatch


def m_topk_softmax_full(O):  # pitfall 12: topk_softmax weighing by the full softmax
    orig = O.gate_weights
    def gw(z, ids, spec):
        if spec.router == "topk_softmax":
            return np.take_along_axis(O.softmax(z), ids, axis=1) * spec.routed_scaling
        return orig(z, ids, spec)
    O.gate_weights = gw


def m_smallest_first(O):
    orig = O.topk_ids
    O.topk_ids = lambda s, k: orig(s, k)[:, ::-1].copy()


def m_unstable_sort(O):
    def dispatch(ids, E):
        eo = np.asarray(ids).reshape(-1)
        perm = np.lexsort((-np.arange(eo.size), eo))  # descending assignment inside a slice
        counts = np.bincount(eo, minlength=E)
        inv = np.empty_like(perm)
        inv[perm] = np.arange(perm.size)
        return perm, inv, counts, np.concatenate([[0], np.cumsum(counts)])
    O.dispatch = dispatch


def m_inv_is_perm(O):
    orig = O.dispatch
    def dispatch(ids, E):
        perm, inv, counts, offsets = orig(ids, E)
        return perm, perm.copy(), counts, offsets
    O.dispatch = dispatch


def m_gelu_tanh(O):
    O.gelu_erf = lambda u: 0.5 * np.asarray(u) * (1 + np.tanh(np.sqrt(2 / np.pi) * (np.asarray(u) + 0.044715 * np.asarray(u) ** 3)))


def m_silu_sign(O):
    O.silu = lambda u: np.asarray(u) * O.sigmoid(-np.asarray(u))


def m_drop_b2(O):
    orig = O.expert_ffn
    O.expert_ffn = lambda xr, act, w1, w2, w3=None, b1=None, b2=None: orig(xr, act, w1, w2, w3, b1, None)


def m_drop_b1(O):
    orig = O.expert_ffn
    O.expert_ffn = lambda xr, act, w1, w2, w3=None, b1=None, b2=None: orig(xr, act, w1, w2, w3, None, b2)


def m_swap_gate_up(O):
    orig = O.expert_ffn
    def ffn(xr, act, w1, w2, w3=None, b1=None, b2=None):
        if act == "swiglu":
            return orig(xr, act, w3, w2, w1, b1, b2)
        return orig(xr, act, w1, w2, w3, b1, b2)
    O.expert_ffn = ffn


def m_transposed_router(O):
    O.router_logits = lambda x, w_g, logit_bias=None: (np.asarray(x, float) @ np.asarray(w_g, float)) + (0 if logit_bias is None else logit_bias)


def m_softmax_no_max_norm(O):
    O.softmax = lambda z: np.exp(np.asarray(z, float)) / np.exp(np.asarray(z, float)).sum(axis=-1, keepdims=True) * 1.0001


def m_combine_no_gate(O):
    def combine(y_sorted, w, inv_perm):
        n, k = np.asarray(w).shape
        return sum(np.asarray(y_sorted, float)[inv_perm[np.arange(n) * k + j]] for j in range(k))
    O.combine = combine


def m_P_over_chosen(O):
    orig = O.load_balance
    def lb(p, ids, E):
        f, _, _ = orig(p, ids, E)
        mask = np.zeros_like(np.asarray(p, float))
        np.put_along_axis(mask, np.asarray(ids), 1.0, axis=1)
        P = (np.asarray(p) * mask).mean(axis=0)
        return f, P, E * float(np.dot(f, P))
    O.load_balance = lb


def m_sigmoid_weights_softmax(O):
    orig = O.gate_weights
    def gw(z, ids, spec):
        if spec.router == "sigmoid":
            s2 = O.Spec(spec.n_experts, spec.top_k, "softmax_topk", spec.norm_topk, spec.routed_scaling, spec.act)
            return orig(z, ids, s2)
        return orig(z, ids, spec)
    O.gate_weights = gw


def m_shared_skipped(O):  # pitfall: the shared expert's term left out of the output
    O.shared_output = lambda x, params, act: np.zeros(np.shape(x))


def m_capacity_token_major(O):  # ranking in token order: a token's 2nd choice beats later 1st choices
    def cd(ids, n_experts, cap):
        ids = np.asarray(ids)
        n, k = ids.shape
        rank = np.zeros((n, k), np.int64)
        seen = np.zeros(n_experts, np.int64)
        for t in range(n):
            for j in range(k):
                rank[t, j] = seen[ids[t, j]]
                seen[ids[t, j]] += 1
        kept = np.minimum(seen, cap)
        offsets = np.concatenate([[0], np.cumsum(kept)])
        return np.where(rank < cap, offsets[ids] + rank, -1).reshape(-1), kept, offsets
    O.capacity_dispatch = cd


def m_capacity_not_even(O):
    O.expert_capacity = lambda k, cf, n, e: int(np.floor(k * cf * n / e))


def m_bw_renorm_jacobian_dropped(O):  # gradient of a renormalised gate taken as if unnormalised
    orig = O.gate_weights_backward
    def gwb(z_row, ids_row, dw, spec):
        if spec.router == "softmax_topk" and spec.norm_topk:
            wt = O.softmax(np.asarray(z_row)[ids_row][None, :])[0]
            dz = np.zeros(len(z_row))
            dz[ids_row] = spec.routed_scaling * wt * dw
            return dz
        return orig(z_row, ids_row, dw, spec)
    O.gate_weights_backward = gwb


def m_bw_silu_derivative(O):  # silu'(g) taken as sigmoid(g)
    orig = O.expert_ffn_backward
    def efb(xr, act, do, w1, w2, w3=None, b1=None, b2=None):
        if act != "swiglu":
            return orig(xr, act, do, w1, w2, w3, b1, b2)
        gt, ut = xr @ np.asarray(w1).T, xr @ np.asarray(w3).T
        sg = O.sigmoid(gt)
        dh = do @ np.asarray(w2)
        du, dg = dh * gt * sg, dh * ut * sg
        return dg @ w1 + du @ w3, {"dw1": dg.T @ xr, "dw3": du.T @ xr, "dw2": do.T @ (gt * sg * ut)}
    O.expert_ffn_backward = efb


def m_bw_aux_ignored(O):  # the load-balancing loss contributes no router gradient
    orig = O.backward
    O.backward = lambda x, params, spec, dy, aux_coef=0.0, z_coef=0.0, logit_bias=None, sel_bias=None: \
        orig(x, params, spec, dy, 0.0, z_coef, logit_bias, sel_bias)


def m_zloss_no_square(O):
    orig = O.z_loss
    O.z_loss = lambda z: float(np.sqrt(orig(z)))


def m_logit_bias_dropped(O):
    O.router_logits = lambda x, w_g, logit_bias=None: np.asarray(x, float) @ np.asarray(w_g, float).T


def m_gap_zero(O):  # every token taken for a near tie: nothing would be compared
    O.topk_gaps = lambda scores, ids: (np.zeros(len(ids)), np.zeros(len(ids)))


def m_gap_from_top(O):  # margin measured from the top choice instead of the k-th
    orig = O.topk_gaps
    def gaps(scores, ids):
        gap, intra = orig(scores, ids)
        s = np.asarray(scores, float)
        top = s[np.arange(len(ids)), ids[:, 0]]
        kth = s[np.arange(len(ids)), ids[:, -1]]
        return gap + (top - kth), intra
    O.topk_gaps = gaps


def m_intra_gap_largest(O):  # the largest adjacent margin inside the top k instead of the smallest
    orig = O.topk_gaps
    def gaps(scores, ids):
        gap, _ = orig(scores, ids)
        s = np.asarray(scores, float)
        ch = np.take_along_axis(s, ids, axis=1)
        intra = np.max(ch[:, :-1] - ch[:, 1:], axis=1) if ids.shape[1] > 1 else np.full(len(ids), np.inf)
        return gap, intra
    O.topk_gaps = gaps


def m_capacity_drops_ignored(O):  # the capacity ranks but nothing is dropped
    orig = O.capacity_dispatch
    def cd(ids, n_experts, cap):
        slot, kept, offsets = orig(ids, n_experts, cap)
        return np.abs(slot), kept, offsets
    O.capacity_dispatch = cd
    fc = O.forward_capacity
    def forward_capacity(x, params, spec, capacity_factor, logit_bias=None, sel_bias=None, ids=None):
        y, r, slot, kept = fc(x, params, spec, float(spec.n_experts) * 8, logit_bias, sel_bias, ids)
        return y, r, orig(r.ids, spec.n_experts, O.expert_capacity(spec.top_k, capacity_factor, len(r.ids),
                                                                   spec.n_experts))[0], kept
    O.forward_capacity = forward_capacity


def m_capacity_renormalised(O):  # the survivors' gates renormalised to sum to one
    def forward_capacity(x, params, spec, capacity_factor, logit_bias=None, sel_bias=None, ids=None):
        x = np.asarray(x, float)
        r = O.route(x, params["w_g"], spec, logit_bias, sel_bias)
        if ids is not None:
            r = O.with_choice(r, ids, spec)
        cap = O.expert_capacity(spec.top_k, capacity_factor, len(x), spec.n_experts)
        slot, kept, _ = O.capacity_dispatch(r.ids, spec.n_experts, cap)
        y = np.zeros_like(x)
        keep = slot.reshape(r.ids.shape) >= 0
        for t in range(len(x)):
            wt = np.where(keep[t], r.w[t], 0.0)
            if wt.sum() > 0:
                wt = wt / wt.sum()
            for j in range(spec.top_k):
                if keep[t, j]:
                    y[t] += wt[j] * O.expert_ffn(x[t][None, :], spec.act, **O._expert(params, int(r.ids[t, j])))[0]
        return y + O.shared_output(x, params, spec.act), r, slot, kept
    O.forward_capacity = forward_capacity


def m_given_choice_ignored(O):  # a given choice silently replaced by the oracle's own
    orig = O.forward_loop
    O.forward_loop = lambda x, params, spec, logit_bias=None, sel_bias=None, ids=None: \
        orig(x, params, spec, logit_bias, sel_bias)


def m_given_choice_old_gates(O):  # a given choice weighed with the gates of the oracle's own choice
    def with_choice(r, ids, spec):
        return O.Route(z=r.z, p=r.p, scores=r.scores, ids=np.asarray(ids), w=r.w, gap=r.gap, intra_gap=r.intra_gap)
    O.with_choice = with_choice


MUTANTS = [v for k, v in sorted(globals().items()) if k.startswith("m_")]


@pytest.mark.parametrize("mutant", MUTANTS, ids=lambda f: f.__name__)
def test_mutant_is_killed(mutant):
    O = fresh_oracle()
    mutant(O)
    killed = []
    for pin in oracle_pins.PINS:
        try:
            pin(O)
        except BaseException as exc:  # an assertion, pytest.fail or a crash all count
            if isinstance(exc, KeyboardInterrupt):
                raise
            killed.append(f"{pin.__name__}: {type(exc).__name__}")
    assert killed, f"no pin fails on mutant {mutant.__name__}"
