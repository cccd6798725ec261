"""GPU parity of the layer's backward (moe_backward, bfloat16) against the CPU oracle's
analytic backward ("Mixture of Experts: routing, sorted dispatch, Switch aux loss, aux-free
bias" (L7.8) §2.1, §2.3, §2.5; "15. Mixture of Experts" (RustingBrain) §15.3), which the
CPU suite pins to central finite differences.

Tolerance (bfloat16 path): the kernels round the recomputed pre-activations, the gate-scaled
hidden activations, the activation gradients and the per-assignment dx to bfloat16 (relative
error 2^-9 each) and every gradient once more on output, with float32 accumulation; so each
gradient tensor must agree to 2e-2 of its largest magnitude element-wise and to 1e-2 in
relative Frobenius norm. Routing must agree exactly (the cases are drawn without near ties).
"""
import sys
from dataclasses import replace

import numpy as np
import pytest
import torch

from gpu_helpers import compare_ids, f64, oracle_params, reference_on_device_choice, spec_of
from mixture_experts_layer_19_amd import binding as B
from mixture_experts_layer_19_amd import workload as W
from oracle import moe_oracle as O

pytestmark = pytest.mark.gpu

TOL_MAX, TOL_FRO = 2e-2, 1e-2
DY = 30  # seed stream of the upstream gradient


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()


def close(name, gpu, ref):
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, f"{name}: shape {gpu.shape} vs {ref.shape}"
    scale = max(np.abs(ref).max(), 1e-30)
    err = np.abs(gpu - ref).max()
    fro = np.linalg.norm(gpu - ref) / max(np.linalg.norm(ref), 1e-30)
    say(f"    {name:10s} max|err| {err:.3e} (of {scale:.3e})  rel fro {fro:.3e}")
    assert err <= TOL_MAX * scale, f"{name}: max|err| {err:.3e} > {TOL_MAX} * {scale:.3e}"
    assert fro <= TOL_FRO, f"{name}: relative Frobenius error {fro:.3e} > {TOL_FRO}"


MARGIN = 1e-5  # score margins the float32 logits cannot flip (their error is ~1e-7 here)


def clean_seed(w, seeds=range(12)):
    """First seed whose oracle routing has no margin below MARGIN, so both sides must route
    alike (asserted token by token below)."""
    for seed in seeds:
        inp = W.make_inputs(w, seed=seed, device="cuda")
        r = O.route(f64(inp["x"]), f64(inp["w_router"]), spec_of(w.cfg), f64(inp["logit_bias"]),
                    f64(inp["sel_bias"]))
        if (r.gap >= MARGIN).all() and (r.intra_gap >= MARGIN).all():
            return seed
    pytest.fail("no tie-free seed")


def run_backward_and_check(w, aux_coef=0.0, z_coef=0.0):
    cfg = w.cfg
    seed = clean_seed(w)
    say(f"[backward] {w.name} {cfg} seed={seed} aux={aux_coef} z={z_coef}")
    inp = W.make_inputs(w, seed=seed, device="cuda")
    dy = W.random_rows(cfg.n_tokens, cfg.d_model, torch.bfloat16, seed=seed, tensor_id=DY)
    out = B.moe_backward(cfg, inp["x"], inp["w_router"], inp["w1"], inp["w3"], inp["w2"], dy, inp["b1"], inp["b2"],
                         inp["logit_bias"], inp["sel_bias"], shared=inp["shared"], aux_coef=aux_coef, z_coef=z_coef)
    torch.cuda.synchronize()
    params = oracle_params(inp)
    spec = spec_of(cfg)
    x = f64(inp["x"])
    ref = O.backward(x, params, spec, f64(dy), aux_coef, z_coef, f64(inp["logit_bias"]), f64(inp["sel_bias"]))
    r = O.route(x, params["w_g"], spec, f64(inp["logit_bias"]), f64(inp["sel_bias"]))
    ids = out["topk_ids"].cpu().numpy()
    assert np.array_equal(ids, r.ids), "routing differs from the oracle's"
    close("dx", f64(out["dx"]), ref["dx"])
    close("dz", f64(out["dz"]), ref["dz"])
    close("dgate", f64(out["dgate"]), ref["dgate"])
    close("dw_router", f64(out["dw_router"]), ref["dw_g"])
    for name in ("dw1", "dw3", "dw2", "db1", "db2"):
        if out.get(name) is not None:
            close(name, f64(out[name]), ref[name])
        else:
            assert name not in ref
    for name in ("ds_w1", "ds_w3", "ds_w2", "ds_b1", "ds_b2"):
        if out.get(name) is not None:
            close(name, f64(out[name]), ref[name])
        else:
            assert name not in ref
    return out, inp, dy


CASES = {
    # SwiGLU, softmax then top-k renormalised; tails in every tile dimension
    "mixtral": (W.WORKLOADS["mixtral"].scaled(n_tokens=300, d_model=136, d_ff=264), 0.01, 1e-3),
    # GELU with biases (b1 / b2 gradients, the b2 term of dgate)
    "gpt2_bias": (W.WORKLOADS["gpt2_small"].scaled(n_tokens=257, d_model=96, d_ff=160), 0.02, 0.0),
    # sigmoid router with renormalisation, routed scaling, selection bias, shared SwiGLU expert
    "deepseek_shared": (W.WORKLOADS["deepseek_v3_shared"].scaled(n_tokens=200, d_model=64, n_experts=16, top_k=4,
                                                                 d_ff=64, d_ff_shared=128, routed_scaling=2.5),
                        0.0, 1e-3),
    # softmax over the chosen logits, GELU without bias, shared GELU expert
    "topk_softmax_shared": (W.WORKLOADS["gpt2_small"].scaled(n_tokens=150, d_model=64, d_ff=96, router="topk_softmax",
                                                             has_bias=False, d_ff_shared=72), 0.01, 0.0),
    # softmax then top-k without renormalisation, 130 experts (router lanes over 3 slots), Zipf logits
    "softmax_raw_e130": (W.WORKLOADS["fine_grained"].scaled(n_tokens=100, d_model=64, n_experts=130, top_k=6, d_ff=64,
                                                            norm_topk=False), 0.05, 1e-2),
    # sigmoid without renormalisation, GELU with biases, shared expert with biases
    "sigmoid_raw_gelu_shared": (W.WORKLOADS["gpt2_small"].scaled(n_tokens=64, d_model=64, n_experts=8, top_k=3,
                                                                 d_ff=96, router="sigmoid", norm_topk=False,
                                                                 routed_scaling=1.7, d_ff_shared=64), 0.0, 0.0),
    # long ragged K over few output tiles: the weight gradients (routed, shared and router)
    # split K into runs reduced in a fixed order
    "split_k": (W.WORKLOADS["mixtral"].scaled(n_tokens=4096, d_model=64, n_experts=4, top_k=1, d_ff=64,
                                              d_ff_shared=64), 0.01, 1e-3),
    # the largest router: E = 1024, k = 32 (16 experts per lane in the router backward)
    "e1024_k32": (W.WORKLOADS["mixtral"].scaled(n_tokens=24, d_model=64, n_experts=1024, top_k=32, d_ff=32),
                  0.02, 1e-3),
    # GELU with biases and top-1 routing
    "gelu_bias_top1": (W.WORKLOADS["gpt2_small"].scaled(n_tokens=333, d_model=72, n_experts=5, top_k=1, d_ff=40,
                                                        router="topk_softmax"), 0.01, 1e-3),
    # one expert for all (k = E = 1): every token in one ragged K of the weight gradients
    "single_expert": (W.WORKLOADS["mixtral"].scaled(n_tokens=70, d_model=64, n_experts=1, top_k=1, d_ff=64), 0.1, 0.1),
    # reductions of 8192 elements or more run the 4-wave grouped GEMM: the SwiGLU and GELU save
    # epilogues of the recomputed up projection (K = d, with a K tail at 8200), and in
    # moe_forward_train the pre-gated down projection (K = d_ff)
    "swiglu_long_k": (W.WORKLOADS["mixtral"].scaled(n_tokens=96, d_model=8200, d_ff=64), 0.01, 1e-3),
    "gelu_long_k": (W.WORKLOADS["gpt2_small"].scaled(n_tokens=64, d_model=8192, d_ff=72), 0.01, 0.0),
    "gelu_bias_long_kff": (W.WORKLOADS["gpt2_small"].scaled(n_tokens=80, d_model=64, d_ff=8200), 0.02, 0.0),
}


@pytest.mark.parametrize("case", list(CASES))
def test_backward_matches_oracle(case):
    w, aux, z = CASES[case]
    w = replace(w, name=case)
    run_backward_and_check(w, aux, z)


def test_backward_routing_matches_forward():
    """The recomputed routing equals moe_forward's (same kernels, same inputs)."""
    w = W.WORKLOADS["mixtral"].scaled(n_tokens=200, d_model=128, d_ff=128)
    inp = W.make_inputs(w, seed=3)
    dy = W.random_rows(200, 128, torch.bfloat16, seed=3, tensor_id=DY)
    f = B.moe_forward(w.cfg, inp["x"], inp["w_router"], inp["w1"], inp["w3"], inp["w2"])
    b = B.moe_backward(w.cfg, inp["x"], inp["w_router"], inp["w1"], inp["w3"], inp["w2"], dy)
    torch.cuda.synchronize()
    for k in ("topk_ids", "topk_w", "counts", "stats"):
        assert torch.equal(f[k], b[k]), k


def test_backward_is_linear_in_dy():
    """Without the auxiliary terms every gradient is linear in dy: dy and 2 dy (exact in
    bfloat16) give gradients that differ by exactly a factor 2 up to rounding."""
    w = W.WORKLOADS["mixtral"].scaled(n_tokens=128, d_model=64, d_ff=64)
    inp = W.make_inputs(w, seed=1)
    dy = W.random_rows(128, 64, torch.bfloat16, seed=1, tensor_id=DY)
    a = B.moe_backward(w.cfg, inp["x"], inp["w_router"], inp["w1"], inp["w3"], inp["w2"], dy)
    b = B.moe_backward(w.cfg, inp["x"], inp["w_router"], inp["w1"], inp["w3"], inp["w2"], 2 * dy)
    torch.cuda.synchronize()
    for k in ("dx", "dw_router", "dw1", "dw3", "dw2", "dz", "dgate"):
        assert torch.equal((2 * a[k].float()).to(a[k].dtype), b[k]), k


def test_backward_empty_and_one_token():
    w = W.WORKLOADS["mixtral"].scaled(n_tokens=0, d_model=64, d_ff=64)
    inp = W.make_inputs(w, seed=0)
    dy = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    out = B.moe_backward(w.cfg, inp["x"], inp["w_router"], inp["w1"], inp["w3"], inp["w2"], dy)
    torch.cuda.synchronize()
    for k in ("dw_router", "dw1", "dw3", "dw2"):
        assert not out[k].any(), k
    run_backward_and_check(replace(W.WORKLOADS["mixtral"].scaled(n_tokens=1, d_model=64, d_ff=64), name="one_token"),
                           0.01, 0.01)


def test_backward_is_deterministic():
    w = W.WORKLOADS["fine_grained"].scaled(n_tokens=333, d_model=128, d_ff=96)
    inp = W.make_inputs(w, seed=2)
    dy = W.random_rows(333, 128, torch.bfloat16, seed=2, tensor_id=DY)
    run = lambda: B.moe_backward(w.cfg, inp["x"], inp["w_router"], inp["w1"], inp["w3"], inp["w2"], dy,
                                 logit_bias=inp["logit_bias"], aux_coef=0.01, z_coef=1e-3)
    a, b = run(), run()
    torch.cuda.synchronize()
    for k in a:
        if a[k] is not None:
            assert torch.equal(a[k], b[k]), k


def test_backward_fullsize_sampled():
    """The Mixtral-shaped backward in the configuration bench.py --mode backward times (full
    N = 8192, d = 4096, d_ff = 14336, preallocated workspace, aux 0.01, z-loss 1e-3, the
    bench's inputs). Routing is checked on every token; dx, dz and dgate on a sample of tokens
    whose two experts are the two sampled experts (so the oracle widens only their weights),
    including tokens at the edges of their slices; dW1, dW3 and dW2 on 6 hidden units of each
    sampled expert, which the oracle's per-expert backward gives exactly from those units'
    weights alone (hidden units do not interact in these gradients)."""
    w = W.WORKLOADS["mixtral"]
    cfg = w.cfg
    N, d, E, k, F = cfg.n_tokens, cfg.d_model, cfg.n_experts, cfg.top_k, cfg.d_ff
    aux, zc = 0.01, 1e-3
    say(f"[backward fullsize] {cfg} aux={aux} z={zc}")
    inp = W.make_inputs(w, seed=0)
    dy = W.random_rows(N, d, cfg.torch_dtype, seed=0, tensor_id=DY)
    ws = B.workspace(cfg, B.Op.BACKWARD)
    out = B.moe_backward(cfg, inp["x"], inp["w_router"], inp["w1"], inp["w3"], inp["w2"], dy, ws=ws,
                         aux_coef=aux, z_coef=zc)
    torch.cuda.synchronize()
    spec = spec_of(cfg)
    x64, dy64 = f64(inp["x"]), f64(dy)
    wg = f64(inp["w_router"])
    r = O.route(x64, wg, spec)
    ids = out["topk_ids"].cpu().numpy()
    near, intra, agree = compare_ids(ids, r, k)
    say(f"    tokens routed differently {int((~agree).sum())}, near ties {int(near.sum())}")
    counts = np.bincount(r.ids.reshape(-1), minlength=E)
    # the two sampled experts: the fullest and the emptiest
    e_hi, e_lo = int(np.argmax(counts)), int(np.argmin(counts))
    pair = {e_hi, e_lo}
    touched = set(ids[~agree].reshape(-1).tolist()) | set(r.ids[~agree].reshape(-1).tolist())
    cand = np.nonzero(agree & np.isin(r.ids, list(pair)).all(axis=1))[0]
    perm, _, _, off = O.dispatch(r.ids, E)
    edge = [int(perm[off[e]] // k) for e in pair] + [int(perm[off[e + 1] - 1] // k) for e in pair]
    rng = np.random.default_rng(5)
    sample = sorted(set([t for t in edge if t in set(cand.tolist())]) |
                    set(rng.choice(cand, size=min(16, cand.size), replace=False).tolist()))
    say(f"    experts {sorted(pair)} rows {[int(counts[e]) for e in sorted(pair)]}, sampled tokens {len(sample)}")
    params = {"w_g": wg, "w1": {}, "w3": {}, "w2": {}}
    for e in pair:
        params["w1"][e], params["w3"][e], params["w2"][e] = f64(inp["w1"][e]), f64(inp["w3"][e]), f64(inp["w2"][e])
    ref = O.backward(x64, params, spec, dy64, aux, zc, tokens=sample)
    st = torch.from_numpy(np.array(sample)).cuda()
    close("dx[sample]", f64(out["dx"][st]), ref["dx"])
    close("dz[sample]", f64(out["dz"][st]), ref["dz"])
    close("dgate[sample]", f64(out["dgate"][st]), ref["dgate"])
    for e in sorted(pair):
        if e in touched:
            say(f"    expert {e}: a differently routed token touches it, weight slices skipped")
            continue
        units = sorted({0, F - 1} | set(np.random.default_rng(e).choice(F, size=4, replace=False).tolist()))
        tok, jj = np.nonzero(r.ids == e)
        xr = x64[tok]
        do = r.w[tok, jj][:, None] * dy64[tok]
        _, g = O.expert_ffn_backward(xr, "swiglu", do, params["w1"][e][units], params["w2"][e][:, units],
                                     params["w3"][e][units])
        u = torch.tensor(units).cuda()
        close(f"dw1[{e}]", f64(out["dw1"][e][u]), g["dw1"])
        close(f"dw3[{e}]", f64(out["dw3"][e][u]), g["dw3"])
        close(f"dw2[{e}]", f64(out["dw2"][e][:, u]), g["dw2"])


SAVED_CASES = ["mixtral", "gpt2_bias", "deepseek_shared", "sigmoid_raw_gelu_shared", "swiglu_long_k", "gelu_long_k",
               "gelu_bias_long_kff"]


@pytest.mark.parametrize("case", SAVED_CASES)
def test_forward_train_and_saved_backward(case):
    """moe_forward_train: routing outputs are moe_forward's bits and y agrees with the oracle
    to the forward's bf16 bound (its h is rounded after the gate). moe_backward(saved) then
    gives exactly the recomputing backward's bits, twice in a row from one forward."""
    w, aux, z = CASES[case]
    cfg = w.cfg
    inp = W.make_inputs(w, seed=0)
    dy = W.random_rows(cfg.n_tokens, cfg.d_model, torch.bfloat16, seed=0, tensor_id=DY)
    args = (cfg, inp["x"], inp["w_router"], inp["w1"], inp["w3"], inp["w2"])
    kw = dict(b1=inp["b1"], b2=inp["b2"], logit_bias=inp["logit_bias"], sel_bias=inp["sel_bias"], shared=inp["shared"])
    fwd = B.moe_forward(*args, **kw)
    ft = B.moe_forward_train(*args, **kw)
    torch.cuda.synchronize()
    for k in ("topk_ids", "topk_w", "counts", "stats"):
        assert torch.equal(fwd[k], ft[k]), k
    params = oracle_params(inp)
    x64, lb, sb = f64(inp["x"]), f64(inp["logit_bias"]), f64(inp["sel_bias"])
    y_own, r = O.forward_loop(x64, params, spec_of(cfg), lb, sb)
    ids = ft["topk_ids"].cpu().numpy()
    compare_ids(ids, r, cfg.top_k)
    y_ref, _ = reference_on_device_choice(x64, params, spec_of(cfg), r, ids, y_own, lb, sb)
    y = f64(ft["y"])
    err, scale = np.abs(y - y_ref).max(), np.abs(y_ref).max()
    say(f"[forward_train] {case}: max|err| {err:.3e} of {scale:.3e} on all {cfg.n_tokens} tokens")
    assert err <= 2e-2 * scale
    bkw = dict(b1=inp["b1"], b2=inp["b2"], logit_bias=inp["logit_bias"], sel_bias=inp["sel_bias"],
               shared=inp["shared"], aux_coef=aux, z_coef=z)
    ref = B.moe_backward(*args, dy, **bkw)
    s1 = B.moe_backward(*args, dy, saved=ft, **bkw)
    s2 = B.moe_backward(*args, dy, saved=ft, **bkw)
    torch.cuda.synchronize()
    for name in B.GRAD_NAMES:
        if ref.get(name) is None:
            continue
        assert torch.equal(ref[name], s1[name]), f"saved backward differs in {name}"
        assert torch.equal(ref[name], s2[name]), f"second saved backward differs in {name}"
