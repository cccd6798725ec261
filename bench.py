"""MoE layer benchmark on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload mixtral] [--no-cpu-baseline]
                [--no-extras] [--mode forward|backward|train] [--weights tiled|rowmajor]

Forward (the default): a step is one whole layer forward (moe_forward: route, dispatch,
expert up and down projections, combine, statistics) over one batch of synthetic tokens
already resident in HBM. Prints ONE JSON line: tokens/s plus the roofline of the dominant
kernel (the fused gate/up expert projection) timed with HIP events that the library records
on its own stream, the near-tie count, the HBM-bound stages timed alone after a MALL flush,
and the CPU baselines: the float64 oracle on a bounded sample (all cores and one core) and a
float32 sorted-dispatch CPU reference on all tokens. The
routed experts' bf16 weights are re-laid out once, before the timed region, into the grouped
GEMM's tiled layout (moe_pack_weights); --weights rowmajor times them as given instead.

Backward: a step is one moe_backward (recomputed routing, dispatch and up projection, then
every gradient) for an upstream gradient dy of the same shape; the JSON line has the same
form, with the roofline of the backward's slowest GEMM stage.
"""
from __future__ import annotations

import argparse
from dataclasses import replace
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3        # MI355X fp32 (vector / matrix)
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
STAGES = ("route", "dispatch", "expert_up", "expert_down", "combine")


def algorithmic(cfg):
    """Algorithmic work per layer call (what the method itself must compute / move)."""
    N, d, E, k, f = cfg.n_tokens, cfg.d_model, cfg.n_experts, cfg.top_k, cfg.d_ff
    A = N * k
    b = 2 if cfg.dtype == "bf16" else 4
    m_up = 2 if cfg.act == "swiglu" else 1
    F = cfg.d_ff_shared
    return {
        "router_flops": 2 * N * d * E,
        "up_flops": 2 * A * d * f * m_up,
        "down_flops": 2 * A * f * d,
        "shared_flops": 2 * N * d * F * m_up + 2 * N * F * d,
        # dispatch: read x once, write x_sorted, ids in / perm / inv_perm (int32)
        "dispatch_bytes": N * d * b + A * d * b + 3 * A * 4,
        # combine (gates already applied upstream): read y_sorted and inv_perm, write y
        "combine_bytes": A * d * b + A * 4 + N * d * b,
    }


def up_bytes(cfg, n_active):
    """Algorithmic HBM bytes of the up projection: the weights (W1, and W3 for SwiGLU, with
    b1) of the n_active experts that received rows, each read once, x_sorted read once and
    the hidden activations written once."""
    A = cfg.n_tokens * cfg.top_k
    b = 2 if cfg.dtype == "bf16" else 4
    m_up = 2 if cfg.act == "swiglu" else 1
    weights = n_active * (m_up * cfg.d_ff * cfg.d_model + (cfg.d_ff if cfg.has_bias else 0)) * b
    return weights + A * cfg.d_model * b + A * cfg.d_ff * b


def file_sha(path):
    with open(path, "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()[:16]


def traffic_for(kernel_src, workload, kernel):
    """HBM bytes per launch of `kernel` (its short name) from committed rocprofv3 counter runs,
    if they were taken on the current text of the file that holds it; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        t = json.load(fh)
    if t.get("sources", {}).get(os.path.basename(kernel_src)) != file_sha(kernel_src):
        return None
    return (t.get("kernels", {}).get(kernel) or {}).get("hbm_bytes_per_launch")


def expert_gemm_kernel(cfg, epi, K):
    """Short name of the grouped GEMM kernel that runs a bf16 expert-projection launch with
    epilogue `epi` (0 GELU up, 1 SwiGLU up, 3 / 4 their saving variants) and reduction K,
    by the library's own rule: the 8-wave kernel with narrow tiles up to 1024 rows per expert,
    else the 4-wave kernel for K >= 4096, else the 8-wave kernel with full tiles only."""
    if cfg.n_tokens * cfg.top_k <= 1024 * cfg.n_experts:
        return f"expert_gemm_bf16_kernel<{epi}, 0, true>"
    if K >= 4096:
        return f"expert_gemm_w4_kernel<{epi}, 0>"
    return f"expert_gemm_bf16_kernel<{epi}, 0, false>"


def algorithmic_backward(cfg):
    """Algorithmic MFMA work of one backward per stage (U = 2 A d f; the up projection and the
    products with W1 / W3 count twice for SwiGLU)."""
    N, d, E, k, f = cfg.n_tokens, cfg.d_model, cfg.n_experts, cfg.top_k, cfg.d_ff
    U = 2 * N * k * d * f
    m = 2 if cfg.act == "swiglu" else 1
    Us = 2 * N * d * cfg.d_ff_shared
    return {"route_dispatch": 2 * N * d * E, "up_recompute": m * U, "act_backward": U, "router_backward": 0,
            "dx_rows": m * U, "dw2": U, "dw13": m * U, "shared": (3 * m + 2) * Us,
            "router_dx_combine": 4 * N * d * E}


def host_info():
    """The host the CPU baselines run on: model name, logical CPUs, CPUs this process may use."""
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except Exception:
        usable = os.cpu_count()
    return {"cpu_model": model, "logical_cpus": os.cpu_count(), "usable_cpus": usable}


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        return os.cpu_count()


def cpu_baseline(w, inp, n_sample=0, target_s=10.0, target_1core_s=8.0, reference=True):
    """The float64 CPU oracle, as it stands, on the first n_sample tokens of the workload
    (n_sample = 0: sized from an 8-token probe to take about target_s seconds), with BLAS on
    every host core; the same on one core (its own sample, sized the same way); and the
    float32 sorted-dispatch CPU reference (oracle/cpu_reference.py) on all N tokens."""
    import numpy as np
    from oracle import moe_oracle as O
    f64 = lambda t: None if t is None else t.float().cpu().numpy().astype(np.float64)
    cfg = w.cfg
    params = {"w_g": f64(inp["w_router"])}
    for name in ("w1", "w3", "w2", "b1", "b2"):
        params[name] = None if inp[name] is None else [f64(inp[name][e]) for e in range(cfg.n_experts)]
    for name, t in (inp.get("shared") or {}).items():
        params[name] = f64(t)
    spec = O.Spec(n_experts=cfg.n_experts, top_k=cfg.top_k, router=cfg.router, norm_topk=cfg.norm_topk,
                  routed_scaling=cfg.routed_scaling, act=cfg.act)
    lb, sb = f64(inp["logit_bias"]), f64(inp["sel_bias"])

    def timed(n_req, n_probe, target):
        if not n_req:
            t0 = time.perf_counter()
            O.forward_loop(f64(inp["x"][:n_probe]), params, spec, lb, sb)
            per_tok = (time.perf_counter() - t0) / n_probe
            n_req = int(min(cfg.n_tokens, max(n_probe, target / max(per_tok, 1e-9))))
        x = f64(inp["x"][:n_req])
        t0 = time.perf_counter()
        O.forward_loop(x, params, spec, lb, sb)
        return n_req, time.perf_counter() - t0

    threads = _blas_threads()
    n_all, dt = timed(n_sample, 8, target_s)
    res = {"value": n_all / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
           "sample": (f"per-token float64 oracle (routing, {cfg.top_k} expert FFNs per token, combine) on the "
                      f"first {n_all} of {cfg.n_tokens} tokens; {dt:.1f} s; weights widened to float64 "
                      f"before the timed region")}
    res.update(host_info())
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            n1, dt1 = timed(0, 2, target_1core_s)
        res["one_core"] = {"value": n1 / dt1, "unit": "tokens/s", "cores": 1,
                           "sample": f"the same oracle on the first {n1} tokens with BLAS limited to one thread; "
                                     f"{dt1:.1f} s"}
    except Exception as exc:  # threadpoolctl missing: say so rather than guess
        res["one_core"] = {"value": None, "note": f"not measured: {exc}"}
    del params
    if reference:
        res["reference_f32"] = cpu_reference_f32(w, inp)
    return res


def cpu_reference_f32(w, inp):
    """The float32 sorted-dispatch CPU reference (oracle/cpu_reference.py) on all N tokens,
    BLAS on every host core; the weights are converted to float32 before the timed region."""
    import numpy as np
    from oracle import cpu_reference as R
    cfg = w.cfg
    f32 = lambda t: None if t is None else t.float().cpu().numpy()
    params = {"w_g": f32(inp["w_router"])}
    for name in ("w1", "w3", "w2", "b1", "b2"):
        params[name] = None if inp[name] is None else [f32(inp[name][e]) for e in range(cfg.n_experts)]
    for name, t in (inp.get("shared") or {}).items():
        params[name] = f32(t)
    x = f32(inp["x"])
    lb, sb = f32(inp["logit_bias"]), f32(inp["sel_bias"])
    t0 = time.perf_counter()
    R.forward_f32(x, params, cfg.n_experts, cfg.top_k, cfg.act, cfg.router, cfg.norm_topk, cfg.routed_scaling,
                  lb, sb)
    dt = time.perf_counter() - t0
    return {"value": cfg.n_tokens / dt, "unit": "tokens/s", "cores": int(_blas_threads()), "kind": "cpu reference",
            "sample": f"NumPy float32 sorted dispatch, one matrix product per expert, all {cfg.n_tokens} tokens; "
                      f"{dt:.2f} s"}


def near_tie_count(cfg, inp):
    """Tokens whose k-th and (k+1)-th selection scores are within 1e-4 on the device (moe_route's
    margin output, same kernels and inputs as the timed forward): their choice may legitimately
    differ from the oracle's, and the parity tests check them on the device's choice."""
    from mixture_experts_layer_19_amd import binding as B
    r = B.moe_route(cfg, inp["x"], inp["w_router"], inp["logit_bias"], inp["sel_bias"], want_gap=True)
    return int((r["gap"] < 1e-4).sum().item())


def isolated_hbm_stages(cfg, inp, out, reps=10, flush_bytes=1 << 30):
    """The HBM-bound stages timed on their own, each repetition preceded by a write of
    flush_bytes of scratch so that the 256 MB MALL holds none of their inputs: moe_dispatch
    (the standalone call: histogram, scan, scatter and row copy of the forward's own ids) and
    moe_combine (the forward's combine: y_sorted already gate-scaled). HIP events on the
    library's stream; median and minimum over reps. GB/s use the algorithmic bytes."""
    import torch
    from mixture_experts_layer_19_amd import binding as B
    work = algorithmic(cfg)
    scratch = torch.empty(flush_bytes // 4, dtype=torch.int32, device="cuda")
    ev = B.HipEvents(2)
    d = B.moe_dispatch(cfg, inp["x"], out["topk_ids"])
    res = {}
    for name in ("dispatch", "combine"):
        ms = []
        for i in range(reps):
            scratch.fill_(i)
            ev.record(0)
            if name == "dispatch":
                d = B.moe_dispatch(cfg, inp["x"], out["topk_ids"], ws=d["ws"])
            else:
                B.moe_combine(cfg, d["x_sorted"], None, d["inv_perm"])
            ev.record(1)
            ms.append(ev.elapsed_ms(0, 1))
        ms.sort()
        med = ms[len(ms) // 2]
        nbytes = work[f"{name}_bytes"]
        res[name] = {"median_us": round(med * 1e3, 2), "min_us": round(ms[0] * 1e3, 2),
                     "gbs": round(nbytes / (med * 1e-3) / 1e9, 1), "frac_of_hbm": round(nbytes / (med * 1e-3) / 1e9 / PEAK_HBM_GBS, 3),
                     "algorithmic_bytes": nbytes}
    # the chip's practical rate for the same traffic: a plain device copy (torch) of half the
    # dispatch's bytes into the other half, timed the same way
    half = work["dispatch_bytes"] // 2 // 16 * 16
    src = torch.empty(half // 2, dtype=torch.int16, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    ms = []
    for i in range(reps):
        scratch.fill_(i)
        ev.record(0)
        dst.copy_(src)
        ev.record(1)
        ms.append(ev.elapsed_ms(0, 1))
    ms.sort()
    med = ms[len(ms) // 2]
    res["plain_copy"] = {"median_us": round(med * 1e3, 2), "gbs": round(2 * half / (med * 1e-3) / 1e9, 1),
                         "frac_of_hbm": round(2 * half / (med * 1e-3) / 1e9 / PEAK_HBM_GBS, 3), "bytes": 2 * half}
    res["note"] = (f"each of {reps} runs after writing {flush_bytes >> 20} MiB of scratch; dispatch is the "
                   f"standalone moe_dispatch (it also histograms and scans the ids, which the forward's "
                   f"routing does for it); x_sorted row-major; plain_copy is torch's device copy of the "
                   f"same number of bytes (half read, half written), the rate a plain copy reaches")
    return res


def cpu_baseline_backward(w, inp, dy, n_sample=0, target_s=15.0, aux_coef=0.0, z_coef=0.0):
    """The float64 CPU oracle's backward, as it stands, on the first n_sample tokens (auto-sized
    from a 4-token probe to about target_s seconds)."""
    import numpy as np
    from oracle import moe_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count()
    f64 = lambda t: None if t is None else t.float().cpu().numpy().astype(np.float64)
    cfg = w.cfg
    params = {"w_g": f64(inp["w_router"])}
    for name in ("w1", "w3", "w2", "b1", "b2"):
        params[name] = None if inp[name] is None else [f64(inp[name][e]) for e in range(cfg.n_experts)]
    for name, t in (inp.get("shared") or {}).items():
        params[name] = f64(t)
    spec = O.Spec(n_experts=cfg.n_experts, top_k=cfg.top_k, router=cfg.router, norm_topk=cfg.norm_topk,
                  routed_scaling=cfg.routed_scaling, act=cfg.act)
    lb, sb = f64(inp["logit_bias"]), f64(inp["sel_bias"])
    if not n_sample:
        t0 = time.perf_counter()
        O.backward(f64(inp["x"][:4]), params, spec, f64(dy[:4]), aux_coef, z_coef, lb, sb)
        per_tok = (time.perf_counter() - t0) / 4
        n_sample = int(min(cfg.n_tokens, max(4, target_s / max(per_tok, 1e-9))))
    t0 = time.perf_counter()
    O.backward(f64(inp["x"][:n_sample]), params, spec, f64(dy[:n_sample]), aux_coef, z_coef, lb, sb)
    dt = time.perf_counter() - t0
    return {"value": n_sample / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": (f"float64 oracle backward (routing, per-assignment expert backward, router and "
                       f"balance-loss gradients) on the first {n_sample} of {cfg.n_tokens} tokens; "
                       f"{dt:.1f} s; weights widened to float64 before the timed region")}


def run_backward(args, w, inp):
    """--mode backward: moe_backward from the state one moe_forward_train left (the training
    path), or with --recompute the self-contained backward that recomputes routing, dispatch
    and the up projection. --mode train: a whole training step, moe_forward_train then
    moe_backward(saved)."""
    import torch
    from mixture_experts_layer_19_amd import binding as B
    from mixture_experts_layer_19_amd import workload as W
    cfg = w.cfg
    dy = W.random_rows(cfg.n_tokens, cfg.d_model, cfg.torch_dtype, seed=0, tensor_id=30)
    ws = B.workspace(cfg, B.Op.BACKWARD)
    aux, zc = 0.01, 1e-3
    fkw = dict(b1=inp["b1"], b2=inp["b2"], logit_bias=inp["logit_bias"], sel_bias=inp["sel_bias"], shared=inp["shared"])
    saved = None if args.recompute else B.moe_forward_train(cfg, inp["x"], inp["w_router"], inp["w1"], inp["w3"],
                                                            inp["w2"], ws=ws, **fkw)
    train = args.mode == "train"
    fwd_ev = B.HipEvents(2) if train else None

    def call(out=None, ev=None):
        if train:
            fwd_ev.record(0)
            B.moe_forward_train(cfg, inp["x"], inp["w_router"], inp["w1"], inp["w3"], inp["w2"], ws=ws,
                                out=saved, **fkw)
            fwd_ev.record(1)
        return B.moe_backward(cfg, inp["x"], inp["w_router"], inp["w1"], inp["w3"], inp["w2"], dy, aux_coef=aux,
                              z_coef=zc, ws=ws, out=out, stage_events=ev, saved=saved, **fkw)
    out = call()
    for _ in range(max(args.warmup - 1, 0)):
        call(out)
    events = [B.HipEvents(B.BWD_EVENTS) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        call(out, events[i].handles)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    stage_ms = {s: 0.0 for s in B.BWD_STAGES}
    for ev in events:
        for j, s in enumerate(B.BWD_STAGES):
            stage_ms[s] += ev.elapsed_ms(j, j + 1) / args.steps
    ms_per_step = wall * 1e3 / args.steps
    work = algorithmic_backward(cfg)
    if saved is not None:
        # nothing recomputed: the routing and up-projection work belongs to the forward
        work["route_dispatch"] = 0
        work["up_recompute"] = 0
    flops = sum(work.values())
    fwd_flops = 0
    if train:
        f = algorithmic(cfg)
        fwd_flops = f["router_flops"] + f["up_flops"] + f["down_flops"] + f["shared_flops"]
        flops += fwd_flops
    peak = PEAK_BF16_TFLOPS
    gemm_stages = ("up_recompute", "act_backward", "dx_rows", "dw2", "dw13")
    rates = {s: work[s] / (stage_ms[s] * 1e-3) / 1e12 for s in gemm_stages + ("shared",)
             if stage_ms[s] > 0 and work[s] > 0}
    dom = max((s for s in gemm_stages if work[s] > 0), key=lambda s: stage_ms[s])
    swi = cfg.act == "swiglu"
    kernel = {"up_recompute": expert_gemm_kernel(cfg, 3 if swi else 4, cfg.d_model),
              "act_backward": "bwd_gemm_kernel<0, 2>" if swi else "bwd_gemm_kernel<0, 3>",
              "dx_rows": "bwd_gemm_kernel<0, 0>", "dw2": "bwd_gemm_kernel<1, 0>", "dw13": "bwd_gemm_kernel<1, 0>"}[dom]
    csrc = os.path.join(ROOT, "mixture_experts_layer_19_amd", "csrc")
    # the weight-gradient kernel serves several launches per call, so its averaged counters
    # do not describe one stage
    traffic = None
    if dom not in ("dw2", "dw13"):
        src = "expert_ffn.hip" if dom == "up_recompute" else "backward.hip"
        traffic = traffic_for(os.path.join(csrc, src), f"{w.name}_backward", kernel)
    E = cfg.n_experts
    what = ("train step (moe_forward_train + moe_backward from its saved state)" if train else
            "bwd tokens/s (recompute + all gradients)" if saved is None else
            "bwd tokens/s (all gradients, from moe_forward_train's saved state)")
    res = {
        "metric": f"MoE layer {what} + active TFLOP/s (% bf16 MFMA peak)",
        "value": cfg.n_tokens / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": f"{w.name} {args.mode}{' (recompute)' if saved is None else ''}: N={cfg.n_tokens} d={cfg.d_model} E={E} k={cfg.top_k} "
                               f"d_ff={cfg.d_ff} {cfg.act} {cfg.router}{'+norm' if cfg.norm_topk else ''} {cfg.dtype}"
                               f" aux_coef={aux} z_coef={zc}",
                   "global_batch": cfg.n_tokens, "parallelism": "single GPU"},
        "active_tflops": flops / (ms_per_step * 1e-3) / 1e12,
        "active_frac_of_peak": flops / (ms_per_step * 1e-3) / 1e12 / peak,
        "stage_ms": {s: round(v, 4) for s, v in stage_ms.items()},
        "stage_tflops": {s: round(v, 1) for s, v in rates.items()},
        "roofline": {"kernel": kernel, "stage": dom, "bound": "mfma", "achieved": rates[dom], "peak": peak,
                     "unit": "TFLOP/s", "frac": rates[dom] / peak, "traffic": traffic,
                     "flops_per_launch": work[dom], "avg_launch_ms": stage_ms[dom]},
        "events_vs_wall": sum(stage_ms.values()) / ms_per_step,
    }
    if train:
        res["forward_train_ms"] = fwd_ev.elapsed_ms(0, 1)  # the last step's
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_backward(w, inp, dy, args.cpu_sample, aux_coef=aux, z_coef=zc)
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mixtral")
    ap.add_argument("--weights", choices=("tiled", "rowmajor"), default="tiled",
                    help="forward: routed experts' weights re-laid out once into the tiled layout "
                         "(moe_pack_weights, outside the timed region) or row-major as given")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="forward: skip the near-tie count and the MALL-flushed isolated stage timings "
                         "(so that a kernel trace holds only the timed forward's kernels)")
    ap.add_argument("--mode", choices=("forward", "backward", "train"), default="forward")
    ap.add_argument("--recompute", action="store_true",
                    help="backward: recompute routing, dispatch and the up projection instead of a saved forward")
    ap.add_argument("--cpu-sample", type=int, default=0, help="tokens in the oracle sample (0: auto)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (reference for the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the library runs one "
              f"GPU's share of the layer and has no multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import torch
    from mixture_experts_layer_19_amd import binding as B
    from mixture_experts_layer_19_amd import workload as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")  # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)  # one elementwise kernel: reads 1 GiB, writes 1 GiB
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "elementwise copy", "bytes_read": 1 << 30, "bytes_written": 1 << 30}))
        return
    w = W.WORKLOADS[args.workload]
    cfg = w.cfg
    inp = W.make_inputs(w, seed=0, device="cuda")
    if args.mode in ("backward", "train"):
        run_backward(args, w, inp)
        return
    ws = B.workspace(cfg, B.Op.FORWARD)
    dev = inp["x"].device
    out = {
        "y": torch.empty((cfg.n_tokens, cfg.d_model), dtype=cfg.torch_dtype, device=dev),
        "topk_ids": torch.empty((cfg.n_tokens, cfg.top_k), dtype=torch.int32, device=dev),
        "topk_w": torch.empty((cfg.n_tokens, cfg.top_k), dtype=torch.float32, device=dev),
        "counts": torch.empty((cfg.n_experts,), dtype=torch.int32, device=dev),
        "stats": torch.empty((2 * cfg.n_experts + 2,), dtype=torch.float32, device=dev),
    }
    def time_forward(c, w1, w3, w2):
        call = lambda ev=None: B.moe_forward(c, inp["x"], inp["w_router"], w1, w3, w2, inp["b1"], inp["b2"],
                                             inp["logit_bias"], inp["sel_bias"], shared=inp["shared"], ws=ws,
                                             out=out, stage_events=ev)
        for _ in range(args.warmup):
            call()
        events = [B.HipEvents(6) for _ in range(args.steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            call(events[i].handles)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        sm = {s: 0.0 for s in STAGES}
        for ev in events:
            for j, s in enumerate(STAGES):
                sm[s] += ev.elapsed_ms(j, j + 1) / args.steps
        return sm, wall * 1e3 / args.steps

    # bf16: the weights re-laid out once into the GEMM's tiled layout (moe_pack_weights, before
    # the timed region, as an engine does when it loads weights), unless --weights rowmajor
    # asks for the row-major weights as given. One layout per run, so that a kernel trace of
    # this command times the launches the roofline reports.
    layout = "tiled" if cfg.dtype == "bf16" and args.weights == "tiled" else "rowmajor"
    if layout == "tiled":
        tcfg = replace(cfg, weight_layout="tiled")
        tw = {n: None if inp[n] is None else B.moe_pack_weights(cfg, 1 if n == "w2" else 0, inp[n])
              for n in ("w1", "w3", "w2")}
        torch.cuda.synchronize()
        stage_ms, ms_per_step = time_forward(tcfg, tw["w1"], tw["w3"], tw["w2"])
    else:
        stage_ms, ms_per_step = time_forward(cfg, inp["w1"], inp["w3"], inp["w2"])
    fwd_ms_events = sum(stage_ms.values())
    work = algorithmic(cfg)
    flops = work["router_flops"] + work["up_flops"] + work["down_flops"] + work["shared_flops"]
    peak = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_F32_TFLOPS
    up_tflops = work["up_flops"] / (stage_ms["expert_up"] * 1e-3) / 1e12
    stats = out["stats"].cpu().numpy()
    E = cfg.n_experts
    counts = out["counts"].cpu().numpy()

    # The up projection's bound: its arithmetic intensity against the ridge point (peak flop
    # rate / HBM bandwidth). Below it the kernel streams its weights (few rows per expert, as
    # in the DeepSeek-V3 shape) and its roofline is HBM bandwidth.
    ub = up_bytes(cfg, int((counts > 0).sum()))
    intensity = work["up_flops"] / ub
    ridge = peak * 1e12 / (PEAK_HBM_GBS * 1e9)
    up_s = stage_ms["expert_up"] * 1e-3
    kname = expert_gemm_kernel(cfg, 1 if cfg.act == "swiglu" else 0, cfg.d_model)
    src = os.path.join(ROOT, "mixture_experts_layer_19_amd", "csrc", "expert_ffn.hip")
    if intensity >= ridge:
        roof = {"kernel": kname, "bound": "mfma", "achieved": up_tflops, "peak": peak, "unit": "TFLOP/s",
                "frac": up_tflops / peak}
    else:
        gbs = ub / up_s / 1e9
        roof = {"kernel": kname, "bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": gbs / PEAK_HBM_GBS, "tflops": up_tflops}
    roof.update({"traffic": traffic_for(src, w.name, kname), "flops_per_launch": work["up_flops"],
                 "bytes_per_launch": ub, "intensity_flop_per_byte": intensity, "ridge_flop_per_byte": ridge,
                 "avg_launch_ms": stage_ms["expert_up"]})
    res = {
        "metric": "MoE layer fwd tokens/s + active TFLOP/s (% bf16 MFMA peak), 8\u00d7top-2 SwiGLU",
        "value": cfg.n_tokens / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": f"{w.name}: N={cfg.n_tokens} d={cfg.d_model} E={E} k={cfg.top_k} "
                               f"d_ff={cfg.d_ff} {cfg.act} {cfg.router}{'+norm' if cfg.norm_topk else ''} {cfg.dtype}",
                   "global_batch": cfg.n_tokens, "parallelism": "single GPU", "weight_layout": layout},
        "active_tflops": flops / (ms_per_step * 1e-3) / 1e12,
        "active_frac_of_peak": flops / (ms_per_step * 1e-3) / 1e12 / peak,
        "stage_ms": {s: round(v, 4) for s, v in stage_ms.items()},
        "stage_rates": {
            "expert_up_tflops": up_tflops,
            # the down stage also runs the shared expert, when there is one
            "expert_down_tflops": (work["down_flops"] + work["shared_flops"]) / (stage_ms["expert_down"] * 1e-3) / 1e12,
            "dispatch_gbs": work["dispatch_bytes"] / (stage_ms["dispatch"] * 1e-3) / 1e9,
            "combine_gbs": work["combine_bytes"] / (stage_ms["combine"] * 1e-3) / 1e9,
        },
        "roofline": roof,
        "switch_loss": float(stats[2 * E]),
        "z_loss": float(stats[2 * E + 1]),
        "expert_rows": {"min": int(counts.min()), "max": int(counts.max()), "empty": int((counts == 0).sum())},
        "events_vs_wall": fwd_ms_events / ms_per_step,
    }
    if not args.no_extras:
        res["near_ties"] = near_tie_count(cfg, inp)
        res["isolated_stages"] = isolated_hbm_stages(cfg, inp, out)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_sample)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
