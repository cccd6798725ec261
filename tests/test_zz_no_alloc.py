"""moe_forward_noalloc (the forward on the library's static device scratch, for callers that
cannot allocate) against moe_forward on the same inputs: identical outputs, bit for bit, on
two calls in a row, the second with a smaller input. (Its refusal of configurations beyond
the scratch is checked on the host in test_abi_cpu.py.)"""
import sys

import pytest
import torch

from mixture_experts_layer_19_amd import binding as B
from mixture_experts_layer_19_amd import workload as W

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def outputs(cfg, dev="cuda"):
    N, d, E, k = cfg.n_tokens, cfg.d_model, cfg.n_experts, cfg.top_k
    return {"y": torch.empty((N, d), dtype=cfg.torch_dtype, device=dev),
            "topk_ids": torch.empty((N, k), dtype=torch.int32, device=dev),
            "topk_w": torch.empty((N, k), dtype=torch.float32, device=dev),
            "counts": torch.empty((E,), dtype=torch.int32, device=dev),
            "stats": torch.empty((2 * E + 2,), dtype=torch.float32, device=dev)}


@pytest.mark.parametrize("base,kw", [("mixtral", dict(n_tokens=128)),
                                     ("deepseek_v3_shared", dict(n_tokens=200, d_model=512, d_ff=256, d_ff_shared=256)),
                                     ("gpt2_small", dict(n_tokens=400, d_model=256, d_ff=520)),
                                     ("tiny_f32", {})])
def test_noalloc_equals_forward(base, kw):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    big = W.WORKLOADS[base].scaled(**kw) if kw else W.WORKLOADS[base]
    small = big.scaled(n_tokens=max(1, big.cfg.n_tokens // 3))
    for w in (big, small):  # two calls in a row, the second smaller
        cfg = w.cfg
        assert B.moe_workspace_size(cfg, B.Op.FORWARD) <= B.NOALLOC_SCRATCH_BYTES
        say(f"[noalloc] {w.name} {cfg}")
        inp = W.make_inputs(w, seed=21)
        args = (inp["x"], inp["w_router"], inp["w1"], inp["w3"], inp["w2"], inp["b1"], inp["b2"], inp["logit_bias"],
                inp["sel_bias"])
        ref = B.moe_forward(cfg, *args, shared=inp["shared"])
        got = B.moe_forward_noalloc(cfg, *args, shared=inp["shared"], out=outputs(cfg))
        torch.cuda.synchronize()
        for key in ("y", "topk_ids", "topk_w", "counts", "stats"):
            assert torch.equal(ref[key], got[key]), f"{key} differs from moe_forward's"
