"""Seeded synthetic workloads for the MoE layer forward (inputs only: this module holds none
of the layer's arithmetic, and both the GPU tests / bench and the CPU oracle's tests draw
their inputs from it).

Recipe (every draw seeded; seed 0 unless stated):
  * x ~ N(0, 1); every weight and bias ~ N(0, 0.02) (0.02 is the standard deviation),
    including the router W_g; drawn in float32 and rounded to bfloat16 (round to nearest
    even) for the bfloat16 workloads.
  * Each tensor (and each expert's slice of a stacked weight) has its own generator, seeded
    from numpy's SeedSequence([seed, tensor_id, expert]), so one expert can be regenerated
    alone. Large tensors are drawn with torch's generator on the target device.
  * fine-grained: a Zipf(s = 1.2) per-expert logit offset, logit_bias_e = -1.2 ln r_e with
    r = 1 + a seeded permutation of 0..E-1, which makes the expert batches heavily ragged.
  * deepseek-v3: a selection-only bias b_e ~ U(-0.1, 0.1).
  * a shared expert (d_ff_shared > 0) draws its weights like a routed expert's, from its own
    streams.
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Dict, Optional

import numpy as np
import torch

from .binding import LayerConfig

X, W_G, W1, W3, W2, B1, B2, ZIPF, SELB, SW1, SW3, SW2, SB1, SB2 = range(14)  # tensor ids of the seed streams


@dataclass(frozen=True)
class Workload:
    name: str
    cfg: LayerConfig
    logit_offset: Optional[str] = None   # "zipf1.2"
    sel_bias: Optional[str] = None       # "uniform0.1"
    weight_std: float = 0.02

    def scaled(self, **kw) -> "Workload":
        """The same recipe at other sizes (for parity cases small enough for the oracle)."""
        return replace(self, cfg=replace(self.cfg, **kw))


WORKLOADS: Dict[str, Workload] = {
    "tiny_f32": Workload("tiny_f32", LayerConfig(256, 64, 4, 2, 256, "softmax_topk", True, "gelu", False, "f32")),
    "gpt2_small": Workload("gpt2_small", LayerConfig(8192, 768, 6, 2, 3072, "softmax_topk", True, "gelu", True, "bf16")),
    "mixtral": Workload("mixtral", LayerConfig(8192, 4096, 8, 2, 14336, "softmax_topk", True, "swiglu", False, "bf16")),
    "fine_grained": Workload("fine_grained", LayerConfig(16384, 2048, 128, 8, 768, "softmax_topk", True, "swiglu", False, "bf16"),
                             logit_offset="zipf1.2"),
    "deepseek_v3": Workload("deepseek_v3", LayerConfig(4096, 7168, 256, 8, 2048, "sigmoid", True, "swiglu", False, "bf16"),
                            sel_bias="uniform0.1"),
    # the same layer with its one shared expert of width f (the pages' DeepSeek setting)
    "deepseek_v3_shared": Workload("deepseek_v3_shared",
                                   LayerConfig(4096, 7168, 256, 8, 2048, "sigmoid", True, "swiglu", False, "bf16",
                                               d_ff_shared=2048), sel_bias="uniform0.1"),
}


def stream_seed(seed: int, tensor_id: int, expert: int = 0) -> int:
    return int(np.random.SeedSequence([seed, tensor_id, expert]).generate_state(1, dtype=np.uint64)[0])


def _gen(seed, tensor_id, expert, device):
    g = torch.Generator(device=device)
    g.manual_seed(stream_seed(seed, tensor_id, expert))
    return g


def _normal(shape, std, seed, tensor_id, expert, device, dtype):
    g = _gen(seed, tensor_id, expert, device)
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)


def make_inputs(w: Workload, seed: int = 0, device="cuda") -> dict:
    """All inputs of one layer call on `device`: x, w_router, w1, w3, w2, b1, b2,
    logit_bias, sel_bias and shared (a dict of the shared expert's weights) (absent ones are
    None)."""
    c = w.cfg
    T = c.torch_dtype
    N, d, E, f = c.n_tokens, c.d_model, c.n_experts, c.d_ff
    s = w.weight_std
    out = {"x": _normal((N, d), 1.0, seed, X, 0, device, T),
           "w_router": _normal((E, d), s, seed, W_G, 0, device, T)}
    w1 = torch.empty((E, f, d), dtype=T, device=device)
    w2 = torch.empty((E, d, f), dtype=T, device=device)
    w3 = torch.empty((E, f, d), dtype=T, device=device) if c.act == "swiglu" else None
    b1 = torch.empty((E, f), dtype=T, device=device) if c.has_bias else None
    b2 = torch.empty((E, d), dtype=T, device=device) if c.has_bias else None
    for e in range(E):
        w1[e] = _normal((f, d), s, seed, W1, e, device, T)
        if w3 is not None:
            w3[e] = _normal((f, d), s, seed, W3, e, device, T)
        w2[e] = _normal((d, f), s, seed, W2, e, device, T)
        if b1 is not None:
            b1[e] = _normal((f,), s, seed, B1, e, device, T)
            b2[e] = _normal((d,), s, seed, B2, e, device, T)
    out.update(w1=w1, w3=w3, w2=w2, b1=b1, b2=b2, logit_bias=None, sel_bias=None, shared=None)
    if c.d_ff_shared:
        F = c.d_ff_shared
        sh = {"s_w1": _normal((F, d), s, seed, SW1, 0, device, T),
              "s_w3": _normal((F, d), s, seed, SW3, 0, device, T) if c.act == "swiglu" else None,
              "s_w2": _normal((d, F), s, seed, SW2, 0, device, T),
              "s_b1": _normal((F,), s, seed, SB1, 0, device, T) if c.has_bias else None,
              "s_b2": _normal((d,), s, seed, SB2, 0, device, T) if c.has_bias else None}
        out["shared"] = sh
    if w.logit_offset == "zipf1.2":
        g = _gen(seed, ZIPF, 0, "cpu")
        r = 1.0 + torch.randperm(E, generator=g).to(torch.float64)
        out["logit_bias"] = (-1.2 * torch.log(r)).to(torch.float32).to(device)
    if w.sel_bias == "uniform0.1":
        g = _gen(seed, SELB, 0, "cpu")
        out["sel_bias"] = (torch.rand(E, generator=g, dtype=torch.float32) * 0.2 - 0.1).to(device)
    return out


IDS, OFFS, YS, GW, PERM = 20, 21, 22, 23, 24  # seed streams of the stage-level inputs


def random_ids(n_tokens: int, n_experts: int, k: int, seed: int = 0, zipf: float = 0.0, device="cuda"):
    """[N,k] int32 expert ids, k distinct per row; with zipf > 0 expert e is drawn with a
    weight ~ (e+1)^-zipf, which leaves the tail experts near-empty or empty."""
    g = _gen(seed, IDS, 0, "cpu")
    u = torch.rand((n_tokens, n_experts), generator=g, dtype=torch.float64)
    keys = torch.log(u) / torch.arange(1, n_experts + 1, dtype=torch.float64).pow(-zipf) if zipf else u
    # Efraimidis-Spirakis weighted sampling without replacement: keep the k largest keys
    ids = torch.topk(keys if zipf else u, k, dim=1).indices
    return ids.to(torch.int32).to(device)


def random_counts(n_rows: int, n_experts: int, seed: int = 0, empty: int = 0):
    """Per-expert row counts summing to n_rows, with `empty` experts holding no rows."""
    rng = np.random.default_rng(stream_seed(seed, OFFS, 0))
    live = np.ones(n_experts, bool)
    if empty:
        live[rng.choice(n_experts, size=min(empty, n_experts - 1), replace=False)] = False
    w = rng.random(n_experts) * live
    cuts = np.sort(rng.choice(n_rows + 1, size=int(live.sum()) - 1, replace=True)) if live.sum() > 1 else np.array([], int)
    parts = np.diff(np.concatenate([[0], cuts, [n_rows]]))
    counts = np.zeros(n_experts, np.int64)
    counts[live] = parts
    return counts


def random_rows(n_rows: int, width: int, dtype, seed: int = 0, tensor_id: int = YS, device="cuda"):
    return _normal((n_rows, width), 1.0, seed, tensor_id, 0, device, dtype)


def random_gates(n_tokens: int, k: int, seed: int = 0, device="cuda"):
    g = _gen(seed, GW, 0, "cpu")
    return torch.rand((n_tokens, k), generator=g, dtype=torch.float32).to(device)


def random_perm(n: int, seed: int = 0, device="cuda"):
    g = _gen(seed, PERM, 0, "cpu")
    return torch.randperm(n, generator=g).to(torch.int32).to(device)
