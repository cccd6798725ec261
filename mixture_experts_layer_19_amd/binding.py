"""Thin ctypes binding over libmoe_mi355x.so, with the C ABI's names.

Argument marshalling only: tensors are checked for device, dtype, shape and contiguity,
outputs are allocated with torch (device memory is PyTorch's job here), and every step of
the layer runs in the library's HIP kernels on torch's current stream. There is no
fallback: if the library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import enum
import os
from dataclasses import dataclass, replace
from typing import Optional, Sequence

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe_mi355x.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_BAD_EXPERT_ID, MOE_ERR_HIP = range(6)
LAYOUTS = {"rowmajor": 0, "tiled": 1}
ROUTERS = {"softmax_topk": 0, "topk_softmax": 1, "sigmoid": 2}
ACTS = {"gelu": 0, "swiglu": 1}
DTYPES = {"f32": 0, "bf16": 1}
TORCH_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


class Op(enum.IntEnum):
    ROUTE = 0
    DISPATCH = 1
    EXPERT_FFN = 2
    COMBINE = 3
    FORWARD = 4
    SHARED_FFN = 5
    BACKWARD = 6


class MoeError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status})")


class MoeConfigStruct(ctypes.Structure):
    _fields_ = [
        ("n_tokens", ctypes.c_int64),
        ("d_model", ctypes.c_int32),
        ("n_experts", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("d_ff", ctypes.c_int32),
        ("router", ctypes.c_int32),
        ("norm_topk", ctypes.c_int32),
        ("act", ctypes.c_int32),
        ("has_bias", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("routed_scaling", ctypes.c_float),
        ("d_ff_shared", ctypes.c_int32),
        ("capacity_factor", ctypes.c_float),
        ("weight_layout", ctypes.c_int32),
    ]


@dataclass(frozen=True)
class LayerConfig:
    """Hyper-parameters of one layer call (mirrors moe_config)."""

    n_tokens: int
    d_model: int
    n_experts: int
    top_k: int
    d_ff: int
    router: str = "softmax_topk"
    norm_topk: bool = True
    act: str = "swiglu"
    has_bias: bool = False
    dtype: str = "bf16"
    routed_scaling: float = 1.0
    d_ff_shared: int = 0     # width S f of the shared expert(s); 0 = none
    capacity_factor: float = 0.0   # moe_forward: 0 = dropless, > 0 = capacity-factor dispatch
    weight_layout: str = "rowmajor"  # w1 / w3 / w2: "rowmajor" [E,N,K], or "tiled" (moe_pack_weights)

    def struct(self) -> MoeConfigStruct:
        if self.router not in ROUTERS or self.act not in ACTS or self.dtype not in DTYPES \
                or self.weight_layout not in LAYOUTS:
            raise ValueError(f"unknown router/act/dtype/weight_layout in {self}")
        return MoeConfigStruct(self.n_tokens, self.d_model, self.n_experts, self.top_k, self.d_ff,
                               ROUTERS[self.router], int(self.norm_topk), ACTS[self.act],
                               int(self.has_bias), DTYPES[self.dtype], float(self.routed_scaling),
                               int(self.d_ff_shared), float(self.capacity_factor), LAYOUTS[self.weight_layout])

    @property
    def torch_dtype(self):
        return TORCH_DTYPES[self.dtype]

    @property
    def n_assign(self) -> int:
        return self.n_tokens * self.top_k

    def with_tokens(self, n: int) -> "LayerConfig":
        return LayerConfig(n, self.d_model, self.n_experts, self.top_k, self.d_ff, self.router,
                           self.norm_topk, self.act, self.has_bias, self.dtype, self.routed_scaling,
                           self.d_ff_shared, self.capacity_factor, self.weight_layout)


_lib = None
_P = ctypes.c_void_p


class MoeGradsStruct(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("dx", "dw_router", "dw1", "dw3", "db1", "dw2", "db2", "ds_w1",
                                               "ds_w3", "ds_b1", "ds_w2", "ds_b2", "dz", "dgate")]


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: run `python -m mixture_experts_layer_19_amd.build` first")
    L = ctypes.CDLL(LIB_PATH)
    S = ctypes.POINTER(MoeConfigStruct)
    L.moe_workspace_size.argtypes = [S, ctypes.c_int]
    L.moe_workspace_size.restype = ctypes.c_size_t
    L.moe_route.argtypes = [S, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
    L.moe_dispatch.argtypes = [S, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
    L.moe_expert_ffn.argtypes = [S, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
    L.moe_combine.argtypes = [S, _P, _P, _P, _P, _P, _P]
    L.moe_shared_ffn.argtypes = [S, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
    L.moe_forward.argtypes = [S] + [_P] * 23 + [ctypes.c_size_t, _P, _P]
    L.moe_forward_noalloc.argtypes = [S] + [_P] * 20
    L.moe_get_device_error.argtypes = [_P, _P]
    L.moe_update_bias.argtypes = [S, _P, _P, ctypes.c_float, _P]
    L.moe_dispatch_capacity.argtypes = [S, ctypes.c_float] + [_P] * 10 + [ctypes.c_size_t, _P]
    L.moe_expert_capacity.argtypes = [ctypes.c_int32, ctypes.c_float, ctypes.c_int64, ctypes.c_int32]
    L.moe_expert_capacity.restype = ctypes.c_int64
    L.moe_backward.argtypes = ([S] + [_P] * 15 + [ctypes.c_float, ctypes.c_float, ctypes.POINTER(MoeGradsStruct)]
                               + [_P] * 4 + [ctypes.c_int, _P, ctypes.c_size_t, _P, _P])
    L.moe_forward_train.argtypes = [S] + [_P] * 20 + [ctypes.c_size_t, _P]
    L.moe_packed_weight_size.argtypes = [S, ctypes.c_int]
    L.moe_packed_weight_size.restype = ctypes.c_size_t
    L.moe_pack_weights.argtypes = [S, ctypes.c_int, _P, _P, _P]
    L.moe_status_string.argtypes = [ctypes.c_int]
    L.moe_status_string.restype = ctypes.c_char_p
    for name in ("moe_route", "moe_dispatch", "moe_expert_ffn", "moe_combine", "moe_forward", "moe_get_device_error",
                 "moe_update_bias", "moe_shared_ffn", "moe_dispatch_capacity", "moe_backward",
                 "moe_forward_train", "moe_pack_weights", "moe_forward_noalloc"):
        getattr(L, name).restype = ctypes.c_int
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().moe_status_string(int(status)).decode()


def _check(status: int, what: str):
    if status != MOE_OK:
        if status in (MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE):
            raise ValueError(f"{what}: {status_string(status)} (status {status})")
        raise MoeError(status, what)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _want(t, name, shape, dtype, optional=False):
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def moe_workspace_size(cfg: LayerConfig, op: Op) -> int:
    return int(lib().moe_workspace_size(ctypes.byref(cfg.struct()), int(op)))


def workspace(cfg: LayerConfig, op: Op, device="cuda") -> torch.Tensor:
    n = moe_workspace_size(cfg, op)
    if n == 0:
        raise ValueError(f"invalid configuration {cfg}")
    return torch.empty(n, dtype=torch.uint8, device=device)


def moe_route(cfg: LayerConfig, x, w_router, logit_bias=None, sel_bias=None, *, want_logits=False,
              want_gap=False, ws=None):
    """Routing and Switch statistics. Returns a dict of device tensors: topk_ids [N,k] int32,
    topk_w [N,k] f32, counts [E] int32, stats [2E+2] f32 (f, P, L, z_loss) and, on request,
    logits [N,E] f32 and gap [N] f32."""
    N, d, E, k = cfg.n_tokens, cfg.d_model, cfg.n_experts, cfg.top_k
    T = cfg.torch_dtype
    _want(x, "x", (N, d), T)
    _want(w_router, "w_router", (E, d), T)
    _want(logit_bias, "logit_bias", (E,), torch.float32, optional=True)
    _want(sel_bias, "sel_bias", (E,), torch.float32, optional=True)
    dev = w_router.device
    out = {
        "topk_ids": torch.empty((N, k), dtype=torch.int32, device=dev),
        "topk_w": torch.empty((N, k), dtype=torch.float32, device=dev),
        "counts": torch.empty((E,), dtype=torch.int32, device=dev),
        "stats": torch.empty((2 * E + 2,), dtype=torch.float32, device=dev),
    }
    out["logits"] = torch.empty((N, E), dtype=torch.float32, device=dev) if want_logits else None
    out["gap"] = torch.empty((N,), dtype=torch.float32, device=dev) if want_gap else None
    ws = workspace(cfg, Op.ROUTE, dev) if ws is None else ws
    st = lib().moe_route(ctypes.byref(cfg.struct()), _ptr(x), _ptr(w_router), _ptr(logit_bias), _ptr(sel_bias),
                         _ptr(out["topk_ids"]), _ptr(out["topk_w"]), _ptr(out["counts"]), _ptr(out["stats"]),
                         _ptr(out["logits"]), _ptr(out["gap"]), _ptr(ws), ws.numel(), _stream())
    _check(st, "moe_route")
    return out


def moe_dispatch(cfg: LayerConfig, x, topk_ids, topk_w=None, *, want_x_sorted=True, ws=None):
    """Sorted dispatch. Returns x_sorted [A,d] (or None), perm [A], inv_perm [A], counts [E],
    offsets [E+1], gate_sorted [A] (when topk_w is given), and the workspace used (its first
    word carries the device error flag, see moe_get_device_error)."""
    N, d, E, k = cfg.n_tokens, cfg.d_model, cfg.n_experts, cfg.top_k
    A = N * k
    _want(topk_ids, "topk_ids", (N, k), torch.int32)
    _want(topk_w, "topk_w", (N, k), torch.float32, optional=True)
    if want_x_sorted:
        _want(x, "x", (N, d), cfg.torch_dtype)
    dev = topk_ids.device
    out = {
        "x_sorted": torch.empty((A, d), dtype=cfg.torch_dtype, device=dev) if want_x_sorted else None,
        "perm": torch.empty((A,), dtype=torch.int32, device=dev),
        "inv_perm": torch.empty((A,), dtype=torch.int32, device=dev),
        "counts": torch.empty((E,), dtype=torch.int32, device=dev),
        "offsets": torch.empty((E + 1,), dtype=torch.int32, device=dev),
        "gate_sorted": torch.empty((A,), dtype=torch.float32, device=dev) if topk_w is not None else None,
    }
    ws = workspace(cfg, Op.DISPATCH, dev) if ws is None else ws
    st = lib().moe_dispatch(ctypes.byref(cfg.struct()), _ptr(x) if want_x_sorted else None, _ptr(topk_ids),
                            _ptr(topk_w), _ptr(out["x_sorted"]), _ptr(out["perm"]), _ptr(out["inv_perm"]),
                            _ptr(out["counts"]), _ptr(out["offsets"]), _ptr(out["gate_sorted"]),
                            _ptr(ws), ws.numel(), _stream())
    _check(st, "moe_dispatch")
    out["ws"] = ws
    return out


def moe_expert_capacity(top_k: int, capacity_factor: float, n_tokens: int, n_experts: int) -> int:
    """floor(k * cf * N / E), raised by one when odd (the library's own computation)."""
    return int(lib().moe_expert_capacity(int(top_k), float(capacity_factor), int(n_tokens), int(n_experts)))


def moe_dispatch_capacity(cfg: LayerConfig, capacity_factor: float, x, topk_ids, topk_w=None, *,
                          want_x=True, ws=None):
    """Capacity-factor (token-dropping) dispatch. Returns a dict of device tensors: slot [A]
    (kept row or -1), kept [E], offsets [E+1], perm_kept [A] (valid below offsets[E]), and
    x_kept [A,d] / gate_kept [A] when requested (valid below offsets[E])."""
    N, d, E, k = cfg.n_tokens, cfg.d_model, cfg.n_experts, cfg.top_k
    A = N * k
    _want(topk_ids, "topk_ids", (N, k), torch.int32)
    _want(topk_w, "topk_w", (N, k), torch.float32, optional=True)
    if want_x:
        _want(x, "x", (N, d), cfg.torch_dtype)
    dev = topk_ids.device
    out = {
        "slot": torch.empty((A,), dtype=torch.int32, device=dev),
        "kept": torch.empty((E,), dtype=torch.int32, device=dev),
        "offsets": torch.empty((E + 1,), dtype=torch.int32, device=dev),
        "perm_kept": torch.empty((A,), dtype=torch.int32, device=dev),
        "x_kept": torch.empty((A, d), dtype=cfg.torch_dtype, device=dev) if want_x else None,
        "gate_kept": torch.empty((A,), dtype=torch.float32, device=dev) if topk_w is not None else None,
    }
    ws = workspace(cfg, Op.DISPATCH, dev) if ws is None else ws
    st = lib().moe_dispatch_capacity(ctypes.byref(cfg.struct()), float(capacity_factor), _ptr(x if want_x else None),
                                     _ptr(topk_ids), _ptr(topk_w), _ptr(out["x_kept"]), _ptr(out["perm_kept"]),
                                     _ptr(out["slot"]), _ptr(out["kept"]), _ptr(out["offsets"]), _ptr(out["gate_kept"]),
                                     _ptr(ws), ws.numel(), _stream())
    _check(st, "moe_dispatch_capacity")
    return out


def moe_expert_ffn(cfg: LayerConfig, x_sorted, offsets, w1, w3, b1, w2, b2, gate_sorted=None, *, ws=None):
    """Expert FFN over the ragged slices; returns y_sorted [A,d] (rows past offsets[E] unwritten)."""
    N, d, E, k, f = cfg.n_tokens, cfg.d_model, cfg.n_experts, cfg.top_k, cfg.d_ff
    A = N * k
    T = cfg.torch_dtype
    _want(x_sorted, "x_sorted", (A, d), T)
    _want(offsets, "offsets", (E + 1,), torch.int32)
    _want(w1, "w1", weight_shape(cfg, 0), T)
    _want(w2, "w2", weight_shape(cfg, 1), T)
    _want(w3, "w3", weight_shape(cfg, 0), T, optional=cfg.act != "swiglu")
    _want(b1, "b1", (E, f), T, optional=not cfg.has_bias)
    _want(b2, "b2", (E, d), T, optional=not cfg.has_bias)
    _want(gate_sorted, "gate_sorted", (A,), torch.float32, optional=True)
    y_sorted = torch.empty((A, d), dtype=T, device=w1.device)
    ws = workspace(cfg, Op.EXPERT_FFN, w1.device) if ws is None else ws
    st = lib().moe_expert_ffn(ctypes.byref(cfg.struct()), _ptr(x_sorted), _ptr(offsets), _ptr(w1), _ptr(w3),
                              _ptr(b1), _ptr(w2), _ptr(b2), _ptr(gate_sorted), _ptr(y_sorted),
                              _ptr(ws), ws.numel(), _stream())
    _check(st, "moe_expert_ffn")
    return y_sorted


TILED_ROWS, TILED_K = 128, 32


def weight_shape(cfg: LayerConfig, which: int):
    """Shape of W1 / W3 (which = 0) or W2 (which = 1) as the calls take them: row-major
    [E,N,K], or for cfg.weight_layout == "tiled" the padded [E,Np,Kp] of moe_pack_weights."""
    N, K = (cfg.d_ff, cfg.d_model) if which == 0 else (cfg.d_model, cfg.d_ff)
    if cfg.weight_layout == "tiled":
        N = -(-N // TILED_ROWS) * TILED_ROWS
        K = -(-K // TILED_K) * TILED_K
    return (cfg.n_experts, N, K)


def moe_packed_weight_size(cfg: LayerConfig, which: int) -> int:
    return int(lib().moe_packed_weight_size(ctypes.byref(cfg.struct()), int(which)))


def moe_pack_weights(cfg: LayerConfig, which: int, w):
    """Tiled copy ([E,Np,Kp] storage in the MOE_WEIGHTS_TILED layout) of the row-major
    weight w: W1 or W3 (which = 0, [E,d_ff,d]) or W2 (which = 1, [E,d,d_ff])."""
    tcfg = replace(cfg, weight_layout="tiled")
    rcfg = replace(cfg, weight_layout="rowmajor")
    _want(w, "w", weight_shape(rcfg, which), cfg.torch_dtype)
    size = moe_packed_weight_size(rcfg, which)
    if size == 0:
        raise ValueError(f"no tiled layout for weight {which} of {cfg} (bf16, valid sizes only)")
    out = torch.empty(weight_shape(tcfg, which), dtype=cfg.torch_dtype, device=w.device)
    assert out.numel() * out.element_size() == size
    st = lib().moe_pack_weights(ctypes.byref(rcfg.struct()), int(which), _ptr(w), _ptr(out), _stream())
    _check(st, "moe_pack_weights")
    return out


def moe_combine(cfg: LayerConfig, y_sorted, topk_w, inv_perm, y_add=None):
    """Gate-weighted combine back through inv_perm, plus y_add [N,d] (the shared expert's
    output) with weight 1 when given; returns y [N,d]."""
    N, d, k = cfg.n_tokens, cfg.d_model, cfg.top_k
    _want(y_sorted, "y_sorted", (N * k, d), cfg.torch_dtype)
    _want(topk_w, "topk_w", (N, k), torch.float32, optional=True)
    _want(inv_perm, "inv_perm", (N * k,), torch.int32)
    _want(y_add, "y_add", (N, d), cfg.torch_dtype, optional=True)
    y = torch.empty((N, d), dtype=cfg.torch_dtype, device=inv_perm.device)
    st = lib().moe_combine(ctypes.byref(cfg.struct()), _ptr(y_sorted), _ptr(topk_w), _ptr(inv_perm), _ptr(y_add),
                           _ptr(y), _stream())
    _check(st, "moe_combine")
    return y


def moe_shared_ffn(cfg: LayerConfig, x, s_w1, s_w3, s_w2, s_b1=None, s_b2=None, *, ws=None):
    """The shared expert (dense MLP of width cfg.d_ff_shared) over all tokens; returns y [N,d]."""
    N, d, F = cfg.n_tokens, cfg.d_model, cfg.d_ff_shared
    T = cfg.torch_dtype
    _want(x, "x", (N, d), T)
    _want(s_w1, "s_w1", (F, d), T)
    _want(s_w3, "s_w3", (F, d), T, optional=cfg.act != "swiglu")
    _want(s_w2, "s_w2", (d, F), T)
    _want(s_b1, "s_b1", (F,), T, optional=not cfg.has_bias)
    _want(s_b2, "s_b2", (d,), T, optional=not cfg.has_bias)
    y = torch.empty((N, d), dtype=T, device=s_w1.device)
    ws = workspace(cfg, Op.SHARED_FFN, s_w1.device) if ws is None else ws
    st = lib().moe_shared_ffn(ctypes.byref(cfg.struct()), _ptr(x), _ptr(s_w1), _ptr(s_w3), _ptr(s_b1), _ptr(s_w2),
                              _ptr(s_b2), _ptr(y), _ptr(ws), ws.numel(), _stream())
    _check(st, "moe_shared_ffn")
    return y


def moe_forward(cfg: LayerConfig, x, w_router, w1, w3, w2, b1=None, b2=None, logit_bias=None, sel_bias=None,
                *, shared: Optional[dict] = None, ws=None, out=None, stage_events: Optional[Sequence[int]] = None,
                want_dispatch: bool = False):
    """The whole layer. Returns dict y [N,d], topk_ids, topk_w, counts, stats. `shared`: the
    shared expert's weights {s_w1, s_w3, s_w2, s_b1, s_b2} when cfg.d_ff_shared > 0. `out` may
    hold preallocated outputs (same keys) and `ws` a preallocated workspace, so that repeated
    calls allocate nothing. stage_events: 6 raw hipEvent_t handles (ints) or None.
    want_dispatch: also return the dispatch arrays the call used, perm [A], inv_perm [A] and
    offsets [E+1] (int32; with a capacity factor: perm_kept, slot and the kept offsets)."""
    N, d, E, k, f = cfg.n_tokens, cfg.d_model, cfg.n_experts, cfg.top_k, cfg.d_ff
    T = cfg.torch_dtype
    sh = shared or {}
    s_w1, s_w3, s_w2, s_b1, s_b2 = (sh.get(n) for n in ("s_w1", "s_w3", "s_w2", "s_b1", "s_b2"))
    if out is None:
        _want(x, "x", (N, d), T)
        _want(w_router, "w_router", (E, d), T)
        _want(w1, "w1", weight_shape(cfg, 0), T)
        _want(w2, "w2", weight_shape(cfg, 1), T)
        _want(w3, "w3", weight_shape(cfg, 0), T, optional=cfg.act != "swiglu")
        _want(b1, "b1", (E, f), T, optional=not cfg.has_bias)
        _want(b2, "b2", (E, d), T, optional=not cfg.has_bias)
        _want(logit_bias, "logit_bias", (E,), torch.float32, optional=True)
        _want(sel_bias, "sel_bias", (E,), torch.float32, optional=True)
        if cfg.d_ff_shared:
            F = cfg.d_ff_shared
            _want(s_w1, "s_w1", (F, d), T)
            _want(s_w3, "s_w3", (F, d), T, optional=cfg.act != "swiglu")
            _want(s_w2, "s_w2", (d, F), T)
            _want(s_b1, "s_b1", (F,), T, optional=not cfg.has_bias)
            _want(s_b2, "s_b2", (d,), T, optional=not cfg.has_bias)
        dev = w_router.device
        out = {
            "y": torch.empty((N, d), dtype=T, device=dev),
            "topk_ids": torch.empty((N, k), dtype=torch.int32, device=dev),
            "topk_w": torch.empty((N, k), dtype=torch.float32, device=dev),
            "counts": torch.empty((E,), dtype=torch.int32, device=dev),
            "stats": torch.empty((2 * E + 2,), dtype=torch.float32, device=dev),
        }
    if want_dispatch and "perm" not in out:
        dev = w_router.device
        out["perm"] = torch.empty((N * k,), dtype=torch.int32, device=dev)
        out["inv_perm"] = torch.empty((N * k,), dtype=torch.int32, device=dev)
        out["offsets"] = torch.empty((E + 1,), dtype=torch.int32, device=dev)
    if ws is None:
        ws = workspace(cfg, Op.FORWARD, w_router.device)
    ev = None
    if stage_events is not None:
        if len(stage_events) != 6:
            raise ValueError("stage_events needs 6 events")
        ev = (ctypes.c_void_p * 6)(*[ctypes.c_void_p(int(e)) for e in stage_events])
    st = lib().moe_forward(ctypes.byref(cfg.struct()), _ptr(x), _ptr(w_router), _ptr(logit_bias), _ptr(sel_bias),
                           _ptr(w1), _ptr(w3), _ptr(b1), _ptr(w2), _ptr(b2), _ptr(s_w1), _ptr(s_w3), _ptr(s_b1),
                           _ptr(s_w2), _ptr(s_b2), _ptr(out["y"]), _ptr(out["topk_ids"]),
                           _ptr(out["topk_w"]), _ptr(out["counts"]), _ptr(out["stats"]), _ptr(out.get("perm")),
                           _ptr(out.get("inv_perm")), _ptr(out.get("offsets")), _ptr(ws), ws.numel(),
                           ev, _stream())
    _check(st, "moe_forward")
    return out


NOALLOC_SCRATCH_BYTES = 128 << 20  # MOE_NOALLOC_SCRATCH_BYTES


def moe_forward_noalloc(cfg: LayerConfig, x, w_router, w1, w3, w2, b1=None, b2=None, logit_bias=None, sel_bias=None,
                        *, shared: Optional[dict] = None, out: dict):
    """moe_forward on the library's static device scratch: the call allocates nothing (the
    outputs in `out` are the caller's: y, topk_ids, topk_w, counts, stats). Calls on one GPU
    must not overlap."""
    sh = shared or {}
    s_w1, s_w3, s_w2, s_b1, s_b2 = (sh.get(n) for n in ("s_w1", "s_w3", "s_w2", "s_b1", "s_b2"))
    st = lib().moe_forward_noalloc(ctypes.byref(cfg.struct()), _ptr(x), _ptr(w_router), _ptr(logit_bias),
                                   _ptr(sel_bias), _ptr(w1), _ptr(w3), _ptr(b1), _ptr(w2), _ptr(b2), _ptr(s_w1),
                                   _ptr(s_w3), _ptr(s_b1), _ptr(s_w2), _ptr(s_b2), _ptr(out["y"]),
                                   _ptr(out["topk_ids"]), _ptr(out["topk_w"]), _ptr(out["counts"]),
                                   _ptr(out["stats"]), _stream())
    _check(st, "moe_forward_noalloc")
    return out


BWD_EVENTS = 10
BWD_STAGES = ("route_dispatch", "up_recompute", "act_backward", "router_backward", "dx_rows", "dw2", "dw13",
              "shared", "router_dx_combine")
GRAD_NAMES = ("dx", "dw_router", "dw1", "dw3", "db1", "dw2", "db2", "ds_w1", "ds_w3", "ds_b1", "ds_w2", "ds_b2",
              "dz", "dgate")


def moe_backward(cfg: LayerConfig, x, w_router, w1, w3, w2, dy, b1=None, b2=None, logit_bias=None, sel_bias=None,
                 *, shared: Optional[dict] = None, aux_coef: float = 0.0, z_coef: float = 0.0, ws=None, out=None,
                 stage_events: Optional[Sequence[int]] = None, saved: Optional[dict] = None):
    """Gradients of <dy, y> + aux_coef L + z_coef z_loss (bfloat16, dropless). Returns a dict
    with dx, dw_router, dw1, dw3, db1, dw2, db2, the shared expert's ds_* (None where the
    weight is absent), dz [N,E] and dgate [N,k] (float32), and the recomputed routing
    (topk_ids, topk_w, counts, stats). `out` / `ws` may hold preallocated buffers;
    stage_events: BWD_EVENTS raw hipEvent_t handles (ints) or None. saved: the dict a
    moe_forward_train call with the same inputs returned (its workspace and routing outputs
    are reused instead of recomputing routing, dispatch and the up projection)."""
    N, d, E, k, f = cfg.n_tokens, cfg.d_model, cfg.n_experts, cfg.top_k, cfg.d_ff
    T = cfg.torch_dtype
    sh = shared or {}
    s_w1, s_w3, s_w2, s_b1, s_b2 = (sh.get(n) for n in ("s_w1", "s_w3", "s_w2", "s_b1", "s_b2"))
    swi, bias, F = cfg.act == "swiglu", cfg.has_bias, cfg.d_ff_shared
    if out is None:
        _want(x, "x", (N, d), T)
        _want(dy, "dy", (N, d), T)
        _want(w_router, "w_router", (E, d), T)
        _want(w1, "w1", (E, f, d), T)
        _want(w2, "w2", (E, d, f), T)
        _want(w3, "w3", (E, f, d), T, optional=not swi)
        _want(b1, "b1", (E, f), T, optional=not bias)
        _want(b2, "b2", (E, d), T, optional=not bias)
        _want(logit_bias, "logit_bias", (E,), torch.float32, optional=True)
        _want(sel_bias, "sel_bias", (E,), torch.float32, optional=True)
        dev = w_router.device
        new = lambda shape, dt=T: torch.empty(shape, dtype=dt, device=dev)
        out = {
            "dx": new((N, d)), "dw_router": new((E, d)), "dw1": new((E, f, d)), "dw3": new((E, f, d)) if swi else None,
            "db1": new((E, f)) if bias else None, "dw2": new((E, d, f)), "db2": new((E, d)) if bias else None,
            "ds_w1": new((F, d)) if F else None, "ds_w3": new((F, d)) if F and swi else None,
            "ds_b1": new((F,)) if F and bias else None, "ds_w2": new((d, F)) if F else None,
            "ds_b2": new((d,)) if F and bias else None,
            "dz": new((N, E), torch.float32), "dgate": new((N, k), torch.float32),
            "topk_ids": new((N, k), torch.int32), "topk_w": new((N, k), torch.float32),
            "counts": new((E,), torch.int32), "stats": new((2 * E + 2,), torch.float32),
        }
    if saved is not None:
        ws = saved["ws"]
        for name in ("topk_ids", "topk_w", "counts", "stats"):
            out[name] = saved[name]
    if ws is None:
        ws = workspace(cfg, Op.BACKWARD, w_router.device)
    g = MoeGradsStruct(*[None if out.get(n) is None else out[n].data_ptr() for n in GRAD_NAMES])
    ev = None
    if stage_events is not None:
        if len(stage_events) != BWD_EVENTS:
            raise ValueError(f"stage_events needs {BWD_EVENTS} events")
        ev = (ctypes.c_void_p * BWD_EVENTS)(*[ctypes.c_void_p(int(e)) for e in stage_events])
    st = lib().moe_backward(ctypes.byref(cfg.struct()), _ptr(x), _ptr(w_router), _ptr(logit_bias), _ptr(sel_bias),
                            _ptr(w1), _ptr(w3), _ptr(b1), _ptr(w2), _ptr(b2), _ptr(s_w1), _ptr(s_w3), _ptr(s_b1),
                            _ptr(s_w2), _ptr(s_b2), _ptr(dy), float(aux_coef), float(z_coef), ctypes.byref(g),
                            _ptr(out["topk_ids"]), _ptr(out["topk_w"]), _ptr(out["counts"]), _ptr(out["stats"]),
                            1 if saved is not None else 0, _ptr(ws), ws.numel(), ev, _stream())
    _check(st, "moe_backward")
    return out


def moe_forward_train(cfg: LayerConfig, x, w_router, w1, w3, w2, b1=None, b2=None, logit_bias=None, sel_bias=None,
                      *, shared: Optional[dict] = None, ws=None, out=None):
    """The forward for training: returns moe_forward's dict (y, topk_ids, topk_w, counts,
    stats) plus "ws", the backward workspace holding what moe_backward(saved=...) reuses."""
    N, d, E, k = cfg.n_tokens, cfg.d_model, cfg.n_experts, cfg.top_k
    sh = shared or {}
    s_w1, s_w3, s_w2, s_b1, s_b2 = (sh.get(n) for n in ("s_w1", "s_w3", "s_w2", "s_b1", "s_b2"))
    if out is None:
        _want(x, "x", (N, d), cfg.torch_dtype)
        _want(w_router, "w_router", (E, d), cfg.torch_dtype)
        dev = w_router.device
        out = {"y": torch.empty((N, d), dtype=cfg.torch_dtype, device=dev),
               "topk_ids": torch.empty((N, k), dtype=torch.int32, device=dev),
               "topk_w": torch.empty((N, k), dtype=torch.float32, device=dev),
               "counts": torch.empty((E,), dtype=torch.int32, device=dev),
               "stats": torch.empty((2 * E + 2,), dtype=torch.float32, device=dev)}
    if ws is None:
        ws = workspace(cfg, Op.BACKWARD, w_router.device)
    out["ws"] = ws
    st = lib().moe_forward_train(ctypes.byref(cfg.struct()), _ptr(x), _ptr(w_router), _ptr(logit_bias),
                                 _ptr(sel_bias), _ptr(w1), _ptr(w3), _ptr(b1), _ptr(w2), _ptr(b2), _ptr(s_w1),
                                 _ptr(s_w3), _ptr(s_b1), _ptr(s_w2), _ptr(s_b2), _ptr(out["y"]),
                                 _ptr(out["topk_ids"]), _ptr(out["topk_w"]), _ptr(out["counts"]),
                                 _ptr(out["stats"]), _ptr(ws), ws.numel(), _stream())
    _check(st, "moe_forward_train")
    return out


def moe_update_bias(cfg: LayerConfig, counts, sel_bias, rate: float):
    """One aux-free balancing step on sel_bias in place (float32 [E]) from counts (int32 [E])."""
    _want(counts, "counts", (cfg.n_experts,), torch.int32)
    _want(sel_bias, "sel_bias", (cfg.n_experts,), torch.float32)
    st = lib().moe_update_bias(ctypes.byref(cfg.struct()), _ptr(counts), _ptr(sel_bias), float(rate), _stream())
    _check(st, "moe_update_bias")
    return sel_bias


def moe_get_device_error(ws: torch.Tensor) -> int:
    """Synchronises the current stream and returns (and clears) the workspace's device error
    status: MOE_OK, MOE_ERR_BAD_EXPERT_ID or MOE_ERR_INVALID_ARG."""
    return int(lib().moe_get_device_error(_ptr(ws), _stream()))


# HIP events for stage timing, straight from the HIP runtime (torch.cuda.Event only times
# work on torch's streams; these are recorded by the library itself on the call's stream).
_hip = None


def _hiprt():
    global _hip
    if _hip is None:
        for name in ("libamdhip64.so", "libamdhip64.so.7", "/opt/rocm/lib/libamdhip64.so"):
            try:
                _hip = ctypes.CDLL(name)
                break
            except OSError:
                continue
        if _hip is None:
            raise RuntimeError("libamdhip64 not found")
        _hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        _hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        _hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), _P, _P]
        _hip.hipEventSynchronize.argtypes = [_P]
        _hip.hipEventDestroy.argtypes = [_P]
        _hip.hipEventRecord.argtypes = [_P, _P]
    return _hip


# hipEventDisableSystemFence: the event only takes a timestamp. Recording a default event
# also writes back and invalidates the caches (a system-scope fence), which the next kernel
# waits for: about 6 us per stage boundary at the Mixtral shape.
HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000


class HipEvents:
    """A handful of raw hipEvent_t handles, timing enabled. timing_only (the default) creates
    them without the system-scope fence, for events that only measure elapsed time."""

    def __init__(self, n: int, timing_only: bool = True):
        h = _hiprt()
        flags = HIP_EVENT_DISABLE_SYSTEM_FENCE if timing_only else 0
        self.handles = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if h.hipEventCreateWithFlags(ctypes.byref(e), ctypes.c_uint(flags)) != 0:
                raise RuntimeError("hipEventCreateWithFlags failed")
            self.handles.append(e.value)

    def record(self, i: int):
        """Records event i on torch's current stream."""
        if _hiprt().hipEventRecord(ctypes.c_void_p(self.handles[i]), _stream()) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, i: int, j: int) -> float:
        h = _hiprt()
        h.hipEventSynchronize(ctypes.c_void_p(self.handles[j]))
        ms = ctypes.c_float()
        if h.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(self.handles[i]), ctypes.c_void_p(self.handles[j])) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def __del__(self):
        try:
            h = _hiprt()
            for e in self.handles:
                h.hipEventDestroy(ctypes.c_void_p(e))
        except Exception:
            pass
