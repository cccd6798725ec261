// C ABI of the MoE layer forward: host-side validation, workspace carving and the launch
// sequences. Nothing here allocates, frees or synchronises (except moe_get_device_error),
// and no HIP call is made before the first launch, so the library loads without a GPU.
#include <algorithm>
#include <cmath>
#include <cstdint>

#include "moe_internal.h"

using namespace moe;

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// Checks of the configuration itself. needs_ff: the call uses d_ff.
moe_status check_config(const moe_config* c, bool needs_ff) {
  if (!c) return MOE_ERR_INVALID_ARG;
  if (c->n_tokens < 0) return MOE_ERR_INVALID_ARG;
  if (c->n_experts < 1 || c->top_k < 1 || c->top_k > c->n_experts) return MOE_ERR_INVALID_ARG;
  if (c->router < MOE_ROUTER_SOFTMAX_TOPK || c->router > MOE_ROUTER_SIGMOID) return MOE_ERR_INVALID_ARG;
  if (c->act < MOE_ACT_GELU || c->act > MOE_ACT_SWIGLU) return MOE_ERR_INVALID_ARG;
  if (c->dtype != MOE_F32 && c->dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if ((c->norm_topk != 0 && c->norm_topk != 1) || (c->has_bias != 0 && c->has_bias != 1)) return MOE_ERR_INVALID_ARG;
  if (c->has_bias && c->act != MOE_ACT_GELU) return MOE_ERR_INVALID_ARG;
  if (!std::isfinite(c->routed_scaling)) return MOE_ERR_INVALID_ARG;
  if (c->n_experts > kMaxExperts || c->top_k > kMaxTopK) return MOE_ERR_UNSUPPORTED;
  if (c->n_tokens * (long long)c->top_k >= (1ll << 31)) return MOE_ERR_UNSUPPORTED;
  if (c->d_model < 8 || c->d_model > 65536 || c->d_model % 8) return MOE_ERR_UNSUPPORTED;
  if (needs_ff && (c->d_ff < 8 || c->d_ff > 65536 || c->d_ff % 8)) return MOE_ERR_UNSUPPORTED;
  if (c->d_ff_shared < 0) return MOE_ERR_INVALID_ARG;
  if (!std::isfinite(c->capacity_factor) || c->capacity_factor < 0.f) return MOE_ERR_INVALID_ARG;
  if (c->d_ff_shared > 0 && (c->d_ff_shared < 8 || c->d_ff_shared > 65536 || c->d_ff_shared % 8))
    return MOE_ERR_UNSUPPORTED;
  if (c->weight_layout != MOE_WEIGHTS_ROWMAJOR && c->weight_layout != MOE_WEIGHTS_TILED) return MOE_ERR_INVALID_ARG;
  if (c->weight_layout == MOE_WEIGHTS_TILED && c->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// A required tensor of the element type: non-null and 16-byte aligned.
moe_status need_t(const void* p) {
  if (!p) return MOE_ERR_INVALID_ARG;
  return aligned16(p) ? MOE_OK : MOE_ERR_UNSUPPORTED;
}
moe_status opt_t(const void* p) { return (!p || aligned16(p)) ? MOE_OK : MOE_ERR_UNSUPPORTED; }
// A required int32 / float32 tensor: non-null and 4-byte aligned.
moe_status need_4(const void* p) {
  if (!p) return MOE_ERR_INVALID_ARG;
  return aligned4(p) ? MOE_OK : MOE_ERR_UNSUPPORTED;
}
moe_status opt_4(const void* p) { return (!p || aligned4(p)) ? MOE_OK : MOE_ERR_UNSUPPORTED; }

// The shared expert's weights: required iff cfg->d_ff_shared > 0, NULL otherwise.
moe_status check_shared(const moe_config* c, const void* s_w1, const void* s_w3, const void* s_b1,
                        const void* s_w2, const void* s_b2) {
  if (c->d_ff_shared == 0) return (s_w1 || s_w3 || s_b1 || s_w2 || s_b2) ? MOE_ERR_INVALID_ARG : MOE_OK;
  moe_status st;
  if ((st = need_t(s_w1)) != MOE_OK || (st = need_t(s_w2)) != MOE_OK) return st;
  if (c->act == MOE_ACT_SWIGLU) {
    if ((st = need_t(s_w3)) != MOE_OK) return st;
  } else if (s_w3) {
    return MOE_ERR_INVALID_ARG;
  }
  if (c->has_bias) {
    if ((st = need_t(s_b1)) != MOE_OK || (st = need_t(s_b2)) != MOE_OK) return st;
  } else if (s_b1 || s_b2) {
    return MOE_ERR_INVALID_ARG;
  }
  return MOE_OK;
}

// What the backward supports beyond check_config: bfloat16, dropless.
moe_status check_backward_config(const moe_config* c) {
  if (c->dtype != MOE_BF16 || c->capacity_factor != 0.f) return MOE_ERR_UNSUPPORTED;
  if (c->weight_layout != MOE_WEIGHTS_ROWMAJOR) return MOE_ERR_UNSUPPORTED;  // row-major weights only
  return MOE_OK;
}

#define MOE_TRY(expr)                  \
  do {                                 \
    const moe_status s_ = (expr);      \
    if (s_ != MOE_OK) return s_;       \
  } while (0)

// Forward-only buffers placed after the stage regions.
void carve_forward_buffers(const moe_config& c, WsCarver& w, WsLayout* L) {
  const size_t A = (size_t)(c.n_tokens * c.top_k);
  const size_t row = (size_t)c.d_model * elem_size(c);
  int* perm = w.take_t<int>(A);
  int* inv = w.take_t<int>(A);
  int* off = w.take_t<int>((size_t)c.n_experts + 1);
  int* fbase = w.take_t<int>(route_base_ints(c));
  int* kept = w.take_t<int>((size_t)c.n_experts);
  float* gs = w.take_t<float>(A);
  // x_sorted: row-major, or tiled (forward_xs_kp) over A rounded up to 128 rows
  const size_t xs_tiled = forward_xs_kp(c) > 0 ? (A + kTiledRows - 1) / kTiledRows * kTiledRows *
                                                     (size_t)forward_xs_kp(c) * elem_size(c) : 0;
  void* xs = w.take(std::max(A * row, xs_tiled));
  void* ys = w.take(A * row);
  if (L) {
    L->perm = perm;
    L->inv_perm = inv;
    L->offsets = off;
    L->fbase = fbase;
    L->kept = kept;
    L->gate_sorted = gs;
    L->x_sorted = xs;
    L->y_sorted = ys;
  }
}

size_t layout(const moe_config& c, int op, char* base, WsLayout* L) {
  WsCarver w(base);
  int* err = w.take_t<int>(kErrWordBytes / sizeof(int));
  if (L) {
    L->base = base;
    L->err = err;
  }
  switch (op) {
    case MOE_OP_ROUTE: carve_route(c, w, L); break;
    case MOE_OP_DISPATCH: carve_dispatch(c, w, L); break;
    case MOE_OP_EXPERT_FFN: carve_ffn(c, w, L); break;
    case MOE_OP_COMBINE: break;
    case MOE_OP_SHARED_FFN: carve_ffn(c, w, L); break;
    case MOE_OP_FORWARD:
      carve_route(c, w, L);
      carve_dispatch(c, w, L);  // the capacity-factor dispatch's scratch
      carve_ffn(c, w, L);
      carve_forward_buffers(c, w, L);
      break;
    case MOE_OP_BACKWARD:
      carve_route(c, w, L);
      carve_ffn(c, w, L);
      carve_forward_buffers(c, w, L);
      carve_backward(c, w, L);
      break;
    default: return 0;
  }
  return w.used();
}

moe_status check_ws(const moe_config& c, int op, void* ws, size_t ws_bytes, WsLayout* L) {
  if (!ws || !aligned16(ws)) return MOE_ERR_WORKSPACE;
  const size_t need = layout(c, op, nullptr, nullptr);
  if (ws_bytes < need) return MOE_ERR_WORKSPACE;
  layout(c, op, static_cast<char*>(ws), L);
  return MOE_OK;
}

moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

}  // namespace

extern "C" {

size_t moe_workspace_size(const moe_config* cfg, int op) {
  const bool needs_ff = op == MOE_OP_EXPERT_FFN || op == MOE_OP_FORWARD || op == MOE_OP_SHARED_FFN ||
                        op == MOE_OP_BACKWARD;
  if (op < MOE_OP_ROUTE || op > MOE_OP_BACKWARD) return 0;
  if (check_config(cfg, needs_ff) != MOE_OK) return 0;
  if (op == MOE_OP_SHARED_FFN && cfg->d_ff_shared <= 0) return 0;
  if (op == MOE_OP_BACKWARD && check_backward_config(cfg) != MOE_OK) return 0;
  return layout(*cfg, op, nullptr, nullptr);
}

moe_status moe_route(const moe_config* cfg, const void* x, const void* w_router,
                     const float* logit_bias, const float* sel_bias, int32_t* topk_ids,
                     float* topk_w, int32_t* counts, float* stats, float* logits_out,
                     float* gap_out, void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(check_config(cfg, false));
  const bool has_tokens = cfg->n_tokens > 0;
  if (has_tokens) {
    MOE_TRY(need_t(x));
    MOE_TRY(need_4(topk_ids));
    MOE_TRY(need_4(topk_w));
  }
  MOE_TRY(need_t(w_router));
  MOE_TRY(need_4(counts));
  MOE_TRY(need_4(stats));
  MOE_TRY(opt_4(logit_bias));
  MOE_TRY(opt_4(sel_bias));
  MOE_TRY(opt_4(logits_out));
  MOE_TRY(opt_4(gap_out));
  WsLayout L{};
  MOE_TRY(check_ws(*cfg, MOE_OP_ROUTE, ws, ws_bytes, &L));
  return hip_status(launch_route(*cfg, L, x, w_router, logit_bias, sel_bias, topk_ids, topk_w, counts,
                                 stats, logits_out, gap_out, false, static_cast<hipStream_t>(stream)));
}

moe_status moe_dispatch(const moe_config* cfg, const void* x, const int32_t* topk_ids,
                        const float* topk_w, void* x_sorted, int32_t* perm, int32_t* inv_perm,
                        int32_t* counts, int32_t* offsets, float* gate_sorted,
                        void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(check_config(cfg, false));
  if (cfg->n_tokens > 0) {
    MOE_TRY(need_4(topk_ids));
    MOE_TRY(need_4(perm));
    MOE_TRY(need_4(inv_perm));
    MOE_TRY(opt_t(x_sorted));
    if (x_sorted) MOE_TRY(need_t(x));
    MOE_TRY(opt_4(topk_w));
    MOE_TRY(opt_4(gate_sorted));
  }
  MOE_TRY(need_4(counts));
  MOE_TRY(need_4(offsets));
  WsLayout L{};
  MOE_TRY(check_ws(*cfg, MOE_OP_DISPATCH, ws, ws_bytes, &L));
  return hip_status(launch_dispatch(*cfg, L, x, topk_ids, topk_w, x_sorted, perm, inv_perm, counts, offsets,
                                    gate_sorted, static_cast<hipStream_t>(stream)));
}

int64_t moe_expert_capacity(int32_t top_k, float capacity_factor, int64_t n_tokens, int32_t n_experts) {
  moe_config c{};
  c.top_k = top_k;
  c.n_tokens = n_tokens;
  c.n_experts = n_experts > 0 ? n_experts : 1;
  return expert_capacity(c, capacity_factor);
}

moe_status moe_dispatch_capacity(const moe_config* cfg, float capacity_factor, const void* x,
                                 const int32_t* topk_ids, const float* topk_w, void* x_kept,
                                 int32_t* perm_kept, int32_t* slot, int32_t* kept, int32_t* offsets,
                                 float* gate_kept, void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(check_config(cfg, false));
  if (!std::isfinite(capacity_factor) || capacity_factor < 0.f) return MOE_ERR_INVALID_ARG;
  if (cfg->n_tokens > 0) {
    MOE_TRY(need_4(topk_ids));
    MOE_TRY(need_4(slot));
    MOE_TRY(opt_4(perm_kept));
    MOE_TRY(opt_t(x_kept));
    if (x_kept) MOE_TRY(need_t(x));
    MOE_TRY(opt_4(topk_w));
    MOE_TRY(opt_4(gate_kept));
  }
  MOE_TRY(need_4(kept));
  MOE_TRY(need_4(offsets));
  WsLayout L{};
  MOE_TRY(check_ws(*cfg, MOE_OP_DISPATCH, ws, ws_bytes, &L));
  return hip_status(launch_dispatch_capacity(*cfg, L, capacity_factor, x, topk_ids, topk_w, x_kept, perm_kept, slot,
                                             kept, offsets, gate_kept, static_cast<hipStream_t>(stream)));
}

moe_status moe_expert_ffn(const moe_config* cfg, const void* x_sorted, const int32_t* offsets,
                          const void* w1, const void* w3, const void* b1, const void* w2,
                          const void* b2, const float* gate_sorted, void* y_sorted, void* ws,
                          size_t ws_bytes, void* stream) {
  MOE_TRY(check_config(cfg, true));
  MOE_TRY(need_4(offsets));
  MOE_TRY(need_t(w1));
  MOE_TRY(need_t(w2));
  if (cfg->act == MOE_ACT_SWIGLU) MOE_TRY(need_t(w3));
  if (cfg->has_bias) {
    MOE_TRY(need_t(b1));
    MOE_TRY(need_t(b2));
  }
  if (cfg->n_tokens > 0) {
    MOE_TRY(need_t(x_sorted));
    MOE_TRY(need_t(y_sorted));
    MOE_TRY(opt_4(gate_sorted));
  }
  WsLayout L{};
  MOE_TRY(check_ws(*cfg, MOE_OP_EXPERT_FFN, ws, ws_bytes, &L));
  hipStream_t s = static_cast<hipStream_t>(stream);
  MOE_TRY(hip_status(launch_ffn_tiles(*cfg, L, offsets, s)));
  MOE_TRY(hip_status(launch_ffn_up(*cfg, L, x_sorted, offsets, w1, w3, b1, s)));
  return hip_status(launch_ffn_down(*cfg, L, offsets, w2, b2, gate_sorted, y_sorted, s));
}

moe_status moe_combine(const moe_config* cfg, const void* y_sorted, const float* topk_w,
                       const int32_t* inv_perm, const void* y_add, void* y, void* stream) {
  MOE_TRY(check_config(cfg, false));
  if (cfg->n_tokens > 0) {
    MOE_TRY(need_t(y_sorted));
    MOE_TRY(need_4(inv_perm));
    MOE_TRY(need_t(y));
    MOE_TRY(opt_4(topk_w));
    MOE_TRY(opt_t(y_add));
  }
  return hip_status(launch_combine(*cfg, y_sorted, topk_w, inv_perm, y_add, y, static_cast<hipStream_t>(stream)));
}

moe_status moe_shared_ffn(const moe_config* cfg, const void* x, const void* s_w1, const void* s_w3,
                          const void* s_b1, const void* s_w2, const void* s_b2, void* y_shared,
                          void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(check_config(cfg, true));
  if (cfg->d_ff_shared <= 0) return MOE_ERR_INVALID_ARG;
  MOE_TRY(check_shared(cfg, s_w1, s_w3, s_b1, s_w2, s_b2));
  if (cfg->n_tokens > 0) {
    MOE_TRY(need_t(x));
    MOE_TRY(need_t(y_shared));
  }
  WsLayout L{};
  MOE_TRY(check_ws(*cfg, MOE_OP_SHARED_FFN, ws, ws_bytes, &L));
  return hip_status(launch_shared(*cfg, L, x, s_w1, s_w3, s_b1, s_w2, s_b2, y_shared,
                                  static_cast<hipStream_t>(stream)));
}

moe_status moe_forward(const moe_config* cfg, const void* x, const void* w_router,
                       const float* logit_bias, const float* sel_bias, const void* w1,
                       const void* w3, const void* b1, const void* w2, const void* b2,
                       const void* s_w1, const void* s_w3, const void* s_b1, const void* s_w2,
                       const void* s_b2, void* y, int32_t* topk_ids, float* topk_w, int32_t* counts,
                       float* stats, int32_t* perm_out, int32_t* inv_perm_out, int32_t* offsets_out, void* ws,
                       size_t ws_bytes, void* const* stage_events, void* stream) {
  MOE_TRY(check_config(cfg, true));
  MOE_TRY(check_shared(cfg, s_w1, s_w3, s_b1, s_w2, s_b2));
  MOE_TRY(opt_4(perm_out));
  MOE_TRY(opt_4(inv_perm_out));
  MOE_TRY(opt_4(offsets_out));
  if (cfg->n_tokens > 0) {
    MOE_TRY(need_t(x));
    MOE_TRY(need_t(y));
    MOE_TRY(need_4(topk_ids));
    MOE_TRY(need_4(topk_w));
  }
  MOE_TRY(need_t(w_router));
  MOE_TRY(need_t(w1));
  MOE_TRY(need_t(w2));
  if (cfg->act == MOE_ACT_SWIGLU) MOE_TRY(need_t(w3));
  if (cfg->has_bias) {
    MOE_TRY(need_t(b1));
    MOE_TRY(need_t(b2));
  }
  MOE_TRY(need_4(counts));
  MOE_TRY(need_4(stats));
  MOE_TRY(opt_4(logit_bias));
  MOE_TRY(opt_4(sel_bias));
  if (stage_events)
    for (int i = 0; i < 6; ++i)
      if (!stage_events[i]) return MOE_ERR_INVALID_ARG;
  WsLayout L{};
  MOE_TRY(check_ws(*cfg, MOE_OP_FORWARD, ws, ws_bytes, &L));
  // dispatch arrays the caller asked for are written in place of the workspace's copies
  if (perm_out) L.perm = perm_out;
  if (inv_perm_out) L.inv_perm = inv_perm_out;
  if (offsets_out) L.offsets = offsets_out;
  hipStream_t s = static_cast<hipStream_t>(stream);
  auto mark = [&](int i) -> moe_status {
    if (!stage_events) return MOE_OK;
    return hip_status(hipEventRecord(static_cast<hipEvent_t>(stage_events[i]), s));
  };
  MOE_TRY(mark(0));
  // Routing's final reduction also writes offsets, the per-block dispatch bases and the
  // m-tile table, so dispatch is a scatter and a row copy.
  MOE_TRY(hip_status(launch_route(*cfg, L, x, w_router, logit_bias, sel_bias, topk_ids, topk_w, counts, stats,
                                  nullptr, nullptr, cfg->capacity_factor <= 0.f, s)));
  MOE_TRY(mark(1));
  if (cfg->capacity_factor > 0.f) {
    // capacity-factor dispatch: k-major ranking, drops; the tile table follows the kept slices
    MOE_TRY(hip_status(launch_dispatch_capacity(*cfg, L, cfg->capacity_factor, x, topk_ids, topk_w, L.x_sorted,
                                                L.perm, L.inv_perm, L.kept, L.offsets, L.gate_sorted, s)));
    MOE_TRY(hip_status(launch_ffn_tiles(*cfg, L, L.offsets, s)));
  } else {
    MOE_TRY(hip_status(launch_dispatch_scanned(*cfg, L, x, topk_ids, topk_w, L.x_sorted, L.perm, L.inv_perm,
                                               L.gate_sorted, s, forward_xs_kp(*cfg))));
  }
  MOE_TRY(mark(2));
  // x_sorted is tiled on the dropless bf16 path (forward_xs_kp), row-major after a capacity dispatch
  MOE_TRY(hip_status(launch_ffn_up(*cfg, L, L.x_sorted, L.offsets, w1, w3, b1, s, forward_xs_kp(*cfg))));
  MOE_TRY(mark(3));
  MOE_TRY(hip_status(launch_ffn_down(*cfg, L, L.offsets, w2, b2, L.gate_sorted, L.y_sorted, s)));
  // Shared(x) of the output equation: its output lands in x_sorted, free after the routed up
  // projection (A >= N rows), and the combine adds it with weight 1.
  const bool shared = cfg->d_ff_shared > 0;
  if (shared) MOE_TRY(hip_status(launch_shared(*cfg, L, x, s_w1, s_w3, s_b1, s_w2, s_b2, L.x_sorted, s)));
  MOE_TRY(mark(4));
  MOE_TRY(hip_status(launch_combine(*cfg, L.y_sorted, nullptr, L.inv_perm, shared ? L.x_sorted : nullptr, y, s)));
  return mark(5);
}

moe_status moe_backward(const moe_config* cfg, const void* x, const void* w_router, const float* logit_bias,
                        const float* sel_bias, const void* w1, const void* w3, const void* b1, const void* w2,
                        const void* b2, const void* s_w1, const void* s_w3, const void* s_b1, const void* s_w2,
                        const void* s_b2, const void* dy, float aux_coef, float z_coef, const moe_grads* grads,
                        int32_t* topk_ids, float* topk_w, int32_t* counts, float* stats, int saved, void* ws,
                        size_t ws_bytes, void* const* stage_events, void* stream) {
  MOE_TRY(check_config(cfg, true));
  MOE_TRY(check_backward_config(cfg));
  MOE_TRY(check_shared(cfg, s_w1, s_w3, s_b1, s_w2, s_b2));
  if (!grads || !std::isfinite(aux_coef) || !std::isfinite(z_coef)) return MOE_ERR_INVALID_ARG;
  if (saved != 0 && saved != 1) return MOE_ERR_INVALID_ARG;
  const moe_grads& g = *grads;
  if (cfg->n_tokens > 0) {
    MOE_TRY(need_t(x));
    MOE_TRY(need_t(dy));
    MOE_TRY(need_t(g.dx));
    MOE_TRY(need_4(topk_ids));
    MOE_TRY(need_4(topk_w));
  }
  MOE_TRY(need_t(w_router));
  MOE_TRY(need_t(w1));
  MOE_TRY(need_t(w2));
  MOE_TRY(need_t(g.dw_router));
  MOE_TRY(need_t(g.dw1));
  MOE_TRY(need_t(g.dw2));
  const bool swi = cfg->act == MOE_ACT_SWIGLU;
  if (swi) {
    MOE_TRY(need_t(w3));
    MOE_TRY(need_t(g.dw3));
  } else if (g.dw3) {
    return MOE_ERR_INVALID_ARG;
  }
  if (cfg->has_bias) {
    MOE_TRY(need_t(b1));
    MOE_TRY(need_t(b2));
    MOE_TRY(need_t(g.db1));
    MOE_TRY(need_t(g.db2));
  } else if (g.db1 || g.db2) {
    return MOE_ERR_INVALID_ARG;
  }
  // the shared expert's gradients follow its weights
  MOE_TRY(check_shared(cfg, g.ds_w1, g.ds_w3, g.ds_b1, g.ds_w2, g.ds_b2));
  MOE_TRY(need_4(counts));
  MOE_TRY(need_4(stats));
  MOE_TRY(opt_4(logit_bias));
  MOE_TRY(opt_4(sel_bias));
  MOE_TRY(opt_4(g.dz));
  MOE_TRY(opt_4(g.dgate));
  if (stage_events)
    for (int i = 0; i < MOE_BWD_EVENTS; ++i)
      if (!stage_events[i]) return MOE_ERR_INVALID_ARG;
  WsLayout L{};
  MOE_TRY(check_ws(*cfg, MOE_OP_BACKWARD, ws, ws_bytes, &L));
  BwdIn in{x, w_router, logit_bias, sel_bias, w1, w3, b1, w2, b2, s_w1, s_w3, s_b1, s_w2, s_b2, dy, aux_coef, z_coef};
  RouteOut ro{topk_ids, topk_w, counts, stats};
  return hip_status(launch_backward(*cfg, L, in, g, ro, saved == 1, stage_events, static_cast<hipStream_t>(stream)));
}

moe_status moe_forward_train(const moe_config* cfg, const void* x, const void* w_router, const float* logit_bias,
                             const float* sel_bias, const void* w1, const void* w3, const void* b1, const void* w2,
                             const void* b2, const void* s_w1, const void* s_w3, const void* s_b1, const void* s_w2,
                             const void* s_b2, void* y, int32_t* topk_ids, float* topk_w, int32_t* counts, float* stats,
                             void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(check_config(cfg, true));
  MOE_TRY(check_backward_config(cfg));
  MOE_TRY(check_shared(cfg, s_w1, s_w3, s_b1, s_w2, s_b2));
  if (cfg->n_tokens > 0) {
    MOE_TRY(need_t(x));
    MOE_TRY(need_t(y));
    MOE_TRY(need_4(topk_ids));
    MOE_TRY(need_4(topk_w));
  }
  MOE_TRY(need_t(w_router));
  MOE_TRY(need_t(w1));
  MOE_TRY(need_t(w2));
  if (cfg->act == MOE_ACT_SWIGLU) MOE_TRY(need_t(w3));
  if (cfg->has_bias) {
    MOE_TRY(need_t(b1));
    MOE_TRY(need_t(b2));
  }
  MOE_TRY(need_4(counts));
  MOE_TRY(need_4(stats));
  MOE_TRY(opt_4(logit_bias));
  MOE_TRY(opt_4(sel_bias));
  WsLayout L{};
  MOE_TRY(check_ws(*cfg, MOE_OP_BACKWARD, ws, ws_bytes, &L));
  BwdIn in{x, w_router, logit_bias, sel_bias, w1, w3, b1, w2, b2, s_w1, s_w3, s_b1, s_w2, s_b2, nullptr, 0.f, 0.f};
  RouteOut ro{topk_ids, topk_w, counts, stats};
  return hip_status(launch_forward_train(*cfg, L, in, y, ro, static_cast<hipStream_t>(stream)));
}

size_t moe_packed_weight_size(const moe_config* cfg, int which) {
  if (check_config(cfg, true) != MOE_OK || cfg->dtype != MOE_BF16 || (which != 0 && which != 1)) return 0;
  return packed_weight_elems(*cfg, which) * 2;
}

moe_status moe_pack_weights(const moe_config* cfg, int which, const void* w, void* w_tiled, void* stream) {
  MOE_TRY(check_config(cfg, true));
  if (which != 0 && which != 1) return MOE_ERR_INVALID_ARG;
  if (cfg->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  MOE_TRY(need_t(w));
  MOE_TRY(need_t(w_tiled));
  const size_t src_bytes = (size_t)cfg->n_experts * cfg->d_ff * cfg->d_model * 2;
  const size_t dst_bytes = packed_weight_elems(*cfg, which) * 2;
  const uintptr_t a = reinterpret_cast<uintptr_t>(w), b = reinterpret_cast<uintptr_t>(w_tiled);
  if (a < b + dst_bytes && b < a + src_bytes) return MOE_ERR_INVALID_ARG;  // overlapping buffers
  return hip_status(launch_pack_weights(*cfg, which, w, w_tiled, static_cast<hipStream_t>(stream)));
}

moe_status moe_update_bias(const moe_config* cfg, const int32_t* counts, float* sel_bias, float rate,
                           void* stream) {
  MOE_TRY(check_config(cfg, false));
  MOE_TRY(need_4(counts));
  MOE_TRY(need_4(sel_bias));
  if (!std::isfinite(rate)) return MOE_ERR_INVALID_ARG;
  return hip_status(launch_update_bias(*cfg, counts, sel_bias, rate, static_cast<hipStream_t>(stream)));
}

moe_status moe_get_device_error(void* ws, void* stream) {
  if (!ws) return MOE_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int v = 0;
  const int zero = 0;
  if (hipMemcpyAsync(&v, ws, sizeof(int), hipMemcpyDeviceToHost, s) != hipSuccess) return MOE_ERR_HIP;
  if (hipStreamSynchronize(s) != hipSuccess) return MOE_ERR_HIP;
  if (hipMemcpyAsync(ws, &zero, sizeof(int), hipMemcpyHostToDevice, s) != hipSuccess) return MOE_ERR_HIP;
  if (hipStreamSynchronize(s) != hipSuccess) return MOE_ERR_HIP;
  if (v == MOE_ERR_BAD_EXPERT_ID || v == MOE_ERR_INVALID_ARG) return static_cast<moe_status>(v);
  return MOE_OK;
}

const char* moe_status_string(moe_status status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported size or alignment";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_BAD_EXPERT_ID: return "expert id out of range";
    case MOE_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

}  // extern "C"
