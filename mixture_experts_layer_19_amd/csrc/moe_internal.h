// Internal declarations shared by the kernel sources and the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe.h"
#include "moe_common.h"

namespace moe {

constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 32;
constexpr size_t kErrWordBytes = 256;  // the device error word lives at the start of every workspace
constexpr size_t kWsAlign = 256;

// Carves 256-byte aligned regions out of a workspace; with a null base it only sizes.
struct WsCarver {
  char* base;
  size_t off = 0;
  explicit WsCarver(char* b) : base(b) {}
  void* take(size_t bytes) {
    off = (off + kWsAlign - 1) / kWsAlign * kWsAlign;
    void* p = base ? base + off : nullptr;
    off += bytes;
    return p;
  }
  template <typename U> U* take_t(size_t n) { return static_cast<U*>(take(n * sizeof(U))); }
  size_t used() const { return (off + kWsAlign - 1) / kWsAlign * kWsAlign; }
};

// Every region a call may use; only the ones its op carves are set.
struct WsLayout {
  char* base = nullptr;
  int* err = nullptr;
  // routing
  float* zpart = nullptr;
  float* part_p = nullptr;
  int* part_hist = nullptr;
  float* part_zl = nullptr;
  // dispatch
  int* d_hist = nullptr;   // [blocks][E] per-block counts
  int* d_base = nullptr;   // [blocks][E] first sorted slot of each block's run of expert e
  int* d_bad = nullptr;    // [blocks] out-of-range id seen
  // expert FFN
  int* tiles = nullptr;    // [1 + max_tiles][4]: count, then (expert, first row, rows) per m-tile
  void* h = nullptr;       // [A][d_ff] T
  // forward intermediates
  int* perm = nullptr;
  int* inv_perm = nullptr;
  int* offsets = nullptr;
  int* counts_tmp = nullptr;
  float* gate_sorted = nullptr;
  void* x_sorted = nullptr;
  void* y_sorted = nullptr;
};

struct RoutePlan {
  int tokens_per_wave, tokens_per_block, n_blocks;
  int n_split, k_chunk;
};

struct RouteArgs {
  const float* zpart;
  int n_split;
  const float* logit_bias;
  const float* sel_bias;
  int n_tokens, n_experts, top_k, router, norm_topk;
  float routed_scaling;
  int tokens_per_wave, tokens_per_block;
  int32_t* topk_ids;
  float* topk_w;
  float* logits_out;
  float* gap_out;
  float* part_p;
  int* part_hist;
  float* part_zl;
};

inline size_t elem_size(const moe_config& c) { return c.dtype == MOE_BF16 ? 2 : 4; }

// Workspace carving per stage (appends regions to w and fills L when non-null).
void carve_route(const moe_config& c, WsCarver& w, WsLayout* L);
void carve_dispatch(const moe_config& c, WsCarver& w, WsLayout* L);
void carve_ffn(const moe_config& c, WsCarver& w, WsLayout* L);

RoutePlan plan_route(const moe_config& c);

// Launch sequences; none of them synchronises.
hipError_t launch_route(const moe_config& c, const WsLayout& L, const void* x, const void* w_router,
                        const float* logit_bias, const float* sel_bias, int32_t* topk_ids,
                        float* topk_w, int32_t* counts, float* stats, float* logits_out,
                        float* gap_out, hipStream_t stream);
hipError_t launch_dispatch(const moe_config& c, const WsLayout& L, const void* x,
                           const int32_t* topk_ids, const float* topk_w, void* x_sorted,
                           int32_t* perm, int32_t* inv_perm, int32_t* counts, int32_t* offsets,
                           float* gate_sorted, hipStream_t stream);
// Builds the per-call m-tile list from offsets (must precede the up and down launches).
hipError_t launch_ffn_tiles(const moe_config& c, const WsLayout& L, const int32_t* offsets, hipStream_t stream);
hipError_t launch_ffn_up(const moe_config& c, const WsLayout& L, const void* x_sorted,
                         const int32_t* offsets, const void* w1, const void* w3, const void* b1,
                         hipStream_t stream);
hipError_t launch_ffn_down(const moe_config& c, const WsLayout& L, const int32_t* offsets,
                           const void* w2, const void* b2, const float* gate_sorted,
                           void* y_sorted, hipStream_t stream);
hipError_t launch_combine(const moe_config& c, const void* y_sorted, const float* topk_w,
                          const int32_t* inv_perm, void* y, hipStream_t stream);

}  // namespace moe
