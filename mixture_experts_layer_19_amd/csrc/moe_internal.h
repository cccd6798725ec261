// Internal declarations shared by the kernel sources and the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe.h"
#include "moe_common.h"
#include "gemm_sched.h"

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
  int* d_offs_all = nullptr;  // [E] capacity dispatch: exclusive scan of all assignments
  int* d_koff = nullptr;      // [E] capacity dispatch: exclusive scan of the kept counts
  // expert FFN
  int* tiles = nullptr;    // m-tile table (kTileHdr + kTileInts per tile ints)
  void* h = nullptr;       // [A][d_ff] T
  float* tail_part = nullptr;  // down projection's tail: K-piece partials (or null: no split)
  // forward intermediates
  int* perm = nullptr;
  int* inv_perm = nullptr;
  int* offsets = nullptr;
  int* fbase = nullptr;    // [route blocks][E] dispatch bases from the routing histograms
  int* kept = nullptr;     // [E] kept rows per expert (capacity-factor dispatch in moe_forward)
  float* gate_sorted = nullptr;
  void* x_sorted = nullptr;
  void* y_sorted = nullptr;
  // backward (its own regions; see carve_backward)
  void* bwd = nullptr;
};

// Exclusive prefix sum of v over the lanes of one wave in lane order, and the wave's total in
// *total, with no LDS; every lane of the wave calls it. The inclusive scan is six DPP moves: row_shr 1, 2, 4, 8 within each row of 16 lanes (lanes
// with no source add the 0 passed as `old`), then row_bcast 15 (lane 15 of rows 0 and 2 into
// rows 1 and 3) and row_bcast 31 (lane 31 into rows 2 and 3). Each is a register move of a
// few cycles, where a shuffle is an LDS-unit permute of about a hundred; the routing
// finalize chains a dozen of these scans.
MOE_DEV int wave_incl_scan(int v) {
  int x = v;
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15, rows 1 and 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31, rows 2 and 3
  return x;
}
MOE_DEV int wave_excl_scan(int v, int* total) {
  const int x = wave_incl_scan(v);
  *total = __builtin_amdgcn_readlane(x, 63);
  return x - v;
}

// Exclusive prefix sum of v over the threads of the block in thread order (threads without
// a value pass 0), and the block's total in *total. Every thread of the block calls it; the
// block size is a multiple of 64. An inclusive scan within each wave (DPP moves), then each
// thread adds the totals of the waves before its own: two barriers at any block size.
// s_tmp: one int per wave.
MOE_DEV int block_excl_scan(int v, int* s_tmp, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int x = wave_incl_scan(v);
  if (lane == 63) s_tmp[wave] = x;
  __syncthreads();
  int before = 0, all = 0;
  for (int w = 0; w < nw; ++w) {
    const int t = s_tmp[w];
    before += w < wave ? t : 0;
    all += t;
  }
  __syncthreads();
  *total = all;
  return before + x - v;
}

// The same over the first E threads (v = 0 beyond), with E <= blockDim.x (s_tmp: one int per
// wave). Every thread of the block calls it and receives *total. (Up to 64 experts this was a
// step-doubling scan through LDS, log2 E steps of two barriers, while the in-wave scan was
// made of shuffles; with DPP moves the two-barrier block scan is shorter at every E.)
MOE_DEV int expert_excl_scan(int v, int E, int* s_tmp, int* total) {
  return block_excl_scan(threadIdx.x < E ? v : 0, s_tmp, total);
}


// The m-tile table, filled by E owners: the caller with e < E owns expert e, whose rows are
// [lo, hi); callers with e >= E only join the scans. Ranges outside [0, rows] or decreasing
// are clamped and the list is capped at max_tiles (so no access leaves the buffers); the
// return value says whether this caller met either. An expert's rows are cut into m-tiles of
// bm rows; a last tile of at most `narrow` rows (0: none) is narrow. scan(v, &total) is an
// exclusive prefix sum over the experts in order that every caller makes alike.
template <class Scan>
MOE_DEV bool tile_table_fill(int e, int lo, int hi, int E, int rows, int bm, int narrow, int max_tiles, int* tiles,
                             Scan scan) {
  bool bad = false;
  if (e < 4) tiles[4 + e] = 0;
  int n = 0, n_nar = 0;
  if (e < E) {
    if (lo < 0 || hi > rows || hi < lo || (e == 0 && lo != 0)) bad = true;
    lo = min(max(lo, 0), rows);
    hi = min(max(hi, lo), rows);
    n = (hi - lo + bm - 1) / bm;
    n_nar = (n > 0 && hi - lo - (n - 1) * bm <= narrow) ? 1 : 0;
  }
  int total, total_full, total_nar;
  const int start = scan(n, &total);
  const int fstart = scan(n - n_nar, &total_full);
  const int nstart = scan(n_nar, &total_nar);
  int* fmap = tiles + kTileHdr + kTileInts * max_tiles;
  int* nmap = fmap + max_tiles;
  if (e < E) {
    const int n_full = n - n_nar;
    for (int t = 0; t < n && start + t < max_tiles; ++t) {
      const int r0 = lo + t * bm;
      int* q = tiles + kTileHdr + kTileInts * (start + t);
      q[0] = e;
      q[1] = r0;
      q[2] = min(bm, hi - r0);
      q[3] = start;
      q[4] = min(n, max_tiles - start);
      q[5] = fstart;
      q[6] = max(0, min(n_full, max_tiles - fstart));
      if (t < n_full && fstart + t < max_tiles) fmap[fstart + t] = start + t;
    }
    if (n_nar && nstart < max_tiles && start + n - 1 < max_tiles) nmap[nstart] = start + n - 1;
    if (e == E - 1) {
      if (total > max_tiles) bad = true;
      // with a clamped list every kept m-tile is counted full (their narrow entries may be gone)
      const bool ok = total <= max_tiles;
      tiles[0] = min(total, max_tiles);
      tiles[1] = ok ? total_full : min(total, max_tiles);
      tiles[2] = kTileHdr + kTileInts * max_tiles;
      tiles[3] = kTileHdr + (kTileInts + 1) * max_tiles;
    }
  }
  return bad;
}

// The tile table from one workgroup of at least E threads (thread e owns expert e); sets *bad
// (LDS) on a clamped range or list. s_scan: kMaxExperts ints of LDS. Every thread of the
// block calls it.
MOE_DEV void build_tile_table(int lo, int hi, int E, int rows, int bm, int narrow, int max_tiles, int* tiles,
                              int* s_scan, int* bad) {
  const int e = threadIdx.x;
  auto scan = [&](int v, int* total) -> int { return expert_excl_scan(e < E ? v : 0, E, s_scan, total); };
  if (tile_table_fill(e, lo, hi, E, rows, bm, narrow, max_tiles, tiles, scan)) *bad = 1;
  __syncthreads();
}

// The same from the 64 lanes of one wave (E <= 64, lane e owns expert e), with no barrier;
// returns whether any lane met a clamped range or list.
MOE_DEV bool build_tile_table_wave(int lo, int hi, int E, int rows, int bm, int narrow, int max_tiles, int* tiles) {
  const int e = threadIdx.x & 63;
  auto scan = [&](int v, int* total) -> int { return wave_excl_scan(e < E ? v : 0, total); };
  return __ballot(tile_table_fill(e, lo, hi, E, rows, bm, narrow, max_tiles, tiles, scan)) != 0;
}

// Routing launch shape. A token is handled by a group of lpt lanes (a power of two: E rounded
// up to one for E <= 64; else 8 to 64, chosen by plan_route from E, k and the token count),
// each lane holding epl experts, so a wave routes 64/lpt tokens at once; tokens_per_wave is a
// multiple of 64/lpt.
struct RoutePlan {
  bool fused;  // bfloat16 with up to 64 experts: projection and routing in one launch
  int lpt, epl;
  int tokens_per_wave, tokens_per_block, n_blocks;
  int n_split, k_chunk;
};

// Final reduction of the routing partials; optionally (moe_forward) also the dispatch scan
// over the same token blocks and the grouped-GEMM tile table.
struct FinalizeArgs {
  const float* part_p;
  const int* part_hist;
  const float* part_zl;
  int n_blocks;
  long long n_tokens;
  int n_experts;
  int32_t* counts;
  float* stats;
  int* offsets;   // [E+1] or null: no dispatch scan
  int* base;      // [n_blocks][E] first sorted slot of each block's run of each expert
  int* err;       // device error word (written 0: routed ids are always valid)
  int* tiles;     // tile table or null
  int tile_bm, tile_narrow, max_tiles;
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
size_t route_base_ints(const moe_config& c);
int route_tokens_per_block(const moe_config& c);

// Launch sequences; none of them synchronises.
// fuse_dispatch (moe_forward): the final routing reduction also writes L.offsets, L.fbase and
// the tile table L.tiles, so dispatch runs only its scatter and copy (launch_dispatch_scanned).
hipError_t launch_route(const moe_config& c, const WsLayout& L, const void* x, const void* w_router,
                        const float* logit_bias, const float* sel_bias, int32_t* topk_ids,
                        float* topk_w, int32_t* counts, float* stats, float* logits_out,
                        float* gap_out, bool fuse_dispatch, hipStream_t stream);
hipError_t launch_dispatch_scanned(const moe_config& c, const WsLayout& L, const void* x,
                                   const int32_t* topk_ids, const float* topk_w, void* x_sorted,
                                   int32_t* perm, int32_t* inv_perm, float* gate_sorted, hipStream_t stream,
                                   int xs_kp = 0);
int ffn_tile_rows(const moe_config& c);
// rows at or below which an expert's last m-tile is narrow (0: no narrow tiles)
int ffn_narrow_rows(const moe_config& c);
// Tiled weights (MOE_WEIGHTS_TILED): rows per block and reduction elements per slab, the
// padded sizes of weight `which` (0: W1 / W3, N = d_ff, K = d; 1: W2, N = d, K = d_ff), its
// element count, and the re-layout kernel.
inline int tiled_n(const moe_config& c, int which) { return ((which ? c.d_model : c.d_ff) + kTiledRows - 1) / kTiledRows * kTiledRows; }
inline int tiled_k(const moe_config& c, int which) { return ((which ? c.d_ff : c.d_model) + kTiledK - 1) / kTiledK * kTiledK; }
inline size_t packed_weight_elems(const moe_config& c, int which) {
  return (size_t)c.n_experts * (size_t)tiled_n(c, which) * (size_t)tiled_k(c, which);
}
hipError_t launch_pack_weights(const moe_config& c, int which, const void* w, void* w_tiled, hipStream_t stream);
// The expert FFN's hidden activations h (moe_expert_ffn, moe_forward) in the same tiled layout
// (rows of h in 128-row blocks of 32-column slabs): bf16.
inline bool ffn_h_tiled(const moe_config& c) { return c.dtype == MOE_BF16; }
// moe_forward's own x_sorted (dropless, bf16) in the tiled layout too, for rows of 4096 or
// more elements: its row pitch, or 0. The dispatch copy then writes 64-byte pieces, which
// costs more than the up projection's contiguous reads gain on shorter rows (same-box A/B:
// d = 2048, k = 8: copy +31 us, up projection -23 us; d = 4096: +9 / -71 us; d = 7168:
// +26 / -239 us).
inline int forward_xs_kp(const moe_config& c) {
  return (c.dtype == MOE_BF16 && c.capacity_factor <= 0.f && c.d_model >= 4096) ? tiled_k(c, 0) : 0;
}
// floor(k cf N / E) raised to the next even integer (the capacity-factor dispatch's capacity)
long long expert_capacity(const moe_config& c, float capacity_factor);
hipError_t launch_dispatch_capacity(const moe_config& c, const WsLayout& L, float capacity_factor, const void* x,
                                    const int32_t* topk_ids, const float* topk_w, void* x_kept, int32_t* perm_kept,
                                    int32_t* slot, int32_t* kept, int32_t* offsets, float* gate_kept,
                                    hipStream_t stream);
int ffn_max_m_tiles(const moe_config& c);
hipError_t launch_dispatch(const moe_config& c, const WsLayout& L, const void* x,
                           const int32_t* topk_ids, const float* topk_w, void* x_sorted,
                           int32_t* perm, int32_t* inv_perm, int32_t* counts, int32_t* offsets,
                           float* gate_sorted, hipStream_t stream);
// Builds the per-call m-tile list from offsets (must precede the up and down launches).
hipError_t launch_ffn_tiles(const moe_config& c, const WsLayout& L, const int32_t* offsets, hipStream_t stream);
hipError_t launch_ffn_up(const moe_config& c, const WsLayout& L, const void* x_sorted,
                         const int32_t* offsets, const void* w1, const void* w3, const void* b1,
                         hipStream_t stream,
                         int xs_kp = 0);
hipError_t launch_ffn_down(const moe_config& c, const WsLayout& L, const int32_t* offsets,
                           const void* w2, const void* b2, const float* gate_sorted,
                           void* y_sorted, hipStream_t stream);
hipError_t launch_update_bias(const moe_config& c, const int32_t* counts, float* bias, float rate,
                              hipStream_t stream);
hipError_t launch_combine(const moe_config& c, const void* y_sorted, const float* topk_w,
                          const int32_t* inv_perm, const void* y_add, void* y, hipStream_t stream);
// The shared expert: dense MLP of width c.d_ff_shared over all N rows of x (tile table and
// hidden activations in L.tiles / L.h, which must be free: after the routed down projection).
hipError_t launch_shared(const moe_config& c, const WsLayout& L, const void* x, const void* s_w1,
                         const void* s_w3, const void* s_b1, const void* s_w2, const void* s_b2,
                         void* y_shared, hipStream_t stream);

// Down projection y = h W2^T (+ b2) times gate over a tile table's rows, K = the hidden width:
// (acc + b2) * gate, or with pre_gated (h already scaled by its row's gate) acc + gate * b2.
// tail_part: the K-split tail's partials (bfloat16; null: one persistent launch).
// w2_tiled: w2 is a moe_pack_weights copy (which = 1). h_kp > 0: h is tiled (as the up
// projection of moe_expert_ffn / moe_forward writes it) with that row pitch.
hipError_t launch_down(const moe_config& c, const int* tiles, int max_m_tiles, const void* h, int K, const void* w2,
                       const void* b2, const float* gate, bool pre_gated, void* y, float* tail_part,
                       hipStream_t stream, bool w2_tiled = false, int h_kp = 0);
// One persistent workgroup per CU: the CU count rounded up to a multiple of 8 (the XCDs).
int persistent_grid();
// Tile table of one dense "expert" covering rows [0, n) in tiles of bm rows.
hipError_t launch_dense_tiles(int n, int bm, int* tiles, hipStream_t stream);
// Backward recompute of the up projection (bfloat16): the tile table's rows of a times W1
// (and W3), writing the pre-activations to pre (SwiGLU: [rows][2 n_out] gate | up; GELU:
// [rows][n_out] with b1) and gate[row] * act(.) to hw [rows][n_out] (gate null: 1).
hipError_t launch_up_save(const moe_config& c, const int* tiles, const void* a, const void* w1, const void* w3,
                          const void* b1, const float* gate, int n_out, void* pre, void* hw, hipStream_t stream);
// The layer's backward (bfloat16, dropless); moe_backward's launch sequence.
struct BwdIn {
  const void* x; const void* w_router; const float* logit_bias; const float* sel_bias;
  const void* w1; const void* w3; const void* b1; const void* w2; const void* b2;
  const void* s_w1; const void* s_w3; const void* s_b1; const void* s_w2; const void* s_b2;
  const void* dy; float aux_coef, z_coef;
};
struct RouteOut {
  int32_t* topk_ids; float* topk_w; int32_t* counts; float* stats;
};
void carve_backward(const moe_config& c, WsCarver& w, WsLayout* L);
// events: null or MOE_BWD_EVENTS events recorded at the stage boundaries (moe.h)
hipError_t launch_backward(const moe_config& c, const WsLayout& L, const BwdIn& in, const moe_grads& gr,
                           const RouteOut& ro, bool saved, void* const* events, hipStream_t stream);
// The forward for training (moe_forward_train): the layer's output, leaving in the backward
// workspace what launch_backward(saved = true) reads instead of recomputing.
hipError_t launch_forward_train(const moe_config& c, const WsLayout& L, const BwdIn& in, void* y, const RouteOut& ro,
                                hipStream_t stream);
// rows of x copied to their sorted slots (x_sorted[inv_perm[n k + j]] = x[n])
// kp > 0: write x_sorted tiled with that row pitch (moe_forward's dropless bf16 path)
void launch_copy(const moe_config& c, const void* x, const int32_t* inv_perm, void* x_sorted, hipStream_t stream,
                 int kp = 0);

}  // namespace moe
