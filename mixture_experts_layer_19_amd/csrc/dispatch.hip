// Sorted dispatch ("Mixture of Experts: routing, sorted dispatch, Switch aux loss, aux-free
// bias" (L7.8) §2.2 and §3): assignment a = n*k + j is stably sorted by expert id as a
// two-level counting sort, with no atomics deciding any position:
//   1. histogram:  per chunk of kChunk assignments, the count of each expert;
//   2. scan:       counts, offsets (exclusive prefix sum, offsets[E] = A), and for every
//                  chunk the first sorted slot of its run of each expert;
//   3. scatter:    within a chunk, an assignment's slot is its chunk base plus the number of
//                  earlier assignments of the same expert in the chunk (wave ballots), so the
//                  order inside each expert's slice is ascending in a (stable);
//   4. row copy:   token-major, each row of x is read once and written to its k slots.
#include <cmath>

#include "moe_internal.h"

namespace moe {

constexpr int kChunk = 2048;  // assignments per workgroup in the histogram / scatter passes

// Expert id of the a-th assignment in the walk order: token-major (a = n k + j, the order of
// the dropless dispatch) or k-major (a = j N + n: every token's first choice, then every
// token's second choice, ...; the ranking order of the capacity-factor dispatch).
template <bool KMAJOR> MOE_DEV int walk_index(int a, int n_tokens, int k) {
  if (!KMAJOR) return a;
  const int j = a / n_tokens;
  return (a - j * n_tokens) * k + j;
}

template <bool KMAJOR>
__global__ __launch_bounds__(256) void dispatch_hist_kernel(
    const int32_t* __restrict__ ids, int A, int E, int n_tokens, int k, int* __restrict__ hist,
    int* __restrict__ bad) {
  __shared__ int s_hist[kMaxExperts];
  __shared__ int s_bad;
  for (int e = threadIdx.x; e < E; e += 256) s_hist[e] = 0;
  if (threadIdx.x == 0) s_bad = 0;
  __syncthreads();
  const int a0 = blockIdx.x * kChunk;
  const int a1 = min(A, a0 + kChunk);
  int my_bad = 0;
  for (int a = a0 + threadIdx.x; a < a1; a += 256) {
    const int e = ids[walk_index<KMAJOR>(a, n_tokens, k)];
    if (e >= 0 && e < E) atomicAdd(&s_hist[e], 1);  // integer counts: order-independent
    else my_bad = 1;
  }
  if (my_bad) s_bad = 1;
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) hist[(size_t)blockIdx.x * E + e] = s_hist[e];
  if (threadIdx.x == 0) bad[blockIdx.x] = s_bad;
}

// One workgroup: per-expert totals over the chunks (chunk order), exclusive scan over
// experts, chunk bases, and the device error word (written, not accumulated).
__global__ __launch_bounds__(1024) void dispatch_scan_kernel(
    const int* __restrict__ hist, const int* __restrict__ bad, int n_chunks, int E,
    int* __restrict__ base, int* __restrict__ counts, int* __restrict__ offsets, int* __restrict__ err) {
  __shared__ int s_scan[kMaxExperts];
  __shared__ int s_bad;
  const int e = threadIdx.x;
  if (e == 0) s_bad = 0;
  int total = 0;
  if (e < E) {
    for (int b = 0; b < n_chunks; ++b) total += hist[(size_t)b * E + e];
    s_scan[e] = total;
  }
  __syncthreads();
  for (int b = threadIdx.x; b < n_chunks; b += blockDim.x)
    if (bad[b]) s_bad = 1;
  // inclusive Hillis-Steele scan over the experts
  for (int o = 1; o < E; o <<= 1) {
    int v = 0;
    if (e < E && e >= o) v = s_scan[e - o];
    __syncthreads();
    if (e < E) s_scan[e] += v;
    __syncthreads();
  }
  if (e < E) {
    const int start = s_scan[e] - total;
    counts[e] = total;
    offsets[e] = start;
    if (e == E - 1) offsets[E] = s_scan[e];
    int run = start;
    for (int b = 0; b < n_chunks; ++b) {
      base[(size_t)b * E + e] = run;
      run += hist[(size_t)b * E + e];
    }
  }
  __syncthreads();
  if (threadIdx.x == 0 && err) err[0] = s_bad ? MOE_ERR_BAD_EXPERT_ID : 0;
}

// Stable scatter. The chunk of `chunk` assignments is walked in order, blockDim.x (64, 128
// or 256) at a time. For an assignment of expert e in wave w: slot = running[e] + (count of
// e in waves < w of this step) + (count of e in lower lanes of wave w). Per-wave counts are
// published in LDS tagged with the step number, so stale entries read as zero without
// clearing. base[blockIdx.x][e] is the first slot of this chunk's run of expert e.
// Capacity scan: like dispatch_scan_kernel over the k-major chunks, plus kept = min(total,
// cap) and koff = exclusive scan of kept; offsets (the kept slices) = koff with koff[E] =
// the number of kept rows.
__global__ __launch_bounds__(1024) void capacity_scan_kernel(
    const int* __restrict__ hist, const int* __restrict__ bad, int n_chunks, int E, int cap,
    int* __restrict__ base, int* __restrict__ offs_all, int* __restrict__ kept, int* __restrict__ koff,
    int* __restrict__ offsets, int* __restrict__ err) {
  __shared__ int s_scan[kMaxExperts];
  __shared__ int s_kscan[kMaxExperts];
  __shared__ int s_bad;
  const int e = threadIdx.x;
  if (e == 0) s_bad = 0;
  int total = 0;
  if (e < E) {
    for (int b = 0; b < n_chunks; ++b) total += hist[(size_t)b * E + e];
    s_scan[e] = total;
    s_kscan[e] = min(total, cap);
  }
  __syncthreads();
  for (int b = threadIdx.x; b < n_chunks; b += blockDim.x)
    if (bad[b]) s_bad = 1;
  for (int o = 1; o < E; o <<= 1) {
    int v = 0, w = 0;
    if (e < E && e >= o) {
      v = s_scan[e - o];
      w = s_kscan[e - o];
    }
    __syncthreads();
    if (e < E) {
      s_scan[e] += v;
      s_kscan[e] += w;
    }
    __syncthreads();
  }
  if (e < E) {
    const int start = s_scan[e] - total;
    const int kk = min(total, cap);
    offs_all[e] = start;
    kept[e] = kk;
    koff[e] = s_kscan[e] - kk;
    offsets[e] = s_kscan[e] - kk;
    if (e == E - 1) offsets[E] = s_kscan[e];
    int run = start;
    for (int b = 0; b < n_chunks; ++b) {
      base[(size_t)b * E + e] = run;
      run += hist[(size_t)b * E + e];
    }
  }
  __syncthreads();
  if (threadIdx.x == 0 && err) err[0] = s_bad ? MOE_ERR_BAD_EXPERT_ID : 0;
}

// Capacity variant (CAP): `pos` is then the assignment's place among all of its expert's
// assignments in k-major order; rank = pos - offs_all[e]; it is kept at row koff[e] + rank
// when rank < cap (perm / inv_perm / gate_sorted refer to the kept rows), else dropped
// (inv_perm = -1).
struct CapArgs {
  int cap;
  const int* offs_all;  // [E] exclusive scan of all assignments per expert
  const int* koff;      // [E] exclusive scan of the kept counts
};

template <bool KMAJOR, bool CAP>
__global__ __launch_bounds__(256) void dispatch_scatter_kernel(
    const int32_t* __restrict__ ids, const float* __restrict__ topk_w, int A, int E, int id_bits, int chunk,
    int n_tokens, int k, const int* __restrict__ base, int32_t* __restrict__ perm, int32_t* __restrict__ inv_perm,
    float* __restrict__ gate_sorted, CapArgs ca) {
  __shared__ int s_run[kMaxExperts];
  __shared__ int s_cnt[4][kMaxExperts];  // (step << 16) | count
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nthr = blockDim.x;
  const int n_waves = nthr >> 6;
  for (int e = threadIdx.x; e < E; e += nthr) {
    s_run[e] = base[(size_t)blockIdx.x * E + e];
    for (int w = 0; w < n_waves; ++w) s_cnt[w][e] = -1;
  }
  __syncthreads();
  const int a0 = blockIdx.x * chunk;
  const int a1 = min(A, a0 + chunk);
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int step = 0, as = a0; as < a1; ++step, as += nthr) {
    const int a = as + threadIdx.x;
    const int ai = (a < a1) ? walk_index<KMAJOR>(a, n_tokens, k) : 0;  // assignment n k + j
    const int e = (a < a1) ? ids[ai] : -1;
    const bool valid = e >= 0 && e < E;
    // lanes of this wave holding the same expert id
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < id_bits; ++b) {
      const uint64_t ones = __ballot(valid && ((e >> b) & 1));
      peers &= ((e >> b) & 1) ? ones : ~ones;
    }
    const int rank = __popcll(peers & lt_mask);
    const int cnt = __popcll(peers);
    const bool leader = valid && rank == 0;
    if (leader) s_cnt[wave][e] = (step << 16) | cnt;
    __syncthreads();
    if (valid) {
      int before = 0;
      for (int w = 0; w < wave; ++w) {
        const int v = s_cnt[w][e];
        if ((v >> 16) == step) before += v & 0xffff;
      }
      int pos = s_run[e] + before + rank;
      if (CAP) {
        const int r = pos - ca.offs_all[e];
        pos = (r < ca.cap) ? ca.koff[e] + r : -1;
      }
      if (pos >= 0) {
        if (perm) perm[pos] = ai;
        if (gate_sorted) gate_sorted[pos] = topk_w[ai];
      }
      inv_perm[ai] = pos;
    } else if (a < a1) {
      inv_perm[ai] = -1;
    }
    __syncthreads();
    if (leader) atomicAdd(&s_run[e], cnt);  // integer adds: the final run is order-independent
    __syncthreads();
  }
}

// Token-major row copy: x_sorted[inv_perm[n*k + j]] = x[n] for j < k. One wave per token:
// the k destinations are wave-uniform, the lanes stream the row in 16-byte pieces, four
// pieces per lane in flight, each read once and written k times. kp > 0: x_sorted is tiled
// (128-row blocks of 32-column slabs, row pitch kp elements; bf16), so four lanes write the
// 64 bytes of one slab of the row.
__global__ __launch_bounds__(256) void dispatch_copy_kernel(
    const uint4* __restrict__ x, const int32_t* __restrict__ inv_perm, uint4* __restrict__ x_sorted,
    long long n_tokens, int k, int vec_per_row, int kp) {
  const int lane = threadIdx.x & 63;
  const long long wave0 = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const long long n_waves = (long long)gridDim.x * 4;
  for (long long n = wave0; n < n_tokens; n += n_waves) {
    const uint4* row = x + (size_t)n * vec_per_row;
    for (int c0 = 0; c0 < vec_per_row; c0 += 4 * 64) {
      uint4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int c = c0 + u * 64 + lane;
        v[u] = c < vec_per_row ? row[c] : make_uint4(0, 0, 0, 0);
      }
      for (int j = 0; j < k; ++j) {
        const int dst = inv_perm[n * k + j];  // wave-uniform
        if (dst < 0) continue;
        // row-major: row dst; tiled: row dst & 127 of block dst / 128 (16-byte units; a slab
        // row is 4 of them and a block's slab 512)
        uint4* out = kp > 0 ? x_sorted + ((size_t)(dst & ~(kTiledRows - 1)) * kp + (dst & (kTiledRows - 1)) * kTiledK) / 8
                            : x_sorted + (size_t)dst * vec_per_row;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int c = c0 + u * 64 + lane;
          if (c < vec_per_row) out[kp > 0 ? (c >> 2) * (kTiledRows * kTiledK / 8) + (c & 3) : c] = v[u];
        }
      }
    }
  }
}

// Row-major x to tiled x_sorted (128-row blocks of 32-column slabs, row pitch kp elements;
// bf16), gathered by destination: x_sorted[i] = x[perm[i] / k]. A workgroup owns 64
// destination rows and kCopySlabs slabs of them; wave w owns rows 16w..16w+15 and lane l
// the 16-byte chunk l & 3 of row l >> 2, so each store instruction writes one slab of 16
// consecutive rows: 1 KiB of contiguous memory (the token-major copy writes the same bytes
// as 64-byte pieces of 128-byte lines, the other half of each line coming from another
// token). A lane's kCopySlabs loads are all in flight before its first store. Each x row is
// read k times (once per destination), so it is used for k <= 2 only. Same-box A/B of the
// dispatch stage against the token-major copy: Mixtral shape (k = 2) 52.1 -> 47.9 us;
// DeepSeek-V3 shape (k = 8) 125 -> 137 us, which keeps the token-major copy.
constexpr int kCopySlabs = 16, kCopyGatherMaxK = 2;
__global__ __launch_bounds__(256) void dispatch_copy_tiled_kernel(
    const uint4* __restrict__ x, const int32_t* __restrict__ perm, uint4* __restrict__ x_sorted, int n_rows, int k,
    int vec_per_row, int kp) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 64 + (threadIdx.x >> 6) * 16 + (lane >> 2);  // destination row
  const int ch = lane & 3;
  if (r >= n_rows) return;
  const uint4* src = x + (size_t)(perm[r] / k) * vec_per_row;
  uint4* dst = x_sorted + ((size_t)(r & ~(kTiledRows - 1)) * kp + (r & (kTiledRows - 1)) * kTiledK) / 8;
  const int s0 = blockIdx.y * kCopySlabs;
  uint4 v[kCopySlabs];
#pragma unroll
  for (int j = 0; j < kCopySlabs; ++j) {
    const int c = (s0 + j) * 4 + ch;
    v[j] = c < vec_per_row ? src[c] : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int j = 0; j < kCopySlabs; ++j) {
    const int c = (s0 + j) * 4 + ch;
    if (c < vec_per_row) dst[(size_t)(s0 + j) * (kTiledRows * kTiledK / 8) + ch] = v[j];
  }
}

static int id_bits_of(int E) {
  int b = 0;
  while ((1 << b) < E) ++b;
  return b;
}

void launch_copy(const moe_config& c, const void* x, const int32_t* inv_perm, void* x_sorted, hipStream_t stream,
                 int kp) {
  if (!x_sorted) return;
  const int vpr = (int)(c.d_model * elem_size(c) / 16);
  const int grid = (int)std::min<long long>((c.n_tokens + 3) / 4, 1 << 16);
  dispatch_copy_kernel<<<grid, 256, 0, stream>>>(static_cast<const uint4*>(x), inv_perm,
                                                 static_cast<uint4*>(x_sorted), c.n_tokens, c.top_k, vpr, kp);
}

void carve_dispatch(const moe_config& c, WsCarver& w, WsLayout* L) {
  const long long A = c.n_tokens * c.top_k;
  const int n_chunks = (int)((A + kChunk - 1) / kChunk);
  const size_t E = (size_t)c.n_experts;
  int* hist = w.take_t<int>((size_t)n_chunks * E);
  int* base = w.take_t<int>((size_t)n_chunks * E);
  int* bad = w.take_t<int>((size_t)n_chunks);
  int* offs_all = w.take_t<int>(E);
  int* koff = w.take_t<int>(E);
  if (L) {
    L->d_hist = hist;
    L->d_base = base;
    L->d_bad = bad;
    L->d_offs_all = offs_all;
    L->d_koff = koff;
  }
}

long long expert_capacity(const moe_config& c, float capacity_factor) {
  const double v = std::floor((double)c.top_k * (double)capacity_factor * (double)c.n_tokens / (double)c.n_experts);
  const long long cap = (long long)v;
  return cap + (cap & 1);
}

hipError_t launch_dispatch_capacity(const moe_config& c, const WsLayout& L, float capacity_factor, const void* x,
                                    const int32_t* topk_ids, const float* topk_w, void* x_kept, int32_t* perm_kept,
                                    int32_t* slot, int32_t* kept, int32_t* offsets, float* gate_kept,
                                    hipStream_t stream) {
  const int A = (int)(c.n_tokens * c.top_k);
  const int E = c.n_experts;
  const int N = (int)c.n_tokens, k = c.top_k;
  const int n_chunks = (A + kChunk - 1) / kChunk;
  // an expert holds at most one assignment per token, so a capacity above N drops nothing
  const int cap = (int)std::min<long long>(expert_capacity(c, capacity_factor), (long long)N);
  if (n_chunks > 0) dispatch_hist_kernel<true><<<n_chunks, 256, 0, stream>>>(topk_ids, A, E, N, k, L.d_hist, L.d_bad);
  capacity_scan_kernel<<<1, 1024, 0, stream>>>(L.d_hist, L.d_bad, n_chunks, E, cap, L.d_base, L.d_offs_all, kept,
                                               L.d_koff, offsets, L.err);
  if (n_chunks > 0) {
    CapArgs ca{cap, L.d_offs_all, L.d_koff};
    const bool gate = gate_kept && topk_w;
    dispatch_scatter_kernel<true, true><<<n_chunks, 256, 0, stream>>>(
        topk_ids, gate ? topk_w : nullptr, A, E, id_bits_of(E), kChunk, N, k, L.d_base, perm_kept, slot,
        gate ? gate_kept : nullptr, ca);
    launch_copy(c, x, slot, x_kept, stream);
  }
  return hipGetLastError();
}

hipError_t launch_dispatch(const moe_config& c, const WsLayout& L, const void* x,
                           const int32_t* topk_ids, const float* topk_w, void* x_sorted,
                           int32_t* perm, int32_t* inv_perm, int32_t* counts, int32_t* offsets,
                           float* gate_sorted, hipStream_t stream) {
  const int A = (int)(c.n_tokens * c.top_k);
  const int E = c.n_experts;
  const int n_chunks = (A + kChunk - 1) / kChunk;
  const int id_bits = id_bits_of(E);
  const int N = (int)c.n_tokens, k = c.top_k;
  if (n_chunks > 0) dispatch_hist_kernel<false><<<n_chunks, 256, 0, stream>>>(topk_ids, A, E, N, k, L.d_hist, L.d_bad);
  dispatch_scan_kernel<<<1, 1024, 0, stream>>>(L.d_hist, L.d_bad, n_chunks, E, L.d_base, counts, offsets, L.err);
  if (n_chunks > 0) {
    dispatch_scatter_kernel<false, false><<<n_chunks, 256, 0, stream>>>(
        topk_ids, (gate_sorted && topk_w) ? topk_w : nullptr, A, E, id_bits, kChunk, N, k, L.d_base, perm, inv_perm,
        (gate_sorted && topk_w) ? gate_sorted : nullptr, CapArgs{});
    launch_copy(c, x, inv_perm, x_sorted, stream);
  }
  return hipGetLastError();
}

// moe_forward's dispatch: the routing finalize already wrote offsets and the per-route-block
// bases (L.fbase), so only the scatter (one chunk per routing block) and the copy remain;
// a tiled x_sorted with k <= 2 is gathered by destination rows, else copied token-major.
hipError_t launch_dispatch_scanned(const moe_config& c, const WsLayout& L, const void* x,
                                   const int32_t* topk_ids, const float* topk_w, void* x_sorted,
                                   int32_t* perm, int32_t* inv_perm, float* gate_sorted, hipStream_t stream,
                                   int xs_kp) {
  const int A = (int)(c.n_tokens * c.top_k);
  if (A == 0) return hipGetLastError();
  const int E = c.n_experts;
  const int chunk = route_tokens_per_block(c) * c.top_k;
  const int n_chunks = (A + chunk - 1) / chunk;
  const int threads = chunk <= 64 ? 64 : chunk <= 128 ? 128 : 256;
  dispatch_scatter_kernel<false, false><<<n_chunks, threads, 0, stream>>>(
      topk_ids, (gate_sorted && topk_w) ? topk_w : nullptr, A, E, id_bits_of(E), chunk, (int)c.n_tokens, c.top_k,
      L.fbase, perm, inv_perm, (gate_sorted && topk_w) ? gate_sorted : nullptr, CapArgs{});
  if (xs_kp > 0 && x_sorted && c.top_k <= kCopyGatherMaxK) {
    const int vpr = (int)(c.d_model * elem_size(c) / 16);
    const dim3 grid((A + 63) / 64, ((vpr + 3) / 4 + kCopySlabs - 1) / kCopySlabs);
    dispatch_copy_tiled_kernel<<<grid, 256, 0, stream>>>(static_cast<const uint4*>(x), perm,
                                                         static_cast<uint4*>(x_sorted), A, c.top_k, vpr, xs_kp);
  } else {
    launch_copy(c, x, inv_perm, x_sorted, stream, xs_kp);
  }
  return hipGetLastError();
}

}  // namespace moe
