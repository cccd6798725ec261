// Routing kernels: router projection z = x W_g^T, then per token softmax, selection score,
// top-k (largest first, ties to the lowest id), gates, and per-block partials of the
// Switch statistics; a final single-workgroup kernel reduces the partials in a fixed order.
//
// Follows "Mixture of Experts: routing, sorted dispatch, Switch aux loss, aux-free bias"
// (L7.8) §2 symbol table and §2.1 routers table, §2.3 load-balancing loss, §2.5 (the bias
// chooses, never weighs); "15. Mixture of Experts" (RustingBrain) §15.2 routing, §15.3 z-loss.
#include <algorithm>

#include "moe_internal.h"

namespace moe {

// The router projection splits its reduction into partial sums added in a fixed order: at
// most 8 (a power of two) for the LDS-tiled projection (E > 64); always kFusedQuarters, one
// per wave pair, in the fused kernel of up to 64 experts, whose lanes keep eight 32-wide
// steps of loads in flight. Before the fusion, Mixtral shape, same-box A/B of the routing
// stage: split 8 with four steps in flight 39.2-39.5 us, split 4 with eight 37.4 us (split 2
// 39.1, split 1 47.5, split 2 with sixteen steps 39.3).
constexpr int kRouterMaxSplit = 8;
constexpr int kFusedQuarters = 4;

// z = the sum of a token's S split partials of one expert, in split order; every partial is
// requested before the first add.
template <int S>
MOE_DEV float split_sum(const float* zp, size_t stride) {
  float zs[S];
#pragma unroll
  for (int sp = 0; sp < S; ++sp) zs[sp] = zp[(size_t)sp * stride];
  float v = 0.f;
#pragma unroll
  for (int sp = 0; sp < S; ++sp) v += zs[sp];
  return v;
}

// ---------------------------------------------------------------------------------------
// Router projection, bfloat16 inputs, float32 accumulation on MFMA (v_mfma_f32_16x16x32_bf16),
// up to 64 experts: route_fused_kernel (below) runs it and the per-token routing in one launch.
// ---------------------------------------------------------------------------------------
// Partial logits of 16 tokens (t0 ..) x 16 NB experts (e0 ..) over the reduction range
// [kb, ke), on v_mfma_f32_16x16x32_bf16: lane l ends with token t0 + 4 (l >> 4) + r of
// acc[b][r], expert e0 + 16 b + (l & 15). Rows past the last token or expert read the last
// one's row, an in-range address, so no load sits behind a per-lane branch (a load there is
// waited for before the next is issued); their outputs are never used. Steps past ke (a
// partial 32-wide step) multiply zeros.
//
// Loads go in batches of kU steps, left to the compiler's schedule, which issues each step's
// loads a few steps ahead of its product (about eight 16-byte loads in flight per lane).
// Same-box A/B at the Mixtral shape (routing kernel, moe_forward): this form 18.7 us; every
// batch's loads issued before its first product 21.0; two batches in flight (the next
// batch's loads issued ahead of this batch's products) 24.2; bounds-checked buffer loads for
// the rows past N or E instead of the clamped rows 20.3.
template <int NB>
MOE_DEV void router_mfma16(const bf16_t* __restrict__ x, const bf16_t* __restrict__ wg, int t0, int e0, int kb, int ke,
                           int n_tokens, int d, int n_experts, int lane, f32x4 (&acc)[NB]) {
  const int row = lane & 15;
  const int kq = (lane >> 4) * 8;
#pragma unroll
  for (int b = 0; b < NB; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
  const bf16_t* arow = x + (size_t)min(t0 + row, n_tokens - 1) * d + kq;
  const bf16_t* brow[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) brow[b] = wg + (size_t)min(e0 + b * 16 + row, n_experts - 1) * d + kq;

  constexpr int kU = NB >= 4 ? 4 : 8;
  const int nb = max(0, ke - kb) / (kU * 32);
  uint4 av[kU], bv[NB][kU];
  for (int i = 0; i < nb; ++i) {
    const int k0 = kb + i * (kU * 32);
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      av[u] = *reinterpret_cast<const uint4*>(arow + k0 + u * 32);
#pragma unroll
      for (int b = 0; b < NB; ++b) bv[b][u] = *reinterpret_cast<const uint4*>(brow[b] + k0 + u * 32);
    }
#pragma unroll
    for (int u = 0; u < kU; ++u)
#pragma unroll
      for (int b = 0; b < NB; ++b)
        acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av[u]),
                                                         __builtin_bit_cast(bf16x8, bv[b][u]), acc[b], 0, 0, 0);
  }
  for (int k = kb + nb * kU * 32; k < ke; k += 32) {  // uniform trip count
    const bool in = k + kq < ke;  // ke is a multiple of 8, so a chunk is wholly in or out
    const int kc = in ? k : ke - 8 - kq;  // lanes past ke re-read the chunk ke - 8 (in range)
    uint4 a1 = *reinterpret_cast<const uint4*>(arow + kc);
    uint4 b1[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) b1[b] = *reinterpret_cast<const uint4*>(brow[b] + kc);
    if (!in) a1 = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      if (!in) b1[b] = make_uint4(0, 0, 0, 0);
      acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a1), __builtin_bit_cast(bf16x8, b1[b]),
                                                       acc[b], 0, 0, 0);
    }
  }
}

// Router projection for E > 64 experts, bfloat16 inputs: workgroup tile 64 tokens x 64 WE
// experts, one wave per 64 experts (2 x 2 blocks of v_mfma_f32_32x32x16_bf16), K walked in
// slabs of 128 or 64 held in LDS, with the next slab loaded into registers while this one
// is multiplied (wider slabs than 32 took the 128-expert projection of 16384 tokens from 44
// to 42 us and the whole routing stage from 94 to 89 us). Sharing each
// x slab across the workgroup's waves and each W_g slab across its 64 tokens keeps the L2
// traffic near one read of x plus one read of W_g per 64 tokens. grid.z splits the
// reduction axis as in router_gemm_bf16_kernel.
template <int WE>
__global__ __launch_bounds__(64 * WE) void router_gemm_tiled_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ wg, float* __restrict__ zpart,
    int n_tokens, int d, int n_experts, int k_chunk) {
  // Slabs of 128 (64 for 256 experts, whose 87 KiB of LDS at 128 would leave one workgroup
  // per CU). LDS rows of kBKr + 8 elements (68 or 36 dwords): 16 lanes reading 16 bytes of 16
  // consecutive rows cover all 64 banks once.
  constexpr int kBMr = 64, kBEr = 64 * WE, kBKr = WE == 2 ? 128 : 64, kLd = kBKr + 8;
  constexpr int kThreads = 64 * WE;
  constexpr int kCh = kBKr / 8;                // 16-byte chunks per row of a slab
  constexpr int kAPer = kBMr * kCh / kThreads;  // 16-byte chunks per thread per slab
  constexpr int kBPer = kBEr * kCh / kThreads;
  __shared__ __attribute__((aligned(16))) uint16_t sA[kBMr * kLd];
  __shared__ __attribute__((aligned(16))) uint16_t sB[kBEr * kLd];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.x * kBMr, e0 = blockIdx.y * kBEr;
  const int kb = blockIdx.z * k_chunk;
  const int ke = min(d, kb + k_chunk);
  const uint16_t* xs = reinterpret_cast<const uint16_t*>(x);
  const uint16_t* ws = reinterpret_cast<const uint16_t*>(wg);

  uint4 ra[kAPer], rb[kBPer];
  auto gload = [&](int k) {
#pragma unroll
    for (int i = 0; i < kAPer; ++i) {
      const int idx = tid + i * kThreads, row = idx / kCh, kk = k + (idx % kCh) * 8;
      const int t = t0 + row;
      ra[i] = (t < n_tokens && kk < ke) ? *reinterpret_cast<const uint4*>(xs + (size_t)t * d + kk)
                                        : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < kBPer; ++i) {
      const int idx = tid + i * kThreads, row = idx / kCh, kk = k + (idx % kCh) * 8;
      const int e = e0 + row;
      rb[i] = (e < n_experts && kk < ke) ? *reinterpret_cast<const uint4*>(ws + (size_t)e * d + kk)
                                         : make_uint4(0, 0, 0, 0);
    }
  };
  auto lstore = [&]() {
#pragma unroll
    for (int i = 0; i < kAPer; ++i) {
      const int idx = tid + i * kThreads;
      *reinterpret_cast<uint4*>(&sA[(idx / kCh) * kLd + (idx % kCh) * 8]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < kBPer; ++i) {
      const int idx = tid + i * kThreads;
      *reinterpret_cast<uint4*>(&sB[(idx / kCh) * kLd + (idx % kCh) * 8]) = rb[i];
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  if (kb < ke) {
    gload(kb);
    lstore();
  }
  __syncthreads();
  for (int k = kb; k < ke; k += kBKr) {
    const bool more = k + kBKr < ke;
    if (more) gload(k + kBKr);
#pragma unroll
    for (int ks = 0; ks < kBKr / 16; ++ks) {
      bf16x8 fa[2], fb[2];
      const int kq = ks * 16 + (lane >> 5) * 8;
#pragma unroll
      for (int i = 0; i < 2; ++i)
        fa[i] = *reinterpret_cast<const bf16x8*>(&sA[(i * 32 + (lane & 31)) * kLd + kq]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        fb[j] = *reinterpret_cast<const bf16x8*>(&sB[(wave * 64 + j * 32 + (lane & 31)) * kLd + kq]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();  // every wave is done reading the slab
    if (more) {
      lstore();
      __syncthreads();
    }
  }
  // lane's element v of a 32 x 32 block: column lane & 31, row 8 (v >> 2) + 4 (lane >> 5) + (v & 3)
  float* zp = zpart + (size_t)blockIdx.z * n_tokens * n_experts;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int e = e0 + wave * 64 + j * 32 + (lane & 31);
    if (e >= n_experts) continue;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int t = t0 + i * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
        if (t < n_tokens) zp[(size_t)t * n_experts + e] = acc[i][j][v];
      }
  }
}

// Router projection for float32 inputs: one wave per token, lanes split the reduction axis,
// float32 FMA accumulation, then a fixed butterfly sum per expert.
__global__ __launch_bounds__(256) void router_gemm_f32_kernel(
    const float* __restrict__ x, const float* __restrict__ wg, float* __restrict__ z,
    int n_tokens, int d, int n_experts) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= n_tokens) return;
  const float* xr = x + (size_t)t * d;
  for (int e = 0; e < n_experts; ++e) {
    const float* wr = wg + (size_t)e * d;
    float s = 0.f;
    for (int k = lane; k < d; k += 64) s = fmaf(xr[k], wr[k], s);
    s = wave_sum(s);
    if (lane == 0) z[(size_t)t * n_experts + e] = s;
  }
}

// ---------------------------------------------------------------------------------------
// Per-token routing. A token is owned by a group of LPT lanes (LPT = E rounded up to a power
// of two, at most 64); lane l of the group holds experts l, l + LPT, ... (EPL of them), so
// one wave routes 64 / LPT tokens side by side and every cross-lane step stays in the group.
// ---------------------------------------------------------------------------------------

// (score desc, id asc): a beats b when its score is larger, or equal with a lower id.
MOE_DEV bool beats(float s, int id, float s2, int id2) { return s > s2 || (s == s2 && id < id2); }

template <int W> MOE_DEV float group_sum(float v) {
#pragma unroll
  for (int o = W / 2; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
template <int W> MOE_DEV float group_max(float v) {
#pragma unroll
  for (int o = W / 2; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// Waves per routing workgroup: 16, or 4 when every lane holds 16 experts (register budget).
constexpr int route_waves(int epl) { return epl >= 16 ? 4 : 16; }

// One pass of a wave's token groups: group grp routes token t (valid when tok; the trip is
// uniform over the wave, so a group past the last token computes on -inf / zeros and writes
// nothing). zf(e) is the token's logit of expert e before the logit bias. Adds the token's
// probabilities to psum and its squared log-sum-exp to zl_acc (lane 0 of the group), and its
// chosen ids to the block histogram s_hist.
template <int LPT, int EPL, typename ZF>
MOE_DEV void route_token(const RouteArgs& a, int t, bool tok, int sub, int grp, ZF&& zf, float (&psum)[EPL],
                         float& zl_acc, int* s_hist) {
  const int E = a.n_experts;
  const int k = a.top_k;
  const bool sigm = a.router == MOE_ROUTER_SIGMOID;
  float z[EPL], s[EPL], ex[EPL];
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = sub + LPT * i;
    const bool ok = e < E;
    float v = 0.f;
    if (ok && tok) {
      v = zf(e);
      if (a.logit_bias) v += a.logit_bias[e];
      if (a.logits_out) a.logits_out[(size_t)t * E + e] = v;
    }
    z[i] = ok ? v : -INFINITY;
    m = fmaxf(m, z[i]);
  }
  m = group_max<LPT>(m);
  float lsum = 0.f;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    ex[i] = (sub + LPT * i < E) ? expf(z[i] - m) : 0.f;
    lsum += ex[i];
  }
  const float sum = group_sum<LPT>(lsum);
  const float inv_sum = 1.0f / sum;
  if (tok && sub == 0) {
    const float lse = m + logf(sum);
    zl_acc += lse * lse;
  }
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = sub + LPT * i;
    const bool ok = e < E;
    psum[i] += (ok && tok) ? ex[i] * inv_sum : 0.f;
    float sc = sigm ? sigmoid_f(z[i]) : z[i];
    if (ok && a.sel_bias) sc += a.sel_bias[e];
    if (sc != sc) sc = -INFINITY;  // a NaN score ranks last, so k valid ids are still chosen
    s[i] = ok ? sc : -INFINITY;
  }

  // k rounds of a group arg-max on (score desc, id asc); one more for the margin. Some
  // lane of the group always holds an untaken valid expert (k <= E), and -inf loses
  // only to a lower id, so the winner is always a valid id.
  uint32_t taken = 0;
  int my_id = -1;
  float my_u = 0.f, last_s = 0.f, gap = INFINITY;
  const int rounds = (k < E) ? k + 1 : k;
  for (int j = 0; j < rounds; ++j) {
    float bs = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = sub + LPT * i;
      if (e < E && !((taken >> i) & 1u) && beats(s[i], e, bs, bi)) {
        bs = s[i];
        bi = e;
      }
    }
#pragma unroll
    for (int o = LPT / 2; o >= 1; o >>= 1) {
      const float os = __shfl_xor(bs, o, kWave);
      const int oi = __shfl_xor(bi, o, kWave);
      if (beats(os, oi, bs, bi)) {
        bs = os;
        bi = oi;
      }
    }
    if (j == k) {  // the best unchosen expert
      gap = last_s - bs;
      break;
    }
    last_s = bs;
    // raw gate of the chosen expert: exp(z - m) for the softmax routers, sigmoid(z) else
    const int slot = bi / LPT;
    const int owner = bi & (LPT - 1);
    float mine = 0.f;
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (i == slot) mine = sigm ? sigmoid_f(z[i]) : ex[i];
    const float u = __shfl(mine, grp * LPT + owner, kWave);
    if (sub == owner) taken |= 1u << slot;
    if (sub == j) {
      my_id = bi;
      my_u = u;
    }
  }
  // gates ([L7.8] §2.1): the softmax routers renormalise exp(z - m) over the chosen set
  // (= p_T / sum p_T = softmax over the chosen logits); without renormalisation the
  // softmax_topk gate is p itself. The sigmoid router renormalises sigmoid(z_T).
  const float usum = group_sum<LPT>(sub < k ? my_u : 0.f);
  if (tok && sub < k) {
    float w;
    if (a.router == MOE_ROUTER_TOPK_SOFTMAX || a.norm_topk) w = my_u / usum;
    else if (a.router == MOE_ROUTER_SOFTMAX_TOPK) w = my_u * inv_sum;
    else w = my_u;
    w *= a.routed_scaling;
    a.topk_ids[(size_t)t * k + sub] = my_id;
    a.topk_w[(size_t)t * k + sub] = w;
    atomicAdd(&s_hist[my_id], 1);  // integer adds: order-independent
  }
  if (a.gap_out && tok && sub == 0) a.gap_out[t] = gap;
}

// Deterministic block partials of NW waves: the groups of a wave combined by a fixed
// butterfly, then the waves in wave order. Every thread of the block calls it.
template <int LPT, int EPL, int NW>
MOE_DEV void route_block_partials(const RouteArgs& a, int lane, int wave, float (&psum)[EPL], float zl_acc,
                                  float (*s_psum)[LPT * EPL], float* s_zl, const int* s_hist) {
  const int E = a.n_experts;
  const int sub = lane & (LPT - 1);
  const int grp = lane / LPT;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
#pragma unroll
    for (int o = 32; o >= LPT; o >>= 1) psum[i] += __shfl_xor(psum[i], o, kWave);
    const int e = sub + LPT * i;
    if (grp == 0 && e < E) s_psum[wave][e] = psum[i];
  }
  const float zl = wave_sum(zl_acc);
  if (lane == 0) s_zl[wave] = zl;
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += NW * kWave) {
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) v += s_psum[w][e];
    a.part_p[(size_t)blockIdx.x * E + e] = v;
    a.part_hist[(size_t)blockIdx.x * E + e] = s_hist[e];
  }
  if (threadIdx.x == 0) {
    float v = 0.f;
    for (int w = 0; w < NW; ++w) v += s_zl[w];
    a.part_zl[blockIdx.x] = v;
  }
}

template <int LPT, int EPL>
__global__ __launch_bounds__(route_waves(EPL) * kWave) void route_tokens_kernel(RouteArgs a) {
  constexpr int kRouteWaves = route_waves(EPL);
  constexpr int kTpw = kWave / LPT;  // tokens routed side by side per wave
  constexpr int kCols = LPT * EPL;   // expert slots of a token group
  __shared__ float s_psum[kRouteWaves][kCols];
  __shared__ int s_hist[kCols];
  __shared__ float s_zl[kRouteWaves];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int sub = lane & (LPT - 1);  // lane within the token's group
  const int grp = lane / LPT;
  const int E = a.n_experts;

  for (int e = threadIdx.x; e < E; e += kRouteWaves * kWave) s_hist[e] = 0;
  __syncthreads();

  float psum[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) psum[i] = 0.f;
  float zl_acc = 0.f;

  const int wave_tok0 = blockIdx.x * a.tokens_per_block + wave * a.tokens_per_wave;
  const size_t zs = (size_t)a.n_tokens * E;
  for (int it = 0; it < a.tokens_per_wave; it += kTpw) {
    const int t = wave_tok0 + it + grp;
    const float* zp = a.zpart + (size_t)t * E;
    auto zf = [&](int e) {
      switch (a.n_split) {  // a power of two up to kRouterMaxSplit
        case 1: return split_sum<1>(zp + e, zs);
        case 2: return split_sum<2>(zp + e, zs);
        case 4: return split_sum<4>(zp + e, zs);
        default: return split_sum<8>(zp + e, zs);
      }
    };
    route_token<LPT, EPL>(a, t, t < a.n_tokens, sub, grp, zf, psum, zl_acc, s_hist);
  }
  route_block_partials<LPT, EPL, kRouteWaves>(a, lane, wave, psum, zl_acc, s_psum, s_zl, s_hist);
}

// ---------------------------------------------------------------------------------------
// Router projection and routing in one launch, bfloat16, up to 64 experts (LPT = E rounded up
// to a power of two, one expert per lane; NB = the 16-expert blocks of the projection). A
// workgroup of 8 waves is one routing block, taken in runs of kFusedTokens = 32 tokens: wave
// w multiplies tokens 16 (w & 1) .. + 15 of the run against every expert over reduction
// quarter w >> 1, the quarter sums of each logit land in LDS and are added in quarter order
// (the order of the split projection's partials), and the token groups then route the run's
// tokens. The block's partials are written as route_tokens_kernel writes them. No logits
// pass through HBM and one launch is saved.
// ---------------------------------------------------------------------------------------
constexpr int kFusedTokens = 32, kFusedWaves = 8;
template <int NB, int LPT>
__global__ __launch_bounds__(kFusedWaves * kWave) void route_fused_kernel(const bf16_t* __restrict__ x,
                                                                          const bf16_t* __restrict__ wg, RouteArgs a,
                                                                          int d, int k_chunk) {
  static_assert(16 * NB >= LPT, "the projection covers every expert slot");
  constexpr int kTpw = kWave / LPT;
  __shared__ float s_z[kFusedQuarters][kFusedTokens][16 * NB];
  __shared__ float s_psum[kFusedWaves][LPT];
  __shared__ int s_hist[LPT];
  __shared__ float s_zl[kFusedWaves];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int E = a.n_experts;
  const int N = a.n_tokens;
  for (int e = threadIdx.x; e < E; e += kFusedWaves * kWave) s_hist[e] = 0;

  const int sub = lane & (LPT - 1);
  const int grp = lane / LPT;
  float psum[1] = {0.f};
  float zl_acc = 0.f;
  // the block's runs of kFusedTokens tokens (uniform over the workgroup)
  for (int r0 = 0; r0 < a.tokens_per_block; r0 += kFusedTokens) {
    const int tb = blockIdx.x * a.tokens_per_block + r0;
    if (tb >= N) break;
    {
      const int half = wave & 1, quarter = wave >> 1;
      const int kb = quarter * k_chunk;
      const int ke = min(d, kb + k_chunk);
      f32x4 acc[NB];
      router_mfma16<NB>(x, wg, tb + 16 * half, 0, kb, ke, N, d, E, lane, acc);
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) s_z[quarter][16 * half + (lane >> 4) * 4 + r][b * 16 + (lane & 15)] = acc[b][r];
    }
    __syncthreads();  // (the first time also the histogram's zeros)
    constexpr int kPasses = (kFusedTokens + kTpw - 1) / kTpw;  // one for E <= 2 (half a pass for E = 1)
    for (int p = wave; p < kPasses; p += kFusedWaves) {  // wave-uniform trip count
      const int tl = p * kTpw + grp;
      const bool tok = tl < kFusedTokens && tb + tl < N;
      auto zf = [&](int e) {
        float v = 0.f;
#pragma unroll
        for (int q = 0; q < kFusedQuarters; ++q) v += s_z[q][tl][e];
        return v;
      };
      route_token<LPT, 1>(a, tb + tl, tok, sub, grp, zf, psum, zl_acc, s_hist);
    }
    __syncthreads();  // every wave is done with s_z before the next run's projection
  }
  route_block_partials<LPT, 1, kFusedWaves>(a, lane, wave, psum, zl_acc, s_psum, s_zl, s_hist);
}

// ---------------------------------------------------------------------------------------
// Final reduction over the routing blocks, one workgroup of T threads (T = 256 up to 64
// experts, else 1024; route_finalize_wave_kernel below is the one-wave form for few blocks).
// Thread (g, e) with g < G = T / E sums expert e's partials over a contiguous range of blocks
// (coalesced over e); the G range sums are then combined in a fixed order, so counts, f, P,
// L and the z-loss are bitwise reproducible. With offsets != null it goes on to the
// dispatch scan of [L7.8] §2.2 over the same blocks: offsets = exclusive scan of counts,
// and base[b][e] = offsets[e] + (assignments of expert e in blocks before b), the first
// sorted slot of block b's run of expert e; then the grouped GEMM's m-tile table.
// ---------------------------------------------------------------------------------------
// 1024 threads above 64 experts; 256 up to 64 (fewer, cheaper barriers for its ~50 steps:
// routing stage at the Mixtral shape 46 -> 41 us together with the router projection's batched
// loads, same-box A/B). Where the one-wave form fits it replaces both: no barrier at all,
// routing stage 37.7 -> 33.9 us at the Mixtral shape, 24.3 -> 21.5 us at the GPT-2-small
// shape (same-box A/B).
template <int NT>
MOE_DEV double block_sum_f64(double v, double* s_red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  __syncthreads();
  if (lane == 0) s_red[wave] = v;
  __syncthreads();
  double r = 0.0;
  for (int w = 0; w < NT / kWave; ++w) r += s_red[w];
  return r;
}

constexpr int kFinChunk = 16;
template <int kFinThreads>
__global__ __launch_bounds__(kFinThreads) void route_finalize_kernel(FinalizeArgs a) {
  __shared__ double s_p[kFinThreads];
  __shared__ int s_c[kFinThreads];
  __shared__ int s_cs[kFinThreads];
  __shared__ int s_off[kMaxExperts + 1];
  __shared__ int s_scan[kMaxExperts];
  __shared__ double s_red[kFinThreads / kWave];
  __shared__ int s_bad;
  const int tid = threadIdx.x;
  const int E = a.n_experts;
  const int nb = a.n_blocks;
  const int G = kFinThreads / E;
  const int g = tid / E;
  const int e = tid - g * E;
  const bool act = g < G;
  const int b0 = act ? (int)((long long)nb * g / G) : 0;
  const int b1 = act ? (int)((long long)nb * (g + 1) / G) : 0;
  if (tid == 0) s_bad = 0;

  // the thread's blocks in chunks of kFinChunk, every load of a chunk unconditional (an index
  // past the thread's range reads its last block, in range, and is dropped), so a chunk is one
  // round trip: a load behind a per-thread condition is waited for before the next is issued
  int c = 0;
  double p = 0.0;
  for (int j0 = b0; j0 < b1; j0 += kFinChunk) {  // b1 > b0 only for active threads
    int hv[kFinChunk];
    float pv[kFinChunk];
#pragma unroll
    for (int j = 0; j < kFinChunk; ++j) {
      const size_t o = (size_t)min(j0 + j, b1 - 1) * E + e;
      hv[j] = a.part_hist[o];
      pv[j] = a.part_p[o];
    }
#pragma unroll
    for (int j = 0; j < kFinChunk; ++j)
      if (j0 + j < b1) {
        c += hv[j];
        p += (double)pv[j];
      }
  }
  s_c[tid] = c;
  s_cs[tid] = c;
  s_p[tid] = p;
  __syncthreads();
  // P: pairwise tree over the groups; counts: inclusive scan over the groups (integers).
  int span = 1;
  while (span < G) span <<= 1;
  for (int h = span >> 1; h >= 1; h >>= 1) {
    if (act && g < h && g + h < G) s_p[tid] += s_p[tid + h * E];
    __syncthreads();
  }
  for (int o = 1; o < G; o <<= 1) {
    const int v = (act && g >= o) ? s_cs[tid - o * E] : 0;
    __syncthreads();
    s_cs[tid] += v;
    __syncthreads();
  }
  const double inv_n = a.n_tokens > 0 ? 1.0 / (double)a.n_tokens : 0.0;
  int total = 0;
  double fp = 0.0;
  if (tid < E) {
    total = s_cs[(G - 1) * E + tid];
    const double f = (double)total * inv_n;
    const double P = s_p[tid] * inv_n;
    a.counts[tid] = total;
    a.stats[tid] = (float)f;
    a.stats[E + tid] = (float)P;
    fp = f * P;
  }
  const double fp_sum = block_sum_f64<kFinThreads>(fp, s_red);
  double zl = 0.0;
  for (int b0z = 0; b0z < nb; b0z += kFinThreads * kFinChunk) {  // uniform trip count
    float zv[kFinChunk];
#pragma unroll
    for (int j = 0; j < kFinChunk; ++j) zv[j] = a.part_zl[min(b0z + j * kFinThreads + tid, nb - 1)];
#pragma unroll
    for (int j = 0; j < kFinChunk; ++j)
      if (b0z + j * kFinThreads + tid < nb) zl += (double)zv[j];
  }
  const double zl_sum = block_sum_f64<kFinThreads>(zl, s_red);
  if (tid == 0) {
    a.stats[2 * E] = (float)((double)E * fp_sum);
    a.stats[2 * E + 1] = (float)(zl_sum * inv_n);
  }
  if (!a.offsets) return;  // uniform over the block

  // offsets: exclusive scan of the counts over the experts
  int all;
  const int ex = expert_excl_scan(tid < E ? total : 0, E, s_scan, &all);
  if (tid < E) {
    s_off[tid] = ex;
    a.offsets[tid] = ex;
  }
  if (tid == 0) {
    s_off[E] = all;
    a.offsets[E] = all;
  }
  __syncthreads();
  // per-block bases: this thread's block range continues after the earlier groups' rows
  if (act) {
    int run = s_off[e] + (s_cs[tid] - s_c[tid]);
    for (int j0 = b0; j0 < b1; j0 += kFinChunk) {
      int hv[kFinChunk];
#pragma unroll
      for (int j = 0; j < kFinChunk; ++j) hv[j] = a.part_hist[(size_t)min(j0 + j, b1 - 1) * E + e];
#pragma unroll
      for (int j = 0; j < kFinChunk; ++j)
        if (j0 + j < b1) {
          a.base[(size_t)(j0 + j) * E + e] = run;
          run += hv[j];
        }
    }
  }
  if (a.tiles) {
    const int lo = tid < E ? s_off[tid] : 0;
    const int hi = tid < E ? s_off[tid + 1] : 0;
    build_tile_table(lo, hi, E, s_off[E], a.tile_bm, a.tile_narrow, a.max_tiles, a.tiles, s_scan, &s_bad);
  }
  __syncthreads();
  if (tid == 0 && a.err) a.err[0] = s_bad ? MOE_ERR_INVALID_ARG : 0;
}

// The same for up to 64 experts when every lane group's run of blocks is at most
// kFinWaveBlocks long: one wave, lane (g, e) = g E + e (g < G = 64 / E) summing expert e over
// group g's blocks, with every cross-lane step a shuffle, so the kernel has no barrier and no
// LDS. All of a lane's partials (counts, P, z-loss) are requested before the first add.
constexpr int kFinWaveBlocks = 32;

MOE_DEV double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__global__ __launch_bounds__(kWave) void route_finalize_wave_kernel(FinalizeArgs a) {
  const int lane = threadIdx.x;
  const int E = a.n_experts;
  const int nb = a.n_blocks;
  const int G = kWave / E;
  const int g = lane / E;  // g == G on the lanes past G E, which hold no group
  const int e = lane - g * E;
  const bool act = g < G;
  const int b0 = act ? nb * g / G : 0;
  const int nmine = act ? nb * (g + 1) / G - b0 : 0;  // <= kFinWaveBlocks (checked by the host)
  int hb[kFinWaveBlocks];
  float pb[kFinWaveBlocks], zb[kFinWaveBlocks];
  // Unconditional loads (an entry past the lane's run reads the last block's, in range, and is
  // zeroed after), so all of them are in flight together: a load behind a per-lane condition
  // is waited for before the next is issued.
  if (nb > 0) {
#pragma unroll
    for (int j = 0; j < kFinWaveBlocks; ++j) {
      const size_t o = (size_t)min(b0 + j, nb - 1) * E + e;  // e < E on every lane
      hb[j] = a.part_hist[o];
      pb[j] = a.part_p[o];
      zb[j] = a.part_zl[min(lane + kWave * j, nb - 1)];  // nb <= G kFinWaveBlocks <= 64 kFinWaveBlocks
    }
  } else {
#pragma unroll
    for (int j = 0; j < kFinWaveBlocks; ++j) {
      hb[j] = 0;
      pb[j] = 0.f;
      zb[j] = 0.f;
    }
  }
#pragma unroll
  for (int j = 0; j < kFinWaveBlocks; ++j) {
    if (j >= nmine) {
      hb[j] = 0;
      pb[j] = 0.f;
    }
    if (lane + kWave * j >= nb) zb[j] = 0.f;
  }
  int c = 0;
  double p = 0.0, zl = 0.0;
#pragma unroll
  for (int j = 0; j < kFinWaveBlocks; ++j) {
    c += hb[j];
    p += (double)pb[j];
    zl += (double)zb[j];
  }
  // P: pairwise tree over the groups; counts: inclusive scan over the groups (integers)
  int span = 1;
  while (span < G) span <<= 1;
  for (int h = span >> 1; h >= 1; h >>= 1) {
    const double o = __shfl(p, min(lane + h * E, kWave - 1), kWave);
    if (act && g < h && g + h < G) p += o;
  }
  int cs = c;
  for (int o = 1; o < G; o <<= 1) {
    const int u = __shfl(cs, max(lane - o * E, 0), kWave);
    if (act && g >= o) cs += u;
  }
  const int total = __shfl(cs, (G - 1) * E + e, kWave);  // expert e's count
  const double inv_n = a.n_tokens > 0 ? 1.0 / (double)a.n_tokens : 0.0;
  double fp = 0.0;
  if (lane < E) {  // group 0: p holds the tree's sum
    const double f = (double)total * inv_n;
    const double P = p * inv_n;
    a.counts[lane] = total;
    a.stats[lane] = (float)f;
    a.stats[E + lane] = (float)P;
    fp = f * P;
  }
  const double fp_sum = wave_sum_f64(fp);
  const double zl_sum = wave_sum_f64(zl);
  if (lane == 0) {
    a.stats[2 * E] = (float)((double)E * fp_sum);
    a.stats[2 * E + 1] = (float)(zl_sum * inv_n);
  }
  if (!a.offsets) return;  // uniform over the wave

  int all;
  const int ex = wave_excl_scan(lane < E ? total : 0, &all);  // offsets over the experts
  if (lane < E) a.offsets[lane] = ex;
  if (lane == 0) a.offsets[E] = all;
  const int off_e = __shfl(ex, e, kWave);
  if (act) {  // per-block bases: this lane's blocks continue after the earlier groups' rows
    int run = off_e + (cs - c);
#pragma unroll
    for (int j = 0; j < kFinWaveBlocks; ++j)
      if (j < nmine) {
        a.base[(size_t)(b0 + j) * E + e] = run;
        run += hb[j];
      }
  }
  bool bad = false;
  if (a.tiles)
    bad = build_tile_table_wave(lane < E ? ex : 0, lane < E ? ex + total : 0, E, all, a.tile_bm, a.tile_narrow,
                                a.max_tiles, a.tiles);
  if (lane == 0 && a.err) a.err[0] = bad ? MOE_ERR_INVALID_ARG : 0;
}

// ---------------------------------------------------------------------------------------
// Aux-free bias step ([L7.8] §2.5): b_e += rate * sign(mean load - load_e). One workgroup;
// the sign is taken exactly as sign(sum - E load_e) in 64-bit integers.
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void update_bias_kernel(const int32_t* __restrict__ counts, float* __restrict__ bias,
                                                           int E, float rate) {
  __shared__ long long s_part[1024 / kWave];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  long long c = 0;
  for (int e = tid; e < E; e += 1024) c += counts[e];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) c += __shfl_xor(c, o, kWave);
  if (lane == 0) s_part[wave] = c;
  __syncthreads();
  long long sum = 0;
  for (int w = 0; w < 1024 / kWave; ++w) sum += s_part[w];
  for (int e = tid; e < E; e += 1024) {
    const long long d = sum - (long long)E * counts[e];
    const float sg = d > 0 ? 1.f : (d < 0 ? -1.f : 0.f);
    bias[e] = bias[e] + rate * sg;
  }
}

hipError_t launch_update_bias(const moe_config& c, const int32_t* counts, float* bias, float rate,
                              hipStream_t stream) {
  update_bias_kernel<<<1, 1024, 0, stream>>>(counts, bias, c.n_experts, rate);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// Host-side launch sequence (no synchronisation).
// ---------------------------------------------------------------------------------------
// Experts per workgroup of the tiled router projection (E > 64).
static int router_tile_experts(int E) { return E <= 128 ? 128 : 256; }

RoutePlan plan_route(const moe_config& c) {
  RoutePlan p{};
  const long long N = c.n_tokens;
  const int E = c.n_experts;
  // Lanes per token (a power of two). Each of a token's k choices is an arg-max reduction
  // over its lanes, so fewer lanes per token mean shorter cross-lane chains and more tokens
  // side by side in a wave. Up to 64 experts a lane holds one. Beyond that a lane holds up
  // to 16 experts, and the lanes per token shrink as long as the token groups (N lpt / 64,
  // one wave pass each) stay at least 4096, about 16 per CU. Fewer groups leave too few
  // waves to hide the reductions' latency: on 128 experts x 16384 tokens and 256 x 4096
  // tokens, 4096 groups timed best of 1024 to 16384. Lane j < k of a group keeps the
  // token's j-th choice, so a group has at least k lanes (k <= kMaxTopK <= 64).
  const int k = c.top_k;
  p.lpt = 1;
  if (E <= kWave) {
    while (p.lpt < E) p.lpt <<= 1;
  } else {
    while (p.lpt < kWave && (p.lpt * 16 < E || p.lpt < k || N * p.lpt < 64ll * 4096)) p.lpt <<= 1;
  }
  p.epl = 1;
  while (p.lpt * p.epl < E) p.epl <<= 1;
  // Blocks of tokens: enough tokens per block that the per-block partial arrays ([blocks][E])
  // stay within 64K entries, which the single-workgroup final reduction reads twice.
  p.fused = c.dtype == MOE_BF16 && E <= kWave;
  if (p.fused) {
    // route_fused_kernel: a block is `iters` consecutive runs of kFusedTokens tokens, the
    // reduction cut into kFusedQuarters quarters of whole 32-wide steps
    const long long iters = std::max<long long>(1, (N * E + 65536ll * kFusedTokens - 1) / (65536ll * kFusedTokens));
    p.tokens_per_block = (int)(kFusedTokens * iters);
    p.tokens_per_wave = p.tokens_per_block;
    p.n_blocks = (int)((N + p.tokens_per_block - 1) / p.tokens_per_block);
    p.n_split = kFusedQuarters;
    p.k_chunk = ((c.d_model + kFusedQuarters - 1) / kFusedQuarters + 31) / 32 * 32;
    return p;
  }
  const int tpw = kWave / p.lpt;
  const int waves = route_waves(p.epl);
  const long long per_block_min = (long long)waves * tpw;
  long long iters = std::max<long long>(1, N * E / (65536ll * per_block_min));
  while (((N + per_block_min * iters - 1) / (per_block_min * iters)) * E > 65536) ++iters;
  p.tokens_per_wave = (int)(tpw * iters);
  p.tokens_per_block = waves * p.tokens_per_wave;
  p.n_blocks = (int)((N + p.tokens_per_block - 1) / p.tokens_per_block);
  if (c.dtype == MOE_BF16) {
    // Split the reduction so that the projection launches several workgroups per CU even
    // for a few thousand tokens; each split writes its own partial z.
    const int e_blocks = (E + router_tile_experts(E) - 1) / router_tile_experts(E);
    const long long base = ((N + 63) / 64) * e_blocks;
    int split = 1;
    while (split < kRouterMaxSplit && base * split < 512 && (c.d_model / (split * 2)) >= 256) split *= 2;
    p.n_split = split;
    p.k_chunk = ((c.d_model / split) + 31) / 32 * 32;
  } else {
    p.n_split = 1;
    p.k_chunk = c.d_model;
  }
  return p;
}

void carve_route(const moe_config& c, WsCarver& w, WsLayout* L) {
  const RoutePlan p = plan_route(c);
  const size_t N = (size_t)c.n_tokens, E = (size_t)c.n_experts;
  float* zpart = w.take_t<float>(p.fused ? 0 : (size_t)p.n_split * N * E);  // the fused kernel keeps z in LDS
  float* part_p = w.take_t<float>((size_t)p.n_blocks * E);
  int* part_hist = w.take_t<int>((size_t)p.n_blocks * E);
  float* part_zl = w.take_t<float>((size_t)p.n_blocks);
  if (L) {
    L->zpart = zpart;
    L->part_p = part_p;
    L->part_hist = part_hist;
    L->part_zl = part_zl;
  }
}

// Per-block dispatch bases of the fused path ([route blocks][E]), carved by moe_forward.
size_t route_base_ints(const moe_config& c) { return (size_t)plan_route(c).n_blocks * c.n_experts; }
int route_tokens_per_block(const moe_config& c) { return plan_route(c).tokens_per_block; }

template <int LPT, int EPL>
static void launch_tokens(const RoutePlan& p, const RouteArgs& ra, hipStream_t stream) {
  route_tokens_kernel<LPT, EPL><<<p.n_blocks, route_waves(EPL) * kWave, 0, stream>>>(ra);
}

hipError_t launch_route(const moe_config& c, const WsLayout& L, const void* x, const void* w_router,
                        const float* logit_bias, const float* sel_bias, int32_t* topk_ids,
                        float* topk_w, int32_t* counts, float* stats, float* logits_out,
                        float* gap_out, bool fuse_dispatch, hipStream_t stream) {
  const RoutePlan p = plan_route(c);
  const int N = (int)c.n_tokens, E = c.n_experts, d = c.d_model;
  if (N > 0) {
    RouteArgs ra{};
    ra.zpart = L.zpart;
    ra.n_split = p.n_split;
    ra.logit_bias = logit_bias;
    ra.sel_bias = sel_bias;
    ra.n_tokens = N;
    ra.n_experts = E;
    ra.top_k = c.top_k;
    ra.router = c.router;
    ra.norm_topk = c.norm_topk;
    ra.routed_scaling = c.routed_scaling;
    ra.tokens_per_wave = p.tokens_per_wave;
    ra.tokens_per_block = p.tokens_per_block;
    ra.topk_ids = topk_ids;
    ra.topk_w = topk_w;
    ra.logits_out = logits_out;
    ra.gap_out = gap_out;
    ra.part_p = L.part_p;
    ra.part_hist = L.part_hist;
    ra.part_zl = L.part_zl;
    if (p.fused) {
      auto xb = static_cast<const bf16_t*>(x);
      auto wb = static_cast<const bf16_t*>(w_router);
      const dim3 grid(p.n_blocks), block(kFusedWaves * kWave);
      switch (p.lpt) {
        case 1: route_fused_kernel<1, 1><<<grid, block, 0, stream>>>(xb, wb, ra, d, p.k_chunk); break;
        case 2: route_fused_kernel<1, 2><<<grid, block, 0, stream>>>(xb, wb, ra, d, p.k_chunk); break;
        case 4: route_fused_kernel<1, 4><<<grid, block, 0, stream>>>(xb, wb, ra, d, p.k_chunk); break;
        case 8: route_fused_kernel<1, 8><<<grid, block, 0, stream>>>(xb, wb, ra, d, p.k_chunk); break;
        case 16: route_fused_kernel<1, 16><<<grid, block, 0, stream>>>(xb, wb, ra, d, p.k_chunk); break;
        case 32: route_fused_kernel<2, 32><<<grid, block, 0, stream>>>(xb, wb, ra, d, p.k_chunk); break;
        default: route_fused_kernel<4, 64><<<grid, block, 0, stream>>>(xb, wb, ra, d, p.k_chunk); break;
      }
    } else {
      if (c.dtype == MOE_BF16) {  // E > 64
        auto xb = static_cast<const bf16_t*>(x);
        auto wb = static_cast<const bf16_t*>(w_router);
        const int te = router_tile_experts(E);
        dim3 grid((N + 63) / 64, (E + te - 1) / te, p.n_split);
        if (te == 128) router_gemm_tiled_kernel<2><<<grid, 128, 0, stream>>>(xb, wb, L.zpart, N, d, E, p.k_chunk);
        else router_gemm_tiled_kernel<4><<<grid, 256, 0, stream>>>(xb, wb, L.zpart, N, d, E, p.k_chunk);
      } else {
        router_gemm_f32_kernel<<<(N + 3) / 4, 256, 0, stream>>>(
            static_cast<const float*>(x), static_cast<const float*>(w_router), L.zpart, N, d, E);
      }
      switch (p.lpt * 100 + p.epl) {
        case 101: launch_tokens<1, 1>(p, ra, stream); break;
        case 201: launch_tokens<2, 1>(p, ra, stream); break;
        case 401: launch_tokens<4, 1>(p, ra, stream); break;
        case 801: launch_tokens<8, 1>(p, ra, stream); break;
        case 1601: launch_tokens<16, 1>(p, ra, stream); break;
        case 3201: launch_tokens<32, 1>(p, ra, stream); break;
        case 6401: launch_tokens<64, 1>(p, ra, stream); break;
        case 816: launch_tokens<8, 16>(p, ra, stream); break;
        case 1608: launch_tokens<16, 8>(p, ra, stream); break;
        case 1616: launch_tokens<16, 16>(p, ra, stream); break;
        case 3204: launch_tokens<32, 4>(p, ra, stream); break;
        case 3208: launch_tokens<32, 8>(p, ra, stream); break;
        case 3216: launch_tokens<32, 16>(p, ra, stream); break;
        case 6402: launch_tokens<64, 2>(p, ra, stream); break;
        case 6404: launch_tokens<64, 4>(p, ra, stream); break;
        case 6408: launch_tokens<64, 8>(p, ra, stream); break;
        default: launch_tokens<64, 16>(p, ra, stream); break;
      }
    }
  }
  FinalizeArgs fa{};
  fa.part_p = L.part_p;
  fa.part_hist = L.part_hist;
  fa.part_zl = L.part_zl;
  fa.n_blocks = p.n_blocks;
  fa.n_tokens = c.n_tokens;
  fa.n_experts = E;
  fa.counts = counts;
  fa.stats = stats;
  if (fuse_dispatch) {
    fa.offsets = L.offsets;
    fa.base = L.fbase;
    fa.err = L.err;
    fa.tiles = L.tiles;
    fa.tile_bm = ffn_tile_rows(c);
    fa.tile_narrow = ffn_narrow_rows(c);
    fa.max_tiles = ffn_max_m_tiles(c);
  }
  if (E <= 64 && (p.n_blocks + kWave / E - 1) / (kWave / E) <= kFinWaveBlocks)
    route_finalize_wave_kernel<<<1, kWave, 0, stream>>>(fa);
  else if (E <= 64) route_finalize_kernel<256><<<1, 256, 0, stream>>>(fa);
  else route_finalize_kernel<1024><<<1, 1024, 0, stream>>>(fa);
  return hipGetLastError();
}

}  // namespace moe
