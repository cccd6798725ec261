// Routing kernels: router projection z = x W_g^T, then per token softmax, selection score,
// top-k (largest first, ties to the lowest id), gates, and per-block partials of the
// Switch statistics; a final single-workgroup kernel reduces the partials in a fixed order.
//
// Follows "Mixture of Experts: routing, sorted dispatch, Switch aux loss, aux-free bias"
// (L7.8) §2 symbol table and §2.1 routers table, §2.3 load-balancing loss, §2.5 (the bias
// chooses, never weighs); "15. Mixture of Experts" (RustingBrain) §15.2 routing, §15.3 z-loss.
#include "moe_internal.h"

namespace moe {

// ---------------------------------------------------------------------------------------
// Router projection, bfloat16 inputs, float32 accumulation on MFMA (v_mfma_f32_16x16x32_bf16).
// Workgroup = 4 waves; each wave owns 16 tokens and NB blocks of 16 experts; grid.z splits
// the reduction axis into independent chunks whose partial sums land in zpart[split][N][E]
// and are added in split order by the epilogue kernel (deterministic, no atomics).
// ---------------------------------------------------------------------------------------
template <int NB>
__global__ __launch_bounds__(256) void router_gemm_bf16_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ wg, float* __restrict__ zpart,
    int n_tokens, int d, int n_experts, int k_chunk) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * 64 + wave * 16;
  const int e0 = blockIdx.y * (16 * NB);
  const int kb = blockIdx.z * k_chunk;
  const int ke = min(d, kb + k_chunk);
  const int row = lane & 15;
  const int kq = (lane >> 4) * 8;

  f32x4 acc[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};

  const bool a_ok = (t0 + row) < n_tokens;
  const bf16_t* arow = x + (size_t)(a_ok ? t0 + row : 0) * d;
  for (int k = kb; k < ke; k += 32) {
    const int kk = k + kq;
    uint4 av = make_uint4(0, 0, 0, 0);
    if (a_ok && kk < ke) av = *reinterpret_cast<const uint4*>(arow + kk);
    bf16x8 a = __builtin_bit_cast(bf16x8, av);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int e = e0 + b * 16 + row;
      uint4 bv = make_uint4(0, 0, 0, 0);
      if (e < n_experts && kk < ke) bv = *reinterpret_cast<const uint4*>(wg + (size_t)e * d + kk);
      acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, bv), acc[b], 0, 0, 0);
    }
  }
  float* zp = zpart + (size_t)blockIdx.z * n_tokens * n_experts;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int e = e0 + b * 16 + (lane & 15);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = t0 + (lane >> 4) * 4 + r;
      if (t < n_tokens && e < n_experts) zp[(size_t)t * n_experts + e] = acc[b][r];
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
// Per-token routing. One wave per token; lane l holds experts l, l+64, ... (up to 16 each).
// ---------------------------------------------------------------------------------------
constexpr int kEpl = kMaxExperts / 64;  // experts per lane, upper bound

// (score desc, id asc): a beats b when its score is larger, or equal with a lower id.
MOE_DEV bool beats(float s, int id, float s2, int id2) { return s > s2 || (s == s2 && id < id2); }

__global__ __launch_bounds__(256) void route_tokens_kernel(RouteArgs a) {
  __shared__ float s_psum[4][kMaxExperts];
  __shared__ int s_hist[kMaxExperts];
  __shared__ float s_zl[4];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int E = a.n_experts;
  const int k = a.top_k;
  const int epl = (E + 63) >> 6;

  for (int e = threadIdx.x; e < E; e += 256) s_hist[e] = 0;
  __syncthreads();

  float psum[kEpl];
#pragma unroll
  for (int i = 0; i < kEpl; ++i) psum[i] = 0.f;
  float zl_acc = 0.f;

  const int tok_begin = blockIdx.x * a.tokens_per_block + wave * a.tokens_per_wave;
  const int tok_end = min((int)a.n_tokens, tok_begin + a.tokens_per_wave);
  for (int t = tok_begin; t < tok_end; ++t) {
    float z[kEpl], s[kEpl], ex[kEpl];
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < kEpl; ++i) {
      const int e = lane + 64 * i;
      z[i] = -INFINITY;
      if (i < epl && e < E) {
        float v = 0.f;
        for (int sp = 0; sp < a.n_split; ++sp) v += a.zpart[((size_t)sp * a.n_tokens + t) * E + e];
        if (a.logit_bias) v += a.logit_bias[e];
        z[i] = v;
        m = fmaxf(m, v);
        if (a.logits_out) a.logits_out[(size_t)t * E + e] = v;
      }
    }
    m = wave_max(m);
    float lsum = 0.f;
#pragma unroll
    for (int i = 0; i < kEpl; ++i) {
      ex[i] = (i < epl && lane + 64 * i < E) ? expf(z[i] - m) : 0.f;
      lsum += ex[i];
    }
    const float sum = wave_sum(lsum);
    const float inv_sum = 1.0f / sum;
    if (lane == 0) {
      const float lse = m + logf(sum);
      zl_acc += lse * lse;
    }
#pragma unroll
    for (int i = 0; i < kEpl; ++i) {
      const int e = lane + 64 * i;
      const bool ok = i < epl && e < E;
      psum[i] += ok ? ex[i] * inv_sum : 0.f;
      float sc = (a.router == MOE_ROUTER_SIGMOID) ? sigmoid_f(z[i]) : z[i];
      if (ok && a.sel_bias) sc += a.sel_bias[e];
      if (sc != sc) sc = -INFINITY;  // a NaN score ranks last, so k valid ids are still chosen
      s[i] = ok ? sc : -INFINITY;
    }

    // k rounds of a wave arg-max on (score desc, id asc); one more for the margin.
    uint32_t taken = 0;
    int my_id = -1;
    float my_u = 0.f, last_s = 0.f, gap = INFINITY;
    const int rounds = (k < E) ? k + 1 : k;
    for (int j = 0; j < rounds; ++j) {
      float bs = -INFINITY;
      int bi = 0x7fffffff;
#pragma unroll
      for (int i = 0; i < kEpl; ++i) {
        const int e = lane + 64 * i;
        if (i < epl && e < E && !((taken >> i) & 1u) && beats(s[i], e, bs, bi)) {
          bs = s[i];
          bi = e;
        }
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        const float os = __shfl_xor(bs, o, 64);
        const int oi = __shfl_xor(bi, o, 64);
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
      const int slot = bi >> 6;
      float mine = 0.f;
#pragma unroll
      for (int i = 0; i < kEpl; ++i)
        if (i == slot) mine = (a.router == MOE_ROUTER_SIGMOID) ? sigmoid_f(z[i]) : ex[i];
      const float u = __shfl(mine, bi & 63, 64);
      if (lane == (bi & 63)) taken |= 1u << slot;
      if (lane == j) {
        my_id = bi;
        my_u = u;
      }
    }
    // gates ([L7.8] §2.1): the softmax routers renormalise exp(z - m) over the chosen set
    // (= p_T / sum p_T = softmax over the chosen logits); without renormalisation the
    // softmax_topk gate is p itself. The sigmoid router renormalises sigmoid(z_T).
    const float usum = wave_sum(lane < k ? my_u : 0.f);
    if (lane < k) {
      float w;
      if (a.router == MOE_ROUTER_TOPK_SOFTMAX || a.norm_topk) w = my_u / usum;
      else if (a.router == MOE_ROUTER_SOFTMAX_TOPK) w = my_u * inv_sum;
      else w = my_u;
      w *= a.routed_scaling;
      a.topk_ids[(size_t)t * k + lane] = my_id;
      a.topk_w[(size_t)t * k + lane] = w;
      if (my_id >= 0 && my_id < E) atomicAdd(&s_hist[my_id], 1);  // integer adds: order-independent
    }
    if (a.gap_out && lane == 0) a.gap_out[t] = gap;
  }

  // Deterministic block partials: waves' per-expert sums combined in wave order.
#pragma unroll
  for (int i = 0; i < kEpl; ++i) {
    const int e = lane + 64 * i;
    if (i < epl && e < E) s_psum[wave][e] = psum[i];
  }
  if (lane == 0) s_zl[wave] = zl_acc;
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) {
    a.part_p[(size_t)blockIdx.x * E + e] = ((s_psum[0][e] + s_psum[1][e]) + s_psum[2][e]) + s_psum[3][e];
    a.part_hist[(size_t)blockIdx.x * E + e] = s_hist[e];
  }
  if (threadIdx.x == 0) a.part_zl[blockIdx.x] = ((s_zl[0] + s_zl[1]) + s_zl[2]) + s_zl[3];
}

// Final statistics: counts, f, P, L = E sum f P and the z-loss, reduced over the block
// partials in block order, in double precision, by one workgroup.
__global__ __launch_bounds__(256) void route_finalize_kernel(
    const float* __restrict__ part_p, const int* __restrict__ part_hist,
    const float* __restrict__ part_zl, int n_blocks, long long n_tokens, int E,
    int* __restrict__ counts, float* __restrict__ stats) {
  __shared__ double s_red[256];
  const double inv_n = n_tokens > 0 ? 1.0 / (double)n_tokens : 0.0;
  double fp_acc = 0.0;
  for (int e = threadIdx.x; e < E; e += 256) {
    long long c = 0;
    double p = 0.0;
    for (int b = 0; b < n_blocks; ++b) {
      c += part_hist[(size_t)b * E + e];
      p += (double)part_p[(size_t)b * E + e];
    }
    counts[e] = (int)c;
    const double f = (double)c * inv_n;
    const double P = p * inv_n;
    stats[e] = (float)f;
    stats[E + e] = (float)P;
    fp_acc += f * P;
  }
  s_red[threadIdx.x] = fp_acc;
  __syncthreads();
  for (int o = 128; o >= 1; o >>= 1) {
    if (threadIdx.x < o) s_red[threadIdx.x] += s_red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    stats[2 * E] = (float)((double)E * s_red[0]);
    double zl = 0.0;
    for (int b = 0; b < n_blocks; ++b) zl += (double)part_zl[b];
    stats[2 * E + 1] = (float)(zl * inv_n);
  }
}

// ---------------------------------------------------------------------------------------
// Host-side launch sequence (no synchronisation).
// ---------------------------------------------------------------------------------------
RoutePlan plan_route(const moe_config& c) {
  RoutePlan p{};
  const long long N = c.n_tokens;
  p.tokens_per_wave = 8;
  p.tokens_per_block = 4 * p.tokens_per_wave;
  p.n_blocks = (int)((N + p.tokens_per_block - 1) / p.tokens_per_block);
  if (c.dtype == MOE_BF16) {
    // Split the reduction so that the projection launches several waves of workgroups per
    // CU even for a few thousand tokens; each split writes its own partial z.
    const int e_blocks = (c.n_experts + 255) / 256;
    const long long base = ((N + 63) / 64) * e_blocks;
    int split = 1;
    while (split < 8 && base * split < 1024 && (c.d_model / (split * 2)) >= 256) split *= 2;
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
  float* zpart = w.take_t<float>((size_t)p.n_split * N * E);
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

hipError_t launch_route(const moe_config& c, const WsLayout& L, const void* x, const void* w_router,
                        const float* logit_bias, const float* sel_bias, int32_t* topk_ids,
                        float* topk_w, int32_t* counts, float* stats, float* logits_out,
                        float* gap_out, hipStream_t stream) {
  const RoutePlan p = plan_route(c);
  const int N = (int)c.n_tokens, E = c.n_experts, d = c.d_model;
  if (N > 0) {
    if (c.dtype == MOE_BF16) {
      const int eb = (E <= 16) ? 1 : (E <= 32) ? 2 : (E <= 64) ? 4 : (E <= 128) ? 8 : 16;
      dim3 grid((N + 63) / 64, (E + 16 * eb - 1) / (16 * eb), p.n_split);
      auto xb = static_cast<const bf16_t*>(x);
      auto wb = static_cast<const bf16_t*>(w_router);
      switch (eb) {
        case 1: router_gemm_bf16_kernel<1><<<grid, 256, 0, stream>>>(xb, wb, L.zpart, N, d, E, p.k_chunk); break;
        case 2: router_gemm_bf16_kernel<2><<<grid, 256, 0, stream>>>(xb, wb, L.zpart, N, d, E, p.k_chunk); break;
        case 4: router_gemm_bf16_kernel<4><<<grid, 256, 0, stream>>>(xb, wb, L.zpart, N, d, E, p.k_chunk); break;
        case 8: router_gemm_bf16_kernel<8><<<grid, 256, 0, stream>>>(xb, wb, L.zpart, N, d, E, p.k_chunk); break;
        default: router_gemm_bf16_kernel<16><<<grid, 256, 0, stream>>>(xb, wb, L.zpart, N, d, E, p.k_chunk); break;
      }
    } else {
      router_gemm_f32_kernel<<<(N + 3) / 4, 256, 0, stream>>>(
          static_cast<const float*>(x), static_cast<const float*>(w_router), L.zpart, N, d, E);
    }
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
    route_tokens_kernel<<<p.n_blocks, 256, 0, stream>>>(ra);
  }
  route_finalize_kernel<<<1, 256, 0, stream>>>(L.part_p, L.part_hist, L.part_zl, p.n_blocks,
                                                c.n_tokens, E, counts, stats);
  return hipGetLastError();
}

}  // namespace moe
