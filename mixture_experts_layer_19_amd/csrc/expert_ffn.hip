// Expert FFN over ragged per-expert slices as grouped GEMMs ("Mixture of Experts: routing,
// sorted dispatch, Switch aux loss, aux-free bias" (L7.8) §2.2: each expert runs once on its
// contiguous slice; "15. Mixture of Experts" (RustingBrain) "Dropless": ragged batches).
//
//   up:   h = gelu(x_s W1^T + b1)              (GELU MLP, optional bias)
//         h = silu(x_s W1^T) * (x_s W3^T)      (SwiGLU; gate and up computed by the same
//                                                workgroup for the same columns, fused)
//   down: y_s = (h W2^T + b2) * gate_sorted    (gate applied before the single rounding)
//
// The m-tiles of every expert are listed once per call by tile_table_kernel from offsets,
// so the GEMM grids are sized from the worst case on the host and idle experts cost
// nothing: they own no tile and their weights are never read.
#include "moe_internal.h"

namespace moe {

enum Epi { kEpiGelu = 0, kEpiSwiglu = 1, kEpiDown = 2 };

// ---------------------------------------------------------------------------------------
// Tile table: tiles[0] = number of m-tiles; tile t is tiles[4 + 4t ..] = (expert, first
// row, rows in the tile). Offsets outside [0, rows] or decreasing are clamped, the list is
// capped at max_tiles (so no access leaves the buffers) and the error word is set.
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void tile_table_kernel(const int* __restrict__ offsets, int E, int rows,
                                                          int bm, int max_tiles, int* __restrict__ tiles,
                                                          int* __restrict__ err) {
  __shared__ int s_scan[kMaxExperts];
  __shared__ int s_bad;
  const int e = threadIdx.x;
  if (e == 0) s_bad = 0;
  __syncthreads();
  int lo = 0, hi = 0, n = 0;
  if (e < E) {
    lo = offsets[e];
    hi = offsets[e + 1];
    if (lo < 0 || hi > rows || hi < lo || (e == 0 && lo != 0)) s_bad = 1;
    lo = min(max(lo, 0), rows);
    hi = min(max(hi, lo), rows);
    n = (hi - lo + bm - 1) / bm;
    s_scan[e] = n;
  }
  __syncthreads();
  for (int o = 1; o < E; o <<= 1) {
    int v = 0;
    if (e < E && e >= o) v = s_scan[e - o];
    __syncthreads();
    if (e < E) s_scan[e] += v;
    __syncthreads();
  }
  if (e < E) {
    const int start = s_scan[e] - n;
    for (int t = 0; t < n && start + t < max_tiles; ++t) {
      const int r0 = lo + t * bm;
      int* q = tiles + 4 + 4 * (start + t);
      q[0] = e;
      q[1] = r0;
      q[2] = min(bm, hi - r0);
    }
    if (e == E - 1) {
      if (s_scan[e] > max_tiles) s_bad = 1;
      tiles[0] = min(s_scan[e], max_tiles);
    }
  }
  __syncthreads();
  if (e == 0 && s_bad && err) err[0] = MOE_ERR_INVALID_ARG;
}

struct GemmArgs {
  const void* a;        // [rows][K] T: x_sorted (up) or h (down)
  const void* b0;       // [E][N_b][K] T: W1 (up) or W2 (down)
  const void* b1;       // [E][N_b][K] T: W3 (SwiGLU up) or null
  const void* bias;     // [E][N_out] T or null
  const float* gate;    // [rows] or null (down only)
  void* c;              // [rows][N_out] T: h (up) or y_sorted (down)
  const int* tiles;     // tile table
  int K, n_out;
};

// ---------------------------------------------------------------------------------------
// bfloat16 grouped GEMM on MFMA (v_mfma_f32_16x16x32_bf16), float32 accumulation.
// Workgroup tile: 128 rows x 128 B-rows (GELU / down: 128 output columns; SwiGLU: 64 gate
// rows and the 64 matching up rows -> 64 output columns), K staged 64 at a time in LDS with
// rows padded to 72 elements so that 16-byte reads of 8 consecutive rows hit distinct banks.
// 4 waves in a 2 x 2 grid; each wave owns 64 rows x 64 B-rows = 4 x 4 MFMA blocks.
// ---------------------------------------------------------------------------------------
constexpr int kBM = 128, kBNB = 128, kBK = 64, kLdsRow = kBK + 8;

template <int EPI>
__global__ __launch_bounds__(256) void expert_gemm_bf16_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[kBM * kLdsRow];
  __shared__ __attribute__((aligned(16))) uint16_t sB[kBNB * kLdsRow];

  const int n_tiles_m = g.tiles[0];
  const int mt = blockIdx.x;
  if (mt >= n_tiles_m) return;
  const int e = g.tiles[4 + 4 * mt];
  const int row0 = g.tiles[5 + 4 * mt];
  const int rows_valid = g.tiles[6 + 4 * mt];
  const int K = g.K;
  const int n_out = g.n_out;
  constexpr int kColsPerTile = (EPI == kEpiSwiglu) ? 64 : 128;
  const int n0 = blockIdx.y * kColsPerTile;
  const int nb_rows = (EPI == kEpiSwiglu) ? n_out : n_out;  // rows of each B matrix

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;

  const uint16_t* A = static_cast<const uint16_t*>(g.a);
  const uint16_t* B0 = static_cast<const uint16_t*>(g.b0) + (size_t)e * nb_rows * K;
  const uint16_t* B1 = (EPI == kEpiSwiglu) ? static_cast<const uint16_t*>(g.b1) + (size_t)e * nb_rows * K : nullptr;

  // Per-thread global chunks: chunk c = tid + 256 q, row = c / 8, 16-byte column = c % 8.
  const uint16_t* a_src[4];
  const uint16_t* b_src[4];
  bool a_ok[4], b_ok[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int c = tid + 256 * q;
    const int r = c >> 3, kc = (c & 7) * 8;
    a_ok[q] = r < rows_valid;
    a_src[q] = A + (size_t)(row0 + (a_ok[q] ? r : 0)) * K + kc;
    int col;
    const uint16_t* base;
    if (EPI == kEpiSwiglu) {
      const int wq = r >> 6, qq = r & 63;
      col = n0 + wq * 32 + (qq & 31);
      base = (qq >= 32) ? B1 : B0;
    } else {
      col = n0 + r;
      base = B0;
    }
    b_ok[q] = col < nb_rows;
    b_src[q] = base + (size_t)(b_ok[q] ? col : 0) * K + kc;
  }

  uint4 ra[4], rb[4];
  auto load_tile = [&](int k0) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int kc = ((tid + 256 * q) & 7) * 8;
      const bool kin = (k0 + kc) < K;
      ra[q] = (a_ok[q] && kin) ? *reinterpret_cast<const uint4*>(a_src[q] + k0) : make_uint4(0, 0, 0, 0);
      rb[q] = (b_ok[q] && kin) ? *reinterpret_cast<const uint4*>(b_src[q] + k0) : make_uint4(0, 0, 0, 0);
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  load_tile(0);
  for (int k0 = 0; k0 < K; k0 += kBK) {
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c = tid + 256 * q;
      const int r = c >> 3, kc = (c & 7) * 8;
      *reinterpret_cast<uint4*>(&sA[r * kLdsRow + kc]) = ra[q];
      *reinterpret_cast<uint4*>(&sB[r * kLdsRow + kc]) = rb[q];
    }
    __syncthreads();
    if (k0 + kBK < K) load_tile(k0 + kBK);
#pragma unroll
    for (int ks = 0; ks < kBK; ks += 32) {
      const int kq = ks + (lane >> 4) * 8;
      bf16x8 af[4], bfr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = wm * 64 + i * 16 + (lane & 15);
        af[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(&sA[r * kLdsRow + kq]));
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = wn * 64 + j * 16 + (lane & 15);
        bfr[j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(&sB[r * kLdsRow + kq]));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  }

  // Epilogue: lane holds rows (lane >> 4) * 4 + r and column lane & 15 of each 16 x 16 block.
  uint16_t* C = static_cast<uint16_t*>(g.c);
  const uint16_t* bias = g.bias ? static_cast<const uint16_t*>(g.bias) + (size_t)e * n_out : nullptr;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int lr = wm * 64 + i * 16 + (lane >> 4) * 4 + r;
      if (lr >= rows_valid) continue;
      const int row = row0 + lr;
      if (EPI == kEpiSwiglu) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int col = n0 + wn * 32 + j * 16 + (lane & 15);
          if (col < n_out) {
            const float gv = acc[i][j][r], uv = acc[i][j + 2][r];
            C[(size_t)row * n_out + col] = f32_to_bf16(silu_f(gv) * uv);
          }
        }
      } else {
        const float gs = (EPI == kEpiDown && g.gate) ? g.gate[row] : 1.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int col = n0 + wn * 64 + j * 16 + (lane & 15);
          if (col < n_out) {
            float v = acc[i][j][r];
            if (bias) v += bf16_to_f32(bias[col]);
            if (EPI == kEpiGelu) v = gelu_erf(v);
            else v *= gs;
            C[(size_t)row * n_out + col] = f32_to_bf16(v);
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
// float32 grouped GEMM with FMA: 64 rows x 64 output columns per workgroup, K staged 16 at
// a time in LDS (k-major, so each thread's 4 x 4 register block reads broadcast rows).
// SwiGLU keeps a gate and an up accumulator for the same columns.
// ---------------------------------------------------------------------------------------
constexpr int kFBM = 64, kFBN = 64, kFBK = 16;

template <int EPI>
__global__ __launch_bounds__(256) void expert_gemm_f32_kernel(GemmArgs g) {
  __shared__ float sA[kFBK][kFBM + 4];
  __shared__ float sB[kFBK][kFBN + 4];
  __shared__ float sU[kFBK][kFBN + 4];
  const int n_tiles_m = g.tiles[0];
  const int mt = blockIdx.x;
  if (mt >= n_tiles_m) return;
  const int e = g.tiles[4 + 4 * mt];
  const int row0 = g.tiles[5 + 4 * mt];
  const int rows_valid = g.tiles[6 + 4 * mt];
  const int K = g.K, n_out = g.n_out;
  const int n0 = blockIdx.y * kFBN;
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const float* A = static_cast<const float*>(g.a);
  const float* B0 = static_cast<const float*>(g.b0) + (size_t)e * n_out * K;
  const float* B1 = (EPI == kEpiSwiglu) ? static_cast<const float*>(g.b1) + (size_t)e * n_out * K : nullptr;

  float acc[4][4] = {}, accu[4][4] = {};
  const int lr = tid >> 2, lk = (tid & 3) * 4;  // loader: row lr, 4 floats at lk
  for (int k0 = 0; k0 < K; k0 += kFBK) {
    const bool kin = (k0 + lk) < K;
    float4 va = make_float4(0, 0, 0, 0), vb = va, vu = va;
    if (lr < rows_valid && kin) va = *reinterpret_cast<const float4*>(A + (size_t)(row0 + lr) * K + k0 + lk);
    if (n0 + lr < n_out && kin) {
      vb = *reinterpret_cast<const float4*>(B0 + (size_t)(n0 + lr) * K + k0 + lk);
      if (EPI == kEpiSwiglu) vu = *reinterpret_cast<const float4*>(B1 + (size_t)(n0 + lr) * K + k0 + lk);
    }
    __syncthreads();
    sA[lk + 0][lr] = va.x; sA[lk + 1][lr] = va.y; sA[lk + 2][lr] = va.z; sA[lk + 3][lr] = va.w;
    sB[lk + 0][lr] = vb.x; sB[lk + 1][lr] = vb.y; sB[lk + 2][lr] = vb.z; sB[lk + 3][lr] = vb.w;
    if (EPI == kEpiSwiglu) {
      sU[lk + 0][lr] = vu.x; sU[lk + 1][lr] = vu.y; sU[lk + 2][lr] = vu.z; sU[lk + 3][lr] = vu.w;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kFBK; ++kk) {
      float av[4], bv[4], uv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = sA[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bv[j] = sB[kk][tx * 4 + j];
        if (EPI == kEpiSwiglu) uv[j] = sU[kk][tx * 4 + j];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
          if (EPI == kEpiSwiglu) accu[i][j] = fmaf(av[i], uv[j], accu[i][j]);
        }
    }
  }
  float* C = static_cast<float*>(g.c);
  const float* bias = g.bias ? static_cast<const float*>(g.bias) + (size_t)e * n_out : nullptr;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int lrow = ty * 4 + i;
    if (lrow >= rows_valid) continue;
    const int row = row0 + lrow;
    const float gs = (EPI == kEpiDown && g.gate) ? g.gate[row] : 1.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + tx * 4 + j;
      if (col >= n_out) continue;
      float v = acc[i][j];
      if (EPI == kEpiSwiglu) v = silu_f(v) * accu[i][j];
      else {
        if (bias) v += bias[col];
        v = (EPI == kEpiGelu) ? gelu_erf(v) : v * gs;
      }
      C[(size_t)row * n_out + col] = v;
    }
  }
}

// ---------------------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------------------
static int tile_rows(const moe_config& c) { return c.dtype == MOE_BF16 ? kBM : kFBM; }

static int max_m_tiles(const moe_config& c) {
  const long long A = c.n_tokens * c.top_k;
  const int bm = tile_rows(c);
  return (int)((A + bm - 1) / bm) + c.n_experts;
}

void carve_ffn(const moe_config& c, WsCarver& w, WsLayout* L) {
  const size_t A = (size_t)(c.n_tokens * c.top_k);
  int* tiles = w.take_t<int>(4 + 4 * (size_t)max_m_tiles(c));
  void* h = w.take(A * (size_t)c.d_ff * elem_size(c));
  if (L) {
    L->tiles = tiles;
    L->h = h;
  }
}

hipError_t launch_ffn_tiles(const moe_config& c, const WsLayout& L, const int32_t* offsets, hipStream_t stream) {
  const int A = (int)(c.n_tokens * c.top_k);
  if (A == 0) return hipGetLastError();
  tile_table_kernel<<<1, 1024, 0, stream>>>(offsets, c.n_experts, A, tile_rows(c), max_m_tiles(c), L.tiles, L.err);
  return hipGetLastError();
}

hipError_t launch_ffn_up(const moe_config& c, const WsLayout& L, const void* x_sorted,
                         const int32_t* offsets, const void* w1, const void* w3, const void* b1,
                         hipStream_t stream) {
  const int A = (int)(c.n_tokens * c.top_k);
  if (A == 0) return hipGetLastError();
  GemmArgs g{};
  g.a = x_sorted;
  g.b0 = w1;
  g.b1 = w3;
  g.bias = (c.act == MOE_ACT_GELU && c.has_bias) ? b1 : nullptr;
  g.c = L.h;
  g.tiles = L.tiles;
  g.K = c.d_model;
  g.n_out = c.d_ff;
  const int mt = max_m_tiles(c);
  if (c.dtype == MOE_BF16) {
    if (c.act == MOE_ACT_SWIGLU) {
      dim3 grid(mt, (c.d_ff + 63) / 64);
      expert_gemm_bf16_kernel<kEpiSwiglu><<<grid, 256, 0, stream>>>(g);
    } else {
      dim3 grid(mt, (c.d_ff + 127) / 128);
      expert_gemm_bf16_kernel<kEpiGelu><<<grid, 256, 0, stream>>>(g);
    }
  } else {
    dim3 grid(mt, (c.d_ff + kFBN - 1) / kFBN);
    if (c.act == MOE_ACT_SWIGLU) expert_gemm_f32_kernel<kEpiSwiglu><<<grid, 256, 0, stream>>>(g);
    else expert_gemm_f32_kernel<kEpiGelu><<<grid, 256, 0, stream>>>(g);
  }
  return hipGetLastError();
}

hipError_t launch_ffn_down(const moe_config& c, const WsLayout& L, const int32_t* offsets,
                           const void* w2, const void* b2, const float* gate_sorted,
                           void* y_sorted, hipStream_t stream) {
  const int A = (int)(c.n_tokens * c.top_k);
  if (A == 0) return hipGetLastError();
  GemmArgs g{};
  g.a = L.h;
  g.b0 = w2;
  g.bias = (c.act == MOE_ACT_GELU && c.has_bias) ? b2 : nullptr;
  g.gate = gate_sorted;
  g.c = y_sorted;
  g.tiles = L.tiles;
  g.K = c.d_ff;
  g.n_out = c.d_model;
  const int mt = max_m_tiles(c);
  if (c.dtype == MOE_BF16) {
    dim3 grid(mt, (c.d_model + 127) / 128);
    expert_gemm_bf16_kernel<kEpiDown><<<grid, 256, 0, stream>>>(g);
  } else {
    dim3 grid(mt, (c.d_model + kFBN - 1) / kFBN);
    expert_gemm_f32_kernel<kEpiDown><<<grid, 256, 0, stream>>>(g);
  }
  return hipGetLastError();
}

}  // namespace moe
