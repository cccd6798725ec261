// Combine ("Mixture of Experts: routing, sorted dispatch, Switch aux loss, aux-free bias"
// (L7.8) §2.2 and §3): y[n] = sum_{j<k} g_{n,j} y_sorted[inv_perm[n*k + j]], accumulated in
// float32 with j ascending and rounded to the element type once. Token-major, 16 bytes per
// lane, so every read and write is a full contiguous row segment.
#include "moe_internal.h"

namespace moe {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// One wave per token: the token's k source rows and gates are wave-uniform (scalar loads),
// and the lanes stream the row in 16-byte pieces, four pieces per source row in flight per
// lane. y_sorted is read once and y written once, so both bypass the caches' reuse policy
// (non-temporal), which leaves the caches to inv_perm and the gates.
template <typename T>
__global__ __launch_bounds__(256) void combine_kernel(
    const uint4* __restrict__ y_sorted, const float* __restrict__ topk_w,
    const int32_t* __restrict__ inv_perm, const uint4* __restrict__ y_add, uint4* __restrict__ y,
    long long n_tokens, int k, int vec_per_row, int n_rows) {
  constexpr int kPer = Elem<T>::kPer16B;
  constexpr int kMaxK = 8;  // gates / sources held in registers; more choices are walked in groups
  const int lane = threadIdx.x & 63;
  const long long wave0 = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const long long n_waves = (long long)gridDim.x * 4;
  for (long long n = wave0; n < n_tokens; n += n_waves) {
    float acc[4][kPer];
    for (int c0 = 0; c0 < vec_per_row; c0 += 4 * 64) {
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int q = 0; q < kPer; ++q) acc[u][q] = 0.f;
      for (int j0 = 0; j0 < k; j0 += kMaxK) {
        int src[kMaxK];
        float gw[kMaxK];
#pragma unroll
        for (int j = 0; j < kMaxK; ++j) {
          const bool in = j0 + j < k;
          const int s = in ? inv_perm[n * k + j0 + j] : -1;
          src[j] = (s >= 0 && s < n_rows) ? s : -1;
          gw[j] = (in && topk_w) ? topk_w[n * k + j0 + j] : 1.0f;
        }
#pragma unroll
        for (int j = 0; j < kMaxK; ++j) {
          if (src[j] < 0) continue;  // wave-uniform
          const uint4* row = y_sorted + (size_t)src[j] * vec_per_row;
          uint4 r[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int c = c0 + u * 64 + lane;
            r[u] = c < vec_per_row ? __builtin_bit_cast(uint4, __builtin_nontemporal_load(
                                         reinterpret_cast<const u32x4*>(row + c)))
                                   : make_uint4(0, 0, 0, 0);
          }
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            float v[kPer];
            unpack16(r[u], v, T{});
#pragma unroll
            for (int q = 0; q < kPer; ++q) acc[u][q] = fmaf(gw[j], v[q], acc[u][q]);
          }
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int c = c0 + u * 64 + lane;
        if (c >= vec_per_row) continue;
        const size_t i = (size_t)n * vec_per_row + c;
        if (y_add) {  // the shared expert's output, weight 1, after the routed terms
          float v[kPer];
          unpack16(y_add[i], v, T{});
#pragma unroll
          for (int q = 0; q < kPer; ++q) acc[u][q] += v[q];
        }
        __builtin_nontemporal_store(__builtin_bit_cast(u32x4, pack16(acc[u], T{})), reinterpret_cast<u32x4*>(y + i));
      }
    }
  }
}

hipError_t launch_combine(const moe_config& c, const void* y_sorted, const float* topk_w,
                          const int32_t* inv_perm, const void* y_add, void* y, hipStream_t stream) {
  const int vpr = (int)(c.d_model * elem_size(c) / 16);
  const long long total = c.n_tokens * vpr;
  if (total == 0) return hipGetLastError();
  const int grid = (int)std::min<long long>((c.n_tokens + 3) / 4, 1 << 16);
  const int n_rows = (int)(c.n_tokens * c.top_k);
  if (c.dtype == MOE_BF16)
    combine_kernel<bf16_t><<<grid, 256, 0, stream>>>(static_cast<const uint4*>(y_sorted), topk_w, inv_perm,
                                                     static_cast<const uint4*>(y_add), static_cast<uint4*>(y),
                                                     c.n_tokens, c.top_k, vpr, n_rows);
  else
    combine_kernel<float><<<grid, 256, 0, stream>>>(static_cast<const uint4*>(y_sorted), topk_w, inv_perm,
                                                    static_cast<const uint4*>(y_add), static_cast<uint4*>(y),
                                                    c.n_tokens, c.top_k, vpr, n_rows);
  return hipGetLastError();
}

}  // namespace moe
