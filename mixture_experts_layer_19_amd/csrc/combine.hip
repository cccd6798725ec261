// Combine ("Mixture of Experts: routing, sorted dispatch, Switch aux loss, aux-free bias"
// (L7.8) §2.2 and §3): y[n] = sum_{j<k} g_{n,j} y_sorted[inv_perm[n*k + j]], accumulated in
// float32 with j ascending and rounded to the element type once. Token-major, 16 bytes per
// lane, so every read and write is a full contiguous row segment.
#include "moe_internal.h"

namespace moe {

template <typename T>
__global__ __launch_bounds__(256) void combine_kernel(
    const uint4* __restrict__ y_sorted, const float* __restrict__ topk_w,
    const int32_t* __restrict__ inv_perm, const uint4* __restrict__ y_add, uint4* __restrict__ y,
    long long n_tokens, int k, int vec_per_row, int n_rows) {
  constexpr int kPer = Elem<T>::kPer16B;
  const long long total = n_tokens * vec_per_row;
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < total; i += (long long)gridDim.x * 256) {
    const long long n = i / vec_per_row;
    const int c = (int)(i - n * vec_per_row);
    float acc[kPer];
#pragma unroll
    for (int q = 0; q < kPer; ++q) acc[q] = 0.f;
    for (int j = 0; j < k; ++j) {
      const int src = inv_perm[n * k + j];
      if (src < 0 || src >= n_rows) continue;
      const float gw = topk_w ? topk_w[n * k + j] : 1.0f;
      float v[kPer];
      unpack16(y_sorted[(size_t)src * vec_per_row + c], v, T{});
#pragma unroll
      for (int q = 0; q < kPer; ++q) acc[q] = fmaf(gw, v[q], acc[q]);
    }
    if (y_add) {  // the shared expert's output, weight 1, after the routed terms
      float v[kPer];
      unpack16(y_add[i], v, T{});
#pragma unroll
      for (int q = 0; q < kPer; ++q) acc[q] += v[q];
    }
    y[i] = pack16(acc, T{});
  }
}

hipError_t launch_combine(const moe_config& c, const void* y_sorted, const float* topk_w,
                          const int32_t* inv_perm, const void* y_add, void* y, hipStream_t stream) {
  const int vpr = (int)(c.d_model * elem_size(c) / 16);
  const long long total = c.n_tokens * vpr;
  if (total == 0) return hipGetLastError();
  const int grid = (int)std::min<long long>((total + 255) / 256, 1 << 16);
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
