// moe_forward_noalloc: the whole-layer forward for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc). Its scratch is a file-scope device array of MOE_NOALLOC_SCRATCH_BYTES, which
// every GPU the library runs on holds from module load to process end; the call allocates
// and frees nothing and runs moe_forward's kernels on that array.
//
// In host code the array's name is only a stand-in for the device symbol: its device address
// is taken once per device with hipGetSymbolAddress (with that device current) and only that
// address is ever handed to kernels.
#include <mutex>

#include "moe_internal.h"

namespace {

static __device__ __align__(256) char scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {nullptr};

// The current device's address of `scratch` (looked up on its first use on that device).
moe_status scratch_ptr(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" moe_status moe_forward_noalloc(const moe_config* cfg, const void* x, const void* w_router,
                                          const float* logit_bias, const float* sel_bias, const void* w1,
                                          const void* w3, const void* b1, const void* w2, const void* b2,
                                          const void* s_w1, const void* s_w3, const void* s_b1, const void* s_w2,
                                          const void* s_b2, void* y, int32_t* topk_ids, float* topk_w,
                                          int32_t* counts, float* stats, void* stream) {
  // the size check comes first, on the host: a configuration whose forward workspace exceeds
  // the static scratch is refused before anything touches the device
  const size_t need = moe_workspace_size(cfg, MOE_OP_FORWARD);
  if (need == 0)  // an invalid configuration: moe_forward's validation names the reason, before any HIP call
    return moe_forward(cfg, x, w_router, logit_bias, sel_bias, w1, w3, b1, w2, b2, s_w1, s_w3, s_b1, s_w2, s_b2, y,
                       topk_ids, topk_w, counts, stats, nullptr, nullptr, nullptr, nullptr, 0, nullptr, stream);
  if (need > (size_t)MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
  void* ws = nullptr;
  const moe_status st = scratch_ptr(&ws);
  if (st != MOE_OK) return st;
  return moe_forward(cfg, x, w_router, logit_bias, sel_bias, w1, w3, b1, w2, b2, s_w1, s_w3, s_b1, s_w2, s_b2, y,
                     topk_ids, topk_w, counts, stats, nullptr, nullptr, nullptr, ws, (size_t)MOE_NOALLOC_SCRATCH_BYTES,
                     nullptr, stream);
}
