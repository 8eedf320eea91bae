// The whole-layer prefill for callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid it): the call's workspace is a fixed array
// in device memory, one per device, that the code object brings with it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "agnes_gdn.h"
#include "launch.h"

namespace agnes {

// The workspace of agnes_gdn_layer_prefill_noalloc.  64 MiB holds the workspace of one
// sequence of up to about 2400 tokens of the 16 / 48-head layer (the size query
// agnes_gdn_layer_prefill_workspace_size decides).  Each device that loads the library holds
// its own copy until the process ends.  In host code `scratch` names a host-side stand-in, not
// device memory: the kernels receive the device address looked up below.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[64] = {};  // device address of `scratch`, per device
}  // namespace

// Device address of `scratch` on the current device, looked up on the first call there (with
// that device current) and kept.
static hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace agnes

extern "C" __attribute__((visibility("default"))) int agnes_gdn_layer_prefill_noalloc(
    const void* x, int64_t x_token_stride, agnes_dtype dtype, const void* conv_weight, const void* conv_bias,
    void* conv_state, const float* g, const float* beta, const int32_t* cu_seqlens, int num_seqs,
    int64_t total_tokens, int num_k_heads, int num_v_heads, int head_dim, float scale, float l2norm_eps,
    const float* initial_state, float* final_state, const void* z, int64_t z_token_stride, const void* norm_weight,
    float norm_eps, void* y, void* o, agnes_dtype out_dtype, void* stream) {
  const size_t need = agnes_gdn_layer_prefill_workspace_size(num_seqs, total_tokens, num_k_heads, num_v_heads,
                                                             head_dim);
  if (need > agnes::kScratchBytes) return AGNES_ERR_UNSUPPORTED;
  void* ws = nullptr;
  if (need > 0) {
    const hipError_t e = agnes::scratch_address(&ws);
    if (e != hipSuccess) return agnes::hip_report(e);
  }
  return agnes::layer_prefill_checked(x, x_token_stride, (int)dtype, conv_weight, conv_bias, conv_state, g, beta,
                                      cu_seqlens, num_seqs, total_tokens, num_k_heads, num_v_heads, head_dim, scale,
                                      l2norm_eps, initial_state, final_state, z, z_token_stride, norm_weight, norm_eps,
                                      y, o, (int)out_dtype, ws, need > 0 ? agnes::kScratchBytes : 0, stream, true);
}
