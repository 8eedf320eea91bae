// C-ABI host layer of libagnes_gdn: argument checks, dtype dispatch and launches.
// Every check runs before anything is enqueued; a failed check launches nothing.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>

#include "agnes_gdn.h"
#include "launch.h"

#define AGNES_API extern "C" __attribute__((visibility("default")))

namespace {

thread_local int g_last_hip_error = 0;
std::atomic<uint32_t> g_wait_limit{0};

constexpr int kHeadDim = 128;

bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) & (n - 1)) == 0; }
bool valid_dtype(int d) { return d == AGNES_F32 || d == AGNES_BF16; }
size_t esize(int d) { return d == AGNES_BF16 ? 2 : 4; }

// Tokens of one call: cu_seqlens are int32.
constexpr int64_t kMaxTokens = INT32_MAX;

// Byte span [lo, hi) touched by `rows` rows of `width` elements at `stride` elements (a NULL
// buffer touches nothing).  The extent is computed exactly in 128 bits; `wraps` marks one that
// runs past the end of the address space, which no buffer can: such a span overlaps every
// non-empty span, so the overlap checks reject it.
struct Span {
  uintptr_t lo, hi;
  bool wraps;
};
Span span(const void* p, int64_t rows, int64_t stride, int64_t width, size_t es) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  if (!p || rows <= 0 || width <= 0) return {lo, lo, false};
  using u128 = unsigned __int128;
  const u128 end = (u128)lo + ((u128)(uint64_t)(rows - 1) * (uint64_t)stride + (uint64_t)width) * es;
  if (stride < 0 || end > UINTPTR_MAX) return {lo, UINTPTR_MAX, true};
  return {lo, (uintptr_t)end, false};
}
bool overlap(Span a, Span b) {
  if (a.lo == a.hi || b.lo == b.hi) return false;
  return a.wraps || b.wraps || (a.lo < b.hi && b.lo < a.hi);
}

int hip_status(hipError_t e) {
  if (e == hipSuccess) return AGNES_OK;
  g_last_hip_error = (int)e;
  return AGNES_ERR_HIP;
}

}  // namespace

namespace agnes {
unsigned prefill_wait_limit() { return g_wait_limit.load(std::memory_order_relaxed); }
}  // namespace agnes

AGNES_API const char* agnes_gdn_status_string(int status) {
  switch (status) {
    case AGNES_OK: return "AGNES_OK";
    case AGNES_ERR_INVALID_ARG: return "AGNES_ERR_INVALID_ARG: invalid argument (pointer, size, stride or overlap)";
    case AGNES_ERR_UNSUPPORTED: return "AGNES_ERR_UNSUPPORTED: outside the supported set of the call (head dims, kernel size, head ratio)";
    case AGNES_ERR_WORKSPACE: return "AGNES_ERR_WORKSPACE: workspace missing or too small";
    case AGNES_ERR_HIP: return "AGNES_ERR_HIP: a HIP launch failed";
    default: return "unknown agnes_status";
  }
}

AGNES_API int agnes_gdn_last_hip_error(void) { return g_last_hip_error; }

AGNES_API const char* agnes_gdn_version(void) { return "0.1.0"; }

AGNES_API int agnes_gdn_conv(const void* x, int64_t x_token_stride, void* y, int64_t y_token_stride,
                             agnes_dtype dtype, const void* weight, const void* bias,
                             const int32_t* cu_seqlens, int num_seqs, int64_t total_tokens, int channels,
                             int kernel_size, void* conv_state, int l2norm_heads, int head_dim,
                             float l2norm_eps, void* stream) {
  if (!valid_dtype(dtype)) return AGNES_ERR_INVALID_ARG;
  if (!x || !y || !weight) return AGNES_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(weight, 4) || (bias && !aligned(bias, 4)) ||
      (conv_state && !aligned(conv_state, 4)))
    return AGNES_ERR_INVALID_ARG;
  if (num_seqs < 0 || total_tokens < 0 || total_tokens > kMaxTokens || channels <= 0 || channels % 8)
    return AGNES_ERR_INVALID_ARG;
  if (x_token_stride < channels || y_token_stride < channels || x_token_stride % 8 || y_token_stride % 8)
    return AGNES_ERR_INVALID_ARG;
  if (l2norm_heads < 0 || !(l2norm_eps >= 0.f) || !std::isfinite(l2norm_eps)) return AGNES_ERR_INVALID_ARG;
  if (kernel_size != 4) return AGNES_ERR_UNSUPPORTED;
  if (l2norm_heads > 0) {
    if (head_dim != kHeadDim) return AGNES_ERR_UNSUPPORTED;
    if ((int64_t)l2norm_heads * head_dim > channels) return AGNES_ERR_INVALID_ARG;
  }
  if (!cu_seqlens) {  // decode mode
    if (!conv_state || total_tokens != num_seqs) return AGNES_ERR_INVALID_ARG;
  } else if (num_seqs == 0 && total_tokens != 0) {
    return AGNES_ERR_INVALID_ARG;
  }
  if ((int64_t)num_seqs > 65535 && !cu_seqlens) return AGNES_ERR_UNSUPPORTED;  // grid.y limit
  if (conv_state && num_seqs > 65535) return AGNES_ERR_UNSUPPORTED;
  if ((total_tokens + 15) / 16 > 65535) return AGNES_ERR_UNSUPPORTED;
  const size_t es = esize(dtype);
  if (overlap(span(x, total_tokens, x_token_stride, channels, es), span(y, total_tokens, y_token_stride, channels, es)))
    return AGNES_ERR_INVALID_ARG;
  if (conv_state && overlap(span(conv_state, num_seqs, (int64_t)channels * 3, (int64_t)channels * 3, es),
                            span(y, total_tokens, y_token_stride, channels, es)))
    return AGNES_ERR_INVALID_ARG;

  agnes::ConvArgs a{x, x_token_stride, y, y_token_stride, (int)dtype, weight, bias, cu_seqlens, num_seqs,
                    total_tokens, channels, conv_state, l2norm_heads, l2norm_eps};
  return hip_status(agnes::launch_conv(a, static_cast<hipStream_t>(stream)));
}

namespace {
// Status of a prefill problem's counts: invalid counts, then shapes outside the supported set
// (head_dim, Hv % Hk, 32-bit (sequence, head) indexing, launches that do not fit the grid limit).
int prefill_shape(int num_seqs, int64_t total_tokens, int num_k_heads, int num_v_heads, int head_dim, bool mfma) {
  if (num_seqs < 0 || total_tokens < 0 || total_tokens > kMaxTokens || num_k_heads <= 0 || num_v_heads <= 0)
    return AGNES_ERR_INVALID_ARG;
  if (head_dim != kHeadDim || num_v_heads % num_k_heads) return AGNES_ERR_UNSUPPORTED;
  if (num_seqs == 0 && total_tokens != 0) return AGNES_ERR_INVALID_ARG;
  if ((int64_t)num_seqs * num_v_heads > INT32_MAX / 8) return AGNES_ERR_UNSUPPORTED;
  const bool fits = mfma ? agnes::prefill_mfma_fits(num_seqs, total_tokens, num_k_heads, num_v_heads)
                         : agnes::prefill_f32_fits(num_seqs, num_v_heads);
  return fits ? AGNES_OK : AGNES_ERR_UNSUPPORTED;
}
}  // namespace

AGNES_API size_t agnes_gdn_prefill_workspace_size(int num_seqs, int64_t total_tokens, int num_k_heads,
                                                  int num_v_heads, int head_dim, agnes_dtype in_dtype) {
  if (in_dtype != AGNES_BF16 || prefill_shape(num_seqs, total_tokens, num_k_heads, num_v_heads, head_dim, true))
    return 0;
  return agnes::prefill_mfma_workspace(num_seqs, total_tokens, num_k_heads, num_v_heads);
}

AGNES_API int agnes_gdn_prefill_chunked(const void* q, const void* k, const void* v, agnes_dtype in_dtype,
                                        int64_t qk_token_stride, int64_t v_token_stride, const float* g,
                                        const float* beta, const int32_t* cu_seqlens, int num_seqs,
                                        int64_t total_tokens, int num_k_heads, int num_v_heads, int head_dim,
                                        float scale, const float* initial_state, float* final_state, void* o,
                                        agnes_dtype o_dtype, void* workspace, size_t workspace_bytes,
                                        void* stream) {
  if (!valid_dtype(in_dtype) || !valid_dtype(o_dtype)) return AGNES_ERR_INVALID_ARG;
  if (const int st = prefill_shape(num_seqs, total_tokens, num_k_heads, num_v_heads, head_dim, in_dtype == AGNES_BF16))
    return st;
  if (num_seqs > 0 && !cu_seqlens) return AGNES_ERR_INVALID_ARG;
  if (total_tokens > 0 && (!q || !k || !v || !g || !beta || !o)) return AGNES_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(g, 4) ||
      !aligned(beta, 4) || !aligned(initial_state, 16) || !aligned(final_state, 16) || !aligned(cu_seqlens, 4))
    return AGNES_ERR_INVALID_ARG;
  if (qk_token_stride < (int64_t)num_k_heads * head_dim || v_token_stride < (int64_t)num_v_heads * head_dim ||
      qk_token_stride % 8 || v_token_stride % 8)
    return AGNES_ERR_INVALID_ARG;
  if (!std::isfinite(scale)) return AGNES_ERR_INVALID_ARG;
  const int64_t sbytes = (int64_t)num_seqs * num_v_heads * head_dim * head_dim;
  const Span s0 = span(initial_state, 1, 0, sbytes, 4), s1 = span(final_state, 1, 0, sbytes, 4);
  if (initial_state && final_state && initial_state != final_state && overlap(s0, s1)) return AGNES_ERR_INVALID_ARG;
  const Span os = span(o, total_tokens, (int64_t)num_v_heads * head_dim, (int64_t)num_v_heads * head_dim, esize(o_dtype));
  if (final_state && overlap(os, s1)) return AGNES_ERR_INVALID_ARG;
  const size_t es = esize(in_dtype);
  if (overlap(os, span(q, total_tokens, qk_token_stride, (int64_t)num_k_heads * head_dim, es)) ||
      overlap(os, span(k, total_tokens, qk_token_stride, (int64_t)num_k_heads * head_dim, es)) ||
      overlap(os, span(v, total_tokens, v_token_stride, (int64_t)num_v_heads * head_dim, es)))
    return AGNES_ERR_INVALID_ARG;
  const size_t need = agnes_gdn_prefill_workspace_size(num_seqs, total_tokens, num_k_heads, num_v_heads, head_dim,
                                                       in_dtype);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 256))) return AGNES_ERR_WORKSPACE;

  agnes::PrefillArgs a{q, k, v, (int)in_dtype, qk_token_stride, v_token_stride, g, beta, cu_seqlens, num_seqs,
                       total_tokens, num_k_heads, num_v_heads, scale, initial_state, final_state, o, (int)o_dtype,
                       workspace, workspace_bytes};
  a.wait_limit = agnes::prefill_wait_limit();
  hipStream_t st = static_cast<hipStream_t>(stream);
  return hip_status(in_dtype == AGNES_BF16 ? agnes::launch_prefill_mfma(a, st) : agnes::launch_prefill_f32(a, st));
}

AGNES_API int agnes_gdn_prefill_fused(const void* x, int64_t x_token_stride, agnes_dtype dtype,
                                      const void* conv_weight, const void* conv_bias, void* conv_state,
                                      const float* g, const float* beta, const int32_t* cu_seqlens, int num_seqs,
                                      int64_t total_tokens, int num_k_heads, int num_v_heads, int head_dim,
                                      float scale, float l2norm_eps, const float* initial_state, float* final_state,
                                      void* o, agnes_dtype o_dtype, void* workspace, size_t workspace_bytes,
                                      void* stream) {
  if (!valid_dtype(dtype) || !valid_dtype(o_dtype)) return AGNES_ERR_INVALID_ARG;
  if (const int st = prefill_shape(num_seqs, total_tokens, num_k_heads, num_v_heads, head_dim, true)) return st;
  if (dtype != AGNES_BF16 || num_seqs > 65535) return AGNES_ERR_UNSUPPORTED;
  if (num_seqs > 0 && (!cu_seqlens || !conv_weight)) return AGNES_ERR_INVALID_ARG;
  if (total_tokens > 0 && (!x || !g || !beta || !o)) return AGNES_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(conv_weight, 16) || !aligned(conv_bias, 16) || !aligned(conv_state, 4) ||
      !aligned(o, 16) || !aligned(g, 4) || !aligned(beta, 4) || !aligned(initial_state, 16) ||
      !aligned(final_state, 16) || !aligned(cu_seqlens, 4))
    return AGNES_ERR_INVALID_ARG;
  const int64_t C = (2 * (int64_t)num_k_heads + num_v_heads) * head_dim;
  if (x_token_stride < C || x_token_stride % 8) return AGNES_ERR_INVALID_ARG;
  if (!std::isfinite(scale) || !(l2norm_eps >= 0.f) || !std::isfinite(l2norm_eps)) return AGNES_ERR_INVALID_ARG;
  const int64_t sbytes = (int64_t)num_seqs * num_v_heads * head_dim * head_dim;
  const Span s0 = span(initial_state, 1, 0, sbytes, 4), s1 = span(final_state, 1, 0, sbytes, 4);
  if (initial_state && final_state && initial_state != final_state && overlap(s0, s1)) return AGNES_ERR_INVALID_ARG;
  const int64_t rowo = (int64_t)num_v_heads * head_dim;
  const Span os = span(o, total_tokens, rowo, rowo, esize(o_dtype));
  const Span xs = span(x, total_tokens, x_token_stride, C, 2);
  const Span cs = span(conv_state, conv_state ? 1 : 0, 0, (int64_t)num_seqs * C * 3, 2);
  const Span ws_span = span(workspace, 1, 0, (int64_t)std::min<size_t>(workspace_bytes, INT64_MAX), 1);
  // outputs and in-place buffers must be disjoint from each other and from every input
  if (overlap(os, xs) || overlap(os, s1) || overlap(os, s0) || overlap(os, cs) || overlap(cs, xs) || overlap(cs, s1) ||
      overlap(cs, s0) || overlap(s1, xs) || overlap(ws_span, os) || overlap(ws_span, xs) || overlap(ws_span, cs) ||
      overlap(ws_span, s1))
    return AGNES_ERR_INVALID_ARG;
  const size_t need = agnes_gdn_prefill_workspace_size(num_seqs, total_tokens, num_k_heads, num_v_heads, head_dim,
                                                       AGNES_BF16);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 256))) return AGNES_ERR_WORKSPACE;

  // the q | k | v channel ranges of x (an empty batch may pass no x at all)
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  const uint16_t* xk = xb ? xb + (int64_t)num_k_heads * head_dim : nullptr;
  const uint16_t* xv = xb ? xb + 2 * (int64_t)num_k_heads * head_dim : nullptr;
  agnes::PrefillArgs a{xb, xk, xv,
                       (int)AGNES_BF16, x_token_stride, x_token_stride, g, beta, cu_seqlens, num_seqs, total_tokens,
                       num_k_heads, num_v_heads, scale, initial_state, final_state, o, (int)o_dtype, workspace,
                       workspace_bytes, conv_weight, conv_bias, conv_state, l2norm_eps};
  a.wait_limit = agnes::prefill_wait_limit();
  return hip_status(agnes::launch_prefill_mfma(a, static_cast<hipStream_t>(stream)));
}

AGNES_API int agnes_gdn_decode_step(const void* q, const void* k, const void* v, agnes_dtype in_dtype,
                                    int64_t qk_token_stride, int64_t v_token_stride, const float* g,
                                    const float* beta, int batch, int num_k_heads, int num_v_heads, int head_dim,
                                    float scale, float* state, void* o, agnes_dtype o_dtype, void* stream) {
  if (!valid_dtype(in_dtype) || !valid_dtype(o_dtype)) return AGNES_ERR_INVALID_ARG;
  if (batch < 0 || num_k_heads <= 0 || num_v_heads <= 0) return AGNES_ERR_INVALID_ARG;
  if (head_dim != kHeadDim || num_v_heads % num_k_heads) return AGNES_ERR_UNSUPPORTED;
  if (batch > 0 && (!q || !k || !v || !g || !beta || !state || !o)) return AGNES_ERR_INVALID_ARG;
  if (!aligned(q, 4) || !aligned(k, 4) || !aligned(v, 4) || !aligned(g, 4) || !aligned(beta, 4) ||
      !aligned(state, 16) || !aligned(o, 4))
    return AGNES_ERR_INVALID_ARG;
  if (qk_token_stride < (int64_t)num_k_heads * head_dim || v_token_stride < (int64_t)num_v_heads * head_dim)
    return AGNES_ERR_INVALID_ARG;
  if (!std::isfinite(scale)) return AGNES_ERR_INVALID_ARG;
  if ((int64_t)batch * num_v_heads > INT32_MAX) return AGNES_ERR_UNSUPPORTED;
  const Span ss = span(state, 1, 0, (int64_t)batch * num_v_heads * head_dim * head_dim, 4);
  const Span os = span(o, batch, (int64_t)num_v_heads * head_dim, (int64_t)num_v_heads * head_dim, esize(o_dtype));
  if (overlap(ss, os)) return AGNES_ERR_INVALID_ARG;
  if (!agnes::decode_fits(batch, num_v_heads)) return AGNES_ERR_UNSUPPORTED;

  agnes::DecodeArgs a{q, k, v, (int)in_dtype, qk_token_stride, v_token_stride, g, beta, batch, num_k_heads,
                      num_v_heads, scale, state, o, (int)o_dtype};
  return hip_status(agnes::launch_decode(a, static_cast<hipStream_t>(stream)));
}

AGNES_API int agnes_gdn_gated_rmsnorm(const void* o, agnes_dtype o_dtype, const void* z, const void* weight,
                                      agnes_dtype zw_dtype, float eps, int64_t rows, int dim, void* y,
                                      agnes_dtype y_dtype, void* stream) {
  if (!valid_dtype(o_dtype) || !valid_dtype(zw_dtype) || !valid_dtype(y_dtype)) return AGNES_ERR_INVALID_ARG;
  if (rows < 0 || !(eps >= 0.f) || !std::isfinite(eps)) return AGNES_ERR_INVALID_ARG;
  if (dim != kHeadDim) return AGNES_ERR_UNSUPPORTED;
  if (rows > 0 && (!o || !z || !weight || !y)) return AGNES_ERR_INVALID_ARG;
  if (!aligned(o, 16) || !aligned(z, 16) || !aligned(weight, 16) || !aligned(y, 16)) return AGNES_ERR_INVALID_ARG;
  const Span ys = span(y, rows, dim, dim, esize(y_dtype));
  const Span osp = span(o, rows, dim, dim, esize(o_dtype));
  const bool exact_alias = (o == y) && (o_dtype == y_dtype);
  if (!exact_alias && overlap(ys, osp)) return AGNES_ERR_INVALID_ARG;
  if (overlap(ys, span(z, rows, dim, dim, esize(zw_dtype)))) return AGNES_ERR_INVALID_ARG;
  if (!agnes::norm_fits(rows)) return AGNES_ERR_UNSUPPORTED;

  agnes::NormArgs a{o, (int)o_dtype, z, weight, (int)zw_dtype, eps, rows, y, (int)y_dtype};
  return hip_status(agnes::launch_gated_rmsnorm(a, static_cast<hipStream_t>(stream)));
}

AGNES_API int agnes_gdn_decode_fused(const void* x, int64_t x_token_stride, agnes_dtype dtype, const void* conv_weight,
                                     const void* conv_bias, void* conv_state, const float* g, const float* beta,
                                     const void* z, const void* norm_weight, float* state, const int32_t* slots,
                                     int num_slots, int batch, int num_k_heads, int num_v_heads, int head_dim,
                                     float scale, float l2norm_eps, float norm_eps, void* y, void* o,
                                     agnes_dtype o_dtype, void* stream) {
  if (!valid_dtype(dtype) || !valid_dtype(o_dtype)) return AGNES_ERR_INVALID_ARG;
  if (batch < 0 || num_slots < 0 || num_k_heads <= 0 || num_v_heads <= 0) return AGNES_ERR_INVALID_ARG;
  if (head_dim != kHeadDim || num_v_heads % num_k_heads) return AGNES_ERR_UNSUPPORTED;
  if (!std::isfinite(scale) || !(l2norm_eps >= 0.f) || !std::isfinite(l2norm_eps) || !(norm_eps >= 0.f) ||
      !std::isfinite(norm_eps))
    return AGNES_ERR_INVALID_ARG;
  if (batch == 0) return AGNES_OK;
  if (!x || !conv_weight || !conv_state || !g || !beta || !z || !norm_weight || !state || !y)
    return AGNES_ERR_INVALID_ARG;
  if (!slots && num_slots < batch) return AGNES_ERR_INVALID_ARG;
  const int64_t C = (2 * (int64_t)num_k_heads + num_v_heads) * head_dim;
  if (x_token_stride < C || x_token_stride % 8) return AGNES_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(conv_weight, 16) || !aligned(conv_bias, 16) || !aligned(conv_state, 16) ||
      !aligned(g, 4) || !aligned(beta, 4) || !aligned(z, 4) || !aligned(norm_weight, 4) || !aligned(state, 16) ||
      !aligned(slots, 4) || !aligned(y, 4) || !aligned(o, 4))
    return AGNES_ERR_INVALID_ARG;
  if ((int64_t)batch * num_k_heads > INT32_MAX || (int64_t)num_slots * num_v_heads > INT32_MAX / 8)
    return AGNES_ERR_UNSUPPORTED;
  const size_t es = esize(dtype), eo = esize(o_dtype);
  const int64_t rowv = (int64_t)num_v_heads * head_dim;
  const Span ys = span(y, batch, rowv, rowv, eo);
  const Span os = o ? span(o, batch, rowv, rowv, eo) : Span{0, 0};
  const Span ss = span(state, 1, 0, (int64_t)num_slots * rowv * head_dim, 4);
  const Span cs = span(conv_state, 1, 0, (int64_t)num_slots * C * 3, es);
  const Span ins[] = {span(x, batch, x_token_stride, C, es), span(conv_weight, 1, 0, C * 4, es),
                      span(conv_bias, conv_bias ? 1 : 0, 0, C, es), span(g, batch, num_v_heads, num_v_heads, 4),
                      span(beta, batch, num_v_heads, num_v_heads, 4), span(z, batch, rowv, rowv, es),
                      span(norm_weight, 1, 0, head_dim, es), span(slots, slots ? 1 : 0, 0, batch, 4)};
  // outputs and in-place buffers must be disjoint from each other and from every input
  const Span outs[] = {ys, os, ss, cs};
  for (int i = 0; i < 4; ++i) {
    for (int j = i + 1; j < 4; ++j)
      if (overlap(outs[i], outs[j])) return AGNES_ERR_INVALID_ARG;
    for (const Span& in : ins)
      if (overlap(outs[i], in)) return AGNES_ERR_INVALID_ARG;
  }
  if (!agnes::decode_fused_fits(batch, num_v_heads)) return AGNES_ERR_UNSUPPORTED;

  agnes::FusedDecodeArgs a{x, x_token_stride, (int)dtype, conv_weight, conv_bias, conv_state, g, beta, z,
                           norm_weight, state, slots, num_slots, batch, num_k_heads, num_v_heads, scale,
                           l2norm_eps, norm_eps, y, o, (int)o_dtype};
  return hip_status(agnes::launch_decode_fused(a, static_cast<hipStream_t>(stream)));
}

AGNES_API size_t agnes_attn_prefill_workspace_size(int num_seqs, int64_t total_tokens) {
  if (num_seqs < 0 || total_tokens < 0 || total_tokens > kMaxTokens) return 0;
  return agnes::attn_prefill_workspace(num_seqs, total_tokens);
}

AGNES_API int agnes_attn_prefill(const void* q, int64_t q_token_stride, const void* k, int64_t k_token_stride,
                                 const void* v, int64_t v_token_stride, const void* gate, int64_t gate_token_stride,
                                 const void* q_norm_weight, const void* k_norm_weight, const int32_t* positions,
                                 int64_t positions_stride, const int32_t* cu_seqlens, int num_seqs,
                                 int64_t total_tokens, int num_q_heads, int num_kv_heads, int head_dim, int rot_dim,
                                 float rope_base, float norm_eps, float scale, void* k_out,
                                 int64_t k_out_token_stride, void* v_out, int64_t v_out_token_stride, void* o,
                                 agnes_dtype o_dtype, void* workspace, size_t workspace_bytes, void* stream) {
  constexpr int kAttnDim = 256;
  if (!valid_dtype(o_dtype)) return AGNES_ERR_INVALID_ARG;
  if (num_seqs < 0 || total_tokens < 0 || total_tokens > kMaxTokens || num_q_heads <= 0 || num_kv_heads <= 0)
    return AGNES_ERR_INVALID_ARG;
  if (head_dim != kAttnDim || rot_dim != 64 || num_q_heads % num_kv_heads) return AGNES_ERR_UNSUPPORTED;
  if (num_seqs == 0 && total_tokens != 0) return AGNES_ERR_INVALID_ARG;
  if (num_seqs > 0 && !cu_seqlens) return AGNES_ERR_INVALID_ARG;
  if (total_tokens > 0 && (!q || !k || !v || !gate || !q_norm_weight || !k_norm_weight || !k_out || !o))
    return AGNES_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(gate, 16) || !aligned(k_out, 16) ||
      !aligned(v_out, 16) || !aligned(o, 16) || !aligned(q_norm_weight, 8) || !aligned(k_norm_weight, 8) ||
      !aligned(positions, 4) || !aligned(cu_seqlens, 4))
    return AGNES_ERR_INVALID_ARG;
  const int64_t qw = (int64_t)num_q_heads * head_dim, kw = (int64_t)num_kv_heads * head_dim;
  if (q_token_stride < qw || gate_token_stride < qw || k_token_stride < kw || v_token_stride < kw ||
      k_out_token_stride < kw || (v_out && v_out_token_stride < kw) || q_token_stride % 8 || gate_token_stride % 8 ||
      k_token_stride % 8 || v_token_stride % 8 || k_out_token_stride % 8 || (v_out && v_out_token_stride % 8))
    return AGNES_ERR_INVALID_ARG;
  if (positions && positions_stride < total_tokens) return AGNES_ERR_INVALID_ARG;
  // 64-row blocks are addressed with 32-bit element offsets
  if (q_token_stride > (1 << 24) || k_token_stride > (1 << 24) || v_token_stride > (1 << 24) ||
      k_out_token_stride > (1 << 24))
    return AGNES_ERR_UNSUPPORTED;
  if (!std::isfinite(rope_base) || rope_base <= 0.f || !std::isfinite(norm_eps) || norm_eps < 0.f ||
      !std::isfinite(scale))
    return AGNES_ERR_INVALID_ARG;
  if (!agnes::attn_prefill_fits(num_seqs, total_tokens, num_q_heads, num_kv_heads)) return AGNES_ERR_UNSUPPORTED;
  const Span os = span(o, total_tokens, qw, qw, esize(o_dtype));
  const Span ks = span(k_out, total_tokens, k_out_token_stride, kw, 2);
  const Span vs = span(v_out, total_tokens, v_out_token_stride, kw, 2);
  const Span ins[4] = {span(q, total_tokens, q_token_stride, qw, 2), span(k, total_tokens, k_token_stride, kw, 2),
                       span(v, total_tokens, v_token_stride, kw, 2),
                       span(gate, total_tokens, gate_token_stride, qw, 2)};
  for (const Span& in : ins)
    if (overlap(os, in) || overlap(ks, in) || overlap(vs, in)) return AGNES_ERR_INVALID_ARG;
  if (overlap(os, ks) || overlap(os, vs) || overlap(ks, vs)) return AGNES_ERR_INVALID_ARG;
  const size_t need = agnes::attn_prefill_workspace(num_seqs, total_tokens);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 256))) return AGNES_ERR_WORKSPACE;

  agnes::AttnArgs a{};
  a.q = q; a.k = k; a.v = v; a.gate = gate;
  a.q_stride = q_token_stride; a.k_stride = k_token_stride; a.v_stride = v_token_stride;
  a.gate_stride = gate_token_stride;
  a.q_norm_w = q_norm_weight; a.k_norm_w = k_norm_weight;
  a.pos3 = positions; a.pos3_stride = positions_stride;
  a.cu = cu_seqlens; a.num_seqs = num_seqs; a.total = total_tokens;
  a.hq = num_q_heads; a.hkv = num_kv_heads;
  a.rope_base = rope_base; a.eps = norm_eps; a.scale = scale;
  a.k_out = k_out; a.k_out_stride = k_out_token_stride;
  a.v_out = v_out; a.v_out_stride = v_out_token_stride;
  a.o = o; a.o_dtype = (int)o_dtype;
  a.workspace = workspace; a.workspace_bytes = workspace_bytes;
  return hip_status(agnes::launch_attn_prefill(a, static_cast<hipStream_t>(stream)));
}

namespace {
constexpr int64_t kMaxCacheLen = (int64_t)1 << 30;
}  // namespace

AGNES_API size_t agnes_attn_decode_workspace_size(int batch, int num_q_heads, int num_kv_heads, int64_t max_len) {
  if (batch <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_len <= 0 || max_len > kMaxCacheLen ||
      num_q_heads % num_kv_heads || !agnes::attn_decode_fits(batch, num_q_heads, num_kv_heads, max_len))
    return 0;
  return agnes::attn_decode_workspace(batch, num_q_heads, num_kv_heads, max_len);
}

AGNES_API int agnes_attn_decode(const void* q, int64_t q_stride, const void* k, int64_t k_stride, const void* v,
                                int64_t v_stride, const void* gate, int64_t gate_stride, const void* q_norm_weight,
                                const void* k_norm_weight, const int32_t* positions, int64_t positions_stride,
                                void* k_cache, void* v_cache, int64_t max_len, const int32_t* cache_lens, int batch,
                                int num_q_heads, int num_kv_heads, int head_dim, int rot_dim, float rope_base,
                                float norm_eps, float scale, void* o, agnes_dtype o_dtype, void* workspace,
                                size_t workspace_bytes, void* stream) {
  constexpr int kAttnDim = 256;
  if (!valid_dtype(o_dtype)) return AGNES_ERR_INVALID_ARG;
  if (batch < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_len <= 0) return AGNES_ERR_INVALID_ARG;
  if (head_dim != kAttnDim || rot_dim != 64 || num_q_heads % num_kv_heads) return AGNES_ERR_UNSUPPORTED;
  if (max_len > kMaxCacheLen) return AGNES_ERR_UNSUPPORTED;
  if (batch == 0) return AGNES_OK;
  if (!q || !k || !v || !gate || !q_norm_weight || !k_norm_weight || !k_cache || !v_cache || !cache_lens || !o)
    return AGNES_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(gate, 16) || !aligned(k_cache, 16) ||
      !aligned(v_cache, 16) || !aligned(o, 16) || !aligned(q_norm_weight, 8) || !aligned(k_norm_weight, 8) ||
      !aligned(positions, 4) || !aligned(cache_lens, 4))
    return AGNES_ERR_INVALID_ARG;
  const int64_t qw = (int64_t)num_q_heads * head_dim, kw = (int64_t)num_kv_heads * head_dim;
  if (q_stride < qw || gate_stride < qw || k_stride < kw || v_stride < kw || q_stride % 8 || gate_stride % 8 ||
      k_stride % 8 || v_stride % 8)
    return AGNES_ERR_INVALID_ARG;
  if (positions && positions_stride < batch) return AGNES_ERR_INVALID_ARG;
  if (!std::isfinite(rope_base) || rope_base <= 0.f || !std::isfinite(norm_eps) || norm_eps < 0.f ||
      !std::isfinite(scale))
    return AGNES_ERR_INVALID_ARG;
  const int64_t cache_rows = (int64_t)batch * max_len;  // of kw elements each
  const Span os = span(o, batch, qw, qw, esize(o_dtype));
  const Span kc = span(k_cache, cache_rows, kw, kw, 2), vc = span(v_cache, cache_rows, kw, kw, 2);
  const Span ins[5] = {span(q, batch, q_stride, qw, 2), span(k, batch, k_stride, kw, 2), span(v, batch, v_stride, kw, 2),
                       span(gate, batch, gate_stride, qw, 2), span(cache_lens, 1, 0, batch, 4)};
  for (const Span& in : ins)
    if (overlap(os, in) || overlap(kc, in) || overlap(vc, in)) return AGNES_ERR_INVALID_ARG;
  if (overlap(os, kc) || overlap(os, vc) || overlap(kc, vc)) return AGNES_ERR_INVALID_ARG;
  if (!agnes::attn_decode_fits(batch, num_q_heads, num_kv_heads, max_len)) return AGNES_ERR_UNSUPPORTED;
  const size_t need = agnes::attn_decode_workspace(batch, num_q_heads, num_kv_heads, max_len);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 256))) return AGNES_ERR_WORKSPACE;

  agnes::AttnArgs a{};
  a.q = q; a.k = k; a.v = v; a.gate = gate;
  a.q_stride = q_stride; a.k_stride = k_stride; a.v_stride = v_stride; a.gate_stride = gate_stride;
  a.q_norm_w = q_norm_weight; a.k_norm_w = k_norm_weight;
  a.pos3 = positions; a.pos3_stride = positions_stride;
  a.total = batch; a.hq = num_q_heads; a.hkv = num_kv_heads;
  a.rope_base = rope_base; a.eps = norm_eps; a.scale = scale;
  a.o = o; a.o_dtype = (int)o_dtype;
  a.workspace = workspace; a.workspace_bytes = workspace_bytes;
  a.k_cache = k_cache; a.v_cache = v_cache; a.max_len = max_len; a.cache_lens = cache_lens;
  return hip_status(agnes::launch_attn_decode(a, static_cast<hipStream_t>(stream)));
}

AGNES_API size_t agnes_gdn_layer_prefill_workspace_size(int num_seqs, int64_t total_tokens, int num_k_heads,
                                                       int num_v_heads, int head_dim) {
  if (prefill_shape(num_seqs, total_tokens, num_k_heads, num_v_heads, head_dim, true) || num_seqs > 65535) return 0;
  return agnes::layer_prefill_workspace(num_seqs, total_tokens, num_k_heads, num_v_heads);
}

namespace agnes {
int hip_report(hipError_t e) { return hip_status(e); }

// agnes_gdn_layer_prefill's checks and launch; single_stage runs the call in one stage (no side
// stream, nothing created on first use).
int layer_prefill_checked(const void* x, int64_t x_token_stride, int dtype, const void* conv_weight,
                          const void* conv_bias, void* conv_state, const float* g, const float* beta,
                          const int32_t* cu_seqlens, int num_seqs, int64_t total_tokens, int num_k_heads,
                          int num_v_heads, int head_dim, float scale, float l2norm_eps, const float* initial_state,
                          float* final_state, const void* z, int64_t z_token_stride, const void* norm_weight,
                          float norm_eps, void* y, void* o, int out_dtype, void* workspace, size_t workspace_bytes,
                          void* stream, bool single_stage) {
  if (!valid_dtype(dtype) || !valid_dtype(out_dtype)) return AGNES_ERR_INVALID_ARG;
  if (const int st = prefill_shape(num_seqs, total_tokens, num_k_heads, num_v_heads, head_dim, true)) return st;
  if (dtype != AGNES_BF16 || num_seqs > 65535) return AGNES_ERR_UNSUPPORTED;
  if (num_seqs > 0 && (!cu_seqlens || !conv_weight || !norm_weight)) return AGNES_ERR_INVALID_ARG;
  if (total_tokens > 0 && (!x || !g || !beta || !z || !y)) return AGNES_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(conv_weight, 16) || !aligned(conv_bias, 16) || !aligned(conv_state, 4) ||
      !aligned(o, 16) || !aligned(y, 16) || !aligned(z, 16) || !aligned(norm_weight, 16) || !aligned(g, 4) ||
      !aligned(beta, 4) || !aligned(initial_state, 16) || !aligned(final_state, 16) || !aligned(cu_seqlens, 4))
    return AGNES_ERR_INVALID_ARG;
  const int64_t C = (2 * (int64_t)num_k_heads + num_v_heads) * head_dim;
  const int64_t rowo = (int64_t)num_v_heads * head_dim;
  if (x_token_stride < C || x_token_stride % 8 || z_token_stride < rowo || z_token_stride % 8)
    return AGNES_ERR_INVALID_ARG;
  if (!std::isfinite(scale) || !(l2norm_eps >= 0.f) || !std::isfinite(l2norm_eps) || !(norm_eps >= 0.f) ||
      !std::isfinite(norm_eps))
    return AGNES_ERR_INVALID_ARG;
  const int64_t sbytes = (int64_t)num_seqs * num_v_heads * head_dim * head_dim;
  const Span s0 = span(initial_state, 1, 0, sbytes, 4), s1 = span(final_state, 1, 0, sbytes, 4);
  if (initial_state && final_state && initial_state != final_state && overlap(s0, s1)) return AGNES_ERR_INVALID_ARG;
  const Span os = span(o, o ? total_tokens : 0, rowo, rowo, esize(out_dtype));
  const Span ys = span(y, total_tokens, rowo, rowo, esize(out_dtype));
  const Span xs = span(x, total_tokens, x_token_stride, C, 2);
  const Span zs = span(z, total_tokens, z_token_stride, rowo, 2);
  const Span cs = span(conv_state, conv_state ? 1 : 0, 0, (int64_t)num_seqs * C * 3, 2);
  const Span ws_span = span(workspace, 1, 0, (int64_t)std::min<size_t>(workspace_bytes, INT64_MAX), 1);
  const Span outs[5] = {os, ys, cs, s1, ws_span};
  const Span ins[4] = {xs, zs, s0, span(norm_weight, 1, 0, head_dim, 2)};
  for (int i = 0; i < 5; ++i) {
    for (const Span& in : ins)
      if (overlap(outs[i], in) && !(i == 3 && in.lo == s0.lo && initial_state == final_state)) return AGNES_ERR_INVALID_ARG;
    for (int k = i + 1; k < 5; ++k)
      if (overlap(outs[i], outs[k])) return AGNES_ERR_INVALID_ARG;
  }
  const size_t need = agnes::layer_prefill_workspace(num_seqs, total_tokens, num_k_heads, num_v_heads);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 256))) return AGNES_ERR_WORKSPACE;

  // the q | k | v channel ranges of x (an empty batch may pass no x at all)
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  const uint16_t* xk = xb ? xb + (int64_t)num_k_heads * head_dim : nullptr;
  const uint16_t* xv = xb ? xb + 2 * (int64_t)num_k_heads * head_dim : nullptr;
  agnes::PrefillArgs a{xb, xk, xv,
                       (int)AGNES_BF16, x_token_stride, x_token_stride, g, beta, cu_seqlens, num_seqs, total_tokens,
                       num_k_heads, num_v_heads, scale, initial_state, final_state, o, (int)out_dtype, workspace,
                       workspace_bytes, conv_weight, conv_bias, conv_state, l2norm_eps};
  a.wait_limit = agnes::prefill_wait_limit();
  a.z = z;
  a.z_stride = z_token_stride;
  a.norm_w = norm_weight;
  a.norm_eps = norm_eps;
  a.y = y;
  a.layer = true;
  a.single_stage = single_stage;
  return hip_status(agnes::launch_layer_prefill(a, static_cast<hipStream_t>(stream)));
}
}  // namespace agnes

AGNES_API int agnes_gdn_layer_prefill(const void* x, int64_t x_token_stride, agnes_dtype dtype,
                                      const void* conv_weight, const void* conv_bias, void* conv_state,
                                      const float* g, const float* beta, const int32_t* cu_seqlens, int num_seqs,
                                      int64_t total_tokens, int num_k_heads, int num_v_heads, int head_dim,
                                      float scale, float l2norm_eps, const float* initial_state, float* final_state,
                                      const void* z, int64_t z_token_stride, const void* norm_weight, float norm_eps,
                                      void* y, void* o, agnes_dtype out_dtype, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  return agnes::layer_prefill_checked(x, x_token_stride, dtype, conv_weight, conv_bias, conv_state, g, beta,
                                      cu_seqlens, num_seqs, total_tokens, num_k_heads, num_v_heads, head_dim, scale,
                                      l2norm_eps, initial_state, final_state, z, z_token_stride, norm_weight, norm_eps,
                                      y, o, out_dtype, workspace, workspace_bytes, stream, false);
}

AGNES_API int agnes_gdn_ceiling_rmw_stream(void* buf, size_t bytes, void* stream) {
  if (!buf || !aligned(buf, 16) || bytes % 16) return AGNES_ERR_INVALID_ARG;
  return hip_status(agnes::launch_rmw_stream(buf, bytes, static_cast<hipStream_t>(stream)));
}

AGNES_API int agnes_gdn_ceiling_mfma(float* sink, int blocks, int iters, void* stream) {
  if (!sink || !aligned(sink, 4) || blocks < 1 || blocks > (1 << 20) || iters < 1 || iters > (1 << 20))
    return AGNES_ERR_INVALID_ARG;
  return hip_status(agnes::launch_mfma_peak(sink, blocks, iters, static_cast<hipStream_t>(stream)));
}

AGNES_API int agnes_gdn_workspace_status(const void* workspace, uint32_t* flags, void* stream) {
  if (!workspace || !flags || !aligned(workspace, 4)) return AGNES_ERR_INVALID_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  uint32_t word = 0;
  hipError_t e = hipMemcpyAsync(&word, workspace, sizeof(word), hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return hip_status(e);
  *flags = word;
  return AGNES_OK;
}

AGNES_API int agnes_gdn_set_wait_limit(uint32_t polls) {
  g_wait_limit.store(polls, std::memory_order_relaxed);
  return AGNES_OK;
}

AGNES_API int agnes_gdn_set_prefill_stages(const int32_t* cuts, int n_cuts) {
  return agnes::set_stage_cuts(cuts, n_cuts) ? AGNES_OK : AGNES_ERR_INVALID_ARG;
}

AGNES_API int agnes_gdn_release(void) { return hip_status(agnes::release_side_queues()); }
