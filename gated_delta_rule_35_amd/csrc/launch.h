// Internal launcher interface between the C-ABI host layer (api.cpp) and the
// kernel translation units.  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace agnes {

struct ConvArgs {
  const void* x;
  int64_t x_stride;
  void* y;
  int64_t y_stride;
  int dtype;
  const void* w;
  const void* bias;
  const int32_t* cu;  // nullptr = decode mode
  int num_seqs;
  int64_t total;
  int channels;
  void* state;  // [N, C, 3] or nullptr
  int l2_heads;
  float eps;
};

struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  int in_dtype;
  int64_t qk_stride;
  int64_t v_stride;
  const float* g;
  const float* beta;
  const int32_t* cu;
  int num_seqs;
  int64_t total;
  int hk;
  int hv;
  float scale;
  const float* s0;
  float* s1;
  void* o;
  int o_dtype;
  void* workspace;
  size_t workspace_bytes;
  // Fused prologue (all null for the plain call): q, k, v above are the q | k | v channel
  // ranges of the raw projection output x (row stride qk_stride == v_stride), and the
  // prefill applies the causal conv + SiLU + L2 of q, k itself.
  const void* conv_w;     // [(2 hk + hv) * 128, 4] bf16
  const void* conv_b;     // [(2 hk + hv) * 128] bf16 or nullptr
  void* conv_hist;        // [num_seqs, (2 hk + hv) * 128, 3] bf16 or nullptr (zeros); advanced after the call
  float l2_eps;
  // Gated RMSNorm epilogue (whole-layer call; nullptr otherwise): y = rmsnorm(o) * w * silu(z)
  // per 128-value head row, in the o dtype; o itself is then optional.
  const void* z;          // [total, hv, 128] bf16, token stride z_stride
  int64_t z_stride;
  const void* norm_w;     // [128] bf16
  float norm_eps;
  void* y;                // [total, hv, 128] contiguous
  // Chunk range of this launch (whole-layer call in stages): local chunks [n_c lo / den,
  // n_c hi / den) of each sequence of n_c chunks; s0 / s1 are then the states at its ends.
  int part_lo = 0, part_hi = 1, part_den = 1;
  int stage = 0;          // whole-layer call: this stage's workgroup ticket counter
  unsigned wait_limit = 0;  // bounded waits poll at most this often (0: each wait's own bound)
  bool single_stage = false;  // run in one stage: no side stream, nothing created on first use
  // The whole-layer call (set even where y is null, as it may be for an empty batch): its first
  // prep clears the exchange words and the workgroup role counters.
  bool layer = false;
};

// Process-wide poll bound handed to every bf16 prefill launch (agnes_gdn_set_wait_limit).
unsigned prefill_wait_limit();
// The C-ABI status of a HIP error (recorded for agnes_gdn_last_hip_error on this thread).
int hip_report(hipError_t e);
// agnes_gdn_layer_prefill's argument checks and launch, on a given workspace.
int layer_prefill_checked(const void* x, int64_t x_token_stride, int dtype, const void* conv_weight,
                          const void* conv_bias, void* conv_state, const float* g, const float* beta,
                          const int32_t* cu_seqlens, int num_seqs, int64_t total_tokens, int num_k_heads,
                          int num_v_heads, int head_dim, float scale, float l2norm_eps, const float* initial_state,
                          float* final_state, const void* z, int64_t z_token_stride, const void* norm_weight,
                          float norm_eps, void* y, void* o, int out_dtype, void* workspace, size_t workspace_bytes,
                          void* stream, bool single_stage);

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  int in_dtype;
  int64_t qk_stride;
  int64_t v_stride;
  const float* g;
  const float* beta;
  int batch;
  int hk;
  int hv;
  float scale;
  float* state;
  void* o;
  int o_dtype;
};

struct FusedDecodeArgs {
  const void* x;       // [batch, (2 hk + hv) * 128], channels q | k | v
  int64_t x_stride;
  int dtype;           // of x, conv_w, conv_b, conv_state, z, norm_w
  const void* conv_w;  // [channels, 4]
  const void* conv_b;  // [channels] or nullptr
  void* conv_state;    // [num_slots, channels, 3]
  const float* g;      // [batch, hv]
  const float* beta;   // [batch, hv]
  const void* z;       // [batch, hv, 128]
  const void* norm_w;  // [128]
  float* state;        // [num_slots, hv, 128, 128]
  const int32_t* slots;  // [batch] or nullptr (slot = entry)
  int num_slots;
  int batch;
  int hk;
  int hv;
  float scale;
  float l2_eps;
  float norm_eps;
  void* y;             // [batch, hv, 128]
  void* o;             // [batch, hv, 128] or nullptr
  int o_dtype;         // of y and o
};

struct NormArgs {
  const void* o;
  int o_dtype;
  const void* z;
  const void* w;
  int zw_dtype;
  float eps;
  int64_t rows;
  void* y;
  int y_dtype;
};

// Global attention layer (query heads hq, KV heads hkv, head dim 256, rotary on dims 0..63).
// Prefill: q, gate [T, hq, 256] and k, v [T, hkv, 256] bf16 rows with the given token strides;
// k_out receives the normalised, rotated k (bf16, token stride k_out_stride) and is what the
// attention reads; v_out (optional) a copy of v.  Decode: one token per batch entry, caches
// [batch, max_len, hkv, 256] bf16, cache_lens[b] tokens already cached.
struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* gate;
  int64_t q_stride, k_stride, v_stride, gate_stride;
  const void* q_norm_w;   // [256] bf16
  const void* k_norm_w;   // [256] bf16
  const int32_t* pos3;    // [3][pos3_stride] positions (text, height, width) or nullptr: text
  int64_t pos3_stride;
  const int32_t* cu;      // prefill: cu_seqlens [num_seqs + 1]
  int num_seqs;
  int64_t total;          // prefill: tokens; decode: batch
  int hq, hkv;
  float rope_base, eps, scale;  // scale <= 0: 1/sqrt(256)
  void* k_out;
  int64_t k_out_stride;
  void* v_out;
  int64_t v_out_stride;
  void* o;                // [T or batch, hq, 256]
  int o_dtype;
  void* workspace;
  size_t workspace_bytes;
  size_t off_off, tab_off;  // set by the launcher
  // decode
  void* k_cache;
  void* v_cache;
  int64_t max_len;
  const int32_t* cache_lens;
};

// The work-items of a launch (blocks x threads per block) are counted in 32 bits.  Each *_fits
// below says whether every launch of a call keeps to that for the given counts; the host layer
// reports AGNES_ERR_UNSUPPORTED, and launches nothing, when one does not.  Token counts reach
// them at most INT32_MAX.
inline bool grid_fits(unsigned __int128 blocks, unsigned threads) { return blocks * threads <= 0xffffffffu; }
bool prefill_mfma_fits(int num_seqs, int64_t total, int hk, int hv);
bool prefill_f32_fits(int num_seqs, int hv);
bool decode_fits(int batch, int hv);
bool decode_fused_fits(int batch, int hv);
bool norm_fits(int64_t rows);
bool attn_prefill_fits(int num_seqs, int64_t total, int hq, int hkv);
bool attn_decode_fits(int batch, int hq, int hkv, int64_t max_len);

hipError_t launch_attn_prefill(AttnArgs a, hipStream_t s);
size_t attn_prefill_workspace(int num_seqs, int64_t total);
hipError_t launch_attn_decode(AttnArgs a, hipStream_t s);
size_t attn_decode_workspace(int64_t batch, int hq, int hkv, int64_t max_len);

hipError_t launch_conv(const ConvArgs& a, hipStream_t s);
hipError_t launch_conv_history(const ConvArgs& a, hipStream_t s);  // final history only
hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t s);
hipError_t launch_prefill_mfma(const PrefillArgs& a, hipStream_t s);
size_t prefill_mfma_workspace(int num_seqs, int64_t total, int hk, int hv);
// Whole-layer prefill (conv + recurrence + gated RMSNorm): the scan workgroups of one value head
// exchange per-token partial sums, so every workgroup of the grid must be resident at once
size_t layer_prefill_workspace(int num_seqs, int64_t total, int hk, int hv);
hipError_t launch_layer_prefill(const PrefillArgs& a, hipStream_t s);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t s);
hipError_t launch_gated_rmsnorm(const NormArgs& a, hipStream_t s);
hipError_t launch_decode_fused(const FusedDecodeArgs& a, hipStream_t s);
hipError_t release_side_queues();
bool set_stage_cuts(const int* cuts, int n);
hipError_t launch_rmw_stream(void* p, size_t bytes, hipStream_t s);
hipError_t launch_mfma_peak(float* sink, int blocks, int iters, hipStream_t s);

}  // namespace agnes
