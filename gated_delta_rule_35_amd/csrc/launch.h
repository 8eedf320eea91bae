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
};

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

hipError_t launch_conv(const ConvArgs& a, hipStream_t s);
hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t s);
hipError_t launch_prefill_mfma(const PrefillArgs& a, hipStream_t s);
size_t prefill_mfma_workspace(int num_seqs, int64_t total, int hk, int hv);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t s);
hipError_t launch_gated_rmsnorm(const NormArgs& a, hipStream_t s);

}  // namespace agnes
