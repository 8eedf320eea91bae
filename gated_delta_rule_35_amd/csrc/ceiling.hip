// Measured ceilings of the machine the layer runs on, for the benchmark's roofline fractions:
// an in-place HBM read-modify-write stream (the access pattern of the decode step's state
// update) and the matrix-core issue rate of bf16 16x16x32 products held in registers.
#include <hip/hip_runtime.h>

#include "launch.h"

namespace agnes {

// p[i] *= a over n4 16-byte vectors, grid-stride.  Each vector is read once and written once,
// with the non-temporal hint on both (the decode step's own access, and the faster of the two
// forms on gfx950).
typedef float f4v __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(256) void rmw_stream_kernel(f4v* __restrict__ p, size_t n4, float a) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += (size_t)gridDim.x * blockDim.x) {
    const f4v v = __builtin_nontemporal_load(p + i);
    __builtin_nontemporal_store(v * a, p + i);
  }
}

// Every wave issues `iters` rounds of 8 independent bf16 16x16x32 products (each accumulator
// is reused 8 products later, which the matrix core issues at its full rate) on operands held
// in registers; one float per wave goes to `sink` so that nothing is optimised away.  The
// products are written as inline assembly so that the accumulators stay in the vector
// registers the products read (no copies between register files inside the loop).
typedef __bf16 bf8v __attribute__((ext_vector_type(8)));
#define AGNES_MFMA_BF16(acc) asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b))
__global__ __launch_bounds__(256) void mfma_peak_kernel(float* sink, int iters) {
  bf8v a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (float)((threadIdx.x + i) & 15));
    b[i] = (__bf16)(0.002f * (float)i);
  }
  f4v c0 = {}, c1 = {}, c2 = {}, c3 = {}, c4 = {}, c5 = {}, c6 = {}, c7 = {};
  for (int it = 0; it < iters; ++it) {
    AGNES_MFMA_BF16(c0);
    AGNES_MFMA_BF16(c1);
    AGNES_MFMA_BF16(c2);
    AGNES_MFMA_BF16(c3);
    AGNES_MFMA_BF16(c4);
    AGNES_MFMA_BF16(c5);
    AGNES_MFMA_BF16(c6);
    AGNES_MFMA_BF16(c7);
  }
  // the products' results are read only after s_nop padding the compiler cannot see through the
  // asm: a full wait for outstanding matrix-core work first
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::);
  const f4v s = c0 + c1 + c2 + c3 + c4 + c5 + c6 + c7;
  if ((threadIdx.x & 63) == 0) sink[(size_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6)] = s[0] + s[1] + s[2] + s[3];
}
#undef AGNES_MFMA_BF16

hipError_t launch_rmw_stream(void* p, size_t bytes, hipStream_t s) {
  const size_t n4 = bytes / 16;
  if (n4 == 0) return hipSuccess;
  hipLaunchKernelGGL(rmw_stream_kernel, dim3(1024), dim3(256), 0, s, static_cast<f4v*>(p), n4, 1.0f);
  return hipGetLastError();
}

hipError_t launch_mfma_peak(float* sink, int blocks, int iters, hipStream_t s) {
  if (blocks <= 0 || iters <= 0) return hipSuccess;
  hipLaunchKernelGGL(mfma_peak_kernel, dim3(blocks), dim3(256), 0, s, sink, iters);
  return hipGetLastError();
}

}  // namespace agnes
