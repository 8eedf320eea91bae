// Depth-wise causal convolution (kernel 4) + SiLU + per-head L2 normalisation of the q and
// k heads, in front of the gated delta rule (model card "Agnes-3.0-Flash Preview", 架构
// table, delta-rule row: causal conv of kernel 4; discosf article "Agnes 3.0 Flash
// 刚上线就刷屏…", section 二.1: the same kernel-4 causal conv).
//
//   y[t, c] = SiLU(bias[c] + sum_j w[c, j] * xh[t - 3 + j, c]),  w[c, 3] on the current token,
//
// with xh taken from the sequence's conv history before its first token.  HBM-bound
// streaming kernels: each thread owns 8 consecutive channels (one 16-byte bf16 vector)
// and walks a block of tokens, keeping the three previous inputs in registers, so x is
// read once (plus a 3-token halo per block) and y written once, with non-temporal stores.
// Sixteen lanes cover one 128-channel head, so the L2 norm is a 16-lane reduction at each
// token.
#include "common.h"
#include "launch.h"

namespace agnes {

constexpr int CONV_TB = 32;       // tokens per block
constexpr int CONV_BATCH = 4;     // tokens whose loads are issued together
constexpr int CONV_THREADS = 256;  // 256 x 8 = 2048 channels per block

template <int DT>
__device__ __forceinline__ void load_hist8(const ConvArgs& a, int n, int c0, int idx, float out[8]) {
  // history entry idx (0 = oldest) of channels c0..c0+7 of sequence n
  const int64_t base = ((int64_t)n * a.channels + c0) * 3;
#pragma unroll
  for (int e = 0; e < 8; ++e) out[e] = load1<DT>(a.state, base + e * 3 + idx);
}

// The whole history of channels c0..c0+7 of sequence n: 24 contiguous elements (entry j of
// channel c0 + e at 3 e + j).  VEC: three 16-byte vectors each way (the host found the history
// 16-byte aligned; an 8-channel group then starts on a 48-byte boundary for bf16, 96 for f32).
template <int DT, bool VEC>
__device__ __forceinline__ void load_hist_all(const ConvArgs& a, int n, int c0, float h[3][8]) {
  if constexpr (VEC) {
    const int64_t base = ((int64_t)n * a.channels + c0) * 3;
    Raw8<DT> r[3];
#pragma unroll
    for (int q = 0; q < 3; ++q) r[q] = load_raw8<DT>(a.state, base + 8 * q);
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
      for (int j = 0; j < 3; ++j) h[j][e] = raw_at<DT>(r, 3 * e + j);
  } else {
#pragma unroll
    for (int j = 0; j < 3; ++j) load_hist8<DT>(a, n, c0, j, h[j]);
  }
}
template <int DT, bool VEC>
__device__ __forceinline__ void store_hist_all(const ConvArgs& a, int n, int c0, const float h0[8], const float h1[8],
                                               const float h2[8]) {
  const int64_t base = ((int64_t)n * a.channels + c0) * 3;
  if constexpr (VEC) {
    float f[24];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      f[3 * e] = h0[e];
      f[3 * e + 1] = h1[e];
      f[3 * e + 2] = h2[e];
    }
#pragma unroll
    for (int q = 0; q < 3; ++q) store8<DT>(a.state, base + 8 * q, f + 8 * q);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      store1<DT>(a.state, base + e * 3 + 0, h0[e]);
      store1<DT>(a.state, base + e * 3 + 1, h1[e]);
      store1<DT>(a.state, base + e * 3 + 2, h2[e]);
    }
  }
}

template <int DT>
__device__ __forceinline__ void conv_token(const ConvArgs& a, const float w[8][4], const float bias[8],
                                           const float h0[8], const float h1[8], const float h2[8],
                                           const float xc[8], bool l2, bool active, float y[8]) {
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float acc = bias[e];
    acc = fmaf(w[e][0], h0[e], acc);
    acc = fmaf(w[e][1], h1[e], acc);
    acc = fmaf(w[e][2], h2[e], acc);
    acc = fmaf(w[e][3], xc[e], acc);
    y[e] = active ? silu(acc) : 0.f;
    ss = fmaf(y[e], y[e], ss);
  }
  ss = sum16_dpp(ss);
  if (l2) {
    const float r = rsqrt_fast(ss + a.eps);
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] *= r;
  }
}

// Taps and bias of channels c0..c0+7.  VEC: as 16-byte vectors (the 32 taps and the 8 biases
// are contiguous), used where the host found weight and bias 16-byte aligned; else one element
// at a time (the C ABI asks only for 4-byte alignment).
template <int DT, bool VEC>
__device__ __forceinline__ void load_params(const ConvArgs& a, int c0, bool active, float w[8][4], float bias[8]) {
  if constexpr (VEC) {
    Raw8<DT> r[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) r[q] = active ? load_raw8<DT>(a.w, (int64_t)c0 * 4 + 8 * q) : Raw8<DT>{};
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
      for (int j = 0; j < 4; ++j) w[e][j] = raw_at<DT>(r, 4 * e + j);
    if (active && a.bias) load8<DT>(a.bias, c0, bias);
    else {
#pragma unroll
      for (int e = 0; e < 8; ++e) bias[e] = 0.f;
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
#pragma unroll
      for (int j = 0; j < 4; ++j) w[e][j] = active ? load1<DT>(a.w, (int64_t)(c0 + e) * 4 + j) : 0.f;
      bias[e] = (active && a.bias) ? load1<DT>(a.bias, c0 + e) : 0.f;
    }
  }
}

// Prefill over a packed batch: grid (channel blocks, token blocks).
template <int DT, bool VEC>
__global__ __launch_bounds__(CONV_THREADS) void conv_prefill_kernel(ConvArgs a) {
  const int c0 = (blockIdx.x * CONV_THREADS + threadIdx.x) * 8;
  const bool active = c0 < a.channels;
  const bool l2 = active && (c0 / 128) < a.l2_heads;
  const int64_t t0 = (int64_t)blockIdx.y * CONV_TB;
  const int64_t t1 = t0 + CONV_TB < a.total ? t0 + CONV_TB : a.total;

  float w[8][4], bias[8];
  load_params<DT, VEC>(a, c0, active, w, bias);

  // sequence holding t0: largest n with cu[n] <= t0
  int lo = 0, hi = a.num_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu_at(a.cu, mid, a.total) <= t0) lo = mid; else hi = mid - 1;
  }
  int n = lo;
  int64_t start = cu_at(a.cu, n, a.total);
  int64_t end = cu_at(a.cu, n + 1, a.total);

  // Fast path (the same for the whole block): its tokens and their 3-token halo lie in one
  // sequence.  Loads are issued a batch of tokens ahead of the arithmetic.
  if (start <= t0 - 3 && t1 <= end && t1 - t0 == CONV_TB) {
    float h[3][8] = {};
    if (active) {
#pragma unroll
      for (int j = 0; j < 3; ++j) load8<DT>(a.x, (t0 - 3 + j) * a.x_stride + c0, h[j]);
    }
    Raw8<DT> xb[2][CONV_BATCH] = {};
    if (active) {
#pragma unroll
      for (int i = 0; i < CONV_BATCH; ++i) xb[0][i] = load_raw8<DT>(a.x, (t0 + i) * a.x_stride + c0);
    }
#pragma unroll
    for (int b = 0; b < CONV_TB / CONV_BATCH; ++b) {
      if (active && b + 1 < CONV_TB / CONV_BATCH) {
#pragma unroll
        for (int i = 0; i < CONV_BATCH; ++i)
          xb[(b + 1) & 1][i] = load_raw8<DT>(a.x, (t0 + (b + 1) * CONV_BATCH + i) * a.x_stride + c0);
      }
#pragma unroll
      for (int i = 0; i < CONV_BATCH; ++i) {
        float xc[8], y[8];
        widen8<DT>(xb[b & 1][i], xc);
        conv_token<DT>(a, w, bias, h[0], h[1], h[2], xc, l2, active, y);
        if (active) store8_nt<DT>(a.y, (t0 + b * CONV_BATCH + i) * a.y_stride + c0, y);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          h[0][e] = h[1][e];
          h[1][e] = h[2][e];
          h[2][e] = xc[e];
        }
      }
    }
    return;
  }

  float h[3][8];
#pragma unroll
  for (int j = 0; j < 3; ++j) {  // h[j] = xh[t0 - 3 + j]
    const int64_t pos = t0 - 3 + j;
    if (!active) {
#pragma unroll
      for (int e = 0; e < 8; ++e) h[j][e] = 0.f;
    } else if (pos >= start) {
      load8<DT>(a.x, pos * a.x_stride + c0, h[j]);
    } else if (a.state) {
      load_hist8<DT>(a, n, c0, (int)(3 - (start - pos)), h[j]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) h[j][e] = 0.f;
    }
  }

  for (int64_t t = t0; t < t1; ++t) {
    if (t >= end) {  // next non-empty sequence starts at t
      while (n + 1 < a.num_seqs && cu_at(a.cu, n + 1, a.total) <= t) ++n;
      start = t;
      end = cu_at(a.cu, n + 1, a.total);
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        if (active && a.state) load_hist8<DT>(a, n, c0, j, h[j]);
        else {
#pragma unroll
          for (int e = 0; e < 8; ++e) h[j][e] = 0.f;
        }
      }
    }
    float xc[8], y[8];
    if (active) load8<DT>(a.x, t * a.x_stride + c0, xc);
    else {
#pragma unroll
      for (int e = 0; e < 8; ++e) xc[e] = 0.f;
    }
    conv_token<DT>(a, w, bias, h[0], h[1], h[2], xc, l2, active, y);
    if (active) store8_nt<DT>(a.y, t * a.y_stride + c0, y);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      h[0][e] = h[1][e];
      h[1][e] = h[2][e];
      h[2][e] = xc[e];
    }
  }
}

// Final history of every sequence, after the prefill kernel has read the old one:
// new[j] = xh[end - 3 + j] (old history for positions before the sequence start).
template <int DT, bool VEC>
__global__ __launch_bounds__(CONV_THREADS) void conv_state_kernel(ConvArgs a) {
  const int c0 = (blockIdx.x * CONV_THREADS + threadIdx.x) * 8;
  const int n = blockIdx.y;
  if (c0 >= a.channels) return;
  const int64_t start = cu_at(a.cu, n, a.total);
  int64_t end = cu_at(a.cu, n + 1, a.total);
  if (end < start) end = start;
  const int64_t len = end - start;
  float old[3][8], nw[3][8];
  load_hist_all<DT, VEC>(a, n, c0, old);
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const int64_t p = len - 3 + j;  // position relative to the sequence start
    if (p >= 0) load8<DT>(a.x, (start + p) * a.x_stride + c0, nw[j]);
    else {
#pragma unroll
      for (int e = 0; e < 8; ++e) nw[j][e] = old[3 + p][e];
    }
  }
  store_hist_all<DT, VEC>(a, n, c0, nw[0], nw[1], nw[2]);
}

// Decode: one token per sequence, history read and advanced in place.
template <int DT, bool VEC>
__global__ __launch_bounds__(CONV_THREADS) void conv_decode_kernel(ConvArgs a) {
  const int c0 = (blockIdx.x * CONV_THREADS + threadIdx.x) * 8;
  const int n = blockIdx.y;
  const bool active = c0 < a.channels;
  const bool l2 = active && (c0 / 128) < a.l2_heads;
  float w[8][4], bias[8], h[3][8] = {}, xc[8], y[8];
  load_params<DT, VEC>(a, c0, active, w, bias);
  if (active) load_hist_all<DT, VEC>(a, n, c0, h);
  if (active) load8<DT>(a.x, (int64_t)n * a.x_stride + c0, xc);
  else {
#pragma unroll
    for (int e = 0; e < 8; ++e) xc[e] = 0.f;
  }
  conv_token<DT>(a, w, bias, h[0], h[1], h[2], xc, l2, active, y);
  if (!active) return;
  store8_nt<DT>(a.y, (int64_t)n * a.y_stride + c0, y);
  store_hist_all<DT, VEC>(a, n, c0, h[1], h[2], xc);
}

static bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }
// Taps, bias and history as 16-byte vectors: every one of them present is 16-byte aligned.
static bool conv_vec(const ConvArgs& a) { return al16(a.w) && al16(a.bias) && al16(a.state); }

template <int DT, bool VEC>
static hipError_t launch_conv_t(const ConvArgs& a, hipStream_t st) {
  const unsigned cblocks = (unsigned)((a.channels / 8 + CONV_THREADS - 1) / CONV_THREADS);
  if (a.cu == nullptr) {
    if (a.num_seqs == 0) return hipSuccess;
    hipLaunchKernelGGL((conv_decode_kernel<DT, VEC>), dim3(cblocks, (unsigned)a.num_seqs), dim3(CONV_THREADS), 0, st,
                       a);
    return hipGetLastError();
  }
  if (a.total > 0) {
    const unsigned tblocks = (unsigned)((a.total + CONV_TB - 1) / CONV_TB);
    hipLaunchKernelGGL((conv_prefill_kernel<DT, VEC>), dim3(cblocks, tblocks), dim3(CONV_THREADS), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.state && a.num_seqs > 0) {
    hipLaunchKernelGGL((conv_state_kernel<DT, VEC>), dim3(cblocks, (unsigned)a.num_seqs), dim3(CONV_THREADS), 0, st,
                       a);
    return hipGetLastError();
  }
  return hipSuccess;
}

template <bool VEC>
static hipError_t launch_history_t(const ConvArgs& a, hipStream_t st) {
  const unsigned cblocks = (unsigned)((a.channels / 8 + CONV_THREADS - 1) / CONV_THREADS);
  if (a.dtype == DT_BF16)
    hipLaunchKernelGGL((conv_state_kernel<DT_BF16, VEC>), dim3(cblocks, (unsigned)a.num_seqs), dim3(CONV_THREADS), 0,
                       st, a);
  else
    hipLaunchKernelGGL((conv_state_kernel<DT_F32, VEC>), dim3(cblocks, (unsigned)a.num_seqs), dim3(CONV_THREADS), 0,
                       st, a);
  return hipGetLastError();
}

hipError_t launch_conv_history(const ConvArgs& a, hipStream_t st) {
  if (!a.state || a.num_seqs == 0) return hipSuccess;
  return al16(a.state) ? launch_history_t<true>(a, st) : launch_history_t<false>(a, st);
}

hipError_t launch_conv(const ConvArgs& a, hipStream_t st) {
  const bool vec = conv_vec(a);
  if (a.dtype == DT_BF16) return vec ? launch_conv_t<DT_BF16, true>(a, st) : launch_conv_t<DT_BF16, false>(a, st);
  return vec ? launch_conv_t<DT_F32, true>(a, st) : launch_conv_t<DT_F32, false>(a, st);
}

}  // namespace agnes
