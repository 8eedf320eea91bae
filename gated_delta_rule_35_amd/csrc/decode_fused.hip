// One decode token per sequence through the whole delta layer in one launch (discosf
// article "Agnes 3.0 Flash 刚上线就刷屏…", section 二.1: stepwise decode of the layer; model
// card "Agnes-3.0-Flash Preview", 架构 table, delta-rule row: kernel-4 causal conv in front,
// gated RMS-norm behind, fp32 recurrent state):
//
//   conv history update + conv + SiLU of the q, k, v channels, L2 norm of the q and k heads,
//   the gated delta-rule step on the fp32 state (rank-one form, as the unfused decode step),
//   then y = o / sqrt(mean(o^2) + eps) * w * SiLU(z) per value head.
//
// One workgroup per (batch entry, key head): it owns the conv channels of that key head's
// q and k heads and of its G = Hv / Hk value heads, so the conv history is read and written
// by one workgroup only, and q, k are convolved and normalised once for the G heads.  Each
// group of 256 threads (four waves) runs the state update of one value head exactly as the
// unfused step does (a row over 16 lanes, one read and one write of the 64 KiB state); its
// state loads are issued before the convolution so that they are in flight meanwhile.  q, k,
// v and o pass through LDS in fp32: nothing is rounded between the steps.
//
// A slot array maps batch entries to state and conv-history slots of a pool (entries whose
// slot is negative or beyond the pool are padding: their y and o rows are zero and nothing
// else is touched).
#include "common.h"
#include "launch.h"

namespace agnes {

constexpr int FD_MAX_GROUPS = 3;  // value heads in flight per workgroup (256 threads each)

template <int DT>
__device__ __forceinline__ void fd_conv_item(const FusedDecodeArgs& a, int b, int slot, int c0, bool l2, float* dst) {
  const int C = (2 * a.hk + a.hv) * 128;
  float x[8], hs[24], w[32], bias[8];
  load8<DT>(a.x, (int64_t)b * a.x_stride + c0, x);
  const int64_t sb = ((int64_t)slot * C + c0) * 3;  // history of channels c0..c0+7, oldest first
  load8<DT>(a.conv_state, sb, hs);
  load8<DT>(a.conv_state, sb + 8, hs + 8);
  load8<DT>(a.conv_state, sb + 16, hs + 16);
#pragma unroll
  for (int j = 0; j < 4; ++j) load8<DT>(a.conv_w, (int64_t)c0 * 4 + 8 * j, w + 8 * j);
  if (a.conv_b) load8<DT>(a.conv_b, c0, bias);
  else {
#pragma unroll
    for (int e = 0; e < 8; ++e) bias[e] = 0.f;
  }
  float y[8], ss = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float acc = bias[e];
    acc = fmaf(w[4 * e + 0], hs[3 * e + 0], acc);
    acc = fmaf(w[4 * e + 1], hs[3 * e + 1], acc);
    acc = fmaf(w[4 * e + 2], hs[3 * e + 2], acc);
    acc = fmaf(w[4 * e + 3], x[e], acc);
    y[e] = silu(acc);
    ss = fmaf(y[e], y[e], ss);
  }
  ss = sum16(ss);  // the 16 items of one head are 16 consecutive lanes
  const float r = l2 ? rsqrt_fast(ss + a.l2_eps) : 1.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) dst[e] = y[e] * r;
  // new history: the two newest old entries, then the current input
  float nh[24];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    nh[3 * e + 0] = hs[3 * e + 1];
    nh[3 * e + 1] = hs[3 * e + 2];
    nh[3 * e + 2] = x[e];
  }
  store8<DT>(a.conv_state, sb, nh);
  store8<DT>(a.conv_state, sb + 8, nh + 8);
  store8<DT>(a.conv_state, sb + 16, nh + 16);
}

template <int DT, int ODT>
__global__ __launch_bounds__(256 * FD_MAX_GROUPS) void decode_fused_kernel(FusedDecodeArgs a) {
  extern __shared__ __align__(16) float fd_smem[];
  const int G = a.hv / a.hk;
  const int ng = G < FD_MAX_GROUPS ? G : FD_MAX_GROUPS;
  const int b = blockIdx.x / a.hk;
  const int kh = blockIdx.x - b * a.hk;
  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  const int gi = tid >> 8;  // value-head group
  const int t = tid & 255;
  const int w = t >> 6, l = t & 63, sub = l >> 4, c = (l & 15) * 4;

  int slot = a.slots ? a.slots[b] : b;
  if (slot < 0 || slot >= a.num_slots) {  // padding entry
    for (int i = tid; i < G * 128; i += nthr) {
      const int64_t idx = ((int64_t)b * a.hv + (int64_t)kh * G) * 128 + i;
      store1<ODT>(a.y, idx, 0.f);
      if (a.o) store1<ODT>(a.o, idx, 0.f);
    }
    return;
  }

  float* qk_s = fd_smem;             // [2][128]: normalised q, k of the key head
  float* v_s = fd_smem + 256;        // [G][128]
  float* o_s = v_s + G * 128;        // [ng][128]

  // state loads of this group's first value head, in flight during the convolution
  float4 s[8][2];
  auto load_state = [&](int j) {
    const float* S = a.state + ((int64_t)slot * a.hv + (int64_t)kh * G + j) * (128 * 128);
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const int row = p * 16 + w * 4 + sub;
      s[p][0] = *reinterpret_cast<const float4*>(S + row * 128 + c);
      s[p][1] = *reinterpret_cast<const float4*>(S + row * 128 + 64 + c);
    }
  };
  if (DT == DT_BF16 && gi < G) load_state(gi);  // (f32 inputs: after the conv, fewer live registers)

  // conv of the q, k and G value heads: 16 items of 8 channels per head
  const int items = (2 + G) * 16;
  for (int it = tid; it < items; it += nthr) {
    const int hl = it >> 4;  // 0 = q head, 1 = k head, 2 + j = value head kh * G + j
    const int base = hl == 0 ? kh * 128 : (hl == 1 ? (a.hk + kh) * 128 : (2 * a.hk + kh * G + hl - 2) * 128);
    float* dst = hl < 2 ? qk_s + hl * 128 : v_s + (hl - 2) * 128;
    fd_conv_item<DT>(a, b, slot, base + (it & 15) * 8, hl < 2, dst + (it & 15) * 8);
  }
  __syncthreads();

  float kv[8], qv[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    kv[e] = qk_s[128 + c + e];
    kv[4 + e] = qk_s[128 + 64 + c + e];
    qv[e] = qk_s[c + e];
    qv[4 + e] = qk_s[64 + c + e];
  }
  float kq = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) kq = fmaf(kv[e], qv[e], kq);
  kq = sum16(kq);

  for (int j0 = 0; j0 < G; j0 += ng) {
    const int j = j0 + gi;
    const bool act = gi < ng && j < G;
    if (act) {
      if (j0 > 0 || DT != DT_BF16) load_state(j);
      const int h = kh * G + j;
      const int64_t bh = (int64_t)b * a.hv + h;
      float* S = a.state + ((int64_t)slot * a.hv + h) * (128 * 128);
      const float alpha = __expf(a.g[bh]);
      const float beta = a.beta[bh];
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        const int row = p * 16 + w * 4 + sub;
        const float x[8] = {s[p][0].x, s[p][0].y, s[p][0].z, s[p][0].w,
                            s[p][1].x, s[p][1].y, s[p][1].z, s[p][1].w};
        float sk = 0.f, sq = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          sk = fmaf(x[e], kv[e], sk);
          sq = fmaf(x[e], qv[e], sq);
        }
        sk = sum16(sk);
        sq = sum16(sq);
        const float d = beta * (v_s[j * 128 + row] - alpha * sk);
        float y[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = fmaf(alpha, x[e], d * kv[e]);
        *reinterpret_cast<float4*>(S + row * 128 + c) = make_float4(y[0], y[1], y[2], y[3]);
        *reinterpret_cast<float4*>(S + row * 128 + 64 + c) = make_float4(y[4], y[5], y[6], y[7]);
        if ((l & 15) == 0) o_s[gi * 128 + row] = a.scale * fmaf(alpha, sq, d * kq);
      }
    }
    __syncthreads();
    if (act && w == 0) {  // gated RMS-norm of head h by the group's first wave, two values a lane
      const int h = kh * G + j;
      const int64_t rb = ((int64_t)b * a.hv + h) * 128;
      const float o0 = o_s[gi * 128 + 2 * l], o1 = o_s[gi * 128 + 2 * l + 1];
      float ss = fmaf(o0, o0, o1 * o1);
      ss = sum16(ss);
      ss += __shfl_xor(ss, 16);
      ss += __shfl_xor(ss, 32);
      const float r = rsqrt_fast(ss * (1.0f / 128.0f) + a.norm_eps);
      const float y0 = o0 * r * load1<DT>(a.norm_w, 2 * l) * silu(load1<DT>(a.z, rb + 2 * l));
      const float y1 = o1 * r * load1<DT>(a.norm_w, 2 * l + 1) * silu(load1<DT>(a.z, rb + 2 * l + 1));
      store1<ODT>(a.y, rb + 2 * l, y0);
      store1<ODT>(a.y, rb + 2 * l + 1, y1);
      if (a.o) {
        store1<ODT>(a.o, rb + 2 * l, o0);
        store1<ODT>(a.o, rb + 2 * l + 1, o1);
      }
    }
    if (j0 + ng < G) __syncthreads();  // o_s is refilled by the next round
  }
}

template <int DT>
static void launch_fd_o(const FusedDecodeArgs& a, dim3 grid, dim3 block, size_t smem, hipStream_t st) {
  if (a.o_dtype == DT_BF16) hipLaunchKernelGGL((decode_fused_kernel<DT, DT_BF16>), grid, block, smem, st, a);
  else hipLaunchKernelGGL((decode_fused_kernel<DT, DT_F32>), grid, block, smem, st, a);
}

hipError_t launch_decode_fused(const FusedDecodeArgs& a, hipStream_t st) {
  if (a.batch == 0) return hipSuccess;
  const int G = a.hv / a.hk;
  const int ng = G < FD_MAX_GROUPS ? G : FD_MAX_GROUPS;
  const dim3 grid((unsigned)a.batch * (unsigned)a.hk), block(256 * ng);
  const size_t smem = (size_t)(2 + G + ng) * 128 * sizeof(float);
  if (a.dtype == DT_BF16) launch_fd_o<DT_BF16>(a, grid, block, smem, st);
  else launch_fd_o<DT_F32>(a, grid, block, smem, st);
  return hipGetLastError();
}

}  // namespace agnes
