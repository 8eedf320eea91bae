// One decode token per sequence through the whole delta layer (discosf article "Agnes 3.0
// Flash 刚上线就刷屏…", section 二.1: stepwise decode of the layer; model card
// "Agnes-3.0-Flash Preview", 架构 table, delta-rule row: kernel-4 causal conv in front, gated
// RMS-norm behind, fp32 recurrent state):
//
//   conv history update + conv + SiLU of the q, k, v channels, L2 norm of the q and k heads,
//   the gated delta-rule step on the fp32 state (rank-one form, as the unfused decode step),
//   then y = o / sqrt(mean(o^2) + eps) * w * SiLU(z) per value head.
//
// One workgroup of 256 threads per (batch entry, value head), laid out as the unfused step: it
// convolves the q and k heads of its key head and its own value head (48 items of 8 channels,
// wave 0), issues the streaming loads of its 64 KiB state, runs the state update (a row over 16
// lanes, one read and one write of the state), and wave 0 applies the gated norm.  The conv goes
// first and the norm's operands are loaded only for the norm, so that the state never shares the
// registers with other inputs: 104 registers, four workgroups per CU (state loads first: 147
// registers and three workgroups per CU, 2 % slower; the norm's z and weight loaded beside the
// state: 108 registers and 8 % slower).
// Each of the G = Hv / Hk workgroups of a key head convolves that key head's q and k channels
// from the old conv history, so that history is advanced only after all of them are done, by a
// second, small launch; a workgroup advances the history of its own value head's channels
// itself.  q, k, v and o pass through LDS in fp32: nothing is rounded between the steps.
//
// A slot array maps batch entries to state and conv-history slots of a pool (entries whose
// slot is negative or beyond the pool are padding: their y and o rows are zero and nothing
// else is touched).
#include "common.h"
#include "launch.h"

namespace agnes {

// New conv history of channels c0..c0+7 of one slot (sb: its first entry): the two newest old
// entries, then the current input (exact copies, oldest first).
template <int DT>
__device__ __forceinline__ void fd_history_store(const FusedDecodeArgs& a, int64_t sb, const Raw8<DT> (&xr)[1],
                                                 const Raw8<DT> (&hr)[3]) {
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    float nh[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int n = 8 * k + i, e = n / 3, j = n % 3;
      nh[i] = j < 2 ? raw_at<DT>(hr, 3 * e + j + 1) : raw_at<DT>(xr, e);
    }
    store8<DT>(a.conv_state, sb + 8 * k, nh);
  }
}

// Conv + SiLU (+ L2 over the 16 lanes of a head) of channels c0..c0+7 of entry b, result to
// dst (LDS); advance: also write the channels' new history.  Inputs stay as loaded (raw) and
// are widened where used.
template <int DT>
__device__ __forceinline__ void fd_conv_item(const FusedDecodeArgs& a, int b, int slot, int c0, bool l2, bool advance,
                                             float* dst) {
  const int C = (2 * a.hk + a.hv) * 128;
  const int64_t sb = ((int64_t)slot * C + c0) * 3;  // history of channels c0..c0+7, oldest first
  Raw8<DT> xr[1], hr[3], wr[4], br[1];
  xr[0] = load_raw8<DT>(a.x, (int64_t)b * a.x_stride + c0);
#pragma unroll
  for (int j = 0; j < 3; ++j) hr[j] = load_raw8<DT>(a.conv_state, sb + 8 * j);
#pragma unroll
  for (int j = 0; j < 4; ++j) wr[j] = load_raw8<DT>(a.conv_w, (int64_t)c0 * 4 + 8 * j);
  if (a.conv_b) br[0] = load_raw8<DT>(a.conv_b, c0);
  float y[8], ss = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float acc = a.conv_b ? raw_at<DT>(br, e) : 0.f;
    acc = fmaf(raw_at<DT>(wr, 4 * e + 0), raw_at<DT>(hr, 3 * e + 0), acc);
    acc = fmaf(raw_at<DT>(wr, 4 * e + 1), raw_at<DT>(hr, 3 * e + 1), acc);
    acc = fmaf(raw_at<DT>(wr, 4 * e + 2), raw_at<DT>(hr, 3 * e + 2), acc);
    acc = fmaf(raw_at<DT>(wr, 4 * e + 3), raw_at<DT>(xr, e), acc);
    y[e] = silu(acc);
    ss = fmaf(y[e], y[e], ss);
  }
  ss = sum16_dpp(ss);  // the 16 items of one head are 16 consecutive lanes
  const float r = l2 ? rsqrt_fast(ss + a.l2_eps) : 1.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) dst[e] = y[e] * r;
  if (advance) fd_history_store<DT>(a, sb, xr, hr);
}

template <int DT, int ODT>
__global__ __launch_bounds__(256) void decode_fused_kernel(FusedDecodeArgs a) {
  __shared__ float qk_s[256];  // normalised q, k of the key head
  __shared__ float v_s[128];
  __shared__ float o_s[128];
  const int G = a.hv / a.hk;
  const int b = blockIdx.x / a.hv;
  const int h = blockIdx.x - b * a.hv;
  const int kh = h / G;
  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, sub = l >> 4, c = (l & 15) * 4;
  const int64_t bh = (int64_t)b * a.hv + h;

  const int slot = a.slots ? a.slots[b] : b;
  if (slot < 0 || slot >= a.num_slots) {  // padding entry
    if (tid < 128) {
      store1<ODT>(a.y, bh * 128 + tid, 0.f);
      if (a.o) store1<ODT>(a.o, bh * 128 + tid, 0.f);
    }
    return;
  }

  if (tid < 48) {  // lanes 0-15: the q head, 16-31: the k head, 32-47: this value head
    const int hl = tid >> 4;
    const int base = hl == 0 ? kh * 128 : (hl == 1 ? (a.hk + kh) * 128 : (2 * a.hk + h) * 128);
    float* dst = hl == 0 ? qk_s : (hl == 1 ? qk_s + 128 : v_s);
    fd_conv_item<DT>(a, b, slot, base + (tid & 15) * 8, hl < 2, hl == 2, dst + (tid & 15) * 8);
  }
  // the state (streaming loads: read once, written once)
  float* S = a.state + ((int64_t)slot * a.hv + h) * (128 * 128);
  f4 s[8][2];
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int row = p * 16 + w * 4 + sub;
    s[p][0] = load_f4_stream(S + row * 128 + c);
    s[p][1] = load_f4_stream(S + row * 128 + 64 + c);
  }
  const float alpha = __expf(a.g[bh]);
  const float beta = a.beta[bh];
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
  kq = sum16_dpp(kq);

#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int row = p * 16 + w * 4 + sub;
    const float x[8] = {s[p][0].x, s[p][0].y, s[p][0].z, s[p][0].w, s[p][1].x, s[p][1].y, s[p][1].z, s[p][1].w};
    float sk = 0.f, sq = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      sk = fmaf(x[e], kv[e], sk);
      sq = fmaf(x[e], qv[e], sq);
    }
    sk = sum16_dpp(sk);
    sq = sum16_dpp(sq);
    const float d = beta * (v_s[row] - alpha * sk);
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = fmaf(alpha, x[e], d * kv[e]);
    store_f4_stream(S + row * 128 + c, f4{y[0], y[1], y[2], y[3]});
    store_f4_stream(S + row * 128 + 64 + c, f4{y[4], y[5], y[6], y[7]});
    if ((l & 15) == 0) o_s[row] = a.scale * fmaf(alpha, sq, d * kq);
  }
  __syncthreads();
  if (w == 0) {  // gated RMS-norm of the head, two values a lane
    const int64_t rb = bh * 128;
    float zn[2], wn[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      zn[i] = load1<DT>(a.z, bh * 128 + 2 * l + i);
      wn[i] = load1<DT>(a.norm_w, 2 * l + i);
    }
    const float o0 = o_s[2 * l], o1 = o_s[2 * l + 1];
    float ss = fmaf(o0, o0, o1 * o1);
    ss = sum16_dpp(ss);
    ss += __shfl_xor(ss, 16);
    ss += __shfl_xor(ss, 32);
    const float r = rsqrt_fast(ss * (1.0f / 128.0f) + a.norm_eps);
    store1<ODT>(a.y, rb + 2 * l, o0 * r * wn[0] * silu(zn[0]));
    store1<ODT>(a.y, rb + 2 * l + 1, o1 * r * wn[1] * silu(zn[1]));
    if (a.o) {
      store1<ODT>(a.o, rb + 2 * l, o0);
      store1<ODT>(a.o, rb + 2 * l + 1, o1);
    }
  }
}

// The conv history of the q and k channels, advanced after every workgroup of the step has read
// it: one thread per (entry, 8 channels); padding entries are left alone.
template <int DT>
__global__ __launch_bounds__(256) void fd_qk_history_kernel(FusedDecodeArgs a) {
  const int per = 2 * a.hk * 16;  // 8-channel items of the q and k heads of one entry
  const int64_t it = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (it >= (int64_t)a.batch * per) return;
  const int b = (int)(it / per), c0 = (int)(it - (int64_t)b * per) * 8;
  const int slot = a.slots ? a.slots[b] : b;
  if (slot < 0 || slot >= a.num_slots) return;
  const int C = (2 * a.hk + a.hv) * 128;
  const int64_t sb = ((int64_t)slot * C + c0) * 3;
  Raw8<DT> xr[1], hr[3];
  xr[0] = load_raw8<DT>(a.x, (int64_t)b * a.x_stride + c0);
#pragma unroll
  for (int j = 0; j < 3; ++j) hr[j] = load_raw8<DT>(a.conv_state, sb + 8 * j);
  fd_history_store<DT>(a, sb, xr, hr);
}

template <int DT>
static hipError_t launch_fd(const FusedDecodeArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)a.batch * (unsigned)a.hv), block(256);
  if (a.o_dtype == DT_BF16) hipLaunchKernelGGL((decode_fused_kernel<DT, DT_BF16>), grid, block, 0, st, a);
  else hipLaunchKernelGGL((decode_fused_kernel<DT, DT_F32>), grid, block, 0, st, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t items = (int64_t)a.batch * 2 * a.hk * 16;
  hipLaunchKernelGGL((fd_qk_history_kernel<DT>), dim3((unsigned)((items + 255) / 256)), dim3(256), 0, st, a);
  return hipGetLastError();
}

// the state update over (entry, value head); the q/k history over (entry, 8 q/k channels), fewer
bool decode_fused_fits(int batch, int hv) { return grid_fits((unsigned __int128)batch * (unsigned)hv, 256); }

hipError_t launch_decode_fused(const FusedDecodeArgs& a, hipStream_t st) {
  if (a.batch == 0) return hipSuccess;
  return a.dtype == DT_BF16 ? launch_fd<DT_BF16>(a, st) : launch_fd<DT_F32>(a, st);
}

}  // namespace agnes
