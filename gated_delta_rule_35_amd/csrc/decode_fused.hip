// One decode token per sequence through the whole delta layer in one launch (discosf
// article "Agnes 3.0 Flash 刚上线就刷屏…", section 二.1: stepwise decode of the layer; model
// card "Agnes-3.0-Flash Preview", 架构 table, delta-rule row: kernel-4 causal conv in front,
// gated RMS-norm behind, fp32 recurrent state):
//
//   conv history update + conv + SiLU of the q, k, v channels, L2 norm of the q and k heads,
//   the gated delta-rule step on the fp32 state (rank-one form, as the unfused decode step),
//   then y = o / sqrt(mean(o^2) + eps) * w * SiLU(z) per value head.
//
// One workgroup of 256 threads per (batch entry, key head): it owns the conv channels of that
// key head's q and k heads and of its G = Hv / Hk value heads, so the conv history is read and
// written by one workgroup only, and q, k are convolved and normalised once for the G heads.
// The workgroup then runs the state updates of the G value heads one after another, each as
// the unfused step does (a row over 16 lanes, one read and one write of the 64 KiB state); the
// first head's state loads are issued before the convolution so that they are in flight
// meanwhile, and two workgroups per CU (the register count allows no more) keep the memory
// busy between heads.  This runs about 2 % faster than three 256-thread groups in one
// workgroup (one head each), and on par with a register-capped build at three workgroups per
// CU.  q, k, v and o pass through LDS in fp32: nothing is rounded between the steps.
//
// A slot array maps batch entries to state and conv-history slots of a pool (entries whose
// slot is negative or beyond the pool are padding: their y and o rows are zero and nothing
// else is touched).
#include "common.h"
#include "launch.h"

namespace agnes {

// Conv + SiLU (+ L2 over the 16 lanes of a head) of channels c0..c0+7 of entry b, result to
// dst (LDS); the history of those channels in slot `slot` advances by the current input.
// Inputs stay as loaded (raw) and are widened where used, to keep registers free for the
// state loads in flight.
template <int DT>
__device__ __forceinline__ void fd_conv_item(const FusedDecodeArgs& a, int b, int slot, int c0, bool l2, float* dst) {
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
  // new history of channel e: its two newest old entries, then the current input (exact copies)
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

template <int DT, int ODT>
__global__ __launch_bounds__(256) void decode_fused_kernel(FusedDecodeArgs a) {
  extern __shared__ __align__(16) float fd_smem[];
  const int G = a.hv / a.hk;
  const int b = blockIdx.x / a.hk;
  const int kh = blockIdx.x - b * a.hk;
  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, sub = l >> 4, c = (l & 15) * 4;

  const int slot = a.slots ? a.slots[b] : b;
  if (slot < 0 || slot >= a.num_slots) {  // padding entry
    for (int i = tid; i < G * 128; i += 256) {
      const int64_t idx = ((int64_t)b * a.hv + (int64_t)kh * G) * 128 + i;
      store1<ODT>(a.y, idx, 0.f);
      if (a.o) store1<ODT>(a.o, idx, 0.f);
    }
    return;
  }

  float* qk_s = fd_smem;       // [2][128]: normalised q, k of the key head
  float* v_s = fd_smem + 256;  // [G][128]
  float* o_s = v_s + G * 128;  // [4][128]: o of head j in slot j % 4, normalised by wave j % 4

  f4 s[8][2];  // streaming loads and stores: each state is read once and written once
  auto load_state = [&](int j) {
    const float* S = a.state + ((int64_t)slot * a.hv + (int64_t)kh * G + j) * (128 * 128);
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const int row = p * 16 + w * 4 + sub;
      s[p][0] = load_f4_stream(S + row * 128 + c);
      s[p][1] = load_f4_stream(S + row * 128 + 64 + c);
    }
  };
  if (DT == DT_BF16) load_state(0);  // (f32 inputs: after the conv, fewer live registers)

  // conv of the q, k and G value heads: 16 items of 8 channels per head
  const int items = (2 + G) * 16;
  for (int it = tid; it < items; it += 256) {
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
  kq = sum16_dpp(kq);

  for (int j = 0; j < G; ++j) {
    if (j > 0 || DT != DT_BF16) load_state(j);
    const int h = kh * G + j;
    const int64_t bh = (int64_t)b * a.hv + h;
    float* S = a.state + ((int64_t)slot * a.hv + h) * (128 * 128);
    float* oj = o_s + (j & 3) * 128;
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
      sk = sum16_dpp(sk);
      sq = sum16_dpp(sq);
      const float d = beta * (v_s[j * 128 + row] - alpha * sk);
      float y[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] = fmaf(alpha, x[e], d * kv[e]);
      store_f4_stream(S + row * 128 + c, f4{y[0], y[1], y[2], y[3]});
      store_f4_stream(S + row * 128 + 64 + c, f4{y[4], y[5], y[6], y[7]});
      if ((l & 15) == 0) oj[row] = a.scale * fmaf(alpha, sq, d * kq);
    }
    // Slot j % 4 is rewritten at head j + 4, after three more barriers that wave j % 4 reaches
    // only once this norm is done.
    __syncthreads();
    if (w == (j & 3)) {  // gated RMS-norm of head h, two values a lane
      const int64_t rb = bh * 128;
      const float o0 = oj[2 * l], o1 = oj[2 * l + 1];
      float ss = fmaf(o0, o0, o1 * o1);
      ss = sum16_dpp(ss);
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
  }
}

template <int DT>
static void launch_fd_o(const FusedDecodeArgs& a, dim3 grid, dim3 block, size_t smem, hipStream_t st) {
  if (a.o_dtype == DT_BF16) hipLaunchKernelGGL((decode_fused_kernel<DT, DT_BF16>), grid, block, smem, st, a);
  else hipLaunchKernelGGL((decode_fused_kernel<DT, DT_F32>), grid, block, smem, st, a);
}

bool decode_fused_fits(int batch, int hk) { return grid_fits((unsigned __int128)batch * (unsigned)hk, 256); }

hipError_t launch_decode_fused(const FusedDecodeArgs& a, hipStream_t st) {
  if (a.batch == 0) return hipSuccess;
  const int G = a.hv / a.hk;
  const dim3 grid((unsigned)a.batch * (unsigned)a.hk), block(256);
  const size_t smem = (size_t)(2 + G + 4) * 128 * sizeof(float);  // <= 63 KiB for G <= 120
  if (a.dtype == DT_BF16) launch_fd_o<DT_BF16>(a, grid, block, smem, st);
  else launch_fd_o<DT_F32>(a, grid, block, smem, st);
  return hipGetLastError();
}

}  // namespace agnes
