// Stepwise decode of the gated delta rule (discosf article "Agnes 3.0 Flash 刚上线就刷屏…",
// section 二.1: the decode path advances the recurrence one token at a time; model card
// "Agnes-3.0-Flash Preview", 架构 table: fp32 recurrent state).
//
// One workgroup per (sequence, value head) performs a single read and a single write of
// that head's 128x128 fp32 state.  Using the rank-one structure of the gated delta rule
// (Gated Delta Networks, ICLR 2025):
//   d_i = beta (v_i - alpha (S k)_i),   o_i = alpha (S q)_i + d_i (k . q),
//   S_i <- alpha S_i + d_i k^T,
// for each value row i.  A row is spread over 16 lanes (8 floats each, as two 16-byte
// vectors 64 columns apart so every load instruction covers contiguous 256-byte row
// halves); the two dot products per row are reduced across those 16 lanes.  The
// 4 waves x 4 rows x 8 passes cover the 128 rows; all 16 state vectors of a lane are
// loaded before any arithmetic so the loads are in flight together.
#include "common.h"
#include "launch.h"

namespace agnes {

template <int IN_DT, int O_DT>
__global__ __launch_bounds__(256) void decode_step_kernel(DecodeArgs a) {
  const int bh = blockIdx.x;  // sequence * Hv + value head
  const int b = bh / a.hv;
  const int h = bh - b * a.hv;
  const int kh = h / (a.hv / a.hk);
  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int l = tid & 63;
  const int sub = l >> 4;
  const int c = (l & 15) * 4;

  float* S = a.state + (int64_t)bh * (128 * 128);
  f4 s[8][2];  // streaming loads and stores: the state is read once and written once
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int row = p * 16 + w * 4 + sub;
    s[p][0] = load_f4_stream(S + row * 128 + c);
    s[p][1] = load_f4_stream(S + row * 128 + 64 + c);
  }

  const int64_t qk_base = (int64_t)b * a.qk_stride + (int64_t)kh * 128;
  float kv[8], qv[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    kv[e] = load1<IN_DT>(a.k, qk_base + c + e);
    kv[4 + e] = load1<IN_DT>(a.k, qk_base + 64 + c + e);
    qv[e] = load1<IN_DT>(a.q, qk_base + c + e);
    qv[4 + e] = load1<IN_DT>(a.q, qk_base + 64 + c + e);
  }
  const int64_t v_base = (int64_t)b * a.v_stride + (int64_t)h * 128;
  float vrow[8];
#pragma unroll
  for (int p = 0; p < 8; ++p) vrow[p] = load1<IN_DT>(a.v, v_base + p * 16 + w * 4 + sub);

  const float alpha = __expf(a.g[bh]);
  const float beta = a.beta[bh];

  float kq = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) kq = fmaf(kv[e], qv[e], kq);
  kq = sum16_dpp(kq);

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
    const float d = beta * (vrow[p] - alpha * sk);
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = fmaf(alpha, x[e], d * kv[e]);
    store_f4_stream(S + row * 128 + c, f4{y[0], y[1], y[2], y[3]});
    store_f4_stream(S + row * 128 + 64 + c, f4{y[4], y[5], y[6], y[7]});
    if ((l & 15) == 0) store1<O_DT>(a.o, (int64_t)bh * 128 + row, a.scale * fmaf(alpha, sq, d * kq));
  }
}

bool decode_fits(int batch, int hv) { return grid_fits((unsigned __int128)batch * (unsigned)hv, 256); }

hipError_t launch_decode(const DecodeArgs& a, hipStream_t st) {
  if (a.batch == 0) return hipSuccess;
  dim3 grid((unsigned)a.batch * (unsigned)a.hv), block(256);
  if (a.in_dtype == DT_BF16) {
    if (a.o_dtype == DT_BF16) hipLaunchKernelGGL((decode_step_kernel<DT_BF16, DT_BF16>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((decode_step_kernel<DT_BF16, DT_F32>), grid, block, 0, st, a);
  } else {
    if (a.o_dtype == DT_BF16) hipLaunchKernelGGL((decode_step_kernel<DT_F32, DT_BF16>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((decode_step_kernel<DT_F32, DT_F32>), grid, block, 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace agnes
