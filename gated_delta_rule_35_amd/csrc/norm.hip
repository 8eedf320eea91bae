// Gated RMSNorm after the recurrence (model card "Agnes-3.0-Flash Preview", 架构 table,
// delta-rule row: gated RMS-norm), per row of 128 values:
//   y = o / sqrt(mean(o^2) + eps) * w * z * sigmoid(z).
// HBM-bound stream: 16 lanes own one row (8 values each, one 16-byte bf16 vector), a
// 256-thread block covers 16 rows per pass and walks NORM_PASSES passes, with the loads of
// all passes issued (kept as loaded, widened at use) before any arithmetic.  y goes out with
// non-temporal stores (5 % faster than plain ones; streaming loads of o and z gain nothing).
#include "common.h"
#include "launch.h"

namespace agnes {

constexpr int NORM_PASSES = 8;
constexpr int NORM_ROWS = 16 * NORM_PASSES;  // rows per block

template <int ODT, int ZDT, int YDT>
__global__ __launch_bounds__(256) void gated_rmsnorm_kernel(NormArgs a) {
  const int lane16 = threadIdx.x & 15;
  const int c0 = lane16 * 8;
  float w[8];
  load8<ZDT>(a.w, c0, w);
  const int64_t row0 = (int64_t)blockIdx.x * NORM_ROWS + (threadIdx.x >> 4);
  Raw8<ODT> orw[NORM_PASSES] = {};
  Raw8<ZDT> zrw[NORM_PASSES] = {};
#pragma unroll
  for (int p = 0; p < NORM_PASSES; ++p) {
    const int64_t r = row0 + p * 16;
    if (r < a.rows) {
      orw[p] = load_raw8<ODT>(a.o, r * 128 + c0);
      zrw[p] = load_raw8<ZDT>(a.z, r * 128 + c0);
    }
  }
#pragma unroll
  for (int p = 0; p < NORM_PASSES; ++p) {
    float o[1][8], z[1][8];
    widen8<ODT>(orw[p], o[0]);
    widen8<ZDT>(zrw[p], z[0]);
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = fmaf(o[0][e], o[0][e], ss);
    ss = sum16(ss);
    const float r = rsqrt_fast(ss * (1.0f / 128.0f) + a.eps);
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = o[0][e] * r * w[e] * silu(z[0][e]);
    const int64_t row = row0 + p * 16;
    if (row < a.rows) store8_nt<YDT>(a.y, row * 128 + c0, y);
  }
}

template <int ODT, int ZDT>
static void launch_y(const NormArgs& a, dim3 g, hipStream_t st) {
  if (a.y_dtype == DT_BF16) hipLaunchKernelGGL((gated_rmsnorm_kernel<ODT, ZDT, DT_BF16>), g, dim3(256), 0, st, a);
  else hipLaunchKernelGGL((gated_rmsnorm_kernel<ODT, ZDT, DT_F32>), g, dim3(256), 0, st, a);
}

bool norm_fits(int64_t rows) { return grid_fits((unsigned __int128)(rows / NORM_ROWS + (rows % NORM_ROWS != 0)), 256); }

hipError_t launch_gated_rmsnorm(const NormArgs& a, hipStream_t st) {
  if (a.rows == 0) return hipSuccess;
  dim3 g((unsigned)((a.rows + NORM_ROWS - 1) / NORM_ROWS));
  if (a.o_dtype == DT_BF16) {
    if (a.zw_dtype == DT_BF16) launch_y<DT_BF16, DT_BF16>(a, g, st);
    else launch_y<DT_BF16, DT_F32>(a, g, st);
  } else {
    if (a.zw_dtype == DT_BF16) launch_y<DT_F32, DT_BF16>(a, g, st);
    else launch_y<DT_F32, DT_F32>(a, g, st);
  }
  return hipGetLastError();
}

}  // namespace agnes
