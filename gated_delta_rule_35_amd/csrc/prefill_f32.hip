// Chunked prefill of the gated delta rule for fp32 inputs: every product in fp32 on the
// vector ALUs (discosf article "Agnes 3.0 Flash 刚上线就刷屏…", section 二.1: chunked
// prefill with chunk 64; model card "Agnes-3.0-Flash Preview", 架构 table: fp32 state).
//
// Chunk algebra (exact re-association of the token recurrence; WY/UT form of Yang et al.,
// "Parallelizing Linear Transformers with the Delta Rule over Sequence Length", NeurIPS
// 2024, with the gate of Gated Delta Networks, ICLR 2025).  Inside a chunk with rows
// r = 0..63, gamma_r = g_0 + ... + g_r and S the state entering the chunk:
//   A  = strict_lower(beta_r exp(gamma_r - gamma_s) k_r.k_s),   X = (I + A)^-1
//   U  = X diag(beta) (V - diag(exp gamma) K S^T)          (pseudo-values)
//   O  = diag(exp gamma) Q S^T + P U,  P = lower_incl(exp(gamma_r - gamma_s) q_r.k_s)
//   S <- exp(gamma_63) S + (diag(exp(gamma_63 - gamma)) U)^T K
// Rows past the end of a partial chunk are zero with beta = g = 0, which makes them
// contribute nothing.  One workgroup per (sequence, value head, block of 32 value rows):
// the value rows of S are independent, so each block carries its own slice of the state.
#include "common.h"
#include "launch.h"

namespace agnes {

namespace f32p {
constexpr int C = 64, D = 128, DVB = 32, NB = D / DVB;
}

template <int O_DT>
__global__ __launch_bounds__(256) void prefill_f32_kernel(PrefillArgs a) {
  using namespace f32p;
  __shared__ float Ks[C][D + 1], Qs[C][D + 1], Ss[DVB][D + 1];
  __shared__ float Vs[C][DVB + 1], Us[C][DVB + 1];
  __shared__ float As[C][C + 1], Ps[C][C + 1], Xs[C][C + 1];
  __shared__ float gam[C], bet[C], eg[C], egl[C];

  const int tid = threadIdx.x;
  const int blk = blockIdx.x % NB;
  const int h = (blockIdx.x / NB) % a.hv;
  const int n = blockIdx.x / (NB * a.hv);
  const int kh = h / (a.hv / a.hk);
  const int dv0 = blk * DVB;
  const int64_t start = cu_at(a.cu, n, a.total);
  int64_t end = cu_at(a.cu, n + 1, a.total);
  if (end < start) end = start;
  const int64_t sbase = ((int64_t)n * a.hv + h) * (D * D);

  for (int idx = tid; idx < DVB * D; idx += 256) {
    const int i = idx / D, j = idx % D;
    Ss[i][j] = a.s0 ? a.s0[sbase + (int64_t)(dv0 + i) * D + j] : 0.f;
  }

  for (int64_t c0 = start; c0 < end; c0 += C) {
    const int L = (int)((end - c0) < C ? (end - c0) : C);
    __syncthreads();  // previous chunk done with every buffer
    for (int idx = tid; idx < C * D; idx += 256) {
      const int r = idx / D, d = idx % D;
      const int64_t off = (c0 + r) * a.qk_stride + (int64_t)kh * D + d;
      Ks[r][d] = r < L ? static_cast<const float*>(a.k)[off] : 0.f;
      Qs[r][d] = r < L ? static_cast<const float*>(a.q)[off] : 0.f;
    }
    for (int idx = tid; idx < C * DVB; idx += 256) {
      const int r = idx / DVB, j = idx % DVB;
      Vs[r][j] = r < L ? static_cast<const float*>(a.v)[(c0 + r) * a.v_stride + (int64_t)h * D + dv0 + j] : 0.f;
    }
    if (tid < 64) {
      const int r = tid;
      float gv = r < L ? a.g[(c0 + r) * a.hv + h] : 0.f;
      const float bv = r < L ? a.beta[(c0 + r) * a.hv + h] : 0.f;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float t = __shfl_up(gv, off, 64);
        if (r >= off) gv += t;
      }
      gam[r] = gv;
      bet[r] = bv;
      eg[r] = expf(gv);
      egl[r] = expf(__shfl(gv, 63, 64) - gv);
    }
    __syncthreads();

    {  // Gram products -> A (strictly lower) and P (lower incl.), 4x4 register blocks
      const int rb = tid / 16, sb = tid % 16;
      float gk[4][4] = {}, gq[4][4] = {};
      for (int d = 0; d < D; ++d) {
        float kr[4], qr[4], ks[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          kr[i] = Ks[4 * rb + i][d];
          qr[i] = Qs[4 * rb + i][d];
          ks[i] = Ks[4 * sb + i][d];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            gk[i][j] = fmaf(kr[i], ks[j], gk[i][j]);
            gq[i][j] = fmaf(qr[i], ks[j], gq[i][j]);
          }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = 4 * rb + i, s = 4 * sb + j;
          const float dec = s <= r ? expf(gam[r] - gam[s]) : 0.f;
          As[r][s] = s < r ? bet[r] * dec * gk[i][j] : 0.f;
          Ps[r][s] = s <= r ? dec * gq[i][j] : 0.f;
        }
    }
    float qs[2][4] = {};
    const int tr = tid / 8, dq = tid % 8;  // rows 2tr, 2tr+1; value cols 4dq..4dq+3
    {  // K S^T and Q S^T, then R' = beta (V - exp(gamma) K S^T) in place of V
      float ks[2][4] = {};
      for (int d = 0; d < D; ++d) {
        float sv[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) sv[j] = Ss[4 * dq + j][d];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const float kv = Ks[2 * tr + i][d], qv = Qs[2 * tr + i][d];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            ks[i][j] = fmaf(kv, sv[j], ks[i][j]);
            qs[i][j] = fmaf(qv, sv[j], qs[i][j]);
          }
        }
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = 2 * tr + i;
#pragma unroll
        for (int j = 0; j < 4; ++j) Vs[r][4 * dq + j] = bet[r] * (Vs[r][4 * dq + j] - eg[r] * ks[i][j]);
      }
    }
    __syncthreads();
    if (tid < 64) {  // X = (I + A)^-1 by forward substitution, one column per lane
      const int col = tid;
      for (int r = 0; r < C; ++r) {
        float acc = r == col ? 1.f : 0.f;
        for (int s = col; s < r; ++s) acc = fmaf(-As[r][s], Xs[s][col], acc);
        Xs[r][col] = acc;  // zero above the diagonal (r < col)
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 2; ++i) {  // U = X R'
      const int r = 2 * tr + i;
      float u[4] = {};
      for (int s = 0; s <= r; ++s) {
        const float xv = Xs[r][s];
#pragma unroll
        for (int j = 0; j < 4; ++j) u[j] = fmaf(xv, Vs[s][4 * dq + j], u[j]);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) Us[r][4 * dq + j] = u[j];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 2; ++i) {  // O = diag(exp gamma) Q S^T + P U
      const int r = 2 * tr + i;
      float ov[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) ov[j] = eg[r] * qs[i][j];
      for (int s = 0; s <= r; ++s) {
        const float pv = Ps[r][s];
#pragma unroll
        for (int j = 0; j < 4; ++j) ov[j] = fmaf(pv, Us[s][4 * dq + j], ov[j]);
      }
      if (r < L) {
        const int64_t ob = ((c0 + r) * a.hv + h) * (int64_t)D + dv0 + 4 * dq;
#pragma unroll
        for (int j = 0; j < 4; ++j) store1<O_DT>(a.o, ob + j, a.scale * ov[j]);
      }
    }
    {  // S <- exp(gamma_63) S + (diag(exp(gamma_63 - gamma)) U)^T K
      const int i = tid / 8, d0 = (tid % 8) * 16;
      const float dec = eg[C - 1];
      float acc[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[j] = dec * Ss[i][d0 + j];
      for (int r = 0; r < C; ++r) {
        const float u = egl[r] * Us[r][i];
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[j] = fmaf(u, Ks[r][d0 + j], acc[j]);
      }
#pragma unroll
      for (int j = 0; j < 16; ++j) Ss[i][d0 + j] = acc[j];
    }
  }
  __syncthreads();
  if (a.s1) {
    for (int idx = tid; idx < DVB * D; idx += 256) {
      const int i = idx / D, j = idx % D;
      a.s1[sbase + (int64_t)(dv0 + i) * D + j] = Ss[i][j];
    }
  }
}

bool prefill_f32_fits(int num_seqs, int hv) {
  return grid_fits((unsigned __int128)num_seqs * (unsigned)hv * f32p::NB, 256);
}

hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t st) {
  const int64_t nblk = (int64_t)a.num_seqs * a.hv * f32p::NB;
  if (nblk == 0) return hipSuccess;
  if (a.o_dtype == DT_BF16) hipLaunchKernelGGL((prefill_f32_kernel<DT_BF16>), dim3((unsigned)nblk), dim3(256), 0, st, a);
  else hipLaunchKernelGGL((prefill_f32_kernel<DT_F32>), dim3((unsigned)nblk), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace agnes
