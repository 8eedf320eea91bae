// Chunked prefill of the gated delta rule on gfx950 matrix cores (discosf article "Agnes 3.0
// Flash 刚上线就刷屏…", section 二.1: chunked prefill with chunk 64; model card
// "Agnes-3.0-Flash Preview", 架构 table: fp32 recurrent state).
//
// Chunk algebra (exact re-association of the token recurrence; WY/UT form of Yang et al.,
// "Parallelizing Linear Transformers with the Delta Rule over Sequence Length", NeurIPS 2024,
// with the gate of Gated Delta Networks, ICLR 2025).  Rows r = 0..63 of a chunk,
// gamma_r = g_0 + ... + g_r, S the state entering the chunk ([value][key]):
//   A = strict_lower(beta_r exp(gamma_r - gamma_s) k_r.k_s),  X = (I + A)^-1
//   R' = diag(beta) (V - diag(exp gamma) K S^T),  U = X R'
//   O  = diag(exp gamma) Q S^T + P U,  P = lower_incl(exp(gamma_r - gamma_s) q_r.k_s)
//   S <- exp(gamma_63) S + (diag(exp(gamma_63 - gamma)) U)^T K
// Rows past the end of a partial chunk are zero with beta = g = 0 and contribute nothing.
//
// Mapping to the hardware:
//  * one workgroup of 4 waves per (sequence, value head, block of DVB value rows): the value
//    rows of S are independent, so every block scans its own [DVB x 128] fp32 slice of the
//    state, which lives in MFMA accumulators for the whole sequence (never leaves the CU);
//  * every product runs on v_mfma_f32_16x16x32_f16 (16x16x16 for the 16-wide triangular
//    blocks) with fp16 operands and fp32 accumulation.  bf16 inputs widen exactly to fp16
//    in its normal range; fp32 intermediates (S, X, R', U, P) are rounded to fp16 once per
//    use, 2^-11 relative, 8x finer than bf16;
//  * X is built blockwise: the four 16x16 diagonal blocks by fp32 forward substitution,
//    the off-diagonal blocks by the block recurrence X_ij = -X_ii sum_k A_ik X_kj on matrix
//    cores, keeping each column block's results in registers (a 16x16x16 result fragment
//    is already laid out as the next product's B operand);
//  * all operands are staged in LDS "k-contiguous" (A as [m][k], B as [n][k]) so every
//    fragment is one 8- or 16-byte LDS read; rows are padded to avoid bank conflicts;
//  * the next chunk's global loads are issued before the current chunk's compute.
#include "common.h"
#include "launch.h"

namespace agnes {

namespace mp {
constexpr int C = 64;       // chunk
constexpr int D = 128;      // head dim (key and value)
constexpr int LDQ = D + 8;  // fp16 row stride of Q, K, S tiles
constexpr int LDT = C + 8;  // fp16 row stride of [*, chunk] tiles
}  // namespace mp

template <int NT>
struct PrefillSmem {
  static constexpr int DVB = 16 * NT;
  _Float16 Qs[mp::C][mp::LDQ];
  _Float16 Ks[mp::C][mp::LDQ];
  _Float16 KTs[mp::D][mp::LDT];     // K^T: [key dim][row]
  _Float16 Ss[DVB][mp::LDQ];        // state slice as fp16 operand: [value][key]
  _Float16 Xs[mp::C][mp::LDT];      // X = (I + A)^-1, lower triangular, row-major
  _Float16 Ls[mp::C][mp::LDT];      // A (off-diagonal blocks), row-major
  _Float16 Ps[mp::C][mp::LDT];      // P, row-major
  _Float16 XTd[4][16][24];          // diagonal blocks of X, transposed
  _Float16 RTs[DVB][mp::LDT];       // R'^T
  _Float16 UTs[DVB][mp::LDT];       // U^T
  _Float16 UdTs[DVB][mp::LDT];      // (diag(exp(gamma_63 - gamma)) U)^T
  float Vs[mp::C][DVB + 4];
  float Ad[4][16][17];              // diagonal blocks of A, fp32
  float gam[mp::C], bet[mp::C], eg[mp::C], egl[mp::C];
};

// Column block J of X = (I + A)^-1 below the diagonal, by the block recurrence
// X_iJ = -X_ii sum_{k=J}^{i-1} A_ik X_kJ.  Each result fragment stays in registers as the
// B operand of the next block row (16x16x16 result order equals its B-operand order).
template <int J, int NT>
__device__ __forceinline__ void offdiag_column(PrefillSmem<NT>& sm, int ln, int lg) {
  f4 xc[3];
#pragma unroll
  for (int i = J + 1; i < 4; ++i) {
    f4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = J; k < i; ++k) {
      const h4 av = *reinterpret_cast<const h4*>(&sm.Ls[16 * i + ln][16 * k + 4 * lg]);
      const h4 bv = (k == J) ? *reinterpret_cast<const h4*>(&sm.XTd[J][ln][4 * lg]) : to_h4(xc[k - J - 1]);
      z = mfma_16x16x16(av, bv, z);
    }
    const h4 xii = *reinterpret_cast<const h4*>(&sm.Xs[16 * i + ln][16 * i + 4 * lg]);
    const f4 zero = {0.f, 0.f, 0.f, 0.f};
    f4 xij = mfma_16x16x16(xii, to_h4(z), zero);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      xij[e] = -xij[e];
      sm.Xs[16 * i + 4 * lg + e][16 * J + ln] = (_Float16)xij[e];
    }
    xc[i - J - 1] = xij;
  }
}

template <int IN_DT, int O_DT, int NT>
__global__ __launch_bounds__(256) void prefill_mfma_kernel(PrefillArgs a) {
  using namespace mp;
  constexpr int DVB = 16 * NT;
  constexpr int NB = D / DVB;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  PrefillSmem<NT>& sm = *reinterpret_cast<PrefillSmem<NT>*>(smem_raw);

  // Workgroups sharing a key group (same q/k rows) are numbered consecutively in `lid`;
  // the hardware deals block ids round-robin over the 8 XCDs, so spread lid across XCDs
  // in contiguous runs to keep those workgroups on one L2.
  const unsigned nblk = gridDim.x;
  unsigned lid = blockIdx.x;
  if ((nblk & 7u) == 0) lid = (blockIdx.x & 7u) * (nblk >> 3) + (blockIdx.x >> 3);
  const int blk = lid % NB;
  const int h = (lid / NB) % a.hv;
  const int n = lid / (NB * a.hv);
  const int kh = h / (a.hv / a.hk);
  const int dv0 = blk * DVB;

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int l = tid & 63;
  const int ln = l & 15;  // fragment column / A-row index
  const int lg = l >> 4;  // fragment k-group

  const int64_t start = cu_at(a.cu, n, a.total);
  int64_t end = cu_at(a.cu, n + 1, a.total);
  if (end < start) end = start;
  const int64_t sbase = ((int64_t)n * a.hv + h) * (D * D);

  // ---- zero the triangular operands once (their upper blocks are never written)
  for (int idx = tid; idx < C * LDT; idx += 256) {
    (&sm.Xs[0][0])[idx] = (_Float16)0.f;
    (&sm.Ls[0][0])[idx] = (_Float16)0.f;
    (&sm.Ps[0][0])[idx] = (_Float16)0.f;
  }

  // ---- state slice: wave w owns key tiles 2w, 2w+1 for all NT value tiles (S^T fragments)
  f4 sacc[2][NT];
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int vt = 0; vt < NT; ++vt) {
      const int dk = 16 * (2 * w + kt) + 4 * lg;
      const int dv = 16 * vt + ln;
      f4 v = {0.f, 0.f, 0.f, 0.f};
      if (a.s0) {
        const float4 t = *reinterpret_cast<const float4*>(a.s0 + sbase + (int64_t)(dv0 + dv) * D + dk);
        v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
      }
      sacc[kt][vt] = v;
      *reinterpret_cast<h4*>(&sm.Ss[dv][dk]) = to_h4(v);
    }

  // ---- chunk loader: Q/K rows in pairs (2 tasks per thread), V slice, g/beta
  uint4 pq[2][2], pk[2][2], pv[NT > 2 ? 2 : 1];
  float pg = 0.f, pb = 0.f;
  auto fetch = [&](int64_t c0) {
    const int L = (int)((end - c0) < C ? (end - c0) : C);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int id = j * 256 + tid;
      const int tp = id >> 4, dg = id & 15;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int r = 2 * tp + u;
        const int64_t off = (c0 + r) * a.qk_stride + (int64_t)kh * D + 8 * dg;
        if (r < L) {
          if constexpr (IN_DT == DT_BF16) {
            pq[j][u] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.q) + off);
            pk[j][u] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.k) + off);
          }
        } else {
          pq[j][u] = make_uint4(0, 0, 0, 0);
          pk[j][u] = make_uint4(0, 0, 0, 0);
        }
      }
    }
    constexpr int VG = DVB / 8;  // 16-byte groups per value row
#pragma unroll
    for (int j = 0; j < (NT > 2 ? 2 : 1); ++j) {
      const int id = j * 256 + tid;
      const int r = id / VG, cg = id % VG;
      if (r < C && r < L)
        pv[j] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.v) + (c0 + r) * a.v_stride +
                                                (int64_t)h * D + dv0 + 8 * cg);
      else
        pv[j] = make_uint4(0, 0, 0, 0);
    }
    if (tid < 64) {
      pg = tid < L ? a.g[(c0 + tid) * a.hv + h] : 0.f;
      pb = tid < L ? a.beta[(c0 + tid) * a.hv + h] : 0.f;
    }
  };
  auto bf16x8_to_h8 = [](uint4 u) {
    h8 r;
    const uint32_t wv[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      r[2 * i] = (_Float16)__uint_as_float(wv[i] << 16);
      r[2 * i + 1] = (_Float16)__uint_as_float(wv[i] & 0xffff0000u);
    }
    return r;
  };

  if (start < end) fetch(start);

  for (int64_t c0 = start; c0 < end; c0 += C) {
    const int L = (int)((end - c0) < C ? (end - c0) : C);
    // ---------------- stage the prefetched chunk into LDS
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int id = j * 256 + tid;
      const int tp = id >> 4, dg = id & 15;
      const h8 q0 = bf16x8_to_h8(pq[j][0]), q1 = bf16x8_to_h8(pq[j][1]);
      const h8 k0 = bf16x8_to_h8(pk[j][0]), k1 = bf16x8_to_h8(pk[j][1]);
      *reinterpret_cast<h8*>(&sm.Qs[2 * tp][8 * dg]) = q0;
      *reinterpret_cast<h8*>(&sm.Qs[2 * tp + 1][8 * dg]) = q1;
      *reinterpret_cast<h8*>(&sm.Ks[2 * tp][8 * dg]) = k0;
      *reinterpret_cast<h8*>(&sm.Ks[2 * tp + 1][8 * dg]) = k1;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        typedef _Float16 h2 __attribute__((ext_vector_type(2)));
        h2 pr;
        pr[0] = k0[e];
        pr[1] = k1[e];
        *reinterpret_cast<h2*>(&sm.KTs[8 * dg + e][2 * tp]) = pr;
      }
    }
    {
      constexpr int VG = DVB / 8;
#pragma unroll
      for (int j = 0; j < (NT > 2 ? 2 : 1); ++j) {
        const int id = j * 256 + tid;
        const int r = id / VG, cg = id % VG;
        if (r < C) {
          const uint32_t wv[4] = {pv[j].x, pv[j].y, pv[j].z, pv[j].w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            sm.Vs[r][8 * cg + 2 * i] = __uint_as_float(wv[i] << 16);
            sm.Vs[r][8 * cg + 2 * i + 1] = __uint_as_float(wv[i] & 0xffff0000u);
          }
        }
      }
    }
    if (tid < 64) {
      float gv = pg;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float t = __shfl_up(gv, off, 64);
        if (tid >= off) gv += t;
      }
      sm.gam[tid] = gv;
      sm.bet[tid] = pb;
      sm.eg[tid] = __expf(gv);
      sm.egl[tid] = __expf(__shfl(gv, 63, 64) - gv);
    }
    if (c0 + C < end) fetch(c0 + C);  // next chunk's loads fly during this chunk
    __syncthreads();

    // ---------------- Gram tiles: A (from K K^T) and P (from Q K^T), lower blocks only
#pragma unroll
    for (int ti = 0; ti < 5; ++ti) {
      const int tix = w + 4 * ti;  // 0..19: 10 K K^T tiles then 10 Q K^T tiles
      const bool isq = tix >= 10;
      int rem = isq ? tix - 10 : tix;
      int bi = 0;
      while (rem > bi) { rem -= bi + 1; ++bi; }
      const int bj = rem;
      const _Float16 (*Arow)[LDQ] = isq ? sm.Qs : sm.Ks;
      f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const h8 av = *reinterpret_cast<const h8*>(&Arow[16 * bi + ln][32 * ks + 8 * lg]);
        const h8 bv = *reinterpret_cast<const h8*>(&sm.Ks[16 * bj + ln][32 * ks + 8 * lg]);
        acc = mfma_16x16x32(av, bv, acc);
      }
      const int s = 16 * bj + ln;
      const float gs = sm.gam[s];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * bi + 4 * lg + i;
        const float dec = s <= r ? __expf(sm.gam[r] - gs) : 0.f;
        if (isq) {
          sm.Ps[r][s] = (_Float16)(s <= r ? dec * acc[i] : 0.f);
        } else if (bi != bj) {
          sm.Ls[r][s] = (_Float16)(sm.bet[r] * dec * acc[i]);
        } else {
          sm.Ad[bi][r - 16 * bi][ln] = s < r ? sm.bet[r] * dec * acc[i] : 0.f;
        }
      }
    }

    // ---------------- Q S^T and K S^T for row tile w; R' = beta (V - exp(gamma) K S^T)
    f4 qsv[NT];
#pragma unroll
    for (int vt = 0; vt < NT; ++vt) {
      f4 aq = {0.f, 0.f, 0.f, 0.f}, ak = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const h8 bv = *reinterpret_cast<const h8*>(&sm.Ss[16 * vt + ln][32 * ks + 8 * lg]);
        const h8 q = *reinterpret_cast<const h8*>(&sm.Qs[16 * w + ln][32 * ks + 8 * lg]);
        const h8 k = *reinterpret_cast<const h8*>(&sm.Ks[16 * w + ln][32 * ks + 8 * lg]);
        aq = mfma_16x16x32(q, bv, aq);
        ak = mfma_16x16x32(k, bv, ak);
      }
      qsv[vt] = aq;
      f4 rp;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * w + 4 * lg + i;
        rp[i] = sm.bet[r] * (sm.Vs[r][16 * vt + ln] - sm.eg[r] * ak[i]);
      }
      *reinterpret_cast<h4*>(&sm.RTs[16 * vt + ln][16 * w + 4 * lg]) = to_h4(rp);
    }
    __syncthreads();

    // ---------------- diagonal blocks of X by forward substitution (wave 0, fp32)
    if (w == 0) {
      const int bb = lg, col = ln;
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float acc = r == col ? 1.f : 0.f;
#pragma unroll
        for (int s = 0; s < r; ++s) acc = fmaf(-sm.Ad[bb][r][s], x[s], acc);
        x[r] = acc;
        sm.Xs[16 * bb + r][16 * bb + col] = (_Float16)acc;
      }
      h8 lo, hi;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        lo[e] = (_Float16)x[e];
        hi[e] = (_Float16)x[8 + e];
      }
      *reinterpret_cast<h8*>(&sm.XTd[bb][col][0]) = lo;
      *reinterpret_cast<h8*>(&sm.XTd[bb][col][8]) = hi;
    }
    __syncthreads();

    // ---------------- off-diagonal blocks: X_ij = -X_ii sum_{k=j}^{i-1} A_ik X_kj (wave j)
    if (w == 0) offdiag_column<0>(sm, ln, lg);
    else if (w == 1) offdiag_column<1>(sm, ln, lg);
    else if (w == 2) offdiag_column<2>(sm, ln, lg);
    __syncthreads();

    // ---------------- U = X R' for row tile w
#pragma unroll
    for (int vt = 0; vt < NT; ++vt) {
      f4 u = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        if (ks == 1 && w < 2) continue;
        const h8 av = *reinterpret_cast<const h8*>(&sm.Xs[16 * w + ln][32 * ks + 8 * lg]);
        const h8 bv = *reinterpret_cast<const h8*>(&sm.RTs[16 * vt + ln][32 * ks + 8 * lg]);
        u = mfma_16x16x32(av, bv, u);
      }
      f4 ud;
#pragma unroll
      for (int i = 0; i < 4; ++i) ud[i] = u[i] * sm.egl[16 * w + 4 * lg + i];
      *reinterpret_cast<h4*>(&sm.UTs[16 * vt + ln][16 * w + 4 * lg]) = to_h4(u);
      *reinterpret_cast<h4*>(&sm.UdTs[16 * vt + ln][16 * w + 4 * lg]) = to_h4(ud);
    }
    __syncthreads();

    // ---------------- O = diag(exp gamma) Q S^T + P U for row tile w
#pragma unroll
    for (int vt = 0; vt < NT; ++vt) {
      f4 o = qsv[vt];
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] *= sm.eg[16 * w + 4 * lg + i];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        if (ks == 1 && w < 2) continue;
        const h8 av = *reinterpret_cast<const h8*>(&sm.Ps[16 * w + ln][32 * ks + 8 * lg]);
        const h8 bv = *reinterpret_cast<const h8*>(&sm.UTs[16 * vt + ln][32 * ks + 8 * lg]);
        o = mfma_16x16x32(av, bv, o);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * w + 4 * lg + i;
        if (r < L)
          store1<O_DT>(a.o, ((c0 + r) * a.hv + h) * (int64_t)D + dv0 + 16 * vt + ln, a.scale * o[i]);
      }
    }

    // ---------------- state: S^T <- exp(gamma_63) S^T + K^T (diag(exp(gamma_63 - gamma)) U)
    {
      const float dec = sm.eg[C - 1];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int vt = 0; vt < NT; ++vt) {
          f4 s = sacc[kt][vt];
#pragma unroll
          for (int i = 0; i < 4; ++i) s[i] *= dec;
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            const h8 av = *reinterpret_cast<const h8*>(&sm.KTs[16 * (2 * w + kt) + ln][32 * ks + 8 * lg]);
            const h8 bv = *reinterpret_cast<const h8*>(&sm.UdTs[16 * vt + ln][32 * ks + 8 * lg]);
            s = mfma_16x16x32(av, bv, s);
          }
          sacc[kt][vt] = s;
          *reinterpret_cast<h4*>(&sm.Ss[16 * vt + ln][16 * (2 * w + kt) + 4 * lg]) = to_h4(s);
        }
    }
    __syncthreads();
  }

  if (a.s1) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int vt = 0; vt < NT; ++vt) {
        const int dk = 16 * (2 * w + kt) + 4 * lg;
        const int dv = 16 * vt + ln;
        const f4 v = sacc[kt][vt];
        *reinterpret_cast<float4*>(a.s1 + sbase + (int64_t)(dv0 + dv) * D + dk) = make_float4(v[0], v[1], v[2], v[3]);
      }
  }
}

template <int O_DT, int NT>
static hipError_t launch_nt_o(const PrefillArgs& a, hipStream_t st) {
  const int64_t nblk = (int64_t)a.num_seqs * a.hv * (mp::D / (16 * NT));
  if (nblk == 0) return hipSuccess;
  const size_t smem = sizeof(PrefillSmem<NT>);
  auto k = prefill_mfma_kernel<DT_BF16, O_DT, NT>;
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(k, dim3((unsigned)nblk), dim3(256), smem, st, a);
  return hipGetLastError();
}

template <int NT>
static hipError_t launch_nt(const PrefillArgs& a, hipStream_t st) {
  return a.o_dtype == DT_BF16 ? launch_nt_o<DT_BF16, NT>(a, st) : launch_nt_o<DT_F32, NT>(a, st);
}

size_t prefill_mfma_workspace(int, int64_t, int, int) { return 0; }

hipError_t launch_prefill_mfma(const PrefillArgs& a, hipStream_t st) { return launch_nt<2>(a, st); }

}  // namespace agnes
