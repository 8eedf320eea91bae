// Chunked prefill of the gated delta rule on gfx950 matrix cores (discosf article "Agnes 3.0
// Flash 刚上线就刷屏…", section 二.1: chunked prefill with chunk 64; model card
// "Agnes-3.0-Flash Preview", 架构 table: fp32 recurrent state).
//
// Chunk algebra (exact re-association of the token recurrence; WY/UT form of Yang et al.,
// "Parallelizing Linear Transformers with the Delta Rule over Sequence Length", NeurIPS 2024,
// with the gate of Gated Delta Networks, ICLR 2025).  Rows r = 0..63 of a chunk,
// gamma_r = g_0 + ... + g_r, S the state entering the chunk ([value][key]):
//   A  = strict_lower(beta_r exp(gamma_r - gamma_s) k_r.k_s)
//   R' = diag(beta) (V - diag(exp gamma) K S^T),   (I + A) U = R'
//   O  = diag(exp gamma) Q S^T + P U,  P = lower_incl(exp(gamma_r - gamma_s) q_r.k_s)
//   S <- exp(gamma_63) S + (diag(exp(gamma_63 - gamma)) U)^T K
// Rows past the end of a partial chunk are zero with beta = g = 0 and contribute nothing.
// (I + A) U = R' is solved by block forward substitution over four 16-row blocks,
//   U_i = X_ii (R'_i - sum_{k<i} A_ik U_k),  X_ii = (I + A_ii)^-1.
//
// Mapping to the hardware.  One workgroup of 4 waves per (sequence, value head, block of 32
// value rows); the value rows of S are independent, so each workgroup scans its own
// [32 x 128] fp32 slice of the state.
//  * Waves 0 and 1 (consumers) own one 16-wide value tile each.  Their state slice lives in
//    matrix-core accumulators for the whole sequence.  Per chunk they run the state-dependent
//    products Q S^T, K S^T, the block substitution for U, P U and the state update, all on
//    v_mfma_f32_16x16x32_f16 / 16x16x16_f16 with fp32 accumulation.  A 16x16 result fragment
//    is reused as the next product's operand without leaving registers: the contraction
//    index of a 16x16x32 product may be permuted as long as both operands use the same
//    permutation, so two result fragments side by side form a B operand and the matching A
//    operand is read from LDS as two 8-byte pieces.  Consumers never write LDS.
//  * Wave 2 (key producer) stages K and K^T of the next chunk, builds the Gram K K^T, the
//    scaled blocks -A_ik and the fp32 inverses of the diagonal blocks (forward substitution).
//  * Wave 3 (query producer) stages Q, the V slice and the gates of the next chunk and builds
//    P from Q K^T.
//  Producers work one chunk ahead in double-buffered LDS, with their global loads (rows and
//  gates) issued one further chunk ahead, so each chunk costs one workgroup barrier.  Each
//  role runs its own loop (same barrier count), so registers are allocated per role.
//  * bf16 inputs widen exactly to fp16 (normal range); fp32 intermediates (S, R', U, P, A,
//    X) are rounded to fp16 once per use (2^-11 relative); the state itself stays fp32.
#include "common.h"
#include "launch.h"

namespace agnes {

namespace mp {
constexpr int C = 64;        // chunk
constexpr int D = 128;       // head dim (key and value)
constexpr int LDQ = D + 8;   // fp16 row stride of Q/K rows
constexpr int LDT = C + 8;   // fp16 row stride of [*, chunk] tiles
constexpr int LDB = 16 + 8;  // fp16 row stride of 16x16 blocks
constexpr int NCW = 2;       // consumer waves, one 16-wide value tile each
constexpr int DVB = 16 * NCW;
constexpr int NB = D / DVB;  // workgroups per value head
}  // namespace mp

struct PrefillSmem {
  _Float16 Qs[2][mp::C][mp::LDQ];
  _Float16 Ks[2][mp::C][mp::LDQ];
  _Float16 KTs[2][mp::D][mp::LDT];    // K^T: [key dim][row]
  _Float16 Ps[2][mp::C][mp::LDT];     // P, row-major, zero above the diagonal
  _Float16 Ln[2][6][16][mp::LDB];     // -A_ik (i > k), row-major blocks
  _Float16 Xd[2][4][16][mp::LDB];     // (I + A_ii)^-1, row-major blocks
  uint16_t Vs[2][mp::C][mp::DVB + 8];  // V slice (bf16 as stored)
  float gam[2][mp::C], bet[2][mp::C], eg[2][mp::C], egl[2][mp::C];
  float Ad[4][16][17];                // key producer: A_ii in fp32
  float pgam[mp::C], pbet[mp::C];     // key producer: its copy of the gates
};

__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

__device__ __forceinline__ h8 cvt8(uint4 u) {
  h8 r;
  const uint32_t wv[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r[2 * i] = (_Float16)__uint_as_float(wv[i] << 16);
    r[2 * i + 1] = (_Float16)__uint_as_float(wv[i] & 0xffff0000u);
  }
  return r;
}

__device__ __forceinline__ h8 cat(h4 a, h4 b) {
  h8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
  r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
  return r;
}

// A operand of a 16x16x32 product whose B operand is two result fragments side by side:
// columns k0+4g..k0+4g+3 and k0+16+4g..k0+16+4g+3 of a row-major fp16 row.
__device__ __forceinline__ h8 a_perm(const _Float16* row, int k0, int lg) {
  return cat(*reinterpret_cast<const h4*>(row + k0 + 4 * lg), *reinterpret_cast<const h4*>(row + k0 + 16 + 4 * lg));
}

__device__ __forceinline__ h8 b_pair(f4 lo, f4 hi) { return cat(to_h4(lo), to_h4(hi)); }

__host__ __device__ constexpr int lblk(int i, int k) { return i * (i - 1) / 2 + k; }

// 64 rows x 128 columns of bf16 as 16 fragments per lane: [tile][kstep] = row 16*tile + (l%16),
// columns 32*kstep + 8*(l/16) .. +7.  Rows >= L read as zero.
__device__ __forceinline__ void load_rows(uint4 (&r)[4][4], const uint16_t* base, int64_t c0, int L,
                                          int64_t stride, int ln, int lg) {
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int row = 16 * t + ln;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      r[t][ks] = row < L ? *reinterpret_cast<const uint4*>(base + (c0 + row) * stride + 32 * ks + 8 * lg)
                         : make_uint4(0, 0, 0, 0);
  }
}

// Per-workgroup constants shared by the three roles.
struct Geo {
  int64_t start, end;
  int nchunks, h, kh, dv0, w, lane, ln, lg;
  int64_t sbase;
  __device__ int len(int c) const {
    const int64_t r = end - start - (int64_t)c * mp::C;
    return (int)(r < mp::C ? r : mp::C);
  }
};

// Key producer: stage K / K^T of chunk c (prefetched in rk, gk/bk) into buffer pb, prefetch
// chunk c+1, then build -A_ik (i > k) and X_ii = (I + A_ii)^-1.
__device__ __forceinline__ void produce_k(PrefillSmem& sm, const PrefillArgs& a, const Geo& G,
                                          const uint16_t* kbase, int c, int pb, uint4 (&rk)[4][4],
                                          float& gk, float& bk) {
  using namespace mp;
  const int ln = G.ln, lg = G.lg, lane = G.lane;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const h8 f = cvt8(rk[t][ks]);
      *reinterpret_cast<h8*>(&sm.Ks[pb][16 * t + ln][32 * ks + 8 * lg]) = f;
#pragma unroll
      for (int e = 0; e < 8; ++e) sm.KTs[pb][32 * ks + 8 * lg + e][16 * t + ln] = f[e];
    }
  float gv = gk;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float t = __shfl_up(gv, off, 64);
    if (lane >= off) gv += t;
  }
  sm.pgam[lane] = gv;
  sm.pbet[lane] = bk;
  if (c + 1 < G.nchunks) {  // prefetch chunk c+1
    const int64_t c1 = G.start + (int64_t)(c + 1) * C;
    const int L1 = G.len(c + 1);
    load_rows(rk, kbase, c1, L1, a.qk_stride, ln, lg);
    gk = lane < L1 ? a.g[(c1 + lane) * a.hv + G.h] : 0.f;
    bk = lane < L1 ? a.beta[(c1 + lane) * a.hv + G.h] : 0.f;
  }
  wave_lds_fence();
  // diagonal blocks of A (fp32) for the substitution
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const h8 kf = *reinterpret_cast<const h8*>(&sm.Ks[pb][16 * b + ln][32 * ks + 8 * lg]);
      acc = mfma_16x16x32(kf, kf, acc);
    }
    const int s = 16 * b + ln;
    const float gs = sm.pgam[s];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * b + 4 * lg + i;
      sm.Ad[b][4 * lg + i][ln] = s < r ? sm.pbet[r] * __expf(sm.pgam[r] - gs) * acc[i] : 0.f;
    }
  }
  // off-diagonal blocks, computed transposed so each lane holds an A-operand row fragment
#pragma unroll
  for (int i = 1; i < 4; ++i) {
    h8 ki[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) ki[ks] = *reinterpret_cast<const h8*>(&sm.Ks[pb][16 * i + ln][32 * ks + 8 * lg]);
    const int r = 16 * i + ln;
    const float gr = sm.pgam[r], br = sm.pbet[r];
#pragma unroll
    for (int k = 0; k < i; ++k) {
      f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        acc = mfma_16x16x32(*reinterpret_cast<const h8*>(&sm.Ks[pb][16 * k + ln][32 * ks + 8 * lg]), ki[ks], acc);
      f4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = -br * __expf(gr - sm.pgam[16 * k + 4 * lg + e]) * acc[e];
      *reinterpret_cast<h4*>(&sm.Ln[pb][lblk(i, k)][ln][4 * lg]) = to_h4(v);
    }
  }
  wave_lds_fence();
  // X_ii = (I + A_ii)^-1, one column per lane (block lg, column ln), right-looking
  float x[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) x[r] = r == ln ? 1.f : 0.f;
#pragma unroll
  for (int s2 = 0; s2 < 16; ++s2)
#pragma unroll
    for (int r = s2 + 1; r < 16; ++r) x[r] = fmaf(-sm.Ad[lg][r][s2], x[s2], x[r]);
#pragma unroll
  for (int r = 0; r < 16; ++r) sm.Xd[pb][lg][r][ln] = (_Float16)x[r];
}

// Query producer: stage Q, V and the gates of chunk c into buffer pb, prefetch chunk c+1,
// then build P = lower_incl(exp(gamma_r - gamma_s) q_r.k_s).
__device__ __forceinline__ void produce_q(PrefillSmem& sm, const PrefillArgs& a, const Geo& G,
                                          const uint16_t* qbase, const uint16_t* kbase, const uint16_t* vrow,
                                          int c, int pb, uint4 (&rq)[4][4], uint4 (&rk)[4][4], uint4 (&rv)[4],
                                          float& gq, float& bq) {
  using namespace mp;
  const int ln = G.ln, lg = G.lg, lane = G.lane;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      *reinterpret_cast<h8*>(&sm.Qs[pb][16 * t + ln][32 * ks + 8 * lg]) = cvt8(rq[t][ks]);
#pragma unroll
  for (int j = 0; j < 4; ++j) *reinterpret_cast<uint4*>(&sm.Vs[pb][lane][8 * j]) = rv[j];
  float gv = gq;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float t = __shfl_up(gv, off, 64);
    if (lane >= off) gv += t;
  }
  sm.gam[pb][lane] = gv;
  sm.bet[pb][lane] = bq;
  sm.eg[pb][lane] = __expf(gv);
  sm.egl[pb][lane] = __expf(__shfl(gv, 63, 64) - gv);
  h8 kf[4][4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) kf[t][ks] = cvt8(rk[t][ks]);
  const bool more = c + 1 < G.nchunks;
  const int64_t c1 = G.start + (int64_t)(c + 1) * C;
  const int L1 = more ? G.len(c + 1) : 0;
  if (more) {
    load_rows(rq, qbase, c1, L1, a.qk_stride, ln, lg);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      rv[j] = lane < L1 ? *reinterpret_cast<const uint4*>(vrow + (c1 + lane) * a.v_stride + 8 * j) : make_uint4(0, 0, 0, 0);
    gq = lane < L1 ? a.g[(c1 + lane) * a.hv + G.h] : 0.f;
    bq = lane < L1 ? a.beta[(c1 + lane) * a.hv + G.h] : 0.f;
  }
  wave_lds_fence();
#pragma unroll
  for (int bi = 0; bi < 4; ++bi) {
    h8 qf[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[ks] = *reinterpret_cast<const h8*>(&sm.Qs[pb][16 * bi + ln][32 * ks + 8 * lg]);
#pragma unroll
    for (int bj = 0; bj <= bi; ++bj) {
      f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) acc = mfma_16x16x32(qf[ks], kf[bj][ks], acc);
      const int s = 16 * bj + ln;
      const float gs = sm.gam[pb][s];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * bi + 4 * lg + i;
        sm.Ps[pb][r][s] = (_Float16)(s <= r ? __expf(sm.gam[pb][r] - gs) * acc[i] : 0.f);
      }
    }
  }
  if (more) load_rows(rk, kbase, c1, L1, a.qk_stride, ln, lg);
}

// Consumer: chunk c from buffer p for value tile G.w; sacc holds S^T fragments [key tile].
template <int O_DT>
__device__ __forceinline__ void consume(PrefillSmem& sm, const PrefillArgs& a, const Geo& G, int c, int p,
                                        f4 (&sacc)[8]) {
  using namespace mp;
  const int ln = G.ln, lg = G.lg, w = G.w;
  const int64_t c0 = G.start + (int64_t)c * C;
  const int L = G.len(c);
  h8 sb[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) sb[ks] = b_pair(sacc[2 * ks], sacc[2 * ks + 1]);
  f4 qs[4], kq[4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    qs[rt] = f4{0.f, 0.f, 0.f, 0.f};
    kq[rt] = f4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      qs[rt] = mfma_16x16x32(a_perm(&sm.Qs[p][16 * rt + ln][0], 32 * ks, lg), sb[ks], qs[rt]);
      kq[rt] = mfma_16x16x32(a_perm(&sm.Ks[p][16 * rt + ln][0], 32 * ks, lg), sb[ks], kq[rt]);
    }
  // R' = beta (V - exp(gamma) K S^T), then block substitution for U
  f4 u[4];
  const f4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f4 wv;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 16 * i + 4 * lg + e;
      const float vv = bf16_to_f32(sm.Vs[p][r][16 * w + ln]);
      wv[e] = sm.bet[p][r] * (vv - sm.eg[p][r] * kq[i][e]);
    }
#pragma unroll
    for (int k = 0; k < i; ++k)
      wv = mfma_16x16x16(*reinterpret_cast<const h4*>(&sm.Ln[p][lblk(i, k)][ln][4 * lg]), to_h4(u[k]), wv);
    u[i] = mfma_16x16x16(*reinterpret_cast<const h4*>(&sm.Xd[p][i][ln][4 * lg]), to_h4(wv), zero);
  }
  // O = diag(exp gamma) Q S^T + P U
  const h8 ub0 = b_pair(u[0], u[1]), ub1 = b_pair(u[2], u[3]);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = qs[i][e] * sm.eg[p][16 * i + 4 * lg + e];
    o = mfma_16x16x32(a_perm(&sm.Ps[p][16 * i + ln][0], 0, lg), ub0, o);
    if (i >= 2) o = mfma_16x16x32(a_perm(&sm.Ps[p][16 * i + ln][0], 32, lg), ub1, o);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 16 * i + 4 * lg + e;
      if (r < L) store1<O_DT>(a.o, ((c0 + r) * a.hv + G.h) * (int64_t)D + G.dv0 + 16 * w + ln, a.scale * o[e]);
    }
  }
  // S^T <- exp(gamma_63) S^T + K^T (diag(exp(gamma_63 - gamma)) U)
  f4 ud[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) ud[i][e] = u[i][e] * sm.egl[p][16 * i + 4 * lg + e];
  const h8 db0 = b_pair(ud[0], ud[1]), db1 = b_pair(ud[2], ud[3]);
  const float dec = sm.eg[p][C - 1];
#pragma unroll
  for (int kt = 0; kt < 8; ++kt) {
    f4 s = sacc[kt];
#pragma unroll
    for (int e = 0; e < 4; ++e) s[e] *= dec;
    s = mfma_16x16x32(a_perm(&sm.KTs[p][16 * kt + ln][0], 0, lg), db0, s);
    s = mfma_16x16x32(a_perm(&sm.KTs[p][16 * kt + ln][0], 32, lg), db1, s);
    sacc[kt] = s;
  }
}

template <int O_DT>
__global__ __launch_bounds__(256) void prefill_mfma_kernel(PrefillArgs a) {
  using namespace mp;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  PrefillSmem& sm = *reinterpret_cast<PrefillSmem*>(smem_raw);

  // Workgroups sharing a key group are consecutive in `lid`; the hardware deals block ids
  // round-robin over the 8 XCDs, so give each XCD a contiguous run of lid (shared L2).
  const unsigned nblk = gridDim.x;
  unsigned lid = blockIdx.x;
  if ((nblk & 7u) == 0) lid = (blockIdx.x & 7u) * (nblk >> 3) + (blockIdx.x >> 3);
  Geo G;
  const int blk = lid % NB;
  G.h = (lid / NB) % a.hv;
  const int n = lid / (NB * a.hv);
  G.kh = G.h / (a.hv / a.hk);
  G.dv0 = blk * DVB;
  G.w = threadIdx.x >> 6;
  G.lane = threadIdx.x & 63;
  G.ln = G.lane & 15;
  G.lg = G.lane >> 4;
  G.start = cu_at(a.cu, n, a.total);
  G.end = cu_at(a.cu, n + 1, a.total);
  if (G.end < G.start) G.end = G.start;
  G.nchunks = (int)((G.end - G.start + C - 1) / C);
  G.sbase = ((int64_t)n * a.hv + G.h) * (D * D);
  const uint16_t* qbase = static_cast<const uint16_t*>(a.q) + (int64_t)G.kh * D;
  const uint16_t* kbase = static_cast<const uint16_t*>(a.k) + (int64_t)G.kh * D;
  const int ln = G.ln, lg = G.lg, lane = G.lane;

  // Every role runs its own loop with exactly one workgroup barrier per chunk after a common
  // prologue barrier, so each role's registers are allocated on their own.
  if (G.w < NCW) {
    f4 sacc[8];
#pragma unroll
    for (int kt = 0; kt < 8; ++kt) {
      f4 v = {0.f, 0.f, 0.f, 0.f};
      if (a.s0) {
        const float4 t = *reinterpret_cast<const float4*>(a.s0 + G.sbase + (int64_t)(G.dv0 + 16 * G.w + ln) * D + 16 * kt + 4 * lg);
        v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
      }
      sacc[kt] = v;
    }
    __syncthreads();
    for (int c = 0; c < G.nchunks; ++c) {
      consume<O_DT>(sm, a, G, c, c & 1, sacc);
      __syncthreads();
    }
    if (a.s1) {
#pragma unroll
      for (int kt = 0; kt < 8; ++kt) {
        const f4 v = sacc[kt];
        *reinterpret_cast<float4*>(a.s1 + G.sbase + (int64_t)(G.dv0 + 16 * G.w + ln) * D + 16 * kt + 4 * lg) =
            make_float4(v[0], v[1], v[2], v[3]);
      }
    }
  } else if (G.w == NCW) {
    uint4 rk[4][4];
    float gk = 0.f, bk = 0.f;
    if (G.nchunks > 0) {
      const int L0 = G.len(0);
      load_rows(rk, kbase, G.start, L0, a.qk_stride, ln, lg);
      gk = lane < L0 ? a.g[(G.start + lane) * a.hv + G.h] : 0.f;
      bk = lane < L0 ? a.beta[(G.start + lane) * a.hv + G.h] : 0.f;
      produce_k(sm, a, G, kbase, 0, 0, rk, gk, bk);
    }
    __syncthreads();
    for (int c = 0; c < G.nchunks; ++c) {
      if (c + 1 < G.nchunks) produce_k(sm, a, G, kbase, c + 1, (c + 1) & 1, rk, gk, bk);
      __syncthreads();
    }
  } else {
    const uint16_t* vrow = static_cast<const uint16_t*>(a.v) + (int64_t)G.h * D + G.dv0;
    uint4 rq[4][4], rk[4][4], rv[4];
    float gq = 0.f, bq = 0.f;
    for (int idx = lane; idx < 2 * C * LDT / 8; idx += 64) {
      const h8 z = {0, 0, 0, 0, 0, 0, 0, 0};
      reinterpret_cast<h8*>(&sm.Ps[0][0][0])[idx] = z;
    }
    if (G.nchunks > 0) {
      const int L0 = G.len(0);
      load_rows(rq, qbase, G.start, L0, a.qk_stride, ln, lg);
      load_rows(rk, kbase, G.start, L0, a.qk_stride, ln, lg);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        rv[j] = lane < L0 ? *reinterpret_cast<const uint4*>(vrow + (G.start + lane) * a.v_stride + 8 * j) : make_uint4(0, 0, 0, 0);
      gq = lane < L0 ? a.g[(G.start + lane) * a.hv + G.h] : 0.f;
      bq = lane < L0 ? a.beta[(G.start + lane) * a.hv + G.h] : 0.f;
      wave_lds_fence();
      produce_q(sm, a, G, qbase, kbase, vrow, 0, 0, rq, rk, rv, gq, bq);
    }
    __syncthreads();
    for (int c = 0; c < G.nchunks; ++c) {
      if (c + 1 < G.nchunks) produce_q(sm, a, G, qbase, kbase, vrow, c + 1, (c + 1) & 1, rq, rk, rv, gq, bq);
      __syncthreads();
    }
  }
}

template <int O_DT>
static hipError_t launch_o(const PrefillArgs& a, hipStream_t st) {
  const int64_t nblk = (int64_t)a.num_seqs * a.hv * mp::NB;
  if (nblk == 0) return hipSuccess;
  const size_t smem = sizeof(PrefillSmem);
  auto k = prefill_mfma_kernel<O_DT>;
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(k, dim3((unsigned)nblk), dim3(256), smem, st, a);
  return hipGetLastError();
}

size_t prefill_mfma_workspace(int, int64_t, int, int) { return 0; }

hipError_t launch_prefill_mfma(const PrefillArgs& a, hipStream_t st) {
  return a.o_dtype == DT_BF16 ? launch_o<DT_BF16>(a, st) : launch_o<DT_F32>(a, st);
}

}  // namespace agnes
