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
// Three launches on the caller's stream:
//  1. chunk_offsets: first chunk index of every sequence (prefix sum of ceil(len / 64)).
//  2. prep (all chunks in parallel, one workgroup per chunk and key group): the Gram matrices
//     K K^T and Q K^T once per key group on matrix cores, then per value head of the group the
//     decay-scaled P, the blocks -A_ik, the fp32 forward-substitution inverses X_ii and the
//     per-row gates, written as one 14 KiB record per (chunk, value head) in the workspace.
//     Everything in it depends only on the inputs, not on the state.
//  3. scan (serial over chunks): one workgroup of 4 waves per (sequence, value head, block of
//     32 value rows); the value rows of S are independent, so each workgroup scans its own
//     [32 x 128] fp32 slice of the state.  Waves 0 and 1 own one 16-wide value tile each and
//     keep their slice of S^T in matrix-core accumulators for the whole sequence; per chunk
//     they run Q S^T, K S^T, the block substitution for U, P U and the state update.  A 16x16
//     result fragment is reused as the next product's operand without leaving registers: the
//     contraction index of a 16x16x32 product may be permuted as long as both operands use
//     the same permutation, so two result fragments side by side form a B operand and the
//     matching A operand is read from LDS as two 8-byte pieces (K^T pieces come straight from
//     the row-major K tile through the gfx950 transposing LDS read).  Waves 2 and 3 only load:
//     they stage chunk c+1 (Q, K; the record and the V slice) into double-buffered LDS while
//     waves 0 and 1 work on chunk c, with their global loads issued a further chunk ahead,
//     so each chunk costs one workgroup barrier.  Each role runs its own loop with the same
//     barrier count, so registers are allocated per role.
// Number formats: bf16 inputs widen exactly to fp16 (normal range); fp32 intermediates
// (S, R', U, P, A, X) are rounded to fp16 once per use (2^-11 relative); every product
// accumulates in fp32 and the state itself stays fp32.
#include "common.h"
#include "launch.h"

namespace agnes {

namespace mp {
constexpr int C = 64;        // chunk
constexpr int D = 128;       // head dim (key and value)
constexpr int LDQ = D + 8;   // fp16 row stride of staged Q/K rows
constexpr int LDT = C + 8;   // fp16 row stride of [*, chunk] tiles
constexpr int LDB = 16 + 8;  // fp16 row stride of 16x16 blocks
constexpr int NCW = 2;       // consumer waves, one 16-wide value tile each
constexpr int DVB = 16 * NCW;
constexpr int NB = D / DVB;  // scan workgroups per value head
constexpr int LDV = DVB + 8; // bf16 row stride of the staged V slice
}  // namespace mp

// Per (chunk, value head) record written by prep and copied verbatim into LDS by scan, so it
// is laid out as the padded LDS image the consumers read (rows padded against bank conflicts).
struct RecImage {
  _Float16 P[mp::C][mp::LDT];      // P, row-major, zero above the diagonal
  _Float16 Ln[6][16][mp::LDB];     // -A_ik (i > k), row-major blocks
  _Float16 Xd[4][16][mp::LDB];     // X_ii = (I + A_ii)^-1, row-major blocks
  float gt[3][mp::C];              // beta, exp(gamma), exp(gamma_63 - gamma)
  float pad[192];                  // to a whole number of 1 KiB copy steps
};
static_assert(sizeof(RecImage) == 18 * 1024, "record image is copied in 1 KiB steps");
namespace mp {
constexpr int REC_BYTES = sizeof(RecImage);
constexpr int REC_P = offsetof(RecImage, P);
constexpr int REC_L = offsetof(RecImage, Ln);
constexpr int REC_X = offsetof(RecImage, Xd);
constexpr int REC_G = offsetof(RecImage, gt);
}  // namespace mp

__host__ __device__ constexpr int lblk(int i, int k) { return i * (i - 1) / 2 + k; }

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
static inline int64_t max_chunks(int64_t total, int num_seqs) { return (total + mp::C - 1) / mp::C + num_seqs; }

// ---------------------------------------------------------------- helpers
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

typedef short s4v __attribute__((ext_vector_type(4)));
typedef uint32_t u4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s4v lds_s4v;

// Transposing LDS read (ds_read_b64_tr_b16): within each 16-lane group, lane i supplies four
// consecutive fp16 values D[i][0..3]; lane 4a+b receives D[a+4e][b], e = 0..3.  With lane
// 16g+i pointing at row (t0 + 4g + i/4), column (c0 + 4(i%4)) of a row-major tile, lane l
// receives tile[t0 + 4g + e][c0 + l%16]: a 16x16x16 A-operand fragment of the transpose.
__device__ __forceinline__ h4 lds_tr4(const _Float16* p) {
  const s4v v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4v*)(p));
  return __builtin_bit_cast(h4, v);
}

// ---------------------------------------------------------------- 1. chunk offsets
__global__ __launch_bounds__(256) void chunk_offsets_kernel(const int32_t* cu, int num_seqs, int64_t total,
                                                            int32_t* off) {
  __shared__ int32_t part[256];
  const int t = threadIdx.x;
  const int per = (num_seqs + 255) / 256;
  const int lo = t * per < num_seqs ? t * per : num_seqs;
  const int hi = lo + per < num_seqs ? lo + per : num_seqs;
  int32_t sum = 0;
  for (int n = lo; n < hi; ++n) {
    const int64_t s = cu_at(cu, n, total), e = cu_at(cu, n + 1, total);
    sum += e > s ? (int32_t)((e - s + mp::C - 1) / mp::C) : 0;
  }
  part[t] = sum;
  __syncthreads();
  if (t == 0) {
    int32_t run = 0;
    for (int i = 0; i < 256; ++i) {
      const int32_t v = part[i];
      part[i] = run;
      run += v;
    }
  }
  __syncthreads();
  int32_t run = part[t];
  for (int n = lo; n < hi; ++n) {
    off[n] = run;
    const int64_t s = cu_at(cu, n, total), e = cu_at(cu, n + 1, total);
    run += e > s ? (int32_t)((e - s + mp::C - 1) / mp::C) : 0;
  }
  if (hi == num_seqs && lo < hi) off[num_seqs] = run;
  if (num_seqs == 0 && t == 0) off[0] = 0;
}

// Sequence holding global chunk j (largest n with off[n] <= j).
__device__ __forceinline__ int seq_of_chunk(const int32_t* off, int num_seqs, int j) {
  int lo = 0, hi = num_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (off[mid] <= j) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// ---------------------------------------------------------------- 2. prep
struct PrepSmem {
  _Float16 Qs[mp::C][mp::LDQ];
  _Float16 Ks[mp::C][mp::LDQ];
  float Gk[mp::C][mp::C + 1];   // K K^T (lower blocks)
  float Gq[mp::C][mp::C + 1];   // Q K^T (lower blocks)
  float gam[mp::C], bet[mp::C];
  float Ad[4][16][17];          // A_ii, fp32
  _Float16 Xs[4][16][16];       // X_ii staged for a coalesced copy
};

__global__ __launch_bounds__(256) void prep_kernel(PrefillArgs a, int64_t maxch) {
  using namespace mp;
  __shared__ PrepSmem sm;
  const int32_t* off = static_cast<const int32_t*>(a.workspace);
  unsigned char* recs = static_cast<unsigned char*>(a.workspace) + align256(4 * (size_t)(a.num_seqs + 1));
  const int j = blockIdx.x;
  const int kh = blockIdx.y;
  if (j >= off[a.num_seqs]) return;
  const int n = seq_of_chunk(off, a.num_seqs, j);
  const int64_t start = cu_at(a.cu, n, a.total);
  const int64_t c0 = start + (int64_t)(j - off[n]) * C;
  int64_t end = cu_at(a.cu, n + 1, a.total);
  const int L = (int)((end - c0) < C ? (end - c0) : C);
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, ln = lane & 15, lg = lane >> 4;

  // ---- Q, K rows of the key group -> fp16 LDS
  const uint16_t* qb = static_cast<const uint16_t*>(a.q) + (int64_t)kh * D;
  const uint16_t* kb = static_cast<const uint16_t*>(a.k) + (int64_t)kh * D;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int task = tid + 256 * i;
    const int r = task >> 4, sg = task & 15;
    const int64_t rr = r < L ? r : 0;
    const uint4 qv = *reinterpret_cast<const uint4*>(qb + (c0 + rr) * a.qk_stride + 8 * sg);
    const uint4 kv = *reinterpret_cast<const uint4*>(kb + (c0 + rr) * a.qk_stride + 8 * sg);
    const uint4 z = make_uint4(0, 0, 0, 0);
    *reinterpret_cast<h8*>(&sm.Qs[r][8 * sg]) = cvt8(r < L ? qv : z);
    *reinterpret_cast<h8*>(&sm.Ks[r][8 * sg]) = cvt8(r < L ? kv : z);
  }
  __syncthreads();

  // ---- Gram tiles (lower blocks): 10 of K K^T, 10 of Q K^T, five per wave
#pragma unroll
  for (int ti = 0; ti < 5; ++ti) {
    const int tix = w + 4 * ti;
    const bool isq = tix >= 10;
    int rem = isq ? tix - 10 : tix, bi = 0;
    while (rem > bi) { rem -= bi + 1; ++bi; }
    const int bj = rem;
    const _Float16 (*Arow)[LDQ] = isq ? sm.Qs : sm.Ks;
    f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      acc = mfma_16x16x32(*reinterpret_cast<const h8*>(&Arow[16 * bi + ln][32 * ks + 8 * lg]),
                          *reinterpret_cast<const h8*>(&sm.Ks[16 * bj + ln][32 * ks + 8 * lg]), acc);
    float (*G)[C + 1] = isq ? sm.Gq : sm.Gk;
#pragma unroll
    for (int i = 0; i < 4; ++i) G[16 * bi + 4 * lg + i][16 * bj + ln] = acc[i];
  }
  __syncthreads();

  const int grp = a.hv / a.hk;
  for (int hh = 0; hh < grp; ++hh) {
    const int h = kh * grp + hh;
    unsigned char* rec = recs + ((size_t)h * (size_t)maxch + (size_t)j) * REC_BYTES;
    if (w == 0) {  // gates: inclusive prefix sum of log-decays; rows >= L get g = beta = 0
      float gv = lane < L ? a.g[(c0 + lane) * a.hv + h] : 0.f;
      const float bv = lane < L ? a.beta[(c0 + lane) * a.hv + h] : 0.f;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const float t = __shfl_up(gv, o, 64);
        if (lane >= o) gv += t;
      }
      sm.gam[lane] = gv;
      sm.bet[lane] = bv;
      float* gr = reinterpret_cast<float*>(rec + REC_G);
      gr[lane] = bv;
      gr[64 + lane] = __expf(gv);
      gr[128 + lane] = __expf(__shfl(gv, 63, 64) - gv);
    }
    __syncthreads();
    {  // P row r, columns s0..s0+15; A for the same positions
      const int r = tid >> 2, s0 = 16 * (tid & 3);
      const int bi = r >> 4, bs = s0 >> 4;
      const float gr = sm.gam[r], br = sm.bet[r];
      h8 p0, p1, l0, l1;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int s = s0 + e;
        const float d = s <= r ? __expf(gr - sm.gam[s]) : 0.f;
        const float pv = s <= r ? d * sm.Gq[r][s] : 0.f;
        const float av = s < r ? br * d * sm.Gk[r][s] : 0.f;
        if (e < 8) { p0[e] = (_Float16)pv; l0[e] = (_Float16)(-av); }
        else { p1[e - 8] = (_Float16)pv; l1[e - 8] = (_Float16)(-av); }
        if (bs == bi) sm.Ad[bi][r & 15][e] = av;
      }
      h8* pp = reinterpret_cast<h8*>(rec + REC_P + (r * LDT + s0) * 2);
      pp[0] = p0;
      pp[1] = p1;
      if (bs < bi) {
        h8* lp = reinterpret_cast<h8*>(rec + REC_L + ((lblk(bi, bs) * 16 + (r & 15)) * LDB) * 2);
        lp[0] = l0;
        lp[1] = l1;
      }
    }
    __syncthreads();
    if (w == 0) {  // X_ii = (I + A_ii)^-1: block lg, column ln, right-looking substitution
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) x[r] = r == ln ? 1.f : 0.f;
#pragma unroll
      for (int s = 0; s < 16; ++s)
#pragma unroll
        for (int r = s + 1; r < 16; ++r) x[r] = fmaf(-sm.Ad[lg][r][s], x[s], x[r]);
#pragma unroll
      for (int r = 0; r < 16; ++r) sm.Xs[lg][r][ln] = (_Float16)x[r];
    }
    __syncthreads();
    if (tid < 128) {  // 64 block rows of 16 fp16 (two 16-byte halves), row stride LDB
      const int q = tid >> 1, hf = tid & 1;
      *reinterpret_cast<uint4*>(rec + REC_X + (q * LDB + 8 * hf) * 2) =
          reinterpret_cast<const uint4*>(&sm.Xs[q >> 4][q & 15][0])[hf];
    }
  }
}

// ---------------------------------------------------------------- 3. scan
typedef __bf16 bf8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;

struct ScanBuf {            // one chunk, filled by direct global -> LDS copies
  uint16_t Qs[mp::C][mp::LDQ];   // bf16 q rows as stored
  uint16_t Ks[mp::C][mp::LDQ];   // bf16 k rows as stored
  RecImage R;                    // prep record of (chunk, value head)
  uint16_t Vs[mp::C][mp::LDV];   // bf16 v slice [row][value col]
};
struct ScanSmem {
  ScanBuf B[2];
  float Os[2][mp::C][mp::DVB + 4];  // output tile, written out by the output wave
};

__device__ __forceinline__ uint32_t fbits(float x) { return __float_as_uint(x); }

// Split fp32 fragment pairs into bf16 hi + lo parts: x = hi + lo with hi = x truncated to
// bf16 and lo = bf16(x - hi), 16 significant bits in all (relative error <= 2^-16).
__device__ __forceinline__ void split_pair(f4 a, f4 b, bf8& hi, bf8& lo) {
  uint32_t h[4], l[4];
  const float x[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t u0 = fbits(x[2 * i]), u1 = fbits(x[2 * i + 1]);
    const float r0 = x[2 * i] - __uint_as_float(u0 & 0xffff0000u);
    const float r1 = x[2 * i + 1] - __uint_as_float(u1 & 0xffff0000u);
    h[i] = (u0 >> 16) | (u1 & 0xffff0000u);
    l[i] = (fbits(r0) >> 16) | (fbits(r1) & 0xffff0000u);
  }
  const uint4 hv = make_uint4(h[0], h[1], h[2], h[3]), lv = make_uint4(l[0], l[1], l[2], l[3]);
  hi = __builtin_bit_cast(bf8, hv);
  lo = __builtin_bit_cast(bf8, lv);
}

__device__ __forceinline__ f4 mfma_bf(bf8 a, bf8 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// bf16 A operand matching a B operand made of two result fragments (see a_perm).
__device__ __forceinline__ bf8 a_perm_bf(const uint16_t* row, int k0, int lg) {
  const u16x4 lo = *reinterpret_cast<const u16x4*>(row + k0 + 4 * lg);
  const u16x4 hi = *reinterpret_cast<const u16x4*>(row + k0 + 16 + 4 * lg);
  const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
  return __builtin_bit_cast(bf8, make_uint4(l2.x, l2.y, h2.x, h2.y));
}

// Transposing read of 4 bf16 values (see lds_tr4) -> 64 raw bits.
__device__ __forceinline__ uint2 lds_tr4_bits(const uint16_t* p) {
  const s4v v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4v*)(p));
  return __builtin_bit_cast(uint2, v);
}

struct Geo {
  int64_t start, end;
  int nchunks, h, kh, dv0, w, lane, ln, lg;
  int64_t sbase;
  size_t rec0;  // byte offset of this sequence's first record for value head h
  __device__ int len(int c) const {
    const int64_t r = end - start - (int64_t)c * mp::C;
    return (int)(r < mp::C ? r : mp::C);
  }
};

// Consumer: chunk in buffer B for value tile G.w; sacc holds S^T fragments [key tile].
__device__ __forceinline__ void consume(const ScanBuf& B, float (*Os)[mp::DVB + 4], const PrefillArgs& a,
                                        const Geo& G, f4 (&sacc)[8]) {
  using namespace mp;
  const int ln = G.ln, lg = G.lg, w = G.w;
  const RecImage& R = B.R;
  f4 bet[4], eg[4], egl[4];
  float vv[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    bet[i] = *reinterpret_cast<const f4*>(&R.gt[0][16 * i + 4 * lg]);
    eg[i] = *reinterpret_cast<const f4*>(&R.gt[1][16 * i + 4 * lg]);
    egl[i] = *reinterpret_cast<const f4*>(&R.gt[2][16 * i + 4 * lg]);
#pragma unroll
    for (int e = 0; e < 4; ++e) vv[i][e] = bf16_to_f32(B.Vs[16 * i + 4 * lg + e][16 * w + ln]);
  }
  h4 lf[6], xf[4];
#pragma unroll
  for (int b = 0; b < 6; ++b) lf[b] = *reinterpret_cast<const h4*>(&R.Ln[b][ln][4 * lg]);
#pragma unroll
  for (int i = 0; i < 4; ++i) xf[i] = *reinterpret_cast<const h4*>(&R.Xd[i][ln][4 * lg]);

  // Q S^T and K S^T on bf16 matrix cores: q, k exact, S as hi + lo
  bf8 shi[4], slo[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) split_pair(sacc[2 * ks], sacc[2 * ks + 1], shi[ks], slo[ks]);
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
      const bf8 qa = a_perm_bf(&B.Qs[16 * rt + ln][0], 32 * ks, lg);
      const bf8 ka = a_perm_bf(&B.Ks[16 * rt + ln][0], 32 * ks, lg);
      qs[rt] = mfma_bf(qa, shi[ks], qs[rt]);
      qs[rt] = mfma_bf(qa, slo[ks], qs[rt]);
      kq[rt] = mfma_bf(ka, shi[ks], kq[rt]);
      kq[rt] = mfma_bf(ka, slo[ks], kq[rt]);
    }
  // R' = beta (V - exp(gamma) K S^T), then block substitution for U (fp16 matrix cores)
  f4 u[4];
  const f4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f4 wv;
#pragma unroll
    for (int e = 0; e < 4; ++e) wv[e] = bet[i][e] * (vv[i][e] - eg[i][e] * kq[i][e]);
#pragma unroll
    for (int k = 0; k < i; ++k) wv = mfma_16x16x16(lf[lblk(i, k)], to_h4(u[k]), wv);
    u[i] = mfma_16x16x16(xf[i], to_h4(wv), zero);
  }
  // O = diag(exp gamma) Q S^T + P U, staged in LDS for the output wave
  const h8 ub0 = b_pair(u[0], u[1]), ub1 = b_pair(u[2], u[3]);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = qs[i][e] * eg[i][e];
    o = mfma_16x16x32(a_perm(&R.P[16 * i + ln][0], 0, lg), ub0, o);
    if (i >= 2) o = mfma_16x16x32(a_perm(&R.P[16 * i + ln][0], 32, lg), ub1, o);
#pragma unroll
    for (int e = 0; e < 4; ++e) Os[16 * i + 4 * lg + e][16 * w + ln] = a.scale * o[e];
  }
  // S^T <- exp(gamma_63) S^T + K^T (diag(exp(gamma_63 - gamma)) U): bf16, U as hi + lo
  f4 ud[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) ud[i][e] = u[i][e] * egl[i][e];
  bf8 dhi[2], dlo[2];
  split_pair(ud[0], ud[1], dhi[0], dlo[0]);
  split_pair(ud[2], ud[3], dhi[1], dlo[1]);
  const float dec = R.gt[1][C - 1];
  const int trow = 4 * lg + (ln >> 2), tcol = 4 * (ln & 3);
#pragma unroll
  for (int kt = 0; kt < 8; ++kt) {
    f4 s = sacc[kt];
#pragma unroll
    for (int e = 0; e < 4; ++e) s[e] *= dec;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const uint2 p0 = lds_tr4_bits(&B.Ks[32 * ks + trow][16 * kt + tcol]);
      const uint2 p1 = lds_tr4_bits(&B.Ks[32 * ks + 16 + trow][16 * kt + tcol]);
      const bf8 kta = __builtin_bit_cast(bf8, make_uint4(p0.x, p0.y, p1.x, p1.y));
      s = mfma_bf(kta, dhi[ks], s);
      s = mfma_bf(kta, dlo[ks], s);
    }
    sacc[kt] = s;
  }
}

// Copy wave: issue the direct global -> LDS loads of chunk c into buffer B (no registers).
// Q/K rows and the V slice are gathered from the strided tensors into padded rows; rows past
// the end of the chunk re-read its first row (finite values that only ever meet zero weights).
__device__ __forceinline__ void issue_chunk(ScanBuf& B, const PrefillArgs& a, const Geo& G,
                                            const unsigned char* recs, int c) {
  using namespace mp;
  const int lane = G.lane;
  const int L = G.len(c);
  const int64_t c0 = G.start + (int64_t)c * C;
  const uint16_t* qb = static_cast<const uint16_t*>(a.q) + c0 * a.qk_stride + (int64_t)G.kh * D;
  const uint16_t* kb = static_cast<const uint16_t*>(a.k) + c0 * a.qk_stride + (int64_t)G.kh * D;
  constexpr int QPR = LDQ / 8;  // 16-byte pieces per padded Q/K row (17)
#pragma unroll
  for (int i = 0; i < C * QPR / 64; ++i) {
    const int j = 64 * i + lane, r = j / QPR, pc = j % QPR;
    const int64_t off = (r < L && pc < D / 8) ? (int64_t)r * a.qk_stride + 8 * pc : 0;
    __builtin_amdgcn_global_load_lds((glb_void*)(qb + off), (lds_void*)(&B.Qs[0][0] + 512 * i), 16, 0, 0);
    __builtin_amdgcn_global_load_lds((glb_void*)(kb + off), (lds_void*)(&B.Ks[0][0] + 512 * i), 16, 0, 0);
  }
  const unsigned char* rec = recs + G.rec0 + (size_t)c * REC_BYTES;
#pragma unroll
  for (int i = 0; i < REC_BYTES / 1024; ++i)
    __builtin_amdgcn_global_load_lds((glb_void*)(rec + 1024 * i + 16 * lane),
                                     (lds_void*)(reinterpret_cast<unsigned char*>(&B.R) + 1024 * i), 16, 0, 0);
  const uint16_t* vb = static_cast<const uint16_t*>(a.v) + c0 * a.v_stride + (int64_t)G.h * D + G.dv0;
  constexpr int VPR = LDV / 8;  // 16-byte pieces per padded V row (5)
#pragma unroll
  for (int i = 0; i < C * VPR / 64; ++i) {
    const int j = 64 * i + lane, r = j / VPR, pc = j % VPR;
    const int64_t off = (r < L && pc < DVB / 8) ? (int64_t)r * a.v_stride + 8 * pc : 0;
    __builtin_amdgcn_global_load_lds((glb_void*)(vb + off), (lds_void*)(&B.Vs[0][0] + 512 * i), 16, 0, 0);
  }
}

// Output wave: write out the output tile of chunk c (rows < L), staged in Os.
template <int O_DT>
__device__ __forceinline__ void write_out(const float (*Os)[mp::DVB + 4], const PrefillArgs& a, const Geo& G,
                                          int c) {
  using namespace mp;
  const int lane = G.lane;
  if (lane >= G.len(c)) return;
  const float* row = &Os[lane][0];
  const int64_t base = ((G.start + (int64_t)c * C + lane) * a.hv + G.h) * (int64_t)D + G.dv0;
#pragma unroll
  for (int j = 0; j < DVB / 8; ++j) {
    float v[8];
    const f4 x0 = *reinterpret_cast<const f4*>(row + 8 * j), x1 = *reinterpret_cast<const f4*>(row + 8 * j + 4);
    v[0] = x0[0]; v[1] = x0[1]; v[2] = x0[2]; v[3] = x0[3];
    v[4] = x1[0]; v[5] = x1[1]; v[6] = x1[2]; v[7] = x1[3];
    store8<O_DT>(a.o, base + 8 * j, v);
  }
}

template <int O_DT>
__global__ __launch_bounds__(256) void scan_kernel(PrefillArgs a, int64_t maxch) {
  using namespace mp;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  ScanSmem& sm = *reinterpret_cast<ScanSmem*>(smem_raw);
  const int32_t* off = static_cast<const int32_t*>(a.workspace);
  const unsigned char* recs = static_cast<const unsigned char*>(a.workspace) + align256(4 * (size_t)(a.num_seqs + 1));

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
  G.rec0 = ((size_t)G.h * (size_t)maxch + (size_t)off[n]) * REC_BYTES;
  const int ln = G.ln, lg = G.lg;

  // Every role runs its own loop with one workgroup barrier per chunk after a common
  // prologue barrier.  Iteration c: consumers on chunk c (buffer c & 1), the copy wave
  // fills buffer (c+1) & 1 and waits for its copies before the barrier, the output wave
  // writes out chunk c-1.
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
      consume(sm.B[c & 1], sm.Os[c & 1], a, G, sacc);
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
    if (G.nchunks > 0) {
      issue_chunk(sm.B[0], a, G, recs, 0);
      __builtin_amdgcn_s_waitcnt(0);
    }
    __syncthreads();
    for (int c = 0; c < G.nchunks; ++c) {
      if (c + 1 < G.nchunks) {
        issue_chunk(sm.B[(c + 1) & 1], a, G, recs, c + 1);
        __builtin_amdgcn_s_waitcnt(0);
      }
      __syncthreads();
    }
  } else {
    __syncthreads();
    for (int c = 0; c < G.nchunks; ++c) {
      if (G.w == NCW + 1 && c >= 1) write_out<O_DT>(sm.Os[(c - 1) & 1], a, G, c - 1);
      __syncthreads();
    }
    if (G.w == NCW + 1 && G.nchunks > 0) write_out<O_DT>(sm.Os[(G.nchunks - 1) & 1], a, G, G.nchunks - 1);
  }
}

// ---------------------------------------------------------------- host side
size_t prefill_mfma_workspace(int num_seqs, int64_t total, int, int hv) {
  if (num_seqs <= 0) return 0;
  return align256(4 * (size_t)(num_seqs + 1)) + (size_t)hv * (size_t)max_chunks(total, num_seqs) * mp::REC_BYTES;
}

template <int O_DT>
static hipError_t launch_o(const PrefillArgs& a, hipStream_t st) {
  if (a.num_seqs == 0) return hipSuccess;
  const int64_t maxch = max_chunks(a.total, a.num_seqs);
  hipLaunchKernelGGL(chunk_offsets_kernel, dim3(1), dim3(256), 0, st, a.cu, a.num_seqs, a.total,
                     static_cast<int32_t*>(a.workspace));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.total > 0) {
    hipLaunchKernelGGL(prep_kernel, dim3((unsigned)maxch, (unsigned)a.hk), dim3(256), 0, st, a, maxch);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const size_t smem = sizeof(ScanSmem);
  auto k = scan_kernel<O_DT>;
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(k, dim3((unsigned)((int64_t)a.num_seqs * a.hv * mp::NB)), dim3(256), smem, st, a, maxch);
  return hipGetLastError();
}

hipError_t launch_prefill_mfma(const PrefillArgs& a, hipStream_t st) {
  return a.o_dtype == DT_BF16 ? launch_o<DT_BF16>(a, st) : launch_o<DT_F32>(a, st);
}

}  // namespace agnes
