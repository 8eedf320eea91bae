// Global attention layer of the model (model card "Agnes-3.0-Flash Preview", 架构 table, rows
// 全局注意力 and 位置编码): 24 query / 4 KV heads (GQA 6 : 1) of dimension 256, RMS-norm on q
// and k, three-axis rotary on the first 64 dims (frequency j on axis j mod 3, base 1e7, dim j
// paired with dim j + 32), causal softmax attention with scale 1/16 inside each sequence, and a
// sigmoid gate on the output.
//
// Prefill: three launches (decode: three more, at the end of this file).
//   1. attn_offsets_kernel: first 128-query block of every sequence (device prefix sum).
//   2. attn_kprep_kernel: per (token, KV head) the normalised, rotated k in bf16 (the KV cache
//      rows, written where the caller says), an optional copy of v, and per token the 32 (cos,
//      sin) pairs of its rotary angles, computed in fp64 and rounded once to fp32.
//   3. attn_fwd_kernel: one 8-wave workgroup per (128-query block, query head).  Each wave owns
//      16 queries; two waves share a SIMD, so one's softmax overlaps the other's products.  The q rows arrive by direct global -> LDS copies and are normalised and
//      rotated in place, scaled by log2(e)/16 and kept as bf16 matrix-core operands.  K and V
//      blocks of 64 keys are double-buffered in LDS (direct copies, 16-byte chunks of a row
//      XOR-swizzled by a permutation of the row's low four bits, so both the 16-byte fragment
//      reads and the transposing reads are free of bank conflicts).  Per block: S^T = K Q^T
//      (each lane then holds scores of one query), an online softmax in base 2, and
//      O^T += V^T P^T with the V^T fragments from the transposing LDS read; every LDS operand
//      is read one step ahead of its products.  The running maximum moves only when a score exceeds it by more than 2^8
//      (the weights stay <= 256, the result is unchanged, and the accumulators are rescaled
//      rarely).  The output is divided by the softmax sum, multiplied by sigmoid(gate) and
//      stored straight from the result layout.
#include "common.h"
#include "launch.h"

namespace agnes {
namespace at {
constexpr int D = 256;        // head dim
constexpr int HROT = 32;      // rotary pairs (dims 0..31 with 32..63)
constexpr int BQ = 128;       // queries per workgroup
constexpr int BK = 64;        // keys per block
constexpr int NW = 4;         // waves per workgroup (decode)
constexpr int NWF = 8;        // waves per workgroup (prefill): two per SIMD
constexpr int QT = BQ / 16 / NWF;  // 16-query tiles per wave (prefill)
constexpr int CH = D / 8;     // 16-byte chunks per row (32)
}  // namespace at

typedef __bf16 abf8 __attribute__((ext_vector_type(8)));
typedef short as4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) as4v alds_s4v;
typedef __attribute__((address_space(3))) void alds_void;
typedef __attribute__((address_space(1))) void aglb_void;

struct AttnSmem {
  uint16_t t[4][at::BK][at::D];  // [0] K, [1] V of even blocks; [2] K, [3] V of odd blocks
};
static_assert(sizeof(AttnSmem) == 128 * 1024, "attention LDS");

// Chunk permutation of a row: ((r & 7) << 1) | bit 3 of r.  For 16 consecutive rows it is a
// bijection on 0..15 (the 16-byte fragment reads of 16 rows hit 16 different bank groups), and
// rows 4a..4a+3 differ in bits 1..2 (the transposing reads of 4 rows x 2 adjacent chunks hit 8).
__device__ __forceinline__ int rsw(int r) { return ((r & 7) << 1) | ((r >> 3) & 1); }

// Swizzled element offset of (row, col) in a [rows][256] bf16 tile: chunk col/8 of the row sits
// at chunk position (col/8) ^ rsw(row).
__device__ __forceinline__ int swz(int row, int col) {
  return row * at::D + ((((col >> 3) ^ rsw(row)) << 3) | (col & 7));
}

__device__ __forceinline__ f4 amfma(abf8 a, abf8 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Transposing LDS read of four 16-bit values (ds_read_b64_tr_b16): within a 16-lane group, lane
// 4a+b receives the b-th value of the reads of lanes a, a+4, a+8, a+12.
__device__ __forceinline__ uint2 atr4(const uint16_t* p) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((alds_s4v*)(p)));
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) x += __shfl_xor(x, m);
  return x;
}

// Sequence containing token t (cu nondecreasing, clamped to [0, total]).
__device__ __forceinline__ int seq_of(const int32_t* cu, int num_seqs, int64_t total, int64_t t) {
  int lo = 0, hi = num_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu_at(cu, mid, total) <= t) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// ---------------------------------------------------------------- 1. block offsets
// off[n] = sum over m < n of ceil(len_m / BQ); off[num_seqs] = the total.  One 256-thread block.
__global__ __launch_bounds__(256) void attn_offsets_kernel(const int32_t* cu, int num_seqs, int64_t total,
                                                           int32_t* off) {
  __shared__ int32_t part[256];
  const int per = (num_seqs + 255) / 256;
  const int a = threadIdx.x * per;
  int32_t s = 0;
  for (int n = a; n < a + per && n < num_seqs; ++n) {
    const int64_t len = cu_at(cu, n + 1, total) - cu_at(cu, n, total);
    s += len > 0 ? (int32_t)((len + at::BQ - 1) / at::BQ) : 0;
  }
  part[threadIdx.x] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    int32_t run = 0;
    for (int i = 0; i < 256; ++i) {
      const int32_t v = part[i];
      part[i] = run;
      run += v;
    }
    off[num_seqs] = run;
  }
  __syncthreads();
  int32_t run = part[threadIdx.x];
  for (int n = a; n < a + per && n < num_seqs; ++n) {
    off[n] = run;
    const int64_t len = cu_at(cu, n + 1, total) - cu_at(cu, n, total);
    run += len > 0 ? (int32_t)((len + at::BQ - 1) / at::BQ) : 0;
  }
}

// ---------------------------------------------------------------- 2. k prep and rotary table
// Rotary angles of frequency j at position p: p * base^(-2j/64), in fp64; (cos, sin) rounded to
// fp32.  pos3 = nullptr: text positions (the index in the sequence on all three axes).
__device__ __forceinline__ float2 rope_cs(const AttnArgs& a, int64_t t, int64_t pos_text, int j) {
  const int64_t p = a.pos3 ? (int64_t)a.pos3[(int64_t)(j % 3) * a.pos3_stride + t] : pos_text;
  const double inv = exp(-(2.0 * j / (2.0 * at::HROT)) * log((double)a.rope_base));
  double s, c;
  sincos((double)p * inv, &s, &c);
  return make_float2((float)c, (float)s);
}

// One wave per (token, KV head); lane l holds dims 4l..4l+3.  Rotary partners (j, j+32) sit in
// lanes l and l^8 of lanes 0..15.
__global__ __launch_bounds__(256) void attn_kprep_kernel(AttnArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wid >= a.total * a.hkv) return;
  const int64_t t = wid / a.hkv;
  const int g = (int)(wid % a.hkv);
  const int n = seq_of(a.cu, a.num_seqs, a.total, t);
  const int64_t pt = t - cu_at(a.cu, n, a.total);
  float2* tab = reinterpret_cast<float2*>(static_cast<unsigned char*>(a.workspace) + a.tab_off) + t * at::HROT;
  if (g == 0 && lane < at::HROT) tab[lane] = rope_cs(a, t, pt, lane);
  const uint16_t* kr = static_cast<const uint16_t*>(a.k) + t * a.k_stride + (int64_t)g * at::D + 4 * lane;
  const uint2 raw = *reinterpret_cast<const uint2*>(kr);
  float x[4] = {bf16_to_f32(raw.x & 0xffffu), bf16_to_f32(raw.x >> 16), bf16_to_f32(raw.y & 0xffffu),
                bf16_to_f32(raw.y >> 16)};
  const float ss = wave_sum(x[0] * x[0] + x[1] * x[1] + x[2] * x[2] + x[3] * x[3]);
  const float r = rsqrt_fast(ss * (1.0f / at::D) + a.eps);
  const uint2 wr = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(a.k_norm_w) + 4 * lane);
  x[0] *= r * bf16_to_f32(wr.x & 0xffffu);
  x[1] *= r * bf16_to_f32(wr.x >> 16);
  x[2] *= r * bf16_to_f32(wr.y & 0xffffu);
  x[3] *= r * bf16_to_f32(wr.y >> 16);
  float y[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) y[e] = __shfl_xor(x[e], 8);
  if (lane < 16) {
    // this lane's pairs j = 4 (lane & 7) + e; the table entry is written by this same token's
    // head-0 wave, so recompute it here rather than wait for it
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float2 cs = rope_cs(a, t, pt, 4 * (lane & 7) + e);
      x[e] = lane < 8 ? x[e] * cs.x - y[e] * cs.y : x[e] * cs.x + y[e] * cs.y;
    }
  }
  uint16_t* ko = static_cast<uint16_t*>(a.k_out) + t * a.k_out_stride + (int64_t)g * at::D + 4 * lane;
  *reinterpret_cast<uint2*>(ko) = make_uint2(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]));
  if (a.v_out) {
    const uint16_t* vr = static_cast<const uint16_t*>(a.v) + t * a.v_stride + (int64_t)g * at::D + 4 * lane;
    uint16_t* vo = static_cast<uint16_t*>(a.v_out) + t * a.v_out_stride + (int64_t)g * at::D + 4 * lane;
    *reinterpret_cast<uint2*>(vo) = *reinterpret_cast<const uint2*>(vr);
  }
}

// ---------------------------------------------------------------- 3. attention
// Direct copies of 64 rows (two per 1 KiB copy) of a [rows][256] bf16 source into a swizzled
// LDS tile: lane i of copy u brings row 2u + i/32, chunk (i % 32) ^ rsw(row), so the LDS slot
// of chunk c of a row is c ^ rsw(row).  Rows at or past `valid` re-read row valid - 1 (their
// results are masked or dropped).  With NWC copying waves, copies u = q + NWC j (j < 32 / NWC)
// are wave q's: row r = 2q + rr + 2 NWC j, whose swizzle rsw(r) depends on j only through its
// parity (2 NWC is 8 or 16: bit 3 of r flips with j or never), so the lane's element offset is
// o[j & 1] + 2 NWC j stride.
struct CopyOffs {
  int32_t o[2];
};
template <int NWC>
__device__ __forceinline__ CopyOffs copy_offs(int64_t stride, int q, int lane) {
  CopyOffs c;
  const int rr = lane >> 5, ch = lane & 31, r0 = 2 * q + rr;
#pragma unroll
  for (int b = 0; b < 2; ++b) c.o[b] = (int32_t)(r0 * stride + 8 * (ch ^ rsw(r0 + 2 * NWC * b)));
  return c;
}
// AUX: cache policy of the direct copies.  The decode passes 2 (non-temporal): each cached row
// is read once per step, and streaming them takes the split-K attention from 415 to 355 us for
// 64 entries of 8191 cached tokens; the prefill keeps 0, its key and value blocks are read again
// by the later query blocks.
template <int NWC, int AUX = 0>
__device__ __forceinline__ void copy_rows(uint16_t* tile, const uint16_t* src, int64_t stride, int row0, int valid,
                                          int q, int lane, const CopyOffs& off) {
  if (row0 + 64 <= valid) {
    const uint16_t* base = src + (int64_t)row0 * stride;
#pragma unroll
    for (int j = 0; j < 32 / NWC; ++j)
      __builtin_amdgcn_global_load_lds((aglb_void*)(base + 2 * NWC * j * stride + off.o[j & 1]),
                                       (alds_void*)(tile + 2 * (q + NWC * j) * at::D), 16, 0, AUX);
    return;
  }
  const int rr = lane >> 5, ch = lane & 31;
  for (int u = q; u < 32; u += NWC) {
    int r = 2 * u + rr;
    const int lr = r;
    if (row0 + r >= valid) r = valid - 1 - row0;
    const uint16_t* s = src + (int64_t)(row0 + r) * stride + 8 * (ch ^ rsw(lr));
    __builtin_amdgcn_global_load_lds((aglb_void*)s, (alds_void*)(tile + 2 * u * at::D), 16, 0, AUX);
  }
}

template <int O_DT>
__global__ __launch_bounds__(64 * at::NWF) void attn_fwd_kernel(AttnArgs a, int nblk_total) {
  using namespace at;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  AttnSmem& sm = *reinterpret_cast<AttnSmem*>(smem_raw);
  const int32_t* off = reinterpret_cast<const int32_t*>(static_cast<const unsigned char*>(a.workspace) + a.off_off);
  const float2* tab = reinterpret_cast<const float2*>(static_cast<const unsigned char*>(a.workspace) + a.tab_off);

  // Workgroups of one query block and its 24 heads are consecutive in lid and share one XCD
  // (block ids go round-robin over the 8 XCDs); heavy (late) query blocks go first.
  const unsigned nb = gridDim.x;
  unsigned lid = blockIdx.x;
  if ((nb & 7u) == 0) lid = (blockIdx.x & 7u) * (nb >> 3) + (blockIdx.x >> 3);
  const int h = (int)(lid % (unsigned)a.hq);
  const int jb = nblk_total - 1 - (int)(lid / (unsigned)a.hq);
  if (jb < 0 || jb >= off[a.num_seqs]) return;
  int n = 0;
  {
    int lo = 0, hi = a.num_seqs - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (off[mid] <= jb) lo = mid;
      else hi = mid - 1;
    }
    n = lo;
  }
  const int64_t start = cu_at(a.cu, n, a.total);
  const int len = (int)(cu_at(a.cu, n + 1, a.total) - start);
  const int q0 = (jb - off[n]) * BQ;  // first query of the block, in the sequence
  const int g = h / (a.hq / a.hkv);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, ln = lane & 15, lg = lane >> 4;
  const int qlast = (q0 + BQ < len ? q0 + BQ : len) - 1;
  const int nkb = qlast / BK + 1;

  const uint16_t* qsrc = static_cast<const uint16_t*>(a.q) + start * a.q_stride + (int64_t)h * D;
  const uint16_t* ksrc = static_cast<const uint16_t*>(a.k_out) + start * a.k_out_stride + (int64_t)g * D;
  const uint16_t* vsrc = static_cast<const uint16_t*>(a.v) + start * a.v_stride + (int64_t)g * D;

  // q rows into tiles 2 and 3 (rows 0..63, 64..127 of the block), K/V block 0 into tiles 0, 1
  const CopyOffs qoff = copy_offs<NWF>(a.q_stride, w, lane), koff = copy_offs<NWF>(a.k_out_stride, w, lane),
                 voff = copy_offs<NWF>(a.v_stride, w, lane);
  copy_rows<NWF>(&sm.t[2][0][0], qsrc, a.q_stride, q0, len, w, lane, qoff);
  copy_rows<NWF>(&sm.t[3][0][0], qsrc, a.q_stride, q0 + BK, len, w, lane, qoff);
  copy_rows<NWF>(&sm.t[0][0][0], ksrc, a.k_out_stride, 0, len, w, lane, koff);
  copy_rows<NWF>(&sm.t[1][0][0], vsrc, a.v_stride, 0, len, w, lane, voff);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // RMS-norm, rotary and the base-2 softmax scale of this wave's 16 q rows, in place; lane l
  // holds dims 4l..4l+3 of a row.
  {
    const uint2 wr = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(a.q_norm_w) + 4 * lane);
    const float wq[4] = {bf16_to_f32(wr.x & 0xffffu), bf16_to_f32(wr.x >> 16), bf16_to_f32(wr.y & 0xffffu),
                         bf16_to_f32(wr.y >> 16)};
    const float qscale = (a.scale > 0.f ? a.scale : 0.0625f) * 1.4426950408889634f;
    for (int i = 0; i < QT * 16; ++i) {
      const int row = 16 * QT * w + i;  // row of the 128-query block
      uint16_t* tile = &sm.t[2 + (row >> 6)][0][0];
      uint16_t* p = tile + swz(row & 63, 4 * lane);
      const uint2 raw = *reinterpret_cast<const uint2*>(p);
      float x[4] = {bf16_to_f32(raw.x & 0xffffu), bf16_to_f32(raw.x >> 16), bf16_to_f32(raw.y & 0xffffu),
                    bf16_to_f32(raw.y >> 16)};
      const float ss = wave_sum(x[0] * x[0] + x[1] * x[1] + x[2] * x[2] + x[3] * x[3]);
      const float r = rsqrt_fast(ss * (1.0f / D) + a.eps);
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] *= r * wq[e];
      float y[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) y[e] = __shfl_xor(x[e], 8);
      int qi = q0 + row;
      if (qi > len - 1) qi = len - 1;
      if (lane < 16) {
        const float4 c2 = *reinterpret_cast<const float4*>(tab + (start + qi) * HROT + 4 * (lane & 7));
        const float4 c3 = *reinterpret_cast<const float4*>(tab + (start + qi) * HROT + 4 * (lane & 7) + 2);
        const float cs[4][2] = {{c2.x, c2.y}, {c2.z, c2.w}, {c3.x, c3.y}, {c3.z, c3.w}};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          x[e] = lane < 8 ? x[e] * cs[e][0] - y[e] * cs[e][1] : x[e] * cs[e][0] + y[e] * cs[e][1];
      }
      *reinterpret_cast<uint2*>(p) =
          make_uint2(pack_bf16x2(x[0] * qscale, x[1] * qscale), pack_bf16x2(x[2] * qscale, x[3] * qscale));
    }
  }
  // Q^T operands: B[k = dim][n = query], lane (ln, lg) holds dims 32 ks + 8 lg .. + 7 of query ln
  abf8 qf[QT][8];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int row = 16 * QT * w + 16 * qt + ln;
    const uint16_t* tile = &sm.t[2 + (row >> 6)][0][0];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[qt][ks] = *reinterpret_cast<const abf8*>(tile + swz(row & 63, 32 * ks + 8 * lg));
  }

  const f4 zero = {0.f, 0.f, 0.f, 0.f};
  f4 acc[QT][16];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt)
#pragma unroll
    for (int d = 0; d < 16; ++d) acc[qt][d] = zero;
  float mrun[QT], lsum[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    mrun[qt] = -INFINITY;
    lsum[qt] = 0.f;
  }
  const int trow = 4 * lg + (ln >> 2), tcol = 4 * (ln & 3);

  for (int kb = 0; kb < nkb; ++kb) {
    if (kb > 0) __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();  // block kb has landed; every wave is done with the other buffer
    // copies of block kb + 1: spread over the K S^T steps below (a copy holds the wave at issue
    // for ~4 products' time) when the block lies inside the sequence, all at once otherwise
    const int nrow = (kb + 1) * BK;
    const bool next = kb + 1 < nkb, spread = next && nrow + BK <= len;
    uint16_t* nK = &sm.t[((kb + 1) & 1) * 2][0][0];
    uint16_t* nV = nK + BK * D;
    const uint16_t* kcp = ksrc + (int64_t)nrow * a.k_out_stride;
    const uint16_t* vcp = vsrc + (int64_t)nrow * a.v_stride;
    if (next && !spread) {
      copy_rows<NWF>(nK, ksrc, a.k_out_stride, nrow, len, w, lane, koff);
      copy_rows<NWF>(nV, vsrc, a.v_stride, nrow, len, w, lane, voff);
    }
    const uint16_t* Kt = &sm.t[(kb & 1) * 2][0][0];
    const uint16_t* Vt = &sm.t[(kb & 1) * 2 + 1][0][0];
    // S^T = K Q^T: D[key 4lg+i of tile kt][query ln]; K fragments one 32-dim step ahead
    f4 st[QT][4];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt)
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) st[qt][kt] = zero;
    abf8 kf[2][4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) kf[0][kt] = *reinterpret_cast<const abf8*>(Kt + swz(16 * kt + ln, 8 * lg));
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      if (spread && ks < 32 / NWF) {
        __builtin_amdgcn_global_load_lds((aglb_void*)(kcp + 2 * NWF * ks * a.k_out_stride + koff.o[ks & 1]),
                                         (alds_void*)(nK + 2 * (w + NWF * ks) * D), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((aglb_void*)(vcp + 2 * NWF * ks * a.v_stride + voff.o[ks & 1]),
                                         (alds_void*)(nV + 2 * (w + NWF * ks) * D), 16, 0, 0);
      }
      if (ks < 7) {
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
          kf[(ks + 1) & 1][kt] = *reinterpret_cast<const abf8*>(Kt + swz(16 * kt + ln, 32 * (ks + 1) + 8 * lg));
      }
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) st[qt][kt] = amfma(kf[ks & 1][kt], qf[qt][ks], st[qt][kt]);
      __builtin_amdgcn_sched_barrier(0);
    }
    // V^T fragments of dim tiles 0 and 1, then the softmax while they load
    uint2 vq[3][4];
#pragma unroll
    for (int d = 0; d < 2; ++d)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        vq[d][2 * j] = atr4(Vt + swz(32 * j + trow, 16 * d + tcol));
        vq[d][2 * j + 1] = atr4(Vt + swz(32 * j + 16 + trow, 16 * d + tcol));
      }
    // causal and end-of-sequence mask, online softmax (base 2), P^T operands
    const int kbase = kb * BK;
    abf8 pf[QT][2];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const int qi = q0 + 16 * QT * w + 16 * qt + ln;
      if (kbase + BK - 1 > qi || kbase + BK > len) {
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int kj = kbase + 16 * kt + 4 * lg + i;
            if (kj > qi || kj >= len) st[qt][kt][i] = -INFINITY;
          }
      }
      float mx = st[qt][0][0];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, st[qt][kt][i]);
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      // move the running maximum only past a margin of 8 (factor 256)
      const bool up = mx > mrun[qt] + 8.0f;
      if (__builtin_amdgcn_ballot_w64(up) != 0) {
        const float mnew = up ? mx : mrun[qt];
        const float alpha = __builtin_amdgcn_exp2f(mrun[qt] - mnew);
        mrun[qt] = mnew;
        lsum[qt] *= alpha;
#pragma unroll
        for (int d = 0; d < 16; ++d) acc[qt][d] *= alpha;
      }
      float ps = 0.f;
      float p[4][4];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[kt][i] = __builtin_amdgcn_exp2f(st[qt][kt][i] - mrun[qt]);
          ps += p[kt][i];
        }
      lsum[qt] += ps;
      // keys 32 j + 4 lg + i (tile 2 j) then 32 j + 16 + 4 lg + i (tile 2 j + 1)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint4 u = make_uint4(pack_bf16x2(p[2 * j][0], p[2 * j][1]), pack_bf16x2(p[2 * j][2], p[2 * j][3]),
                                   pack_bf16x2(p[2 * j + 1][0], p[2 * j + 1][1]),
                                   pack_bf16x2(p[2 * j + 1][2], p[2 * j + 1][3]));
        pf[qt][j] = __builtin_bit_cast(abf8, u);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // O^T += V^T P^T: A[m = dim 16 d + ln][k] from the transposing read of the V rows, two dim
    // tiles ahead
#pragma unroll
    for (int d = 0; d < 16; ++d) {
      if (d < 14) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          vq[(d + 2) % 3][2 * j] = atr4(Vt + swz(32 * j + trow, 16 * (d + 2) + tcol));
          vq[(d + 2) % 3][2 * j + 1] = atr4(Vt + swz(32 * j + 16 + trow, 16 * (d + 2) + tcol));
        }
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint2 lo = vq[d % 3][2 * j], hi = vq[d % 3][2 * j + 1];
        const abf8 vf = __builtin_bit_cast(abf8, make_uint4(lo.x, lo.y, hi.x, hi.y));
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) acc[qt][d] = amfma(vf, pf[qt][j], acc[qt][d]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // O = O^T / l * sigmoid(gate): lane holds dims 16 d + 4 lg .. + 3 of query ln
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    float l = lsum[qt];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    const float inv = 1.0f / l;
    const int qi = q0 + 16 * QT * w + 16 * qt + ln;
    if (qi < len) {
      const int64_t t = start + qi;
      const uint16_t* gp = static_cast<const uint16_t*>(a.gate) + t * a.gate_stride + (int64_t)h * D + 4 * lg;
#pragma unroll
      for (int d = 0; d < 16; ++d) {
        const uint2 gr = *reinterpret_cast<const uint2*>(gp + 16 * d);
        const float gv[4] = {bf16_to_f32(gr.x & 0xffffu), bf16_to_f32(gr.x >> 16), bf16_to_f32(gr.y & 0xffffu),
                             bf16_to_f32(gr.y >> 16)};
        f4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = acc[qt][d][e] * inv * __builtin_amdgcn_rcpf(1.0f + __expf(-gv[e]));
        store4<O_DT>(a.o, (t * a.hq + h) * (int64_t)D + 16 * d + 4 * lg, o);
      }
    }
  }
}

// ---------------------------------------------------------------- decode
// One new token per batch entry b; the caches [batch][max_len][hkv][256] hold cache_lens[b]
// earlier tokens and the new one goes to index L = cache_lens[b].  An entry with L outside
// [0, max_len) is padding: no cache write, zero output.
typedef short ds4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int entry_len(const AttnArgs& a, int b) {
  const int L = a.cache_lens[b];
  return (L >= 0 && (int64_t)L < a.max_len) ? L : -1;
}

__device__ __forceinline__ f4 amfma16(ds4v a, ds4v b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// 1. One wave per (entry, row): rows 0..hq-1 are the query heads (normalised, rotated, scaled by
// log2(e) times the softmax scale, bf16 into the workspace), rows hq.. the KV heads (k normalised
// and rotated into the k cache, v copied into the v cache, both at index L).
__global__ __launch_bounds__(256) void attn_decode_prep_kernel(AttnArgs a) {
  const int lane = threadIdx.x & 63;
  const int rows = a.hq + a.hkv;
  const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wid >= a.total * rows) return;
  const int b = (int)(wid / rows), r = (int)(wid % rows);
  const int L = entry_len(a, b);
  if (L < 0) return;
  const bool isq = r < a.hq;
  const int hd = isq ? r : r - a.hq;
  const uint16_t* src = isq ? static_cast<const uint16_t*>(a.q) + b * a.q_stride + (int64_t)hd * at::D
                            : static_cast<const uint16_t*>(a.k) + b * a.k_stride + (int64_t)hd * at::D;
  const uint2 raw = *reinterpret_cast<const uint2*>(src + 4 * lane);
  float x[4] = {bf16_to_f32(raw.x & 0xffffu), bf16_to_f32(raw.x >> 16), bf16_to_f32(raw.y & 0xffffu),
                bf16_to_f32(raw.y >> 16)};
  const float ss = wave_sum(x[0] * x[0] + x[1] * x[1] + x[2] * x[2] + x[3] * x[3]);
  const float rr = rsqrt_fast(ss * (1.0f / at::D) + a.eps);
  const uint2 wr = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(isq ? a.q_norm_w : a.k_norm_w) +
                                                   4 * lane);
  x[0] *= rr * bf16_to_f32(wr.x & 0xffffu);
  x[1] *= rr * bf16_to_f32(wr.x >> 16);
  x[2] *= rr * bf16_to_f32(wr.y & 0xffffu);
  x[3] *= rr * bf16_to_f32(wr.y >> 16);
  float y[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) y[e] = __shfl_xor(x[e], 8);
  if (lane < 16) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float2 cs = rope_cs(a, b, L, 4 * (lane & 7) + e);
      x[e] = lane < 8 ? x[e] * cs.x - y[e] * cs.y : x[e] * cs.x + y[e] * cs.y;
    }
  }
  if (isq) {
    const float qs = (a.scale > 0.f ? a.scale : 0.0625f) * 1.4426950408889634f;
    uint16_t* qb = reinterpret_cast<uint16_t*>(static_cast<unsigned char*>(a.workspace) + a.off_off) +
                   ((int64_t)b * a.hq + hd) * at::D + 4 * lane;
    *reinterpret_cast<uint2*>(qb) = make_uint2(pack_bf16x2(x[0] * qs, x[1] * qs), pack_bf16x2(x[2] * qs, x[3] * qs));
  } else {
    const int64_t row = (((int64_t)b * a.max_len + L) * a.hkv + hd) * at::D + 4 * lane;
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.k_cache) + row) =
        make_uint2(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]));
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.v_cache) + row) =
        *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(a.v) + b * a.v_stride + (int64_t)hd * at::D +
                                        4 * lane);
  }
}

// 2. Split-K attention: one workgroup per (entry, KV head, key range of sk keys).  The query
// heads of the KV head's group are the rows of one 16-row tile (the rest zero).  64-key blocks
// are double-buffered in LDS as in the prefill; wave w takes keys 16w..16w+15 of each block:
// S^T = K Q^T (16 keys x 16 rows), an online softmax per row, and O^T += V^T P^T on 16x16x16
// products whose B operand is the score fragment as it stands.  The waves' partial results are
// merged through LDS into one (max, sum, O) per query head of the range, in the workspace.
__global__ __launch_bounds__(256) void attn_decode_kernel(AttnArgs a, int ns, int sk) {
  using namespace at;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  AttnSmem& sm = *reinterpret_cast<AttnSmem*>(smem_raw);
  const int G = a.hq / a.hkv;
  const int s = blockIdx.x % ns, g = (blockIdx.x / ns) % a.hkv, b = blockIdx.x / (ns * a.hkv);
  const int L = entry_len(a, b);
  if (L < 0) return;
  float* part = reinterpret_cast<float*>(static_cast<unsigned char*>(a.workspace) + a.tab_off) +
                (((int64_t)b * a.hkv + g) * ns + s) * G * (2 + D);
  const int k0 = s * sk, k1 = (k0 + sk < L + 1 ? k0 + sk : L + 1);
  const int lane = threadIdx.x & 63, ln = lane & 15, lg = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (k0 >= k1) {  // empty range: a partial that weighs nothing
    if (threadIdx.x < G) {
      part[threadIdx.x * (2 + D)] = -INFINITY;
      part[threadIdx.x * (2 + D) + 1] = 0.f;
    }
    return;
  }
  const int nblk = (k1 - k0 + BK - 1) / BK, valid = k1 - k0;
  const int64_t ts = (int64_t)a.hkv * D;  // cache token stride
  const uint16_t* ksrc = static_cast<const uint16_t*>(a.k_cache) + (((int64_t)b * a.max_len + k0) * a.hkv + g) * D;
  const uint16_t* vsrc = static_cast<const uint16_t*>(a.v_cache) + (((int64_t)b * a.max_len + k0) * a.hkv + g) * D;
  const CopyOffs off = copy_offs<NW>(ts, w, lane);
  copy_rows<NW, 2>(&sm.t[0][0][0], ksrc, ts, 0, valid, w, lane, off);
  copy_rows<NW, 2>(&sm.t[1][0][0], vsrc, ts, 0, valid, w, lane, off);
  // Q^T operands: rows ln < G are the query heads g G + ln
  abf8 qf[8];
  {
    const uint16_t* qb = reinterpret_cast<const uint16_t*>(static_cast<const unsigned char*>(a.workspace) + a.off_off) +
                         ((int64_t)b * a.hq + g * G + (ln < G ? ln : 0)) * D;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const uint4 u = *reinterpret_cast<const uint4*>(qb + 32 * ks + 8 * lg);
      qf[ks] = __builtin_bit_cast(abf8, ln < G ? u : make_uint4(0, 0, 0, 0));
    }
  }
  const f4 zero = {0.f, 0.f, 0.f, 0.f};
  f4 acc[16];
#pragma unroll
  for (int d = 0; d < 16; ++d) acc[d] = zero;
  float mrun = -INFINITY, lsum = 0.f;
  const int trow = 4 * lg + (ln >> 2), tcol = 4 * (ln & 3);
  for (int kb = 0; kb < nblk; ++kb) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();  // block kb has landed; every wave is done with the other buffer
    if (kb + 1 < nblk) {
      const int nb = ((kb + 1) & 1) * 2;
      copy_rows<NW, 2>(&sm.t[nb][0][0], ksrc, ts, (kb + 1) * BK, valid, w, lane, off);
      copy_rows<NW, 2>(&sm.t[nb + 1][0][0], vsrc, ts, (kb + 1) * BK, valid, w, lane, off);
    }
    const uint16_t* Kt = &sm.t[(kb & 1) * 2][0][0];
    const uint16_t* Vt = &sm.t[(kb & 1) * 2 + 1][0][0];
    f4 st = zero;
    abf8 kf[2];
    kf[0] = *reinterpret_cast<const abf8*>(Kt + swz(16 * w + ln, 8 * lg));
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      if (ks < 7) kf[(ks + 1) & 1] = *reinterpret_cast<const abf8*>(Kt + swz(16 * w + ln, 32 * (ks + 1) + 8 * lg));
      st = amfma(kf[ks & 1], qf[ks], st);
    }
    // keys k0 + 64 kb + 16 w + 4 lg + i at or past k1 do not exist
    const int kidx = kb * BK + 16 * w + 4 * lg;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (kidx + i >= valid) st[i] = -INFINITY;
    float m = fmaxf(fmaxf(st[0], st[1]), fmaxf(st[2], st[3]));
    m = fmaxf(m, __shfl_xor(m, 16));
    m = fmaxf(m, __shfl_xor(m, 32));
    const bool up = m > mrun + 8.0f;  // move the running maximum only past a margin of 8
    if (__builtin_amdgcn_ballot_w64(up) != 0) {
      const float mnew = up ? m : mrun;
      const float alpha = __builtin_amdgcn_exp2f(mrun - mnew);
      mrun = mnew;
      lsum *= alpha;
#pragma unroll
      for (int d = 0; d < 16; ++d) acc[d] *= alpha;
    }
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {  // a missing key weighs 0 (also while no key of this row exists)
      p[i] = st[i] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(st[i] - mrun);
      lsum += p[i];
    }
    const ds4v pb = __builtin_bit_cast(ds4v, make_uint2(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])));
#pragma unroll
    for (int d = 0; d < 16; ++d) {
      const ds4v va = __builtin_bit_cast(ds4v, atr4(Vt + swz(16 * w + trow, 16 * d + tcol)));
      acc[d] = amfma16(va, pb, acc[d]);
    }
  }
  // merge the four waves: row q = ln, dims 16 d + 4 lg + i
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);
  __syncthreads();  // every wave is done with the tiles
  float* red = reinterpret_cast<float*>(smem_raw);  // [wave][16 rows][2 + 256]
  float* mine = red + (w * 16 + ln) * (2 + D);
  if (lg == 0) {
    mine[0] = mrun;
    mine[1] = lsum;
  }
#pragma unroll
  for (int d = 0; d < 16; ++d)
#pragma unroll
    for (int i = 0; i < 4; ++i) mine[2 + 16 * d + 4 * lg + i] = acc[d][i];
  __syncthreads();
  const int dim = threadIdx.x;  // 256 threads, one dim each
  for (int q = 0; q < G; ++q) {
    float mw[NW], M = -INFINITY;
#pragma unroll
    for (int v = 0; v < NW; ++v) {
      mw[v] = red[(v * 16 + q) * (2 + D)];
      M = fmaxf(M, mw[v]);
    }
    float l = 0.f, o = 0.f;
#pragma unroll
    for (int v = 0; v < NW; ++v) {
      const float wv = mw[v] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw[v] - M);
      l += wv * red[(v * 16 + q) * (2 + D) + 1];
      o += wv * red[(v * 16 + q) * (2 + D) + 2 + dim];
    }
    float* pq = part + q * (2 + D);
    if (dim == 0) {
      pq[0] = M;
      pq[1] = l;
    }
    pq[2 + dim] = o;
  }
}

// 3. One wave per (entry, query head): merge the key ranges, divide by the softmax sum, apply
// sigmoid(gate) and store; padding entries get zeros.
template <int O_DT>
__global__ __launch_bounds__(256) void attn_decode_combine_kernel(AttnArgs a, int ns) {
  const int lane = threadIdx.x & 63;
  const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wid >= a.total * a.hq) return;
  const int b = (int)(wid / a.hq), h = (int)(wid % a.hq);
  const int G = a.hq / a.hkv, g = h / G, q = h % G;
  const int64_t oi = ((int64_t)b * a.hq + h) * at::D + 4 * lane;
  const int L = entry_len(a, b);
  f4 o = {0.f, 0.f, 0.f, 0.f};
  if (L >= 0) {
    const float* part = reinterpret_cast<const float*>(static_cast<const unsigned char*>(a.workspace) + a.tab_off) +
                        (((int64_t)b * a.hkv + g) * ns) * G * (2 + at::D) + q * (2 + at::D);
    float M = -INFINITY;
    for (int s = 0; s < ns; ++s) M = fmaxf(M, part[(int64_t)s * G * (2 + at::D)]);
    float l = 0.f;
    for (int s = 0; s < ns; ++s) {
      const float* ps = part + (int64_t)s * G * (2 + at::D);
      const float ms = ps[0];
      if (ms == -INFINITY) continue;  // an empty key range (its values are not written)
      const float wv = __builtin_amdgcn_exp2f(ms - M);
      l += wv * ps[1];
      const float4 v = *reinterpret_cast<const float4*>(ps + 2 + 4 * lane);
      o[0] += wv * v.x;
      o[1] += wv * v.y;
      o[2] += wv * v.z;
      o[3] += wv * v.w;
    }
    const uint2 gr = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(a.gate) + b * a.gate_stride +
                                                     (int64_t)h * at::D + 4 * lane);
    const float gv[4] = {bf16_to_f32(gr.x & 0xffffu), bf16_to_f32(gr.x >> 16), bf16_to_f32(gr.y & 0xffffu),
                         bf16_to_f32(gr.y >> 16)};
    const float inv = 1.0f / l;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] *= inv * __builtin_amdgcn_rcpf(1.0f + __expf(-gv[e]));
  }
  store4<O_DT>(a.o, oi, o);
}

// Decode split: about 1024 workgroups over the batch and KV heads, ranges of at least 64 keys.
static void decode_split(int64_t batch, int hkv, int64_t max_len, int& ns, int& sk) {
  const int64_t pairs = batch * hkv > 0 ? batch * hkv : 1;
  int64_t n = (1024 + pairs - 1) / pairs;
  const int64_t nmax = (max_len + at::BK - 1) / at::BK;
  if (n > nmax) n = nmax;
  if (n < 1) n = 1;
  int64_t k = (max_len + n - 1) / n;
  k = (k + at::BK - 1) / at::BK * at::BK;
  sk = (int)k;
  ns = (int)((max_len + k - 1) / k);
}

// prep over (entry, query or KV head), attention over (entry, KV head, key split), combine over
// (entry, query head); max_len is at most 2^30.
bool attn_decode_fits(int batch, int hq, int hkv, int64_t max_len) {
  using u128 = unsigned __int128;
  int ns, sk;
  decode_split(batch, hkv, max_len, ns, sk);
  return grid_fits(((u128)batch * ((u128)hq + (u128)hkv) + 3) / 4, 256) &&
         grid_fits((u128)batch * (u128)hkv * (u128)ns, 256) && grid_fits(((u128)batch * (u128)hq + 3) / 4, 256);
}

size_t attn_decode_workspace(int64_t batch, int hq, int hkv, int64_t max_len) {
  if (batch <= 0 || hkv <= 0) return 0;
  int ns, sk;
  decode_split(batch, hkv, max_len, ns, sk);
  const size_t qb = ((size_t)batch * hq * at::D * 2 + 255) & ~size_t(255);
  return qb + (size_t)batch * hq * ns * (2 + at::D) * 4;
}

hipError_t launch_attn_decode(AttnArgs a, hipStream_t st) {
  if (a.total == 0) return hipSuccess;
  int ns, sk;
  decode_split(a.total, a.hkv, a.max_len, ns, sk);
  a.off_off = 0;  // bf16 [batch][hq][256] prepared queries
  a.tab_off = ((size_t)a.total * a.hq * at::D * 2 + 255) & ~size_t(255);  // partial results
  const int64_t waves = a.total * (a.hq + a.hkv);
  hipLaunchKernelGGL(attn_decode_prep_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t smem = sizeof(AttnSmem);
  static const hipError_t a0 = hipFuncSetAttribute(reinterpret_cast<const void*>(attn_decode_kernel),
                                                   hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (a0 != hipSuccess) return a0;
  hipLaunchKernelGGL(attn_decode_kernel, dim3((unsigned)(a.total * a.hkv * ns)), dim3(256), smem, st, a, ns, sk);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t cw = a.total * a.hq;
  if (a.o_dtype == DT_BF16)
    hipLaunchKernelGGL(attn_decode_combine_kernel<DT_BF16>, dim3((unsigned)((cw + 3) / 4)), dim3(256), 0, st, a, ns);
  else
    hipLaunchKernelGGL(attn_decode_combine_kernel<DT_F32>, dim3((unsigned)((cw + 3) / 4)), dim3(256), 0, st, a, ns);
  return hipGetLastError();
}

// ---------------------------------------------------------------- host side
// offsets in one block, key preparation over (token, KV head), attention over (query block,
// query head) with at most total / BQ + num_seqs query blocks.
bool attn_prefill_fits(int num_seqs, int64_t total, int hq, int hkv) {
  using u128 = unsigned __int128;
  const u128 nblk = (u128)((total + at::BQ - 1) / at::BQ) + (u128)num_seqs;
  return grid_fits(((u128)total * (u128)hkv + 3) / 4, 256) && grid_fits(nblk * (u128)hq, 64 * at::NWF);
}

size_t attn_prefill_workspace(int num_seqs, int64_t total) {
  if (num_seqs <= 0) return 0;
  const size_t off = ((size_t)(num_seqs + 1) * 4 + 255) & ~size_t(255);
  return off + (size_t)total * at::HROT * 8;
}

hipError_t launch_attn_prefill(AttnArgs a, hipStream_t st) {
  if (a.num_seqs == 0 || a.total == 0) return hipSuccess;
  a.off_off = 0;
  a.tab_off = ((size_t)(a.num_seqs + 1) * 4 + 255) & ~size_t(255);
  int32_t* off = reinterpret_cast<int32_t*>(static_cast<unsigned char*>(a.workspace) + a.off_off);
  hipLaunchKernelGGL(attn_offsets_kernel, dim3(1), dim3(256), 0, st, a.cu, a.num_seqs, a.total, off);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t waves = a.total * a.hkv;
  hipLaunchKernelGGL(attn_kprep_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, st, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nblk = (int)((a.total + at::BQ - 1) / at::BQ) + a.num_seqs;  // bound on query blocks
  const size_t smem = sizeof(AttnSmem);
  auto k = a.o_dtype == DT_BF16 ? attn_fwd_kernel<DT_BF16> : attn_fwd_kernel<DT_F32>;
  static const hipError_t a0 = hipFuncSetAttribute(reinterpret_cast<const void*>(attn_fwd_kernel<DT_BF16>),
                                                   hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  static const hipError_t a1 = hipFuncSetAttribute(reinterpret_cast<const void*>(attn_fwd_kernel<DT_F32>),
                                                   hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (a0 != hipSuccess) return a0;
  if (a1 != hipSuccess) return a1;
  hipLaunchKernelGGL(k, dim3((unsigned)((int64_t)nblk * a.hq)), dim3(64 * at::NWF), smem, st, a, nblk);
  return hipGetLastError();
}

}  // namespace agnes
