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
// X = (I + A)^-1 is lower triangular and depends only on the inputs, so U = X R' is one
// product; X is built by blocks of 16: X_ii = (I + A_ii)^-1 by forward substitution, then
// X_ij = -X_ii sum_{k=j..i-1} A_ik X_kj for i > j, by increasing i - j.
//
// Three launches on the caller's stream:
//  1. chunk_offsets: first chunk index of every sequence (prefix sum of ceil(len / 64)).
//  2. prep (all chunks in parallel, one workgroup per chunk and key group, four waves per
//     value head of the group): the Gram matrices K K^T and Q K^T on matrix cores, then per
//     value head in fp32 the decay-scaled P, A and X (the blocks of X off the diagonal on
//     fp32 matrix cores), written as one 13 KiB record per (chunk, value head), and the fp16
//     image of the chunk's q and k rows, 33 KiB per (chunk, key group).  Everything in them
//     depends only on the inputs, not on the state.
//  3. scan (serial over chunks): one workgroup of 8 waves per (sequence, value head, block of
//     32 value rows); the value rows of S are independent, so each workgroup scans its own
//     [32 x 128] fp32 slice of the state.  The chain wave keeps that slice of S^T in matrix-core
//     accumulators for the whole sequence and per chunk runs K S^T, U = X R' and the state
//     update (the serial path); the output wave computes Q S^T and, one chunk later, P U and
//     the output rows, with the fp16 state and U operands handed over through LDS.  A 16x16
//     result fragment is reused as the next product's operand without leaving registers: the
//     contraction index of a 16x16x32 product may be permuted as long as both operands use
//     the same permutation, so two result fragments side by side form a B operand and the
//     matching A operand is read from LDS as two 8-byte pieces (K^T pieces come straight from
//     the row-major K tile through the gfx950 transposing LDS read).  Six copy waves fill the
//     other half of a double buffer with the next chunk (q/k image, record, V slice) by direct
//     global -> LDS loads.  Each chunk costs one workgroup barrier; each role runs its own
//     loop with the same barrier count, so registers are allocated per role.
// Fused prologue (same kernels, compiled a second time): q, k, v are the channel ranges of
// the raw projection output x, and the causal conv (kernel 4) + SiLU + L2 of q and k run
// inside the prefill instead of in a separate pass over x.  prep convolves the chunk's q and
// k rows (a 3-token halo from x, or from the conv history before a sequence's first token)
// straight into its fp16 staging; in the scan the copy waves bring the raw x rows of the V
// slice one chunk early and convolve them while the next chunk's copies are in flight.  The
// conv history is advanced by a fourth launch once every read of the old one is done.
// Number formats: bf16 inputs widen exactly to fp16 (normal range); fp32 intermediates
// (S, R', U, P, X) are rounded to fp16 once per use (2^-11 relative); every product
// accumulates in fp32 and the state itself stays fp32.
#include <hip/hip_ext.h>

#include <mutex>

#include "common.h"
#include "launch.h"

namespace agnes {

namespace mp {
constexpr int C = 64;        // chunk
constexpr int D = 128;       // head dim (key and value)
constexpr int LDQ = D + 8;   // fp16 row stride of staged Q/K rows
constexpr int NVT = 2;       // 16-wide value tiles per scan workgroup
// Value tiles per chain wave and per output wave (measured at T = 8192).  One tile per wave
// (two chain and two output waves, one SIMD each) halves each wave's serial work, but every wave
// then streams the whole K, Q, X and P tiles from LDS for half the products, and ten waves leave
// each at most 170 registers: the prefill calls run 5 % faster so, the whole-layer call (whose
// two tile waves then share SIMDs with the chain or output waves) no faster.
constexpr int tpw(bool norm) { return norm ? 2 : 1; }
constexpr int npair(bool norm) { return NVT / tpw(norm); }  // chain waves (and as many output waves)
constexpr int NCP = 6;       // copy waves
constexpr int nwaves(bool norm) { return 2 * npair(norm) + NCP; }  // chain, output, copy waves
constexpr int MAX_WAVES = 2 * NVT + NCP;
constexpr int DVB = 16 * NVT;
constexpr int RING = 8;      // whole-layer call: chunk slots of the partial-sum exchange
static_assert(RING >= 4 && (RING & (RING - 1)) == 0, "exchange ring: no slot reused before it is read");
constexpr int NB = D / DVB;  // scan workgroups per value head
constexpr int LDV = DVB + 8; // bf16 row stride of the staged V slice
constexpr int VR_ROWS = 80;  // raw x rows of a V slice (fused): 3 halo + 64, to 5 x 1 KiB copies
}  // namespace mp

// Per (chunk, value head) record written by prep and copied verbatim into LDS by scan, so it
// is laid out as the LDS image the consumers read.  P and X are stored as the six 16x32
// A-operand fragments the scan multiplies by: row block f, columns 0..31 (f = 0..3), and row
// blocks 2, 3, columns 32..63 (f = 4, 5).  Lane 16g + m of fragment f holds row 16 rb(f) + m,
// columns k0 + 4g .. + 3 and k0 + 16 + 4g .. + 3 (the order of a_perm), so a lane reads its
// operand with one 16-byte LDS read.  The blocks above the diagonal inside the fragments, (0,1)
// and (2,3), hold zeros; the other blocks above the diagonal are not stored.
struct RecImage {
  h8 P[6][64];                     // P = lower_incl(exp(gamma_r - gamma_s) q_r.k_s)
  h8 X[6][64];                     // X = (I + A)^-1
  float gt[3][mp::C];              // beta, exp(gamma), exp(gamma_63 - gamma)
  float pad[64];                   // to a whole number of 1 KiB copy steps
};
static_assert(sizeof(RecImage) == 13 * 1024, "record image is copied in 1 KiB steps");
// Byte offset in a fragment-packed P or X of the four values (r, s .. s + 3), s a multiple of 4
// and (r, s) inside a stored fragment.
__host__ __device__ constexpr int frag_off(int r, int s) {
  return ((((r >> 4) + 2 * (s >> 5)) * 64 + 16 * ((s & 15) >> 2) + (r & 15)) * 8 + 4 * ((s & 31) >> 4)) * 2;
}
static_assert(frag_off(0, 0) == 0 && frag_off(0, 16) == 8 && frag_off(1, 4) == 16 * 17 &&
                  frag_off(32, 32) == 4 * 64 * 16 && frag_off(63, 60) == (5 * 64 + 63) * 16 + 8,
              "fragment packing");
// Per (chunk, key group) image of the fp16 q and k rows (rows past the chunk end are zero).  Q
// is read only as the A operand of Q S^T, so it is stored as those sixteen 16x32 fragments
// (fragment 4 ks + rt: rows 16 rt .. + 15, columns 32 ks .. + 31, lanes as for P and X); K is
// also read transposed, so it stays row-major (rows padded against bank conflicts).
struct QKImage {
  h8 Q[16][64];
  _Float16 K[mp::C][mp::LDQ];
};
static_assert(sizeof(QKImage) == 33 * 1024, "q/k image is copied in 1 KiB steps");
// Byte offset in the fragment-packed Q of the four values (r, s .. s + 3), s a multiple of 4.
__host__ __device__ constexpr int qfrag_off(int r, int s) {
  return ((((s >> 5) * 4 + (r >> 4)) * 64 + 16 * ((s & 15) >> 2) + (r & 15)) * 8 + 4 * ((s & 31) >> 4)) * 2;
}
static_assert(qfrag_off(0, 0) == 0 && qfrag_off(16, 0) == 64 * 16 && qfrag_off(0, 32) == 4 * 64 * 16 &&
                  qfrag_off(63, 124) == (15 * 64 + 63) * 16 + 8,
              "fragment packing");
namespace mp {
constexpr int REC_BYTES = sizeof(RecImage);
constexpr int QK_BYTES = sizeof(QKImage);
}  // namespace mp

// Workspace: [status word, 256 bytes] [chunk offsets (N+1) int32, 256-aligned] [records: Hv x maxch]
// [q/k images: Hk x maxch] ...
struct WsLayout {
  static constexpr size_t OFF = 256;  // chunk offsets; the status word sits at byte 0
  static constexpr size_t SINK = 64;  // 64 bytes of the header that stores may hit and nothing reads
  size_t rec, qk, bytes;
  size_t mid;  // calls in stages: the states carried between the stages
  // whole-layer call only: per (sequence, value head) RING chunk slots, each with one 64-bit
  // (chunk tag, partial sum of squares) word per output row and workgroup of the head; the
  // workgroup role counters of the stages (all zeroed by the first stage's prep)
  size_t ring, tick, layer_bytes;
  __host__ __device__ WsLayout(int num_seqs, int hv, int hk, int64_t maxch) {
    rec = (OFF + 4 * (size_t)(num_seqs + 1) + 255) & ~size_t(255);
    qk = rec + (size_t)hv * (size_t)maxch * mp::REC_BYTES;
    mid = qk + (size_t)hk * (size_t)maxch * mp::QK_BYTES;
    bytes = mid + (size_t)num_seqs * hv * mp::D * mp::D * 4;
    ring = (bytes + 255) & ~size_t(255);
    tick = ring + (size_t)num_seqs * hv * mp::RING * mp::NB * mp::C * 8;
    layer_bytes = tick + 256;
  }
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
__host__ __device__ inline const int32_t* ws_offsets(const void* ws) {
  return reinterpret_cast<const int32_t*>(static_cast<const unsigned char*>(ws) + WsLayout::OFF);
}

// Status word of the workspace (byte 0): sticky bits, cleared by the first launch of every call
// (the chunk offsets), set with an atomic OR where a bounded wait gives up or an operand leaves
// the fp16 range of the matrix-core path.  The host reads it after the call
// (agnes_gdn_workspace_status); the bit values are the AGNES_WS_* constants of the header.
namespace wsbits {
constexpr unsigned WAIT_LDS = 1u;       // a wait for another wave of the workgroup gave up
constexpr unsigned WAIT_EXCHANGE = 2u;  // a wait for another workgroup's partial sums gave up
constexpr unsigned WAIT_ROLE = 4u;      // a workgroup found no role to claim and did nothing
constexpr unsigned RANGE = 8u;          // an fp16 operand or the final state left +-65504 / was not finite
}  // namespace wsbits
__device__ __forceinline__ void ws_report(void* ws, unsigned bits) {
  __hip_atomic_fetch_or(static_cast<unsigned*>(ws), bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Poll bound of a wait: the caller's limit (tests force waits to give up with a small one), else
// the wait's own default.
__device__ __forceinline__ int wait_bound(unsigned limit, int def) {
  return limit && limit < (unsigned)def ? (int)limit : def;
}
// fp16 range of a value about to become a matrix-core operand.
__device__ __forceinline__ bool fp16_range(float v) { return __builtin_fabsf(v) <= 65504.f; }
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

// Workgroup barrier ordering LDS only: global stores issued before it may still be in flight
// (a full __syncthreads would wait for them).  Direct global -> LDS copies are not covered:
// the issuing wave waits for them (s_waitcnt) before the barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Barrier of the copy waves of the fused scan, which order their own LDS traffic with explicit
// waits (the direct copies that must land before the barrier, and the conv's LDS accesses, which
// wait for themselves): a workgroup release fence here would make the compiler wait for every
// direct copy in flight, the raw rows of the chunk after next included.
__device__ __forceinline__ void copy_barrier() { __builtin_amdgcn_s_barrier(); }

// ---------------------------------------------------------------- 1. chunk offsets
__global__ __launch_bounds__(256) void chunk_offsets_kernel(const int32_t* cu, int num_seqs, int64_t total,
                                                            int32_t* off, unsigned* status) {
  if (threadIdx.x == 0) *status = 0u;
  __shared__ int32_t wsum[4];
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int per = (num_seqs + 255) / 256;
  const int lo = t * per < num_seqs ? t * per : num_seqs;
  const int hi = lo + per < num_seqs ? lo + per : num_seqs;
  int32_t sum = 0;
  for (int n = lo; n < hi; ++n) {
    const int64_t s = cu_at(cu, n, total), e = cu_at(cu, n + 1, total);
    sum += e > s ? (int32_t)((e - s + mp::C - 1) / mp::C) : 0;
  }
  // exclusive prefix of the per-thread sums: within each wave by shuffles, then over the waves
  int32_t incl = sum;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int32_t u = __shfl_up(incl, o, 64);
    if (lane >= o) incl += u;
  }
  if (lane == 63) wsum[wv] = incl;
  __syncthreads();
  int32_t run = incl - sum;
  for (int i = 0; i < wv; ++i) run += wsum[i];
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
typedef __bf16 bf8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;

namespace mp {
constexpr int PH = 3;       // value heads per prep workgroup (four waves each)
}

// Lower 16x16 block (i, j), i >= j, of a [chunk, chunk] matrix stored block by block.
__host__ __device__ constexpr int tri(int i, int j) { return i * (i + 1) / 2 + j; }

struct PrepSmem {
  union U {
    struct {
      uint16_t Q[mp::C][mp::LDQ];   // bf16 q rows as stored (rows >= L: copies of row 0); fused: fp16
      uint16_t K[mp::C][mp::LDQ];   // bf16 k rows as stored; fused: fp16
      uint16_t Xq[mp::C + 4][mp::D];  // fused: raw x rows c0 - 3 .. c0 + 64 of the q head (bf16)
      uint16_t Xk[mp::C + 4][mp::D];  // fused: the same for the k head
    } qk;                           // until the Gram products are done
    struct Head {
      float A[10][16][17];          // lower blocks of A, fp32
      float X[10][16][17];          // lower blocks of X = (I + A)^-1, fp32
    } hd[mp::PH];
  } u;
  float gam[mp::PH][mp::C], bet[mp::PH][mp::C];
};

// Lower 16x16 block pair p = 0..9 -> (bi, bj), bi >= bj: (0,0) (1,0) (1,1) (2,0) (2,1) ...
__device__ __forceinline__ void pair_of(int p, int& bi, int& bj) {
  bi = 0;
  while (p > bi) {
    p -= bi + 1;
    ++bi;
  }
  bj = p;
}

__device__ __forceinline__ f4 mfma_bf(bf8 a, bf8 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f4 mfma_f32(float a, float b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// z + A_ik X_kj on fp32 matrix cores (four 16x16x4 steps; lane (m, g) of step s holds
// A[m][4s+g] and X[4s+g][m]).
__device__ __forceinline__ f4 blk_ax(const PrepSmem::U::Head& hd, int i, int k, int j, int ln, int lg, f4 z) {
  float av[4], xv[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    av[s] = hd.A[tri(i, k)][ln][4 * s + lg];
    xv[s] = hd.X[tri(k, j)][4 * s + lg][ln];
  }
#pragma unroll
  for (int s = 0; s < 4; ++s) z = mfma_f32(av[s], xv[s], z);
  return z;
}
// -X_ii z with z in result layout (lane (n, g) holds z[4g+e][n]): step s contracts over the
// rows 4g+s of z, which are the lanes' own element s.
__device__ __forceinline__ f4 blk_xz(const PrepSmem::U::Head& hd, int i, int ln, int lg, f4 z) {
  f4 r = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 4; ++s) r = mfma_f32(-hd.X[tri(i, i)][ln][4 * lg + s], z[s], r);
  return r;
}

// One workgroup per (chunk, key group, round of up to PH value heads of the group): the q/k
// rows, the Gram products and the fp16 q/k image are shared; each value head of the round
// has four waves of its own for the decay-scaled A, P and X.
template <bool FUSED>
__global__ __launch_bounds__(256 * mp::PH) __attribute__((amdgpu_waves_per_eu(6))) void prep_kernel(PrefillArgs a, int64_t maxch) {
  using namespace mp;
  __shared__ PrepSmem sm;
  const int32_t* off = ws_offsets(a.workspace);
  const WsLayout ws(a.num_seqs, a.hv, a.hk, maxch);
  unsigned char* base = static_cast<unsigned char*>(a.workspace);
  const int grp = a.hv / a.hk;
  const unsigned rounds = (unsigned)((grp + PH - 1) / PH);
  const unsigned nblk = gridDim.x;
  unsigned lid = blockIdx.x;
  if ((nblk & 7u) == 0) lid = (blockIdx.x & 7u) * (nblk >> 3) + (blockIdx.x >> 3);
  const int rd = (int)(lid % rounds);
  const int j = (int)((lid / rounds) % (unsigned)maxch);
  const int kh = (int)(lid / (rounds * (unsigned)maxch));
  if (a.layer && a.part_lo == 0) {  // whole-layer call, first stage: no partial sum published yet
    // (tag 0 matches no chunk), no ticket taken
    uint4* r = reinterpret_cast<uint4*>(base + ws.ring);
    const size_t n16 = (ws.layer_bytes - ws.ring) / 16;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (size_t)nblk * blockDim.x)
      r[i] = make_uint4(0u, 0u, 0u, 0u);
  }
  if (j >= off[a.num_seqs]) return;
  const int n = seq_of_chunk(off, a.num_seqs, j);
  if (a.part_den > 1) {  // a stage of the whole-layer call: its chunk range only
    const int ncs = off[n + 1] - off[n], jl = j - off[n];
    if (jl < (int)((int64_t)ncs * a.part_lo / a.part_den) || jl >= (int)((int64_t)ncs * a.part_hi / a.part_den)) return;
  }
  const int64_t start = cu_at(a.cu, n, a.total);
  const int64_t c0 = start + (int64_t)(j - off[n]) * C;
  const int64_t end = cu_at(a.cu, n + 1, a.total);
  const int L = (int)((end - c0) < C ? (end - c0) : C);
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, ln = lane & 15, lg = lane >> 4;
  const int slot = w >> 2, v = w & 3, ts = tid & 255;
  const int z = rd * PH + slot;
  bool bad = false;  // a value that leaves the fp16 range on its way to the matrix cores
  const bool act = z < grp;
  const int h = kh * grp + (act ? z : 0);
  unsigned char* rec = base + ws.rec + ((size_t)h * maxch + j) * REC_BYTES;
  PrepSmem::U::Head& hd = sm.u.hd[slot];
  // The gates of the chunk (one value head per four waves), requested before the row copies.
  float gv = 0.f, bv = 0.f;
  if (v == 0 && act) {
    gv = lane < L ? a.g[(c0 + lane) * a.hv + h] : 0.f;
    bv = lane < L ? a.beta[(c0 + lane) * a.hv + h] : 0.f;
  }
  // Fused prologue: the conv taps and bias of this thread's 8 channels of the conv pass below,
  // requested first so that their latency overlaps the row copies.
  uint4 cw[4] = {}, cb = make_uint4(0, 0, 0, 0);
  if constexpr (FUSED) {
    const int ch = (((tid >> 4) & 1) ? a.hk + kh : kh) * D + 8 * (tid & 15);
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) cw[q4] = load_raw8<DT_BF16>(a.conv_w, (int64_t)ch * 4 + 8 * q4).u[0];
    if (a.conv_b) cb = load_raw8<DT_BF16>(a.conv_b, ch).u[0];
  }

  if constexpr (FUSED) {
    // ---- raw x rows c0 - 3 .. c0 + 64 of the q and k heads -> LDS (direct copies, 17 x 1 KiB
    // per head); rows outside the sequence re-read row c0 (the halo before the sequence start is
    // taken from the conv history in the conv pass below).
    const uint16_t* xq = static_cast<const uint16_t*>(a.q) + (int64_t)kh * D;  // a.q: channel 0 of x
    const uint16_t* xk = static_cast<const uint16_t*>(a.k) + (int64_t)kh * D;
#pragma unroll
    for (int t = 0; t < (34 + 4 * PH - 1) / (4 * PH); ++t) {
      const int i = w + 4 * PH * t;
      if (i >= 34) break;
      const int ii = i < 17 ? i : i - 17;
      const int jj = 64 * ii + lane, row = jj >> 4, pc = jj & 15;
      const int64_t pos = c0 - 3 + row;
      const int64_t o = (pos >= start && row < 3 + L ? pos : c0) * a.qk_stride + 8 * pc;
      uint16_t* dst = (i < 17 ? &sm.u.qk.Xq[0][0] : &sm.u.qk.Xk[0][0]) + 512 * ii;
      __builtin_amdgcn_global_load_lds((glb_void*)((i < 17 ? xq : xk) + o), (lds_void*)dst, 16, 0, 0);
    }
  } else {
    // ---- q, k rows of the chunk -> LDS (direct copies, 17 x 1 KiB per matrix, spread over
    // the waves; the 17th 16-byte piece of a row is padding and re-reads the row's start)
    constexpr int QPR = LDQ / 8;
    const uint16_t* qb = static_cast<const uint16_t*>(a.q) + c0 * a.qk_stride + (int64_t)kh * D;
    const uint16_t* kb = static_cast<const uint16_t*>(a.k) + c0 * a.qk_stride + (int64_t)kh * D;
#pragma unroll
    for (int t = 0; t < (2 * QPR + 4 * PH - 1) / (4 * PH); ++t) {
      const int i = w + 4 * PH * t;
      if (i >= 2 * QPR) break;
      const int ii = i < QPR ? i : i - QPR;
      const int jj = 64 * ii + lane, r = jj / QPR, pc = jj % QPR;
      const int64_t o = (int64_t)(r < L ? r : 0) * a.qk_stride + (pc < D / 8 ? 8 * pc : 0);
      const uint16_t* src = (i < QPR ? qb : kb) + o;
      uint16_t* dst = (i < QPR ? &sm.u.qk.Q[0][0] : &sm.u.qk.K[0][0]) + 512 * ii;
      __builtin_amdgcn_global_load_lds((glb_void*)src, (lds_void*)dst, 16, 0, 0);
    }
  }
  // gates: inclusive prefix sum of log-decays (loaded at the top); rows >= L get g = beta = 0.
  // The record's copy is stored after the barrier so that the wait below covers loads only.
  if (v == 0 && act) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float t = __shfl_up(gv, o, 64);
      if (lane >= o) gv += t;
    }
    sm.gam[slot][lane] = gv;
    sm.bet[slot][lane] = bv;
  }
  __builtin_amdgcn_s_waitcnt(0);
  lds_barrier();
  if constexpr (FUSED) {
    // ---- conv + SiLU + L2 of the staged rows, fp16 into Q / K (rows >= L zero).  Thread
    // (row group rr, head hs, 8 channels col) takes rows rr, rr + 24, rr + 48; the 16 lanes of a
    // (row, head) are consecutive, so the L2 norm is a 16-lane sum.
    const int col = tid & 15, hs = (tid >> 4) & 1, rr = tid >> 5;
    const int Ctot = (2 * a.hk + a.hv) * D;
    const int ch = (hs ? a.hk + kh : kh) * D + 8 * col;
    float bs[8];
    {
      Raw8<DT_BF16> br;
      br.u[0] = cb;
      widen8<DT_BF16>(br, bs);
    }
    const uint16_t (*X)[D] = hs ? sm.u.qk.Xk : sm.u.qk.Xq;
    const uint16_t* hist = static_cast<const uint16_t*>(a.conv_hist);
    // the first round of a key group also writes the fp16 q/k image, straight from the conv
    QKImage* img = reinterpret_cast<QKImage*>(base + ws.qk + ((size_t)kh * maxch + j) * QK_BYTES);
    const bool head = c0 - 3 < start;  // the sequence's first chunk: the halo is the history
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      const int r = rr + 24 * k;
      if (r >= C) break;
      uint4 xr[4];
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) xr[jt] = *reinterpret_cast<const uint4*>(&X[r + jt][8 * col]);
      if (head) {
#pragma unroll
        for (int jt = 0; jt < 3; ++jt) {
          const int i = r + jt;  // staged row i = x row c0 - 3 + i
          if (c0 - 3 + i < start) {  // before the sequence start: history entry i (oldest first)
            const uint16_t* hp = hist + ((int64_t)n * Ctot + ch) * 3 + i;
            xr[jt] = hist ? make_uint4(hp[0] | (uint32_t)hp[3] << 16, hp[6] | (uint32_t)hp[9] << 16,
                                       hp[12] | (uint32_t)hp[15] << 16, hp[18] | (uint32_t)hp[21] << 16)
                          : make_uint4(0, 0, 0, 0);
          }
        }
      }
      float y[8], ss = 0.f;
      conv4_bf16x8(xr, cw, bs, y);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        y[e] = silu(y[e]);
        ss = fmaf(y[e], y[e], ss);
      }
      ss = sum16_dpp(ss);
      const float rs = rsqrt_fast(ss + a.l2_eps);
      h8 hv;
#pragma unroll
      for (int e = 0; e < 8; ++e) hv[e] = r < L ? (_Float16)(y[e] * rs) : (_Float16)0.f;
      *reinterpret_cast<h8*>(hs ? &sm.u.qk.K[r][8 * col] : &sm.u.qk.Q[r][8 * col]) = hv;
      if (rd == 0) {
        if (hs) {
          *reinterpret_cast<h8*>(&img->K[r][8 * col]) = hv;
        } else {
          unsigned char* qb = reinterpret_cast<unsigned char*>(img->Q);
          *reinterpret_cast<h4*>(qb + qfrag_off(r, 8 * col)) = h4{hv[0], hv[1], hv[2], hv[3]};
          *reinterpret_cast<h4*>(qb + qfrag_off(r, 8 * col + 4)) = h4{hv[4], hv[5], hv[6], hv[7]};
        }
      }
    }
    lds_barrier();
  }
  if (v == 0 && act) {
    float* gr = reinterpret_cast<float*>(rec + offsetof(RecImage, gt));
    gr[lane] = bv;
    gr[64 + lane] = __expf(gv);
    gr[128 + lane] = __expf(__shfl(gv, 63, 64) - gv);
  }

  // ---- Gram blocks K K^T and Q K^T (bf16 matrix cores): wave w < 10 takes lower block pair w.
  // The first round of a key group of the plain call also writes the fp16 q/k image (rows >= L zero).
  f4 gk = {0.f, 0.f, 0.f, 0.f}, gq = gk;
  int bi = 0, bj = 0;
  if (w < 10) {
    pair_of(w, bi, bj);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int col = 32 * ks + 8 * lg;
      // gq is the transpose, K_bj Q_bi^T, so that a lane holds four consecutive columns of a row
      // of P (one 8-byte store per head below)
      if constexpr (FUSED) {  // fp16 rows
        const h8 kbv = *reinterpret_cast<const h8*>(&sm.u.qk.K[16 * bj + ln][col]);
        gk = mfma_16x16x32(*reinterpret_cast<const h8*>(&sm.u.qk.K[16 * bi + ln][col]), kbv, gk);
        gq = mfma_16x16x32(kbv, *reinterpret_cast<const h8*>(&sm.u.qk.Q[16 * bi + ln][col]), gq);
      } else {
        const bf8 kbv = *reinterpret_cast<const bf8*>(&sm.u.qk.K[16 * bj + ln][col]);
        gk = mfma_bf(*reinterpret_cast<const bf8*>(&sm.u.qk.K[16 * bi + ln][col]), kbv, gk);
        gq = mfma_bf(kbv, *reinterpret_cast<const bf8*>(&sm.u.qk.Q[16 * bi + ln][col]), gq);
      }
    }
  }
  if (!FUSED && rd == 0) {  // the fp16 q/k image of the plain call (the fused one wrote it in the conv)
    QKImage* img = reinterpret_cast<QKImage*>(base + ws.qk + ((size_t)kh * maxch + j) * QK_BYTES);
    for (int i = tid; i < 2 * C * (D / 8); i += 256 * PH) {
      const bool isk = i >= C * (D / 8);
      const int r = (i >> 4) & (C - 1), col = 8 * (i & 15);
      const uint4 u = *reinterpret_cast<const uint4*>(isk ? &sm.u.qk.K[r][col] : &sm.u.qk.Q[r][col]);
      if (r < L) {  // bf16 magnitudes from 65536 up (0x4780) do not fit fp16
        const uint32_t wv[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) bad |= (wv[e] & 0x7fffu) >= 0x4780u || ((wv[e] >> 16) & 0x7fffu) >= 0x4780u;
      }
      const h8 hv = cvt8(r < L ? u : make_uint4(0, 0, 0, 0));
      if (isk) {
        *reinterpret_cast<h8*>(&img->K[r][col]) = hv;
      } else {
        unsigned char* qb = reinterpret_cast<unsigned char*>(img->Q);
        *reinterpret_cast<h4*>(qb + qfrag_off(r, col)) = h4{hv[0], hv[1], hv[2], hv[3]};
        *reinterpret_cast<h4*>(qb + qfrag_off(r, col + 4)) = h4{hv[4], hv[5], hv[6], hv[7]};
      }
    }
  }
  lds_barrier();  // q/k rows are dead from here

  // ---- per value head of the round, straight from the Gram fragments of block pair (bi, bj):
  // A (fp32, LDS) and P (fp16, record, zero above the diagonal).  Waves 10, 11 write the two
  // blocks of P above the diagonal that the scan reads, (0,1) and (2,3), as zeros.
  if (w < 10) {
    const int s2 = 16 * bj + ln, r0 = 16 * bi + 4 * lg;  // gk: rows r0 + e, column s2
    const int pr = 16 * bi + ln, ps = 16 * bj + 4 * lg;  // gq: row pr, columns ps + e
#pragma unroll
    for (int zz = 0; zz < PH; ++zz) {
      if (rd * PH + zz >= grp) break;
      const int hz = kh * grp + rd * PH + zz;
      unsigned char* rz = base + ws.rec + ((size_t)hz * maxch + j) * REC_BYTES;
      const f4 gr = *reinterpret_cast<const f4*>(&sm.gam[zz][r0]);
      const f4 br = *reinterpret_cast<const f4*>(&sm.bet[zz][r0]);
      const float gs = sm.gam[zz][s2];
      const float gpr = sm.gam[zz][pr];
      const f4 gps = *reinterpret_cast<const f4*>(&sm.gam[zz][ps]);
      h4 pv4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = r0 + e;
        const float d = s2 < r ? __expf(gr[e] - gs) : 0.f;
        sm.u.hd[zz].A[w][4 * lg + e][ln] = br[e] * d * gk[e];
        const float pv = ps + e <= pr ? __expf(gpr - gps[e]) * gq[e] : 0.f;
        bad |= !fp16_range(pv);
        pv4[e] = (_Float16)pv;
      }
      *reinterpret_cast<h4*>(rz + offsetof(RecImage, P) + frag_off(pr, ps)) = pv4;
    }
  } else {
    for (int i = tid - 640; i < PH * 2 * 64; i += 128) {  // (head, block, lane): the lane's upper half
      const int zz = i >> 7, blk = (i >> 6) & 1, l = i & 63;
      if (rd * PH + zz < grp) {
        const int hz = kh * grp + rd * PH + zz;
        unsigned char* rz = base + ws.rec + ((size_t)hz * maxch + j) * REC_BYTES;
        *reinterpret_cast<uint2*>(rz + offsetof(RecImage, P) + frag_off(32 * blk + (l & 15), 16 + 32 * blk + 4 * (l >> 4))) =
            make_uint2(0, 0);
      }
    }
  }
  lds_barrier();
  if (v == 0 && act) {  // diagonal blocks X_bb = (I + A_bb)^-1: block lg, column ln, right-looking
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) x[r] = r == ln ? 1.f : 0.f;
    const int tb = tri(lg, lg);
#pragma unroll
    for (int s2 = 0; s2 < 16; ++s2)
#pragma unroll
      for (int r = s2 + 1; r < 16; ++r) x[r] = fmaf(-hd.A[tb][r][s2], x[s2], x[r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) hd.X[tb][r][ln] = x[r];
  }
  lds_barrier();
  // off-diagonal blocks by levels d = i - j: X_ij = -X_ii sum_{k=j}^{i-1} A_ik X_kj (fp32)
  const f4 zf = {0.f, 0.f, 0.f, 0.f};
  if (v < 3 && act) {  // d = 1: blocks (v+1, v)
    const int i = v + 1;
    const f4 x = blk_xz(hd, i, ln, lg, blk_ax(hd, i, v, v, ln, lg, zf));
#pragma unroll
    for (int e = 0; e < 4; ++e) hd.X[tri(i, v)][4 * lg + e][ln] = x[e];
  }
  lds_barrier();
  if (v < 2 && act) {  // d = 2: blocks (v+2, v)
    const int i = v + 2;
    f4 zz = blk_ax(hd, i, v, v, ln, lg, zf);
    zz = blk_ax(hd, i, v + 1, v, ln, lg, zz);
    const f4 x = blk_xz(hd, i, ln, lg, zz);
#pragma unroll
    for (int e = 0; e < 4; ++e) hd.X[tri(i, v)][4 * lg + e][ln] = x[e];
  }
  lds_barrier();
  if (v == 0 && act) {  // d = 3: block (3, 0)
    f4 zz = blk_ax(hd, 3, 0, 0, ln, lg, zf);
    zz = blk_ax(hd, 3, 1, 0, ln, lg, zz);
    zz = blk_ax(hd, 3, 2, 0, ln, lg, zz);
    const f4 x = blk_xz(hd, 3, ln, lg, zz);
#pragma unroll
    for (int e = 0; e < 4; ++e) hd.X[tri(3, 0)][4 * lg + e][ln] = x[e];
  }
  lds_barrier();
  // X -> record (fp16 fragments, zero above the diagonal): item t is lane t % 64 of fragment t / 64
  if (act) {
    for (int t = ts; t < 6 * 64; t += 256) {
      const int f = t >> 6, g = (t >> 4) & 3, bi = f < 4 ? f : f - 2, r = 16 * bi + (t & 15);
      h8 xv;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int s0 = (f < 4 ? 0 : 32) + 16 * hh + 4 * g, bj = s0 >> 4;
        const float* xr = &hd.X[bj <= bi ? tri(bi, bj) : 0][r & 15][s0 & 15];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float xe = s0 + e <= r ? xr[e] : 0.f;
          bad |= !fp16_range(xe);
          xv[4 * hh + e] = (_Float16)xe;
        }
      }
      *reinterpret_cast<h8*>(rec + offsetof(RecImage, X) + 16 * t) = xv;
    }
  }
  if (__any(bad) && lane == 0) ws_report(a.workspace, wsbits::RANGE);
}

// ---------------------------------------------------------------- 3. scan
struct ScanBuf {            // one chunk, filled by direct global -> LDS copies
  QKImage QK;                    // fp16 q, k rows of the key group
  RecImage R;                    // prep record of (chunk, value head)
  uint16_t Vs[mp::C][mp::LDV];   // bf16 v slice [row][value col]
};
// Hand-over from the chain wave of a value tile to its output wave (lane-major 16-byte
// pieces): the fp16 operands of S^T entering a chunk and of U.
struct ExBuf {
  h8 s[mp::NVT][4][64];
  h8 u[mp::NVT][2][64];
};
struct ScanSmem {
  ScanBuf B[2];                      // by chunk parity
  float Os[mp::C][mp::DVB + 4];      // output tile staging of the output wave
  ExBuf X[2];                        // by chunk parity
  uint16_t Vr[2][mp::VR_ROWS][mp::DVB];  // fused prologue: raw x rows of the V slice, by chunk parity
  int ks_done[mp::NVT];              // c + 1 once chain wave p's K S^T of chunk c is done
  int os_ready;                      // whole-layer call: (output waves) x (c + 1) once chunk c's tile is in Os
  unsigned ticket;                   // whole-layer call: this workgroup's place in start order
};
static_assert(sizeof(ScanSmem) <= 160 * 1024, "scan LDS");

struct Geo {
  int64_t start, end;  // rows of this launch's chunks (a stage: the chunk range only)
  int64_t hstart;      // the sequence's first row: the conv reads the history before it
  int cbase;           // the sequence's chunk index of local chunk 0 (stages)
  int nchunks, h, kh, dv0, w, lane, ln, lg;
  int64_t sbase;
  size_t rec0;  // workspace byte offset of this sequence's first record for value head h
  size_t qk0;   // workspace byte offset of this sequence's first q/k image for key group kh
  __device__ int len(int c) const {
    const int64_t r = end - start - (int64_t)c * mp::C;
    return (int)(r < mp::C ? r : mp::C);
  }
};

// Transposing read of 4 bf16 values (same lane pattern as lds_tr4), widened to fp32.
__device__ __forceinline__ f4 lds_tr4_bf16(const uint16_t* p) {
  const s4v v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4v*)(p));
  const uint2 u = __builtin_bit_cast(uint2, v);
  return f4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
            __uint_as_float(u.y & 0xffff0000u)};
}

// K^T operand of the state update for key tile kt, token half ks (see lds_tr4).
__device__ __forceinline__ h8 kt_operand(const ScanBuf& B, int kt, int ks, int trow, int tcol) {
  return cat(lds_tr4(&B.QK.K[32 * ks + trow][16 * kt + tcol]), lds_tr4(&B.QK.K[32 * ks + 16 + trow][16 * kt + tcol]));
}

// Bounded wait for an LDS flag that another wave of the workgroup raises, with relaxed loads.
// ks_done only orders work in time (its data hand-over goes through a barrier); os_ready hands
// over the staged output tile, so its writer releases (workgroup scope, LDS) before raising it
// and its readers acquire after the wait.  The bound (never reached when the flag works) keeps
// a broken one from hanging the GPU.
__device__ __forceinline__ void wait_flag(const int* f, int target, const PrefillArgs& a) {
  const int n = wait_bound(a.wait_limit, 1 << 20);
  for (int i = 0; i < n; ++i) {
    if (__hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) >= target) return;
    __builtin_amdgcn_s_sleep(1);
  }
  if ((threadIdx.x & 63) == 0) ws_report(a.workspace, wsbits::WAIT_LDS);
}

// Gates of the rows a lane holds in result layout (rows 16i + 4g + e of tile i, e = 0..3):
// four 16-byte LDS reads of a [64] gate row.
__device__ __forceinline__ void gate_rows16(const float* gt, int lg, float (&o)[16]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f4 v = *reinterpret_cast<const f4*>(gt + 16 * i + 4 * lg);
    o[4 * i] = v[0]; o[4 * i + 1] = v[1]; o[4 * i + 2] = v[2]; o[4 * i + 3] = v[3];
  }
}

// Raw transposing read of 4 bf16 values (see lds_tr4); widened later by bf16x4_to_f4.
__device__ __forceinline__ uint2 lds_tr4_raw(const uint16_t* p) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4v*)(p)));
}
__device__ __forceinline__ f4 h4_to_f4(h4 v) { return f4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]}; }
__device__ __forceinline__ f4 bf16x4_to_f4(uint2 u) {
  return f4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
            __uint_as_float(u.y & 0xffff0000u)};
}

// Chain wave on the chunk in buffer B, for its TPW value tiles t0 .. t0 + TPW - 1 (every LDS
// operand feeds one product per tile): K S^T, R' = beta (V - exp(gamma) K S^T), U = X R', and
// the state update S^T <- exp(gamma_63) S^T + K^T diag(exp(gamma_63 - gamma)) U.  sb holds the
// fp16 B operands of S^T entering the chunk and leaves with those of the next chunk; U goes to
// exU and the next chunk's S^T operands to exS for the output wave.  38 products of 16x16x32
// per tile.
// The wave issues in order, so the code is laid out by hand: operands are read a step ahead,
// and the results of a product are first used several products later.
template <int TPW, bool VF16>
__device__ __forceinline__ void chain_step(const ScanBuf& B, ExBuf& exU, ExBuf& exS, int t0, int lane, int ln, int lg,
                                           f4 (&sacc)[TPW][8], h8 (&sb)[TPW][4], int* ks_done, int c) {
  using namespace mp;
  const RecImage& R = B.R;
  const f4 zero = {0.f, 0.f, 0.f, 0.f};
  const int trow = 4 * lg + (ln >> 2), tcol = 4 * (ln & 3);
  h8 ka[2][4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) ka[0][rt] = a_perm(&B.QK.K[16 * rt + ln][0], 0, lg);
  const float dec = R.gt[1][C - 1];
  f4 kq[TPW][4];
#pragma unroll
  for (int t = 0; t < TPW; ++t)
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) kq[t][rt] = zero;
  __builtin_amdgcn_sched_barrier(0);
  // K S^T; alongside, the V slices, X operands and the decay of the state (sacc is not an
  // operand until the update: the products use the fp16 copy sb)
  h8 xa[6];
  uint2 vr[TPW][4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    if (ks < 3) {
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) ka[(ks + 1) & 1][rt] = a_perm(&B.QK.K[16 * rt + ln][0], 32 * (ks + 1), lg);
    }
    if (ks == 1) {
#pragma unroll
      for (int t = 0; t < TPW; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) vr[t][i] = lds_tr4_raw(&B.Vs[16 * i + 4 * lg + (ln >> 2)][16 * (t0 + t) + 4 * (ln & 3)]);
    }
    if (ks == 2) {
#pragma unroll
      for (int i = 0; i < 6; ++i) xa[i] = R.X[i][lane];
    }
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int t = 0; t < TPW; ++t) kq[t][rt] = mfma_16x16x32(ka[ks & 1][rt], sb[t][ks], kq[t][rt]);
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sacc[t][2 * ks][e] *= dec;
        sacc[t][2 * ks + 1][e] *= dec;
      }
    __builtin_amdgcn_sched_barrier(0);
  }
  // the LDS-heavy start of the chunk is over: let the output wave begin (a timing hint only)
  if (lane == 0) __hip_atomic_store(ks_done, c + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  // K^T operands of the first two key tiles, then R' and U for both tiles
  h8 kta[2][2];
  kta[0][0] = kt_operand(B, 0, 0, trow, tcol);
  kta[0][1] = kt_operand(B, 0, 1, trow, tcol);
  float bb[16], gg[16];
  gate_rows16(R.gt[0], lg, bb);
  gate_rows16(R.gt[1], lg, gg);
  h8 rb[TPW][2];
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    f4 rp[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f4 vv = VF16 ? h4_to_f4(__builtin_bit_cast(h4, vr[t][i])) : bf16x4_to_f4(vr[t][i]);
#pragma unroll
      for (int e = 0; e < 4; ++e) rp[i][e] = bb[4 * i + e] * (vv[e] - gg[4 * i + e] * kq[t][i][e]);
    }
    rb[t][0] = b_pair(rp[0], rp[1]);
    rb[t][1] = b_pair(rp[2], rp[3]);
  }
  f4 u[TPW][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int t = 0; t < TPW; ++t) u[t][i] = mfma_16x16x32(xa[i], rb[t][0], zero);
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    u[t][2] = mfma_16x16x32(xa[4], rb[t][1], u[t][2]);
    u[t][3] = mfma_16x16x32(xa[5], rb[t][1], u[t][3]);
  }
  kta[1][0] = kt_operand(B, 1, 0, trow, tcol);
  kta[1][1] = kt_operand(B, 1, 1, trow, tcol);
  float ll[16];
  gate_rows16(R.gt[2], lg, ll);
  __builtin_amdgcn_sched_barrier(0);
  h8 db[TPW][2];
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    f4 ud[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) ud[i][e] = u[t][i][e] * ll[4 * i + e];
    db[t][0] = b_pair(ud[0], ud[1]);
    db[t][1] = b_pair(ud[2], ud[3]);
  }
  __builtin_amdgcn_sched_barrier(0);
  // state update, K^T operands two key tiles ahead; the hand-over of U meanwhile
#pragma unroll
  for (int kt = 0; kt < 8; ++kt) {
    h8 n0, n1;
    if (kt < 6) {
      n0 = kt_operand(B, kt + 2, 0, trow, tcol);
      n1 = kt_operand(B, kt + 2, 1, trow, tcol);
    }
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      sacc[t][kt] = mfma_16x16x32(kta[kt & 1][0], db[t][0], sacc[t][kt]);
      sacc[t][kt] = mfma_16x16x32(kta[kt & 1][1], db[t][1], sacc[t][kt]);
    }
    if (kt == 1) {
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        exU.u[t0 + t][0][lane] = b_pair(u[t][0], u[t][1]);
        exU.u[t0 + t][1][lane] = b_pair(u[t][2], u[t][3]);
      }
    }
    if (kt < 6) {
      kta[kt & 1][0] = n0;
      kta[kt & 1][1] = n1;
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  // fp16 operands of the new state for the next chunk (and the output wave)
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      sb[t][ks] = b_pair(sacc[t][2 * ks], sacc[t][2 * ks + 1]);
      exS.s[t0 + t][ks][lane] = sb[t][ks];
    }
}

// Output wave, part 1 (chunk c in buffer B, value tiles t0 .. t0 + TPW - 1): Q S^T with the S^T
// operands the chain wave handed over, and the operands of P and the gates exp(gamma) kept for
// part 2.
template <int TPW>
__device__ __forceinline__ void qs_step(const ScanBuf& B, const ExBuf& exS, int t0, int lane, int ln, int lg,
                                        f4 (&qs)[TPW][4], h8 (&pa)[6], float (&ge)[16]) {
  using namespace mp;
  const f4 zero = {0.f, 0.f, 0.f, 0.f};
  h8 sb[TPW][4];
#pragma unroll
  for (int t = 0; t < TPW; ++t)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) sb[t][ks] = exS.s[t0 + t][ks][lane];
  h8 qa[2][4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) qa[0][rt] = B.QK.Q[rt][lane];
#pragma unroll
  for (int t = 0; t < TPW; ++t)
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) qs[t][rt] = zero;
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    if (ks < 3) {
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) qa[(ks + 1) & 1][rt] = B.QK.Q[4 * (ks + 1) + rt][lane];
    } else {
#pragma unroll
      for (int i = 0; i < 6; ++i) pa[i] = B.R.P[i][lane];
      gate_rows16(B.R.gt[1], lg, ge);
    }
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int t = 0; t < TPW; ++t) qs[t][rt] = mfma_16x16x32(qa[ks & 1][rt], sb[t][ks], qs[t][rt]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Output wave, part 2 (the chunk c of part 1, one iteration later): O = diag(exp gamma) Q S^T
// + P U for its tiles, staged in their columns of Os by this wave and written out from there
// (rows < L, 2 TPW lanes per row, eight values each).
template <int TPW, int O_DT, bool STAGE>
__device__ __forceinline__ void o_step(const ExBuf& exU, float (*Os)[mp::DVB + 4], int* os_ready, const PrefillArgs& a,
                                       const Geo& G, int c, int t0, const f4 (&qs)[TPW][4], const h8 (&pa)[6],
                                       const float (&gg)[16]) {
  using namespace mp;
  const int lane = G.lane, ln = G.ln, lg = G.lg;
  // All products first, then all stores: each result is used only after every product has
  // been issued, and the staging reads are unconditional, so nothing waits on one latency at
  // a time.
  h8 ub[TPW][2];
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    ub[t][0] = exU.u[t0 + t][0][lane];
    ub[t][1] = exU.u[t0 + t][1][lane];
  }
  f4 o[TPW][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
#pragma unroll
      for (int e = 0; e < 4; ++e) o[t][i][e] = qs[t][i][e] * gg[4 * i + e];
      o[t][i] = mfma_16x16x32(pa[i], ub[t][0], o[t][i]);
    }
#pragma unroll
  for (int i = 2; i < 4; ++i)
#pragma unroll
    for (int t = 0; t < TPW; ++t) o[t][i] = mfma_16x16x32(pa[i + 2], ub[t][1], o[t][i]);
#pragma unroll
  for (int t = 0; t < TPW; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) Os[16 * i + 4 * lg + e][16 * (t0 + t) + ln] = a.scale * o[t][i][e];
  if constexpr (STAGE) {
    // hand the tile to the tile waves, which write it out: the wave's LDS writes are complete
    // before its count is added (one per chunk from each output wave), and the tile is
    // not rewritten before the next barrier
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    if (lane == 0) __hip_atomic_fetch_add(os_ready, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    return;
  }
  // Os is written and read back by this wave only: LDS keeps a wave's accesses in order.
  constexpr int LPR = 2 * TPW, RPP = 64 / LPR;  // lanes per row, rows per pass
  const int L = G.len(c);
  const int part = lane % LPR, col = 16 * t0 + 8 * part;
  f4 x[C / RPP][2];
#pragma unroll
  for (int rg = 0; rg < C / RPP; ++rg) {
    const int r = RPP * rg + lane / LPR;
    x[rg][0] = *reinterpret_cast<const f4*>(&Os[r][col]);
    x[rg][1] = *reinterpret_cast<const f4*>(&Os[r][col + 4]);
  }
#pragma unroll
  for (int rg = 0; rg < C / RPP; ++rg) {
    const int r = RPP * rg + lane / LPR;
    if (r < L) {
      const float v[8] = {x[rg][0][0], x[rg][0][1], x[rg][0][2], x[rg][0][3],
                          x[rg][1][0], x[rg][1][1], x[rg][1][2], x[rg][1][3]};
      store8_nt<O_DT>(a.o, ((G.start + (int64_t)c * C + r) * a.hv + G.h) * (int64_t)D + G.dv0 + col, v);
    }
  }
}

// ---- whole-layer call: gated RMSNorm y = o / sqrt(mean(o^2) + eps) * w * silu(z) of the output
// rows, whose 128 values are spread over the NB workgroups of a value head.  The output wave
// only stages its [64 x DVB] tile in Os and raises os_ready; the first NTW copy waves (tile
// waves, 32 rows each) issue no copies and run the norm.  They are the only waves that store
// rows, and their loads and stores never share a wait counter with the copies: a copy wave
// waiting for its copies never waits on a row store or an exchange load.
//
// Exchange: a row's partial sum of squares over this block's DVB columns travels with its chunk
// tag in one 64-bit word, written and read as a relaxed atomic at agent scope: a reader that
// sees the tag sees the sum stored with it, so no fence (on this chip, a write-back or
// invalidation of a whole L2) is needed.  Chunk c (counted from the sequence start, so that
// the stages of a call never take each other's words) uses slot c mod RING.  In step c a tile wave
// (1) waits for the words of chunk c - 3 (loaded at the end of step c - 1, reloaded while a tag
// is older) and computes y of chunk c - 3; (2) loads the gates of chunk c - 2 and stores y of
// chunk c - 3; (3) takes chunk c - 1 from Os and publishes its sums; (4) loads the words of chunk
// c - 2.  Chunk k is published in step k + 1 and read in
// steps k + 2 .. k + 3; slot k is next written (chunk k + RING) in step k + RING + 1, after the
// writer's wait for chunk k + RING - 2, which every reader publishes in step k + RING - 1 after
// its own read of chunk k (step k + 3): RING >= 4 suffices.  Every wait ends (the workgroups
// take their roles in start order, see the kernel); the bound only keeps a lost word from
// hanging the GPU.
namespace mp {
constexpr int NTW = 2;                  // tile waves
constexpr int TLPR = DVB / 8;           // lanes per row piece (8 values each)
constexpr int TRPP = 64 / TLPR;         // rows per pass of a tile wave
static_assert(TLPR == 4 && TRPP == 16, "tile-wave lane layout");
}  // namespace mp

struct NormCtx {
  unsigned long long* ring;  // this (sequence, value head): [RING][NB][64] tagged words
  int blk;                   // this block
  int r0;                    // first row of this tile wave
  int cbase;                 // the sequence's chunk index of local chunk 0: tags and slots use it
  float w[8];                // norm weights of the lane's 8 columns
  void* sink;                // where the row stores of rows past the chunk end go (see tile_store_y)
};

// The lane's pieces of rows r0 + 16 g + lane / 4 (g < NG) of the staged tile, columns
// 8 (lane % 4) .. + 7.
template <int NG>
__device__ __forceinline__ void tile_take(const float (*Os)[mp::DVB + 4], int r0, int lane, float (&x)[NG][8]) {
  const int col = 8 * (lane % mp::TLPR);
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const int r = r0 + mp::TRPP * g + lane / mp::TLPR;
    const f4 a0 = *reinterpret_cast<const f4*>(&Os[r][col]);
    const f4 a1 = *reinterpret_cast<const f4*>(&Os[r][col + 4]);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[g][e] = a0[e];
      x[g][e + 4] = a1[e];
    }
  }
}

// Row pieces out with non-temporal stores (nothing here reads them back; measured 3 us faster
// on the T = 8192 layer call than plain stores).
template <int O_DT, int NG>
__device__ __forceinline__ void tile_store(void* dst, const PrefillArgs& a, const Geo& G, int c, int r0, int lane,
                                           const float (&x)[NG][8]) {
  const int L = G.len(c), col = 8 * (lane % mp::TLPR);
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const int r = r0 + mp::TRPP * g + lane / mp::TLPR;
    if (r < L) store8_nt<O_DT>(dst, ((G.start + (int64_t)c * mp::C + r) * a.hv + G.h) * (int64_t)mp::D + G.dv0 + col, x[g]);
  }
}

__device__ __forceinline__ unsigned long long* ring_word(const NormCtx& nc_, int c, int b, int r) {
  return nc_.ring + (((c + nc_.cbase) & (mp::RING - 1)) * mp::NB + b) * mp::C + r;
}

// Partial sums of squares of the lane's rows over this block's columns (every lane of a row
// gets the row's sum).
template <int NG>
__device__ __forceinline__ void row_sums(const float (&x)[NG][8], float (&ss)[NG]) {
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    float s2 = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) s2 += x[g][e] * x[g][e];
#pragma unroll
    for (int m = 1; m < mp::TLPR; m <<= 1) s2 += __shfl_xor(s2, m);
    ss[g] = s2;
  }
}

template <int NG>
__device__ __forceinline__ void norm_publish(const NormCtx& nc_, int c, int lane, const float (&ss)[NG]) {
  if (lane % mp::TLPR) return;
#pragma unroll
  for (int g = 0; g < NG; ++g)
    __hip_atomic_store(ring_word(nc_, c, nc_.blk, nc_.r0 + mp::TRPP * g + lane / mp::TLPR),
                       ((unsigned long long)__float_as_uint(ss[g]) << 32) | (unsigned)(c + nc_.cbase + 1), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

// Loads of chunk c for the norm: lane l takes the other blocks' words of row r0 + (l % 32)
// (lanes l and l + 32 alike) and the gates of its own row pieces.
template <int NG>
struct NormIn {
  unsigned long long w[mp::NB - 1];
  uint4 z[NG];
};

template <int NG>
__device__ __forceinline__ void norm_load_words(const NormCtx& nc_, int c, int lane, NormIn<NG>& g) {
  static_assert(NG * mp::TRPP == 32, "a tile wave's rows fit half a wave");
#pragma unroll
  for (int i = 0; i < mp::NB - 1; ++i)
    g.w[i] = __hip_atomic_load(ring_word(nc_, c, i + (i >= nc_.blk), nc_.r0 + (lane & 31)), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
}

template <int NG>
__device__ __forceinline__ void norm_load_z(const NormCtx& nc_, const PrefillArgs& a, const Geo& G, int c, int lane,
                                            NormIn<NG>& g) {
  const int L = G.len(c), col = 8 * (lane % mp::TLPR);
#pragma unroll
  for (int q = 0; q < NG; ++q) {
    const int r = nc_.r0 + mp::TRPP * q + lane / mp::TLPR;
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 zz = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
        static_cast<const uint16_t*>(a.z) + (G.start + (int64_t)c * mp::C + (r < L ? r : 0)) * a.z_stride +
        (int64_t)G.h * mp::D + G.dv0 + col));  // read once: streamed past the cache
    g.z[q] = make_uint4(zz[0], zz[1], zz[2], zz[3]);
  }
}

// An empty use of the exchange loads' registers: the compiler waits for those loads here.  At the
// start of every step this tells it that no load is pending when the step issues the next ones;
// without it, it waits for everything in flight before issuing them (vector memory counts retire
// in order), the row stores of the same step included.
template <int NG>
__device__ __forceinline__ void consume(const NormIn<NG>& g) {
  static_assert(mp::NB - 1 == 3 && NG == 2, "operand list below");
  asm volatile("" ::"v"(g.w[0]), "v"(g.w[1]), "v"(g.w[2]), "v"(g.z[0].x), "v"(g.z[0].y), "v"(g.z[0].z),
               "v"(g.z[0].w), "v"(g.z[1].x), "v"(g.z[1].y), "v"(g.z[1].z), "v"(g.z[1].w));
}

// Waits until every other block has published chunk c, then computes y of chunk c from the
// lane's row pieces x, their own sums ss and the gates in g.
template <int NG>
__device__ __forceinline__ void norm_compute(const NormCtx& nc_, const PrefillArgs& a, int c, int lane, NormIn<NG>& g,
                                             const float (&x)[NG][8], const float (&ss)[NG], float (&y)[NG][8]) {
  const int bound = wait_bound(a.wait_limit, 1 << 24);
  bool ready = false;
  for (int it = 0; it < bound; ++it) {
    bool ok = true;
#pragma unroll
    for (int i = 0; i < mp::NB - 1; ++i) ok = ok && (unsigned)g.w[i] == (unsigned)(c + nc_.cbase + 1);
    if (__all(ok)) {
      ready = true;
      break;
    }
    __builtin_amdgcn_s_sleep(1);
    norm_load_words(nc_, c, lane, g);
    consume(g);  // a reload is waited for here, not where the next step's loads are issued
  }
  if (!ready && lane == 0) ws_report(a.workspace, wsbits::WAIT_EXCHANGE);
  float oth = 0.f;
#pragma unroll
  for (int i = 0; i < mp::NB - 1; ++i) oth += __uint_as_float((unsigned)(g.w[i] >> 32));
#pragma unroll
  for (int q = 0; q < NG; ++q) {
    const float tot = ss[q] + __shfl(oth, mp::TRPP * q + lane / mp::TLPR);
    const float rs = rsqrt_fast(tot * (1.0f / mp::D) + a.norm_eps);
    const uint32_t zw[4] = {g.z[q].x, g.z[q].y, g.z[q].z, g.z[q].w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float zv = __uint_as_float((e & 1) ? (zw[e >> 1] & 0xffff0000u) : (zw[e >> 1] << 16));
      y[q][e] = x[q][e] * rs * nc_.w[e] * silu(zv);
    }
  }
}

// y rows of chunk c out (c < 0: none).  Every lane stores, the rows past the chunk end (and all
// rows for c < 0) into the sink, 64 bytes of the workspace header that nothing reads: the store
// sequence has no branch, so the compiler's count of the memory operations in flight is exact on
// every path through the step.
template <int O_DT, int NG>
__device__ __forceinline__ void tile_store_y(const NormCtx& nc_, const PrefillArgs& a, const Geo& G, int c, int lane,
                                             const float (&y)[NG][8]) {
  const int L = c >= 0 ? G.len(c) : 0, col = 8 * (lane % mp::TLPR);
  constexpr int ES = O_DT == DT_BF16 ? 2 : 4;
#pragma unroll
  for (int q = 0; q < NG; ++q) {
    const int r = nc_.r0 + mp::TRPP * q + lane / mp::TLPR;
    const int64_t idx = ((G.start + (int64_t)c * mp::C + r) * a.hv + G.h) * (int64_t)mp::D + G.dv0 + col;
    store8_nt<O_DT>(r < L ? static_cast<void*>(static_cast<unsigned char*>(a.y) + idx * ES) : nc_.sink, 0, y[q]);
  }
}

// A tile wave's steps (as many LDS barriers as every other wave).  qt: this tile wave.
template <int O_DT>
__device__ __forceinline__ void tile_wave(ScanSmem& sm, const PrefillArgs& a, const Geo& G, const WsLayout& wl, int n,
                                          int nc, int qt) {
  using namespace mp;
  constexpr int NG = C / TRPP / NTW;  // row passes per tile wave
  const int lane = G.lane;
  const int r0 = qt * (C / NTW);
  lds_barrier();  // the copy waves' two prologue steps
  lds_barrier();
  NormCtx nctx;
  nctx.ring = reinterpret_cast<unsigned long long*>(static_cast<unsigned char*>(a.workspace) + wl.ring) +
              ((int64_t)n * a.hv + G.h) * (RING * NB * C);
  nctx.blk = G.dv0 / DVB;
  nctx.r0 = r0;
  nctx.cbase = G.cbase;
  nctx.sink = static_cast<unsigned char*>(a.workspace) + WsLayout::SINK;
  load8<DT_BF16>(a.norm_w, G.dv0 + 8 * (lane % TLPR), nctx.w);
  float xa[NG][8], xb[NG][8], sa[NG], sb[NG];  // chunks c - 3 and c - 2 at the start of step c
  float y[NG][8] = {};                          // y of chunk c - 3, stored at the end of step c
  NormIn<NG> gin = {};
  for (int c = 0; c < nc + 1; ++c) {
    consume(gin);
    if (c >= 3) norm_compute<NG>(nctx, a, c - 3, lane, gin, xa, sa, y);
    // the gates of chunk c - 2 (from HBM) a whole step before their use, and y of chunk c - 3
    // out, before the wait for the staged tile: neither lies on the way to the barrier
    if (c >= 2) norm_load_z<NG>(nctx, a, G, c - 2, lane, gin);
    tile_store_y<O_DT, NG>(nctx, a, G, c - 3, lane, y);  // steps 0 .. 2: all into the sink
#pragma unroll
    for (int q = 0; q < NG; ++q) {
      sa[q] = sb[q];
#pragma unroll
      for (int e = 0; e < 8; ++e) xa[q][e] = xb[q][e];
    }
    if (c >= 1) {
      wait_flag(&sm.os_ready, npair(true) * c, a);  // chunk c - 1 staged by every output wave
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
      tile_take<NG>(sm.Os, r0, lane, xb);
      row_sums<NG>(xb, sb);
      norm_publish<NG>(nctx, c - 1, lane, sb);
      if (a.o) tile_store<O_DT, NG>(a.o, a, G, c - 1, r0, lane, xb);
    }
    if (c >= 2) norm_load_words<NG>(nctx, c - 2, lane, gin);
    lds_barrier();
  }
  // chunks nc - 2 (words and gates in flight) and nc - 1
  if (nc >= 2) {
    norm_compute<NG>(nctx, a, nc - 2, lane, gin, xa, sa, y);
    tile_store_y<O_DT, NG>(nctx, a, G, nc - 2, lane, y);
  }
  if (nc >= 1) {
    norm_load_z<NG>(nctx, a, G, nc - 1, lane, gin);
    norm_load_words<NG>(nctx, nc - 1, lane, gin);
    norm_compute<NG>(nctx, a, nc - 1, lane, gin, xb, sb, y);
    tile_store_y<O_DT, NG>(nctx, a, G, nc - 1, lane, y);
  }
}

// Copy waves: issue the direct global -> LDS loads (no registers) of chunk c into buffer
// B[c & 1] (c < 0: none) and, for the fused prologue, of the raw x rows of chunk cv's V slice
// into Vr[cv & 1] (cv < 0: none).  A chunk is 51 copies of 1 KiB (q/k image 33, record 13, V
// slice 5) landing back to back in the buffer; copy wave q of NCOPY issues the copies u = q,
// q + NCOPY, ...  The q/k image and the record are contiguous; the V slice is gathered from
// the strided tensor into padded rows, rows past the end of the chunk re-reading its first
// row (finite values that only ever meet beta = 0).  The raw rows of the fused path are the
// chunk's 64 rows after a 3-row halo (x rows c0 - 3 .. c0 + 76); rows outside the sequence
// re-read row c0 (the halo before the sequence start comes from the conv history instead).
// Each wave issues at most about one direct copy per 100 cycles, hence several.
// First copy index u >= base with u = q (mod NCP).
template <int NCOPY>
__device__ __forceinline__ int first_copy(int base, int q) {
  const int r = (q - base) % NCOPY;
  return base + (r < 0 ? r + NCOPY : r);
}

// Number of direct copies copy wave q issues for one chunk (issue_chunk with c >= 0 and cv >= 0).
template <bool FUSED, int NCOPY>
__device__ __forceinline__ int copies_of_wave(int q) {
  using namespace mp;
  constexpr int NQK = QK_BYTES / 1024, NREC = REC_BYTES / 1024, NV = C * (LDV / 8) / 64;
  const int nqk = (NQK - q + NCOPY - 1) / NCOPY;
  const int f = first_copy<NCOPY>(NQK, q);
  const int nrec = f < NQK + NREC ? (NQK + NREC - f + NCOPY - 1) / NCOPY : 0;
  if constexpr (FUSED) return nqk + nrec + (q < 4 ? 2 : 0);
  const int fv = first_copy<NCOPY>(NQK + NREC, q);
  return nqk + nrec + (fv < NQK + NREC + NV ? (NQK + NREC + NV - fv + NCOPY - 1) / NCOPY : 0);
}

// s_waitcnt on the vector memory count only (expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt is six bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
// The same for a wave-uniform count n in [0, 24) (larger counts wait for everything).
__device__ __forceinline__ void wait_vm_n(int n) {
  switch (n) {
#define AGNES_WAIT_CASE(k) case k: wait_vm<k>(); break;
    AGNES_WAIT_CASE(1) AGNES_WAIT_CASE(2) AGNES_WAIT_CASE(3) AGNES_WAIT_CASE(4) AGNES_WAIT_CASE(5)
    AGNES_WAIT_CASE(6) AGNES_WAIT_CASE(7) AGNES_WAIT_CASE(8) AGNES_WAIT_CASE(9) AGNES_WAIT_CASE(10)
    AGNES_WAIT_CASE(11) AGNES_WAIT_CASE(12) AGNES_WAIT_CASE(13) AGNES_WAIT_CASE(14) AGNES_WAIT_CASE(15)
    AGNES_WAIT_CASE(16) AGNES_WAIT_CASE(17) AGNES_WAIT_CASE(18) AGNES_WAIT_CASE(19) AGNES_WAIT_CASE(20)
    AGNES_WAIT_CASE(21) AGNES_WAIT_CASE(22) AGNES_WAIT_CASE(23)
#undef AGNES_WAIT_CASE
    default: wait_vm<0>(); break;
  }
}

template <bool FUSED, int NCOPY>
__device__ __forceinline__ void issue_chunk(ScanSmem& sm, const PrefillArgs& a, const Geo& G,
                                            const unsigned char* ws, int c, int cv, int q) {
  using namespace mp;
  constexpr int NQK = QK_BYTES / 1024, NREC = REC_BYTES / 1024, NV = C * (LDV / 8) / 64;
  static_assert(sizeof(ScanBuf) == (NQK + NREC + NV) * 1024, "chunk buffer is a whole number of copies");
  static_assert(VR_ROWS * DVB * 2 == NV * 1024, "raw V rows take as many copies as the V slice");
  // q is wave-uniform (a scalar): every loop below runs on scalar counters, and a copy costs
  // an address add, an m0 add and the load.
  const int lane = G.lane;
  const uint16_t* vb = static_cast<const uint16_t*>(a.v) + (int64_t)G.h * D + G.dv0;
  if (c >= 0) {
    unsigned char* dst = reinterpret_cast<unsigned char*>(&sm.B[c & 1]);
    const unsigned char* qk = ws + G.qk0 + (size_t)c * QK_BYTES + 16 * lane;
    for (int u = q; u < NQK; u += NCOPY)
      __builtin_amdgcn_global_load_lds((glb_void*)(qk + 1024 * u), (lds_void*)(dst + 1024 * u), 16, 0, 0);
    const unsigned char* rec = ws + G.rec0 + (size_t)c * REC_BYTES + 16 * lane - 1024 * NQK;
    for (int u = first_copy<NCOPY>(NQK, q); u < NQK + NREC; u += NCOPY)
      __builtin_amdgcn_global_load_lds((glb_void*)(rec + 1024 * u), (lds_void*)(dst + 1024 * u), 16, 0, 0);
    if constexpr (!FUSED) {
      constexpr int VPR = LDV / 8;  // 16-byte pieces per padded V row (5)
      const int L = G.len(c);
      for (int u = first_copy<NCOPY>(NQK + NREC, q); u < NQK + NREC + NV; u += NCOPY) {
        const int j = 64 * (u - NQK - NREC) + lane, r = j / VPR, pc = j % VPR;
        const uint16_t* src = vb + (G.start + (int64_t)c * C) * a.v_stride +
                              ((r < L && pc < DVB / 8) ? (int64_t)r * a.v_stride + 8 * pc : 0);
        __builtin_amdgcn_global_load_lds((glb_void*)src, (lds_void*)(dst + 1024 * u), 16, 0, 0);
      }
    }
  }
  if constexpr (FUSED) {
    // raw rows: conv wave q (< 4) copies pieces q and q + 1 (raw rows 16 q .. 16 q + 31), all
    // that its own conv items (chunk rows 16 q .. 16 q + 15) read, so that the conv waits only
    // for its own copies
    if (cv >= 0 && q < 4) {
      static_assert(NV == 5, "four conv waves, two overlapping 16-row pieces each");
      const int64_t c0 = G.start + (int64_t)cv * C;
      for (int u = NQK + NREC + q; u < NQK + NREC + q + 2; ++u) {
        const int jv = 64 * (u - NQK - NREC) + lane, i = jv >> 2, pc = jv & 3;
        const int64_t pos = c0 - 3 + i;
        const bool in = pos >= G.hstart && i < 3 + G.len(cv);
        const uint16_t* src = vb + (in ? pos : c0) * a.v_stride + 8 * pc;
        __builtin_amdgcn_global_load_lds((glb_void*)src, (lds_void*)(&sm.Vr[cv & 1][0][0] + 512 * (u - NQK - NREC)), 16,
                                         0, 0);
      }
    }
  }
}

// LDS reads and the write of the V-slice conv, written out so that the compiler does not wait
// for the copy wave's direct copies in flight before them: it cannot tell the parity-indexed
// rows apart from the copies' destinations and would wait for every copy to land (vector memory
// counts) before the conv could start.  The conv reads Vr[cc & 1] (landed a step earlier) and
// writes B[cc & 1].Vs, and the copies in flight write B[cc & 1].QK / .R and Vr[(cc + 1) & 1]:
// disjoint bytes.  Each block waits for its own LDS operations.
__device__ __forceinline__ void lds_read4_b128(const void* p0, const void* p1, const void* p2, const void* p3,
                                               uint4 (&x)[4]) {
  const unsigned a0 = (unsigned)(uintptr_t)(const lds_void*)p0, a1 = (unsigned)(uintptr_t)(const lds_void*)p1,
                 a2 = (unsigned)(uintptr_t)(const lds_void*)p2, a3 = (unsigned)(uintptr_t)(const lds_void*)p3;
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  u32x4 r0, r1, r2, r3;
  asm volatile(
      "ds_read_b128 %0, %4\n\t"
      "ds_read_b128 %1, %5\n\t"
      "ds_read_b128 %2, %6\n\t"
      "ds_read_b128 %3, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3)
      : "v"(a0), "v"(a1), "v"(a2), "v"(a3)
      : "memory");
  x[0] = make_uint4(r0[0], r0[1], r0[2], r0[3]);
  x[1] = make_uint4(r1[0], r1[1], r1[2], r1[3]);
  x[2] = make_uint4(r2[0], r2[1], r2[2], r2[3]);
  x[3] = make_uint4(r3[0], r3[1], r3[2], r3[3]);
}
__device__ __forceinline__ void lds_write_b128(void* p, h8 v) {
  const unsigned a = (unsigned)(uintptr_t)(lds_void*)p;
  asm volatile("ds_write_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" ::"v"(a), "v"(v) : "memory");
}

// Copy waves, fused prologue: the V slice of chunk cc = SiLU(causal conv) of its raw x rows in
// Vr[cc & 1] (row r of the chunk reads raw rows r .. r + 3), fp16 into B[cc & 1].Vs.  For the
// sequence's first chunk the halo rows are the conv history (zeros without one).  Item
// q * 64 + lane < 256: chunk row item / 4, value columns 8 (item % 4) .. + 7; the lane's conv
// taps (packed bf16, as stored) and biases of those 8 channels are loaded once per sequence.
__device__ __forceinline__ void conv_vslice(ScanSmem& sm, const PrefillArgs& a, const Geo& G, int n, int cc, int q,
                                            const uint4 (&wt)[4], const float (&bs)[8]) {
  using namespace mp;
  const int item = q * 64 + G.lane;
  if (item >= C * DVB / 8) return;
  const int r = item >> 2, cg = item & 3;
  uint4 xr[4];
  lds_read4_b128(&sm.Vr[cc & 1][r][8 * cg], &sm.Vr[cc & 1][r + 1][8 * cg], &sm.Vr[cc & 1][r + 2][8 * cg],
                 &sm.Vr[cc & 1][r + 3][8 * cg], xr);
  if (cc == 0 && G.start == G.hstart) {  // staged rows 0 .. 2 lie before the sequence start
#pragma unroll
    for (int jt = 0; jt < 3; ++jt) {
      const int i = r + jt;
      if (i < 3) {
        const uint16_t* hist = static_cast<const uint16_t*>(a.conv_hist);
        const int64_t ch = (int64_t)(2 * a.hk + G.h) * D + G.dv0 + 8 * cg;
        const int64_t Ctot = (int64_t)(2 * a.hk + a.hv) * D;
        const uint16_t* hp = hist + ((int64_t)n * Ctot + ch) * 3 + i;
        xr[jt] = hist ? make_uint4(hp[0] | (uint32_t)hp[3] << 16, hp[6] | (uint32_t)hp[9] << 16,
                                   hp[12] | (uint32_t)hp[15] << 16, hp[18] | (uint32_t)hp[21] << 16)
                      : make_uint4(0, 0, 0, 0);
      }
    }
  }
  float acc[8];
  conv4_bf16x8(xr, wt, bs, acc);
  h8 o;
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = (_Float16)silu(acc[e]);
  lds_write_b128(&sm.B[cc & 1].Vs[r][8 * cg], o);
}

// Waves: NPAIR chain waves, NPAIR output waves (pair p for value tiles TPW p .. TPW p + TPW - 1),
// then NCP copy waves.  Iteration c (one LDS barrier each, n + 1 in all): the chain waves on
// chunk c; the output waves finish and write out chunk c-1 and start chunk c; the copy waves
// fill the other buffer with chunk c+1.
template <int O_DT, bool FUSED, bool NORM = false>
__global__ __launch_bounds__(64 * mp::nwaves(NORM)) void scan_kernel(PrefillArgs a, int64_t maxch) {
  using namespace mp;
  constexpr int TPW = tpw(NORM), NPAIR = npair(NORM);
  extern __shared__ __align__(16) unsigned char smem_raw[];
  ScanSmem& sm = *reinterpret_cast<ScanSmem*>(smem_raw);
  const int32_t* off = ws_offsets(a.workspace);
  const unsigned char* ws = static_cast<const unsigned char*>(a.workspace);
  const WsLayout wl(a.num_seqs, a.hv, a.hk, maxch);

  // Workgroups sharing a key group are consecutive in `lid`; the hardware deals block ids
  // round-robin over the 8 XCDs, so each key group's workgroups go to one XCD (shared L2), and
  // the key groups are dealt to the XCDs in turn (kg mod 8), so that every XCD gets an even
  // share of every sequence when the grid is larger than the chip.
  const unsigned nblk = gridDim.x;
  const unsigned kgw = (unsigned)(NB * (a.hv / a.hk));  // workgroups per key group
  unsigned lid = blockIdx.x;
  if ((nblk % (8u * kgw)) == 0) {
    const unsigned i = blockIdx.x >> 3;
    lid = ((i / kgw) * 8u + (blockIdx.x & 7u)) * kgw + i % kgw;
  }
  if constexpr (NORM) {
    // The NB workgroups of a value head wait for each other, so their roles are claimed in the
    // order workgroups start, not taken from the block index.  The roles are cut into 8 ranges
    // of whole key groups, one per XCD (range y: key groups y, y + 8, y + 16, ..., dealt like the
    // block index above, so every XCD gets its share of every sequence); a workgroup claims the next role of its own XCD's range
    // (from the XCC_ID register) with an atomic counter, or, once that range is used up, the
    // next role of a range that is not.  Each range is claimed in order, so at most one head
    // per range has members still to start: at most 24 workgroups wait on partners that have
    // not started, and the others run to the end and free their compute units.  No residency of
    // the whole grid is assumed, only room for more than 24 of these workgroups at a time.  The
    // XCC_ID only steers the 12 workgroups of a key group to one L2 (a wrong value costs
    // locality, not correctness).
    if (threadIdx.x == 0) {
      unsigned* cnt = reinterpret_cast<unsigned*>(const_cast<unsigned char*>(ws) + wl.tick) + 8 * a.stage;
      const unsigned cap = nblk >> 3;
      unsigned role = 0;
      bool claimed = true;
      if ((nblk % (8u * NB * (unsigned)(a.hv / a.hk))) == 0) {
        const unsigned x = __builtin_amdgcn_s_getreg(0xf814) & 7u;  // hwreg(HW_REG_XCC_ID)
        unsigned t = __hip_atomic_fetch_add(&cnt[x], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        unsigned y = x;
        if (t >= cap) {  // this XCD's range is used up: another range still has a role for every such claim
          bool got = false;
          const int bound = wait_bound(a.wait_limit, 1 << 16);
          for (int it = 0; it < bound && !got; ++it)
            for (y = 0; y < 8 && !got; ++y) {
              if (__hip_atomic_load(&cnt[y], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= cap) continue;
              t = __hip_atomic_fetch_add(&cnt[y], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              got = t < cap;
            }
          if (got) --y;  // the loop advanced past the range it claimed from
          if (!got) {  // (never when every workgroup claims once): no role, nothing is touched
            ws_report(a.workspace, wsbits::WAIT_ROLE);
            claimed = false;
          }
        }
        // claim t of range y: its key groups are y, y + 8, y + 16, ... (dealt as the block ids)
        const unsigned kgw2 = (unsigned)(NB * (a.hv / a.hk));
        role = ((t / kgw2) * 8u + y) * kgw2 + t % kgw2;
      } else {
        role = __hip_atomic_fetch_add(&cnt[0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // plain start order
      }
      if (claimed && role >= nblk) {  // (never when the counters were cleared for this call)
        ws_report(a.workspace, wsbits::WAIT_ROLE);
        claimed = false;
      }
      sm.ticket = claimed ? role : ~0u;
    }
    __syncthreads();
    lid = sm.ticket;
    if (lid == ~0u) return;
  }
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
  G.hstart = G.start;
  const int ncs = (int)((G.end - G.start + C - 1) / C);
  const int cb = (int)((int64_t)ncs * a.part_lo / a.part_den), ce = (int)((int64_t)ncs * a.part_hi / a.part_den);
  G.cbase = cb;
  G.start += (int64_t)cb * C;
  if (G.end > G.hstart + (int64_t)ce * C) G.end = G.hstart + (int64_t)ce * C;
  if (G.end < G.start) G.end = G.start;
  G.nchunks = ce - cb;
  G.sbase = ((int64_t)n * a.hv + G.h) * (D * D);
  G.rec0 = wl.rec + ((size_t)G.h * (size_t)maxch + (size_t)(off[n] + cb)) * REC_BYTES;
  G.qk0 = wl.qk + ((size_t)G.kh * (size_t)maxch + (size_t)(off[n] + cb)) * QK_BYTES;
  const int ln = G.ln, lg = G.lg, lane = G.lane;
  const int nc = G.nchunks;
  if (threadIdx.x < NPAIR) sm.ks_done[threadIdx.x] = 0;  // ordered before every use by the prologue barrier
  if (threadIdx.x == 0) sm.os_ready = 0;
  static_assert(!NORM || FUSED, "the whole-layer call is the fused one");

  if (G.w < NPAIR) {  // chain wave
    const int pr = NPAIR == 1 ? 0 : G.w, t0 = TPW * pr;
    f4 sacc[TPW][8];
    h8 sb[TPW][4];
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
#pragma unroll
      for (int kt = 0; kt < 8; ++kt) {
        f4 v = {0.f, 0.f, 0.f, 0.f};
        if (a.s0) {
          const float4 x =
              *reinterpret_cast<const float4*>(a.s0 + G.sbase + (int64_t)(G.dv0 + 16 * (t0 + t) + ln) * D + 16 * kt + 4 * lg);
          v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
        }
        sacc[t][kt] = v;
      }
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        sb[t][ks] = b_pair(sacc[t][2 * ks], sacc[t][2 * ks + 1]);
        sm.X[0].s[t0 + t][ks][lane] = sb[t][ks];
      }
    }
    if constexpr (FUSED) lds_barrier();  // (the copy waves' extra prologue step)
    lds_barrier();
    for (int c = 0; c < nc + 1; ++c) {
      if (c < nc)
        chain_step<TPW, FUSED>(sm.B[c & 1], sm.X[c & 1], sm.X[(c + 1) & 1], t0, lane, ln, lg, sacc, sb, &sm.ks_done[pr], c);
      lds_barrier();
    }
    // An fp16 operand out of range anywhere in the sequence leaves the state out of range or not
    // finite (inf and NaN persist through the decay and the updates), so one check at the end
    // covers the state and U operands of every chunk.
    bool in_range = true;
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
      for (int kt = 0; kt < 8; ++kt)
#pragma unroll
        for (int e = 0; e < 4; ++e) in_range = in_range && fp16_range(sacc[t][kt][e]);
    if (!__all(in_range) && lane == 0) ws_report(a.workspace, wsbits::RANGE);
    if (a.s1) {
#pragma unroll
      for (int t = 0; t < TPW; ++t)
#pragma unroll
        for (int kt = 0; kt < 8; ++kt) {
          const f4 v = sacc[t][kt];
          *reinterpret_cast<float4*>(a.s1 + G.sbase + (int64_t)(G.dv0 + 16 * (t0 + t) + ln) * D + 16 * kt + 4 * lg) =
              make_float4(v[0], v[1], v[2], v[3]);
        }
    }
  } else if (G.w < 2 * NPAIR) {  // output wave
    const int pr = NPAIR == 1 ? 0 : G.w - NPAIR, t0 = TPW * pr;
    f4 qs[TPW][4];
    h8 pa[6];
    float ge[16] = {};
    if constexpr (FUSED) lds_barrier();
    lds_barrier();
    for (int c = 0; c < nc + 1; ++c) {
      // Start once the chain wave is past K S^T: run beside it, the output wave's LDS reads
      // slow the chain's operand reads (the serial path) by about a third.
      if (c < nc) wait_flag(&sm.ks_done[pr], c + 1, a);
      if (c >= 1) o_step<TPW, O_DT, NORM>(sm.X[(c - 1) & 1], sm.Os, &sm.os_ready, a, G, c - 1, t0, qs, pa, ge);
      if (c < nc) qs_step<TPW>(sm.B[c & 1], sm.X[c & 1], t0, lane, ln, lg, qs, pa, ge);
      lds_barrier();
    }
  } else {  // copy wave
    const int q = __builtin_amdgcn_readfirstlane(G.w - 2 * NPAIR);  // wave-uniform: scalar copy loop
    if constexpr (FUSED) {
      // Whole-layer call: the first NTW copy waves are tile waves; the others copy (and the conv
      // takes four of them).
      constexpr int NTWF = NORM ? NTW : 0, NCOPY = NCP - NTWF;
      static_assert(NCOPY >= 4, "the conv of a V slice takes four waves");
      if constexpr (NORM) {
        if (q < NTW) {
          tile_wave<O_DT>(sm, a, G, wl, n, nc, q);
          return;
        }
      }
      const int qc = q - NTWF, qv = NORM ? q - (NCP - 4) : q;  // copy index; conv index (< 0 or > 3: none)
      // Step c: copies of chunk c+1 and raw rows of chunk c+2 in flight while the raw rows of
      // chunk c+1 (landed during step c-1) are convolved into its V slice.
      uint4 wt[4];  // conv taps of the lane's 8 value channels, packed bf16 as stored
      float bs[8];
      const int64_t ch = (int64_t)(2 * a.hk + G.h) * D + G.dv0 + 8 * (lane & 3);
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) wt[q4] = load_raw8<DT_BF16>(a.conv_w, ch * 4 + 8 * q4).u[0];
      if (a.conv_b) load8<DT_BF16>(a.conv_b, ch, bs);
      else {
#pragma unroll
        for (int e = 0; e < 8; ++e) bs[e] = 0.f;
      }
      if (nc > 0) issue_chunk<true, NCOPY>(sm, a, G, ws, 0, 0, qc);
      if (nc > 1) issue_chunk<true, NCOPY>(sm, a, G, ws, -1, 1, qc);
      __builtin_amdgcn_s_waitcnt(0);
      lds_barrier();  // raw rows of chunk 0 visible to every copy wave
      if (nc > 0 && qv >= 0 && qv < 4) conv_vslice(sm, a, G, n, 0, qv, wt, bs);
      lds_barrier();
      // A conv wave's raw rows of chunk c + 2 (its last two copies of step c) may still be in
      // flight at the end of step c: only its own conv of step c + 1 reads them, after a wait
      // for everything but that step's own copies.  Every other copy lands before the barrier.
      const bool conv_wave = qv >= 0 && qv < 4;
      for (int c = 0; c < nc + 1; ++c) {
        if (c + 1 < nc) {
          const bool raw = c + 2 < nc;
          issue_chunk<true, NCOPY>(sm, a, G, ws, c + 1, raw ? c + 2 : -1, qc);
          if (conv_wave) {
            wait_vm_n(copies_of_wave<true, NCOPY>(qc) - (raw ? 0 : 2));  // raw rows of chunk c + 1
            conv_vslice(sm, a, G, n, c + 1, qv, wt, bs);
            if (raw) wait_vm<2>();
            else wait_vm<0>();
          } else {
            __builtin_amdgcn_s_waitcnt(0);
          }
        }
        copy_barrier();
      }
    } else {
      if (nc > 0) {
        issue_chunk<false, NCP>(sm, a, G, ws, 0, -1, q);
        __builtin_amdgcn_s_waitcnt(0);
      }
      lds_barrier();
      for (int c = 0; c < nc + 1; ++c) {
        if (c + 1 < nc) {
          issue_chunk<false, NCP>(sm, a, G, ws, c + 1, -1, q);
          __builtin_amdgcn_s_waitcnt(0);
        }
        lds_barrier();
      }
    }
  }
}

// ---------------------------------------------------------------- host side
size_t prefill_mfma_workspace(int num_seqs, int64_t total, int hk, int hv) {
  if (num_seqs <= 0) return 0;
  return WsLayout(num_seqs, hv, hk, max_chunks(total, num_seqs)).bytes;
}

size_t layer_prefill_workspace(int num_seqs, int64_t total, int hk, int hv) {
  if (num_seqs <= 0) return 0;
  return WsLayout(num_seqs, hv, hk, max_chunks(total, num_seqs)).layer_bytes;
}

// prep over (chunk, key group, round of value heads), scan over (sequence, value head, row block);
// the whole-layer call's conv history launch is bounded by its 65535 sequences.
bool prefill_mfma_fits(int num_seqs, int64_t total, int hk, int hv) {
  using u128 = unsigned __int128;
  const int64_t rounds = (hv / hk + mp::PH - 1) / mp::PH;
  return grid_fits((u128)max_chunks(total, num_seqs) * (u128)hk * (u128)rounds, 256 * mp::PH) &&
         grid_fits((u128)num_seqs * (u128)hv * mp::NB, 64 * mp::MAX_WAVES);
}

template <int O_DT, bool FUSED, bool NORM>
static hipError_t scan_attr() {
  static const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(scan_kernel<O_DT, FUSED, NORM>),
                                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)sizeof(ScanSmem));
  return e;
}

static hipError_t launch_offsets(const PrefillArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(chunk_offsets_kernel, dim3(1), dim3(256), 0, st, a.cu, a.num_seqs, a.total,
                     const_cast<int32_t*>(ws_offsets(a.workspace)), static_cast<unsigned*>(a.workspace));
  return hipGetLastError();
}

// done (optional): an event completed with the kernel itself (no marker of its own in the queue)
template <bool FUSED>
static hipError_t launch_prep(const PrefillArgs& a, int64_t maxch, hipStream_t st, hipEvent_t done = nullptr) {
  const int64_t rounds = (a.hv / a.hk + mp::PH - 1) / mp::PH;
  const dim3 grid((unsigned)(maxch * a.hk * rounds)), block(256 * mp::PH);
  if (done) {
    hipExtLaunchKernelGGL((prep_kernel<FUSED>), grid, block, 0, st, nullptr, done, 0, a, maxch);
  } else {
    // (the whole-layer call's first prep also clears the exchange words and role counters, so it
    // runs even when every sequence is empty)
    if (a.total == 0 && !(a.layer && a.part_lo == 0)) return hipSuccess;
    hipLaunchKernelGGL((prep_kernel<FUSED>), grid, block, 0, st, a, maxch);
  }
  return hipGetLastError();
}

template <int O_DT, bool FUSED, bool NORM>
static hipError_t launch_scan(const PrefillArgs& a, int64_t maxch, hipStream_t st) {
  const hipError_t e = scan_attr<O_DT, FUSED, NORM>();
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)((int64_t)a.num_seqs * a.hv * mp::NB)), block(64 * mp::nwaves(NORM));
  hipLaunchKernelGGL((scan_kernel<O_DT, FUSED, NORM>), grid, block, sizeof(ScanSmem), st, a, maxch);
  return hipGetLastError();
}

// advance the conv history once every read of the old one (prep, scan) is done
static hipError_t launch_history(const PrefillArgs& a, hipStream_t st) {
  if (!a.conv_hist) return hipSuccess;
  const ConvArgs h{a.q, a.qk_stride, nullptr, 0, DT_BF16, a.conv_w, a.conv_b, a.cu, a.num_seqs, a.total,
                   (2 * a.hk + a.hv) * mp::D, a.conv_hist, 0, 0.f};
  return launch_conv_history(h, st);
}

template <int O_DT, bool FUSED, bool NORM>
static hipError_t launch_o(const PrefillArgs& a, hipStream_t st) {
  if (a.num_seqs == 0) return hipSuccess;
  const int64_t maxch = max_chunks(a.total, a.num_seqs);
  hipError_t e = launch_offsets(a, st);
  if (e == hipSuccess) e = launch_prep<FUSED>(a, maxch, st);
  if (e == hipSuccess) e = launch_scan<O_DT, FUSED, NORM>(a, maxch, st);
  if (e == hipSuccess && FUSED) e = launch_history(a, st);
  return e;
}

// ---- prefill calls in stages.  The scan of a single long sequence occupies 4 compute units per
// value head (192 of 256 for the layer) for its whole length, while prep uses the whole chip for
// a short time before it.  So the call runs as prep(first part of every sequence) -> scan(first
// part) on the caller's stream, with prep(next part) on a side stream beside that scan (on the
// compute units the scan leaves free), then scan(next part) carrying the state over.  Prep beside
// a scan runs ~3x slower than alone, so the first part is the larger: 13/20 of the chunks for the
// whole-layer call, 7/10 for the prefill calls (their scan is faster without the norm).  More
// stages shorten the exposed first prep but cost more at each hand-over than they save (at
// T = 8192: two stages 356 us, three 373-380 us, four 398 us).  Used when the scan leaves a
// quarter of the chip free and sequences are long enough.  The cuts are a process-wide setting
// (agnes_gdn_set_prefill_stages, for every kind of call once set), read under the side-queue
// lock at each launch.
constexpr int SPLIT_DEN = 40;    // stage boundaries in 1/40 of each sequence's chunks
constexpr int MAX_STAGES = 8;    // the workspace holds role counters for 8 stages
struct StageCuts {
  int n = 1;                     // number of cuts: the call runs in n + 1 stages
  int cut[MAX_STAGES - 1] = {26};  // stage k covers [cut[k-1], cut[k]) of SPLIT_DEN
  bool custom = false;           // set by the caller (else each kind of call takes its default)
};
constexpr int LAYER_CUT = 26, PREFILL_CUT = 28;  // defaults (measured at T = 8192)

namespace {
// The side streams of the calls in stages: one per caller stream, up to SIDE_PER_DEV per device
// (beyond that the least recently used one is shared with the new caller stream: its work stays
// ordered on the side stream and every wait is enqueued against the event record it follows, so
// sharing costs only concurrency).  Callers on different streams thus run their side-stream
// preparation side by side.
constexpr int SIDE_PER_DEV = 4;
struct SideQueue {
  hipStream_t s = nullptr;
  hipEvent_t prepped[MAX_STAGES] = {};
  hipStream_t owner = nullptr;  // the caller stream it last served
  unsigned long long used = 0;  // when (g_side_tick)
  int cus = 0;
};
std::mutex g_side_mu;  // held while a call enqueues: a side queue's events are shared
SideQueue g_side[64][SIDE_PER_DEV];
unsigned long long g_side_tick = 0;
StageCuts g_cuts;      // under g_side_mu
}  // namespace

static hipError_t destroy_side_queue(SideQueue& q) {
  hipError_t first = hipSuccess;
  for (int k = 0; k < MAX_STAGES; ++k)
    if (q.prepped[k]) {
      const hipError_t e = hipEventDestroy(q.prepped[k]);
      if (first == hipSuccess) first = e;
    }
  if (q.s) {
    const hipError_t e = hipStreamDestroy(q.s);
    if (first == hipSuccess) first = e;
  }
  q = SideQueue{};
  return first;
}

// The side queue of `caller` on the current device (under g_side_mu), created on first use.
static hipError_t side_queue(hipStream_t caller, SideQueue*& q) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  SideQueue* row = g_side[dev];
  SideQueue* pick = nullptr;
  for (int i = 0; i < SIDE_PER_DEV && !pick; ++i)
    if (row[i].s && row[i].owner == caller) pick = &row[i];
  for (int i = 0; i < SIDE_PER_DEV && !pick; ++i)
    if (!row[i].s) pick = &row[i];
  if (!pick) {
    pick = &row[0];
    for (int i = 1; i < SIDE_PER_DEV; ++i)
      if (row[i].used < pick->used) pick = &row[i];
  }
  if (!pick->s) {
    SideQueue n;
    e = hipDeviceGetAttribute(&n.cus, hipDeviceAttributeMultiprocessorCount, dev);
    for (int k = 0; k < MAX_STAGES && e == hipSuccess; ++k) e = hipEventCreate(&n.prepped[k]);
    if (e == hipSuccess) e = hipStreamCreateWithFlags(&n.s, hipStreamNonBlocking);  // default priority
    if (e != hipSuccess) {
      destroy_side_queue(n);
      return e;
    }
    *pick = n;
  }
  pick->owner = caller;
  pick->used = ++g_side_tick;
  q = pick;
  return hipSuccess;
}

// Destroys the side queues (streams and events) the calls in stages created, after waiting for
// their work; the next such call creates them again.  No HIP call at all when none exists.
hipError_t release_side_queues() {
  std::lock_guard<std::mutex> lock(g_side_mu);
  bool any = false;
  for (const auto& row : g_side)
    for (const SideQueue& q : row) any = any || q.s != nullptr;
  if (!any) return hipSuccess;
  int cur = 0;
  hipError_t first = hipGetDevice(&cur);
  for (int d = 0; d < 64; ++d) {
    for (SideQueue& q : g_side[d]) {
      if (!q.s) continue;
      hipError_t e = hipSetDevice(d);
      if (e == hipSuccess) e = hipStreamSynchronize(q.s);
      if (e == hipSuccess) e = destroy_side_queue(q);  // (kept, with its work, if the wait failed)
      if (first == hipSuccess) first = e;
    }
  }
  const hipError_t e = hipSetDevice(cur);
  return first != hipSuccess ? first : e;
}

// Sets the stage cuts of the later calls: n cuts strictly increasing inside (0, SPLIT_DEN),
// n < MAX_STAGES (n = 0: one stage), or n = -1: back to each kind of call's default.  False, and
// nothing changed, for any other list.
bool set_stage_cuts(const int* cuts, int n) {
  if (n < -1 || n >= MAX_STAGES || (n > 0 && !cuts)) return false;
  for (int i = 0; i < n; ++i)
    if (cuts[i] <= (i ? cuts[i - 1] : 0) || cuts[i] >= SPLIT_DEN) return false;
  std::lock_guard<std::mutex> lock(g_side_mu);
  g_cuts = StageCuts{};
  if (n < 0) return true;
  g_cuts.custom = true;
  g_cuts.n = n;
  for (int i = 0; i < n; ++i) g_cuts.cut[i] = cuts[i];
  return true;
}

template <int O_DT, bool FUSED, bool NORM>
static hipError_t launch_staged(const PrefillArgs& a, hipStream_t st) {
  if (a.num_seqs == 0) return hipSuccess;
  if (a.single_stage) return launch_o<O_DT, FUSED, NORM>(a, st);
  std::lock_guard<std::mutex> lock(g_side_mu);
  StageCuts cuts = g_cuts;
  if (!cuts.custom) cuts.cut[0] = NORM ? LAYER_CUT : PREFILL_CUT;
  if (cuts.n == 0) return launch_o<O_DT, FUSED, NORM>(a, st);
  SideQueue* q = nullptr;
  hipError_t e = side_queue(st, q);
  if (e != hipSuccess) return e;
  const int64_t grid = (int64_t)a.num_seqs * a.hv * mp::NB;
  const bool split = 4 * grid <= 3 * (int64_t)q->cus && a.total >= (int64_t)a.num_seqs * 8 * mp::C;
  if (!split) return launch_o<O_DT, FUSED, NORM>(a, st);
  const int nstage = cuts.n + 1;
  const int64_t maxch = max_chunks(a.total, a.num_seqs);
  const WsLayout wl(a.num_seqs, a.hv, a.hk, maxch);
  float* mid = reinterpret_cast<float*>(static_cast<unsigned char*>(a.workspace) + wl.mid);
  PrefillArgs sp[MAX_STAGES];
  for (int k = 0; k < nstage; ++k) {
    sp[k] = a;
    sp[k].part_lo = k == 0 ? 0 : cuts.cut[k - 1];
    sp[k].part_hi = k == nstage - 1 ? SPLIT_DEN : cuts.cut[k];
    sp[k].part_den = SPLIT_DEN;
    sp[k].stage = k;
    if (k > 0) sp[k].s0 = mid;           // a workgroup reads its state slice before it writes it,
    if (k < nstage - 1) sp[k].s1 = mid;  // so a middle stage updates the carried state in place
  }
  // Under stream capture the events are recorded as their own nodes (a kernel-completion event
  // is not a capturable dependency); the side stream then joins the capture through them.
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if ((e = hipStreamIsCapturing(st, &cap)) != hipSuccess) return e;
  const bool capturing = cap != hipStreamCaptureStatusNone;
  if ((e = launch_offsets(a, st)) != hipSuccess) return e;
  if ((e = launch_prep<FUSED>(sp[0], maxch, st, capturing ? nullptr : q->prepped[0])) != hipSuccess) return e;
  if (capturing && (e = hipEventRecord(q->prepped[0], st)) != hipSuccess) return e;
  for (int k = 0; k < nstage; ++k) {
    if (k > 0 && (e = hipStreamWaitEvent(st, q->prepped[k], 0)) != hipSuccess) return e;
    if ((e = launch_scan<O_DT, FUSED, NORM>(sp[k], maxch, st)) != hipSuccess) return e;
    if (k + 1 == nstage) break;
    if (k == 0 && (e = hipStreamWaitEvent(q->s, q->prepped[0], 0)) != hipSuccess) return e;
    hipEvent_t done = q->prepped[k + 1];
    if ((e = launch_prep<FUSED>(sp[k + 1], maxch, q->s, capturing ? nullptr : done)) != hipSuccess) return e;
    if (capturing && (e = hipEventRecord(done, q->s)) != hipSuccess) return e;
  }
  return FUSED ? launch_history(a, st) : hipSuccess;
}

hipError_t launch_layer_prefill(const PrefillArgs& a, hipStream_t st) {
  return a.o_dtype == DT_BF16 ? launch_staged<DT_BF16, true, true>(a, st) : launch_staged<DT_F32, true, true>(a, st);
}

hipError_t launch_prefill_mfma(const PrefillArgs& a, hipStream_t st) {
  if (a.conv_w)
    return a.o_dtype == DT_BF16 ? launch_staged<DT_BF16, true, false>(a, st) : launch_staged<DT_F32, true, false>(a, st);
  return a.o_dtype == DT_BF16 ? launch_staged<DT_BF16, false, false>(a, st) : launch_staged<DT_F32, false, false>(a, st);
}

}  // namespace agnes
