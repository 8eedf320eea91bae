// Host-side checks of the libagnes_gdn C ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer (the library's host code and this driver both).
//
// Every compute call below is built to stop at one of the library's argument checks, so no
// pointer value is ever dereferenced and nothing reaches the device; the remaining calls are
// host-only queries and settings.  Besides the ordinary rejects, the cases push every size,
// stride and count to its extreme (INT64_MAX tokens, strides that wrap the address space,
// head counts whose channel sums overflow 32 bits) so that the sanitizers see the arithmetic
// of the checks at the edges of their domain.
//
// Exit status 0: every call returned the expected status (a sanitizer report aborts the run).
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <limits>

#include "agnes_gdn.h"

namespace {

int g_fail = 0;

#define EXPECT(call, want)                                                                          \
  do {                                                                                              \
    const long long got_ = (long long)(call);                                                       \
    if (got_ != (long long)(want)) {                                                                \
      std::fprintf(stderr, "%s:%d: %s returned %lld, expected %lld\n", __FILE__, __LINE__, #call, got_, \
                   (long long)(want));                                                              \
      ++g_fail;                                                                                     \
    }                                                                                               \
  } while (0)

// A struct of default arguments, then one statement that changes them.
#define WITH(T, stmt) ([&] { T a; stmt; return a; }())

constexpr int OK = AGNES_OK, INV = AGNES_ERR_INVALID_ARG, UNS = AGNES_ERR_UNSUPPORTED, WS = AGNES_ERR_WORKSPACE;
constexpr agnes_dtype BF16 = AGNES_BF16, F32 = AGNES_F32;
constexpr int64_t I64MAX = std::numeric_limits<int64_t>::max();
constexpr int IMAX = std::numeric_limits<int>::max();
constexpr int64_t BIG_STRIDE = I64MAX & ~int64_t(7);  // a multiple of 8 whose extent wraps
const float NaN = std::nanf(""), Inf = INFINITY;

// Distinct, 256-byte aligned addresses that are never dereferenced.
void* P(int i) { return reinterpret_cast<void*>(uintptr_t(0x10000000) * uintptr_t(i + 1)); }
template <class T = void>
T* Pt(int i, uintptr_t off = 0) {
  return reinterpret_cast<T*>(reinterpret_cast<uintptr_t>(P(i)) + off);
}
// 16 TiB apart: for problems whose buffers are too large for P's spacing.
template <class T = void>
T* Far(int i) {
  return reinterpret_cast<T*>(uintptr_t(i + 1) << 44);
}
const agnes_dtype BAD_DT = static_cast<agnes_dtype>(7);

// ---- agnes_gdn_conv
struct Conv {
  const void* x = P(0); int64_t xs = 512; void* y = P(1); int64_t ys = 512; agnes_dtype dt = BF16;
  const void* w = P(2); const void* b = nullptr; const int32_t* cu = Pt<int32_t>(3); int n = 2; int64_t T = 10;
  int C = 512; int K = 4; void* st = nullptr; int l2 = 2; int hd = 128; float eps = 1e-6f;
};
int conv(const Conv& a) {
  return agnes_gdn_conv(a.x, a.xs, a.y, a.ys, a.dt, a.w, a.b, a.cu, a.n, a.T, a.C, a.K, a.st, a.l2, a.hd, a.eps,
                        nullptr);
}

void conv_cases() {
  EXPECT(conv(WITH(Conv, a.x = nullptr)), INV);
  EXPECT(conv(WITH(Conv, a.dt = BAD_DT)), INV);
  EXPECT(conv(WITH(Conv, a.x = Pt(0, 8))), INV);
  EXPECT(conv(WITH(Conv, (a.C = 500, a.xs = 500, a.ys = 500))), INV);
  EXPECT(conv(WITH(Conv, a.xs = 256)), INV);
  EXPECT(conv(WITH(Conv, a.K = 3)), UNS);
  EXPECT(conv(WITH(Conv, a.hd = 64)), UNS);
  EXPECT(conv(WITH(Conv, a.l2 = 5)), INV);
  EXPECT(conv(WITH(Conv, a.eps = NaN)), INV);
  EXPECT(conv(WITH(Conv, (a.cu = nullptr, a.n = 10, a.T = 10))), INV);
  EXPECT(conv(WITH(Conv, (a.cu = nullptr, a.n = 4, a.T = 10, a.st = P(4)))), INV);
  EXPECT(conv(WITH(Conv, a.n = 0)), INV);
  EXPECT(conv(WITH(Conv, a.y = Pt(0, 512))), INV);
  // extremes
  EXPECT(conv(WITH(Conv, a.T = I64MAX)), INV);             // more tokens than int32 cu_seqlens can hold
  EXPECT(conv(WITH(Conv, a.T = int64_t(1) << 31)), INV);
  EXPECT(conv(WITH(Conv, a.xs = BIG_STRIDE)), INV);        // x's extent wraps the address space
  EXPECT(conv(WITH(Conv, a.ys = BIG_STRIDE)), INV);
  EXPECT(conv(WITH(Conv, (a.C = IMAX & ~7, a.xs = IMAX & ~7, a.ys = IMAX & ~7, a.l2 = IMAX))), INV);
  EXPECT(conv(WITH(Conv, (a.cu = nullptr, a.n = IMAX, a.T = IMAX, a.st = P(4)))), UNS);
  EXPECT(conv(WITH(Conv, (a.n = IMAX, a.st = P(4)))), UNS);
  EXPECT(conv(WITH(Conv, a.n = -1)), INV);
  EXPECT(conv(WITH(Conv, a.T = -1)), INV);
}

// ---- agnes_gdn_prefill_chunked
struct Prefill {
  const void* q = P(0); const void* k = P(1); const void* v = P(2); agnes_dtype dt = BF16; int64_t qs = 2 * 128;
  int64_t vs = 6 * 128; const float* g = Pt<float>(3); const float* b = Pt<float>(4); const int32_t* cu = Pt<int32_t>(5);
  int n = 1; int64_t T = 64; int hk = 2; int hv = 6; int hd = 128; float sc = 1.f; const float* s0 = Pt<float>(6);
  float* s1 = Pt<float>(7); void* o = P(8); agnes_dtype odt = F32; void* ws = nullptr; size_t wsb = 0;
};
int prefill(const Prefill& a) {
  return agnes_gdn_prefill_chunked(a.q, a.k, a.v, a.dt, a.qs, a.vs, a.g, a.b, a.cu, a.n, a.T, a.hk, a.hv, a.hd, a.sc,
                                   a.s0, a.s1, a.o, a.odt, a.ws, a.wsb, nullptr);
}

void prefill_cases() {
  EXPECT(prefill(WITH(Prefill, a.hd = 64)), UNS);
  EXPECT(prefill(WITH(Prefill, a.hv = 5)), UNS);
  EXPECT(prefill(WITH(Prefill, a.q = nullptr)), INV);
  EXPECT(prefill(WITH(Prefill, a.cu = nullptr)), INV);
  EXPECT(prefill(WITH(Prefill, a.q = Pt(0, 2))), INV);
  EXPECT(prefill(WITH(Prefill, a.qs = 100)), INV);
  EXPECT(prefill(WITH(Prefill, a.qs = 2 * 128 + 4)), INV);
  EXPECT(prefill(WITH(Prefill, a.n = 0)), INV);
  EXPECT(prefill(WITH(Prefill, a.n = -1)), INV);
  EXPECT(prefill(WITH(Prefill, a.s1 = Pt<float>(6, 1024))), INV);
  EXPECT(prefill(WITH(Prefill, a.o = Pt(0, 64))), INV);
  EXPECT(prefill(WITH(Prefill, a.sc = Inf)), INV);
  EXPECT(prefill(WITH(Prefill, a.odt = BAD_DT)), INV);
  const size_t need = agnes_gdn_prefill_workspace_size(1, 64, 2, 6, 128, BF16);
  EXPECT(need > 0 && need % 256 == 0, 1);
  EXPECT(prefill(Prefill{}), WS);
  EXPECT(prefill(WITH(Prefill, (a.ws = P(9), a.wsb = need - 1))), WS);
  EXPECT(prefill(WITH(Prefill, (a.ws = Pt(9, 16), a.wsb = need))), WS);
  EXPECT(agnes_gdn_prefill_workspace_size(3, 1000, 2, 6, 128, BF16) > need, 1);
  EXPECT(agnes_gdn_prefill_workspace_size(1, 64, 2, 6, 128, F32), 0);
  EXPECT(agnes_gdn_prefill_workspace_size(1, 64, 2, 6, 64, BF16), 0);
  EXPECT(agnes_gdn_prefill_workspace_size(1, 64, 2, 5, 128, BF16), 0);
  // extremes
  EXPECT(prefill(WITH(Prefill, a.T = I64MAX)), INV);
  EXPECT(prefill(WITH(Prefill, a.qs = BIG_STRIDE)), INV);
  EXPECT(prefill(WITH(Prefill, a.vs = BIG_STRIDE)), INV);
  EXPECT(prefill(WITH(Prefill, (a.hk = IMAX, a.hv = IMAX, a.qs = BIG_STRIDE, a.vs = BIG_STRIDE))), UNS);
  EXPECT(prefill(WITH(Prefill, (a.n = IMAX, a.hv = 6))), UNS);
  EXPECT(agnes_gdn_prefill_workspace_size(1, I64MAX, 2, 6, 128, BF16), 0);
  EXPECT(agnes_gdn_prefill_workspace_size(1 << 18, int64_t(1) << 18, 1, 4, 128, BF16) > 0, 1);
  EXPECT(agnes_gdn_prefill_workspace_size(1 << 18, int64_t(1) << 18, 1, 8, 128, BF16), 0);  // 2^23 scan blocks
  EXPECT(prefill(WITH(Prefill, (a.n = 1 << 18, a.T = 1 << 18, a.hk = 1, a.hv = 8, a.qs = 128, a.vs = 8 * 128,
                                a.q = Far(0), a.k = Far(1), a.v = Far(2), a.o = Far(3), a.s0 = Far<float>(4),
                                a.s1 = Far<float>(5)))), UNS);
  EXPECT(agnes_gdn_prefill_workspace_size(IMAX, IMAX, 1, 1, 128, BF16), 0);
  EXPECT(agnes_gdn_prefill_workspace_size(1, IMAX, 1, 1 << 26, 128, BF16), 0);
  EXPECT(agnes_gdn_prefill_workspace_size(-1, 64, 2, 6, 128, BF16), 0);
  EXPECT(agnes_gdn_prefill_workspace_size(1, -1, 2, 6, 128, BF16), 0);
}

// ---- agnes_gdn_prefill_fused
struct PFused {
  const void* x = P(0); int64_t xs = 10 * 128; agnes_dtype dt = BF16; const void* w = P(1); const void* b = nullptr;
  void* cs = nullptr; const float* g = Pt<float>(3); const float* be = Pt<float>(4); const int32_t* cu = Pt<int32_t>(5);
  int n = 1; int64_t T = 64; int hk = 2; int hv = 6; int hd = 128; float sc = 1.f; float eps = 1e-6f;
  const float* s0 = nullptr; float* s1 = Pt<float>(7); void* o = P(8); agnes_dtype odt = F32; void* ws = nullptr;
  size_t wsb = 0;
};
int pfused(const PFused& a) {
  return agnes_gdn_prefill_fused(a.x, a.xs, a.dt, a.w, a.b, a.cs, a.g, a.be, a.cu, a.n, a.T, a.hk, a.hv, a.hd, a.sc,
                                 a.eps, a.s0, a.s1, a.o, a.odt, a.ws, a.wsb, nullptr);
}

void pfused_cases() {
  EXPECT(pfused(WITH(PFused, a.dt = F32)), UNS);
  EXPECT(pfused(WITH(PFused, a.hd = 64)), UNS);
  EXPECT(pfused(WITH(PFused, (a.hv = 5, a.xs = 9 * 128))), UNS);
  EXPECT(pfused(WITH(PFused, a.w = nullptr)), INV);
  EXPECT(pfused(WITH(PFused, a.x = nullptr)), INV);
  EXPECT(pfused(WITH(PFused, a.xs = 10 * 128 - 8)), INV);
  EXPECT(pfused(WITH(PFused, a.x = Pt(0, 8))), INV);
  EXPECT(pfused(WITH(PFused, a.eps = -1.f)), INV);
  EXPECT(pfused(WITH(PFused, a.o = Pt(0, 64))), INV);
  EXPECT(pfused(WITH(PFused, a.cs = Pt(0, 128))), INV);
  EXPECT(pfused(WITH(PFused, a.n = 0)), INV);
  const size_t need = agnes_gdn_prefill_workspace_size(1, 64, 2, 6, 128, BF16);
  EXPECT(pfused(PFused{}), WS);
  EXPECT(pfused(WITH(PFused, (a.ws = P(9), a.wsb = need - 1))), WS);
  // extremes
  EXPECT(pfused(WITH(PFused, a.T = I64MAX)), INV);
  EXPECT(pfused(WITH(PFused, a.xs = BIG_STRIDE)), INV);
  EXPECT(pfused(WITH(PFused, (a.hk = 1 << 30, a.hv = 1 << 30, a.xs = BIG_STRIDE))), UNS);  // 3 * 2^30 channels
  EXPECT(pfused(WITH(PFused, (a.hk = IMAX, a.hv = IMAX, a.xs = BIG_STRIDE))), UNS);
  // a workspace claimed to run to the end of memory, from below every other buffer
  EXPECT(pfused(WITH(PFused, (a.ws = reinterpret_cast<void*>(256), a.wsb = std::numeric_limits<size_t>::max()))), INV);
  EXPECT(pfused(WITH(PFused, (a.T = 0, a.n = 0, a.x = nullptr, a.o = nullptr))), OK);  // empty batch
}

// ---- agnes_gdn_decode_step
struct Decode {
  const void* q = P(0); const void* k = P(1); const void* v = P(2); agnes_dtype dt = BF16; int64_t qs = 2 * 128;
  int64_t vs = 6 * 128; const float* g = Pt<float>(3); const float* b = Pt<float>(4); int B = 4; int hk = 2; int hv = 6;
  int hd = 128; float sc = 1.f; float* st = Pt<float>(5); void* o = P(6); agnes_dtype odt = F32;
};
int decode(const Decode& a) {
  return agnes_gdn_decode_step(a.q, a.k, a.v, a.dt, a.qs, a.vs, a.g, a.b, a.B, a.hk, a.hv, a.hd, a.sc, a.st, a.o,
                               a.odt, nullptr);
}

void decode_cases() {
  EXPECT(decode(WITH(Decode, a.hd = 96)), UNS);
  EXPECT(decode(WITH(Decode, a.hv = 7)), UNS);
  EXPECT(decode(WITH(Decode, a.st = nullptr)), INV);
  EXPECT(decode(WITH(Decode, a.st = Pt<float>(5, 4))), INV);
  EXPECT(decode(WITH(Decode, a.o = Pt(5, 4096))), INV);
  EXPECT(decode(WITH(Decode, a.B = -1)), INV);
  EXPECT(decode(WITH(Decode, a.vs = 100)), INV);
  // extremes
  EXPECT(decode(WITH(Decode, (a.B = IMAX, a.hk = IMAX, a.hv = IMAX, a.qs = BIG_STRIDE, a.vs = BIG_STRIDE))), UNS);
  EXPECT(decode(WITH(Decode, (a.B = 1 << 24, a.hk = 1, a.hv = 1 << 7, a.vs = BIG_STRIDE))), UNS);  // 2^31 heads
  EXPECT(decode(WITH(Decode, (a.B = 1 << 23, a.hk = 1, a.hv = 1 << 7, a.vs = BIG_STRIDE, a.o = Pt(5, 64)))), INV);
  EXPECT(decode(WITH(Decode, (a.qs = BIG_STRIDE, a.vs = BIG_STRIDE, a.o = Pt(5, 64)))), INV);
  // 2^25 (sequence, head) blocks of 256 threads: beyond one launch
  EXPECT(decode(WITH(Decode, (a.B = 1 << 20, a.hk = 1, a.hv = 32, a.vs = 32 * 128, a.st = Far<float>(0),
                              a.o = Far(2)))), UNS);
}

// ---- agnes_gdn_gated_rmsnorm
struct Norm {
  const void* o = P(0); agnes_dtype odt = BF16; const void* z = P(1); const void* w = P(2); agnes_dtype zdt = BF16;
  float eps = 1e-6f; int64_t rows = 100; int dim = 128; void* y = P(3); agnes_dtype ydt = BF16;
};
int norm(const Norm& a) {
  return agnes_gdn_gated_rmsnorm(a.o, a.odt, a.z, a.w, a.zdt, a.eps, a.rows, a.dim, a.y, a.ydt, nullptr);
}

void norm_cases() {
  EXPECT(norm(WITH(Norm, a.dim = 64)), UNS);
  EXPECT(norm(WITH(Norm, a.rows = -1)), INV);
  EXPECT(norm(WITH(Norm, a.o = nullptr)), INV);
  EXPECT(norm(WITH(Norm, a.y = Pt(0, 256))), INV);
  EXPECT(norm(WITH(Norm, (a.y = P(0), a.ydt = F32))), INV);
  EXPECT(norm(WITH(Norm, a.y = Pt(1, 16))), INV);
  EXPECT(norm(WITH(Norm, a.eps = -1.f)), INV);
  // extremes
  EXPECT(norm(WITH(Norm, a.rows = I64MAX)), INV);           // the rows' extent wraps the address space
  EXPECT(norm(WITH(Norm, (a.rows = int64_t(1) << 40, a.y = P(0)))), INV);  // 256 TiB rows of y run into z
  // 2^34 rows: more blocks than one launch can count
  EXPECT(norm(WITH(Norm, (a.rows = int64_t(1) << 34, a.o = Far(0), a.z = Far(1), a.w = Far(2), a.y = Far(3)))), UNS);
}

// ---- agnes_gdn_decode_fused
struct DFused {
  const void* x = P(0); int64_t xs = 10 * 128; agnes_dtype dt = BF16; const void* w = P(1); const void* b = nullptr;
  void* cs = P(2); const float* g = Pt<float>(3); const float* be = Pt<float>(4); const void* z = P(5);
  const void* nw = P(6); float* st = Pt<float>(7); const int32_t* sl = nullptr; int S = 4; int B = 4; int hk = 2;
  int hv = 6; int hd = 128; float sc = 1.f; float e1 = 1e-6f; float e2 = 1e-6f; void* y = P(8); void* o = nullptr;
  agnes_dtype odt = BF16;
};
int dfused(const DFused& a) {
  return agnes_gdn_decode_fused(a.x, a.xs, a.dt, a.w, a.b, a.cs, a.g, a.be, a.z, a.nw, a.st, a.sl, a.S, a.B, a.hk,
                                a.hv, a.hd, a.sc, a.e1, a.e2, a.y, a.o, a.odt, nullptr);
}

void dfused_cases() {
  EXPECT(dfused(WITH(DFused, (a.B = 0, a.x = nullptr, a.y = nullptr))), OK);
  EXPECT(dfused(WITH(DFused, a.hd = 64)), UNS);
  EXPECT(dfused(WITH(DFused, a.hv = 7)), UNS);
  EXPECT(dfused(WITH(DFused, a.x = nullptr)), INV);
  EXPECT(dfused(WITH(DFused, a.cs = nullptr)), INV);
  EXPECT(dfused(WITH(DFused, a.S = 3)), INV);
  EXPECT(dfused(WITH(DFused, a.xs = 10 * 128 - 8)), INV);
  EXPECT(dfused(WITH(DFused, a.xs = 10 * 128 + 4)), INV);
  EXPECT(dfused(WITH(DFused, a.x = Pt(0, 8))), INV);
  EXPECT(dfused(WITH(DFused, a.st = Pt<float>(7, 4))), INV);
  EXPECT(dfused(WITH(DFused, a.dt = static_cast<agnes_dtype>(5))), INV);
  EXPECT(dfused(WITH(DFused, a.e2 = NaN)), INV);
  EXPECT(dfused(WITH(DFused, a.sc = Inf)), INV);
  EXPECT(dfused(WITH(DFused, a.B = -1)), INV);
  EXPECT(dfused(WITH(DFused, a.y = Pt(7, 4096))), INV);
  EXPECT(dfused(WITH(DFused, a.o = Pt(8, 256))), INV);
  EXPECT(dfused(WITH(DFused, a.cs = Pt(0, 1024))), INV);
  EXPECT(dfused(WITH(DFused, a.y = Pt(5, 64))), INV);
  // extremes
  EXPECT(dfused(WITH(DFused, (a.hk = 1 << 30, a.hv = 1 << 30, a.xs = BIG_STRIDE))), UNS);
  EXPECT(dfused(WITH(DFused, (a.hk = IMAX, a.hv = IMAX, a.xs = BIG_STRIDE))), UNS);
  EXPECT(dfused(WITH(DFused, a.xs = BIG_STRIDE)), INV);
  EXPECT(dfused(WITH(DFused, (a.S = IMAX, a.B = IMAX))), UNS);
  EXPECT(dfused(WITH(DFused, (a.B = 1 << 24, a.S = 4, a.sl = Far<int32_t>(9), a.x = Far(0), a.w = Far(1),
                              a.cs = Far(2), a.g = Far<float>(3), a.be = Far<float>(4), a.z = Far(5),
                              a.nw = Far(6), a.st = Far<float>(7), a.y = Far(8)))), UNS);
}

// ---- agnes_gdn_layer_prefill and its fixed-workspace variant
struct Layer {
  const void* x = P(0); int64_t xs = 10 * 128; agnes_dtype dt = BF16; const void* w = P(1); const void* b = nullptr;
  void* cs = nullptr; const float* g = Pt<float>(3); const float* be = Pt<float>(4); const int32_t* cu = Pt<int32_t>(5);
  int n = 1; int64_t T = 64; int hk = 2; int hv = 6; int hd = 128; float sc = 1.f; float eps = 1e-6f;
  const float* s0 = nullptr; float* s1 = Pt<float>(7); const void* z = P(2); int64_t zs = 6 * 128;
  const void* nw = P(6); float neps = 1e-6f; void* y = P(8); void* o = nullptr; agnes_dtype odt = BF16;
  void* ws = nullptr; size_t wsb = 0;
};
int layer(const Layer& a) {
  return agnes_gdn_layer_prefill(a.x, a.xs, a.dt, a.w, a.b, a.cs, a.g, a.be, a.cu, a.n, a.T, a.hk, a.hv, a.hd, a.sc,
                                 a.eps, a.s0, a.s1, a.z, a.zs, a.nw, a.neps, a.y, a.o, a.odt, a.ws, a.wsb, nullptr);
}
int layer_noalloc(const Layer& a) {
  return agnes_gdn_layer_prefill_noalloc(a.x, a.xs, a.dt, a.w, a.b, a.cs, a.g, a.be, a.cu, a.n, a.T, a.hk, a.hv, a.hd,
                                         a.sc, a.eps, a.s0, a.s1, a.z, a.zs, a.nw, a.neps, a.y, a.o, a.odt, nullptr);
}

void layer_cases() {
  EXPECT(layer(WITH(Layer, a.dt = F32)), UNS);
  EXPECT(layer(WITH(Layer, a.hd = 64)), UNS);
  EXPECT(layer(WITH(Layer, a.z = nullptr)), INV);
  EXPECT(layer(WITH(Layer, a.y = nullptr)), INV);
  EXPECT(layer(WITH(Layer, a.nw = nullptr)), INV);
  EXPECT(layer(WITH(Layer, a.zs = 6 * 128 - 8)), INV);
  EXPECT(layer(WITH(Layer, a.zs = 6 * 128 + 4)), INV);
  EXPECT(layer(WITH(Layer, a.neps = -1.f)), INV);
  EXPECT(layer(WITH(Layer, a.neps = NaN)), INV);
  EXPECT(layer(WITH(Layer, a.y = Pt(2, 256))), INV);
  EXPECT(layer(WITH(Layer, a.o = Pt(8, 512))), INV);
  EXPECT(layer(WITH(Layer, a.y = Pt(0, 64))), INV);
  EXPECT(layer(WITH(Layer, a.n = 0)), INV);
  const size_t need = agnes_gdn_layer_prefill_workspace_size(1, 64, 2, 6, 128);
  EXPECT(need >= agnes_gdn_prefill_workspace_size(1, 64, 2, 6, 128, BF16), 1);
  EXPECT(layer(Layer{}), WS);
  EXPECT(layer(WITH(Layer, (a.ws = P(9), a.wsb = need - 1))), WS);
  EXPECT(agnes_gdn_layer_prefill_workspace_size(1, 64, 2, 5, 128), 0);
  // extremes
  EXPECT(layer(WITH(Layer, a.T = I64MAX)), INV);
  EXPECT(layer(WITH(Layer, a.xs = BIG_STRIDE)), INV);
  EXPECT(layer(WITH(Layer, a.zs = BIG_STRIDE)), INV);
  EXPECT(layer(WITH(Layer, (a.hk = 1 << 30, a.hv = 1 << 30, a.xs = BIG_STRIDE, a.zs = BIG_STRIDE))), UNS);
  EXPECT(layer(WITH(Layer, (a.hk = IMAX, a.hv = IMAX, a.xs = BIG_STRIDE, a.zs = BIG_STRIDE))), UNS);
  EXPECT(agnes_gdn_layer_prefill_workspace_size(1, I64MAX, 2, 6, 128), 0);
  EXPECT(agnes_gdn_layer_prefill_workspace_size(IMAX, IMAX, IMAX, IMAX, 128), 0);
  // the fixed-workspace variant: checks that need no device call
  EXPECT(layer_noalloc(WITH(Layer, a.hd = 64)), UNS);
  EXPECT(layer_noalloc(WITH(Layer, (a.T = 8192, a.hk = 16, a.hv = 48, a.xs = 80 * 128, a.zs = 48 * 128))), UNS);
  EXPECT(layer_noalloc(WITH(Layer, a.T = I64MAX)), INV);
  EXPECT(layer_noalloc(WITH(Layer, (a.T = 0, a.n = 0, a.x = nullptr))), OK);
}

// ---- global attention
struct Attn {
  const void* q = P(0); int64_t qs = 24 * 256; const void* k = P(1); int64_t ks = 4 * 256; const void* v = P(2);
  int64_t vs = 4 * 256; const void* g = P(3); int64_t gs = 24 * 256; const void* qw = P(4);
  const void* kw = Pt(4, 512); const int32_t* pos = nullptr; int64_t ps = 0; const int32_t* cu = Pt<int32_t>(5);
  int n = 1; int64_t T = 100; int hq = 24; int hkv = 4; int hd = 256; int rd = 64; float base = 1e7f;
  float eps = 1e-6f; float sc = 0.f; void* ko = P(6); int64_t kos = 4 * 256; void* vo = nullptr; int64_t vos = 0;
  void* o = P(7); agnes_dtype odt = BF16; void* ws = nullptr; size_t wsb = 0;
};
int attn(const Attn& a) {
  return agnes_attn_prefill(a.q, a.qs, a.k, a.ks, a.v, a.vs, a.g, a.gs, a.qw, a.kw, a.pos, a.ps, a.cu, a.n, a.T, a.hq,
                            a.hkv, a.hd, a.rd, a.base, a.eps, a.sc, a.ko, a.kos, a.vo, a.vos, a.o, a.odt, a.ws, a.wsb,
                            nullptr);
}

void attn_cases() {
  EXPECT(attn(WITH(Attn, (a.n = 0, a.T = 0, a.q = nullptr, a.k = nullptr, a.v = nullptr, a.g = nullptr,
                          a.ko = nullptr, a.o = nullptr))), OK);
  EXPECT(attn(WITH(Attn, a.hd = 128)), UNS);
  EXPECT(attn(WITH(Attn, a.rd = 32)), UNS);
  EXPECT(attn(WITH(Attn, a.hq = 10)), UNS);
  EXPECT(attn(WITH(Attn, a.ko = nullptr)), INV);
  EXPECT(attn(WITH(Attn, a.g = nullptr)), INV);
  EXPECT(attn(WITH(Attn, a.qw = nullptr)), INV);
  EXPECT(attn(WITH(Attn, a.qs = 24 * 256 - 8)), INV);
  EXPECT(attn(WITH(Attn, a.ks = 4 * 256 + 4)), INV);
  EXPECT(attn(WITH(Attn, a.q = Pt(0, 8))), INV);
  EXPECT(attn(WITH(Attn, a.qw = Pt(4, 2))), INV);
  EXPECT(attn(WITH(Attn, (a.pos = Pt<int32_t>(8), a.ps = 99))), INV);
  EXPECT(attn(WITH(Attn, a.base = 0.f)), INV);
  EXPECT(attn(WITH(Attn, a.eps = NaN)), INV);
  EXPECT(attn(WITH(Attn, a.odt = static_cast<agnes_dtype>(5))), INV);
  EXPECT(attn(WITH(Attn, a.n = 0)), INV);
  EXPECT(attn(WITH(Attn, a.o = Pt(0, 512))), INV);
  EXPECT(attn(WITH(Attn, a.ko = P(1))), INV);
  EXPECT(attn(WITH(Attn, (a.vo = Pt(7, 1024), a.vos = 1024))), INV);
  const size_t need = agnes_attn_prefill_workspace_size(1, 100);
  EXPECT(need > 0, 1);
  EXPECT(attn(Attn{}), WS);
  EXPECT(attn(WITH(Attn, (a.ws = P(9), a.wsb = need - 1))), WS);
  EXPECT(attn(WITH(Attn, (a.ws = Pt(9, 16), a.wsb = need))), WS);
  // extremes
  EXPECT(attn(WITH(Attn, a.T = I64MAX)), INV);
  EXPECT(attn(WITH(Attn, (a.T = I64MAX, a.pos = Pt<int32_t>(8), a.ps = I64MAX))), INV);
  EXPECT(attn(WITH(Attn, (a.hq = IMAX, a.hkv = 1, a.qs = BIG_STRIDE, a.gs = BIG_STRIDE))), UNS);
  EXPECT(attn(WITH(Attn, (a.vo = Pt(10), a.vos = BIG_STRIDE))), INV);  // v_out's extent wraps
  // 2^29 tokens of 24 query heads: more query blocks than one launch can count
  EXPECT(attn(WITH(Attn, (a.T = int64_t(1) << 29, a.q = Far(0), a.k = Far(1), a.v = Far(2), a.g = Far(3),
                          a.ko = Far(4), a.o = Far(5)))), UNS);
  EXPECT(agnes_attn_prefill_workspace_size(IMAX, I64MAX), 0);
  EXPECT(agnes_attn_prefill_workspace_size(-1, 100), 0);
}

struct ADec {
  const void* q = P(0); int64_t qs = 24 * 256; const void* k = P(1); int64_t ks = 4 * 256; const void* v = P(2);
  int64_t vs = 4 * 256; const void* g = P(3); int64_t gs = 24 * 256; const void* qw = P(4);
  const void* kw = Pt(4, 512); const int32_t* pos = nullptr; int64_t ps = 0; void* kc = P(5); void* vc = P(6);
  int64_t L = 1000; const int32_t* lens = Pt<int32_t>(7); int B = 8; int hq = 24; int hkv = 4; int hd = 256;
  int rd = 64; float base = 1e7f; float eps = 1e-6f; float sc = 0.f; void* o = P(8); agnes_dtype odt = BF16;
  void* ws = nullptr; size_t wsb = 0;
};
int adec(const ADec& a) {
  return agnes_attn_decode(a.q, a.qs, a.k, a.ks, a.v, a.vs, a.g, a.gs, a.qw, a.kw, a.pos, a.ps, a.kc, a.vc, a.L,
                           a.lens, a.B, a.hq, a.hkv, a.hd, a.rd, a.base, a.eps, a.sc, a.o, a.odt, a.ws, a.wsb,
                           nullptr);
}

void adec_cases() {
  EXPECT(adec(WITH(ADec, (a.B = 0, a.q = nullptr, a.kc = nullptr))), OK);
  EXPECT(adec(WITH(ADec, a.hd = 128)), UNS);
  EXPECT(adec(WITH(ADec, a.hq = 22)), UNS);
  EXPECT(adec(WITH(ADec, a.L = 0)), INV);
  EXPECT(adec(WITH(ADec, a.kc = nullptr)), INV);
  EXPECT(adec(WITH(ADec, a.lens = nullptr)), INV);
  EXPECT(adec(WITH(ADec, a.qs = 24 * 256 - 8)), INV);
  EXPECT(adec(WITH(ADec, a.vs = 4 * 256 + 4)), INV);
  EXPECT(adec(WITH(ADec, a.kc = Pt(5, 8))), INV);
  EXPECT(adec(WITH(ADec, (a.pos = Pt<int32_t>(9), a.ps = 7))), INV);
  EXPECT(adec(WITH(ADec, a.sc = NaN)), INV);
  EXPECT(adec(WITH(ADec, a.vc = Pt(5, 4096))), INV);
  EXPECT(adec(WITH(ADec, a.o = Pt(0, 1024))), INV);
  const size_t need = agnes_attn_decode_workspace_size(8, 24, 4, 1000);
  EXPECT(need > 0, 1);
  EXPECT(adec(ADec{}), WS);
  EXPECT(adec(WITH(ADec, (a.ws = P(10), a.wsb = need - 1))), WS);
  // extremes
  EXPECT(adec(WITH(ADec, a.L = I64MAX)), UNS);
  EXPECT(adec(WITH(ADec, (a.B = IMAX, a.hq = IMAX, a.hkv = IMAX, a.L = 1 << 30, a.qs = BIG_STRIDE,
                          a.ks = BIG_STRIDE, a.vs = BIG_STRIDE, a.gs = BIG_STRIDE))), INV);  // o's extent wraps
  EXPECT(adec(WITH(ADec, (a.B = IMAX, a.L = 1 << 30))), INV);   // 2^61 cache rows: the caches overlap
  EXPECT(adec(WITH(ADec, (a.B = 1 << 24, a.L = 1, a.q = Far(0), a.k = Far(1), a.v = Far(2), a.g = Far(3),
                          a.kc = Far(4), a.vc = Far(5), a.lens = Far<int32_t>(6), a.o = Far(7)))), UNS);
  EXPECT(agnes_attn_decode_workspace_size(IMAX, IMAX, IMAX, I64MAX), 0);
  EXPECT(agnes_attn_decode_workspace_size(IMAX, IMAX, 1, 1 << 30), 0);
}

// ---- status, settings and measurement calls
void misc_cases() {
  EXPECT(agnes_gdn_version() != nullptr, 1);
  for (int s = -8; s <= 4; ++s) EXPECT(agnes_gdn_status_string(s) != nullptr, 1);
  uint32_t flags = 7;
  EXPECT(agnes_gdn_workspace_status(nullptr, &flags, nullptr), INV);
  EXPECT(agnes_gdn_workspace_status(P(0), nullptr, nullptr), INV);
  EXPECT(agnes_gdn_workspace_status(Pt(0, 2), &flags, nullptr), INV);
  EXPECT(flags, 7u);
  EXPECT(agnes_gdn_set_wait_limit(0), OK);
  EXPECT(agnes_gdn_set_wait_limit(0xffffffffu), OK);
  EXPECT(agnes_gdn_set_wait_limit(0), OK);
  EXPECT(agnes_gdn_ceiling_rmw_stream(nullptr, 1024, nullptr), INV);
  EXPECT(agnes_gdn_ceiling_rmw_stream(P(0), 1000, nullptr), INV);
  EXPECT(agnes_gdn_ceiling_rmw_stream(Pt(0, 8), 1024, nullptr), INV);
  EXPECT(agnes_gdn_ceiling_mfma(nullptr, 4, 4, nullptr), INV);
  EXPECT(agnes_gdn_ceiling_mfma(Pt<float>(0), 0, 4, nullptr), INV);
  EXPECT(agnes_gdn_ceiling_mfma(Pt<float>(0), 4, (1 << 20) + 1, nullptr), INV);
  EXPECT(agnes_gdn_ceiling_mfma(Pt<float>(0), IMAX, IMAX, nullptr), INV);
  const int32_t bad[][8] = {{0}, {40}, {24, 24}, {30, 20}, {-1}, {1, 2, 3, 4, 5, 6, 7, 8}, {IMAX}};
  const int nbad[] = {1, 1, 2, 2, 1, 8, 1};
  for (int i = 0; i < 7; ++i) EXPECT(agnes_gdn_set_prefill_stages(bad[i], nbad[i]), INV);
  EXPECT(agnes_gdn_set_prefill_stages(nullptr, 1), INV);
  EXPECT(agnes_gdn_set_prefill_stages(nullptr, -2), INV);
  EXPECT(agnes_gdn_set_prefill_stages(nullptr, -IMAX - 1), INV);
  EXPECT(agnes_gdn_set_prefill_stages(nullptr, IMAX), INV);
  EXPECT(agnes_gdn_set_prefill_stages(nullptr, 0), OK);
  const int32_t seven[] = {1, 2, 3, 4, 5, 6, 39};
  EXPECT(agnes_gdn_set_prefill_stages(seven, 7), OK);
  const int32_t dflt[] = {26};
  EXPECT(agnes_gdn_set_prefill_stages(dflt, 1), OK);
  EXPECT(agnes_gdn_set_prefill_stages(nullptr, -1), OK);  // the defaults again
  EXPECT(agnes_gdn_last_hip_error(), 0);
  EXPECT(agnes_gdn_release(), OK);  // nothing was created: no device call
}

}  // namespace

int main() {
  conv_cases();
  prefill_cases();
  pfused_cases();
  decode_cases();
  norm_cases();
  dfused_cases();
  layer_cases();
  attn_cases();
  adec_cases();
  misc_cases();
  EXPECT(agnes_gdn_last_hip_error(), 0);  // no case reached the device
  if (g_fail) {
    std::fprintf(stderr, "%d check(s) failed\n", g_fail);
    return 1;
  }
  std::printf("abi host checks: all passed\n");
  return 0;
}
