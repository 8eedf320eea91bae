// Device helpers shared by the gfx950 kernels of the gated delta-rule layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace agnes {

enum : int { DT_F32 = 0, DT_BF16 = 1 };

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- bf16 storage
__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two fp32 values rounded to nearest even into packed bf16 (low half = lo); NaN stays NaN.
// One hardware conversion on gfx950.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}
__device__ __forceinline__ uint32_t f32_to_bf16(float f) { return pack_bf16x2(f, 0.f) & 0xffffu; }

// 8 consecutive elements of a DT tensor as fp32 (16-byte aligned for bf16, 32 for f32).
template <int DT>
__device__ __forceinline__ void load8(const void* base, int64_t idx, float out[8]) {
  if constexpr (DT == DT_BF16) {
    uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + idx);
    uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(w[i] << 16);
      out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + idx);
    float4 a = p[0], b = p[1];
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
    out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
  }
}

// 8 consecutive elements kept as loaded (bf16: one 16-byte vector, f32: two), so that many
// can be in flight in few registers; widen8 converts to fp32 at the point of use.
template <int DT>
struct Raw8 {
  uint4 u[DT == DT_BF16 ? 1 : 2];
};
template <int DT>
__device__ __forceinline__ Raw8<DT> load_raw8(const void* base, int64_t idx) {
  Raw8<DT> r;
  if constexpr (DT == DT_BF16) {
    r.u[0] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + idx);
  } else {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const float*>(base) + idx);
    r.u[0] = p[0];
    r.u[1] = p[1];
  }
  return r;
}
template <int DT>
__device__ __forceinline__ void widen8(const Raw8<DT>& r, float out[8]) {
  if constexpr (DT == DT_BF16) {
    const uint32_t w[4] = {r.u[0].x, r.u[0].y, r.u[0].z, r.u[0].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(w[i] << 16);
      out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  } else {
    const uint32_t w[8] = {r.u[0].x, r.u[0].y, r.u[0].z, r.u[0].w, r.u[1].x, r.u[1].y, r.u[1].z, r.u[1].w};
#pragma unroll
    for (int i = 0; i < 8; ++i) out[i] = __uint_as_float(w[i]);
  }
}

// Element i (0..8n-1) of n consecutive raw 8-element loads, as fp32.
template <int DT>
__device__ __forceinline__ float raw_at(const Raw8<DT>* r, int i) {
  if constexpr (DT == DT_BF16) {
    const uint4 u = r[i >> 3].u[0];
    const uint32_t wd = ((i & 7) >> 1) == 0 ? u.x : ((i & 7) >> 1) == 1 ? u.y : ((i & 7) >> 1) == 2 ? u.z : u.w;
    return __uint_as_float((i & 1) ? (wd & 0xffff0000u) : (wd << 16));
  } else {
    const uint4 u = r[i >> 3].u[(i & 7) >> 2];
    const uint32_t wd = (i & 3) == 0 ? u.x : (i & 3) == 1 ? u.y : (i & 3) == 2 ? u.z : u.w;
    return __uint_as_float(wd);
  }
}

template <int DT>
__device__ __forceinline__ void store8(void* base, int64_t idx, const float v[8]) {
  if constexpr (DT == DT_BF16) {
    uint4 u;
    u.x = pack_bf16x2(v[0], v[1]);
    u.y = pack_bf16x2(v[2], v[3]);
    u.z = pack_bf16x2(v[4], v[5]);
    u.w = pack_bf16x2(v[6], v[7]);
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(base) + idx) = u;
  } else {
    float4* p = reinterpret_cast<float4*>(static_cast<float*>(base) + idx);
    p[0] = make_float4(v[0], v[1], v[2], v[3]);
    p[1] = make_float4(v[4], v[5], v[6], v[7]);
  }
}

// store8 with non-temporal stores (outputs nothing in the same kernel reads back).  For a
// streamed output they leave the caches to the inputs: the conv's y this way runs 30 % faster
// than with plain stores.
template <int DT>
__device__ __forceinline__ void store8_nt(void* base, int64_t idx, const float v[8]) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  if constexpr (DT == DT_BF16) {
    const u32x4 u = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                     pack_bf16x2(v[6], v[7])};
    __builtin_nontemporal_store(u, reinterpret_cast<u32x4*>(static_cast<uint16_t*>(base) + idx));
  } else {
    f32x4* p = reinterpret_cast<f32x4*>(static_cast<float*>(base) + idx);
    __builtin_nontemporal_store(f32x4{v[0], v[1], v[2], v[3]}, p);
    __builtin_nontemporal_store(f32x4{v[4], v[5], v[6], v[7]}, p + 1);
  }
}

// A 16-byte fp32 vector read or written with the non-temporal hint, for data a kernel streams
// through exactly once in each direction, such as a recurrent state updated in place: on gfx950
// the pair (streaming load, then streaming store of the same line) runs the decode step's
// read-modify-write 12 % faster than plain accesses (measured; either one alone does not help).
__device__ __forceinline__ f4 load_f4_stream(const float* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const f4*>(p));
}
__device__ __forceinline__ void store_f4_stream(float* p, f4 v) { __builtin_nontemporal_store(v, reinterpret_cast<f4*>(p)); }

// 4 consecutive values (8-byte aligned for bf16, 16 for f32).
template <int DT>
__device__ __forceinline__ void store4(void* base, int64_t idx, f4 v) {
  if constexpr (DT == DT_BF16) {
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(base) + idx) =
        make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
  } else {
    *reinterpret_cast<float4*>(static_cast<float*>(base) + idx) = make_float4(v[0], v[1], v[2], v[3]);
  }
}

template <int DT>
__device__ __forceinline__ float load1(const void* base, int64_t idx) {
  if constexpr (DT == DT_BF16) return bf16_to_f32(static_cast<const uint16_t*>(base)[idx]);
  else return static_cast<const float*>(base)[idx];
}

template <int DT>
__device__ __forceinline__ void store1(void* base, int64_t idx, float v) {
  if constexpr (DT == DT_BF16) static_cast<uint16_t*>(base)[idx] = (uint16_t)f32_to_bf16(v);
  else static_cast<float*>(base)[idx] = v;
}

// ---------------------------------------------------------------- causal conv, kernel 4
// bias + sum_j w[e][j] x_j[e] for 8 channels e of one output row: x_j are the row's four input
// rows (bf16 as loaded, oldest first), w the channels' taps as stored ([channel][4] bf16: for
// channel e, dword 2e holds taps 0, 1 and dword 2e+1 taps 2, 3).  Each channel takes two bf16
// dot products (exact bf16 x bf16 products, fp32 sums); pairs of one channel's inputs from two
// rows are gathered with byte permutes.
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, a), __builtin_bit_cast(bf16x2v, b), c, false);
}
__device__ __forceinline__ uint32_t dw(const uint4& u, int i) { return i == 0 ? u.x : i == 1 ? u.y : i == 2 ? u.z : u.w; }
__device__ __forceinline__ void conv4_bf16x8(const uint4 (&x)[4], const uint4 (&w)[4], const float (&bias)[8],
                                             float (&acc)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {  // dword i of a row: channels 2i (low half), 2i+1 (high half)
    const uint32_t a0 = dw(x[0], i), a1 = dw(x[1], i), a2 = dw(x[2], i), a3 = dw(x[3], i);
    const uint32_t p01l = __builtin_amdgcn_perm(a1, a0, 0x05040100u), p01h = __builtin_amdgcn_perm(a1, a0, 0x07060302u);
    const uint32_t p23l = __builtin_amdgcn_perm(a3, a2, 0x05040100u), p23h = __builtin_amdgcn_perm(a3, a2, 0x07060302u);
    acc[2 * i] = dot2_bf16(dw(w[i], 1), p23l, dot2_bf16(dw(w[i], 0), p01l, bias[2 * i]));
    acc[2 * i + 1] = dot2_bf16(dw(w[i], 3), p23h, dot2_bf16(dw(w[i], 2), p01h, bias[2 * i + 1]));
  }
}

// ---------------------------------------------------------------- reductions
// Sum over each aligned group of 16 lanes (a DPP row); every lane gets its group's sum.
__device__ __forceinline__ float sum16(float v) {
  v += __shfl_xor(v, 1, 16);
  v += __shfl_xor(v, 2, 16);
  v += __shfl_xor(v, 4, 16);
  v += __shfl_xor(v, 8, 16);
  return v;
}
// The same sum through DPP lane moves within each 16-lane row (one VALU operation per step
// instead of an LDS permute and its index arithmetic): swap neighbours, swap pairs, then add the
// mirrored half-row and the mirrored row.  Each step adds lane values from the other half of the
// current group, so after four steps every lane holds its row's sum (in another summation order
// than sum16).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xf, 0xf, true));
}
__device__ __forceinline__ float sum16_dpp(float v) {
  v += dpp_f<0xB1>(v);   // quad_perm [1, 0, 3, 2]: lane ^ 1
  v += dpp_f<0x4E>(v);   // quad_perm [2, 3, 0, 1]: lane ^ 2
  v += dpp_f<0x141>(v);  // row_half_mirror: lane 7 - i of each 8
  v += dpp_f<0x140>(v);  // row_mirror: lane 15 - i of each 16
  return v;
}

// x * sigmoid(x) with the hardware exp2 and reciprocal (each within about 1 ulp).
__device__ __forceinline__ float silu(float u) { return u * __builtin_amdgcn_rcpf(1.0f + __expf(-u)); }
// 1 / sqrt(x), hardware estimate (within about 1 ulp).
__device__ __forceinline__ float rsqrt_fast(float x) { return __builtin_amdgcn_rsqf(x); }

// ---------------------------------------------------------------- matrix cores
// D = A(16x32) B(32x16) + C.  Lane l holds A[l%16][8(l/16)+e], B[8(l/16)+e][l%16],
// and D[4(l/16)+i][l%16] (i = 0..3).
__device__ __forceinline__ f4 mfma_16x16x32(h8 a, h8 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
// D = A(16x16) B(16x16) + C.  Lane l holds A[l%16][4(l/16)+e], B[4(l/16)+e][l%16],
// D[4(l/16)+i][l%16]: the D fragment is already in B-operand order.
__device__ __forceinline__ f4 mfma_16x16x16(h4 a, h4 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ h4 to_h4(f4 v) {
  h4 r;
  r[0] = (_Float16)v[0]; r[1] = (_Float16)v[1]; r[2] = (_Float16)v[2]; r[3] = (_Float16)v[3];
  return r;
}

// Clamp a device cu_seqlens entry into [0, total].
__device__ __forceinline__ int64_t cu_at(const int32_t* cu, int i, int64_t total) {
  int64_t v = cu[i];
  return v < 0 ? 0 : (v > total ? total : v);
}

}  // namespace agnes
