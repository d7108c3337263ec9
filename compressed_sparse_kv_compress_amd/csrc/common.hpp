// Device helpers shared by the gfx950 kernels of the CSA / HCA library.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Storage element types.  bf16 is carried as its raw 16-bit pattern.
struct bf16_t {
  uint16_t bits;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest even (finite inputs; NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u) return static_cast<uint16_t>((u >> 16) | ((u & 0xffff) ? 0x40 : 0));
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Unpack the low / high bf16 of a 32-bit word.
__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return static_cast<uint32_t>(f32_to_bf16(a)) | (static_cast<uint32_t>(f32_to_bf16(b)) << 16);
}

// 2^x on the hardware exp unit (inputs are already scaled by log2(e)).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Cross-lane data movement by DPP (a VALU operand modifier, no LDS round
// trip as with __shfl): row_shr:n reads lane i-n within a row of 16 lanes;
// row_bcast:15 and row_bcast:31 read the last lane of the previous row
// (rows 1, 3) and lane 31 (rows 2, 3).  Lanes with no source keep `id`.
template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ uint32_t dpp(uint32_t id, uint32_t v) {
  return static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(static_cast<int>(id), static_cast<int>(v), CTRL, ROWS, 0xf, false));
}
constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118;
constexpr int kRowBcast15 = 0x142, kRowBcast31 = 0x143;

// Value of lane 63 as a wave-uniform scalar.
__device__ __forceinline__ uint32_t last_lane(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 63));
}

// Inclusive scan of op over the 64 lanes (identity id); lane 63 ends with the total.
template <typename Op>
__device__ __forceinline__ float wave_scan_f(float v, uint32_t id, Op op) {
  v = op(v, __uint_as_float(dpp<kRowShr1>(id, __float_as_uint(v))));
  v = op(v, __uint_as_float(dpp<kRowShr2>(id, __float_as_uint(v))));
  v = op(v, __uint_as_float(dpp<kRowShr4>(id, __float_as_uint(v))));
  v = op(v, __uint_as_float(dpp<kRowShr8>(id, __float_as_uint(v))));
  v = op(v, __uint_as_float(dpp<kRowBcast15, 0xa>(id, __float_as_uint(v))));
  v = op(v, __uint_as_float(dpp<kRowBcast31, 0xc>(id, __float_as_uint(v))));
  return v;
}

// Sum / max over the four 16-lane groups of a wavefront (lanes l, l^16, l^32,
// l^48), returned to all four: the gfx950 row-swap permutes exchange the
// groups pairwise without an LDS round trip.
__device__ __forceinline__ float group_sum4(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto p = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const float y = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  const uint32_t v = __float_as_uint(y);
  const auto q = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}
__device__ __forceinline__ float group_max4(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto p = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const float y = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
  const uint32_t v = __float_as_uint(y);
  const auto q = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}

// Max / sum over the wavefront, returned to every lane (wave-uniform).
__device__ __forceinline__ float wave_max(float v) {
  v = wave_scan_f(v, 0xff800000u, [](float a, float b) { return fmaxf(a, b); });
  return __uint_as_float(last_lane(__float_as_uint(v)));
}
__device__ __forceinline__ float wave_sum(float v) {
  v = wave_scan_f(v, 0u, [](float a, float b) { return a + b; });
  return __uint_as_float(last_lane(__float_as_uint(v)));
}

// Order-preserving map float -> uint32 with -0 and +0 mapped together.
__device__ __forceinline__ uint32_t float_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u << 1) == 0) u = 0;  // -0 -> +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_float(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}

}  // namespace csa
