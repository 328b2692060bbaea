// Device helpers shared by the libpagedkv kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf162_t __attribute__((ext_vector_type(2)));

enum { DT_F16 = 0, DT_BF16 = 1 };

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

// a.x*b.x + a.y*b.y + c on two packed 16-bit pairs, float32 accumulate
// (v_dot2c_f32_f16 / v_dot2c_f32_bf16); the 16-bit products are exact in f32.
template <int DT>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c);

template <>
__device__ __forceinline__ float dot2<DT_F16>(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b), c,
                                false);
}

template <>
__device__ __forceinline__ float dot2<DT_BF16>(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, a),
                                         __builtin_bit_cast(bf162_t, b), c, false);
}

// Dot product of 8 packed elements held by one lane.
template <int DT>
__device__ __forceinline__ float dot8(const u32x4 &q, const u32x4 &k) {
  float acc = dot2<DT>(q.x, k.x, 0.f);
  acc = dot2<DT>(q.y, k.y, acc);
  acc = dot2<DT>(q.z, k.z, acc);
  acc = dot2<DT>(q.w, k.w, acc);
  return acc;
}

// Low / high element of a packed pair, widened exactly to f32.
template <int DT>
__device__ __forceinline__ float lo16(uint32_t w);
template <int DT>
__device__ __forceinline__ float hi16(uint32_t w);

template <>
__device__ __forceinline__ float lo16<DT_F16>(uint32_t w) {
  return (float)__builtin_bit_cast(half2_t, w).x;
}
template <>
__device__ __forceinline__ float hi16<DT_F16>(uint32_t w) {
  return (float)__builtin_bit_cast(half2_t, w).y;
}
template <>
__device__ __forceinline__ float lo16<DT_BF16>(uint32_t w) {
  return __uint_as_float(w << 16);
}
template <>
__device__ __forceinline__ float hi16<DT_BF16>(uint32_t w) {
  return __uint_as_float(w & 0xFFFF0000u);
}

// f32 -> 16-bit pattern, round to nearest even.
template <int DT>
__device__ __forceinline__ uint16_t to16(float x);

template <>
__device__ __forceinline__ uint16_t to16<DT_F16>(float x) {
  return __builtin_bit_cast(uint16_t, (_Float16)x);
}
template <>
__device__ __forceinline__ uint16_t to16<DT_BF16>(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0;  // NaN stays NaN
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Cross-lane moves inside a 16-lane DPP row (row_mask / bank_mask all on).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
constexpr int DPP_QUAD_XOR1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_XOR2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int DPP_ROW_HALF_MIRROR = 0x141;
constexpr int DPP_ROW_MIRROR = 0x140;

// Sum over groups of N consecutive lanes (N = 8 or 16); every lane of the
// group ends with the same bits (each step adds a value to its mirror image,
// which is commutative).
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 8 || N == 16, "group of 8 or 16 lanes");
  x += dpp<DPP_QUAD_XOR1>(x);
  x += dpp<DPP_QUAD_XOR2>(x);
  x += dpp<DPP_ROW_HALF_MIRROR>(x);
  if constexpr (N == 16) x += dpp<DPP_ROW_MIRROR>(x);
  return x;
}

// A 16-byte piece of a K/V row, read once per call.  NT: a non-temporal
// load (the line is streamed past the caches and does not displace reused
// data); else an ordinary cached load, for pools whose blocks are read more
// than once in a call (shared prefixes).
template <bool NT>
__device__ __forceinline__ u32x4 ld_kv(const void *p) {
  if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
  else return *reinterpret_cast<const u32x4 *>(p);
}

// 8 bytes of a K/V row (FP8 pools), the same load policy.
template <bool NT>
__device__ __forceinline__ uint32_t __attribute__((ext_vector_type(2))) ld_kv8(const void *p) {
  typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
  if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const u32x2_t *>(p));
  else return *reinterpret_cast<const u32x2_t *>(p);
}

// 2^x on the hardware unit (v_exp_f32); 2^0 is exactly 1 and 2^-inf is 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Workgroup ids are handed to the 8 XCDs round-robin.  Remap so that G
// consecutive logical items run on one XCD (they share its L2) while
// successive groups still spread over all XCDs.  `grid` must be a multiple of
// 8 * G.
template <int G>
__device__ __forceinline__ int xcd_remap(int i) {
  const int x = i & 7;
  const int j = i >> 3;
  return (j / G) * (8 * G) + x * G + (j % G);
}

// FP8 (OCP e4m3) quantisation, shared by the append and the decode step:
// code = the e4m3 value nearest to float32(x * inv), ties to even, with the
// product saturated to +-448 first (the conversion itself does not
// saturate); NaN stays NaN.
__device__ __forceinline__ float sat448(float y) { return (y != y) ? y : fminf(fmaxf(y, -448.f), 448.f); }

__device__ __forceinline__ uint32_t quant4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(sat448(a), sat448(b), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(sat448(c), sat448(d), w, true);
  return (uint32_t)w;
}

// 16 consecutive 16-bit elements (two 16-byte pieces) -> their 16 codes.
template <int DT>
__device__ __forceinline__ u32x4 quant16(const u32x4 &a, const u32x4 &b, float inv) {
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  uint32_t o[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    o[j] = quant4(lo16<DT>(w[2 * j]) * inv, hi16<DT>(w[2 * j]) * inv, lo16<DT>(w[2 * j + 1]) * inv,
                  hi16<DT>(w[2 * j + 1]) * inv);
  return u32x4{o[0], o[1], o[2], o[3]};
}

}  // namespace pkv
