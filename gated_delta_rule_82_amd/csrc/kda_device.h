// kda_device.h - device-side numerics shared by the libkda kernels:
// bf16 conversion, the transcendentals of the gate, and the DPP / row-swap
// cross-lane moves of a 64-lane wavefront.  Included by the .hip sources
// only; everything has internal linkage.
#ifndef KDA_DEVICE_H_
#define KDA_DEVICE_H_

#include <hip/hip_runtime.h>

#include <cstdint>

namespace kda {
namespace {

constexpr int kWave = 64;
constexpr int kXcds = 8;

// ---------------------------------------------------------------------------
// numbers
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// fp32 -> bf16, round to nearest, ties to even; NaN stays a quiet NaN.
// The gfx950 conversion instruction (v_cvt_pk_bf16_f32) does it for two
// values at once; on the GPU it matched the bit formula
// (u + 0x7fff + ((u >> 16) & 1)) >> 16, NaN quieted, on every one of 16.7 M
// inputs (ties at every exponent, denormals, infinities, NaN payloads).
// The formula costs about five instructions per value, which is what a
// multi-token decode on a bf16 pool is short of.
typedef __bf16 kda_bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t f32x2_to_bf16x2_rne(float lo, float hi) {
  const kda_bf16x2 h = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, h);   // lo in bits 0..15
}

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

// Transcendentals use the hardware exp2 / log2 / rcp / rsqrt instructions
// (about 1 ulp each).  ln(1 + y) keeps full relative accuracy for small y
// through the correction of Goldberg, "What every computer scientist should
// know about floating-point arithmetic" (1991), Theorem 4:
// ln(1 + y) = y * ln(w) / (w - 1) with w = fl(1 + y), and = y when w == 1.
// The correction factor is within a few ulps of 1, so it takes the
// hardware reciprocal (1 ulp) rather than an IEEE division (a ten-
// instruction sequence, per channel and token).
__device__ __forceinline__ float exp_f(float x) { return __expf(x); }

__device__ __forceinline__ float log1p_f(float y) {
  const float w = 1.0f + y;
  return w == 1.0f ? y : __logf(w) * (y * __builtin_amdgcn_rcpf(w - 1.0f));
}

__device__ __forceinline__ float softplus_f(float x) {
  return fmaxf(x, 0.0f) + log1p_f(exp_f(-fabsf(x)));
}

__device__ __forceinline__ float sigmoid_f(float x) {
  return __builtin_amdgcn_rcpf(1.0f + exp_f(-x));
}

__device__ __forceinline__ float rsqrt_f(float x) { return __builtin_amdgcn_rsqf(x); }

// ---------------------------------------------------------------------------
// cross-lane moves: DPP reads a neighbour lane inside a 16-lane row;
// v_permlane16_swap / v_permlane32_swap (gfx950) exchange whole rows
// ---------------------------------------------------------------------------

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
constexpr int kDppXor1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int kDppQuadReverse = 0x1B;  // quad_perm [3,2,1,0]: lane ^ 3
constexpr int kDppHalfMirror = 0x141;  // lane 7 - i within each group of 8
constexpr int kDppRowRor4 = 0x124;     // lane (i + 4) mod 16 of the row
constexpr int kDppRowRor8 = 0x128;     // lane (i + 8) mod 16 = lane ^ 8

// lane ^ 4: the half-row mirror (7 - i) read through the quad reversal (i ^ 3)
__device__ __forceinline__ float dpp_xor4(float x) {
  return dpp<kDppQuadReverse>(dpp<kDppHalfMirror>(x));
}

// Both return keep + the partner's value, where lanes in the lower half of
// each pair of rows keep `lo` and the upper half keep `hi`:
//   swap16: partner lane ^ 16; swap32: partner lane ^ 32.
__device__ __forceinline__ float swap16_add(float lo, float hi) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(lo), __float_as_uint(hi), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

__device__ __forceinline__ float swap32_add(float lo, float hi) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(lo), __float_as_uint(hi), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// One transpose-reduce level through a within-row DPP move: lanes whose
// level bit is clear (up == false) keep `lo` and receive the partner's `lo`,
// the others keep `hi` and receive the partner's `hi`.
template <int XOR>
__device__ __forceinline__ float dpp_level(bool up, float lo, float hi) {
  const float send = up ? lo : hi;
  const float keep = up ? hi : lo;
  if constexpr (XOR == 1) return keep + dpp<kDppXor1>(send);
  else if constexpr (XOR == 2) return keep + dpp<kDppXor2>(send);
  else if constexpr (XOR == 4) return keep + dpp_xor4(send);
  else return keep + dpp<kDppRowRor8>(send);
}

__device__ __forceinline__ float wave_sum(float x) {
  x += dpp<kDppXor1>(x);
  x += dpp<kDppXor2>(x);
  x += dpp<kDppRowRor4>(x);
  x += dpp<kDppRowRor8>(x);
  x = swap16_add(x, x);
  return swap32_add(x, x);
}

}  // namespace
}  // namespace kda

#endif  // KDA_DEVICE_H_
