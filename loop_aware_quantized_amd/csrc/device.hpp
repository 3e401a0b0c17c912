// device.hpp -- small device helpers shared by the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace lkv {

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

__device__ __forceinline__ float f16_to_f32(uint32_t bits16) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits16)));
}

__device__ __forceinline__ uint16_t f16_bits_rne(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
}

// Next fp16 bit pattern towards -inf / +inf (finite or infinite input).
__device__ __forceinline__ uint16_t f16_next_down(uint16_t h) {
  if ((h & 0x7fffu) == 0) return 0x8001u;          // +-0 -> -min subnormal
  return (h & 0x8000u) ? static_cast<uint16_t>(h + 1) : static_cast<uint16_t>(h - 1);
}
__device__ __forceinline__ uint16_t f16_next_up(uint16_t h) {
  if ((h & 0x7fffu) == 0) return 0x0001u;
  return (h & 0x8000u) ? static_cast<uint16_t>(h - 1) : static_cast<uint16_t>(h + 1);
}

// Largest fp16 <= x and smallest fp16 >= x (directed conversions built on
// the hardware's round-to-nearest-even conversion).
__device__ __forceinline__ uint16_t f16_round_down_bits(float x) {
  uint16_t h = f16_bits_rne(x);
  if (f16_to_f32(h) > x) h = f16_next_down(h);
  return h;
}
__device__ __forceinline__ uint16_t f16_round_up_bits(float x) {
  uint16_t h = f16_bits_rne(x);
  if (f16_to_f32(h) < x) h = f16_next_up(h);
  return h;
}

// Quantizer parameters of one group: zero = fp16 round-down of the minimum,
// scale = fp16 round-up of fp32((max - zero) / levels).
struct QParams {
  uint16_t zbits, sbits;
  float z, s;
};

__device__ __forceinline__ QParams qparams(float mn, float mx, float levels) {
  QParams q;
  q.zbits = f16_round_down_bits(mn);
  q.z = f16_to_f32(q.zbits);
  const float r = mx - q.z;          // IEEE fp32 subtraction
  const float s32 = r / levels;      // IEEE fp32 division (no fast-math)
  q.sbits = f16_round_up_bits(s32);
  q.s = f16_to_f32(q.sbits);
  return q;
}

// code = clamp(rint_even(fp32(fp32(x - z) / s)), 0, levels); 0 when s == 0.
__device__ __forceinline__ uint32_t qcode(float x, const QParams& q, float levels) {
  if (!(q.s > 0.0f)) return 0u;
  const float t = (x - q.z) / q.s;
  float c = __builtin_rintf(t);
  c = fminf(fmaxf(c, 0.0f), levels);
  return static_cast<uint32_t>(c);
}

template <typename T>
__device__ __forceinline__ T wave_max(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Sum over the 32 lanes of each half-wave.
__device__ __forceinline__ float half_wave_sum(float v) {
#pragma unroll
  for (int o = 16; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// ---- wave reductions on DPP row operations (no LDS round trips) ----------
// DPP controls: quad_perm [1,0,3,2] = 0xB1, quad_perm [2,3,0,1] = 0x4E,
// row_half_mirror = 0x141, row_mirror = 0x140.
template <int kCtrl>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF, false));
}

// Sum over the lanes l' with l' = l (mod kStride), kStride in {1, 2, 4, 8}:
// DPP row rotations within each 16-lane row (VALU), then the gfx950 lane
// swaps across rows (the sum of a swap's two results is v[l] + v[l ^ 16],
// resp. v[l] + v[l ^ 32], in every lane).  No LDS round trips.
template <int kStride>
__device__ __forceinline__ float strided_sum(float v) {
  static_assert(kStride == 1 || kStride == 2 || kStride == 4 || kStride == 8, "stride");
  if (kStride <= 1) v += dpp_f<0x121>(v);    // row_ror:1
  if (kStride <= 2) v += dpp_f<0x122>(v);    // row_ror:2
  if (kStride <= 4) v += dpp_f<0x124>(v);    // row_ror:4
  v += dpp_f<0x128>(v);                      // row_ror:8
  const uint32_t u = __float_as_uint(v);
  const auto r16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  v = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
  const uint32_t w = __float_as_uint(v);
  const auto r32 = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return __uint_as_float(r32[0]) + __uint_as_float(r32[1]);
}

// Inclusive prefix sum over the 64 lanes of a wave: Hillis-Steele within
// each 16-lane row (DPP row_shr, lanes without a source add 0), then row
// 15's total into rows 1 and 3 (row_bcast:15) and lane 31's into rows 2
// and 3 (row_bcast:31).
template <int kCtrl, int kRowMask>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, kCtrl, kRowMask, 0xF, false);
}
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += dpp_i<0x111, 0xF>(v);   // row_shr:1
  v += dpp_i<0x112, 0xF>(v);   // row_shr:2
  v += dpp_i<0x114, 0xF>(v);   // row_shr:4
  v += dpp_i<0x118, 0xF>(v);   // row_shr:8
  v += dpp_i<0x142, 0xA>(v);   // row_bcast:15 into rows 1, 3
  v += dpp_i<0x143, 0xC>(v);   // row_bcast:31 into rows 2, 3
  return v;
}

// every lane of each 16-lane row receives the row's sum / max
__device__ __forceinline__ float row_sum(float v) {
  v += dpp_f<0xB1>(v);
  v += dpp_f<0x4E>(v);
  v += dpp_f<0x141>(v);
  v += dpp_f<0x140>(v);
  return v;
}
__device__ __forceinline__ float row_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));
  v = fmaxf(v, dpp_f<0x4E>(v));
  v = fmaxf(v, dpp_f<0x141>(v));
  v = fmaxf(v, dpp_f<0x140>(v));
  return v;
}
__device__ __forceinline__ float lane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
// wave-uniform sum / max of a 64-lane wave
__device__ __forceinline__ float dpp_wave_sum(float v) {
  v = row_sum(v);
  return (lane_f(v, 0) + lane_f(v, 16)) + (lane_f(v, 32) + lane_f(v, 48));
}
__device__ __forceinline__ float dpp_wave_max(float v) {
  v = row_max(v);
  return fmaxf(fmaxf(lane_f(v, 0), lane_f(v, 16)), fmaxf(lane_f(v, 32), lane_f(v, 48)));
}

// wave-uniform maximum of an unsigned value (DPP row max + four lanes)
template <int kCtrl>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), kCtrl, 0xF, 0xF, false));
}
__device__ __forceinline__ uint32_t dpp_wave_max_u32(uint32_t v) {
  v = max(v, dpp_u<0xB1>(v));
  v = max(v, dpp_u<0x4E>(v));
  v = max(v, dpp_u<0x141>(v));
  v = max(v, dpp_u<0x140>(v));
  const uint32_t a = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 0));
  const uint32_t b = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 16));
  const uint32_t c = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 32));
  const uint32_t d = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 48));
  return max(max(a, b), max(c, d));
}

// Wave-uniform maximum of a float that is not NaN, as an integer maximum:
// flipping the magnitude bits of negative values makes the signed integer
// order the float order, and DPP integer maxima need no NaN canonicalizing.
__device__ __forceinline__ int f32_order_key(float x) {
  const int i = __float_as_int(x);
  return i ^ ((i >> 31) & 0x7fffffff);
}
__device__ __forceinline__ float dpp_wave_max_ordered(float x) {
  int v = f32_order_key(x);
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false));
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false));
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false));
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false));
  const int m = max(max(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
                    max(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
  return __int_as_float(m ^ ((m >> 31) & 0x7fffffff));   // the key map is its own inverse
}

__device__ __forceinline__ float byte_f(uint32_t w, int k) {
  return static_cast<float>((w >> (8 * k)) & 0xffu);
}

}  // namespace lkv
