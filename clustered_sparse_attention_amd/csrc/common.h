// Device-side helpers shared by the gfx950 kernels of the layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define AC_DEV __device__ __forceinline__

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

namespace ac {

constexpr int kWave = 64;

// bf16 bit pattern -> fp32 (exact).
AC_DEV float bf2f(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// fp32 -> bf16 bit pattern, round to nearest even (finite inputs).
AC_DEV uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// fp64 -> bf16 bit pattern with a single rounding to 8 significant bits
// (nearest, ties to even), for values in the bf16 normal range or zero:
// round the binary64 significand at bit 45, then narrow exactly to fp32.
AC_DEV uint16_t d2bf(double x) {
  uint64_t u = (uint64_t)__double_as_longlong(x);
  u += 0x00000FFFFFFFFFFFull + ((u >> 45) & 1ull);
  u &= ~0x00001FFFFFFFFFFFull;
  float f = (float)__longlong_as_double((long long)u);  // exact: <= 8 significant bits
  return (uint16_t)(__float_as_uint(f) >> 16);
}

// Split an fp32 value into bf16 parts whose sum reproduces it: hi = bf16(x),
// mid = bf16(x - hi), lo = bf16(x - hi - mid).  The differences are exact in fp32.
AC_DEV void split3(float x, uint16_t &hi, uint16_t &mid, uint16_t &lo) {
  hi = f2bf(x);
  float r1 = x - bf2f(hi);
  mid = f2bf(r1);
  float r2 = r1 - bf2f(mid);
  lo = f2bf(r2);
}

// Order-preserving map of fp32 to uint32 (larger float -> larger integer).
AC_DEV uint32_t f2ord(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// SplitMix64 step from state z (Steele, Lea and Flood 2014): add the golden
// gamma, then the xor-shift-multiply finaliser.
AC_DEV uint64_t splitmix64(uint64_t z) {
  z += 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// Counter-based uniform in [0, 1) for (seed, stream, counter).
AC_DEV double uniform01(uint64_t seed, uint64_t stream, uint64_t counter) {
  uint64_t x = splitmix64(seed);
  x = splitmix64(x ^ stream);
  x = splitmix64(x ^ counter);
  return (double)(x >> 11) * (1.0 / 9007199254740992.0);
}

// Random stream of one k-means++ run: head, role (0 queries, 1 keys), stage.
AC_DEV uint64_t stream_id(uint64_t bh, uint32_t role, uint32_t stage) {
  return ((bh & ((1ull << 44) - 1)) << 20) | ((uint64_t)(role & 0xF) << 16) | (stage & 0xFFFF);
}

// DPP moves within a wave.  Controls used: quad permutes 0x00-0xFF, row
// shifts right 0x111-0x11F, wave shift right by one 0x138, row mirror 0x140,
// half-row mirror 0x141, row broadcasts of lanes 15 and 31 0x142 / 0x143.
// Lanes that the row and bank masks leave out, or whose source lane lies
// outside the row (or wave), get 0.
template <int CTRL, int ROWS = 0xF, int BANKS = 0xF>
AC_DEV uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROWS, BANKS, false);
}
template <int CTRL, int ROWS = 0xF, int BANKS = 0xF>
AC_DEV float dpp_f32(float v) {
  return __uint_as_float(dpp_u32<CTRL, ROWS, BANKS>(__float_as_uint(v)));
}
// sum over each row of 16 lanes, left in every lane of the row: after each
// step the groups of 2, 4, 8, 16 lanes hold equal values, so the mirrors
// pair every lane with the other half of its group
AC_DEV float row16_sum(float v) {
  v += dpp_f32<0xB1>(v);   // quad: xor 1
  v += dpp_f32<0x4E>(v);   // quad: xor 2
  v += dpp_f32<0x141>(v);  // half-row mirror
  v += dpp_f32<0x140>(v);  // row mirror
  return v;
}
// fp64 through the same moves, one 32-bit half at a time (both halves from
// the same source lane, or both 0)
template <int CTRL, int ROWS = 0xF, int BANKS = 0xF>
AC_DEV double dpp_f64(double v) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = dpp_u32<CTRL, ROWS, BANKS>((uint32_t)b), hi = dpp_u32<CTRL, ROWS, BANKS>((uint32_t)(b >> 32));
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
// inclusive prefix sum over the 64 lanes: within each row of 16 by row
// shifts of 1, 2, 4, 8, then row 0's total into row 1 and row 2's into row 3
// (row broadcast of lane 15), then lane 31's total into rows 2 and 3
AC_DEV double wave_incl_scan(double v) {
  v += dpp_f64<0x111>(v);
  v += dpp_f64<0x112>(v);
  v += dpp_f64<0x114>(v);
  v += dpp_f64<0x118>(v);
  v += dpp_f64<0x142, 0xA>(v);
  v += dpp_f64<0x143, 0xC>(v);
  return v;
}
// the previous lane's value (0 in lane 0), bit for bit: a wave shift by one
AC_DEV double wave_prev(double v) { return dpp_f64<0x138>(v); }
// the value lane l holds (uniform)
AC_DEV float lane_f32(float v, int l) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l)); }

template <typename T>
AC_DEV T wave_sum(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

AC_DEV float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

}  // namespace ac
