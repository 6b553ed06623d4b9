// angle_fixed.hpp -- the fixed-point angle format shared by the angle scan
// and the decode step's streaming state.
//
// An angle is held as a 48-bit fraction of a turn (uint64, low 48 bits;
// arithmetic mod 2^48 is arithmetic mod 2 pi), offset by half a turn (2^47)
// so that the conversion back lands in [-pi, pi).  Sums of converted fp32
// steps are exact; both the full-sequence scan and the token-by-token decode
// state use these two conversions, so they produce bit-identical angles.
// ("Why Do Accumulated Transformations Extrapolate?" Sec. 5: a route of
// commuting SO(2) steps is a rotation by the summed angle, mod 2 pi.)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace arp {

constexpr uint64_t MASK48 = (1ull << 48) - 1;
constexpr uint64_t FIXED_ZERO = 1ull << 47;  // the empty sum, with the half-turn offset
constexpr double INV_2PI = 0.15915494309189533577;
constexpr double TWO_PI = 6.28318530717958647693;

// Radians (fp32) -> fixed-point turns, low 48 bits meaningful.
// n is the nearest whole number of turns; fma(a, 1/(2 pi), 24 - n) rounds
// a / (2 pi) - n + 24 once, to a multiple of 2^-48 (the result lies in
// [23.5, 24.5], so its exponent is that of 16), and the low 48 mantissa bits
// are the fraction of the turn.  Branch-free and exact in n for any finite
// angle below 2^50 turns.
__device__ __forceinline__ uint64_t to_fixed(float a) {
#pragma clang fp contract(off)
  const double x = (double)a;
  const double n = __builtin_rint(x * INV_2PI);
  const double y = __builtin_fma(x, INV_2PI, 24.0 - n);
  return (uint64_t)__double_as_longlong(y) & MASK48;
}

// Fixed-point turns (already offset by 2^47) -> radians in [-pi, pi).
// The 48 bits become the mantissa of a double in [16, 17); subtracting 16.5
// is exact and yields the signed turn in [-1/2, 1/2).
__device__ __forceinline__ float to_radians_offset(uint64_t u) {
#pragma clang fp contract(off)
  const uint64_t bits = (0x4030000000000000ull) | (u & MASK48);
  const double z = __longlong_as_double((long long)bits) - 16.5;
  return (float)(z * TWO_PI);
}

}  // namespace arp
