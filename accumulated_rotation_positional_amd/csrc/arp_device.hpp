// arp_device.hpp -- device helpers shared by the gfx950 kernels of libarp.
//
// Vector types for the bf16 matrix-core builtins, bf16 packing, and the
// pair rotation R(a) = [[cos a, -sin a], [sin a, cos a]] on (x[2p], x[2p+1])
// ("AdaRoPE: Not All Attention Heads Should Rotate and Scale Equally",
// Sec. 2.1 eq. (1)).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace arp {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float LOG2E = 1.44269504088896341f;

// ---------------------------------------------------------------------------
// bf16 <-> fp32
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}
// Two fp32 -> packed bf16 pair (round to nearest even; one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 r;
  r[0] = (__bf16)lo;
  r[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// ---------------------------------------------------------------------------
// Pair rotation.  (a, b) -> (a c - b s, a s + b c); the inverse uses -s.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void rotate_pair(float& a, float& b, float c, float s) {
  float x = a * c - b * s;
  float y = a * s + b * c;
  a = x;
  b = y;
}

}  // namespace arp
