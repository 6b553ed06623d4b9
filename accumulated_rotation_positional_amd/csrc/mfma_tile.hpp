// mfma_tile.hpp -- operand-layout helpers shared by the bf16 attention kernels
// (forward and backward) on the gfx950 matrix cores.
//
// All products use v_mfma_f32_32x32x16_bf16.  For lane l = 32 hf + ln:
//   A operand: A[m = ln][k = 8 hf .. 8 hf + 7]
//   B operand: B[k = 8 hf .. 8 hf + 7][n = ln]
//   accumulator element r: C[m = 8 (r / 4) + 4 hf + r % 4][n = ln]
// When the 32 (or 64) rows of an A tile sit in LDS in the order swap_bits23,
// accumulator element r of lane (ln, hf) holds logical row
// 16 (r >> 3) + 8 hf + (r & 7): elements 0..7 and 8..15 are then the B operand
// of the next product along that row index, with no data movement.
#pragma once

#include <hip/hip_runtime.h>

#include "arp_device.hpp"

namespace arp {

typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef const __attribute__((address_space(1))) void* global_void_ptr;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4* lds_s16x4_ptr;

// LDS transpose read (ds_read_b64_tr_b16): each group of 16 lanes names a
// 16 x 4 block of 16-bit elements (lane j of the group: four consecutive
// elements at p); lane i of the group receives element i % 4 of the rows named
// by lanes 4 e + i / 4, e = 0..3.
// The four elements come back packed in two dwords (element 0 in the low
// half of the first).
__device__ __forceinline__ u32x2 lds_read_tr16(const void* p) {
  return __builtin_bit_cast(
      u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(const_cast<void*>(p))));
}

// Row order of K~ in LDS: bits 2 and 3 of the key index swapped (an involution).
__device__ __forceinline__ int swap_bits23(int x) {
  return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1);
}

// LDS swizzle: the 16-byte chunk c of a row of ROWB bytes is stored at chunk
// c ^ swz(row).  A 128-bit LDS read serves 16 lanes per cycle from 64 banks,
// i.e. 256 bytes; the operand reads of 16 consecutive rows must therefore hit
// 16 distinct 16-byte bank groups, which this choice guarantees for 64-, 128-
// and 256-byte rows.
template <int ROWB>
__device__ __forceinline__ int swz(int row) {
  static_assert(ROWB == 64 || ROWB == 128 || ROWB == 256, "row size");
  return ROWB == 64 ? ((row >> 2) & 3) : ROWB == 128 ? ((row >> 1) & 7) : (row & 15);
}

// LDS swizzle of the natural V rows (64-bit transpose reads): one read
// instruction of 32 lanes covers 4 consecutive rows x 64 bytes (four 16-byte
// chunks, 4b .. 4b + 3), which must land in the four distinct 64-byte quarters
// of the 256-byte bank period.  128-byte rows: consecutive rows already sit
// in opposite halves, so rows r and r + 2 swap the 64-byte blocks of their
// half (chunk bit 2 from row bit 1); 256-byte rows: row r % 4 picks the block.
template <int ROWB>
__device__ __forceinline__ int swzv(int row) {
  static_assert(ROWB == 128 || ROWB == 256, "row size");
  return ROWB == 128 ? ((row >> 1) & 1) << 2 : (row & 3) << 2;
}

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Max and sum of a value over the two half-waves (lanes l and l ^ 32), with
// one v_permlane32_swap: afterwards each lane holds both halves' values.
__device__ __forceinline__ float halves_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Wait until at most N global->LDS loads of this wave are still in flight
// (s_waitcnt vmcnt(N), the other counters untouched).
template <int N>
__device__ __forceinline__ void wait_loads() {
  static_assert(N >= 0 && N < 16, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

}  // namespace arp
