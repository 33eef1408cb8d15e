// Device-side types and helpers shared by the gfx950 kernels of the library.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dpg {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// FP32 -> BF16 bits, round to nearest even (gfx950 converts natively).
__device__ __forceinline__ uint32_t bf16_bits(float f) {
  __bf16 h = (__bf16)f;
  return (uint32_t)__builtin_bit_cast(unsigned short, h);
}

__device__ __forceinline__ float bf16_value(uint32_t bits16) {
  return __builtin_bit_cast(float, bits16 << 16);
}

// Two FP32 values -> one dword holding two BF16 (lo half = first).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return bf16_bits(lo) | (bf16_bits(hi) << 16);
}

// BF16x3 split of one FP32 value: hi = bf16(a), lo = bf16(a - hi).  a - hi is
// exact in FP32 because hi is a rounding of a to fewer bits.
__device__ __forceinline__ void split3(float a, uint32_t& hi, uint32_t& lo) {
  hi = bf16_bits(a);
  lo = bf16_bits(a - bf16_value(hi));
}

// Split 8 FP32 values into an 8-wide BF16 hi vector and lo vector.
__device__ __forceinline__ void split3_x8(const f32x4& v0, const f32x4& v1, u32x4& hi, u32x4& lo) {
  uint32_t h[8], l[8];
  split3(v0[0], h[0], l[0]);
  split3(v0[1], h[1], l[1]);
  split3(v0[2], h[2], l[2]);
  split3(v0[3], h[3], l[3]);
  split3(v1[0], h[4], l[4]);
  split3(v1[1], h[5], l[5]);
  split3(v1[2], h[6], l[6]);
  split3(v1[3], h[7], l[7]);
  hi = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
  lo = u32x4{l[0] | (l[1] << 16), l[2] | (l[3] << 16), l[4] | (l[5] << 16), l[6] | (l[7] << 16)};
}

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) { return __builtin_bit_cast(bf16x8, v); }

// Transposing 64-bit LDS read (gfx950 ds_read_b64_tr_b16).  Within each group
// of 16 lanes, lane i receives element (i % 4) of the 4-element chunk addressed
// by lanes i/4, 4 + i/4, 8 + i/4 and 12 + i/4 of its group, in that order.
__device__ __forceinline__ u32x2 lds_read_tr16(const __bf16* lds_ptr) {
  i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(lds_ptr));
  return __builtin_bit_cast(u32x2, v);
}

// K partition of a split plan: S splits over KB reduction blocks (64
// elements, or 64 tokens, each); with q = KB / S and r = KB % S the first r
// splits take q + 1 blocks and the others q, so split s starts at block
// s q + min(s, r): sizes differ by at most one block, none is empty while
// S <= KB, and with two splits the first takes ceil(KB / 2) blocks.  q and r
// come from one division per kernel (split_parts), not one per unit.
struct SplitParts {
  int q, r;
};
__device__ __forceinline__ SplitParts split_parts(int S, int KB) {
  const int q = KB / S;
  return SplitParts{q, KB - q * S};
}
__device__ __forceinline__ int split_begin(int s, const SplitParts& sp) { return s * sp.q + min(s, sp.r); }

// Map a linear workgroup id so that the workgroups the dispatcher sends to one
// XCD (ids congruent mod 8) cover a contiguous range of tile ids.  A bijection
// on [0, total).
__device__ __forceinline__ int xcd_remap(int bid, int total) {
  constexpr int kXcds = 8;
  if (total < kXcds) return bid;
  const int per = (total + kXcds - 1) / kXcds;      // ids per "tall" XCD
  const int tall = total - (per - 1) * kXcds;        // XCDs that get `per` ids
  const int xcd = bid % kXcds;
  const int local = bid / kXcds;
  if (xcd < tall) return xcd * per + local;
  return tall * per + (xcd - tall) * (per - 1) + local;
}

}  // namespace dpg
