// Device helpers shared by the CSA/HCA kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// bf16 <-> fp32.  fp32 -> bf16 rounds to nearest, ties to even (finite inputs).
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u) return static_cast<uint16_t>((u >> 16) | ((u & 0xffff) ? 0x40 : 0));
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}
// E4M3 ("fn") encoding with round-to-nearest-even and saturation to +-448, from the format's
// bit fields (bias 7, 3 mantissa bits, subnormal quantum 2^-9).
__device__ __forceinline__ uint8_t e4m3_rne(float x) {
  const uint8_t sign = (__float_as_uint(x) >> 24) & 0x80;
  const float a = fabsf(x);
  uint32_t code;
  if (!(a < 448.f)) {
    code = 0x7e;
  } else if (a < 0.015625f) {  // below 2^-6: subnormal quantum 2^-9
    code = static_cast<uint32_t>(rintf(a * 512.f));  // 8 -> 0x08 = 2^-6, still correct
  } else {
    int ex;
    const float f = frexpf(a, &ex);  // a = f * 2^ex, f in [0.5, 1)
    uint32_t mant = static_cast<uint32_t>(rintf((f * 2.f - 1.f) * 8.f));
    uint32_t field = static_cast<uint32_t>(ex + 6);
    if (mant == 8) {
      mant = 0;
      ++field;
    }
    code = (field << 3) | mant;
    if (code > 0x7e) code = 0x7e;
  }
  return static_cast<uint8_t>(code | sign);
}

// E2M1 (OCP MXFP4 element: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6) nearest to x, ties to the even
// code, saturating at 6; the sign bit (bit 3) follows x's sign bit.
__device__ __forceinline__ uint32_t e2m1_rne(float x) {
  const float a = fabsf(x);
  const uint32_t mag = a > 5.f     ? 7u
                       : a >= 3.5f ? 6u
                       : a > 2.5f  ? 5u
                       : a >= 1.75f ? 4u
                       : a > 1.25f ? 3u
                       : a >= 0.75f ? 2u
                       : a > 0.25f ? 1u
                                   : 0u;
  return mag | ((__float_as_uint(x) >> 28) & 8u);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

// Order-preserving map fp32 -> uint32 (larger float <=> larger key; -0 is folded to +0).
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// RoPE angle p * inv_freq, reduced in fp64 to a fraction of a turn in [-1/2, 1/2] before the
// hardware sin/cos (v_sin_f32 / v_cos_f32 take turns), so positions up to 2^31 keep an absolute
// angle error around 1e-6 rad instead of the ~0.06 rad an fp32 product would give at 2^20.
__device__ __forceinline__ void rope_cos_sin(int pos, float inv_freq, float& c, float& s) {
  const double inv_two_pi = 0.15915494309189533577;
  double turns = static_cast<double>(pos) * static_cast<double>(inv_freq) * inv_two_pi;
  turns -= rint(turns);
  const float tf = static_cast<float>(turns);
  s = __builtin_amdgcn_sinf(tf);
  c = __builtin_amdgcn_cosf(tf);
}

__device__ __forceinline__ float wave_max_xor(float v, int from_mask) {
  // reduce over lanes that differ only in the bits of from_mask (16 and/or 32)
  if (from_mask & 16) v = fmaxf(v, __shfl_xor(v, 16, 64));
  if (from_mask & 32) v = fmaxf(v, __shfl_xor(v, 32, 64));
  return v;
}
// v summed over the four lanes l, l^16, l^32, l^48 with the lane-swap instructions
// (v_permlane16_swap / v_permlane32_swap: VALU, no LDS round trip).  Swapping a register with
// itself leaves, in each lane, its own value in one result and its partner's in the other.
__device__ __forceinline__ float wave_sum_xor16_32(float v) {
  auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(s16[0]) + __uint_as_float(s16[1]);
  auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(s32[0]) + __uint_as_float(s32[1]);
}
// Whole-wave integer scans and reductions from DPP lane moves and the lane-swap instructions,
// all VALU: no LDS round trip per step.
// Inclusive prefix sum over lanes 0..l: shifts by 1, 2, 4, 8 inside each 16-lane row (lanes
// without a source read 0), then row r adds the total of row r-1 (rows 1, 3) and the total of
// rows 0-1 (rows 2, 3) through the row broadcasts of lanes 15 and 31.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  const int v = static_cast<int>(x);
  int s = v + __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true);   // row_shr:1
  s += __builtin_amdgcn_update_dpp(0, s, 0x112, 0xf, 0xf, true);          // row_shr:2
  s += __builtin_amdgcn_update_dpp(0, s, 0x114, 0xf, 0xf, true);          // row_shr:4
  s += __builtin_amdgcn_update_dpp(0, s, 0x118, 0xf, 0xf, true);          // row_shr:8
  s += __builtin_amdgcn_update_dpp(0, s, 0x142, 0xa, 0xf, false);         // row_bcast:15
  s += __builtin_amdgcn_update_dpp(0, s, 0x143, 0xc, 0xf, false);         // row_bcast:31
  return static_cast<uint32_t>(s);
}
// x reduced over all 64 lanes: lanes l^1 and l^2 (quad permutes), then the mirrored half-row
// and row, then l^16 and l^32 (lane swaps).
template <typename Op>
__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t x, Op op) {
  x = op(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0xb1, 0xf,
                                                              0xf, false)));  // [1,0,3,2]
  x = op(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x4e, 0xf,
                                                              0xf, false)));  // [2,3,0,1]
  x = op(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x141, 0xf,
                                                              0xf, false)));  // row_half_mirror
  x = op(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x140, 0xf,
                                                              0xf, false)));  // row_mirror
  auto s16 = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  x = op(s16[0], s16[1]);
  auto s32 = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return op(s32[0], s32[1]);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  return wave_reduce_u32(x, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) {
  return wave_reduce_u32(x, [](uint32_t a, uint32_t b) { return a < b ? a : b; });
}
__device__ __forceinline__ float wave_sum_xor(float v, int from_mask) {
  if (from_mask & 16) v += __shfl_xor(v, 16, 64);
  if (from_mask & 32) v += __shfl_xor(v, 32, 64);
  return v;
}

// MFMA wrappers.  16x16 outputs: lane l holds D[row = 4*(l/16) + i][col = l%16], i = 0..3.
// A operand: lane l supplies row l%16 and a K slice chosen by l/16; B operand: column l%16 and
// the same K slice.  Any fixed assignment of K values to (lane/16, element) works as long as
// A and B use the same one, which every caller below does.
__device__ __forceinline__ f32x4 mfma_bf16_16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_fp8_16x16x32(long a, long b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a, b, c, 0, 0, 0);
}
// 16x16x128 with both operands E4M3 (format code 0) and unit block scales (E8M0 127 = 2^0).
__device__ __forceinline__ f32x4 mfma_fp8_16x16x128(i32x8 a, i32x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// 16x16x128 with A E4M3 (unit scale) and B FP4 E2M1 (format code 4) in the low four dwords of
// b, scaled by 2^(scale_b - 127) per lane: each lane's scale covers the 32 K values it holds.
__device__ __forceinline__ f32x4 mfma_fp8_fp4_16x16x128(i32x8 a, i32x8 b, f32x4 c, int scale_b) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 4, 0, 127, 0, scale_b);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// LDS transpose read (ds_read_b64_tr_b16): within each group of 16 lanes, lane 4*i0+q points
// at 4 consecutive 16-bit values (row i0, columns 4q..4q+3) of a 4x16 block; lane j receives
// column j of that block, rows 0..3 in order.  p must point into LDS, 8-byte aligned.
__device__ __forceinline__ bf16x4 lds_read_tr16(const uint16_t* p) {
  typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p));
}

}  // namespace csa
