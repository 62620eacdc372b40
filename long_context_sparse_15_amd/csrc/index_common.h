// Device helpers shared by the indexer's scoring kernels (index.hip) and the top-k kernels
// (topk.hip): the visible length of a query row and the score-row element access.
#pragma once

#include "common.h"
#include "kernels.h"

namespace csa {

// Visible entries of a query row: min(n_entries[b], floor((t+1)/m)), clamped to [0, n_max]
// so a bad n_entries can never send a read past the cache.
// Both loads go out together (one memory round trip, not two dependent ones).  `row` may
// differ between lanes.
__device__ __forceinline__ int visible(const int32_t* n_entries, const int32_t* pos, int row,
                                       int nq, int m, int n_max) {
  const int b = row / nq;
  int ne = n_entries[b];
  int tp = *(pos ? pos + row : n_entries + b);
  asm volatile("" : "+v"(ne), "+v"(tp) : : "memory");
  const long t = pos ? tp : (row % nq);
  long v = (t + 1) / m;
  const int n = min(ne, n_max);
  if (v > n) v = n;
  return static_cast<int>(v < 0 ? 0 : v);
}

// Score rows in the workspace: fp32, or bf16 bit patterns (ST = uint16_t).  at() reads one score
// as fp32 (bf16 widens exactly), four() the four scores from element e (e % 4 == 0: one 16-byte
// or 8-byte load), put() stores one (bf16: nearest even).
template <typename ST> struct Scores;
template <> struct Scores<float> {
  static __device__ __forceinline__ float at(const float* r, int e) { return r[e]; }
  static __device__ __forceinline__ void four(const float* r, int e, float (&f)[4]) {
    const float4 v = *reinterpret_cast<const float4*>(r + e);
    f[0] = v.x;
    f[1] = v.y;
    f[2] = v.z;
    f[3] = v.w;
  }
  static __device__ __forceinline__ void put(float* r, int e, float v) { r[e] = v; }
  static __device__ __forceinline__ float stored(float v) { return v; }  // what put keeps
  static __device__ __forceinline__ void put4(float* r, int e, f32x4 v) {
    *reinterpret_cast<f32x4*>(r + e) = v;
  }
};
template <> struct Scores<uint16_t> {
  static __device__ __forceinline__ float at(const uint16_t* r, int e) { return bf16_to_f32(r[e]); }
  static __device__ __forceinline__ void four(const uint16_t* r, int e, float (&f)[4]) {
    const uint2 v = *reinterpret_cast<const uint2*>(r + e);
    f[0] = __uint_as_float(v.x << 16);
    f[1] = __uint_as_float(v.x & 0xffff0000u);
    f[2] = __uint_as_float(v.y << 16);
    f[3] = __uint_as_float(v.y & 0xffff0000u);
  }
  static __device__ __forceinline__ void put(uint16_t* r, int e, float v) { r[e] = f32_to_bf16(v); }
  static __device__ __forceinline__ float stored(float v) { return bf16_to_f32(f32_to_bf16(v)); }
  static __device__ __forceinline__ void put4(uint16_t* r, int e, f32x4 v) {
    *reinterpret_cast<uint2*>(r + e) = uint2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
  }
};

// Score rows: fp32 (or bf16) values, row stride a multiple of 64 elements.
inline int score_stride(int n_max) { return (n_max + 63) & ~63; }

}  // namespace csa
