// Pieces shared by the attention kernels (mqa.hip, mqa_hb.hip): the launch parameters, bf16
// packing, the LDS row swizzle and the span merge that every output goes through.
#pragma once

#include <cmath>

#include "common.h"
#include "kernels.h"

namespace csa {

struct MqaParams {
  const uint16_t* q;
  const uint16_t* entries;
  const uint16_t* window;
  const int32_t* idx;
  const int32_t* n_entries;
  const int32_t* pos;
  const float* sink;
  const float* inv_freq;
  int nq, n_heads, r, k, m, n_win, win_slots, n_max;
  PageMap pages;  // entries in a block pool (PAGED kernels)
  float scale_log2;
  int split_rows, n_splits, head_groups, n_work;
  float* part;  // span partials: bf16 O / l of each span in the MFMA lane order (see mqa_kernel)
  float* ml;    // [rows, n_splits, n_heads, 2]: (max, sum) of each span
  uint16_t* out;
  float* lse_out;
};

__device__ __forceinline__ f32x16 mfma_bf16_32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Physical 16-byte chunk of logical chunk c in LDS row `row`: the low four bits of the chunk
// index are XORed with a permutation of row % 16 (bits of row&3 and (row>>2)&3 swapped).
// 16 consecutive rows at one logical chunk land in 16 distinct bank groups, and so do the
// 4 rows x 4 chunks addressed by 32 lanes of a transposed read.
__device__ __forceinline__ int swz(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }

__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};  // RNE
  return __builtin_bit_cast(uint32_t, v);
}

// fp32 rounded to bf16 (nearest even) and back: the value a span partial holds
__device__ __forceinline__ float bf16_round(float x) {
  return static_cast<float>(static_cast<__bf16>(x));
}
// four bf16 values packed low first (as pack2 writes them) to fp32
__device__ __forceinline__ f32x4 unpack_b4(uint2 v) {
  return f32x4{__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u),
               __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xffff0000u)};
}

// Merge of a query's span partials, in span order, plus the sink, in the log2 domain.  A span
// contributes its maximum m, its sum l of exp2(z - m) and O / l stored in bf16.  Every list, split
// into one span or many, is normalised by exactly these operations (contraction off, so the
// rounding is the same wherever they are inlined): the combine kernel folds the stored partials,
// a single-span workgroup folds its own partial, rounded to bf16 as it would have been stored.
struct SpanMerge {
  float M;     // running reference: the sink logit, raised to the spans' maxima
  float lsum;  // sum over merged spans of l * exp2(m - M)
};
__device__ __forceinline__ SpanMerge sm_start(float sink2) { return SpanMerge{sink2, 0.f}; }
// raise the reference to Mn >= M; returns the factor the merged O must be multiplied by
__device__ __forceinline__ float sm_raise(SpanMerge& st, float Mn) {
#pragma clang fp contract(off)
  if (Mn == st.M) return 1.f;
  const float a = (st.M == -INFINITY) ? 0.f : exp2f(st.M - Mn);
  st.lsum *= a;
  st.M = Mn;
  return a;
}
// adds a span (maximum m <= M, sum l); returns the weight of its O / l (0 for an empty span)
__device__ __forceinline__ float sm_add(SpanMerge& st, float m, float l) {
#pragma clang fp contract(off)
  if (m == -INFINITY) return 0.f;
  const float w = l * exp2f(m - st.M);
  st.lsum += w;
  return w;
}
__device__ __forceinline__ float sm_fold(float o, float ov, float w) {
#pragma clang fp contract(off)
  return o + ov * w;
}
// 1 / (sum + the sink's term); 0 when nothing is attended and there is no sink
__device__ __forceinline__ float sm_inv(const SpanMerge& st, bool has_sink, float sink2) {
#pragma clang fp contract(off)
  const float den = st.lsum + ((has_sink && st.M != -INFINITY) ? exp2f(sink2 - st.M) : 0.f);
  return den > 0.f ? 1.f / den : 0.f;
}
// natural-log sum of exp(z) without the sink
__device__ __forceinline__ float sm_lse(const SpanMerge& st) {
  return st.lsum > 0.f ? (st.M + log2f(st.lsum)) * kLn2 : -INFINITY;
}

// As store_out4, with cos/sin of the rotation angles of position t read from a table (pair i of
// the RoPE dims at entry i).
__device__ __forceinline__ void store_out4_tab(uint16_t* dst, float o0, float o1, float o2,
                                               float o3, int d0, int c, int r,
                                               const float2* cs_tab) {
  float o[4] = {o0, o1, o2, o3};
#pragma unroll
  for (int pr = 0; pr < 2; ++pr) {
    const int d = d0 + 2 * pr;
    if (d >= c - r) {
      const float2 e = cs_tab[(d - (c - r)) >> 1];
      const float x0 = o[2 * pr], x1 = o[2 * pr + 1];
      o[2 * pr] = x0 * e.x + x1 * e.y;       // rotation by -angle
      o[2 * pr + 1] = -x0 * e.y + x1 * e.x;
    }
  }
  uint2 v;
  v.x = pack2(o[0], o[1]);
  v.y = pack2(o[2], o[3]);
  *reinterpret_cast<uint2*>(dst) = v;
}

// Epilogue shared by the in-place path and the combine kernel: o (4 consecutive dims d0..d0+3
// of one head) is rotated back by -t on the RoPE dims and stored as bf16.
__device__ __forceinline__ void store_out4(uint16_t* dst, float o0, float o1, float o2, float o3,
                                           int d0, int c, int r, int t, const float* inv_freq) {
  float o[4] = {o0, o1, o2, o3};
#pragma unroll
  for (int pr = 0; pr < 2; ++pr) {
    const int d = d0 + 2 * pr;
    if (d >= c - r) {
      float cs, sn;
      rope_cos_sin(t, inv_freq[(d - (c - r)) >> 1], cs, sn);
      const float x0 = o[2 * pr], x1 = o[2 * pr + 1];
      o[2 * pr] = x0 * cs + x1 * sn;       // rotation by -angle
      o[2 * pr + 1] = -x0 * sn + x1 * cs;
    }
  }
  uint2 v;
  v.x = pack2(o[0], o[1]);
  v.y = pack2(o[2], o[3]);
  *reinterpret_cast<uint2*>(dst) = v;
}

// (x0, x1) rotated back by the angle with cosine cs and sine sn
__device__ __forceinline__ void rot_back(float& x0, float& x1, float cs, float sn) {
#pragma clang fp contract(off)
  const float a = x0 * cs + x1 * sn;
  const float b = -x0 * sn + x1 * cs;
  x0 = a;
  x1 = b;
}

// s_waitcnt until at most N vector-memory operations of this wave are outstanding (loads
// complete in issue order), leaving the LDS and export counters alone
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Every launch parameter requested in one batch at kernel entry: scalar loads complete out of
// order, so each later batch the compiler would issue on demand costs a full wait on all of them.
__device__ __forceinline__ void mqa_preload_params(const MqaParams& p) {
  asm volatile("" ::"s"(p.q), "s"(p.entries), "s"(p.window), "s"(p.idx), "s"(p.n_entries),
               "s"(p.pos), "s"(p.sink), "s"(p.inv_freq), "s"(p.nq), "s"(p.n_heads), "s"(p.r),
               "s"(p.k), "s"(p.m), "s"(p.n_win), "s"(p.win_slots), "s"(p.n_max));
  asm volatile("" ::"s"(p.pages.table), "s"(p.pages.stride), "s"(p.pages.shift),
               "s"(p.scale_log2), "s"(p.split_rows), "s"(p.n_splits), "s"(p.head_groups),
               "s"(p.n_work), "s"(p.part), "s"(p.ml), "s"(p.out), "s"(p.lse_out));
}

// The position of query row `row` requested through the vector path (a valid address when there
// is no position array); take it with mqa_position_take after the loads that do not need it.
__device__ __forceinline__ int mqa_position_request(const MqaParams& p, int row) {
  int rv = p.pos ? row : 0;
  asm volatile("" : "+v"(rv));
  return (p.pos ? p.pos : p.n_entries)[rv];
}
__device__ __forceinline__ int mqa_position_take(const MqaParams& p, int row, int t_vec) {
  asm volatile("" : "+v"(t_vec) : : "memory");
  return p.pos ? __builtin_amdgcn_readfirstlane(t_vec) : (row % p.nq);
}

// Workgroup -> (head group, span, query row); row = -1 for a workgroup past the work.  Workgroups
// are dealt round-robin over the 8 XCDs (bid % 8).  With at least 8 rows every span and head
// group of a row runs on the XCD row % 8, so the row's query (and, for head groups, its gathered
// rows) is fetched into one L2.  With fewer rows that would leave XCDs idle, so the work items
// (row, span) are spread over the XCDs instead, a work item's head groups still on one XCD.
// mqa_grid gives the matching grid size.
__device__ __forceinline__ void mqa_work_item(const MqaParams& p, int bid, int& hg, int& split,
                                             int& row) {
  const int rows = p.n_work / p.n_splits;
  const int xcd = bid & 7, k8 = bid >> 3;
  hg = k8 % p.head_groups;
  if (rows >= 8) {
    split = (k8 / p.head_groups) % p.n_splits;
    row = (k8 / p.head_groups / p.n_splits) * 8 + xcd;
    if (row >= rows) row = -1;
  } else {
    const int w = (k8 / p.head_groups) * 8 + xcd;
    split = w % p.n_splits;
    row = w < p.n_work ? w / p.n_splits : -1;
  }
}
inline unsigned mqa_grid(int rows, int n_splits, int head_groups) {
  const long n = rows >= 8 ? static_cast<long>((rows + 7) / 8 * 8) * n_splits
                           : static_cast<long>((rows * n_splits + 7) / 8 * 8);
  return static_cast<unsigned>(n * head_groups);
}

// Head-block attention for c = 512 (mqa_hb.hip): launches the kernel and, with several spans,
// its combine.
hipError_t launch_mqa_hb(const MqaParams& prm, int rows, hipStream_t s);
// Runs of queries (prefill) with up to 64 heads, c = 512, one span per query of up to
// kHbqMaxList rows: two queries per workgroup (mqa_hb.hip).
constexpr int kHbqMaxList = 1024;  // key-list rows a query may bring (its index list in LDS)
hipError_t launch_mqa_hbq(const MqaParams& prm, int rows, hipStream_t s);

}  // namespace csa
