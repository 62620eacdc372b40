// Lightning indexer scoring and exact top-k selection for gfx950.
//
// Method: "DeepSeek V4 模型技术大全", chapter "Attention", section "CSA 的完整路径":
//   I_{t,s} = sum_h w^I_{t,h} ReLU(q^I_{t,h} . K^IComp_s)  for s < floor((t+1)/m),
//   I_t = TopK_k { I_{t,s} }.
// Operands are E4M3 codes with float32 scales; since the scales are positive,
//   w_h ReLU(sq_h sk_s x) = sk_s (w_h sq_h) ReLU(x),
// so the MFMA works on raw codes and the epilogue applies (w_h sq_h) per head and sk_s per entry.
//
// Top-k is exact with the lower index winning ties.  Scores become order-preserving 32-bit
// keys.  Decode rows (few rows, many entries) use a first-level histogram of the top 12 key bits
// built by the scoring kernel, a multi-workgroup collect of everything above the threshold bin
// plus the (few) candidates inside it, and a per-row finalize that sorts the candidates and
// emits the selection in ascending index order.  Prefill rows (many rows, <= 16384 entries
// each) use one workgroup per row with the keys held in LDS: a 4-pass radix select finds the
// k-th key, and an index-ordered compaction emits the selection already sorted.
#include "common.h"
#include "kernels.h"

namespace csa {

// Visible entries of a query row: min(n_entries[b], floor((t+1)/m)), clamped to [0, n_max]
// so a bad n_entries can never send a read past the cache.
__device__ __forceinline__ int visible(const int32_t* n_entries, const int32_t* pos, int row,
                                       int nq, int m, int n_max) {
  const int b = row / nq;
  const long t = pos ? pos[row] : (row % nq);
  long v = (t + 1) / m;
  const int n = min(n_entries[b], n_max);
  if (v > n) v = n;
  return static_cast<int>(v < 0 ? 0 : v);
}

// ============================================================================ scoring
// One workgroup scores `chunk` consecutive entries of one query row.  Each wave takes 16-entry
// tiles; a tile is an MFMA with the indexer heads as the M dimension (A operand, resident in
// registers for the whole chunk) and 16 entries as N (B operand, streamed from HBM).
template <int DI, int HT>
__global__ __launch_bounds__(256) void index_score_kernel(
    const uint8_t* __restrict__ qi, const float* __restrict__ qi_scale,
    const float* __restrict__ wi, const uint8_t* __restrict__ keys,
    const float* __restrict__ kscale, const int32_t* __restrict__ n_entries,
    const int32_t* __restrict__ pos, int nq, int n_max, int H_I, int m, int chunk,
    float* __restrict__ scores, int sstride, uint32_t* __restrict__ hist, int nchunks) {
  constexpr int KB = DI / 4;   // key bytes per lane (its lane group's K slice)
  constexpr int KK = DI / 32;  // 8-byte MFMA steps per slice
  __shared__ uint32_t lhist[kHistBins];

  const int row = blockIdx.x / nchunks;
  const int b = row / nq;
  const int n_vis = visible(n_entries, pos, row, nq, m, n_max);
  const int e0 = (blockIdx.x % nchunks) * chunk;
  const int e1 = min(n_vis, e0 + chunk);
  const int tid = threadIdx.x;
  const int l = lane_id(), g = l >> 4, c16 = l & 15, wave = tid >> 6;

  if (hist) {
    for (int i = tid; i < kHistBins; i += 256) lhist[i] = 0;
    __syncthreads();
  }

  if (e0 < e1) {
    // A operand: query codes of head ht*16 + c16, K slice g.
    long aq[HT][KK];
    float wq[HT][4];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      const int head = ht * 16 + c16;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) aq[ht][kk] = 0;
      if (head < H_I) {
        const long* src = reinterpret_cast<const long*>(
            qi + (static_cast<size_t>(row) * H_I + head) * DI + g * KB);
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) aq[ht][kk] = src[kk];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int hh = ht * 16 + g * 4 + i;
        wq[ht][i] = hh < H_I ? wi[static_cast<size_t>(row) * H_I + hh] *
                                   qi_scale[static_cast<size_t>(row) * H_I + hh]
                             : 0.f;
      }
    }

    const uint8_t* kbase = keys + static_cast<size_t>(b) * n_max * DI + g * KB;
    const float* sbase = kscale + static_cast<size_t>(b) * n_max;
    float* srow = scores + static_cast<size_t>(row) * sstride;
    const int ntile = (e1 - e0 + 15) >> 4;

    auto load = [&](int tile, long (&bk)[KK], float& ks) {
      const int e = e0 + tile * 16 + c16;
      if (e < e1) {
        const long* src = reinterpret_cast<const long*>(kbase + static_cast<size_t>(e) * DI);
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) bk[kk] = __builtin_nontemporal_load(src + kk);
        ks = sbase[e];
      } else {
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) bk[kk] = 0;
        ks = 0.f;
      }
    };
    auto compute = [&](int tile, const long (&bk)[KK], float ks) {
      f32x4 acc[HT];
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) acc[ht] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) acc[ht] = mfma_fp8_16x16x32(aq[ht][kk], bk[kk], acc[ht]);
      float part = 0.f;
#pragma unroll
      for (int ht = 0; ht < HT; ++ht)
#pragma unroll
        for (int i = 0; i < 4; ++i) part += wq[ht][i] * fmaxf(acc[ht][i], 0.f);
      part = wave_sum_xor(part, 48);
      const int e = e0 + tile * 16 + c16;
      if (g == 0 && e < e1) {
        const float s = part * ks;
        srow[e] = s;
        if (hist) atomicAdd(&lhist[order_key(s) >> 20], 1u);
      }
    };

    // two tiles in flight per wave: tile j+4 loads while tile j computes
    long k0[KK], k1[KK];
    float s0 = 0.f, s1 = 0.f;
    int tile = wave;
    if (tile < ntile) load(tile, k0, s0);
    while (tile < ntile) {
      if (tile + 4 < ntile) load(tile + 4, k1, s1);
      compute(tile, k0, s0);
      tile += 4;
      if (tile >= ntile) break;
      if (tile + 4 < ntile) load(tile + 4, k0, s0);
      compute(tile, k1, s1);
      tile += 4;
    }
  }

  if (hist) {
    __syncthreads();
    uint32_t* grow = hist + static_cast<size_t>(row) * kHistBins;
    for (int i = tid; i < kHistBins; i += 256) {
      const uint32_t v = lhist[i];
      if (v) atomicAdd(grow + i, v);
    }
  }
}

// ============================================================================ block helpers
// Threshold bin of a row: the bin tb such that (#keys in bins > tb) < kk <= (#keys in bins >= tb).
__device__ int find_threshold_bin(const uint32_t* __restrict__ h, int kk, uint32_t* s_sum,
                                  int* s_out) {
  const int tid = threadIdx.x;  // 256 threads, 16 bins each
  uint32_t loc[16];
  uint32_t tot = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    loc[j] = h[tid * 16 + j];
    tot += loc[j];
  }
  s_sum[tid] = tot;
  __syncthreads();
  // reverse inclusive scan: s_sum[t] = sum over t' >= t
  for (int off = 1; off < 256; off <<= 1) {
    const uint32_t v = (tid + off < 256) ? s_sum[tid + off] : 0u;
    __syncthreads();
    s_sum[tid] += v;
    __syncthreads();
  }
  const uint32_t above = s_sum[tid] - tot;
  if (above < static_cast<uint32_t>(kk) && static_cast<uint32_t>(kk) <= above + tot) {
    uint32_t cum = above;
    for (int j = 15; j >= 0; --j) {
      if (cum + loc[j] >= static_cast<uint32_t>(kk)) {
        *s_out = tid * 16 + j;
        break;
      }
      cum += loc[j];
    }
  }
  __syncthreads();
  return *s_out;
}

// wave-aggregated append: returns the slot of this lane (valid only if pred)
__device__ __forceinline__ uint32_t wave_append(bool pred, uint32_t* counter) {
  const unsigned long long mask = __ballot(pred);
  if (!mask) return 0;
  const int l = lane_id();
  const int leader = __ffsll(static_cast<long long>(mask)) - 1;
  uint32_t base = 0;
  if (l == leader) base = atomicAdd(counter, static_cast<uint32_t>(__popcll(mask)));
  base = __shfl(base, leader, 64);
  const unsigned long long lower = (l == 0) ? 0ull : (mask & ((1ull << l) - 1ull));
  return base + static_cast<uint32_t>(__popcll(lower));
}

// ============================================================================ multi-WG top-k
__global__ __launch_bounds__(256) void topk_collect_kernel(
    const float* __restrict__ scores, int sstride, const uint32_t* __restrict__ hist,
    const int32_t* __restrict__ n_entries, const int32_t* __restrict__ pos, int nq, int m, int k,
    int n_max, int chunk, int nchunks, uint32_t* __restrict__ counters, int32_t* __restrict__ sel,
    uint64_t* __restrict__ cand) {
  __shared__ uint32_t s_sum[256];
  __shared__ int s_tb;
  const int row = blockIdx.x / nchunks;
  const int n_vis = visible(n_entries, pos, row, nq, m, n_max);
  if (threadIdx.x == 0) s_tb = -1;
  if (n_vis <= k) return;  // everything is selected; finalize handles it
  const int e0 = (blockIdx.x % nchunks) * chunk;
  const int e1 = min(n_vis, e0 + chunk);
  if (e0 >= e1) return;
  const int tb = find_threshold_bin(hist + static_cast<size_t>(row) * kHistBins, k, s_sum, &s_tb);
  const float* srow = scores + static_cast<size_t>(row) * sstride;
  uint32_t* cnt = counters + 2 * row;
  for (int base = e0; base < e1; base += 256) {
    const int e = base + threadIdx.x;
    uint32_t key = 0;
    int bin = -1;
    if (e < e1) {
      key = order_key(srow[e]);
      bin = static_cast<int>(key >> 20);
    }
    const bool is_sel = bin > tb;
    const bool is_cand = bin == tb;
    const uint32_t ps = wave_append(is_sel, cnt + 0);
    if (is_sel && ps < static_cast<uint32_t>(k)) sel[static_cast<size_t>(row) * k + ps] = e;
    const uint32_t pc = wave_append(is_cand, cnt + 1);
    if (is_cand && pc < static_cast<uint32_t>(kCandCap))
      cand[static_cast<size_t>(row) * kCandCap + pc] =
          (static_cast<uint64_t>(key) << 32) | (0xffffffffu - static_cast<uint32_t>(e));
  }
}

template <typename T, bool kDescending>
__device__ void bitonic_sort(T* a, int n) {  // n power of two, 256 threads
  for (int k2 = 2; k2 <= n; k2 <<= 1) {
    for (int j = k2 >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < n; i += 256) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const bool up = ((i & k2) == 0) == kDescending;  // this pair wants a[i] >= a[ixj]
          const T x = a[i], y = a[ixj];
          if (up ? (x < y) : (x > y)) {
            a[i] = y;
            a[ixj] = x;
          }
        }
      }
      __syncthreads();
    }
  }
}

__device__ __forceinline__ int next_pow2(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

// Exact selection of one row by a single workgroup streaming the row (used when a row's
// threshold bin holds more candidates than kCandCap, e.g. massive ties).  Radix select over
// the 32-bit keys finds the kk-th largest key T; an index-ordered pass then takes every key > T
// and the first (lowest-index) keys == T, emitting indices in ascending order.
__device__ void select_row_exact(const float* __restrict__ srow, int n_vis, int kk, int k,
                                 int32_t* __restrict__ out, float* __restrict__ sout,
                                 uint32_t* s_hist /*256*/, int* s_misc /*8*/) {
  const int tid = threadIdx.x;
  uint32_t prefix = 0, mask = 0;
  int remaining = kk;
  for (int shift = 24; shift >= 0; shift -= 8) {
    s_hist[tid] = 0;
    __syncthreads();
    for (int e = tid; e < n_vis; e += 256) {
      const uint32_t key = order_key(srow[e]);
      if ((key & mask) == prefix) atomicAdd(&s_hist[(key >> shift) & 255], 1u);
    }
    __syncthreads();
    if (tid == 0) {
      int cum = 0;
      for (int d = 255; d >= 0; --d) {
        const int c = static_cast<int>(s_hist[d]);
        if (cum + c >= remaining) {
          s_misc[0] = d;
          s_misc[1] = remaining - cum;
          break;
        }
        cum += c;
      }
    }
    __syncthreads();
    prefix |= static_cast<uint32_t>(s_misc[0]) << shift;
    mask |= 255u << shift;
    remaining = s_misc[1];
    __syncthreads();
  }
  const uint32_t T = prefix;
  const int need_eq = remaining;
  // index-ordered compaction
  __shared__ int s_wcnt[2][4];
  int taken = 0, eq_seen = 0;
  const int wave = tid >> 6, l = lane_id();
  for (int base = 0; base < n_vis; base += 256) {
    const int e = base + tid;
    uint32_t key = 0;
    if (e < n_vis) key = order_key(srow[e]);
    const bool eq = (e < n_vis) && key == T;
    const unsigned long long meq = __ballot(eq);
    const unsigned long long lower = (l == 0) ? 0ull : ((1ull << l) - 1ull);
    if (l == 0) s_wcnt[0][wave] = __popcll(meq);
    __syncthreads();
    int eq_before = eq_seen;
    for (int w = 0; w < wave; ++w) eq_before += s_wcnt[0][w];
    eq_before += __popcll(meq & lower);
    const bool take = (e < n_vis) && (key > T || (eq && eq_before < need_eq));
    const unsigned long long mt = __ballot(take);
    if (l == 0) s_wcnt[1][wave] = __popcll(mt);
    __syncthreads();
    int slot = taken;
    for (int w = 0; w < wave; ++w) slot += s_wcnt[1][w];
    slot += __popcll(mt & lower);
    if (take && slot < k) {
      out[slot] = e;
      if (sout) sout[slot] = srow[e];
    }
    int add_eq = 0, add_t = 0;
    for (int w = 0; w < 4; ++w) {
      add_eq += s_wcnt[0][w];
      add_t += s_wcnt[1][w];
    }
    eq_seen += add_eq;
    taken += add_t;
    __syncthreads();
  }
  for (int j = kk + tid; j < k; j += 256) {
    out[j] = -1;
    if (sout) sout[j] = -INFINITY;
  }
}

__global__ __launch_bounds__(256) void topk_finalize_kernel(
    const float* __restrict__ scores, int sstride, const int32_t* __restrict__ n_entries,
    const int32_t* __restrict__ pos, int nq, int m, int k, int n_max,
    const uint32_t* __restrict__ counters,
    const int32_t* __restrict__ sel, const uint64_t* __restrict__ cand,
    int32_t* __restrict__ idx_out, float* __restrict__ score_out) {
  extern __shared__ __align__(16) unsigned char smem[];
  uint64_t* cbuf = reinterpret_cast<uint64_t*>(smem);                  // kCandCap
  int32_t* list = reinterpret_cast<int32_t*>(cbuf + kCandCap);         // kMaxTopK
  __shared__ uint32_t s_hist[256];
  __shared__ int s_misc[8];
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const int n_vis = visible(n_entries, pos, row, nq, m, n_max);
  const int kk = min(k, n_vis);
  int32_t* out = idx_out + static_cast<size_t>(row) * k;
  float* sout = score_out ? score_out + static_cast<size_t>(row) * k : nullptr;
  const float* srow = scores + static_cast<size_t>(row) * sstride;
  if (n_vis <= k) {
    for (int j = tid; j < k; j += 256) {
      out[j] = j < n_vis ? j : -1;
      if (sout) sout[j] = j < n_vis ? srow[j] : -INFINITY;
    }
    return;
  }
  const int n_gt = static_cast<int>(counters[2 * row]);
  const int nc = static_cast<int>(counters[2 * row + 1]);
  // the candidate path needs n_gt < kk <= n_gt + nc <= n_gt + kCandCap; anything else (massive
  // ties in the threshold bin) takes the exact streaming path
  if (nc > kCandCap || n_gt >= kk || n_gt + nc < kk) {
    select_row_exact(srow, n_vis, kk, k, out, sout, s_hist, s_misc);
    return;
  }
  const int need = kk - n_gt;
  const int p2c = next_pow2(nc);
  for (int j = tid; j < p2c; j += 256)
    cbuf[j] = j < nc ? cand[static_cast<size_t>(row) * kCandCap + j] : 0ull;
  __syncthreads();
  bitonic_sort<uint64_t, true>(cbuf, p2c);
  const int p2k = next_pow2(kk);
  for (int j = tid; j < p2k; j += 256) {
    int32_t v = 0x7fffffff;
    if (j < n_gt)
      v = sel[static_cast<size_t>(row) * k + j];
    else if (j < kk)
      v = static_cast<int32_t>(0xffffffffu - static_cast<uint32_t>(cbuf[j - n_gt] & 0xffffffffu));
    list[j] = v;
  }
  __syncthreads();
  bitonic_sort<int32_t, false>(list, p2k);
  for (int j = tid; j < k; j += 256) {
    const int v = j < kk ? list[j] : -1;
    out[j] = v;
    if (sout) sout[j] = j < kk ? srow[v] : -INFINITY;
  }
}

// ============================================================================ per-row top-k
__global__ __launch_bounds__(256) void topk_row_kernel(
    const float* __restrict__ scores, int sstride, const int32_t* __restrict__ n_entries,
    const int32_t* __restrict__ pos, int nq, int m, int k, int n_max, int32_t* __restrict__ idx_out,
    float* __restrict__ score_out) {
  extern __shared__ __align__(16) unsigned char smem[];
  uint32_t* keys = reinterpret_cast<uint32_t*>(smem);  // kRowTopkMaxN
  __shared__ uint32_t s_hist[256];
  __shared__ int s_misc[8];
  __shared__ int s_wcnt[2][4];
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const int n_vis = visible(n_entries, pos, row, nq, m, n_max);
  const int kk = min(k, n_vis);
  int32_t* out = idx_out + static_cast<size_t>(row) * k;
  float* sout = score_out ? score_out + static_cast<size_t>(row) * k : nullptr;
  const float* srow = scores + static_cast<size_t>(row) * sstride;
  if (n_vis <= k) {
    for (int j = tid; j < k; j += 256) {
      out[j] = j < n_vis ? j : -1;
      if (sout) sout[j] = j < n_vis ? srow[j] : -INFINITY;
    }
    return;
  }
  if (n_vis > kRowTopkMaxN) {
    select_row_exact(srow, n_vis, kk, k, out, sout, s_hist, s_misc);
    return;
  }
  for (int e = tid; e < n_vis; e += 256) keys[e] = order_key(srow[e]);
  __syncthreads();
  uint32_t prefix = 0, mask = 0;
  int remaining = kk;
  for (int shift = 24; shift >= 0; shift -= 8) {
    s_hist[tid] = 0;
    __syncthreads();
    for (int e = tid; e < n_vis; e += 256) {
      const uint32_t key = keys[e];
      if ((key & mask) == prefix) atomicAdd(&s_hist[(key >> shift) & 255], 1u);
    }
    __syncthreads();
    if (tid < 64) {
      // digit search by one wave: suffix sums over 256 digits, 4 per lane
      const int l = tid;
      uint32_t c4[4];
      uint32_t tot = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        c4[j] = s_hist[l * 4 + j];
        tot += c4[j];
      }
      // inclusive suffix scan of tot across lanes (lane l gets sum over lanes >= l)
      uint32_t suf = tot;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t v = __shfl_down(suf, off, 64);
        if (l + off < 64) suf += v;
      }
      const uint32_t above = suf - tot;
      if (above < static_cast<uint32_t>(remaining) &&
          static_cast<uint32_t>(remaining) <= above + tot) {
        uint32_t cum = above;
        for (int j = 3; j >= 0; --j) {
          if (cum + c4[j] >= static_cast<uint32_t>(remaining)) {
            s_misc[0] = l * 4 + j;
            s_misc[1] = remaining - static_cast<int>(cum);
            break;
          }
          cum += c4[j];
        }
      }
    }
    __syncthreads();
    prefix |= static_cast<uint32_t>(s_misc[0]) << shift;
    mask |= 255u << shift;
    remaining = s_misc[1];
    __syncthreads();
  }
  const uint32_t T = prefix;
  const int need_eq = remaining;
  int taken = 0, eq_seen = 0;
  const int wave = tid >> 6, l = lane_id();
  const unsigned long long lower = (l == 0) ? 0ull : ((1ull << l) - 1ull);
  for (int base = 0; base < n_vis; base += 256) {
    const int e = base + tid;
    const uint32_t key = e < n_vis ? keys[e] : 0u;
    const bool eq = (e < n_vis) && key == T;
    const unsigned long long meq = __ballot(eq);
    const bool gt = (e < n_vis) && key > T;
    if (l == 0) s_wcnt[0][wave] = __popcll(meq);
    __syncthreads();
    int eq_before = eq_seen + __popcll(meq & lower);
    for (int w = 0; w < wave; ++w) eq_before += s_wcnt[0][w];
    const bool take = gt || (eq && eq_before < need_eq);
    const unsigned long long mt = __ballot(take);
    if (l == 0) s_wcnt[1][wave] = __popcll(mt);
    __syncthreads();
    int slot = taken + __popcll(mt & lower);
    for (int w = 0; w < wave; ++w) slot += s_wcnt[1][w];
    if (take && slot < k) {
      out[slot] = e;
      if (sout) sout[slot] = srow[e];
    }
    for (int w = 0; w < 4; ++w) {
      eq_seen += s_wcnt[0][w];
      taken += s_wcnt[1][w];
    }
    __syncthreads();
  }
  for (int j = kk + tid; j < k; j += 256) {
    out[j] = -1;
    if (sout) sout[j] = -INFINITY;
  }
}

// ============================================================================ fill
__global__ void fill_u32_kernel(uint32_t* __restrict__ p, uint32_t v, size_t n) {
  for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<size_t>(gridDim.x) * blockDim.x)
    p[i] = v;
}

hipError_t launch_fill_u32(uint32_t* p, uint32_t v, size_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const size_t blocks = (n + 255) / 256;
  const unsigned grid = static_cast<unsigned>(blocks < 4096 ? blocks : 4096);
  fill_u32_kernel<<<grid, 256, 0, s>>>(p, v, n);
  return hipGetLastError();
}

// ============================================================================ launchers
static size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

static int score_stride(int n_max) { return (n_max + 63) & ~63; }

size_t index_topk_workspace(int rows, int n_max, int k, bool multi) {
  size_t b = align256(static_cast<size_t>(rows) * score_stride(n_max) * sizeof(float));
  if (multi) {
    b += align256(static_cast<size_t>(rows) * kHistBins * 4);
    b += align256(static_cast<size_t>(rows) * 2 * 4);
    b += align256(static_cast<size_t>(rows) * k * 4);
    b += align256(static_cast<size_t>(rows) * kCandCap * 8);
  }
  return b;
}

template <int DI, int HT>
static void launch_scores_t(const IndexArgs& a, int chunk, int nchunks, uint32_t* hist,
                            hipStream_t s) {
  const unsigned grid = static_cast<unsigned>(nchunks) * static_cast<unsigned>(a.B * a.nq);
  index_score_kernel<DI, HT><<<grid, 256, 0, s>>>(a.qi, a.qi_scale, a.wi, a.keys, a.kscale,
                                                  a.n_entries, a.pos, a.nq, a.n_max, a.H_I, a.m,
                                                  chunk, a.scores, a.sstride, hist, nchunks);
}

static hipError_t launch_scores(const IndexArgs& a, int chunk, uint32_t* hist, hipStream_t s) {
  const int nchunks = (a.n_max + chunk - 1) / chunk;
  const int ht = (a.H_I + 15) / 16;
#define CSA_SCORE_CASE(DI_, HT_)                        \
  if (a.d_I == DI_ && ht == HT_) {                     \
    launch_scores_t<DI_, HT_>(a, chunk, nchunks, hist, s); \
    return hipGetLastError();                          \
  }
  CSA_SCORE_CASE(128, 4)
  CSA_SCORE_CASE(128, 3)
  CSA_SCORE_CASE(128, 2)
  CSA_SCORE_CASE(128, 1)
  CSA_SCORE_CASE(64, 4)
  CSA_SCORE_CASE(64, 3)
  CSA_SCORE_CASE(64, 2)
  CSA_SCORE_CASE(64, 1)
  CSA_SCORE_CASE(32, 4)
  CSA_SCORE_CASE(32, 3)
  CSA_SCORE_CASE(32, 2)
  CSA_SCORE_CASE(32, 1)
#undef CSA_SCORE_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_index_topk(const IndexArgs& a, bool multi, hipStream_t s) {
  const int rows = a.B * a.nq;
  hipError_t e;
  if (multi) {
    // histogram + counters must start at zero
    e = launch_fill_u32(a.hist, 0u, static_cast<size_t>(rows) * kHistBins, s);
    if (e != hipSuccess) return e;
    e = launch_fill_u32(a.counters, 0u, static_cast<size_t>(rows) * 2, s);
    if (e != hipSuccess) return e;
  }
  const int chunk = 2048;
  e = launch_scores(a, chunk, multi ? a.hist : nullptr, s);
  if (e != hipSuccess) return e;
  if (multi) {
    const int cchunk = 4096;
    const int ncc = (a.n_max + cchunk - 1) / cchunk;
    const unsigned grid = static_cast<unsigned>(ncc) * static_cast<unsigned>(rows);
    topk_collect_kernel<<<grid, 256, 0, s>>>(a.scores, a.sstride, a.hist, a.n_entries, a.pos,
                                             a.nq, a.m, a.k, a.n_max, cchunk, ncc, a.counters,
                                             a.sel, a.cand);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t lds = kCandCap * 8 + kMaxTopK * 4;
    topk_finalize_kernel<<<rows, 256, lds, s>>>(a.scores, a.sstride, a.n_entries, a.pos, a.nq,
                                                a.m, a.k, a.n_max, a.counters, a.sel, a.cand,
                                                a.idx_out, a.score_out);
    return hipGetLastError();
  }
  const size_t lds = kRowTopkMaxN * 4;
  static bool attr_set = false;
  if (!attr_set) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(topk_row_kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  topk_row_kernel<<<rows, 256, lds, s>>>(a.scores, a.sstride, a.n_entries, a.pos, a.nq, a.m,
                                         a.k, a.n_max, a.idx_out, a.score_out);
  return hipGetLastError();
}

hipError_t launch_index_prefill(const IndexArgs& a, hipStream_t s) {
  return launch_index_topk(a, false, s);
}

}  // namespace csa
