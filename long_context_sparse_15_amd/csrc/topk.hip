// Exact top-k selection of the indexer scores for gfx950.
//
// Method: "DeepSeek V4 模型技术大全", chapter "Attention", section "CSA 的完整路径":
//   I_t = TopK_k { I_{t,s} | s < floor((t+1)/m) }.
//
// Top-k is exact with the lower index winning ties.  Scores (fp32, or bf16 widened exactly)
// become order-preserving 32-bit keys.  Rows of up to 32768 entries use one workgroup per row
// with the keys in registers or LDS: a sampled threshold, an exact select among the few
// candidates above it (or a radix select) and an index-ordered compaction that emits the
// selection sorted.  Longer rows (decode at long context, few rows) are cut into 4096-entry
// chunks, one workgroup each, that take thresholds of their own and write their candidates; a
// finalize workgroup per row selects among them and emits the selection in ascending index
// order.
#include "topk_common.h"

namespace csa {

// Index-ordered emission of a row's selection: every key > T, then the first need_eq keys == T
// in index order; indices come out ascending.  key(e) reads the row's key of entry e.  Each wave
// owns a contiguous segment of the row: a counting pass (ballots), one exchange of per-wave
// counts, and an emitting pass whose slots come from ballot prefix counts.
template <int THREADS, typename KeyFn, typename EmitFn>
__device__ void ordered_emit_fn(KeyFn key, int n, uint32_t T, int need_eq, int cap, EmitFn emit) {
  constexpr int NWAVE = THREADS / 64;
  __shared__ uint32_t s_gt[NWAVE], s_eq[NWAVE];
  const int l = lane_id(), wave = threadIdx.x >> 6;
  const unsigned long long lower = (l == 0) ? 0ull : ((1ull << l) - 1ull);
  const int seg = ((n + NWAVE - 1) / NWAVE + 63) & ~63;
  const int s0 = min(n, wave * seg), s1 = min(n, s0 + seg);
  uint32_t cgt = 0, ceq = 0;
  for (int base = s0; base < s1; base += 64) {
    const int e = base + l;
    const uint32_t kv = e < s1 ? key(e) : 0u;
    cgt += __popcll(__ballot(e < s1 && kv > T));
    ceq += __popcll(__ballot(e < s1 && kv == T));
  }
  if (l == 0) {
    s_gt[wave] = cgt;
    s_eq[wave] = ceq;
  }
  __syncthreads();
  // keys > T and == T in the earlier waves' segments; the == T keys taken before this wave are
  // the first min(need_eq, eq_seen) of them (a loop of constant length: its reads go out
  // together)
  int eq_seen = 0, gt_seen = 0;
#pragma unroll
  for (int w2 = 0; w2 < NWAVE - 1; ++w2) {
    if (w2 < wave) {
      gt_seen += static_cast<int>(s_gt[w2]);
      eq_seen += static_cast<int>(s_eq[w2]);
    }
  }
  int slot_base = gt_seen + min(need_eq, eq_seen);
  for (int base = s0; base < s1; base += 64) {
    const int e = base + l;
    const uint32_t kv = e < s1 ? key(e) : 0u;
    const bool eq = e < s1 && kv == T;
    const bool gt = e < s1 && kv > T;
    const unsigned long long meq = __ballot(eq);
    const bool take = gt || (eq && eq_seen + __popcll(meq & lower) < need_eq);
    const unsigned long long mt = __ballot(take);
    const int slot = slot_base + __popcll(mt & lower);
    if (take && slot < cap) emit(slot, e);
    slot_base += __popcll(mt);
    eq_seen += __popcll(meq);
  }
  __syncthreads();  // s_gt / s_eq are reused by the next call
}

// Emission straight into a row of the output (and its scores), padded with -1 / -inf.
template <int THREADS, typename KeyFn, typename ST>
__device__ void ordered_emit(KeyFn key, int n, uint32_t T, int need_eq, int kk, int k,
                             const ST* __restrict__ srow, int32_t* __restrict__ out,
                             float* __restrict__ sout, uint32_t* s_tmp) {
  ordered_emit_fn<THREADS>(key, n, T, need_eq, k, [&](int slot, int e) {
    out[slot] = e;
    if (sout) sout[slot] = Scores<ST>::at(srow, e);
  });
  for (int j = kk + threadIdx.x; j < k; j += THREADS) {
    out[j] = -1;
    if (sout) sout[j] = -INFINITY;
  }
  (void)s_tmp;
}

// Radix select of the kk-th largest key among n keys with 12 + 12 + 8 bit passes over a 4096-bin
// histogram.  Returns T (the kk-th largest key) and need_eq (how many keys == T are taken).
template <int THREADS, typename KeyFn>
__device__ void radix_select(KeyFn key, int n, int kk, uint32_t* hist /*4096*/, uint32_t* s_tmp,
                             int* s_res, uint32_t& T, int& need_eq) {
  const int tid = threadIdx.x;
  uint32_t prefix = 0, mask = 0;
  uint32_t remaining = static_cast<uint32_t>(kk);
  const int shifts[3] = {20, 8, 0};
  const int widths[3] = {12, 12, 8};
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = shifts[pass];
    const int nb = 1 << widths[pass];
    for (int i = tid; i < nb; i += THREADS) hist[i] = 0;
    __syncthreads();
    for (int e = tid; e < n; e += THREADS) {
      const uint32_t kv = key(e);
      if ((kv & mask) == prefix) atomicAdd(&hist[(kv >> shift) & (nb - 1)], 1u);
    }
    __syncthreads();
    if (nb >= THREADS) {
      block_find_crossing<THREADS>(hist, nb, remaining, s_tmp, s_res);
    } else {  // 256 bins with more than 256 threads: first 256 threads only
      if (tid < 64) {
        const int l = tid;
        uint32_t c4[4], own = 0;
        for (int j = 0; j < 4; ++j) {
          c4[j] = hist[l * 4 + j];
          own += c4[j];
        }
        const uint32_t inc = wave_incl_scan(own);
        const uint32_t above = __builtin_amdgcn_readlane(inc, 63) - inc;
        if (above < remaining && remaining <= above + own) {
          uint32_t cum = above;
          for (int j = 3; j >= 0; --j) {
            if (cum + c4[j] >= remaining) {
              s_res[0] = l * 4 + j;
              s_res[1] = static_cast<int>(remaining - cum);
              break;
            }
            cum += c4[j];
          }
        }
      }
      __syncthreads();
    }
    const uint32_t d = static_cast<uint32_t>(s_res[0]);
    remaining = static_cast<uint32_t>(s_res[1]);
    prefix |= d << shift;
    mask |= static_cast<uint32_t>(nb - 1) << shift;
    __syncthreads();
  }
  T = prefix;
  need_eq = static_cast<int>(remaining);
}

// Exact kk-th largest key (T) among n keys that all lie in [lo, hi], and how many keys equal
// to T are taken (need_eq).  A 12-bit histogram over the bits just below the common prefix of
// lo and hi (so the bins split the keys' actual range); while the crossing bin holds more than
// 64 keys (crowded or tied scores) the next 12 bits of that bin are histogrammed, until it is
// small or every bit is fixed.  A small bin's keys are gathered and ranked by pairwise
// comparison in one wave.  (Each pass after the first counts only the keys in the crossing bin
// and fixes 12 more bits; the 4096 bins hold the bin's few bits above them at one value.)
template <int THREADS, typename KeyFn>
__device__ void select_kth(KeyFn key, int n, int kk, uint32_t lo, uint32_t hi,
                           uint32_t* hist /*4096*/, uint32_t* s_tmp, int* s_res, uint32_t& T,
                           int& need_eq, bool zeroed = false) {
  __shared__ uint32_t s_bin[64];
  __shared__ uint32_t s_nb;
  const int tid = threadIdx.x;
  const uint32_t diff = lo ^ hi;
  const int top = diff ? 32 - __clz(diff) : 0;  // bits below the common prefix
  int shift = top > 12 ? top - 12 : 0;
  uint32_t pmask = top >= 32 ? 0u : ~((1u << top) - 1u);
  uint32_t prefix = lo & pmask;
  uint32_t c1 = radix_pass<THREADS>(key, n, prefix, pmask, shift, 4096,
                                    static_cast<uint32_t>(kk), hist, s_tmp, s_res, zeroed);
  uint32_t d1 = static_cast<uint32_t>(s_res[0]);
  uint32_t r1 = static_cast<uint32_t>(s_res[1]);
  __syncthreads();
  while (c1 > 64 && shift > 0) {  // (uniform: every thread holds the same values)
    prefix = (prefix | (d1 << shift)) & ~((1u << shift) - 1u);
    pmask = ~((1u << shift) - 1u);
    shift = shift > 12 ? shift - 12 : 0;
    c1 = radix_pass<THREADS>(key, n, prefix, pmask, shift, 4096, r1, hist, s_tmp, s_res);
    d1 = static_cast<uint32_t>(s_res[0]);
    r1 = static_cast<uint32_t>(s_res[1]);
    __syncthreads();
  }
  if (c1 > 64) {  // every bit fixed: the bin is one key value, T, of which r1 are taken
    T = (prefix & pmask) | d1;
    need_eq = static_cast<int>(r1);
    return;
  }
  if (tid == 0) s_nb = 0;
  __syncthreads();
  for (int e = tid; e < n; e += THREADS) {
    const uint32_t kv = key(e);
    if ((kv & pmask) == prefix && ((kv >> shift) & 4095u) == d1) s_bin[atomicAdd(&s_nb, 1u)] = kv;
  }
  __syncthreads();
  if (tid < 64) {  // wave 0: rank the bin's keys; the r1-th largest is T
    const int nbk = static_cast<int>(s_nb);
    const uint32_t mine = tid < nbk ? s_bin[tid] : 0u;
    int gt = 0, eq = 0;
    for (int j = 0; j < nbk; ++j) {  // key j from lane j's register, no LDS round trip
      const uint32_t o = __builtin_amdgcn_readlane(mine, j);
      gt += o > mine;
      eq += o == mine;
    }
    if (tid < nbk && gt < static_cast<int>(r1) && static_cast<int>(r1) <= gt + eq) {
      s_res[0] = static_cast<int>(mine);  // every lane holding T writes the same values
      s_res[1] = static_cast<int>(r1) - gt;
    }
  }
  __syncthreads();
  T = static_cast<uint32_t>(s_res[0]);
  need_eq = s_res[1];
  __syncthreads();
}

// ============================================================================ per-row top-k
// One workgroup per query row; the row's keys live in LDS when n_vis <= CAP, otherwise they are
// re-read from the score row in global memory on every pass (exact, slower).
template <int THREADS, int CAP, typename ST>
__global__ __launch_bounds__(THREADS) void topk_row_kernel(
    const ST* __restrict__ scores, int sstride, const int32_t* __restrict__ n_entries,
    const int32_t* __restrict__ pos, int nq, int m, int k, int n_max, int32_t* __restrict__ idx_out,
    float* __restrict__ score_out) {
  extern __shared__ __align__(16) unsigned char smem[];
  uint32_t* keys = reinterpret_cast<uint32_t*>(smem);  // CAP
  uint32_t* hist = keys + CAP;                          // 4096
  __shared__ uint32_t s_tmp[THREADS / 64];
  __shared__ int s_res[2];
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const int n_vis = visible(n_entries, pos, row, nq, m, n_max);
  const int kk = min(k, n_vis);
  int32_t* out = idx_out + static_cast<size_t>(row) * k;
  float* sout = score_out ? score_out + static_cast<size_t>(row) * k : nullptr;
  const ST* srow = scores + static_cast<size_t>(row) * sstride;
  if (n_vis <= k) {
    for (int j = tid; j < k; j += THREADS) {
      out[j] = j < n_vis ? j : -1;
      if (sout) sout[j] = j < n_vis ? Scores<ST>::at(srow, j) : -INFINITY;
    }
    return;
  }
  uint32_t T;
  int need_eq;
  if (n_vis <= CAP) {
    const int n4 = n_vis >> 2;
    for (int i = tid; i < n4; i += THREADS) {
      float v[4];
      Scores<ST>::four(srow, 4 * i, v);
#pragma unroll
      for (int j = 0; j < 4; ++j) keys[4 * i + j] = order_key(v[j]);
    }
    for (int e = 4 * n4 + tid; e < n_vis; e += THREADS) keys[e] = order_key(Scores<ST>::at(srow, e));
    __syncthreads();
    auto kf = [&](int e) { return keys[e]; };
    radix_select<THREADS>(kf, n_vis, kk, hist, s_tmp, s_res, T, need_eq);
    ordered_emit<THREADS>(kf, n_vis, T, need_eq, kk, k, srow, out, sout, s_tmp);
  } else {
    auto kf = [&](int e) { return order_key(Scores<ST>::at(srow, e)); };
    radix_select<THREADS>(kf, n_vis, kk, hist, s_tmp, s_res, T, need_eq);
    ordered_emit<THREADS>(kf, n_vis, T, need_eq, kk, k, srow, out, sout, s_tmp);
  }
}

// ============================================================================ sampled row top-k
// One workgroup per row; thread t holds in registers the keys of the row's 16-byte chunks
// i*THREADS + t, i < PER/4 (coalesced loads), so chunk column i of all threads precedes column
// i+1 in index order.
//  1. the first key of every fourth chunk is a sample (1 in 16); the lower edge of the 12-bit
//     bin holding the r-th largest sample (r a little above kk/16 with a margin of 4 standard
//     deviations; refined by a second pass when that bin is crowded) is a threshold T_lo that
//     almost surely has between kk and kCandCap keys at or above it;
//  2. each thread counts its candidates (keys >= T_lo) per chunk column, two 16-bit counts to a
//     word; one block prefix sum over those words places every candidate (key, index) in LDS in
//     ascending index order;
//  3. select_kth finds the kk-th candidate key T and how many keys equal to T are taken;
//  4. the index-ordered emission over the candidate list writes the keys above T and the first
//     ties, so the selection comes out sorted with the lowest indices winning ties.
// If the count misses [kk, kCandCap] (ties, adversarial data) the exact streaming select runs.
// CLAMP (runs of query rows, whose causal lengths vary): the row's visible length is read first
// and chunk loads past it re-read the row's last visible chunk (a cache hit), so a row moves
// only its visible scores from HBM; otherwise (decode: full rows, few of them) every chunk load
// goes out before the length is known, one memory round trip sooner.
template <int THREADS, int PER, typename ST, bool CLAMP = false>
__global__ __launch_bounds__(THREADS) void topk_sample_kernel(
    const ST* __restrict__ scores, int sstride, const int32_t* __restrict__ n_entries,
    const int32_t* __restrict__ pos, int nq, int m, int k, int n_max, int32_t* __restrict__ idx_out,
    float* __restrict__ score_out) {
  constexpr int CH = PER / 4;             // chunks per thread
  constexpr int SPT = CH / 4;             // samples per thread
  constexpr int NS = THREADS * SPT;       // sample slots
  constexpr int NWAVE = THREADS / 64;
  constexpr int CW = CH / 2;              // count words per thread, two chunk columns each
  static_assert(CH % 4 == 0 && CW <= 4, "chunk and count layout");
  static_assert(THREADS * 4 <= 0xffff, "a column's candidate count fits 16 bits");
  __shared__ uint32_t s_samp[NS];
  __shared__ uint32_t s_hist[kHistBins];
  __shared__ uint32_t s_ckey[kCandCap];
  __shared__ int32_t s_cidx[kCandCap];
  __shared__ u32x4 s_wcnt[NWAVE];
  __shared__ uint32_t s_tmp[NWAVE];
  __shared__ int s_res[2];
  __shared__ uint32_t s_max;
  const int row = blockIdx.x;
  const int tid = threadIdx.x, l = lane_id(), wave = tid >> 6;
  const ST* srow = scores + static_cast<size_t>(row) * sstride;
  // keys; every chunk load is issued (clamped into the row) and masked, the row's last partial
  // chunk is read element by element.  The addresses depend only on the row length, so the
  // loads go out first, before the row's position and entry count are known, and all of them
  // before any is used (pinned: otherwise the compiler splits them and sinks the pieces into
  // per-element branches, each behind a wait).
  float f[CH][4];
  int n_vis;
  if constexpr (CLAMP) {
    n_vis = visible(n_entries, pos, row, nq, m, n_max);
    const int last = max(n_vis - 1, 0) & ~3;  // start of the chunk holding the last visible key
#pragma unroll
    for (int i = 0; i < CH; ++i) Scores<ST>::four(srow, min((i * THREADS + tid) * 4, last), f[i]);
    asm volatile("" ::: "memory");
  } else {
#pragma unroll
    for (int i = 0; i < CH; ++i)
      Scores<ST>::four(srow, min((i * THREADS + tid) * 4, sstride - 4), f[i]);
    asm volatile("" ::: "memory");
    n_vis = visible(n_entries, pos, row, nq, m, n_max);
  }
  const int kk = min(k, n_vis);
  int32_t* out = idx_out + static_cast<size_t>(row) * k;
  float* sout = score_out ? score_out + static_cast<size_t>(row) * k : nullptr;
  if (n_vis <= k) {
    for (int j = tid; j < k; j += THREADS) {
      out[j] = j < n_vis ? j : -1;
      if (sout) sout[j] = j < n_vis ? Scores<ST>::at(srow, j) : -INFINITY;
    }
    return;
  }
  uint32_t kr[PER];
  {
#pragma unroll
    for (int i = 0; i < CH; ++i)
      asm volatile("" : "+v"(f[i][0]), "+v"(f[i][1]), "+v"(f[i][2]), "+v"(f[i][3]) : : "memory");
    // keys past n_vis are 0, below every key of a finite score (order_key >= 0x007fffff), so
    // the candidate passes below compare keys only; one bound check per chunk (the row's partial
    // last chunk is filled in below)
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const bool full = (i * THREADS + tid) * 4 + 4 <= n_vis;
#pragma unroll
      for (int j = 0; j < 4; ++j) kr[i * 4 + j] = full ? order_key(f[i][j]) : 0u;
    }
  }
  // the first histogram pass finds it cleared (written while the loads are in flight)
  for (int i = tid; i < kHistBins; i += THREADS) s_hist[i] = 0u;
  {
    const int last = (n_vis - 1) & ~3;  // start of the chunk holding the last visible entry
    if (n_vis & 3) {
#pragma unroll
      for (int i = 0; i < CH; ++i)
        if ((i * THREADS + tid) * 4 == last) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (last + j < n_vis) kr[i * 4 + j] = order_key(Scores<ST>::at(srow, last + j));
        }
    }
  }
  // samples: slot (i/4)*THREADS + t holds the first key of chunk i*THREADS + t (i % 4 == 0);
  // entries grow with the slot, so the visible samples are a prefix of ns slots
#pragma unroll
  for (int i = 0; i < CH; i += 4) {
    const int base = (i * THREADS + tid) * 4;
    s_samp[(i / 4) * THREADS + tid] = base < n_vis ? kr[i * 4] : 0u;
  }
  const int qch = (n_vis + 3) / 4;  // chunks that start below n_vis
  int ns = 0;
#pragma unroll
  for (int g = 0; g < SPT; ++g) ns += max(0, min(THREADS, qch - 4 * g * THREADS));
  if (tid == 0) s_max = 0u;
  __syncthreads();
  const float expect = static_cast<float>(kk) * static_cast<float>(ns) / static_cast<float>(n_vis);
  int r = static_cast<int>(ceilf(expect + 4.f * sqrtf(expect) + 4.f));
  if (r > ns) r = ns;
  // T_lo: the lower edge of the 12-bit bin that holds the r-th largest sample (refined by a
  // second 12-bit pass when that bin holds more than 64 samples)
  auto sf = [&](int j) { return s_samp[j]; };
  uint32_t Tlo;
  {
    const uint32_t cb = radix_pass<THREADS>(sf, ns, 0u, 0u, 20, 4096, static_cast<uint32_t>(r),
                                            s_hist, s_tmp, s_res, /*zeroed=*/true);
    const uint32_t d1 = static_cast<uint32_t>(s_res[0]);
    const uint32_t r1 = static_cast<uint32_t>(s_res[1]);
    __syncthreads();
    Tlo = d1 << 20;
    if (cb > 64) {
      radix_pass<THREADS>(sf, ns, d1 << 20, 0xfff00000u, 8, 4096, r1, s_hist, s_tmp, s_res);
      Tlo |= static_cast<uint32_t>(s_res[0]) << 8;
      __syncthreads();
    }
  }
  // candidates (visible keys >= T_lo; past n_vis every key is 0 < Tc) per chunk column, packed
  // two columns to a word, and the largest key (a candidate whenever any key is one)
  const uint32_t Tc = max(Tlo, 1u);
  uint32_t cw[CW], kmax = 0;
#pragma unroll
  for (int w = 0; w < CW; ++w) cw[w] = 0u;
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    uint32_t c = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      c += kr[i * 4 + j] >= Tc ? 1u : 0u;
      kmax = max(kmax, kr[i * 4 + j]);
    }
    cw[i / 2] += c << (16 * (i & 1));
  }
  uint32_t inc[CW];
#pragma unroll
  for (int w = 0; w < CW; ++w) inc[w] = wave_incl_scan(cw[w]);
  kmax = wave_max_u32(kmax);
  if (l == 63) {
    u32x4 t4 = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int w = 0; w < CW; ++w) t4[w] = inc[w];
    s_wcnt[wave] = t4;
  }
  if (l == 0 && kmax) atomicMax(&s_max, kmax);
  // select_kth's histogram pass finds it cleared
  for (int i = tid; i < kHistBins; i += THREADS) s_hist[i] = 0u;
  __syncthreads();
  // lane j < NWAVE takes wave j's totals; a scan across those lanes gives every wave the words
  // of the waves before it and the block totals
  uint32_t before[CW], tot[CW];
  {
    const int uw = __builtin_amdgcn_readfirstlane(wave);
    const u32x4 mine = l < NWAVE ? s_wcnt[l] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int w = 0; w < CW; ++w) {
      const uint32_t sc = wave_incl_scan(mine[w]);
      tot[w] = __builtin_amdgcn_readlane(sc, NWAVE - 1);
      const uint32_t prev = uw > 0 ? __builtin_amdgcn_readlane(sc, uw > 0 ? uw - 1 : 0) : 0u;
      before[w] = inc[w] - cw[w] + prev;
    }
  }
  uint32_t cnt = 0;
  uint32_t slot[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    slot[i] = cnt + ((before[i / 2] >> (16 * (i & 1))) & 0xffffu);
    cnt += (tot[i / 2] >> (16 * (i & 1))) & 0xffffu;
  }
  if (cnt >= static_cast<uint32_t>(kk) && cnt <= static_cast<uint32_t>(kCandCap)) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      uint32_t sl = slot[i];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (kr[i * 4 + j] >= Tc) {
          s_ckey[sl] = kr[i * 4 + j];
          s_cidx[sl] = (i * THREADS + tid) * 4 + j;
          ++sl;
        }
      }
    }
    __syncthreads();
    uint32_t T;
    int need_eq;
    auto cf = [&](int j) { return s_ckey[j]; };
    select_kth<THREADS>(cf, static_cast<int>(cnt), kk, Tlo, s_max, s_hist, s_tmp, s_res, T,
                        need_eq, /*zeroed=*/true);
    ordered_emit_fn<THREADS>(cf, static_cast<int>(cnt), T, need_eq, k, [&](int o, int j) {
      const int e = s_cidx[j];
      out[o] = e;
      if (sout) sout[o] = Scores<ST>::at(srow, e);
    });
    for (int j = kk + tid; j < k; j += THREADS) {
      out[j] = -1;
      if (sout) sout[j] = -INFINITY;
    }
    return;
  }
  uint32_t T;
  int need_eq;
  auto gk = [&](int e) { return order_key(Scores<ST>::at(srow, e)); };
  radix_select<THREADS>(gk, n_vis, kk, s_hist, s_tmp, s_res, T, need_eq);
  ordered_emit<THREADS>(gk, n_vis, T, need_eq, kk, k, srow, out, sout, s_tmp);
}

// ============================================================================ multi-WG top-k
// For rows longer than one workgroup's register file (decode at long context).  A row is cut
// into chunks, each of which selects its candidates itself: the decode scorer's workgroups do so
// for the entries they have just scored (index.hip), otherwise one 1024-thread workgroup per
// kCollectChunk entries reads them back (topk_collect_kernel).  A chunk selects its
// candidates with a threshold of its own: T_c, the lower edge of the 12-bit bin (refined
// by 12 more bits when crowded) holding its r-th largest key, r = the chunk's expected share of
// the row's top kk plus four standard deviations.  It writes the (key, index) pairs >= T_c in
// ascending index order into its own region (block prefix sum, no global atomics) with the
// count and T_c.  A finalize workgroup per row (a second launch: a device-scope handoff inside
// one launch costs an L2 write-back per workgroup on this multi-XCD part) concatenates the
// regions (a list in ascending index order), finds the kk-th key T of the list with one
// histogram pass over its actual range and emits the keys above it plus the first ties in index
// order.  The list holds every key >= T of the row exactly when T >= every chunk's T_c (a key
// >= T is then >= its chunk's threshold).  Otherwise (a chunk holding far more than its share
// of the top keys) the chunks with T_c > T are read again for every key >= T and the list is
// rebuilt around them (see the finalize); on a region overflow, too few candidates or too many
// such chunks the exact streaming select of the row runs instead.
constexpr int kSCandCap = 8192;  // candidates of a row held by its finalize workgroup
constexpr int kRepairChunks = 16;  // chunks a finalize re-reads when their thresholds cut T
constexpr size_t kMultiLds = static_cast<size_t>(kSCandCap) * 8 + kHistBins * 4;

template <typename ST>
__global__ __launch_bounds__(1024) void topk_collect_kernel(
    const ST* __restrict__ scores, int sstride, const int32_t* __restrict__ n_entries,
    const int32_t* __restrict__ pos, int nq, int m, int k, int n_max, int nchunks,
    uint32_t* __restrict__ ccount, uint64_t* __restrict__ cand) {
  constexpr int THREADS = 1024, PER = kCollectChunk / THREADS;
  static_assert(PER == 4, "one 16-byte load of keys per thread");
  __shared__ uint32_t s_key[kCollectChunk];
  __shared__ uint32_t hist[kHistBins];
  __shared__ uint32_t s_tmp[THREADS / 64];
  __shared__ int s_res[2];
  asm volatile("" ::"s"(scores), "s"(sstride), "s"(n_entries), "s"(pos), "s"(nq), "s"(m), "s"(k),
               "s"(n_max), "s"(nchunks), "s"(ccount), "s"(cand));  // all parameters at once
  const int row = blockIdx.x / nchunks;
  const int chunk = blockIdx.x % nchunks;
  const int tid = threadIdx.x;
  const ST* srow = scores + static_cast<size_t>(row) * sstride;
  const int e0 = chunk * kCollectChunk;
  // this chunk's keys (one 16-byte load per thread, clamped into the row) go out first, before
  // the row's position and entry count are known; also to LDS for the histogram pass, which is
  // cleared while the loads are in flight
  float f[4];
  Scores<ST>::four(srow, min(e0 + tid * PER, sstride - 4), f);
  asm volatile("" ::: "memory");
  const int n_vis = visible(n_entries, pos, row, nq, m, n_max);
  const int kk = min(k, n_vis);
  if (n_vis <= k) return;  // everything is selected; finalize does not read the regions
  const int used = (n_vis + kCollectChunk - 1) / kCollectChunk;  // chunks holding visible keys
  if (chunk >= used) return;
  const size_t rc = static_cast<size_t>(row) * nchunks + chunk;
  const int len = min(kCollectChunk, n_vis - e0);
  uint32_t key[PER];
  {
    const int base = e0 + tid * PER;
    asm volatile("" : "+v"(f[0]), "+v"(f[1]), "+v"(f[2]), "+v"(f[3]) : : "memory");  // one load
#pragma unroll
    for (int j = 0; j < 4; ++j) key[j] = base + j < n_vis ? order_key(f[j]) : 0u;
  }
  for (int i = tid; i < kHistBins; i += THREADS) hist[i] = 0u;
#pragma unroll
  for (int j = 0; j < PER; ++j) s_key[tid * PER + j] = key[j];
  __syncthreads();
  collect_candidates<THREADS, PER>(key, s_key, e0, len, n_vis, kk, hist, s_tmp, s_res,
                                   cand + rc * kCandPerChunk, ccount + 2 * rc);
}

template <typename ST>
__global__ __launch_bounds__(1024) void topk_finalize_kernel(
    const ST* __restrict__ scores, int sstride, const int32_t* __restrict__ n_entries,
    const int32_t* __restrict__ pos, int nq, int m, int k, int n_max, int nchunks,
    const uint32_t* __restrict__ ccount, const uint64_t* __restrict__ cand,
    int32_t* __restrict__ idx_out, float* __restrict__ score_out, int cchunk) {
  constexpr int THREADS = 1024;
  extern __shared__ __align__(16) unsigned char smem[];
  uint32_t* ckey = reinterpret_cast<uint32_t*>(smem);              // kSCandCap
  int32_t* cidx = reinterpret_cast<int32_t*>(ckey + kSCandCap);    // kSCandCap
  uint32_t* hist = reinterpret_cast<uint32_t*>(cidx + kSCandCap);  // kHistBins
  __shared__ uint32_t s_off[1025];
  __shared__ uint32_t s_tmp[THREADS / 64];
  __shared__ int s_res[2];
  __shared__ int s_flag;
  __shared__ uint32_t s_lo, s_hi, s_tmax;
  __shared__ int s_rchunk[kRepairChunks];       // chunks re-read for keys >= T
  __shared__ uint32_t s_rcount[kRepairChunks];  // their counts of such keys
  asm volatile("" ::"s"(scores), "s"(sstride), "s"(n_entries), "s"(pos), "s"(nq), "s"(m), "s"(k),
               "s"(n_max), "s"(nchunks), "s"(ccount), "s"(cand), "s"(idx_out),
               "s"(score_out), "s"(cchunk));  // all parameters at once
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  // this thread's chunk (count, threshold) goes out first, before the row's position and entry
  // count are known (it is used only for chunks that hold visible keys)
  uint32_t cc_raw = 0u, ct_raw = 0u;
  {
    const size_t rc = static_cast<size_t>(row) * nchunks + min(tid, nchunks - 1);
    cc_raw = ccount[2 * rc];
    ct_raw = ccount[2 * rc + 1];
  }
  asm volatile("" ::: "memory");
  const int n_vis = visible(n_entries, pos, row, nq, m, n_max);
  const int kk = min(k, n_vis);
  int32_t* out = idx_out + static_cast<size_t>(row) * k;
  float* sout = score_out ? score_out + static_cast<size_t>(row) * k : nullptr;
  const ST* srow = scores + static_cast<size_t>(row) * sstride;
  if (n_vis <= k) {  // everything is selected
    for (int j = tid; j < k; j += THREADS) {
      out[j] = j < n_vis ? j : -1;
      if (sout) sout[j] = j < n_vis ? Scores<ST>::at(srow, j) : -INFINITY;
    }
    return;
  }
  const int used = (n_vis + cchunk - 1) / cchunk;  // <= nchunks
  if (tid == 0) {
    s_flag = used > THREADS ? 1 : 0;  // 1 = take the exact fallback
    s_lo = 0xffffffffu;
    s_hi = 0u;
    s_tmax = 0u;
  }
  __syncthreads();
  if (!s_flag) {
    const uint32_t c = tid < used ? cc_raw : 0u;
    const uint32_t tc = wave_max_u32(tid < used ? ct_raw : 0u);
    if (lane_id() == 0) atomicMax(&s_tmax, tc);
    if (c > static_cast<uint32_t>(kCandPerChunk)) s_flag = 1;
    uint32_t tot;
    const uint32_t o = block_excl_scan<THREADS>(c, s_tmp, &tot);
    if (tid < used) s_off[tid] = o;
    if (tid == 0) {
      s_off[used] = tot;
      if (tot > static_cast<uint32_t>(kSCandCap) || tot < static_cast<uint32_t>(kk)) s_flag = 1;
    }
    __syncthreads();
  }
  if (s_flag) {
    uint32_t T;
    int need_eq;
    auto kf = [&](int e) { return order_key(Scores<ST>::at(srow, e)); };
    radix_select<THREADS>(kf, n_vis, kk, hist, s_tmp, s_res, T, need_eq);
    ordered_emit<THREADS>(kf, n_vis, T, need_eq, kk, k, srow, out, sout, s_tmp);
    return;
  }
  const int nc = static_cast<int>(s_off[used]);
  uint32_t lo = 0xffffffffu, hi = 0u;
  // tpr threads per region (16; 8 for chunks of up to 2048 entries, whose regions hold about
  // half as many pairs and are twice as many), each region's pairs to its place in the
  // concatenated list; a thread's first eight pairs are requested together (one round trip for
  // regions up to 8 tpr pairs)
  const int tpr = cchunk <= 2048 ? 8 : 16;
  const int tsh = cchunk <= 2048 ? 3 : 4;
  auto copy_region = [&](int c) {
    const uint32_t o = s_off[c], n = s_off[c + 1] - o;
    const uint64_t* src = cand + (static_cast<size_t>(row) * nchunks + c) * kCandPerChunk;
    const uint32_t j0 = tid & (tpr - 1), last = n > 0 ? n - 1 : 0;
    uint64_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = src[min(j0 + tpr * u, last)];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint32_t j = j0 + tpr * u;
      if (j < n) {
        const uint32_t kv = static_cast<uint32_t>(v[u] >> 32);
        ckey[o + j] = kv;
        cidx[o + j] = static_cast<int32_t>(v[u] & 0xffffffffu);
        lo = min(lo, kv);
        hi = max(hi, kv);
      }
    }
    for (uint32_t j = j0 + 8 * tpr; j < n; j += tpr) {
      const uint64_t w = src[j];
      const uint32_t kv = static_cast<uint32_t>(w >> 32);
      ckey[o + j] = kv;
      cidx[o + j] = static_cast<int32_t>(w & 0xffffffffu);
      lo = min(lo, kv);
      hi = max(hi, kv);
    }
  };
  for (int c = tid >> tsh; c < used; c += THREADS >> tsh) copy_region(c);
  lo = wave_min_u32(lo);
  hi = wave_max_u32(hi);
  if (lane_id() == 0) {
    atomicMin(&s_lo, lo);
    atomicMax(&s_hi, hi);
  }
  __syncthreads();
  uint32_t T;
  int need_eq;
  auto ck = [&](int j) { return ckey[j]; };
  select_kth<THREADS>(ck, nc, kk, s_lo, s_hi, hist, s_tmp, s_res, T, need_eq);
  int n_list = nc;
  if (T < s_tmax) {
    // Some chunk's threshold cut keys that reach T (a chunk holding far more than its share of
    // the row's top keys, e.g. the newest entries of a prompt).  Those chunks (T_c > T) are
    // read again for every key >= T, the others keep their regions (all keys >= T_c, T_c <=
    // T), and the list is rebuilt in index order: it then holds every key >= T of the row, so
    // its kk-th key T' >= T is the row's and every key >= T' is in it.  Up to kRepairChunks
    // chunks are re-read; more, or a list over kSCandCap, take the exact streaming select.
    const uint32_t Tr = T;
    const bool aff = tid < used && ct_raw > Tr;
    uint32_t n_aff;
    const uint32_t ai = block_excl_scan<THREADS>(aff ? 1u : 0u, s_tmp, &n_aff);
    if (aff && ai < static_cast<uint32_t>(kRepairChunks)) s_rchunk[ai] = tid;
    __syncthreads();
    bool ok = n_aff <= static_cast<uint32_t>(kRepairChunks);
    // a re-read chunk of cchunk <= 4096 entries takes the first cchunk / 4 threads
    const bool in_chunk = tid * 4 < cchunk;
    if (ok) {
      // keys >= Tr of each re-read chunk, counted (4 keys a thread, one 16-byte load)
      for (uint32_t a = 0; a < n_aff; ++a) {
        const int e = s_rchunk[a] * cchunk + tid * 4;
        float f[4];
        Scores<ST>::four(srow, min(e, sstride - 4), f);
        uint32_t c = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          c += (in_chunk && e + j < n_vis && order_key(f[j]) >= Tr) ? 1u : 0u;
        uint32_t tot;
        block_excl_scan<THREADS>(c, s_tmp, &tot);
        if (tid == 0) s_rcount[a] = tot;
      }
      __syncthreads();
      const uint32_t cnew = tid < used ? (aff ? s_rcount[ai] : cc_raw) : 0u;
      uint32_t tot;
      const uint32_t o = block_excl_scan<THREADS>(cnew, s_tmp, &tot);
      if (tid < used) s_off[tid] = o;
      if (tid == 0) {
        s_off[used] = tot;
        s_lo = 0xffffffffu;
        s_hi = 0u;
      }
      ok = tot <= static_cast<uint32_t>(kSCandCap);
      n_list = static_cast<int>(tot);
      __syncthreads();
    }
    if (!ok) {  // exact streaming select over the row
      auto kf = [&](int e) { return order_key(Scores<ST>::at(srow, e)); };
      radix_select<THREADS>(kf, n_vis, kk, hist, s_tmp, s_res, T, need_eq);
      ordered_emit<THREADS>(kf, n_vis, T, need_eq, kk, k, srow, out, sout, s_tmp);
      return;
    }
    // regions of the chunks that keep them, 16 threads each
    lo = 0xffffffffu;
    hi = 0u;
    for (int c = tid >> tsh; c < used; c += THREADS >> tsh)
      if (ccount[2 * (static_cast<size_t>(row) * nchunks + c) + 1] <= Tr) copy_region(c);
    uint32_t lo2 = lo, hi2 = hi;
    // the re-read chunks' keys >= Tr, in index order
    for (uint32_t a = 0; a < n_aff; ++a) {
      const int c = s_rchunk[a];
      const int e = c * cchunk + tid * 4;
      float f[4];
      Scores<ST>::four(srow, min(e, sstride - 4), f);
      uint32_t kv[4], cnt = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        kv[j] = (in_chunk && e + j < n_vis) ? order_key(f[j]) : 0u;
        cnt += kv[j] >= Tr && kv[j] != 0u ? 1u : 0u;
      }
      uint32_t tot;
      uint32_t o = s_off[c] + block_excl_scan<THREADS>(cnt, s_tmp, &tot);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (kv[j] >= Tr && kv[j] != 0u) {
          ckey[o] = kv[j];
          cidx[o] = e + j;
          lo2 = min(lo2, kv[j]);
          hi2 = max(hi2, kv[j]);
          ++o;
        }
      }
    }
    lo2 = wave_min_u32(lo2);
    hi2 = wave_max_u32(hi2);
    if (lane_id() == 0) {
      atomicMin(&s_lo, lo2);
      atomicMax(&s_hi, hi2);
    }
    __syncthreads();
    select_kth<THREADS>(ck, n_list, kk, s_lo, s_hi, hist, s_tmp, s_res, T, need_eq);
  }
  // the candidate list is in ascending index order
  ordered_emit_fn<THREADS>(ck, n_list, T, need_eq, k, [&](int slot, int j) {
    out[slot] = cidx[j];
    if (sout) sout[slot] = Scores<ST>::at(srow, cidx[j]);
  });
  for (int j = kk + tid; j < k; j += THREADS) {
    out[j] = -1;
    if (sout) sout[j] = -INFINITY;
  }
}

// ============================================================================ launchers
static size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// Rows longer than the 1024-thread sampled select holds (and not too many of them) use the
// multi-workgroup select (measured slower than the one-workgroup select at 32K entries).
bool index_use_multi(int rows, int n_max) {
  return n_max > kRowTopkBigN && rows <= kMultiMaxRows;
}

// Chunks a row is cut into for the multi-workgroup select: the decode scorer's own chunks when
// it collects the candidates, kCollectChunk otherwise; 0 when the row selection runs instead.
static int chunk_entries(int rows, int nq, int n_max, int d_I, int H_I) {
  if (index_fused_collect(nq, d_I, H_I, rows, n_max)) return index_score_chunk();
  return index_use_multi(rows, n_max) ? kCollectChunk : 0;
}

size_t index_topk_workspace(int rows, int nq, int n_max, int d_I, int H_I, bool score_bf16) {
  const size_t sb = score_bf16 ? 2 : 4;
  size_t b = align256(static_cast<size_t>(rows) * score_stride(n_max) * sb);
  if (const int ch = chunk_entries(rows, nq, n_max, d_I, H_I)) {
    const size_t rc = static_cast<size_t>(rows) * ((n_max + ch - 1) / ch);
    b += align256(rc * 8);  // (count, threshold) per chunk
    b += align256(rc * kCandPerChunk * 8);
  }
  return b;
}

void index_topk_layout(IndexArgs& a, void* ws, int rows) {
  unsigned char* p = static_cast<unsigned char*>(ws);
  a.sstride = score_stride(a.n_max);
  a.scores = p;
  p += align256(static_cast<size_t>(rows) * a.sstride * (a.score_bf16 ? 2 : 4));
  a.counters = nullptr;
  a.cand = nullptr;
  if (const int ch = chunk_entries(rows, a.nq, a.n_max, a.d_I, a.H_I)) {
    const size_t rc = static_cast<size_t>(rows) * ((a.n_max + ch - 1) / ch);
    a.counters = reinterpret_cast<uint32_t*>(p);
    p += align256(rc * 8);
    a.cand = reinterpret_cast<uint64_t*>(p);
  }
}

template <int THREADS, int CAP, typename ST>
static hipError_t launch_row_topk(const IndexArgs& a, int rows, hipStream_t s) {
  const size_t lds = (static_cast<size_t>(CAP) + kHistBins) * 4;
  if (hipError_t e =
          ensure_max_lds(reinterpret_cast<const void*>(topk_row_kernel<THREADS, CAP, ST>), lds))
    return e;
  ProfScope ps("topk_row", s);
  topk_row_kernel<THREADS, CAP, ST><<<rows, THREADS, lds, s>>>(
      static_cast<const ST*>(a.scores), a.sstride, a.n_entries, a.pos, a.nq, a.m, a.k, a.n_max,
      a.idx_out, a.score_out);
  return hipGetLastError();
}

template <typename ST>
static hipError_t launch_index_topk_t(const IndexArgs& a, hipStream_t s) {
  const int rows = a.B * a.nq;
  const bool fused = index_fused_collect(a.nq, a.d_I, a.H_I, rows, a.n_max);
  const bool multi = fused || index_use_multi(rows, a.n_max);
  hipError_t e = fused ? launch_index_scores_collect(a, s) : launch_index_scores(a, s);
  if (e != hipSuccess) return e;
  const ST* sc = static_cast<const ST*>(a.scores);
  if (!multi) {
    if (a.n_max <= 4096) return launch_row_topk<256, kRowTopkMaxN, ST>(a, rows, s);
    // runs of query rows (causal lengths) read only their visible scores
    const bool clamp = a.nq >= 16;
    if (a.n_max <= 16384) {
      ProfScope ps("topk_sample", s);
      // 512 threads x 32 keys (measured 1.83 ms against 2.89 ms for 256 x 64 and 3.68 ms for
      // 1024 x 32 on the 64K-token prefill rows)
      if (clamp)
        topk_sample_kernel<512, 32, ST, true><<<rows, 512, 0, s>>>(
            sc, a.sstride, a.n_entries, a.pos, a.nq, a.m, a.k, a.n_max, a.idx_out, a.score_out);
      else
        topk_sample_kernel<512, 32, ST><<<rows, 512, 0, s>>>(
            sc, a.sstride, a.n_entries, a.pos, a.nq, a.m, a.k, a.n_max, a.idx_out, a.score_out);
      return hipGetLastError();
    }
    ProfScope ps("topk_sample", s);
    if (clamp)
      topk_sample_kernel<1024, 32, ST, true><<<rows, 1024, 0, s>>>(
          sc, a.sstride, a.n_entries, a.pos, a.nq, a.m, a.k, a.n_max, a.idx_out, a.score_out);
    else
      topk_sample_kernel<1024, 32, ST><<<rows, 1024, 0, s>>>(
          sc, a.sstride, a.n_entries, a.pos, a.nq, a.m, a.k, a.n_max, a.idx_out, a.score_out);
    return hipGetLastError();
  }
  const int cch = fused ? index_score_chunk() : kCollectChunk;
  const int ncc = (a.n_max + cch - 1) / cch;
  if (!fused) {
    ProfScope ps("topk_collect", s);
    topk_collect_kernel<ST><<<static_cast<unsigned>(ncc) * rows, 1024, 0, s>>>(
        sc, a.sstride, a.n_entries, a.pos, a.nq, a.m, a.k, a.n_max, ncc, a.counters, a.cand);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if ((e = ensure_max_lds(reinterpret_cast<const void*>(topk_finalize_kernel<ST>), kMultiLds)))
    return e;
  ProfScope ps("topk_finalize", s);
  topk_finalize_kernel<ST><<<rows, 1024, kMultiLds, s>>>(sc, a.sstride, a.n_entries, a.pos,
                                                         a.nq, a.m, a.k, a.n_max, ncc,
                                                         a.counters, a.cand, a.idx_out,
                                                         a.score_out, cch);
  return hipGetLastError();
}

hipError_t launch_index_topk(const IndexArgs& a, hipStream_t s) {
  return a.score_bf16 ? launch_index_topk_t<uint16_t>(a, s) : launch_index_topk_t<float>(a, s);
}

}  // namespace csa
