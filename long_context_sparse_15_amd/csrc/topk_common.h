// Block-wide pieces of the top-k selection shared by the selection kernels (topk.hip) and the
// decode scorer (index.hip), which collects the candidates of its own chunk of a row.
#pragma once

#include "index_common.h"

namespace csa {

// Block-wide search over a histogram of `nbins` counts for the bin d with
//   sum(bins > d) < remaining <= sum(bins >= d).
// Writes d to s_res[0] and remaining - sum(bins > d) to s_res[1].  All THREADS threads call it.
template <int THREADS>
__device__ void block_find_crossing(const uint32_t* bins, int nbins, uint32_t remaining,
                                    uint32_t* s_tmp, int* s_res) {
  constexpr int NWAVE = THREADS / 64;
  const int tid = threadIdx.x, l = lane_id(), wave = tid >> 6;
  const int per = nbins / THREADS;  // nbins is a multiple of THREADS
  uint32_t own = 0;
  for (int j = 0; j < per; ++j) own += bins[tid * per + j];
  // inclusive suffix sum inside the wave (lane l: sum over lanes >= l) from the prefix sum
  const uint32_t inc = wave_incl_scan(own);
  const uint32_t wtot = __builtin_amdgcn_readlane(inc, 63);
  const uint32_t suf = wtot - inc + own;
  if (l == 0) s_tmp[wave] = wtot;
  __syncthreads();
  uint32_t later = 0;  // (a loop of constant length: its reads go out together)
#pragma unroll
  for (int w2 = 1; w2 < NWAVE; ++w2)
    if (w2 > wave) later += s_tmp[w2];
  const uint32_t above = suf - own + later;
  if (above < remaining && remaining <= above + own) {
    uint32_t cum = above;
    for (int j = per - 1; j >= 0; --j) {
      const uint32_t c = bins[tid * per + j];
      if (cum + c >= remaining) {
        s_res[0] = tid * per + j;
        s_res[1] = static_cast<int>(remaining - cum);
        break;
      }
      cum += c;
    }
  }
  __syncthreads();
}

// Exclusive block scan of one uint32 per thread; returns the thread's prefix, *total the sum.
template <int THREADS>
__device__ uint32_t block_excl_scan(uint32_t v, uint32_t* s_tmp, uint32_t* total) {
  constexpr int NWAVE = THREADS / 64;
  const int tid = threadIdx.x, l = lane_id(), wave = tid >> 6;
  const uint32_t inc = wave_incl_scan(v);
  if (l == 63) s_tmp[wave] = inc;
  __syncthreads();
  uint32_t before = 0, tot = 0;
  for (int w2 = 0; w2 < NWAVE; ++w2) {
    const uint32_t x = s_tmp[w2];
    if (w2 < wave) before += x;
    tot += x;
  }
  __syncthreads();
  *total = tot;
  return before + inc - v;
}

// One histogram pass of radix select: counts keys matching (prefix, mask) into nb bins of the
// bits at `shift`, then finds the crossing bin of `remaining` (s_res[0], s_res[1]); returns the
// crossing bin's count.
template <int THREADS, typename KeyFn>
__device__ uint32_t radix_pass(KeyFn key, int n, uint32_t prefix, uint32_t mask, int shift,
                               int nb, uint32_t remaining, uint32_t* hist, uint32_t* s_tmp,
                               int* s_res, bool zeroed = false) {
  const int tid = threadIdx.x;
  if (!zeroed) {  // a caller that cleared hist before its last barrier skips this
    for (int i = tid; i < nb; i += THREADS) hist[i] = 0;
    __syncthreads();
  }
  for (int e = tid; e < n; e += THREADS) {
    const uint32_t kv = key(e);
    if ((kv & mask) == prefix) atomicAdd(&hist[(kv >> shift) & (nb - 1)], 1u);
  }
  __syncthreads();
  block_find_crossing<THREADS>(hist, nb, remaining, s_tmp, s_res);
  return hist[s_res[0]];
}

// Candidates of one chunk of a row for the multi-workgroup select.  The chunk's threshold T_c
// is the lower edge of the 12-bit bin (refined by 12 more bits when crowded) holding its r-th
// largest key, r = the chunk's expected share of the row's top kk plus four standard
// deviations and 4; the chunk's (key, index) pairs >= T_c go to its region in ascending index
// order (block prefix sum, no global atomics), then its count and T_c.  Thread tid holds the
// keys of entries e0 + tid*PER .. +PER-1 (0 past the row's visible length n_vis); s_key holds
// the chunk's len keys for the histogram passes; hist must be zeroed, and a barrier passed
// since s_key and hist were written.  All THREADS threads call it.
template <int THREADS, int PER>
__device__ void collect_candidates(const uint32_t (&key)[PER], const uint32_t* s_key, int e0,
                                   int len, int n_vis, int kk, uint32_t* hist, uint32_t* s_tmp,
                                   int* s_res, uint64_t* cdst, uint32_t* cc) {
  const int tid = threadIdx.x;
  const float expect = static_cast<float>(kk) * static_cast<float>(len) / static_cast<float>(n_vis);
  const int r = static_cast<int>(ceilf(expect + 4.f * sqrtf(expect) + 4.f));
  uint32_t Tc = 0u;  // keep the whole chunk when it holds no more than r keys
  if (r < len) {
    auto kf = [&](int e) { return s_key[e]; };
    const uint32_t cb = radix_pass<THREADS>(kf, len, 0u, 0u, 20, 4096, static_cast<uint32_t>(r),
                                            hist, s_tmp, s_res, /*zeroed=*/true);
    const uint32_t d1 = static_cast<uint32_t>(s_res[0]);
    const uint32_t r1 = static_cast<uint32_t>(s_res[1]);
    __syncthreads();
    Tc = d1 << 20;
    if (cb > 64) {  // crowded bin: refine by the next 12 bits
      radix_pass<THREADS>(kf, len, d1 << 20, 0xfff00000u, 8, 4096, r1, hist, s_tmp, s_res);
      Tc |= static_cast<uint32_t>(s_res[0]) << 8;
      __syncthreads();
    }
  }
  uint32_t own = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) own += (e0 + tid * PER + i < n_vis && key[i] >= Tc) ? 1u : 0u;
  uint32_t total;
  uint32_t off = block_excl_scan<THREADS>(own, s_tmp, &total);
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = e0 + tid * PER + i;
    if (e < n_vis && key[i] >= Tc) {
      if (off < static_cast<uint32_t>(kCandPerChunk))
        cdst[off] = (static_cast<uint64_t>(key[i]) << 32) | static_cast<uint32_t>(e);
      ++off;
    }
  }
  if (tid == 0) {
    cc[0] = total;
    cc[1] = Tc;
  }
}

}  // namespace csa
