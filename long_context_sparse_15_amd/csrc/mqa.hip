// Shared-KV multi-query attention over compressed entries + sliding window + sink (gfx950).
//
// Method: "DeepSeek V4 模型技术大全", chapter "Attention": component table (shared K=V MQA with
// one KV head; attention sink p = exp(z) / (exp(a_h) + sum exp(z)); window W_t of the last
// n_win tokens) and section "注意力实现细节" (partial RoPE on the last dims of q and keys, the
// core-attention output rotated back).  CSA attends the top-k selected entries, HCA every closed
// entry j < floor((t+1)/m') ("HCA 的完整路径"); both add the window rows and share one softmax.
//
// Layout of the work: a workgroup owns one query row, 16*NW heads (16 per wave) and a span of
// the query's key list (selected or visible entries, then window tokens).  Key rows are staged
// through LDS 32 at a time and shared by all waves.  Per wave and 32-row tile:
//   S^T[32 rows x 16 heads] = E . Q^T        (A = entry rows from LDS, B = query in registers)
//   online softmax per head in the log2 domain (rows spread over the 4 lane groups)
//   O^T[C dims x 16 heads] += E^T . P^T      (A = entry columns from LDS, B = P^T straight from
//                                             the S^T accumulator layout, no LDS round trip)
// With several spans per query each workgroup writes (max, sum, unnormalised O) and a combine
// kernel merges them in a fixed order, adds the sink and normalises; with one span the same
// epilogue runs in place.  Spans are fixed by the plan, not by timing, so results are
// run-to-run deterministic.
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
  float scale_log2;
  int split_rows, n_splits, head_groups, n_work;
  float* part;  // [rows, n_splits, n_heads, C + 4]: C unnormalised sums, (max, sum), pad
  uint16_t* out;
  float* lse_out;
};

template <int C>
struct Tile {
  static constexpr int kRows = 32;
  static constexpr int kStride = C + 8;  // bf16 elements per LDS row (16-byte pad)
  static constexpr int kElems = kRows * kStride;
};

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
  v.x = pack_bf16x2(o[0], o[1]);
  v.y = pack_bf16x2(o[2], o[3]);
  *reinterpret_cast<uint2*>(dst) = v;
}

// One workgroup: one query row, HT head tiles of 16 heads, DS dim slices per head tile
// (NW = HT*DS waves).  Wave (h, s) owns heads h*16..h*16+15 and dims s*C/DS..(s+1)*C/DS-1:
// it computes the partial logits of its dim slice, the DS partials of a head tile are summed
// through LDS (every slice then runs the identical softmax), and it accumulates the output
// of its own dims only.  Rows are staged through a single LDS tile of 32 rows whose global
// loads for the next tile are in flight (in registers) while the current tile is computed.
template <int C, int HT, int DS>
__global__ __launch_bounds__(64 * HT * DS) void mqa_kernel(MqaParams p) {
  using TL = Tile<C>;
  constexpr int NW = HT * DS;
  constexpr int NT = 64 * NW;
  constexpr int CH = C / 8;                             // 16-byte chunks per row
  constexpr int LOADS = (TL::kRows * CH + NT - 1) / NT;
  constexpr int CS = C / DS;                            // dims per slice
  constexpr int KSL = CS / 32;                          // MFMA K steps of a slice
  constexpr int DTL = CS / 16;                          // output dim tiles of a slice
  extern __shared__ __align__(16) unsigned char smem[];
  uint16_t* E = reinterpret_cast<uint16_t*>(smem);                          // [32][C+8]
  float* SX = reinterpret_cast<float*>(smem + TL::kElems * sizeof(uint16_t));  // [NW][8][64]
  int* s_idx = reinterpret_cast<int*>(SX + NW * 8 * 64);                     // [split_rows]
  __shared__ long s_off[3][TL::kRows];
  __shared__ int s_valid[3][TL::kRows];

  const int tid = threadIdx.x;
  const int l = lane_id(), g = l >> 4, c16 = l & 15, wave = tid >> 6;
  const int hsub = wave % HT, slice = wave / HT;
  // Work item w = (row, split); head groups of one work item are blocks 8 apart (same XCD).
  const int bid = blockIdx.x;
  const int w = (bid / (8 * p.head_groups)) * 8 + (bid & 7);
  const int hg = (bid >> 3) % p.head_groups;
  if (w >= p.n_work) return;
  const int split = w % p.n_splits;
  const int row = w / p.n_splits;
  const int b = row / p.nq;
  const int t = p.pos ? p.pos[row] : (row % p.nq);
  const int n_ent = max(0, min(p.n_entries[b], p.n_max));
  const int n_w = min(p.n_win, t + 1);
  const int wlo = t - n_w + 1;
  int n_sel;
  if (p.idx) {
    n_sel = p.k;
  } else {
    const long v = (static_cast<long>(t) + 1) / p.m;
    n_sel = static_cast<int>(v < n_ent ? v : n_ent);
  }
  const int R = n_sel + n_w;
  const int j0 = split * p.split_rows;
  const int j1 = min(R, j0 + p.split_rows);
  const int head = (hg * HT + hsub) * 16 + c16;
  const bool head_ok = head < p.n_heads;
  const int dbase = slice * CS;

  // the span's selected entry indices go to LDS first, so that the tile loop issues no global
  // load other than the row gathers (whose completion the compiler then tracks exactly)
  if (p.idx) {
    const int e1 = min(j1, n_sel);
    for (int j = j0 + tid; j < e1; j += NT) s_idx[j - j0] = p.idx[static_cast<size_t>(row) * p.k + j];
  }

  // ---- query fragments of this slice (B operand of S^T), rotated at t on the RoPE dims
  bf16x8 bq[KSL];
  {
    const uint16_t* qrow = p.q + (static_cast<size_t>(row) * p.n_heads + (head_ok ? head : 0)) * C;
#pragma unroll
    for (int kk = 0; kk < KSL; ++kk) {
      const int d0 = dbase + kk * 32 + g * 8;
      u32x4 raw = head_ok ? *reinterpret_cast<const u32x4*>(qrow + d0) : u32x4{0, 0, 0, 0};
      if (d0 + 8 > C - p.r) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int d = d0 + 2 * j;
          if (d >= C - p.r) {
            float cs, sn;
            rope_cos_sin(t, p.inv_freq[(d - (C - p.r)) >> 1], cs, sn);
            const float x0 = bf16_to_f32(static_cast<uint16_t>(raw[j] & 0xffff));
            const float x1 = bf16_to_f32(static_cast<uint16_t>(raw[j] >> 16));
            raw[j] = pack_bf16x2(x0 * cs - x1 * sn, x0 * sn + x1 * cs);
          }
        }
      }
      bq[kk] = as_bf16x8(raw);
    }
  }

  f32x4 acc[DTL];
#pragma unroll
  for (int dt = 0; dt < DTL; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // m_ref: the reference maximum the probabilities are taken against (log2 domain); it moves
  // only when a logit exceeds it by more than 8, so the accumulators are rarely rescaled and
  // every probability stays below 2^8.
  float m_ref = -INFINITY, l_run = 0.f;

  auto resolve = [&](int slot, int jt) {  // row offsets of the tile starting at list row jt
    if (tid < TL::kRows) {
      const int j = jt + tid;
      long off = static_cast<long>(b) * p.n_max * C;  // safe in-bounds row for masked slots
      int ok = 0;
      if (j < j1) {
        if (j < n_sel) {
          const int e = p.idx ? s_idx[j - j0] : j;
          ok = (e >= 0 && e < n_ent) ? 1 : 0;
          off = (static_cast<long>(b) * p.n_max + (ok ? e : 0)) * C;
        } else {
          const int u = wlo + (j - n_sel);
          ok = 1;
          off = -1 - (static_cast<long>(b) * p.win_slots + (u % p.win_slots)) * C;  // window
        }
      }
      s_off[slot][tid] = off;
      s_valid[slot][tid] = ok;
    }
  };
  // two register stages: while tile `it` is computed, tiles it+1 and it+2 are in flight
  u32x4 stage0[LOADS], stage1[LOADS];
  // Every lane always issues its loads (an invalid row reads a valid row of the cache and is
  // zeroed when stored to LDS), so the instruction stream does not branch and the compiler waits
  // for exactly the stage being stored while the other stage stays in flight.
  static_assert(LOADS * NT == TL::kRows * CH, "tile chunks must split evenly over the threads");
  auto gload = [&](int slot, u32x4 (&st)[LOADS]) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int ch = tid + i * NT;
      const int rr = ch / CH, cc = ch % CH;
      const long off = s_off[slot][rr];
      const uint16_t* src = off >= 0 ? p.entries + off : p.window + (-1 - off);
      st[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src) + cc);
    }
  };
  auto sstore = [&](int slot, const u32x4 (&st)[LOADS]) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int ch = tid + i * NT;
      const int rr = ch / CH, cc = ch % CH;
      const u32x4 v = s_valid[slot][rr] ? st[i] : u32x4{0, 0, 0, 0};
      *reinterpret_cast<u32x4*>(E + rr * TL::kStride + cc * 8) = v;
    }
  };

  const int ntiles = j1 > j0 ? (j1 - j0 + TL::kRows - 1) / TL::kRows : 0;
  __syncthreads();  // s_idx
  if (ntiles > 0) {
    resolve(0, j0);
    if (ntiles > 1) resolve(1, j0 + TL::kRows);
    __syncthreads();
    gload(0, stage0);
    if (ntiles > 1) gload(1, stage1);
  }
  const int i0 = c16 >> 2, q4 = c16 & 3;
  auto tile_step = [&](int it, u32x4 (&st)[LOADS]) {
    const int slot = it % 3;
    __syncthreads();  // every wave is done with the previous tile (E and SX)
    sstore(slot, st);  // waits for this tile's loads only; the next tile's stay in flight
    if (it + 2 < ntiles) resolve((it + 2) % 3, j0 + (it + 2) * TL::kRows);
    __syncthreads();  // tile `it` is in LDS; offsets of tile it+2 are known
    if (it + 2 < ntiles) gload((it + 2) % 3, st);
    // partial S^T of this slice: rows rt*16 + c16 (A from LDS) x heads (B in registers)
    f32x4 sacc[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      sacc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
      const uint16_t* er = E + (rt * 16 + c16) * TL::kStride + dbase + g * 8;
#pragma unroll
      for (int kk = 0; kk < KSL; ++kk) {
        const bf16x8 a = as_bf16x8(*reinterpret_cast<const u32x4*>(er + kk * 32));
        sacc[rt] = mfma_bf16_16x16x32(a, bq[kk], sacc[rt]);
      }
    }
    if constexpr (DS > 1) {  // sum the DS slice partials of this head tile
      float* mine = SX + (wave * 8) * 64 + l;
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) mine[(rt * 4 + i) * 64] = sacc[rt][i];
      __syncthreads();
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v = 0.f;
#pragma unroll
          for (int s2 = 0; s2 < DS; ++s2) v += SX[((s2 * HT + hsub) * 8 + rt * 4 + i) * 64 + l];
          sacc[rt][i] = v;
        }
    }
    // online softmax (log2 domain); lane holds rows rt*16 + 4g + i for head c16
    float s[2][4];
    float tmax = -INFINITY;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rr = rt * 16 + g * 4 + i;
        const bool ok = s_valid[slot][rr] && (j0 + it * TL::kRows + rr < j1);
        s[rt][i] = ok ? sacc[rt][i] * p.scale_log2 : -INFINITY;
        tmax = fmaxf(tmax, s[rt][i]);
      }
    tmax = wave_max_xor(tmax, 48);
    const bool move = tmax > m_ref + 8.f;
    if (__ballot(move)) {  // wave-uniform: some head's reference has to move up
      const float m_new = move ? tmax : m_ref;
      const float alpha = (m_new == m_ref) ? 1.f : exp2f(m_ref - m_new);
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < DTL; ++dt) acc[dt] *= alpha;
      m_ref = m_new;
    }
    float pv[2][4];
    float psum = 0.f;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pv[rt][i] = (s[rt][i] == -INFINITY) ? 0.f : exp2f(s[rt][i] - m_ref);
        psum += pv[rt][i];
      }
    l_run += psum;
    u32x4 pr;
    pr[0] = pack_bf16x2(pv[0][0], pv[0][1]);
    pr[1] = pack_bf16x2(pv[0][2], pv[0][3]);
    pr[2] = pack_bf16x2(pv[1][0], pv[1][1]);
    pr[3] = pack_bf16x2(pv[1][2], pv[1][3]);
    const bf16x8 bp = as_bf16x8(pr);
    // O^T += E^T . P^T on this slice's dims.  K slots of lane group g: rows 4g..4g+3 and
    // 16+4g..16+4g+3; the A operand comes from two LDS transpose reads (within each 16-lane
    // group, lane 4*i0+q addresses row base+i0, dims +4q..+4q+3 of a 4x16 block; lane j gets
    // dim j of rows base..base+3).
    const uint16_t* ta = E + (g * 4 + i0) * TL::kStride + dbase + 4 * q4;
    const uint16_t* tb = ta + 16 * TL::kStride;
#pragma unroll
    for (int dt = 0; dt < DTL; ++dt) {
      const bf16x4 lo = lds_read_tr16(ta + dt * 16);
      const bf16x4 hi = lds_read_tr16(tb + dt * 16);
      const bf16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      acc[dt] = mfma_bf16_16x16x32(a, bp, acc[dt]);
    }
  };
  for (int it = 0; it < ntiles; it += 2) {  // unrolled by the two stages (static register indexing)
    tile_step(it, stage0);
    if (it + 1 < ntiles) tile_step(it + 1, stage1);
  }

  const float l_tot = wave_sum_xor(l_run, 48);
  const size_t orow = static_cast<size_t>(row) * p.n_heads + head;
  if (!head_ok) return;
  if (p.n_splits == 1) {
    const float a2 = p.sink ? p.sink[head] * kLog2e : -INFINITY;
    const float M = fmaxf(m_ref, a2);
    const float f = (m_ref == -INFINITY) ? 0.f : exp2f(m_ref - M);
    const float den = l_tot * f + ((a2 == -INFINITY) ? 0.f : exp2f(a2 - M));
    const float inv = den > 0.f ? f / den : 0.f;
    uint16_t* orow_p = p.out + orow * C;
#pragma unroll
    for (int dt = 0; dt < DTL; ++dt) {
      const int d0 = dbase + dt * 16 + g * 4;
      store_out4(orow_p + d0, acc[dt][0] * inv, acc[dt][1] * inv, acc[dt][2] * inv,
                 acc[dt][3] * inv, d0, C, p.r, t, p.inv_freq);
    }
    if (p.lse_out && g == 0 && slice == 0)
      p.lse_out[orow] = l_tot > 0.f ? (m_ref + log2f(l_tot)) * kLn2 : -INFINITY;
  } else {
    float* prow = p.part + ((static_cast<size_t>(row) * p.n_splits + split) * p.n_heads + head) *
                               (C + 4);
#pragma unroll
    for (int dt = 0; dt < DTL; ++dt)
      *reinterpret_cast<f32x4*>(prow + dbase + dt * 16 + g * 4) = acc[dt];
    if (g == 0 && slice == 0) {
      prow[C] = m_ref;
      prow[C + 1] = l_tot;
    }
  }
}

// Merge of the spans of one (query row, head): fixed order over spans, sink added once.
template <int C>
__global__ __launch_bounds__(64) void mqa_combine_kernel(MqaParams p) {
  const int rh = blockIdx.x;  // row * n_heads + head
  const int row = rh / p.n_heads, head = rh % p.n_heads;
  const int t = p.pos ? p.pos[row] : (row % p.nq);
  const int l = threadIdx.x;
  const float* base = p.part + (static_cast<size_t>(row) * p.n_splits * p.n_heads + head) * (C + 4);
  const size_t sstride = static_cast<size_t>(p.n_heads) * (C + 4);
  float M = p.sink ? p.sink[head] * kLog2e : -INFINITY;
  for (int s = 0; s < p.n_splits; ++s) M = fmaxf(M, base[s * sstride + C]);
  float den = (p.sink && M != -INFINITY) ? exp2f(p.sink[head] * kLog2e - M) : 0.f;
  float lsum = 0.f;
  constexpr int PER = C / 64;  // dims per thread (multiple of 4 for C >= 256; C=128 -> 2)
  float o[PER > 0 ? PER : 1];
#pragma unroll
  for (int i = 0; i < PER; ++i) o[i] = 0.f;
  for (int s = 0; s < p.n_splits; ++s) {
    const float ms = base[s * sstride + C];
    if (ms == -INFINITY) continue;
    const float f = exp2f(ms - M);
    lsum += base[s * sstride + C + 1] * f;
#pragma unroll
    for (int i = 0; i < PER; ++i) o[i] += base[s * sstride + l * PER + i] * f;
  }
  den += lsum;
  const float inv = den > 0.f ? 1.f / den : 0.f;
  uint16_t* dst = p.out + (static_cast<size_t>(row) * p.n_heads + head) * C;
  // each thread owns PER consecutive dims starting at l*PER (even, so RoPE pairs stay local)
#pragma unroll
  for (int i = 0; i < PER; i += 2) {
    const int d = l * PER + i;
    float x0 = o[i] * inv, x1 = o[i + 1] * inv;
    if (d >= C - p.r) {
      float cs, sn;
      rope_cos_sin(t, p.inv_freq[(d - (C - p.r)) >> 1], cs, sn);
      const float y0 = x0 * cs + x1 * sn, y1 = -x0 * sn + x1 * cs;
      x0 = y0;
      x1 = y1;
    }
    *reinterpret_cast<uint32_t*>(dst + d) = pack_bf16x2(x0, x1);
  }
  if (p.lse_out && l == 0)
    p.lse_out[rh] = lsum > 0.f ? (M + log2f(lsum)) * kLn2 : -INFINITY;
}

// ---------------------------------------------------------------- planning and launch
// ---------------------------------------------------------------- planning and launch
static int round_up(int x, int a) { return (x + a - 1) / a * a; }

// Shapes: many query rows (prefill) -> 64 heads x 2 slices per workgroup and no spans; few rows
// over long dense lists (HCA decode) -> 64 heads x 2 slices, spans of >= 512 rows; few rows
// over short sparse lists (CSA decode) -> 16 heads x 4 slices per workgroup (the head groups of
// a row share the gathered rows through L2) and spans chosen to fill the chip.
MqaPlan plan_mqa(int rows, int n_heads, int c, int max_list) {
  MqaPlan pl;
  const int tiles = (n_heads + 15) / 16;
  const bool many_rows = rows >= 1024;
  const bool dense_long = max_list > 4096;
  if (many_rows || dense_long) {
    pl.head_tiles = tiles < 4 ? tiles : 4;
    if (pl.head_tiles == 3) pl.head_tiles = 4;
    pl.slices = 2;
  } else {
    pl.head_tiles = 1;
    pl.slices = c >= 256 ? 4 : 2;
  }
  pl.heads_per_wg = 16 * pl.head_tiles;
  pl.head_groups = (n_heads + pl.heads_per_wg - 1) / pl.heads_per_wg;
  const long base = static_cast<long>(rows) * pl.head_groups;
  const long target = dense_long ? 256 : 256;
  const int min_rows = dense_long ? 512 : 128;
  int splits = base >= target ? 1 : static_cast<int>((target + base - 1) / base);
  int sr = round_up((max_list + splits - 1) / splits, 32);
  if (sr < min_rows) sr = round_up(min_rows < max_list ? min_rows : max_list, 32);
  pl.split_rows = sr;
  pl.n_splits = (max_list + sr - 1) / sr;
  if (pl.n_splits < 1) pl.n_splits = 1;
  return pl;
}

size_t mqa_workspace(const MqaPlan& p, int rows, int n_heads, int c) {
  if (p.n_splits <= 1) return 0;
  return static_cast<size_t>(rows) * p.n_splits * n_heads * (c + 4) * sizeof(float);
}

template <int C, int HT, int DS>
static hipError_t launch_t(const MqaParams& prm, int rows, hipStream_t s) {
  const size_t lds = Tile<C>::kElems * sizeof(uint16_t) + HT * DS * 8 * 64 * sizeof(float) +
                     (prm.idx ? static_cast<size_t>(prm.split_rows) * sizeof(int) : 0);
  static size_t attr = 0;
  if (attr < lds) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(mqa_kernel<C, HT, DS>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(lds));
    if (e != hipSuccess) return e;
    attr = lds;
  }
  MqaParams q = prm;
  q.n_work = rows * prm.n_splits;
  const unsigned grid = static_cast<unsigned>((q.n_work + 7) / 8 * 8) * prm.head_groups;
  {
    ProfScope ps(prm.idx ? "mqa_sparse" : "mqa_dense", s);
    mqa_kernel<C, HT, DS><<<grid, 64 * HT * DS, lds, s>>>(q);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || prm.n_splits == 1) return e;
  ProfScope ps("mqa_combine", s);
  mqa_combine_kernel<C><<<static_cast<unsigned>(rows) * prm.n_heads, 64, 0, s>>>(prm);
  return hipGetLastError();
}

template <int C>
static hipError_t launch_c(const MqaParams& prm, const MqaPlan& pl, int rows, hipStream_t s) {
  if (pl.head_tiles == 1 && pl.slices == 4) return launch_t<C, 1, 4>(prm, rows, s);
  if (pl.head_tiles == 1 && pl.slices == 2) return launch_t<C, 1, 2>(prm, rows, s);
  if (pl.head_tiles == 2 && pl.slices == 2) return launch_t<C, 2, 2>(prm, rows, s);
  if (pl.head_tiles == 4 && pl.slices == 2) return launch_t<C, 4, 2>(prm, rows, s);
  return hipErrorInvalidValue;
}

hipError_t launch_mqa(const MqaArgs& a, const MqaPlan& pl, hipStream_t s) {
  MqaParams p;
  p.q = a.q;
  p.entries = a.entries;
  p.window = a.window;
  p.idx = a.idx;
  p.n_entries = a.n_entries;
  p.pos = a.pos;
  p.sink = a.sink;
  p.inv_freq = a.inv_freq;
  p.nq = a.nq;
  p.n_heads = a.n_heads;
  p.r = a.r;
  p.k = a.k;
  p.m = a.m;
  p.n_win = a.n_win;
  p.win_slots = a.win_slots;
  p.n_max = a.n_max;
  p.scale_log2 = a.scale * kLog2e;
  p.split_rows = pl.split_rows;
  p.n_splits = pl.n_splits;
  p.head_groups = pl.head_groups;
  p.part = a.part;
  p.out = a.out;
  p.lse_out = a.lse_out;
  const int rows = a.B * a.nq;
  switch (a.c) {
    case 128: return launch_c<128>(p, pl, rows, s);
    case 256: return launch_c<256>(p, pl, rows, s);
    case 512: return launch_c<512>(p, pl, rows, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace csa
