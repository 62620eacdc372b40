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

template <int C, int NW>
__global__ __launch_bounds__(64 * NW) void mqa_kernel(MqaParams p) {
  using TL = Tile<C>;
  constexpr int NT = 64 * NW;
  constexpr int CH = C / 8;                       // 16-byte chunks per row
  constexpr int LOADS = (TL::kRows * CH + NT - 1) / NT;
  constexpr int KS = C / 32;                      // MFMA K steps over the head dim
  constexpr int DT = C / 16;                      // output dim tiles
  extern __shared__ __align__(16) unsigned char smem[];
  uint16_t* lds = reinterpret_cast<uint16_t*>(smem);   // 2 tiles
  __shared__ long s_off[2][TL::kRows];                 // element offset of each staged row
  __shared__ int s_valid[2][TL::kRows];

  const int tid = threadIdx.x;
  const int l = lane_id(), g = l >> 4, c16 = l & 15, wave = tid >> 6;
  // Work item w = (row, split); its head groups run as blocks 8 apart so that, with blocks
  // dealt round-robin over the 8 XCDs, all groups of one work item share an XCD and its L2.
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
  const int head = hg * 16 * NW + wave * 16 + c16;
  const bool head_ok = head < p.n_heads;

  // ---- query fragments (B operand of S^T), rotated at t on the RoPE dims
  bf16x8 bq[KS];
  {
    const uint16_t* qrow = p.q + (static_cast<size_t>(row) * p.n_heads + (head_ok ? head : 0)) * C;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      const int d0 = kk * 32 + g * 8;
      u32x4 raw = head_ok ? *reinterpret_cast<const u32x4*>(qrow + d0) : u32x4{0, 0, 0, 0};
      if (d0 + 8 > C - p.r) {
        float x[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          x[2 * j] = bf16_to_f32(static_cast<uint16_t>(raw[j] & 0xffff));
          x[2 * j + 1] = bf16_to_f32(static_cast<uint16_t>(raw[j] >> 16));
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int d = d0 + 2 * j;
          if (d >= C - p.r) {
            float cs, sn;
            rope_cos_sin(t, p.inv_freq[(d - (C - p.r)) >> 1], cs, sn);
            const float x0 = x[2 * j], x1 = x[2 * j + 1];
            x[2 * j] = x0 * cs - x1 * sn;
            x[2 * j + 1] = x0 * sn + x1 * cs;
          }
          raw[j] = pack_bf16x2(x[2 * j], x[2 * j + 1]);
        }
      }
      bq[kk] = as_bf16x8(raw);
    }
  }

  f32x4 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  auto resolve = [&](int buf, int jt) {  // row offsets of the tile starting at list row jt
    if (tid < TL::kRows) {
      const int j = jt + tid;
      long off = 0;
      int ok = 0;
      if (j < j1) {
        if (j < n_sel) {
          const int e = p.idx ? p.idx[static_cast<size_t>(row) * p.k + j] : j;
          ok = (e >= 0 && e < n_ent) ? 1 : 0;
          off = (static_cast<long>(b) * p.n_max + (ok ? e : 0)) * C;
        } else {
          const int u = wlo + (j - n_sel);
          ok = 1;
          off = -1 - (static_cast<long>(b) * p.win_slots + (u % p.win_slots)) * C;  // window
        }
      }
      s_off[buf][tid] = off;
      s_valid[buf][tid] = ok;
    }
  };
  u32x4 stage[LOADS];
  auto gload = [&](int buf) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int ch = tid + i * NT;
      stage[i] = u32x4{0, 0, 0, 0};
      if (ch < TL::kRows * CH) {
        const int rr = ch / CH, cc = ch % CH;
        if (s_valid[buf][rr]) {
          const long off = s_off[buf][rr];
          const uint16_t* src = off >= 0 ? p.entries + off : p.window + (-1 - off);
          stage[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src) + cc);
        }
      }
    }
  };
  auto sstore = [&](int buf) {
    uint16_t* dst = lds + buf * TL::kElems;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int ch = tid + i * NT;
      if (ch < TL::kRows * CH) {
        const int rr = ch / CH, cc = ch % CH;
        *reinterpret_cast<u32x4*>(dst + rr * TL::kStride + cc * 8) = stage[i];
      }
    }
  };

  const int ntiles = j1 > j0 ? (j1 - j0 + TL::kRows - 1) / TL::kRows : 0;
  if (ntiles > 0) {
    resolve(0, j0);
    __syncthreads();
    gload(0);
    sstore(0);
    if (ntiles > 1) resolve(1, j0 + TL::kRows);
    __syncthreads();
  }
  for (int it = 0; it < ntiles; ++it) {
    const int buf = it & 1;
    const bool more = it + 1 < ntiles;
    if (more) gload(buf ^ 1);  // global loads of the next tile overlap this tile's math
    const uint16_t* E = lds + buf * TL::kElems;

    // S^T = E . Q^T for the two 16-row halves
    f32x4 sacc[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      sacc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
      const uint16_t* er = E + (rt * 16 + c16) * TL::kStride + g * 8;
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        const bf16x8 a = as_bf16x8(*reinterpret_cast<const u32x4*>(er + kk * 32));
        sacc[rt] = mfma_bf16_16x16x32(a, bq[kk], sacc[rt]);
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
        const bool ok = s_valid[buf][rr] && (j0 + it * TL::kRows + rr < j1);
        s[rt][i] = ok ? sacc[rt][i] * p.scale_log2 : -INFINITY;
        tmax = fmaxf(tmax, s[rt][i]);
      }
    tmax = wave_max_xor(tmax, 48);
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = (m_new == -INFINITY) ? 1.f : exp2f(m_run - m_new);
    float pv[2][4];
    float psum = 0.f;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pv[rt][i] = (s[rt][i] == -INFINITY) ? 0.f : exp2f(s[rt][i] - m_new);
        psum += pv[rt][i];
      }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    if (__ballot(alpha != 1.f)) {  // wave-uniform: skip once the running maxima have settled
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) acc[dt] *= alpha;
    }
    u32x4 pr;
    pr[0] = pack_bf16x2(pv[0][0], pv[0][1]);
    pr[1] = pack_bf16x2(pv[0][2], pv[0][3]);
    pr[2] = pack_bf16x2(pv[1][0], pv[1][1]);
    pr[3] = pack_bf16x2(pv[1][2], pv[1][3]);
    const bf16x8 bp = as_bf16x8(pr);
    // O^T += E^T . P^T.  The K slots of lane group g are rows 4g..4g+3 and 16+4g..16+4g+3 (the
    // S^T accumulator layout); the A operand (dims x rows) comes from two LDS transpose reads:
    // within each 16-lane group, lane 4*i0+q addresses row (base+i0), dims dt*16+4q..+3 of a
    // 4x16 block, and lane j receives dim dt*16+j of rows base..base+3.
    const int i0 = c16 >> 2, q4 = c16 & 3;
    const uint16_t* ta = E + (g * 4 + i0) * TL::kStride + 4 * q4;
    const uint16_t* tb = ta + 16 * TL::kStride;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const bf16x4 lo = lds_read_tr16(ta + dt * 16);
      const bf16x4 hi = lds_read_tr16(tb + dt * 16);
      const bf16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      acc[dt] = mfma_bf16_16x16x32(a, bp, acc[dt]);
    }
    __syncthreads();  // everyone is done with this buffer and with s_valid[buf]
    if (more) {
      sstore(buf ^ 1);
      if (it + 2 < ntiles) resolve(buf, j0 + (it + 2) * TL::kRows);
    }
    __syncthreads();
  }

  const float l_tot = wave_sum_xor(l_run, 48);
  const size_t orow = static_cast<size_t>(row) * p.n_heads + head;
  if (p.n_splits == 1) {
    if (!head_ok) return;
    const float a2 = p.sink ? p.sink[head] * kLog2e : -INFINITY;
    const float M = fmaxf(m_run, a2);
    const float f = (m_run == -INFINITY) ? 0.f : exp2f(m_run - M);
    const float den = l_tot * f + ((a2 == -INFINITY) ? 0.f : exp2f(a2 - M));
    const float inv = den > 0.f ? f / den : 0.f;
    uint16_t* orow_p = p.out + orow * C;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int d0 = dt * 16 + g * 4;
      store_out4(orow_p + d0, acc[dt][0] * inv, acc[dt][1] * inv, acc[dt][2] * inv,
                 acc[dt][3] * inv, d0, C, p.r, t, p.inv_freq);
    }
    if (p.lse_out && g == 0)
      p.lse_out[orow] = l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
  } else {
    if (!head_ok) return;
    float* prow = p.part + ((static_cast<size_t>(row) * p.n_splits + split) * p.n_heads + head) *
                               (C + 4);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      *reinterpret_cast<f32x4*>(prow + dt * 16 + g * 4) = acc[dt];
    if (g == 0) {
      prow[C] = m_run;
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
static int round_up(int x, int a) { return (x + a - 1) / a * a; }

MqaPlan plan_mqa(int rows, int n_heads, int c, int max_list) {
  MqaPlan pl;
  // at most 4 waves (64 heads) per workgroup: 16 heads x 512 dims of fp32 accumulator per wave
  // plus the query fragments already fill most of a wave's registers
  int nw = (n_heads + 15) / 16;
  if (nw > 4) nw = 4;
  if (nw == 3) nw = 4;
  if (c >= 512 && nw < 2) nw = 2;  // one wave would need 2x the staging registers
  pl.heads_per_wg = 16 * nw;
  pl.head_groups = (n_heads + pl.heads_per_wg - 1) / pl.heads_per_wg;
  const long base = static_cast<long>(rows) * pl.head_groups;
  const long target = 512;
  int splits = base >= target ? 1 : static_cast<int>((target + base - 1) / base);
  int sr = round_up((max_list + splits - 1) / splits, 32);
  if (sr < 64 && max_list > 64) sr = 64;
  if (sr < 32) sr = 32;
  pl.split_rows = sr;
  pl.n_splits = (max_list + sr - 1) / sr;
  if (pl.n_splits < 1) pl.n_splits = 1;
  return pl;
}

size_t mqa_workspace(const MqaPlan& p, int rows, int n_heads, int c) {
  if (p.n_splits <= 1) return 0;
  return static_cast<size_t>(rows) * p.n_splits * n_heads * (c + 4) * sizeof(float);
}

template <int C, int NW>
static hipError_t launch_t(const MqaParams& prm, int rows, hipStream_t s) {
  const size_t lds = 2 * Tile<C>::kElems * sizeof(uint16_t);
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(mqa_kernel<C, NW>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(lds));
    if (e != hipSuccess) return e;
    attr = true;
  }
  MqaParams q = prm;
  q.n_work = rows * prm.n_splits;
  const unsigned grid = static_cast<unsigned>((q.n_work + 7) / 8 * 8) * prm.head_groups;
  {
    ProfScope ps(prm.idx ? "mqa_sparse" : "mqa_dense", s);
    mqa_kernel<C, NW><<<grid, 64 * NW, lds, s>>>(q);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || prm.n_splits == 1) return e;
  ProfScope ps("mqa_combine", s);
  mqa_combine_kernel<C><<<static_cast<unsigned>(rows) * prm.n_heads, 64, 0, s>>>(prm);
  return hipGetLastError();
}

template <int C>
static hipError_t launch_c(const MqaParams& prm, int nw, int rows, hipStream_t s) {
  switch (nw) {
    case 1: return launch_t<C, 1>(prm, rows, s);
    case 2: return launch_t<C, 2>(prm, rows, s);
    case 4: return launch_t<C, 4>(prm, rows, s);
  }
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
  const int nw = pl.heads_per_wg / 16;
  switch (a.c) {
    case 128: return launch_c<128>(p, nw, rows, s);
    case 256: return launch_c<256>(p, nw, rows, s);
    case 512: return launch_c<512>(p, nw, rows, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace csa
