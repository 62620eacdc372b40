// Shared-KV multi-query attention over compressed entries + sliding window + sink (gfx950).
//
// Method: "DeepSeek V4 模型技术大全", chapter "Attention": component table (shared K=V MQA with
// one KV head; attention sink p = exp(z) / (exp(a_h) + sum exp(z)); window W_t of the last
// n_win tokens) and section "注意力实现细节" (partial RoPE on the last dims of q and keys, the
// core-attention output rotated back).  CSA attends the top-k selected entries, HCA every closed
// entry j < floor((t+1)/m') ("HCA 的完整路径"); both add the window rows and share one softmax.
//
// Layout of the work.  A workgroup owns one query row, 32*HP heads and a span of the query's
// key list (selected or visible entries, then window tokens).  Key rows are gathered 32 at a
// time into LDS and shared by all waves; while one tile is computed the next two are in flight
// in registers.  Wave (hp, s) owns heads hp*32..hp*32+31 and, for C = 512, the dim slice
// s*256..s*256+255 (DS = 2 slices; one slice for C <= 256).  Per wave and tile, with 32x32x16
// bf16 MFMAs:
//   S^T[32 rows x 32 heads] = E . Q^T over the slice  (A = entry rows from LDS, B = q in regs);
//   the DS slice partials are summed through LDS;
//   online softmax per head in the log2 domain (lane l: head l%32, 16 of the 32 rows);
//   O^T[slice dims x 32 heads] += E^T . P^T  (A = transposed LDS reads, B = P^T taken straight
//   from the S^T accumulator layout).
// LDS rows are unpadded with 16-byte chunks XOR-swizzled by row, which keeps both the row reads
// of the S phase and the transposed reads of the PV phase free of bank conflicts.  With several
// spans per query each workgroup writes (max, sum, O / sum in bf16) and a combine kernel merges
// them in a fixed order, adds the sink and normalises; with one span the workgroup runs the same
// merge on its own partial in place.  The span size depends on the key list's length and on
// whether the call brings one query per sequence or a run of them, never on the batch size, so a
// sequence's output bits do not depend on which other sequences share the call.
#include <algorithm>
#include <cmath>

#include "mqa_common.h"

namespace csa {

template <int C, int HP_>
struct MqaShape {
  static constexpr int HP = HP_;
  static constexpr int DS = C == 512 ? 2 : 1;   // dim slices
  static constexpr int NW = HP * DS;            // waves
  static constexpr int NT = 64 * NW;
  static constexpr int CS = C / DS;             // dims per slice (256 or 128)
  static constexpr int KK = CS / 16;            // S^T MFMA steps over the slice
  static constexpr int DT = CS / 32;            // 32-dim output tiles of the slice
  static constexpr int CPR = C / 8;             // 16-byte chunks per row
  static constexpr int LOADS = 32 * CPR / NT;   // chunks per thread per tile
  static constexpr int TILE = 32 * C;           // bf16 elements per LDS tile
  static constexpr size_t lds_sx() { return 2 * TILE * sizeof(uint16_t); }
  static constexpr size_t lds_freq() { return lds_sx() + (DS > 1 ? NW * 1024 * sizeof(float) : 0); }
  static constexpr size_t lds_fixed() { return lds_freq() + (C / 2) * sizeof(float); }
};

// PAGED: entries live in a block pool; the span's entry list (selected indices, or the visible
// range for the dense case) is translated to pool rows once, into LDS, and those rows are
// gathered (-1: masked).
template <int C, int HP, bool PAGED = false>
__global__ __launch_bounds__((MqaShape<C, HP>::NT)) void mqa_kernel(MqaParams p) {
  using SH = MqaShape<C, HP>;
  constexpr int DS = SH::DS, NW = SH::NW, NT = SH::NT, CS = SH::CS, KK = SH::KK, DT = SH::DT;
  constexpr int CPR = SH::CPR, LOADS = SH::LOADS, TILE = SH::TILE;
  static_assert(LOADS * NT == 32 * CPR, "tile chunks must split evenly over the threads");
  static_assert(CPR == 64 || 64 % CPR == 0, "a load step covers whole rows");
  static_assert(NT >= 64, "one thread per RoPE frequency (rope_dim <= 128 is checked at the API)");
  extern __shared__ __align__(16) unsigned char smem[];
  uint16_t* E = reinterpret_cast<uint16_t*>(smem);                         // [2][32][C] swizzled
  float* SX = reinterpret_cast<float*>(smem + SH::lds_sx());       // [NW][4][64][4]
  float* s_freq = reinterpret_cast<float*>(smem + SH::lds_freq());  // [r/2] RoPE frequencies
  int* s_idx = reinterpret_cast<int*>(smem + SH::lds_fixed());      // [split_rows]

  const int tid = threadIdx.x;
  const int l = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hp = wave % HP, slice = wave / HP;
  const int h = l >> 5, n32 = l & 31;
  // Work item w = (row, split); head groups of one work item are blocks 8 apart (same XCD).
  const int bid = blockIdx.x;
  const int w = (bid / (8 * p.head_groups)) * 8 + (bid & 7);
  const int hg = (bid >> 3) % p.head_groups;
  if (w >= p.n_work) return;
  const int split = w % p.n_splits;
  const int row = w / p.n_splits;
  const int b = row / p.nq;
  const int j0 = split * p.split_rows;
  // the first two tiles' selected indices depend only on (row, split): their loads go out
  // before the position and entry count they are checked against (two dependent memory round
  // trips before the first gathers instead of three)
  int pre0 = 0, pre1 = 0;
  if (p.idx && l < 32) {
    const int32_t* ir = p.idx + static_cast<size_t>(row) * p.k;
    pre0 = ir[min(j0 + l, p.k - 1)];
    pre1 = ir[min(j0 + 32 + l, p.k - 1)];
  }
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
  const int j1 = min(R, j0 + p.split_rows);
  const int head = (hg * HP + hp) * 32 + n32;
  const bool head_ok = head < p.n_heads;
  const int dbase = slice * CS;
  // pool row of logical entry e (-1 if e is not a closed entry)
  auto xlate = [&](int e) {
    return (e >= 0 && e < n_ent) ? static_cast<int>(entry_row(p.pages, p.n_max, b, e)) : -1;
  };
  if constexpr (PAGED) {
    if (l < 32) {
      pre0 = xlate(p.idx ? pre0 : j0 + l);
      pre1 = xlate(p.idx ? pre1 : j0 + 32 + l);
    }
  }

  // Row pointers of the tile starting at list row jt, computed by lanes 0..31 (one row each).
  // Rows that are masked (past the span, an index outside the visible entries) point at the
  // window row of token t, which every call holds, and are excluded through the valid mask,
  // so every lane always issues its loads and no gathered value is ever undefined.
  const uint16_t* const safe_row =
      p.window + (static_cast<size_t>(b) * p.win_slots + (t % p.win_slots)) * C;
  auto resolve = [&](int jt, int pre, const uint16_t*& ptr, uint32_t& mask) {
    const int j = jt + l;
    const uint16_t* pr = safe_row;
    bool ok = false;
    if (l < 32 && j < j1) {
      if (j < n_sel) {
        const int e = (p.idx || PAGED) ? (pre >= -1 ? pre : s_idx[j - j0]) : j;
        if constexpr (PAGED) {
          ok = e >= 0;
          if (ok) pr = p.entries + static_cast<size_t>(e) * C;
        } else {
          ok = e >= 0 && e < n_ent;
          if (ok) pr = p.entries + (static_cast<size_t>(b) * p.n_max + e) * C;
        }
      } else {
        const int u = wlo + (j - n_sel);
        ok = true;
        pr = p.window + (static_cast<size_t>(b) * p.win_slots + (u % p.win_slots)) * C;
      }
    }
    ptr = pr;
    mask = static_cast<uint32_t>(__ballot(ok));
  };
  auto gload = [&](const uint16_t* ptr, u32x4 (&st)[LOADS]) {
    const uint64_t pv = reinterpret_cast<uint64_t>(ptr);
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int ch = tid + i * NT;
      const int cc = ch % CPR;
      uint64_t rp;
      if constexpr (CPR == 64) {  // one row per wave and load step: a wave-uniform pointer
        const int rr = wave + i * NW;
        const uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(pv), rr);
        const uint32_t hi = __builtin_amdgcn_readlane(static_cast<uint32_t>(pv >> 32), rr);
        rp = (static_cast<uint64_t>(hi) << 32) | lo;
      } else {
        const int rr = ch / CPR;
        const uint32_t lo = __shfl(static_cast<uint32_t>(pv), rr, 64);
        const uint32_t hi = __shfl(static_cast<uint32_t>(pv >> 32), rr, 64);
        rp = (static_cast<uint64_t>(hi) << 32) | lo;
      }
      st[i] = *(reinterpret_cast<const __attribute__((address_space(1))) u32x4*>(rp) + cc);
    }
  };

  // The tile count is odd (padded with a masked tile): the first tile is peeled, the rest run
  // in pairs with static register stages and LDS buffers.  Every tile step prefetches two tiles
  // ahead unconditionally (tiles past the span resolve to masked rows), so both register stages
  // are always in flight in the same order.  The first two tiles are issued before anything
  // else, with their indices read straight from global memory (pre0, pre1).
  const int ntiles = j1 > j0 ? (((j1 - j0 + 31) / 32) | 1) : 0;
  u32x4 stage0[LOADS], stage1[LOADS];
  uint32_t mask0 = 0, mask1 = 0;
  if (ntiles > 0) {
    const uint16_t* p0;
    const uint16_t* p1;
    resolve(j0, pre0 < -1 ? -1 : pre0, p0, mask0);
    resolve(j0 + 32, pre1 < -1 ? -1 : pre1, p1, mask1);
    gload(p0, stage0);
    gload(p1, stage1);
  }

  // All other global loads of the prologue follow right behind, so that their latencies overlap
  // with the gathers': the query fragments, the sink, the RoPE frequencies and the span's
  // selected entry indices (the last two go to LDS: the tile loop then issues no global load
  // but the row gathers, and the epilogue does not read frequencies behind its own stores).
  u32x4 qraw[KK];
  {
    const uint16_t* qrow = p.q + (static_cast<size_t>(row) * p.n_heads + (head_ok ? head : 0)) * C;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      qraw[kk] = head_ok ? *reinterpret_cast<const u32x4*>(qrow + dbase + kk * 16 + h * 8)
                         : u32x4{0, 0, 0, 0};
  }
  const float sink_v = (p.sink && head_ok) ? p.sink[head] : 0.f;
  const float freq_v = tid < (p.r >> 1) ? p.inv_freq[tid] : 0.f;  // r/2 <= C/2 <= NT
  if (p.idx || PAGED) {
    constexpr int IPT = 8;  // indices per thread and pass, all loaded before any is stored
    const int e1 = min(j1, n_sel);
    for (int base = j0; base < e1; base += NT * IPT) {
      int v[IPT];
#pragma unroll
      for (int i = 0; i < IPT; ++i) {
        const int j = base + tid + i * NT;
        v[i] = j < e1 ? (p.idx ? p.idx[static_cast<size_t>(row) * p.k + j] : j) : 0;
      }
      if constexpr (PAGED) {
#pragma unroll
        for (int i = 0; i < IPT; ++i) v[i] = xlate(v[i]);
      }
#pragma unroll
      for (int i = 0; i < IPT; ++i) {
        const int j = base + tid + i * NT;
        if (j < e1) s_idx[j - j0] = v[i];
      }
    }
  }
  if (tid < (p.r >> 1)) s_freq[tid] = freq_v;
  __syncthreads();  // s_idx, s_freq

  // ---- query fragments (B operand of S^T): head l%32, dims dbase + 16kk + 8h .. +7, rotated
  // at t on the RoPE dims
  bf16x8 bq[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    const int d0 = dbase + kk * 16 + h * 8;
    u32x4 raw = qraw[kk];
    if (d0 + 8 > C - p.r) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = d0 + 2 * j;
        if (d >= C - p.r) {
          float cs, sn;
          rope_cos_sin(t, s_freq[(d - (C - p.r)) >> 1], cs, sn);
          const float x0 = bf16_to_f32(static_cast<uint16_t>(raw[j] & 0xffff));
          const float x1 = bf16_to_f32(static_cast<uint16_t>(raw[j] >> 16));
          raw[j] = pack2(x0 * cs - x1 * sn, x0 * sn + x1 * cs);
        }
      }
    }
    bq[kk] = as_bf16x8(raw);
  }
  // the query fragments are complete before the tile loop (otherwise the first use inside the
  // loop would wait for every load in flight, on every iteration)
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) asm volatile("" ::"v"(bq[kk]) : "memory");

  f32x16 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x16{};
  // m_ref: the reference maximum the probabilities are taken against (log2 domain, scaled); it
  // moves only when a scaled logit exceeds it by more than 8, so the accumulators are rarely
  // rescaled and every probability stays below 2^8.
  float m_ref = -INFINITY, l_run = 0.f;

  // LDS byte offsets that do not change from tile to tile (the buffer, the upper 16-chunk block
  // of a row and the second 16-row half are added as immediates)
  uint32_t st_off[LOADS];  // store of load step i: row ch / CPR, chunk ch % CPR
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int ch = tid + i * NT;
    const int rr = ch / CPR, cc = ch % CPR;
    st_off[i] = static_cast<uint32_t>(rr * C + ((cc ^ swz(rr)) << 3)) * 2u;
  }
  // S phase (A operand): lane row n32, logical chunk (dbase>>3) + 2kk + h; the swizzle only
  // touches the low four chunk bits, so kk >= 8 adds 256 bytes to the offset of kk - 8.
  uint32_t sa_off[8];
#pragma unroll
  for (int k8 = 0; k8 < 8; ++k8)
    sa_off[k8] = static_cast<uint32_t>(n32 * C + (dbase & ~127) +
                                       (((((dbase >> 3) & 15) + 2 * k8 + h) ^ swz(n32)) << 3)) * 2u;
  // PV phase (transposed A operand): rows 16mm + 4h + i0 (first read) and +8 (second read),
  // logical chunk (dbase>>3) + 4dt + 2(G&1) + q/2, element 4(q&1) in the chunk.  Row swizzles:
  // (i0<<2)|h and (i0<<2)|(2+h), independent of mm; dt>>2 adds 256 bytes, mm adds 16 rows.
  const int G = l >> 4, i0 = (l & 15) >> 2, q4 = l & 3;
  uint32_t ta_off[4], tb_off[4];
#pragma unroll
  for (int d3 = 0; d3 < 4; ++d3) {
    const int low = 4 * d3 + 2 * (G & 1) + (q4 >> 1);
    const int ra = 4 * h + i0, rb = ra + 8;
    ta_off[d3] = static_cast<uint32_t>(ra * C + (dbase & ~127) + ((low ^ swz(ra)) << 3) +
                                       4 * (q4 & 1)) * 2u;
    tb_off[d3] = static_cast<uint32_t>(rb * C + (dbase & ~127) + ((low ^ swz(rb)) << 3) +
                                       4 * (q4 & 1)) * 2u;
  }

  // tile step, front part: tile `it` (held in stage st) goes to LDS buffer buf, tile it+2 is
  // resolved and its gathers issued into the same stage; returns tile it's valid mask
  auto front = [&](int it, u32x4 (&st)[LOADS], uint32_t& mask, int buf) -> uint32_t {
    if constexpr (DS == 1) __syncthreads();  // every wave is done with the buffer's last tile
#pragma unroll
    for (int i = 0; i < LOADS; ++i)
      *reinterpret_cast<u32x4*>(smem + st_off[i] + buf * TILE * 2) = st[i];
    const uint32_t msk = mask;
    const uint16_t* pn;
    resolve(j0 + (it + 2) * 32, -2, pn, mask);  // -2: read the index from LDS
    __syncthreads();  // tile `it` is in LDS
    gload(pn, st);
    return msk;
  };
  // partial S^T of this wave's slice from LDS buffer buf
  auto s_phase = [&](int buf) -> f32x16 {
    const unsigned char* Eb = smem + buf * TILE * 2;
    f32x16 sacc = f32x16{};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const bf16x8 a =
          as_bf16x8(*reinterpret_cast<const u32x4*>(Eb + sa_off[kk & 7] + (kk >> 3) * 256));
      sacc = mfma_bf16_32x32x16(a, bq[kk], sacc);
    }
    return sacc;
  };
  // O^T += E^T . P^T on this slice's dims from LDS buffer buf.  K slots of lane half h in MFMA
  // mm: rows 16mm + 4h + 0..3 and 16mm + 8 + 4h + 0..3, read transposed (within each 16-lane
  // group, lane 4*i0+q addresses row base+i0, dims +4q..+4q+3 of a 4x16 block; lane j receives
  // dim j of rows base..base+3).
  auto pv_phase = [&](int buf, const bf16x8 (&bp)[2]) {
    const unsigned char* Eb = smem + buf * TILE * 2;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int mm = 0; mm < 2; ++mm) {
        const uint32_t imm = (dt >> 2) * 256 + mm * 16 * C * 2;
        const bf16x4 lo = lds_read_tr16(reinterpret_cast<const uint16_t*>(Eb + ta_off[dt & 3] + imm));
        const bf16x4 hi = lds_read_tr16(reinterpret_cast<const uint16_t*>(Eb + tb_off[dt & 3] + imm));
        const bf16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        acc[dt] = mfma_bf16_32x32x16(a, bp[mm], acc[dt]);
      }
    }
  };
  // slice sum, mask, online softmax of one tile; P^T (bf16, B operand of the PV MFMAs) to bp
  auto softmax = [&](f32x16 sacc, uint32_t msk, bf16x8 (&bp)[2]) {
    if constexpr (DS > 1) {  // sum the slice partials of this head pair
      f32x4* mine = reinterpret_cast<f32x4*>(SX + wave * 1024);
#pragma unroll
      for (int qq = 0; qq < 4; ++qq)
        mine[qq * 64 + l] = f32x4{sacc[4 * qq], sacc[4 * qq + 1], sacc[4 * qq + 2], sacc[4 * qq + 3]};
      __syncthreads();
      const f32x4* other = reinterpret_cast<const f32x4*>(SX + (hp + (1 - slice) * HP) * 1024);
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const f32x4 v = other[qq * 64 + l];
#pragma unroll
        for (int e = 0; e < 4; ++e) sacc[4 * qq + e] += v[e];
      }
    }
    // element i of the accumulator holds row 8*(i/4) + 4h + i%4 of the tile, head l%32
    if (msk != 0xffffffffu) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int rr = 8 * (i >> 2) + 4 * h + (i & 3);
        if (!((msk >> rr) & 1u)) sacc[i] = -INFINITY;
      }
    }
    float mx = sacc[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sacc[i]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * p.scale_log2;
    const bool move = mx > m_ref + 8.f;
    if (__ballot(move)) {  // wave-uniform: some head's reference has to move up
      const float m_new = move ? mx : m_ref;
      const float alpha = (m_new == m_ref) ? 1.f : __builtin_amdgcn_exp2f(m_ref - m_new);
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) acc[dt] *= alpha;
      m_ref = m_new;
    }
    const float mu = (m_ref == -INFINITY) ? 0.f : m_ref;
    float psum = 0.f;
#pragma unroll
    for (int mm = 0; mm < 2; ++mm) {
      u32x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[8 * mm + 2 * e], p.scale_log2, -mu));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[8 * mm + 2 * e + 1], p.scale_log2, -mu));
        psum += p0 + p1;
        v[e] = pack2(p0, p1);
      }
      bp[mm] = as_bf16x8(v);
    }
    l_run += psum;
  };

  if (ntiles > 0) {
    bf16x8 bpA[2], bpB[2];
    {
      const uint32_t msk = front(0, stage0, mask0, 0);
      softmax(s_phase(0), msk, bpA);
    }
    // step it: S of tile it interleaves with PV of tile it-1 (independent MFMA chains on
    // different LDS buffers), then the slice sum and softmax of tile it
    for (int it = 1; it < ntiles; it += 2) {
      uint32_t msk = front(it, stage1, mask1, 1);
      f32x16 sacc = s_phase(1);
      pv_phase(0, bpA);
      softmax(sacc, msk, bpB);
      msk = front(it + 1, stage0, mask0, 0);
      sacc = s_phase(0);
      pv_phase(1, bpB);
      softmax(sacc, msk, bpA);
    }
    pv_phase(0, bpA);  // the last tile (even index)
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const size_t orow = static_cast<size_t>(row) * p.n_heads + head;
  if (!head_ok) return;
  // output element i of acc[dt]: head l%32, dim dbase + 32dt + 8*(i/4) + 4h + i%4
  const float il = l_tot > 0.f ? 1.f / l_tot : 0.f;  // the partial is O / l of the span
  if (p.n_splits == 1) {
    // the combine's merge of this one partial (rounded to bf16 as it would have been stored)
    const float a2 = p.sink ? sink_v * kLog2e : -INFINITY;
    SpanMerge sm = sm_start(a2);
    sm_raise(sm, fmaxf(sm.M, m_ref));
    const float wgt = sm_add(sm, m_ref, l_tot);
    const float inv = sm_inv(sm, p.sink != nullptr, a2);
    auto fin = [&](float v) { return sm_fold(0.f, bf16_round(v * il), wgt) * inv; };
    uint16_t* orow_p = p.out + orow * C;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = dbase + dt * 32 + g4 * 8 + 4 * h;
        store_out4(orow_p + d0, fin(acc[dt][4 * g4]), fin(acc[dt][4 * g4 + 1]),
                   fin(acc[dt][4 * g4 + 2]), fin(acc[dt][4 * g4 + 3]), d0, C, p.r, t, s_freq);
      }
    if (p.lse_out && h == 0 && slice == 0) p.lse_out[orow] = sm_lse(sm);
  } else {
    // span partials in the MFMA lane order: per (row, span, head group, wave) DT*4 chunks of
    // 64 lanes x 4 values, so every store instruction writes 512 bytes contiguous; the values
    // are O / l of the span (|O / l| <= max |entry|) in bf16 (fp32's exponent range: no
    // overflow whatever the entries' magnitudes)
    uint16_t* pw = reinterpret_cast<uint16_t*>(p.part) +
                   ((((static_cast<size_t>(row) * p.n_splits + split) * p.head_groups + hg) * NW +
                     wave) * (DT * 4) * 256);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
        *reinterpret_cast<uint2*>(pw + ((dt * 4 + g4) * 64 + l) * 4) =
            uint2{pack2(acc[dt][4 * g4] * il, acc[dt][4 * g4 + 1] * il),
                  pack2(acc[dt][4 * g4 + 2] * il, acc[dt][4 * g4 + 3] * il)};
    if (h == 0 && slice == 0) {
      float* mlp = p.ml + ((static_cast<size_t>(row) * p.n_splits + split) * p.n_heads + head) * 2;
      mlp[0] = m_ref;
      mlp[1] = l_tot;
    }
  }
}

// ---------------------------------------------------------------- eight-wave variant, C = 512
// Wave (hp, s) of eight owns heads hp*32..hp*32+31 and the 128-dim slice s*128..s*128+127: its
// output accumulators take 64 registers and two waves share each SIMD.  The four slice partials
// of S^T are summed through LDS with a change of ownership: wave (hp, s) finishes the softmax of
// heads 8s..8s+7 of its pair over all 32 rows of the tile (lane l: head 8s + l%8, rows
// 4(l/8)..4(l/8)+3), so the per-head maximum is a reduction across lanes of one wave (DPP and
// lane-swap instructions, no LDS round trip).  The owner publishes P^T (bf16, in the K-slot
// order of the PV MFMAs) and the rescale factor of each head.
//
// Two barriers per tile step i:
//   phase A: tile i+1 from registers into LDS, this wave's S partial of tile i out, gathers of
//            tile i+3 issued; barrier
//   phase B: rescale by the factors of tile i-1; slice sums and softmax of tile i (P^T and
//            factors out); PV of tile i-1; S of tile i+1; rows of tile i+4 resolved; barrier
// Phase B is one branch-free block apart from the rare rescale, so the scheduler can spread
// its 16 MFMAs over the softmax and address work.  Key tiles live in a ring of three LDS buffers
// (tile t in buffer t % 3); P^T and the factors alternate between two buffers by tile parity.
template <int C>
struct MqaWideShape {
  static constexpr int HP = 2, DS = 4, NW = HP * DS, NT = 64 * NW;
  static constexpr int CS = C / DS;             // dims per slice
  static constexpr int KK = CS / 16;            // S^T MFMA steps over the slice
  static constexpr int DT = CS / 32;            // 32-dim output tiles of the slice
  static constexpr int CPR = C / 8;             // 16-byte chunks per row
  static constexpr int LOADS = 32 * CPR / NT;   // chunks per thread per tile
  static constexpr int TILE = 32 * C;           // bf16 elements per LDS tile
  static constexpr int NBUF = 3;
  static constexpr size_t off_sx = NBUF * TILE * sizeof(uint16_t);  // [HP][DS][4][64] f32x4
  static constexpr size_t off_sp = off_sx + HP * DS * 4 * 64 * 16;  // [2][HP][8][32] 4 x bf16
  static constexpr size_t off_sa = off_sp + 2 * HP * 8 * 32 * 8;    // [2][HP][32] factors
  static constexpr size_t off_sl = off_sa + 2 * HP * 32 * 4;        // [HP][32] (max, sum)
  static constexpr size_t off_cs = off_sl + HP * 32 * 8;            // [64] cos/sin of the RoPE pairs
  static constexpr size_t lds_fixed() { return off_cs + 64 * sizeof(float2); }
};

// x combined with lane l ^ 8, l ^ 16 and l ^ 32 (a reduction over the eight lanes l % 8 + 8j)
__device__ __forceinline__ float max_over_xor8_16_32(float x) {
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xf, 0xf,
                                                          false)));  // row_ror:8 = lane ^ 8
  auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(s16[0]), __uint_as_float(s16[1]));
  auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(s32[0]), __uint_as_float(s32[1]));
}
__device__ __forceinline__ float sum_over_xor8_16_32(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xf, 0xf, false));
  auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(s16[0]) + __uint_as_float(s16[1]);
  auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(s32[0]) + __uint_as_float(s32[1]);
}

// PAGED: as mqa_kernel's, the span's entries are translated to pool rows in the prologue.
// MIXED: entries are rows of c + r bytes, the c - r unrotated dims as E4M3 codes then the r RoPE
// dims in bf16; a gathered entry row is widened to bf16 (exact) as it is stored to LDS, so the
// tiles and everything after them are unchanged.  Window rows stay bf16.
template <int C, bool SPARSE, bool PAGED = false, bool MIXED = false>
__global__ __launch_bounds__((MqaWideShape<C>::NT)) void mqa_wide_kernel(MqaParams p) {
  using SH = MqaWideShape<C>;
  constexpr int HP = SH::HP, DS = SH::DS, NW = SH::NW, NT = SH::NT, CS = SH::CS, KK = SH::KK,
                DT = SH::DT, CPR = SH::CPR, LOADS = SH::LOADS, TILE = SH::TILE;
  constexpr uint32_t TB = TILE * 2;  // bytes per LDS tile
  static_assert(CPR == 64 && LOADS * NT == 32 * CPR, "one row per wave and load step");
  static_assert(KK <= 8 && DT <= 4, "offset tables below cover one 128-dim block");
  static_assert(NT >= C / 2 && NT * LOADS * 16 >= TB, "prologue work splits over the threads");
  static_assert(HP * 32 * (C + 8) * 2 <= SH::NBUF * TB && (HP * 32 * (C / 8)) % NT == 0,
                "the output rows fit the tile ring and split evenly over the threads");
  extern __shared__ __align__(16) unsigned char smem[];
  f32x4* SX = reinterpret_cast<f32x4*>(smem + SH::off_sx);
  uint2* SP = reinterpret_cast<uint2*>(smem + SH::off_sp);
  float* SA = reinterpret_cast<float*>(smem + SH::off_sa);
  float2* SL = reinterpret_cast<float2*>(smem + SH::off_sl);
  float2* s_cs = reinterpret_cast<float2*>(smem + SH::off_cs);  // cos, sin of pair i at t
  int* s_idx = reinterpret_cast<int*>(smem + SH::lds_fixed());  // [split_rows] (LIST)
  constexpr bool LIST = SPARSE || PAGED;  // rows come from the span's list in s_idx

  const int tid = threadIdx.x;
  const int l = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hp = wave % HP, slice = wave / HP;
  const int h = l >> 5, n32 = l & 31;
  const int r4 = l >> 3, hh = 8 * slice + (l & 7);  // softmax share: head hh, rows 4r4..4r4+3
  mqa_preload_params(p);
  const int bid = blockIdx.x;
  int hg, split, row;
  mqa_work_item(p, bid, hg, split, row);
  if (row < 0) return;
  const int b = row / p.nq;
  const int j0 = split * p.split_rows;
  const int head = (hg * HP + hp) * 32 + n32;
  const bool head_ok = head < p.n_heads;
  const int dbase = slice * CS;
  // Loads go out in the order they are needed and none is conditional, so each wait below
  // covers only what it needs (vector loads complete in order): the span's first indices, its
  // index list, sink and RoPE frequencies; then the query slice; the first gathers last.
  constexpr int IPT = (kMaxTopK + NT - 1) / NT;  // index-list entries per thread: any span
  // position and entry count first, through the vector path (one round trip, waited for once
  // below, not two scalar round trips each behind a wait for every scalar load)
  int rv = p.pos ? row : b, bv = b;
  asm volatile("" : "+v"(rv), "+v"(bv));
  int t_vec = (p.pos ? p.pos : p.n_entries)[rv];
  int ne_vec = p.n_entries[bv];
  asm volatile("" ::: "memory");
  int pre0 = 0, pre1 = 0;
  int iv[IPT];
  if constexpr (SPARSE) {
    const int32_t* ir = p.idx + static_cast<size_t>(row) * p.k;
    pre0 = ir[min(j0 + (l & 31), p.k - 1)];
    pre1 = ir[min(j0 + 32 + (l & 31), p.k - 1)];
#pragma unroll
    for (int i = 0; i < IPT; ++i) iv[i] = ir[min(j0 + i * NT + tid, p.k - 1)];
  }
  const float sink_raw = *(p.sink ? p.sink + (head_ok ? head : 0) : p.inv_freq);
  const float freq_v = p.inv_freq[min(tid, (p.r >> 1) - 1)];
  u32x4 qraw[KK];
  {
    const uint16_t* qrow = p.q + (static_cast<size_t>(row) * p.n_heads + (head_ok ? head : 0)) * C;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      qraw[kk] = *reinterpret_cast<const u32x4*>(qrow + dbase + kk * 16 + h * 8);
  }
  asm volatile("" : "+v"(t_vec), "+v"(ne_vec) : : "memory");  // after Q is requested
  const int t = p.pos ? __builtin_amdgcn_readfirstlane(t_vec) : (row % p.nq);
  const int n_ent = max(0, min(__builtin_amdgcn_readfirstlane(ne_vec), p.n_max));
  const int n_w = min(p.n_win, t + 1);
  const int wlo = t - n_w + 1;
  int n_sel;
  if (SPARSE) {
    n_sel = p.k;
  } else {
    const long v = (static_cast<long>(t) + 1) / p.m;
    n_sel = static_cast<int>(v < n_ent ? v : n_ent);
  }
  const int R = n_sel + n_w;
  const int j1 = min(R, j0 + p.split_rows);

  // Row pointers of the tile at list row jt (lanes 0..31; other lanes' values are unused).
  // Masked rows (past the span, an index outside the visible entries) read the window row of t.
  // Branch-free: the index is always read (clamped into the span's index list) and both
  // candidate pointers are formed, then selected.
  const int ES = MIXED ? (C + p.r) / 2 : C;  // entry row stride in 16-bit units
  const uint16_t* const ent_base =
      PAGED ? p.entries : p.entries + static_cast<size_t>(b) * p.n_max * ES;
  const uint16_t* const win_base = p.window + static_cast<size_t>(b) * p.win_slots * C;
  const uint16_t* const safe_row = win_base + static_cast<size_t>(t % p.win_slots) * C;
  // PAGED lists hold pool rows, already checked against the visible entries (-1: masked)
  const int e_lim = PAGED ? 0x7fffffff : n_ent;
  // em (MIXED): which rows of the tile are entry rows (the rest are bf16 window rows)
  auto resolve_e = [&](int j, int e, const uint16_t*& ptr, uint32_t& mask, uint32_t& em) {
    const bool in_span = l < 32 && j < j1;
    const bool sel = j < n_sel;
    const bool ok_e = e >= 0 && e < e_lim;
    const int u = max(wlo + (j - n_sel), 0);
    const uint16_t* pe = ent_base + static_cast<size_t>(ok_e ? e : 0) * ES;
    const uint16_t* pw = win_base + static_cast<size_t>(u % p.win_slots) * C;
    const bool ok = in_span && (!sel || ok_e);
    ptr = ok ? (sel ? pe : pw) : safe_row;
    mask = static_cast<uint32_t>(__ballot(ok));
    if constexpr (MIXED) em = static_cast<uint32_t>(__ballot(ok && sel));
  };
  auto resolve = [&](int jt, const uint16_t*& ptr, uint32_t& mask, uint32_t& em) {
    const int j = jt + l;
    int e = j;
    if constexpr (LIST) e = s_idx[min(max(j - j0, 0), p.split_rows - 1)];
    resolve_e(j, e, ptr, mask, em);
  };
  // MIXED: an entry row holds ncc 16-byte chunks of codes, then r/8 chunks of RoPE dims.  Lane l
  // fills bf16 chunk l of the LDS row either way: lanes below 2*ncc load the code chunk l/2 and
  // widen its half l%2 (8 codes), the others load RoPE chunk l - ncc as is.
  const int ncc = (C - p.r) >> 4;
  const int mixed_ch = l < 2 * ncc ? (l >> 1) : l - ncc;
  // wave `wave` loads rows wave, wave+8, wave+16, wave+24 of the tile, 16 bytes per lane
  auto gload = [&](const uint16_t* ptr, uint32_t em, u32x4 (&st)[LOADS]) {
    const uint64_t pv = reinterpret_cast<uint64_t>(ptr);
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int rr = wave + i * NW;
      const uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(pv), rr);
      const uint32_t hi = __builtin_amdgcn_readlane(static_cast<uint32_t>(pv >> 32), rr);
      const uint64_t rp = (static_cast<uint64_t>(hi) << 32) | lo;
      int ch = l;
      if constexpr (MIXED) ch = ((em >> rr) & 1u) ? mixed_ch : l;
      st[i] = *(reinterpret_cast<const __attribute__((address_space(1))) u32x4*>(rp) + ch);
    }
  };

  // even tile count (a masked tile pads odd spans); tiles 0 and 1 are gathered first, their
  // indices read straight from global memory
  const int ntiles = j1 > j0 ? ((j1 - j0 + 63) / 64) * 2 : 0;
  // (an empty span gathers masked rows, the window row of t, and never uses them)
  u32x4 stage0[LOADS], stage1[LOADS];
  uint32_t mq0 = 0, mq1 = 0, mq2 = 0, mq3 = 0;  // valid masks of tiles i .. i+3
  uint32_t em0 = 0, em1 = 0, em2 = 0, em3 = 0;  // entry-row masks of the same tiles (MIXED)
  // pool row of logical entry e (-1 if e is not a closed entry)
  auto xlate = [&](int e) {
    return (e >= 0 && e < n_ent) ? static_cast<int>(entry_row(p.pages, p.n_max, b, e)) : -1;
  };
  {
    const uint16_t* p0;
    const uint16_t* p1;
    int f0 = SPARSE ? pre0 : j0 + l, f1 = SPARSE ? pre1 : j0 + 32 + l;
    if constexpr (PAGED) {
      f0 = xlate(f0);
      f1 = xlate(f1);
    }
    resolve_e(j0 + l, f0, p0, mq0, em0);
    resolve_e(j0 + 32 + l, f1, p1, mq1, em1);
    gload(p0, em0, stage0);
    gload(p1, em1, stage1);
  }

  if constexpr (LIST) {
    const int e1 = min(j1, n_sel);
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
      const int j = j0 + i * NT + tid;
      int v = SPARSE ? iv[i] : j;
      if constexpr (PAGED) v = j < e1 ? xlate(v) : -1;
      if (j < e1) s_idx[j - j0] = v;
    }
  }
  if (tid < (p.r >> 1)) {
    float cs, sn;
    rope_cos_sin(t, freq_v, cs, sn);
    s_cs[tid] = float2{cs, sn};
  }
  // the step before tile 0 runs a PV on buffer 2 with P = 0 and factors 1: zero both
#pragma unroll
  for (int i = 0; i < LOADS; ++i)
    reinterpret_cast<u32x4*>(smem + 2 * TB)[tid + i * NT] = u32x4{0, 0, 0, 0};
  if (tid < HP * 8 * 32) SP[HP * 8 * 32 + tid] = uint2{0, 0};
  if (tid < HP * 32) SA[HP * 32 + tid] = 1.f;
  __syncthreads();  // s_idx, s_cs, zeroed buffers

  bf16x8 bq[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    const int d0 = dbase + kk * 16 + h * 8;
    u32x4 raw = head_ok ? qraw[kk] : u32x4{0u, 0u, 0u, 0u};
    if (d0 + 8 > C - p.r) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = d0 + 2 * j;
        if (d >= C - p.r) {
          const float2 e = s_cs[(d - (C - p.r)) >> 1];
          const float cs = e.x, sn = e.y;
          const float x0 = bf16_to_f32(static_cast<uint16_t>(raw[j] & 0xffff));
          const float x1 = bf16_to_f32(static_cast<uint16_t>(raw[j] >> 16));
          raw[j] = pack2(x0 * cs - x1 * sn, x0 * sn + x1 * cs);
        }
      }
    }
    bq[kk] = as_bf16x8(raw);
  }
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) asm volatile("" ::"v"(bq[kk]) : "memory");

  f32x16 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x16{};
  // online softmax state of this lane's share (head hh, four rows): the reference maximum moves
  // only when a scaled logit exceeds it by more than 8; l_part sums this lane's probabilities
  float m_ref = -INFINITY, l_part = 0.f;

  uint32_t st_off[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int rr = wave + i * NW;
    st_off[i] = static_cast<uint32_t>(rr * C + ((l ^ swz(rr)) << 3)) * 2u;
  }
  // S phase (A operand): row n32, logical chunk (dbase>>3) + 2kk + h; the slice is one 16-chunk
  // block, so the swizzle stays inside it
  uint32_t sa_off[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk)
    sa_off[kk] = static_cast<uint32_t>(n32 * C + dbase + (((2 * kk + h) ^ swz(n32)) << 3)) * 2u;
  // PV phase (transposed A operand): rows 16mm + 4h + i0 and +8, logical chunk
  // (dbase>>3) + 4dt + 2(G&1) + q/2, element 4(q&1); mm adds 16 rows as an immediate
  const int G = l >> 4, i0 = (l & 15) >> 2, q4 = l & 3;
  uint32_t ta_off[DT], tb_off[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    const int low = 4 * dt + 2 * (G & 1) + (q4 >> 1);
    const int ra = 4 * h + i0, rb = ra + 8;
    ta_off[dt] = static_cast<uint32_t>(ra * C + dbase + ((low ^ swz(ra)) << 3) + 4 * (q4 & 1)) * 2u;
    tb_off[dt] = static_cast<uint32_t>(rb * C + dbase + ((low ^ swz(rb)) << 3) + 4 * (q4 & 1)) * 2u;
  }

  auto store_tile = [&](const u32x4 (&st)[LOADS], uint32_t em, uint32_t bo) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      u32x4 v = st[i];
      if constexpr (MIXED) {  // entry-row code lanes: 8 codes of dwords 2(l%2), 2(l%2)+1
        const int rr = wave + i * NW;
        const bool widen = ((em >> rr) & 1u) && l < 2 * ncc;
        const uint32_t w0 = (l & 1) ? v[2] : v[0], w1 = (l & 1) ? v[3] : v[1];
        const u32x4 wv = {
            __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.f, false)),
            __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.f, true)),
            __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.f, false)),
            __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.f, true))};
        v = widen ? wv : v;
      }
      *reinterpret_cast<u32x4*>(smem + st_off[i] + bo) = v;
    }
  };
  auto s_phase = [&](uint32_t bo) -> f32x16 {
    const unsigned char* Eb = smem + bo;
    u32x4 ea[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) ea[kk] = *reinterpret_cast<const u32x4*>(Eb + sa_off[kk]);
    f32x16 sacc = f32x16{};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) sacc = mfma_bf16_32x32x16(as_bf16x8(ea[kk]), bq[kk], sacc);
    return sacc;
  };
  // P^T of a tile for head n32 in the K-slot order of the PV MFMAs (rows 16mm + 4h + 0..3, then
  // 16mm + 8 + 4h + 0..3)
  auto read_p = [&](int par, bf16x8 (&bp)[2]) {
    const uint2* sp = SP + (par * HP + hp) * 256 + n32;
#pragma unroll
    for (int mm = 0; mm < 2; ++mm) {
      const uint2 lo = sp[(4 * mm + h) * 32];
      const uint2 hi = sp[(4 * mm + 2 + h) * 32];
      bp[mm] = as_bf16x8(u32x4{lo.x, lo.y, hi.x, hi.y});
    }
  };
  auto pv_phase = [&](uint32_t bo, const bf16x8 (&bp)[2]) {
    const unsigned char* Eb = smem + bo;
    bf16x8 ev[DT][2];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int mm = 0; mm < 2; ++mm) {
        const uint32_t imm = mm * 16 * C * 2;
        const bf16x4 lo = lds_read_tr16(reinterpret_cast<const uint16_t*>(Eb + ta_off[dt] + imm));
        const bf16x4 hi = lds_read_tr16(reinterpret_cast<const uint16_t*>(Eb + tb_off[dt] + imm));
        ev[dt][mm] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int mm = 0; mm < 2; ++mm) acc[dt] = mfma_bf16_32x32x16(ev[dt][mm], bp[mm], acc[dt]);
  };
  // this wave's S^T partial to LDS: element i of sacc holds row 8*(i/4) + 4h + i%4, head n32
  auto x_write = [&](const f32x16& sacc) {
    f32x4* mine = SX + (hp * DS + slice) * 256;
#pragma unroll
    for (int g = 0; g < 4; ++g)
      mine[g * 64 + l] = f32x4{sacc[4 * g], sacc[4 * g + 1], sacc[4 * g + 2], sacc[4 * g + 3]};
  };
  // slice sums of this lane's share (rows 4r4..4r4+3 of head hh sit in lane 32*(r4&1) + hh,
  // elements 4*(r4/2)..+3, of each slice's partial), mask, online softmax, P^T and the rescale
  // factor to LDS (buffer par); branch-free
  auto softmax = [&](uint32_t msk, int par) {
    const f32x4* src = SX + hp * DS * 256 + (r4 >> 1) * 64 + 32 * (r4 & 1) + hh;
    f32x4 s = src[0];
#pragma unroll
    for (int ss = 1; ss < DS; ++ss) s += src[ss * 256];
#pragma unroll
    for (int e = 0; e < 4; ++e) s[e] = ((msk >> (4 * r4 + e)) & 1u) ? s[e] : -INFINITY;
    const float mx =
        max_over_xor8_16_32(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]))) * p.scale_log2;
    const bool move = mx > m_ref + 8.f;
    const float m_new = move ? mx : m_ref;
    const float alpha = move ? __builtin_amdgcn_exp2f(m_ref - m_new) : 1.f;
    l_part *= alpha;
    m_ref = m_new;
    const float mu = (m_ref == -INFINITY) ? 0.f : m_ref;
    float pr[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) pr[e] = __builtin_amdgcn_exp2f(fmaf(s[e], p.scale_log2, -mu));
    l_part += (pr[0] + pr[1]) + (pr[2] + pr[3]);
    SP[((par * HP + hp) * 8 + r4) * 32 + hh] = uint2{pack2(pr[0], pr[1]), pack2(pr[2], pr[3])};
    SA[(par * HP + hp) * 32 + hh] = alpha;  // the eight lanes of a head write the same value
  };

  if (ntiles > 0) {
    // tile 0 into buffer 0, tile 2 gathered into its registers, S(0); tile 3 is resolved
    const uint16_t* pnext;
    {
      const uint16_t* p2;
      resolve(j0 + 64, p2, mq2, em2);
      resolve(j0 + 96, pnext, mq3, em3);
      store_tile(stage0, em0, 0);
      __syncthreads();
      gload(p2, em2, stage0);
    }
    f32x16 sacc = s_phase(0);
    bf16x8 bp[2];
    uint32_t bo_prev = 2 * TB, bo_next = TB;  // buffers of tiles i-1 and i+1
    auto step = [&](int i, u32x4 (&st)[LOADS]) {
      const int par = i & 1;
      // phase A: tile i+1 to LDS, S partial of tile i out, gathers of tile i+3
      store_tile(st, em1, bo_next);
      x_write(sacc);
      gload(pnext, em3, st);
      __syncthreads();
      // phase B
      {
        const float alpha = SA[((par ^ 1) * HP + hp) * 32 + n32];  // factor of tile i-1
        if (__ballot(alpha != 1.f)) {
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) acc[dt] *= alpha;
        }
      }
      read_p(par ^ 1, bp);
      softmax(mq0, par);
      pv_phase(bo_prev, bp);
      sacc = s_phase(bo_next);
      uint32_t mn, en = 0;
      resolve(j0 + (i + 4) * 32, pnext, mn, en);
      mq0 = mq1;
      mq1 = mq2;
      mq2 = mq3;
      mq3 = mn;
      em0 = em1;
      em1 = em2;
      em2 = em3;
      em3 = en;
      __syncthreads();
      bo_prev = bo_prev == 2 * TB ? 0 : bo_prev + TB;  // tile i, i.e. i-1 of the next step
      bo_next = bo_next == 2 * TB ? 0 : bo_next + TB;
    };
    for (int i = 0; i < ntiles; i += 2) {
      step(i, stage1);
      step(i + 1, stage0);
    }
    // PV of the last tile (odd index: P^T in buffer 1)
    {
      const float alpha = SA[(1 * HP + hp) * 32 + n32];
      if (__ballot(alpha != 1.f)) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) acc[dt] *= alpha;
      }
    }
    read_p(1, bp);
    pv_phase(bo_prev, bp);
  }

  // the owners publish (reference, sum) per head; every wave normalises its own dims
  {
    const float l_tot = sum_over_xor8_16_32(l_part);
    if (r4 == 0) SL[hp * 32 + hh] = float2{m_ref, l_tot};
  }
  __syncthreads();
  const float2 mlv = SL[hp * 32 + n32];
  const float m_fin = mlv.x, l_fin = mlv.y;
  const size_t orow = static_cast<size_t>(row) * p.n_heads + head;
  // output element i of acc[dt]: head n32, dim dbase + 32dt + 8*(i/4) + 4h + i%4
  const float il = l_fin > 0.f ? 1.f / l_fin : 0.f;  // the partial is O / l of the span
  if (p.n_splits == 1) {
    // the combine's merge of this one partial (rounded to bf16 as it would have been stored)
    const float a2 = (p.sink && head_ok) ? sink_raw * kLog2e : -INFINITY;
    SpanMerge sm = sm_start(a2);
    sm_raise(sm, fmaxf(sm.M, m_fin));
    const float wgt = sm_add(sm, m_fin, l_fin);
    const float inv = sm_inv(sm, p.sink != nullptr, a2);
    auto fin = [&](float v) { return sm_fold(0.f, bf16_round(v * il), wgt) * inv; };
    // The normalised, rotated rows of the workgroup's heads are assembled in LDS (the tile ring
    // is free after the barrier above; a row pitch of C + 8 elements spreads consecutive heads
    // over the banks) and leave as whole rows: each store instruction writes 1 KiB contiguous.
    constexpr int OP = C + 8;
    constexpr int CPR16 = C / 8;  // 16-byte chunks per row
    uint16_t* so = reinterpret_cast<uint16_t*>(smem);
    uint16_t* so_row = so + (hp * 32 + n32) * OP;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = dbase + dt * 32 + g4 * 8 + 4 * h;
        store_out4_tab(so_row + d0, fin(acc[dt][4 * g4]), fin(acc[dt][4 * g4 + 1]),
                       fin(acc[dt][4 * g4 + 2]), fin(acc[dt][4 * g4 + 3]), d0, C, p.r, s_cs);
      }
    if (p.lse_out && head_ok && h == 0 && slice == 0) p.lse_out[orow] = sm_lse(sm);
    __syncthreads();
    const int head0 = hg * HP * 32;
    uint16_t* obase = p.out + (static_cast<size_t>(row) * p.n_heads + head0) * C;
#pragma unroll
    for (int i = 0; i < HP * 32 * CPR16 / NT; ++i) {
      const int c = i * NT + tid;
      const int hr = c / CPR16, col = c % CPR16;
      if (head0 + hr < p.n_heads)
        *reinterpret_cast<u32x4*>(obase + static_cast<size_t>(hr) * C + col * 8) =
            *reinterpret_cast<const u32x4*>(so + hr * OP + col * 8);
    }
  } else {
    if (!head_ok) return;
    // span partials as in mqa_kernel: O / l of the span in bf16, MFMA lane order
    uint16_t* pw = reinterpret_cast<uint16_t*>(p.part) +
                   ((((static_cast<size_t>(row) * p.n_splits + split) * p.head_groups + hg) * NW +
                     wave) * (DT * 4) * 256);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
        *reinterpret_cast<uint2*>(pw + ((dt * 4 + g4) * 64 + l) * 4) =
            uint2{pack2(acc[dt][4 * g4] * il, acc[dt][4 * g4 + 1] * il),
                  pack2(acc[dt][4 * g4 + 2] * il, acc[dt][4 * g4 + 3] * il)};
    if (h == 0 && slice == 0) {
      float* mlp = p.ml + ((static_cast<size_t>(row) * p.n_splits + split) * p.n_heads + head) * 2;
      mlp[0] = m_fin;
      mlp[1] = l_fin;
    }
  }
}

// Merge of the spans of one (query row, 64-head group): a thread takes CPT of the DT*4 chunks a
// lane of one wave held (same head, 4 dims each), merges the spans in a fixed order, adds the
// sink once, normalises, rotates back and stores bf16.  Loads of up to NS spans are in flight
// together: NS covers every span of a CSA decode list (one pass, one round trip), and the RoPE
// frequencies of the thread's dims are requested with them, so the rotation at the end waits
// for nothing.  Fewer (row, head group) pairs than the device has CUs take one chunk per thread
// (twice the workgroups); larger batches two.
constexpr int kCombineMax = 24;

template <int C, class SH, int NS, int CPT>
__global__ __launch_bounds__((SH::NT)) void mqa_combine_kernel(MqaParams p) {
  constexpr int HP = SH::HP, NW = SH::NW, CS = SH::CS, DT = SH::DT;
  constexpr int GROUPS = DT * 4 / CPT;   // thread groups per (row, head group)
  const int bid = blockIdx.x;
  const int cgp = bid % GROUPS;
  const int hg = (bid / GROUPS) % p.head_groups;
  const int row = bid / (GROUPS * p.head_groups);
  const int tid = threadIdx.x, l = lane_id();
  const int wave = tid >> 6;
  const int hp = wave % HP, slice = wave / HP;
  const int h = l >> 5, n32 = l & 31;
  const int head = (hg * HP + hp) * 32 + n32;
  mqa_preload_params(p);
  if (head >= p.n_heads) return;
  const int t_vec = mqa_position_request(p, row);  // needed only for the rotation at the end
  const int dbase = slice * CS;
  // chunk cc = dt*4 + g4 holds dims dbase + 32dt + 8g4 + 4h .. +3: the frequencies of its two
  // RoPE pairs (a clamped pair for unrotated dims, unused)
  int dpos[CPT];
  float fq[CPT][2];
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int cc = cgp * CPT + c;
    dpos[c] = dbase + (cc >> 2) * 32 + (cc & 3) * 8 + 4 * h;
#pragma unroll
    for (int pr = 0; pr < 2; ++pr)
      fq[c][pr] = p.inv_freq[max(0, min(dpos[c] + 2 * pr - (C - p.r), p.r - 2)) >> 1];
  }
  const size_t span_stride = static_cast<size_t>(p.head_groups) * NW * (DT * 4) * 256;
  const uint16_t* pw0 = reinterpret_cast<const uint16_t*>(p.part) +
                        (((static_cast<size_t>(row) * p.n_splits) * p.head_groups + hg) * NW +
                         wave) * (DT * 4) * 256 + (cgp * CPT * 64 + l) * 4;
  const float* ml0 = p.ml + (static_cast<size_t>(row) * p.n_splits * p.n_heads + head) * 2;
  const size_t ml_stride = static_cast<size_t>(p.n_heads) * 2;

  // one pass per NS spans: their (max, sum) and O loads go out together, and the running
  // reference M moves (rescaling what was merged) only between passes
  // the sink is requested now and taken after the first pass's loads are out
  float sink_raw = *(p.sink ? p.sink + head : p.inv_freq);
  float sink2 = -INFINITY;
  SpanMerge sm = sm_start(-INFINITY);
  f32x4 o[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) o[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < p.n_splits; s0 += NS) {
    float mv[NS], lv[NS];
    uint2 ov[NS][CPT];
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const int sp = min(s0 + j, p.n_splits - 1);
      mv[j] = s0 + j < p.n_splits ? ml0[sp * ml_stride] : -INFINITY;
      lv[j] = ml0[sp * ml_stride + 1];
#pragma unroll
      for (int c = 0; c < CPT; ++c)
        ov[j][c] = *reinterpret_cast<const uint2*>(pw0 + sp * span_stride + c * 256);
    }
    if (s0 == 0) {
      asm volatile("" : "+v"(sink_raw) : : "memory");
      sink2 = p.sink ? sink_raw * kLog2e : -INFINITY;
      sm = sm_start(sink2);
    }
    float Mn = sm.M;
#pragma unroll
    for (int j = 0; j < NS; ++j) Mn = fmaxf(Mn, mv[j]);
    const float a = sm_raise(sm, Mn);
#pragma unroll
    for (int c = 0; c < CPT; ++c) o[c] *= a;
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const float wgt = sm_add(sm, mv[j], lv[j]);  // partials are O / l
      if (wgt == 0.f && mv[j] == -INFINITY) continue;
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        const f32x4 v = unpack_b4(ov[j][c]);
#pragma unroll
        for (int e = 0; e < 4; ++e) o[c][e] = sm_fold(o[c][e], v[e], wgt);
      }
    }
  }
  const float inv = sm_inv(sm, p.sink != nullptr, sink2);
  const int t = mqa_position_take(p, row, t_vec);
  uint2 packed[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int d0 = dpos[c];
    float x[4] = {o[c][0] * inv, o[c][1] * inv, o[c][2] * inv, o[c][3] * inv};
#pragma unroll
    for (int pr = 0; pr < 2; ++pr) {
      const int d = d0 + 2 * pr;
      if (d >= C - p.r) {
        float cs, sn;
        rope_cos_sin(t, fq[c][pr], cs, sn);
        const float x0 = x[2 * pr], x1 = x[2 * pr + 1];
        x[2 * pr] = x0 * cs + x1 * sn;
        x[2 * pr + 1] = -x0 * sn + x1 * cs;
      }
    }
    packed[c].x = pack2(x[0], x[1]);
    packed[c].y = pack2(x[2], x[3]);
  }
  uint16_t* dst = p.out + (static_cast<size_t>(row) * p.n_heads + head) * C;
#pragma unroll
  for (int c = 0; c < CPT; ++c) *reinterpret_cast<uint2*>(dst + dpos[c]) = packed[c];
  if (p.lse_out && cgp == 0 && h == 0 && slice == 0)
    p.lse_out[static_cast<size_t>(row) * p.n_heads + head] = sm_lse(sm);
}

// ---------------------------------------------------------------- planning and launch
static int round_up(int x, int a) { return (x + a - 1) / a * a; }

// Runs of queries (prefill) with up to 64 heads, c = 512, bf16 entries and lists of up to
// kHbqMaxList rows: the two-query head-block kernel (mqa_hb.hip), one span per query.
//
// Heads.  Sliced kernels: up to 64 heads per workgroup (two 32-head pairs), more heads as
// separate 64-head groups whose workgroups sit on the same XCD and share the gathered rows
// through its L2.  Decode over a long list (more than kMaxTopK rows, HCA over a long cache) with
// more than 64 heads, c = 512 and bf16 entries: the head-block kernel (mqa_hb.hip), 128 heads
// per workgroup, so every gathered row serves all of a query's heads in one pass.  Its fixed
// cost per workgroup (about 10 us of prologue and epilogue on MI355X) pays off only over long
// spans, so shorter lists stay on the sliced kernels.
//
// Spans.  How a query's key list is cut into spans decides the order in which its softmax terms
// are summed, so it must not depend on the batch: the plan reads the list's length (top_k +
// n_win for CSA, the cache's n_max + n_win for HCA) and whether the call brings one query per
// sequence (decode) or a run of kManyQueries or more (prefill), never the number of sequences.
// A sequence decoded alone or inside any batch, at any slot, gets the same bits.
//  * runs of queries: one span per query (lists up to kMaxTopK rows) -- the rows already fill
//    the device, and a split would only add the partials' round trip;
//  * decode, lists up to kMaxTopK rows (every CSA decode): spans of kDecodeSpan rows;
//  * decode, longer lists (HCA over a long cache): eight spans, sixteen for the head-block
//    kernel (each of its workgroups covers twice the heads, so twice the spans fill the device;
//    it always runs several spans).
constexpr int kManyQueries = 16;
constexpr int kDecodeSpan = 128;
constexpr int kLongListSpans = 8;
constexpr int kLongListSpansHb = 16;

MqaPlan plan_mqa(int nq, int n_heads, int c, int max_list, bool mixed) {
  MqaPlan pl;
  const int list0 = max_list > 0 ? max_list : 1;
  const bool hb =
      c == 512 && !mixed && n_heads > 64 && nq < kManyQueries && list0 > kMaxTopK;
  const bool hbq = c == 512 && !mixed && n_heads <= 64 && nq >= kManyQueries &&
                   round_up(list0, 32) <= kHbqMaxList;
  pl.kind = hb ? kMqaHeadBlock : (hbq ? kMqaHeadBlockQ : kMqaSliced);
  pl.head_pairs = hb ? 4 : 2;  // sliced: one instantiation, 64 heads (fewer leave waves idle)
  pl.slices = hb ? 1 : (c == 512 ? 4 : 1);  // eight waves of 128-dim slices for c = 512
  pl.heads_per_wg = 32 * pl.head_pairs;
  pl.head_groups = (n_heads + pl.heads_per_wg - 1) / pl.heads_per_wg;
  const int list = max_list > 0 ? max_list : 1;
  const int long_spans = hb ? kLongListSpansHb : kLongListSpans;
  int sr;
  if (nq >= kManyQueries) sr = round_up(list, 32);
  else if (list <= kMaxTopK) sr = kDecodeSpan;
  else sr = round_up((list + long_spans - 1) / long_spans, hb ? 32 : 64);
  pl.split_rows = std::min(sr, kMaxTopK);  // a span's list fits its LDS slots
  pl.n_splits = (list + pl.split_rows - 1) / pl.split_rows;
  return pl;
}

// partials: rows x spans x head groups x heads_per_wg heads x c bf16, then (max, sum) floats
// for rows x spans x heads (the head-block kernel indexes them by its padded head count)
size_t mqa_workspace(const MqaPlan& p, int rows, int n_heads, int c) {
  if (p.n_splits <= 1) return 0;
  const size_t heads = static_cast<size_t>(p.head_groups) * p.heads_per_wg;
  const size_t o = static_cast<size_t>(rows) * p.n_splits * heads * c;
  const size_t ml = static_cast<size_t>(rows) * p.n_splits *
                    (p.kind == kMqaHeadBlock ? heads : static_cast<size_t>(n_heads)) * 2;
  return o * sizeof(uint16_t) + ml * sizeof(float);  // bf16 partials, then fp32 (max, sum)
}

template <int C, class SH, bool WIDE, bool PAGED, bool MIXED = false>
static hipError_t launch_t(const MqaParams& prm, int rows, hipStream_t s) {
  const size_t lds = SH::lds_fixed() + ((prm.idx || PAGED)
                                            ? static_cast<size_t>(prm.split_rows) * sizeof(int)
                                            : 0);
  {
    hipError_t e;
    if constexpr (WIDE) {
      e = prm.idx ? ensure_max_lds(
                        reinterpret_cast<const void*>(mqa_wide_kernel<C, true, PAGED, MIXED>), lds)
                  : ensure_max_lds(
                        reinterpret_cast<const void*>(mqa_wide_kernel<C, false, PAGED, MIXED>), lds);
    } else {
      e = ensure_max_lds(reinterpret_cast<const void*>(mqa_kernel<C, SH::HP, PAGED>), lds);
    }
    if (e != hipSuccess) return e;
  }
  MqaParams q = prm;
  q.n_work = rows * prm.n_splits;
  const unsigned grid = mqa_grid(rows, prm.n_splits, prm.head_groups);
  {
    ProfScope ps(prm.idx ? "mqa_sparse" : "mqa_dense", s);
    if constexpr (WIDE) {
      if (prm.idx) mqa_wide_kernel<C, true, PAGED, MIXED><<<grid, SH::NT, lds, s>>>(q);
      else mqa_wide_kernel<C, false, PAGED, MIXED><<<grid, SH::NT, lds, s>>>(q);
    }
    else mqa_kernel<C, SH::HP, PAGED><<<grid, SH::NT, lds, s>>>(q);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || prm.n_splits == 1) return e;
  ProfScope ps("mqa_combine", s);
  constexpr int G2 = SH::DT * 4 / 2;  // workgroups per (row, head group) at two chunks a thread
  const unsigned pairs = static_cast<unsigned>(rows) * prm.head_groups;
  const bool one_chunk = pairs * G2 < 256;
  const bool wide = prm.n_splits > 8;
  const unsigned cgrid = pairs * (one_chunk ? 2 * G2 : G2);
  if (one_chunk) {
    if (wide) mqa_combine_kernel<C, SH, kCombineMax, 1><<<cgrid, SH::NT, 0, s>>>(prm);
    else mqa_combine_kernel<C, SH, 8, 1><<<cgrid, SH::NT, 0, s>>>(prm);
  } else {
    if (wide) mqa_combine_kernel<C, SH, kCombineMax, 2><<<cgrid, SH::NT, 0, s>>>(prm);
    else mqa_combine_kernel<C, SH, 8, 2><<<cgrid, SH::NT, 0, s>>>(prm);
  }
  return hipGetLastError();
}

template <int C>
static hipError_t launch_c(const MqaParams& prm, const MqaPlan& pl, int rows, bool mixed,
                           hipStream_t s) {
  const bool paged = prm.pages.table != nullptr;
  if constexpr (C == 512) {
    if (pl.kind == kMqaHeadBlock) {
      if (mixed || pl.head_pairs != 4) return hipErrorInvalidValue;
      return launch_mqa_hb(prm, rows, s);
    }
    if (pl.kind == kMqaHeadBlockQ) {
      if (mixed || pl.n_splits != 1) return hipErrorInvalidValue;
      return launch_mqa_hbq(prm, rows, s);
    }
    if (pl.head_pairs != 2) return hipErrorInvalidValue;
    using W = MqaWideShape<C>;
    if (mixed)
      return paged ? launch_t<C, W, true, true, true>(prm, rows, s)
                   : launch_t<C, W, true, false, true>(prm, rows, s);
    return paged ? launch_t<C, W, true, true>(prm, rows, s)
                 : launch_t<C, W, true, false>(prm, rows, s);
  } else {
    if (mixed || pl.kind != kMqaSliced || pl.head_pairs != 2) return hipErrorInvalidValue;
    return paged ? launch_t<C, MqaShape<C, 2>, false, true>(prm, rows, s)
                 : launch_t<C, MqaShape<C, 2>, false, false>(prm, rows, s);
  }
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
  p.pages = a.pages;
  p.scale_log2 = a.scale * kLog2e;
  p.split_rows = pl.split_rows;
  p.n_splits = pl.n_splits;
  p.head_groups = pl.head_groups;
  p.part = a.part;
  p.ml = a.part + static_cast<size_t>(a.B) * a.nq * pl.n_splits * pl.head_groups *
                      pl.heads_per_wg * a.c / 2;  // after the bf16 partials
  p.out = a.out;
  p.lse_out = a.lse_out;
  const int rows = a.B * a.nq;
  switch (a.c) {
    case 128: return launch_c<128>(p, pl, rows, a.entry_mixed, s);
    case 256: return launch_c<256>(p, pl, rows, a.entry_mixed, s);
    case 512: return launch_c<512>(p, pl, rows, a.entry_mixed, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace csa
