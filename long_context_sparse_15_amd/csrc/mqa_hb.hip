// Head-block shared-KV attention for head dim 512 (gfx950): decode over a long key list (HCA over
// a long cache) when a query has more than 64 heads.
//
// Method: "DeepSeek V4 模型技术大全", chapter "Attention": shared K = V MQA with one KV head over
// the selected (CSA) or all closed (HCA, "HCA 的完整路径") compressed entries plus the window rows
// of the last n_win tokens, one softmax with the attention sink, partial RoPE on the last dims
// and the output rotated back ("注意力实现细节").  The arithmetic of the softmax, the span
// partials and their merge is the one of mqa.hip (mqa_common.h); only the division of the work
// differs.
//
// Layout of the work.  A workgroup of four waves owns one query row, 128 heads and a span of the
// query's key list (the list is always cut into several spans); wave w owns heads 32w..32w+31
// over all 512 dims, so one gathered row serves every head of the query in one pass and no wave
// needs another's partial logits.  Each workgroup writes its span's partial (bf16 O / l and the
// span's (max, sum)); the combine kernel below merges them, adds the sink and rotates back.  Per 32-row
// tile and wave, with 32x32x16 bf16 MFMAs:
//   S^T[32 rows x 32 heads]  = E[32 rows x 512] . Q^T[512 x 32 heads]     32 K steps
//   O^T[512 dims x 32 heads] += E^T[512 x 32 rows] . P^T[32 rows x 32 heads]  16 dim blocks x 2
// Q^T stays in registers (128 VGPRs), O^T in the 256 accumulation registers, S^T and P^T never
// leave the wave: K slot s of lane half h in PV step kb is row 16kb + 4h + s (s < 4) or
// 16kb + 8 + 4h + s - 4, exactly the rows whose logits that lane's S^T accumulators hold.
// Key rows go from global memory straight into LDS (global_load_lds, one instruction per 1 KiB
// row) in a ring of four tiles: tile i+2 is requested while tile i is scored and tile i-1's PV
// runs, so a tile has two steps to arrive, and one barrier per tile suffices.  Rows that are
// masked (past the span's end inside its last tile, an index outside the visible entries) read
// the window row of t and are excluded from the softmax, so every row of a tile is loaded
// unconditionally; tiles past the span are not requested.
#include <algorithm>
#include <cmath>

#include "mqa_common.h"

namespace csa {

struct MqaHbShape {
  static constexpr int NW = 4, NT = 64 * NW, HPW = 32, HPG = HPW * NW;
  static constexpr int C = 512;
  static constexpr int NBUF = 4;
  static constexpr uint32_t TB = 32 * C * 2;   // bytes per tile
  static constexpr int RPW = 32 / NW;          // rows each wave requests per tile
  static constexpr size_t off_cs = NBUF * TB;  // [64] cos/sin of the RoPE pairs at t
  static constexpr size_t lds_fixed() { return off_cs + 64 * sizeof(float2); }
};
static_assert(MqaHbShape::HPW * MqaHbShape::C * 2 == MqaHbShape::TB,
              "a wave's output rows are staged in one tile buffer");

// max of v over lanes l and l ^ 32 (lane-swap instruction, no LDS round trip)
__device__ __forceinline__ float max_xor32(float v) {
  auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float sum_xor32(float v) {
  auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

// The output accumulators (32 heads x 512 dims = 256 registers a wave) live in the accumulation
// registers while the logits, the query and everything else use the 256 vector registers.  The
// file is compiled with MFMAs in vector-register form (so the S^T MFMAs and their consumers stay
// in vector registers), and the PV MFMAs are written out with accumulation-register operands.
// The compiler cannot see that these statements are MFMAs, so the wait states they require are
// issued explicitly (CDNA3/CDNA4 instruction set, MFMA dependency rules):
//  * a VALU write of a vector register read as an MFMA A/B operand: 2 wait states;
//  * an MFMA result read by a VALU (v_accvgpr_read) or overwritten by one: up to 18 wait states
//    after a 16-pass MFMA (32x32x16 bf16 takes 8 passes on gfx950; 18 covers both);
//  * a v_accvgpr_write read as SrcC by an MFMA: 2 wait states (3 issued).
// Back-to-back MFMAs that accumulate into the same registers are avoided altogether (the two
// steps into one block are issued 16 MFMAs apart).  The fences take the accumulators as operands
// so that no read or write of them can be scheduled across the waits.
__device__ __forceinline__ void mfma_32x32x16_agpr(f32x16& acc, bf16x8 a, bf16x8 b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b) : "memory");
}
// The S^T MFMAs are written out as well (vector-register accumulators), so that every operand
// read stays where the source puts it, two steps ahead of its MFMA; the first of a tile starts
// from a literal zero.  An MFMA that accumulates into exactly the registers the previous one
// wrote needs no wait states.
__device__ __forceinline__ void mfma_32x32x16_v0(f32x16& acc, bf16x8 a, bf16x8 b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b) : "memory");
}
__device__ __forceinline__ void mfma_32x32x16_v(f32x16& acc, bf16x8 a, bf16x8 b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b) : "memory");
}
__device__ __forceinline__ void hb_v_fence_after_mfma(f32x16& acc) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" : "+v"(acc));
}
__device__ __forceinline__ void hb_nops_valu_to_mfma() { asm volatile("s_nop 2"); }

// 16 bytes a lane from global memory (base + voff, base wave-uniform) straight into LDS at
// lds_addr + 16 * lane.  Written out so that the compiler does not see an LDS store in flight:
// otherwise it waits for every outstanding gather before each LDS read of the tile ring, which
// would serialise the ring.  The caller orders the DMA against the reads itself: a wave waits
// for its own gathers of a tile (vmcnt; loads complete in issue order) and a barrier follows.
// M0 holds the LDS address (one wait state between its write and the DMA); M0 is reserved to
// the compiler and cannot be declared clobbered, and nothing else in these kernels uses it (the
// LDS instructions of gfx950 do not read it).
//
// The row's base address comes from a lane of a vector register (v_readlane into an SGPR pair),
// and a vector memory instruction may read an SGPR written by a VALU instruction only 5 wait
// states later.  The compiler does not see the DMA's read, so the callers take every address
// (row_addr, which pins it in place) before the previous DMA of the sequence is issued: that
// DMA's three instructions and this one's M0 write and wait state make the 5.  The first DMA of
// a sequence has only the next address's two readlanes in between and waits 3 more (FIRST).
struct RowAddr {
  uint32_t lo, hi;
};
__device__ __forceinline__ RowAddr row_addr(uint64_t pv, int rr) {
  RowAddr a{static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<uint32_t>(pv), rr)),
            static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<uint32_t>(pv >> 32), rr))};
  asm volatile("" : : "s"(a.lo), "s"(a.hi));  // read here, ahead of the DMAs that precede its own
  return a;
}
template <bool FIRST = false>
__device__ __forceinline__ void lds_dma16(RowAddr a, uint32_t voff, uint32_t lds_addr) {
  const uint64_t base = (static_cast<uint64_t>(a.hi) << 32) | a.lo;
  if constexpr (FIRST)
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 3\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(voff), "s"(base), "s"(lds_addr));
  else
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(voff), "s"(base), "s"(lds_addr));
}
__device__ __forceinline__ void hb_acc_fence_after_mfma(f32x16 (&acc)[16]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3"
               : "+a"(acc[0]), "+a"(acc[1]), "+a"(acc[2]), "+a"(acc[3]), "+a"(acc[4]),
                 "+a"(acc[5]), "+a"(acc[6]), "+a"(acc[7]), "+a"(acc[8]), "+a"(acc[9]),
                 "+a"(acc[10]), "+a"(acc[11]), "+a"(acc[12]), "+a"(acc[13]), "+a"(acc[14]),
                 "+a"(acc[15]));
}
__device__ __forceinline__ void hb_acc_fence_before_mfma(f32x16 (&acc)[16]) {
  asm volatile("s_nop 2"
               : "+a"(acc[0]), "+a"(acc[1]), "+a"(acc[2]), "+a"(acc[3]), "+a"(acc[4]),
                 "+a"(acc[5]), "+a"(acc[6]), "+a"(acc[7]), "+a"(acc[8]), "+a"(acc[9]),
                 "+a"(acc[10]), "+a"(acc[11]), "+a"(acc[12]), "+a"(acc[13]), "+a"(acc[14]),
                 "+a"(acc[15]));
}

template <bool SPARSE, bool PAGED>
__global__ __launch_bounds__(MqaHbShape::NT) void mqa_hb_kernel(MqaParams p) {
  using SH = MqaHbShape;
  constexpr int NW = SH::NW, NT = SH::NT, C = SH::C, RPW = SH::RPW;
  constexpr uint32_t TB = SH::TB;
  constexpr bool LIST = SPARSE || PAGED;  // rows come from the span's list in s_idx
  typedef __attribute__((address_space(3))) unsigned char lds_uchar;
  extern __shared__ __align__(16) unsigned char smem[];
  float2* s_cs = reinterpret_cast<float2*>(smem + SH::off_cs);  // cos, sin of pair i at t
  int* s_idx = reinterpret_cast<int*>(smem + SH::lds_fixed());  // [split_rows] (LIST)

  const int tid = threadIdx.x;
  const int l = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = l >> 5, n32 = l & 31;
  mqa_preload_params(p);
  const int bid = blockIdx.x;
  int hg, split, row;
  mqa_work_item(p, bid, hg, split, row);
  if (row < 0) return;
  const int b = row / p.nq;
  const int j0 = split * p.split_rows;
  const int head = hg * SH::HPG + wave * SH::HPW + n32;
  const bool head_ok = head < p.n_heads;

  // ---- prologue loads, in the order they are needed: the span's first indices, the position
  // and entry count, sink and RoPE frequency, then the query slice
  int pre0 = 0, pre1 = 0;
  if constexpr (SPARSE) {
    const int32_t* ir = p.idx + static_cast<size_t>(row) * p.k;
    pre0 = ir[min(j0 + n32, p.k - 1)];
    pre1 = ir[min(j0 + 32 + n32, p.k - 1)];
  }
  // (both loads go out together through the vector path, first: one memory round trip before
  // the gathers, not two scalar round trips each behind a wait for every scalar load)
  int rv = p.pos ? row : b, bv = b;
  asm volatile("" : "+v"(rv), "+v"(bv));
  int t_vec = (p.pos ? p.pos : p.n_entries)[rv];
  int ne_vec = p.n_entries[bv];
  float freq_v = p.inv_freq[min(tid, (p.r >> 1) - 1)];
  asm volatile("" ::: "memory");  // the three small loads go out before the query's
  u32x4 qv[32];  // Q^T B operand: head n32, dims 16kk + 8h .. +7
  {
    const uint16_t* qrow = p.q + (static_cast<size_t>(row) * p.n_heads + (head_ok ? head : 0)) * C;
#pragma unroll
    for (int kk = 0; kk < 32; ++kk)
      qv[kk] = *reinterpret_cast<const u32x4*>(qrow + kk * 16 + h * 8);
  }
  // the three small loads are waited for here, once, after Q is requested and before the
  // gathers are (a later wait counted by the compiler would not know of the gathers)
  asm volatile("" : "+v"(t_vec), "+v"(ne_vec), "+v"(freq_v) : : "memory");
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

  const uint16_t* const ent_base =
      PAGED ? p.entries : p.entries + static_cast<size_t>(b) * p.n_max * C;
  const uint16_t* const win_base = p.window + static_cast<size_t>(b) * p.win_slots * C;
  const uint16_t* const safe_row = win_base + static_cast<size_t>(t % p.win_slots) * C;
  const int e_lim = PAGED ? 0x7fffffff : n_ent;  // PAGED lists hold pool rows (-1: masked)
  auto xlate = [&](int e) {
    return (e >= 0 && e < n_ent) ? static_cast<int>(entry_row(p.pages, p.n_max, b, e)) : -1;
  };
  // row pointer of list row j (lanes 0..31, one row each) and the tile's valid mask
  auto resolve_e = [&](int j, int e, const uint16_t*& ptr, uint32_t& mask) {
    const bool in_span = l < 32 && j < j1;
    const bool sel = j < n_sel;
    const bool ok_e = e >= 0 && e < e_lim;
    const int u = max(wlo + (j - n_sel), 0);
    const uint16_t* pe = ent_base + static_cast<size_t>(ok_e ? e : 0) * C;
    const uint16_t* pw = win_base + static_cast<size_t>(u % p.win_slots) * C;
    const bool ok = in_span && (!sel || ok_e);
    ptr = ok ? (sel ? pe : pw) : safe_row;
    mask = static_cast<uint32_t>(__ballot(ok));
  };
  auto resolve = [&](int jt, const uint16_t*& ptr, uint32_t& mask) {
    const int j = jt + n32;
    int e = j;
    if constexpr (LIST) e = s_idx[min(max(j - j0, 0), p.split_rows - 1)];
    resolve_e(j, e, ptr, mask);
  };
  // this wave's rows of a tile (rows wave, wave + NW, ...) straight into LDS buffer buf; logical
  // chunk c of row rr lands at chunk c ^ swz(rr)
  const uint32_t lds_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_uchar*)smem));
  auto addr_of = [&](const uint16_t* ptr, int q) {  // row wave + NW q of a tile
    return row_addr(reinterpret_cast<uint64_t>(ptr), wave + q * NW);
  };
  auto gload = [&](const uint16_t* ptr, int buf) {  // all of this wave's rows of a tile
    RowAddr a = addr_of(ptr, 0);
#pragma unroll
    for (int q = 0; q < RPW; ++q) {
      RowAddr nx = a;
      if (q + 1 < RPW) nx = addr_of(ptr, q + 1);
      const int rr = wave + q * NW;
      const uint32_t voff = static_cast<uint32_t>(l ^ swz(rr)) << 4;
      const uint32_t la = lds_base + static_cast<uint32_t>(buf) * TB + static_cast<uint32_t>(rr) * (C * 2);
      if (q == 0) lds_dma16<true>(a, voff, la);
      else lds_dma16(a, voff, la);
      a = nx;
    }
  };

  // tiles 0 and 1 are requested first (their indices read straight from global memory)
  const int ntiles = j1 > j0 ? (j1 - j0 + 31) / 32 : 0;
  uint32_t mk0 = 0, mk1 = 0, mk2 = 0, mk3 = 0;  // valid masks of tiles i .. i+3
  {
    const uint16_t* p0;
    const uint16_t* p1;
    int f0 = SPARSE ? pre0 : j0 + n32, f1 = SPARSE ? pre1 : j0 + 32 + n32;
    if constexpr (PAGED) {
      f0 = xlate(f0);
      f1 = xlate(f1);
    }
    resolve_e(j0 + n32, f0, p0, mk0);
    resolve_e(j0 + 32 + n32, f1, p1, mk1);
    if (ntiles > 0) gload(p0, 0);
    if (ntiles > 1) gload(p1, 1);
  }
  if constexpr (LIST) {
    const int e1 = min(j1, n_sel);
    for (int j = j0 + tid; j < e1; j += NT) {
      int v = SPARSE ? p.idx[static_cast<size_t>(row) * p.k + j] : j;
      if constexpr (PAGED) v = xlate(v);
      s_idx[j - j0] = v;
    }
  }
  if (tid < (p.r >> 1)) {
    float cs, sn;
    rope_cos_sin(t, freq_v, cs, sn);
    s_cs[tid] = float2{cs, sn};
  }
  __syncthreads();  // s_idx, s_cs

  // query fragments rotated at t on the RoPE dims
  // (rope_dim <= 128, so only the last 8 K steps can hold RoPE dims; branch-free selects)
  bf16x8 bq[32];
#pragma unroll
  for (int kk = 0; kk < 32; ++kk) {
    u32x4 raw = qv[kk];  // (a head past n_heads reads head 0: its outputs are never stored)
    if (kk >= 24) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int d = kk * 16 + h * 8 + 2 * jj;
        const int rel = d - (C - p.r);
        const float2 e = s_cs[max(rel, 0) >> 1];
        const float x0 = bf16_to_f32(static_cast<uint16_t>(raw[jj] & 0xffff));
        const float x1 = bf16_to_f32(static_cast<uint16_t>(raw[jj] >> 16));
        const uint32_t rot = pack2(x0 * e.x - x1 * e.y, x0 * e.y + x1 * e.x);
        raw[jj] = rel >= 0 ? rot : raw[jj];
      }
    }
    bq[kk] = as_bf16x8(raw);
  }

  // LDS byte offsets that do not change from tile to tile.  S (A operand): row n32, logical
  // chunk 2kk + h; kk = 8k' + kr adds 256 k' bytes to kr's offset (the swizzle stays within 16
  // chunks).  PV (transposed A operand): lane 4*i0 + q4 of 16-lane group G points at row
  // 4h + i0 (K slots 0..3) or 4h + i0 + 8 (slots 4..7), logical chunk 4dt + 2(G&1) + q4/2,
  // half q4&1; dt = 4k' + d' adds 256 k' bytes to d''s offset and step kb adds 16 rows.
  uint32_t sa_off[8];
#pragma unroll
  for (int kr = 0; kr < 8; ++kr)
    sa_off[kr] = static_cast<uint32_t>(n32 * C + (((2 * kr + h) ^ swz(n32)) << 3)) * 2u;
  const int G = l >> 4, i0 = (l & 15) >> 2, q4 = l & 3;
  const int ra = 4 * h + i0, rb = ra + 8;
  uint32_t ta_off[4], tb_off[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const int low = 4 * d + 2 * (G & 1) + (q4 >> 1);
    ta_off[d] = static_cast<uint32_t>(ra * C + ((low ^ swz(ra)) << 3) + 4 * (q4 & 1)) * 2u;
    tb_off[d] = static_cast<uint32_t>(rb * C + ((low ^ swz(rb)) << 3) + 4 * (q4 & 1)) * 2u;
  }
  constexpr uint32_t kStep16 = 16u * C * 2u;  // byte offset of rows 16..31

  f32x16 acc[16];  // O^T: acc[dt][4i + e] = dim 32dt + 8i + 4h + e of head n32
#pragma unroll
  for (int dt = 0; dt < 16; ++dt) acc[dt] = f32x16{};
  hb_acc_fence_before_mfma(acc);
  // online softmax of head n32 (log2 domain, scaled): the reference maximum moves only when a
  // logit exceeds it by more than 8; l_part sums this lane's probabilities (its 16 rows)
  float m_ref = -INFINITY, l_part = 0.f;

  // Operand reads: S step kk (row n32, dims 16kk + 8h..) and PV step k (kb = k / 16,
  // dt = k % 16: dims 32dt + l%32, K slots of rows 16kb + 4h + 0..3 and +8).
  auto read_s = [&](const unsigned char* Eb, int kk) {
    return as_bf16x8(*reinterpret_cast<const u32x4*>(Eb + sa_off[kk & 7] + (kk >> 3) * 256));
  };
  auto read_pv = [&](const unsigned char* Eb, int k) {
    const int dt = k & 15, kb = k >> 4;
    const uint32_t o = (dt >> 2) * 256 + kb * kStep16;
    const bf16x4 lo = lds_read_tr16(reinterpret_cast<const uint16_t*>(Eb + ta_off[dt & 3] + o));
    const bf16x4 hi = lds_read_tr16(reinterpret_cast<const uint16_t*>(Eb + tb_off[dt & 3] + o));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  };
  // PV of the last tile alone
  auto pv_only = [&](uint32_t bo, const bf16x8 (&P)[2]) {
    const unsigned char* Ep = smem + bo;
    bf16x8 t0 = read_pv(Ep, 0), t1 = read_pv(Ep, 1);
    hb_nops_valu_to_mfma();
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      bf16x8 t2 = t1;
      if (k + 2 < 32) t2 = read_pv(Ep, k + 2);
      mfma_32x32x16_agpr(acc[k & 15], t0, P[k >> 4]);
      t0 = t1;
      t1 = t2;
    }
  };
  // rescale of the output accumulators when some head's reference maximum moved up (rare)
  auto rescale = [&](float alpha) {
    if (__ballot(alpha != 1.f)) {  // wave-uniform branch
      hb_acc_fence_after_mfma(acc);
      // one 16-register block at a time: the fence ties block dt+1's reads to block dt's writes
#pragma unroll
      for (int dt = 0; dt < 16; ++dt) {
        acc[dt] *= alpha;
        if (dt + 1 < 16) asm volatile("" : "+a"(acc[dt]), "+a"(acc[dt + 1]));
      }
      hb_acc_fence_before_mfma(acc);
    }
  };

  {
    const uint16_t* pn2;
    const uint16_t* pn3;
    resolve(j0 + 64, pn2, mk2);
    bf16x8 Pprev[2] = {as_bf16x8(u32x4{0u, 0u, 0u, 0u}), as_bf16x8(u32x4{0u, 0u, 0u, 0u})};
    for (int i = 0; i < ntiles; ++i) {
      const uint32_t bo = static_cast<uint32_t>(i & 3) * TB;
      const uint32_t bo_prev = static_cast<uint32_t>((i + 3) & 3) * TB;
      // this wave's rows of tile i have landed (tile i+1's, when it exists, may still fly)
      if (i + 1 < ntiles) wait_vm<RPW>();
      else wait_vm<0>();
      __syncthreads();  // every wave's rows of tile i are in LDS; tile i-2's buffer is free
      // S of tile i with the PV of tile i-1 (its buffer is not refilled before i+3).  Tile 0 runs
      // the same code with P = 0 over its own rows, which are finite or attended anyway, so the
      // accumulators stay exactly zero (one code path keeps the registers within the file).
      const unsigned char* Eb = smem + bo;
      const unsigned char* Ep = smem + (i > 0 ? bo_prev : bo);
      const bool dma = i + 2 < ntiles;  // only tiles of the span are requested
      const int dbuf = (i + 2) & 3;
      bf16x8 t0 = read_pv(Ep, 0), t1 = read_pv(Ep, 1);
      // PV block j of the previous tile: operands read two blocks ahead
      auto pv_step = [&](int j) {
        bf16x8 t2 = t1;
        if (j + 2 < 32) t2 = read_pv(Ep, j + 2);
        mfma_32x32x16_agpr(acc[j & 15], t0, Pprev[j >> 4]);
        t0 = t1;
        t1 = t2;
        __builtin_amdgcn_sched_barrier(0);
      };
      // phase 1: tile i+2 requested, then the 32 K steps of S^T with PV blocks 0..15 after the
      // odd steps (the requests issued together at the start of the phase measured 4% faster per
      // tile than one after every fourth step)
      f32x16 sacc;
      {
        if (dma) gload(pn2, dbuf);
        bf16x8 s0 = read_s(Eb, 0), s1 = read_s(Eb, 1);
        hb_nops_valu_to_mfma();  // P was written by VALU code
#pragma unroll
        for (int k = 0; k < 32; ++k) {
          bf16x8 s2 = s1;
          if (k + 2 < 32) s2 = read_s(Eb, k + 2);
          if (k == 0) mfma_32x32x16_v0(sacc, s0, bq[0]);
          else mfma_32x32x16_v(sacc, s0, bq[k]);
          s0 = s1;
          s1 = s2;
          if (k & 1) pv_step(k >> 1);
        }
        hb_v_fence_after_mfma(sacc);
      }
      // phase 2: PV blocks 16..31 with the masked online softmax of tile i in stages between
      // them (element 4r + e of sacc is row 8r + 4h + e; P^T comes out in the K-slot order)
      float v[16], pr[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) v[e] = sacc[e];
      if (mk0 != 0xffffffffu) {  // a tile with masked rows (wave-uniform)
        const uint32_t mh = mk0 >> (4 * h);  // bit 8r + e: row 8r + 4h + e
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            v[4 * r + e] = ((mh >> (8 * r + e)) & 1u) ? v[4 * r + e] : -INFINITY;
      }
      // (each stage's results are pinned by an empty statement so that no stage moves past
      // the MFMA that follows it)
      float mx = fmaxf(fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])),
                       fmaxf(fmaxf(v[4], v[5]), fmaxf(v[6], v[7])));
      asm volatile("" : "+v"(mx));
      pv_step(16);
      mx = fmaxf(mx, fmaxf(fmaxf(fmaxf(v[8], v[9]), fmaxf(v[10], v[11])),
                           fmaxf(fmaxf(v[12], v[13]), fmaxf(v[14], v[15]))));
      mx = max_xor32(mx) * p.scale_log2;
      const bool move = mx > m_ref + 8.f;
      const float m_new = move ? mx : m_ref;
      // nothing summed yet (reference still -inf): the accumulators are zero, no rescale
      float alpha = (move && m_ref != -INFINITY) ? __builtin_amdgcn_exp2f(m_ref - m_new) : 1.f;
      float mu = (m_new == -INFINITY) ? 0.f : m_new;
      asm volatile("" : "+v"(alpha), "+v"(mu));
      pv_step(17);
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
#pragma unroll
        for (int e = 4 * g4; e < 4 * g4 + 4; ++e)
          pr[e] = __builtin_amdgcn_exp2f(fmaf(v[e], p.scale_log2, -mu));
        asm volatile("" : "+v"(pr[4 * g4]), "+v"(pr[4 * g4 + 1]), "+v"(pr[4 * g4 + 2]),
                     "+v"(pr[4 * g4 + 3]));
        pv_step(18 + g4);
      }
      float ls = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) ls += pr[e];
      l_part = l_part * alpha + ls;
      m_ref = m_new;
      bf16x8 Pn[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        Pn[kb] = as_bf16x8(u32x4{pack2(pr[8 * kb], pr[8 * kb + 1]),
                                 pack2(pr[8 * kb + 2], pr[8 * kb + 3]),
                                 pack2(pr[8 * kb + 4], pr[8 * kb + 5]),
                                 pack2(pr[8 * kb + 6], pr[8 * kb + 7])});
      asm volatile("" : "+v"(Pn[0]), "+v"(Pn[1]), "+v"(l_part));
      pv_step(22);
      resolve(j0 + (i + 3) * 32, pn3, mk3);
#pragma unroll
      for (int j = 23; j < 32; ++j) pv_step(j);
      rescale(alpha);  // after every PV MFMA of tile i-1
      Pprev[0] = Pn[0];
      Pprev[1] = Pn[1];
      pn2 = pn3;
      mk0 = mk1;
      mk1 = mk2;
      mk2 = mk3;
    }
    if (ntiles > 0) pv_only(static_cast<uint32_t>((ntiles - 1) & 3) * TB, Pprev);
  }
  hb_acc_fence_after_mfma(acc);
  __syncthreads();  // every wave is done with the ring before it stages the outputs

  // ---- epilogue: the span's partial (bf16 O / l) of this wave's 32 heads staged in tile
  // buffer `wave` and written as whole 1 KiB rows, and its (max, sum).  Staging position of
  // the 8 bytes (chunk c, half hf) of head row n: chunk c ^ ((n >> 1) & 15), half hf ^ (n & 1),
  // so the 32 lanes of one half-wave write 32 distinct 8-byte slots of every bank group.
  // (Stores of 8 bytes a lane straight from the registers took 70% longer: 32 rows a store.)
  const float l_tot = sum_xor32(l_part);
  const float il = l_tot > 0.f ? 1.f / l_tot : 0.f;  // the partial is O / l of the span
  const size_t hrow = static_cast<size_t>(p.head_groups) * SH::HPG;  // padded heads of a row
  // block (row, span, head group, wave) of the partials: [dt][i][lane][4 dims], every store
  // 512 contiguous bytes; element e of lane l in (dt, i) is head 32 wave + l % 32 of the group,
  // dim 32 dt + 8 i + 4 (l / 32) + e
  uint16_t* pw = reinterpret_cast<uint16_t*>(p.part) +
                 ((((static_cast<size_t>(row) * p.n_splits + split) * p.head_groups + hg) * NW +
                   wave) * (SH::HPW * C));
#pragma unroll
  for (int dt = 0; dt < 16; ++dt) {
    if (dt > 0) asm volatile("" : "+a"(acc[dt - 1]), "+a"(acc[dt]));  // one block at a time
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<uint2*>(pw + ((dt * 4 + i) * 64 + l) * 4) =
          uint2{pack2(acc[dt][4 * i] * il, acc[dt][4 * i + 1] * il),
                pack2(acc[dt][4 * i + 2] * il, acc[dt][4 * i + 3] * il)};
  }
  if (h == 0) {
    float* mlp = p.ml + ((static_cast<size_t>(row) * p.n_splits + split) * hrow + head) * 2;
    mlp[0] = m_ref;
    mlp[1] = l_tot;
  }
}

// Merge of the span partials of the head-block kernel: a thread takes dims 8c..8c+7 of one
// (row, head), i.e. the words of lanes n and n + 32 at step c = 4 dt + i of its partial blocks
// (consecutive threads take consecutive lanes, so a wave's loads are two 256-byte runs), merges
// the spans in order, adds the sink once, normalises, rotates back and stores bf16.  Loads of up
// to kHbCombineMax spans are in flight together, and the RoPE frequencies of the thread's dims go
// out with the first loads, so the rotation at the end waits for nothing.
constexpr int kHbCombineMax = 8;

__global__ __launch_bounds__(256) void mqa_combine_hb_kernel(MqaParams p, int rows) {
  constexpr int C = MqaHbShape::C, HPW = MqaHbShape::HPW, BLK = HPW * C;
  const int nblk = p.head_groups * MqaHbShape::NW;  // 32-head blocks of a row
  const size_t hrow = static_cast<size_t>(nblk) * HPW;
  const size_t gid = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  const int n = static_cast<int>(gid % HPW);
  const int c = static_cast<int>((gid / HPW) % (C / 8));
  const int blk = static_cast<int>((gid / (HPW * (C / 8))) % nblk);
  const int row = static_cast<int>(gid / (static_cast<size_t>(HPW) * (C / 8) * nblk));
  const int head = blk * HPW + n;
  mqa_preload_params(p);
  if (row >= rows || head >= p.n_heads) return;
  const int t_vec = mqa_position_request(p, row);  // needed only for the rotation at the end
  const int d0 = c * 8;
  float fq[4];  // frequencies of the thread's RoPE pairs, requested now (clamped, unused if unrotated)
#pragma unroll
  for (int pr2 = 0; pr2 < 4; ++pr2)
    fq[pr2] = p.inv_freq[max(0, min(d0 + 2 * pr2 - (C - p.r), p.r - 2)) >> 1];
  const uint16_t* pw = reinterpret_cast<const uint16_t*>(p.part) +
                       (static_cast<size_t>(row) * p.n_splits * nblk + blk) * BLK +
                       (c * 64 + n) * 4;
  const float* ml = p.ml + (static_cast<size_t>(row) * p.n_splits * hrow + head) * 2;
  const size_t pstride = static_cast<size_t>(nblk) * BLK, mstride = hrow * 2;
  // the sink is requested now and taken after the first pass's loads are out
  float sink_raw = *(p.sink ? p.sink + head : p.inv_freq);
  float sink2 = -INFINITY;
  SpanMerge sm = sm_start(-INFINITY);
  float o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = 0.f;
  for (int s0 = 0; s0 < p.n_splits; s0 += kHbCombineMax) {
    float mv[kHbCombineMax], lv[kHbCombineMax];
    uint2 ova[kHbCombineMax], ovb[kHbCombineMax];
#pragma unroll
    for (int j = 0; j < kHbCombineMax; ++j) {
      const int sp = min(s0 + j, p.n_splits - 1);
      mv[j] = s0 + j < p.n_splits ? ml[sp * mstride] : -INFINITY;
      lv[j] = ml[sp * mstride + 1];
      ova[j] = *reinterpret_cast<const uint2*>(pw + sp * pstride);
      ovb[j] = *reinterpret_cast<const uint2*>(pw + sp * pstride + 32 * 4);
    }
    if (s0 == 0) {
      asm volatile("" : "+v"(sink_raw) : : "memory");
      sink2 = p.sink ? sink_raw * kLog2e : -INFINITY;
      sm = sm_start(sink2);
    }
    float Mn = sm.M;
#pragma unroll
    for (int j = 0; j < kHbCombineMax; ++j) Mn = fmaxf(Mn, mv[j]);
    const float a = sm_raise(sm, Mn);
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] *= a;
#pragma unroll
    for (int j = 0; j < kHbCombineMax; ++j) {
      const float wgt = sm_add(sm, mv[j], lv[j]);  // partials are O / l
      if (mv[j] == -INFINITY) continue;
      const f32x4 va = unpack_b4(ova[j]), vb = unpack_b4(ovb[j]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        o[e] = sm_fold(o[e], va[e], wgt);
        o[4 + e] = sm_fold(o[4 + e], vb[e], wgt);
      }
    }
  }
  const float inv = sm_inv(sm, p.sink != nullptr, sink2);
  const int t = mqa_position_take(p, row, t_vec);
  float x[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = o[e] * inv;
#pragma unroll
  for (int pr2 = 0; pr2 < 4; ++pr2) {
    const int d = d0 + 2 * pr2;
    if (d >= C - p.r) {
      float cs, sn;
      rope_cos_sin(t, fq[pr2], cs, sn);
      rot_back(x[2 * pr2], x[2 * pr2 + 1], cs, sn);
    }
  }
  *reinterpret_cast<u32x4*>(p.out + (static_cast<size_t>(row) * p.n_heads + head) * C + d0) =
      u32x4{pack2(x[0], x[1]), pack2(x[2], x[3]), pack2(x[4], x[5]), pack2(x[6], x[7])};
  if (p.lse_out && c == 0) p.lse_out[static_cast<size_t>(row) * p.n_heads + head] = sm_lse(sm);
}

// ---------------------------------------------------------------- runs of queries (prefill)
// Two query rows per workgroup, one span each (the whole key list, up to kHbqMaxList rows):
// waves 2s and 2s+1 own heads 0..31 and 32..63 of query slot s over all 512 dims, with the same
// MFMA layout as the kernel above.  Each query has a ring of two tiles in LDS (tile i+1 is
// requested while tile i is computed: S^T, softmax, PV), so four waves work on two independent
// key lists with one barrier per step.  A query whose list has fewer tiles computes fully
// masked tiles in the remaining steps (no effect on its sums).  The output is merged with the
// sink and normalised (the combine's span-merge arithmetic for one span, folded into one factor
// per head), rotated back in place and leaves as whole 1 KiB rows.
struct MqaHbqShape {
  static constexpr int NW = 4, NT = 64 * NW, HPW = 32, QPW = 2, HPQ = 64;
  static constexpr int C = 512;
  static constexpr uint32_t TB = 32 * C * 2;   // bytes per tile
  static constexpr int RPW = 32 / 2;           // rows each wave requests per tile (2 a query)
  static constexpr size_t off_cs = 4 * TB;     // [2][64] cos/sin of the RoPE pairs at t
  static constexpr size_t lds_fixed() { return off_cs + 2 * 64 * sizeof(float2); }
};

template <bool SPARSE, bool PAGED>
__global__ __launch_bounds__(MqaHbqShape::NT) void mqa_hbq_kernel(MqaParams p) {
  using SH = MqaHbqShape;
  constexpr int NT = SH::NT, C = SH::C, RPW = SH::RPW;
  constexpr uint32_t TB = SH::TB;
  constexpr bool LIST = SPARSE || PAGED;
  typedef __attribute__((address_space(3))) unsigned char lds_uchar;
  extern __shared__ __align__(16) unsigned char smem[];

  const int tid = threadIdx.x;
  const int l = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qs = wave >> 1, hb = wave & 1;  // query slot, head block
  const int tq = tid & 127;                 // thread within the query slot's two waves
  const int h = l >> 5, n32 = l & 31;
  mqa_preload_params(p);
  const int rows = p.n_work;  // one span per query
  const int row0 = blockIdx.x * 2;
  if (row0 >= rows) return;
  const bool live = row0 + qs < rows;  // the slot past an odd row count mirrors the last row
  const int row = min(row0 + qs, rows - 1);
  const int b = row / p.nq;
  const int head = hb * SH::HPW + n32;
  const bool head_ok = head < p.n_heads;
  float2* s_cs = reinterpret_cast<float2*>(smem + SH::off_cs) + qs * 64;
  int* s_idx = reinterpret_cast<int*>(smem + SH::lds_fixed()) + qs * p.split_rows;

  int pre0 = 0;
  if constexpr (SPARSE) pre0 = p.idx[static_cast<size_t>(row) * p.k + min(n32, p.k - 1)];
  // position and entry count of both rows of the workgroup (the step count is the larger of
  // the two lists'), the query's index list (every load issued now, clamped into its k
  // indices, and stored to LDS once the list length is known: one round trip instead of one
  // per 128 indices), sink and RoPE frequency, then the query slice
  const int rowo = min(row0 + (qs ^ 1), rows - 1);
  int t_vec = mqa_position_request(p, row), to_vec = mqa_position_request(p, rowo);
  int ne_vec = p.n_entries[b], neo_vec = p.n_entries[rowo / p.nq];
  constexpr int IPT = kHbqMaxList / 128;  // index-list entries per thread of a query slot
  int idxv[IPT];
#pragma unroll
  for (int u = 0; u < IPT; ++u)
    idxv[u] = SPARSE ? p.idx[static_cast<size_t>(row) * p.k + min(tq + 128 * u, p.k - 1)] : 0;
  float sink_raw = *(p.sink ? p.sink + (head_ok ? head : 0) : p.inv_freq);
  float freq_v = p.inv_freq[min(tq, (p.r >> 1) - 1)];
  asm volatile("" ::: "memory");
  u32x4 qv[32];
  {
    const uint16_t* qrow = p.q + (static_cast<size_t>(row) * p.n_heads + (head_ok ? head : 0)) * C;
#pragma unroll
    for (int kk = 0; kk < 32; ++kk)
      qv[kk] = *reinterpret_cast<const u32x4*>(qrow + kk * 16 + h * 8);
  }
  asm volatile("" : "+v"(ne_vec), "+v"(neo_vec), "+v"(sink_raw), "+v"(freq_v) : : "memory");
#pragma unroll
  for (int u = 0; u < IPT; ++u) asm volatile("" : "+v"(idxv[u]) : : "memory");
  const int t = mqa_position_take(p, row, t_vec);
  const int to = mqa_position_take(p, rowo, to_vec);
  auto list_len = [&](int tt, int ne_raw) {  // n_sel + n_w of a row at position tt
    const int ne = max(0, min(ne_raw, p.n_max));
    int ns;
    if (SPARSE) {
      ns = p.k;
    } else {
      const long v = (static_cast<long>(tt) + 1) / p.m;
      ns = static_cast<int>(v < ne ? v : ne);
    }
    return ns + min(p.n_win, tt + 1);
  };
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
  const int R = min(n_sel + n_w, p.split_rows);
  const int R_o = min(list_len(to, __builtin_amdgcn_readfirstlane(neo_vec)), p.split_rows);
  const int ntiles = (max(R, R_o) + 31) / 32;  // steps of the workgroup

  const uint16_t* const ent_base =
      PAGED ? p.entries : p.entries + static_cast<size_t>(b) * p.n_max * C;
  const uint16_t* const win_base = p.window + static_cast<size_t>(b) * p.win_slots * C;
  const uint16_t* const safe_row = win_base + static_cast<size_t>(t % p.win_slots) * C;
  const int e_lim = PAGED ? 0x7fffffff : n_ent;
  auto xlate = [&](int e) {
    return (e >= 0 && e < n_ent) ? static_cast<int>(entry_row(p.pages, p.n_max, b, e)) : -1;
  };
  auto resolve_e = [&](int j, int e, const uint16_t*& ptr, uint32_t& mask) {
    const bool in_span = l < 32 && j < R;
    const bool sel = j < n_sel;
    const bool ok_e = e >= 0 && e < e_lim;
    const int u = max(wlo + (j - n_sel), 0);
    const uint16_t* pe = ent_base + static_cast<size_t>(ok_e ? e : 0) * C;
    const uint16_t* pw = win_base + static_cast<size_t>(u % p.win_slots) * C;
    const bool ok = in_span && (!sel || ok_e);
    ptr = ok ? (sel ? pe : pw) : safe_row;
    mask = static_cast<uint32_t>(__ballot(ok));
  };
  auto resolve = [&](int jt, const uint16_t*& ptr, uint32_t& mask) {
    const int j = jt + n32;
    int e = j;
    if constexpr (LIST) e = s_idx[min(max(j, 0), p.split_rows - 1)];
    resolve_e(j, e, ptr, mask);
  };
  // rows hb, hb + 2, .. of the slot's tile into the slot's buffer buf (rows of one query
  // split over its two waves)
  const uint32_t lds_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_uchar*)smem));
  auto gload = [&](const uint16_t* ptr, int buf) {
    const uint64_t pv = reinterpret_cast<uint64_t>(ptr);
    RowAddr a = row_addr(pv, hb);
#pragma unroll
    for (int q = 0; q < RPW; ++q) {
      const int rr = hb + 2 * q;
      RowAddr nx = a;
      if (q + 1 < RPW) nx = row_addr(pv, rr + 2);  // one DMA ahead of its own
      const uint32_t voff = static_cast<uint32_t>(l ^ swz(rr)) << 4;
      const uint32_t la = lds_base + static_cast<uint32_t>(qs * 2 + buf) * TB +
                          static_cast<uint32_t>(rr) * (C * 2);
      if (q == 0) lds_dma16<true>(a, voff, la);
      else lds_dma16(a, voff, la);
      a = nx;
    }
  };

  uint32_t mk = 0;  // valid mask of the tile being computed
  if (ntiles > 0) {
    const uint16_t* p0;
    int f0 = SPARSE ? pre0 : n32;
    if constexpr (PAGED) f0 = xlate(f0);
    resolve_e(n32, f0, p0, mk);
    gload(p0, 0);
  }
  if constexpr (LIST) {
    const int e1 = min(R, n_sel);
#pragma unroll
    for (int u = 0; u < IPT; ++u) {
      const int j = tq + 128 * u;
      if (j < e1) {
        int v = SPARSE ? idxv[u] : j;
        if constexpr (PAGED) v = xlate(v);
        s_idx[j] = v;
      }
    }
  }
  if (tq < (p.r >> 1)) {
    float cs, sn;
    rope_cos_sin(t, freq_v, cs, sn);
    s_cs[tq] = float2{cs, sn};
  }
  __syncthreads();  // s_idx, s_cs

  bf16x8 bq[32];
#pragma unroll
  for (int kk = 0; kk < 32; ++kk) {
    u32x4 raw = qv[kk];
    if (kk >= 24) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int d = kk * 16 + h * 8 + 2 * jj;
        const int rel = d - (C - p.r);
        const float2 e = s_cs[max(rel, 0) >> 1];
        const float x0 = bf16_to_f32(static_cast<uint16_t>(raw[jj] & 0xffff));
        const float x1 = bf16_to_f32(static_cast<uint16_t>(raw[jj] >> 16));
        const uint32_t rot = pack2(x0 * e.x - x1 * e.y, x0 * e.y + x1 * e.x);
        raw[jj] = rel >= 0 ? rot : raw[jj];
      }
    }
    bq[kk] = as_bf16x8(raw);
  }

  uint32_t sa_off[8];
#pragma unroll
  for (int kr = 0; kr < 8; ++kr)
    sa_off[kr] = static_cast<uint32_t>(n32 * C + (((2 * kr + h) ^ swz(n32)) << 3)) * 2u;
  const int G = l >> 4, i0 = (l & 15) >> 2, q4 = l & 3;
  const int ra = 4 * h + i0, rb = ra + 8;
  uint32_t ta_off[4], tb_off[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const int low = 4 * d + 2 * (G & 1) + (q4 >> 1);
    ta_off[d] = static_cast<uint32_t>(ra * C + ((low ^ swz(ra)) << 3) + 4 * (q4 & 1)) * 2u;
    tb_off[d] = static_cast<uint32_t>(rb * C + ((low ^ swz(rb)) << 3) + 4 * (q4 & 1)) * 2u;
  }
  constexpr uint32_t kStep16 = 16u * C * 2u;

  f32x16 acc[16];
#pragma unroll
  for (int dt = 0; dt < 16; ++dt) acc[dt] = f32x16{};
  hb_acc_fence_before_mfma(acc);
  float m_ref = -INFINITY, l_part = 0.f;

  auto read_s = [&](const unsigned char* Eb, int kk) {
    return as_bf16x8(*reinterpret_cast<const u32x4*>(Eb + sa_off[kk & 7] + (kk >> 3) * 256));
  };
  auto read_pv = [&](const unsigned char* Eb, int k) {
    const int dt = k & 15, kb = k >> 4;
    const uint32_t o = (dt >> 2) * 256 + kb * kStep16;
    const bf16x4 lo = lds_read_tr16(reinterpret_cast<const uint16_t*>(Eb + ta_off[dt & 3] + o));
    const bf16x4 hi = lds_read_tr16(reinterpret_cast<const uint16_t*>(Eb + tb_off[dt & 3] + o));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  };

  for (int i = 0; i < ntiles; ++i) {
    const unsigned char* Eb = smem + static_cast<uint32_t>(qs * 2 + (i & 1)) * TB;
    wait_vm<0>();     // this wave's rows of tile i have landed
    __syncthreads();  // both waves' rows of tile i are in LDS; tile i-1's buffer is free
    uint32_t mk_next = 0;
    if (i + 1 < ntiles) {
      const uint16_t* pn;
      resolve((i + 1) * 32, pn, mk_next);
      gload(pn, (i + 1) & 1);
    }
    // S^T of tile i, operands two steps ahead
    f32x16 sacc;
    {
      bf16x8 s0 = read_s(Eb, 0), s1 = read_s(Eb, 1);
#pragma unroll
      for (int k = 0; k < 32; ++k) {
        bf16x8 s2 = s1;
        if (k + 2 < 32) s2 = read_s(Eb, k + 2);
        if (k == 0) mfma_32x32x16_v0(sacc, s0, bq[0]);
        else mfma_32x32x16_v(sacc, s0, bq[k]);
        s0 = s1;
        s1 = s2;
      }
      hb_v_fence_after_mfma(sacc);
    }
    // the first PV operands go out while the softmax runs
    bf16x8 t0 = read_pv(Eb, 0), t1 = read_pv(Eb, 1);
    float v[16], pr[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) v[e] = sacc[e];
    if (mk != 0xffffffffu) {  // a tile with masked rows (wave-uniform)
      const uint32_t mh = mk >> (4 * h);
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          v[4 * r + e] = ((mh >> (8 * r + e)) & 1u) ? v[4 * r + e] : -INFINITY;
    }
    float mx = v[0];
#pragma unroll
    for (int e = 1; e < 16; ++e) mx = fmaxf(mx, v[e]);
    mx = max_xor32(mx) * p.scale_log2;
    const bool move = mx > m_ref + 8.f;
    const float m_new = move ? mx : m_ref;
    // nothing summed yet (reference still -inf): the accumulators are zero, no rescale
    const float alpha = (move && m_ref != -INFINITY) ? __builtin_amdgcn_exp2f(m_ref - m_new) : 1.f;
    const float mu = (m_new == -INFINITY) ? 0.f : m_new;
#pragma unroll
    for (int e = 0; e < 16; ++e) pr[e] = __builtin_amdgcn_exp2f(fmaf(v[e], p.scale_log2, -mu));
    float ls = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) ls += pr[e];
    l_part = l_part * alpha + ls;
    m_ref = m_new;
    bf16x8 P[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
      P[kb] = as_bf16x8(u32x4{pack2(pr[8 * kb], pr[8 * kb + 1]), pack2(pr[8 * kb + 2], pr[8 * kb + 3]),
                              pack2(pr[8 * kb + 4], pr[8 * kb + 5]),
                              pack2(pr[8 * kb + 6], pr[8 * kb + 7])});
    if (__ballot(alpha != 1.f)) {  // some head's reference moved up: rescale what was summed
      hb_acc_fence_after_mfma(acc);
#pragma unroll
      for (int dt = 0; dt < 16; ++dt) {
        acc[dt] *= alpha;
        if (dt + 1 < 16) asm volatile("" : "+a"(acc[dt]), "+a"(acc[dt + 1]));
      }
      hb_acc_fence_before_mfma(acc);
    }
    // PV of tile i (kb-major: the two MFMAs into one block are 16 apart)
    hb_nops_valu_to_mfma();  // P was just written by VALU code
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      bf16x8 t2 = t1;
      if (k + 2 < 32) t2 = read_pv(Eb, k + 2);
      mfma_32x32x16_agpr(acc[k & 15], t0, P[k >> 4]);
      t0 = t1;
      t1 = t2;
    }
    mk = mk_next;
  }
  hb_acc_fence_after_mfma(acc);
  __syncthreads();  // every wave is done with the rings before it stages its outputs

  // ---- epilogue: the span merged with the sink (the combine's arithmetic for one span: the
  // weight of the span and the normalisation by the sum with the sink's term, folded into one
  // factor per head), the rotation back on the RoPE dims (the last four blocks: rope_dim <=
  // 128), staged in tile buffer `wave` (chunk c of head row n at c ^ ((n >> 1) & 15), halves
  // swapped for odd n) and written as whole 1 KiB rows
  const float l_tot = sum_xor32(l_part);
  const float il = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const float a2 = (p.sink && head_ok) ? sink_raw * kLog2e : -INFINITY;
  SpanMerge sm = sm_start(a2);
  sm_raise(sm, fmaxf(sm.M, m_ref));
  const float wgt = sm_add(sm, m_ref, l_tot);
  const float inv = sm_inv(sm, p.sink != nullptr, a2);
  const float fsc = il * wgt * inv;  // O -> output
  const int rope0 = C - p.r;
  unsigned char* so = smem + wave * TB;
  const int sw_c = (n32 >> 1) & 15, sw_h = h ^ (n32 & 1);
#pragma unroll
  for (int dt = 0; dt < 16; ++dt) {
    if (dt > 0) asm volatile("" : "+a"(acc[dt - 1]), "+a"(acc[dt]));  // one block at a time
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float x[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = acc[dt][4 * i + e] * fsc;
      if (dt >= 12) {
#pragma unroll
        for (int pr2 = 0; pr2 < 2; ++pr2) {
          const int d = dt * 32 + i * 8 + 4 * h + 2 * pr2;
          const float2 e = s_cs[max(d - rope0, 0) >> 1];
          float y0 = x[2 * pr2], y1 = x[2 * pr2 + 1];
          rot_back(y0, y1, e.x, e.y);
          x[2 * pr2] = d >= rope0 ? y0 : x[2 * pr2];
          x[2 * pr2 + 1] = d >= rope0 ? y1 : x[2 * pr2 + 1];
        }
      }
      const int c = 4 * dt + i;
      *reinterpret_cast<uint2*>(so + n32 * (C * 2) + ((c ^ sw_c) << 4) + (sw_h << 3)) =
          uint2{pack2(x[0], x[1]), pack2(x[2], x[3])};
    }
  }
  if (live && p.lse_out && head_ok && h == 0)
    p.lse_out[static_cast<size_t>(row) * p.n_heads + head] = sm_lse(sm);
  __syncthreads();
  const int head0 = hb * SH::HPW;
  const int n_rows = live ? min(SH::HPW, p.n_heads - head0) : 0;
  uint16_t* obase = p.out + (static_cast<size_t>(row) * p.n_heads + head0) * C;
  // eight rows at a time: their LDS reads all issued before the first store
#pragma unroll 1
  for (int n0 = 0; n0 < n_rows; n0 += 8) {
    u32x4 w4[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int n = min(n0 + u, n_rows - 1);
      w4[u] = *reinterpret_cast<const u32x4*>(so + n * (C * 2) + ((l ^ ((n >> 1) & 15)) << 4));
      if (n & 1) w4[u] = u32x4{w4[u][2], w4[u][3], w4[u][0], w4[u][1]};
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (n0 + u < n_rows)
        *reinterpret_cast<u32x4*>(obase + static_cast<size_t>(n0 + u) * C + l * 8) = w4[u];
  }
}

template <bool SPARSE, bool PAGED>
static hipError_t launch_hbq_t(const MqaParams& prm, int rows, hipStream_t s) {
  using SH = MqaHbqShape;
  if (prm.n_splits != 1 || prm.split_rows > kHbqMaxList || prm.n_heads > SH::HPQ)
    return hipErrorInvalidValue;
  const size_t lds = SH::lds_fixed() +
                     ((SPARSE || PAGED) ? 2 * static_cast<size_t>(prm.split_rows) * sizeof(int) : 0);
  hipError_t e = ensure_max_lds(reinterpret_cast<const void*>(mqa_hbq_kernel<SPARSE, PAGED>), lds);
  if (e != hipSuccess) return e;
  MqaParams q = prm;
  q.n_work = rows;
  ProfScope ps(SPARSE ? "mqa_sparse" : "mqa_dense", s);
  mqa_hbq_kernel<SPARSE, PAGED><<<static_cast<unsigned>((rows + 1) / 2), SH::NT, lds, s>>>(q);
  return hipGetLastError();
}

hipError_t launch_mqa_hbq(const MqaParams& prm, int rows, hipStream_t s) {
  const bool paged = prm.pages.table != nullptr;
  if (prm.idx) return paged ? launch_hbq_t<true, true>(prm, rows, s) : launch_hbq_t<true, false>(prm, rows, s);
  return paged ? launch_hbq_t<false, true>(prm, rows, s) : launch_hbq_t<false, false>(prm, rows, s);
}

template <bool SPARSE, bool PAGED>
static hipError_t launch_hb_t(const MqaParams& prm, int rows, hipStream_t s) {
  using SH = MqaHbShape;
  const size_t lds =
      SH::lds_fixed() + ((SPARSE || PAGED) ? static_cast<size_t>(prm.split_rows) * sizeof(int) : 0);
  if (prm.n_splits < 2) return hipErrorInvalidValue;  // the kernel writes span partials only
  hipError_t e = ensure_max_lds(reinterpret_cast<const void*>(mqa_hb_kernel<SPARSE, PAGED>), lds);
  if (e != hipSuccess) return e;
  MqaParams q = prm;
  q.n_work = rows * prm.n_splits;
  const unsigned grid = mqa_grid(rows, prm.n_splits, prm.head_groups);
  {
    ProfScope ps(SPARSE ? "mqa_sparse" : "mqa_dense", s);
    mqa_hb_kernel<SPARSE, PAGED><<<grid, SH::NT, lds, s>>>(q);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  ProfScope ps("mqa_combine", s);
  const size_t threads = static_cast<size_t>(rows) * prm.head_groups * SH::HPG * (SH::C / 8);
  mqa_combine_hb_kernel<<<static_cast<unsigned>((threads + 255) / 256), 256, 0, s>>>(prm, rows);
  return hipGetLastError();
}

hipError_t launch_mqa_hb(const MqaParams& prm, int rows, hipStream_t s) {
  const bool paged = prm.pages.table != nullptr;
  if (prm.idx) return paged ? launch_hb_t<true, true>(prm, rows, s) : launch_hb_t<true, false>(prm, rows, s);
  return paged ? launch_hb_t<false, true>(prm, rows, s) : launch_hb_t<false, false>(prm, rows, s);
}

}  // namespace csa
