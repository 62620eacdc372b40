// Lightning indexer scoring and exact top-k selection for gfx950.
//
// Method: "DeepSeek V4 模型技术大全", chapter "Attention", section "CSA 的完整路径":
//   I_{t,s} = sum_h w^I_{t,h} ReLU(q^I_{t,h} . K^IComp_s)  for s < floor((t+1)/m),
//   I_t = TopK_k { I_{t,s} }.
// Operands are E4M3 codes with float32 scales; since the scales are positive,
//   w_h ReLU(sq_h sk_s x) = sk_s (w_h sq_h) ReLU(x),
// so the MFMA works on raw codes and the epilogue applies (w_h sq_h) per head and sk_s per entry.
//
// The indexer query may be MXFP4 too (both operands FP4: E2M1 codes with an E8M0 scale per 32
// dims on each side, applied inside the scaled MFMA).  Scores may be stored as fp32 or, rounded
// to nearest even, as bf16 ("index scores FP32 -> BF16"); the top-k then ranks the bf16 values.
//
// Top-k is exact with the lower index winning ties.  Scores become order-preserving 32-bit
// keys.  Rows of up to 32768 entries use one workgroup per row with the keys in registers or
// LDS: a sampled threshold, an exact select among the few candidates above it (or a radix
// select) and an index-ordered compaction that emits the selection sorted.  Longer rows
// (decode at long context, few rows) are cut into 4096-entry chunks, one workgroup each,
// that share a sampled threshold and write their candidates; the last workgroup of a row selects
// among them and emits the selection in ascending index order.
#include "common.h"
#include "kernels.h"

#ifndef CSA_STREAM_LOAD
#define CSA_STREAM_LOAD(p) __builtin_nontemporal_load(p)
#endif

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
  static __device__ __forceinline__ void put4(uint16_t* r, int e, f32x4 v) {
    *reinterpret_cast<uint2*>(r + e) = uint2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
  }
};

// ============================================================================ scoring
// One workgroup scores `chunk` consecutive entries of one query row.  Each wave takes 16-entry
// tiles; a tile is an MFMA with the indexer heads as the M dimension (A operand, resident in
// registers for the whole chunk) and 16 entries as N (B operand, streamed from HBM).
// MX = true: the keys are MXFP4 (E2M1 codes, E8M0 scale per 32 dims).  The scaled MFMA takes
// the query as E4M3 and the keys as FP4 with each lane's block scale; its FP4 operand gives
// lane group g the 32 dims 32g..32g+31 (16 contiguous bytes of the packed key), while its FP8
// operand gives lane group g dims 16g..16g+15 and 64+16g..64+16g+15 (both checked on the GPU).
// PAGED: keys and scales live in a block pool (blocks of >= 16 entries, so a 16-entry tile lies
// in one block); each tile's block comes from one scalar-cache load of the block table.
// QX (with MX): the query is MXFP4 too, the scaled MFMA's FP4 A operand: lane group g takes dims
// 32g..32g+31 of its head (16 bytes of the packed row) and that block's E8M0 scale byte.
// ST: the score type written (float, or uint16_t for bf16 scores).
template <int DI, int HT, int TPW, bool MX = false, bool PAGED = false, bool QX = false,
          typename ST = float>
__global__ __launch_bounds__(256) void index_score_kernel(
    const uint8_t* __restrict__ qi, const float* __restrict__ qi_scale,
    const float* __restrict__ wi, const uint8_t* __restrict__ keys,
    const float* __restrict__ kscale, const int32_t* __restrict__ n_entries,
    const int32_t* __restrict__ pos, int nq, int n_max, int H_I, int m, int chunk,
    ST* __restrict__ scores, int sstride, int nchunks, PageMap pm) {
  static_assert(!QX || MX, "an FP4 query is paired with FP4 keys");
  constexpr int KB = DI / 4;   // key bytes per lane (its lane group's K slice)
  constexpr int KK = DI / 32;  // 8-byte MFMA steps per slice

  const int row = blockIdx.x / nchunks;
  const int b = row / nq;
  const int e0 = (blockIdx.x % nchunks) * chunk;
  const int tid = threadIdx.x;
  const int l = lane_id(), g = l >> 4, c16 = l & 15, wave = tid >> 6;

  // A operand: query codes of head ht*16 + c16, K slice g.  For DI = 128 (one 16x16x128 MFMA
  // per head tile) lane group g holds bytes 16g..16g+15 and 64+16g..64+16g+15 of the row, and
  // of each key: the four lane groups of an entry then read 64 contiguous bytes per load.
  // Other DI: bytes 32g.. in 8-byte steps of 16x16x32 MFMAs.
  constexpr bool kWide = DI == 128 || MX;
  // E4M3 keys of 128 bytes are loaded as whole 128-byte lines: in each of two loads, lanes
  // 8i..8i+7 take the eight 16-byte chunks of one entry (entries i and 8+i of the 16-entry
  // tile), then two rounds of lane permutes (ds_bpermute) regroup them so that lane (g, n) holds
  // bytes 32g..32g+31 of entry n, the MFMA's B layout.  (Loading each lane's own 32 bytes
  // directly touches every line from two instructions: 13% slower at 128K.)
  constexpr bool kLine = DI == 128 && !MX;
  constexpr int KROW = MX ? DI / 2 : DI;  // key bytes per entry
  constexpr int NBLK = DI / 32;           // MXFP4 blocks per key
  i32x8 aw[HT];
  long aq[HT][KK];
  float wq[HT][4];
  int sq[HT];  // QX: this lane's query block scale (E8M0)
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    const int head = ht * 16 + c16;
    sq[ht] = 127;
    if constexpr (QX) {  // packed E2M1 row of DI/2 bytes; blocks past DI are zero codes
      const size_t rh = static_cast<size_t>(row) * H_I + (head < H_I ? head : 0);
      const u32x4 v = (head < H_I && g < NBLK)
                          ? reinterpret_cast<const u32x4*>(qi + rh * (DI / 2))[g]
                          : u32x4{0, 0, 0, 0};
      aw[ht] = i32x8{static_cast<int>(v[0]), static_cast<int>(v[1]), static_cast<int>(v[2]),
                     static_cast<int>(v[3]), 0, 0, 0, 0};
      if (head < H_I && g < NBLK)
        sq[ht] = static_cast<int>((reinterpret_cast<const uint32_t*>(qi_scale)[rh] >> (8 * g)) &
                                  0xffu);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int hh = ht * 16 + g * 4 + i;
        wq[ht][i] = hh < H_I ? wi[static_cast<size_t>(row) * H_I + hh] : 0.f;  // scale in MFMA
      }
      continue;
    }
    const uint8_t* qrow = qi + (static_cast<size_t>(row) * H_I + (head < H_I ? head : 0)) * DI;
    const uint8_t* src = qrow + g * KB;
    if constexpr (kWide) {  // dims past DI (MXFP4 with DI < 128) are zero
      // E4M3 keys: lane group g takes bytes 32g..32g+31 (chunks 2g, 2g+1; see kLine below);
      // MXFP4: the FP8 operand order the scaled MFMA pairs with the FP4 keys (chunks g, 4+g)
      const u32x4* q16 = reinterpret_cast<const u32x4*>(qrow);
      const int c0 = kLine ? 2 * g : g, c1 = kLine ? 2 * g + 1 : 4 + g;
      const u32x4 lo = (head < H_I && c0 < DI / 16) ? q16[c0] : u32x4{0, 0, 0, 0};
      const u32x4 hi = (head < H_I && c1 < DI / 16) ? q16[c1] : u32x4{0, 0, 0, 0};
      aw[ht] = i32x8{static_cast<int>(lo[0]), static_cast<int>(lo[1]), static_cast<int>(lo[2]),
                     static_cast<int>(lo[3]), static_cast<int>(hi[0]), static_cast<int>(hi[1]),
                     static_cast<int>(hi[2]), static_cast<int>(hi[3])};
    } else {
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        aq[ht][kk] = head < H_I ? reinterpret_cast<const long*>(src)[kk] : 0;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hh = ht * 16 + g * 4 + i;
      wq[ht][i] = hh < H_I ? wi[static_cast<size_t>(row) * H_I + hh] *
                                 qi_scale[static_cast<size_t>(row) * H_I + hh]
                           : 0.f;
    }
  }

  const size_t seq0 = PAGED ? 0 : static_cast<size_t>(b) * n_max;  // row of entry 0
  const uint8_t* kbase = keys + seq0 * KROW + (kWide ? 0 : g * KB);
  const float* sbase = kscale + seq0;
  const uint32_t* swbase = reinterpret_cast<const uint32_t*>(sbase);  // MXFP4 scale bytes
  ST* srow = scores + static_cast<size_t>(row) * sstride;

  // Wave `wave` scores tiles wave, wave+4, ... (TPW tiles of 16 entries).  The sequence is
  // fully unrolled straight-line code with PD tiles in flight; loads are unconditional (past
  // the end they re-read the last visible entry, whose extra scores are never stored), so the
  // compiler waits for exactly the tile it is about to use.
  auto tile_entry = [&](int t) { return e0 + (wave + 4 * t) * 16 + c16; };
  struct KeyTile {
    i32x8 w;
    u32x4 p, q;  // kLine: the two whole-line loads, arranged for the two permute rounds
    long n[KK];
    float ks;
    uint32_t sw;
  };
  // kLine regroup.  Load X: lane s holds chunk s%8 of entry s/8; load Y: chunk (s%8)^1 of entry
  // 8 + s/8.  Even lanes offer (X, Y), odd lanes (Y, X) to rounds 1 and 2: target lane (g, n)
  // reads round 1 from lane 8(n%8) + 2g + (n >= 8) and round 2 from lane 8(n%8) + 2g + (n < 8),
  // which yields chunks 2g and 2g+1 of entry n for every n.
  const int n8 = c16 & 7, hiN = c16 >> 3;
  const int perm1 = (8 * n8 + 2 * g + hiN) * 4, perm2 = (8 * n8 + 2 * g + (hiN ^ 1)) * 4;
  auto load = [&](int t, KeyTile& kt, int emax) {
    const int el = min(tile_entry(t), emax);
    size_t e = el;
    if constexpr (PAGED) {  // the tile's entries (clamped ones included) share one block
      const int tb = min(e0 + (wave + 4 * t) * 16, emax & ~15);
      e = block_base_uniform(pm, b, tb >> pm.shift) + (el & ((1 << pm.shift) - 1));
    }
    if constexpr (MX) {
      const u32x4* src = reinterpret_cast<const u32x4*>(kbase + static_cast<size_t>(e) * KROW);
      const u32x4 v = g < NBLK ? CSA_STREAM_LOAD(src + g) : u32x4{0, 0, 0, 0};
      kt.w = i32x8{static_cast<int>(v[0]), static_cast<int>(v[1]), static_cast<int>(v[2]),
                   static_cast<int>(v[3]), 0, 0, 0, 0};
      kt.sw = swbase[e];
      return;
    } else if constexpr (kLine) {
      // rows of entries tb + s/8 and tb + 8 + s/8 of this tile (clamped like el)
      const int tb = min(e0 + (wave + 4 * t) * 16, emax & ~15);
      const int ex = min(tb + (l >> 3), emax), ey = min(tb + 8 + (l >> 3), emax);
      size_t rx = ex, ry = ey;
      if constexpr (PAGED) {
        const size_t base = e - (el & ((1 << pm.shift) - 1)) + (tb & ((1 << pm.shift) - 1)) - tb;
        rx = base + ex;
        ry = base + ey;
      }
      const u32x4 X = CSA_STREAM_LOAD(reinterpret_cast<const u32x4*>(kbase + rx * DI) + (l & 7));
      const u32x4 Y =
          CSA_STREAM_LOAD(reinterpret_cast<const u32x4*>(kbase + ry * DI) + ((l & 7) ^ 1));
      kt.p = (l & 1) ? Y : X;
      kt.q = (l & 1) ? X : Y;
    } else if constexpr (kWide) {
      const u32x4* src = reinterpret_cast<const u32x4*>(kbase + static_cast<size_t>(e) * DI);
      const u32x4 lo = CSA_STREAM_LOAD(src + g), hi = CSA_STREAM_LOAD(src + 4 + g);
      kt.w = i32x8{static_cast<int>(lo[0]), static_cast<int>(lo[1]), static_cast<int>(lo[2]),
                   static_cast<int>(lo[3]), static_cast<int>(hi[0]), static_cast<int>(hi[1]),
                   static_cast<int>(hi[2]), static_cast<int>(hi[3])};
    } else {
      const long* src = reinterpret_cast<const long*>(kbase + static_cast<size_t>(e) * DI);
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) kt.n[kk] = CSA_STREAM_LOAD(src + kk);
    }
    kt.ks = sbase[e];
  };
  auto compute = [&](int t, const KeyTile& kt, int e1) {
    f32x4 acc[HT];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) acc[ht] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (MX) {
      // this lane's block scale (unit for the zero blocks past DI)
      const int sb = g < NBLK ? static_cast<int>((kt.sw >> (8 * g)) & 0xffu) : 127;
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) {
        if constexpr (QX)
          acc[ht] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aw[ht], kt.w, acc[ht], 4, 4,
                                                                     0, sq[ht], 0, sb);
        else
          acc[ht] = mfma_fp8_fp4_16x16x128(aw[ht], kt.w, acc[ht], sb);
      }
    } else if constexpr (kLine) {
      i32x8 w;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        w[k] = __builtin_amdgcn_ds_bpermute(perm1, static_cast<int>(kt.p[k]));
        w[4 + k] = __builtin_amdgcn_ds_bpermute(perm2, static_cast<int>(kt.q[k]));
      }
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) acc[ht] = mfma_fp8_16x16x128(aw[ht], w, acc[ht]);
    } else if constexpr (kWide) {
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) acc[ht] = mfma_fp8_16x16x128(aw[ht], kt.w, acc[ht]);
    } else {
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) acc[ht] = mfma_fp8_16x16x32(aq[ht][kk], kt.n[kk], acc[ht]);
    }
    // ReLU as a signed integer max of the float's bits with 0 (one instruction)
    float part = 0.f;
#pragma unroll
    for (int ht = 0; ht < HT; ++ht)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        part = fmaf(wq[ht][i], __int_as_float(max(__float_as_int(acc[ht][i]), 0)), part);
    part = wave_sum_xor16_32(part);
    const int e = tile_entry(t);
    if (g == 0 && e < e1) {
      const float sc = MX ? part : part * kt.ks;  // MXFP4 scales act inside the MFMA
      Scores<ST>::put(srow, e, sc);
    }
  };
  // The first tiles are loaded before the row's visible length is known (clamped to the
  // allocated entries; scores past the visible end are never stored), so no wave waits for
  // the position and entry-count loads before its first key loads.
  constexpr int PD = 3, NB = PD + 1;  // a spare buffer: tile t+PD's loads go out before tile t
  KeyTile kb[NB];                      // is computed
#pragma unroll
  for (int t = 0; t < PD; ++t) load(t, kb[t], n_max - 1);
  const int n_vis = visible(n_entries, pos, row, nq, m, n_max);
  const int e1 = min(n_vis, e0 + chunk);
  if (e0 < e1) {
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      if (t + PD < TPW) load(t + PD, kb[(t + PD) % NB], e1 - 1);
      compute(t, kb[t % NB], e1);
    }
  }
}
// ============================================================================ scoring, many rows
// Prefill: many query rows share the keys, so scoring is a batched product over heads.  A
// workgroup takes 16 consecutive query rows of one sequence and holds their indexer queries
// (all heads, E4M3 codes) in LDS.  Each wave takes groups of 64 entries, four 16-entry blocks
// held in registers as A operands, and for every head h reads the 16 queries' codes of h once
// (B operand) for four 16x16x128 MFMAs, one per block (K = 128: one head's whole product):
//   D[entry][query] = K_e . Q_{q,h}                    (raw codes, exact in fp32)
//   acc[entry][query] += max(D, 0) * (w_{q,h} sq_{q,h})
// then multiplies by the entry scale sk_e.  The next group's keys and scales are loaded while
// the current one is computed.
constexpr int kGemmQ = 16;   // query rows per workgroup
constexpr int kGemmWaves = 8;  // two waves per SIMD: one's epilogue overlaps another's MFMAs
constexpr int kGemmThreads = 64 * kGemmWaves;
constexpr int kGemmH = 64;   // largest head count held in LDS
constexpr int kGemmDI = 128;
// LDS: query codes [h][q][128 B], head factors [h][q] fp32, query block scales [h][q] (4 E8M0
// bytes, FP4 queries), visible counts [q]
constexpr size_t kGemmLds = kGemmH * kGemmQ * kGemmDI + 2 * kGemmH * kGemmQ * 4 + kGemmQ * 4;

// 16-byte chunk swizzle of the query rows in LDS: the 16 queries read at one chunk position
// land in 16 distinct bank groups (rows are 128 bytes apart).
__device__ __forceinline__ int qswz(int q) { return (q >> 1) & 7; }

// MX = true: MXFP4 keys as the FP4 A operand (lane group g: dims 32g..32g+31, the lane's block
// scale); the query codes then go in the FP8 operand's order (lane group g: dims 16g..16g+15 and
// 64+16g..64+16g+15, i.e. 16-byte chunks g and 4+g of the query row).
// PAGED: keys and scales in a block pool (blocks of >= 16 entries); each 16-entry block's pool
// block comes from a scalar-cache load of the block table.
// QX (with MX): the queries are MXFP4 too, the scaled MFMA's FP4 B operand (lane group g: dims
// 32g..32g+31 of the query's head, i.e. 16-byte chunk g of its 64-byte packed row, and that
// block's E8M0 scale byte).  ST: the score type written (float, or uint16_t for bf16 scores).
template <bool MX, bool PAGED = false, bool QX = false, typename ST = float>
__global__ __launch_bounds__(kGemmThreads) void index_gemm_kernel(
    const uint8_t* __restrict__ qi, const float* __restrict__ qi_scale,
    const float* __restrict__ wi, const uint8_t* __restrict__ keys,
    const float* __restrict__ kscale, const int32_t* __restrict__ n_entries,
    const int32_t* __restrict__ pos, int nq, int n_max, int H_I, int m, int qtiles,
    ST* __restrict__ scores, int sstride, PageMap pm) {
  static_assert(!QX || MX, "an FP4 query is paired with FP4 keys");
  constexpr int DI = kGemmDI;
  constexpr int KROW = MX ? DI / 2 : DI;  // key bytes per entry
  constexpr int QROW = QX ? DI / 2 : DI;  // query bytes per head
  extern __shared__ __align__(16) unsigned char smem[];
  uint8_t* s_q = smem;                                                   // [h][q][128] swizzled
  float* s_c = reinterpret_cast<float*>(smem + kGemmH * kGemmQ * DI);    // [h][q]: w * sq
  uint32_t* s_qs = reinterpret_cast<uint32_t*>(s_c + kGemmH * kGemmQ);   // [h][q]: E8M0 x 4
  int* s_nv = reinterpret_cast<int*>(s_qs + kGemmH * kGemmQ);            // [q]: visible entries
  // causal rows: the last query tiles carry the most entries and are dispatched first
  const int b = blockIdx.x / qtiles;
  const int t0 = (qtiles - 1 - blockIdx.x % qtiles) * kGemmQ;
  const int tid = threadIdx.x, l = lane_id(), wave = tid >> 6;
  const int g = l >> 4, c16 = l & 15;

  constexpr int QCH = QROW / 16;  // 16-byte chunks of a query head
  for (int ch = tid; ch < H_I * kGemmQ * QCH; ch += kGemmThreads) {
    const int h = ch / (kGemmQ * QCH), q = (ch / QCH) % kGemmQ, c = ch % QCH;
    u32x4 v = u32x4{0, 0, 0, 0};
    if (t0 + q < nq)
      v = *reinterpret_cast<const u32x4*>(
          qi + (static_cast<size_t>(b * nq + t0 + q) * H_I + h) * QROW + c * 16);
    *reinterpret_cast<u32x4*>(s_q + (h * kGemmQ + q) * DI + ((c ^ qswz(q)) << 4)) = v;
  }
  for (int i = tid; i < H_I * kGemmQ; i += kGemmThreads) {
    const int h = i / kGemmQ, q = i % kGemmQ;
    const size_t rh = static_cast<size_t>(b * nq + t0 + q) * H_I + h;
    const bool ok = t0 + q < nq;
    if constexpr (QX) {  // the scales act inside the MFMA; s_c is the head weight alone
      s_c[i] = ok ? wi[rh] : 0.f;
      s_qs[i] = ok ? reinterpret_cast<const uint32_t*>(qi_scale)[rh] : 0x7f7f7f7fu;
    } else {
      s_c[i] = ok ? wi[rh] * qi_scale[rh] : 0.f;
    }
  }
  if (tid < kGemmQ)
    s_nv[tid] = (t0 + tid < nq) ? visible(n_entries, pos, b * nq + t0 + tid, nq, m, n_max) : 0;
  __syncthreads();
  int nv_max = 0;
#pragma unroll
  for (int q = 0; q < kGemmQ; ++q) nv_max = max(nv_max, s_nv[q]);
  const int my_nv = s_nv[c16];
  const int ngroups = (nv_max + 63) / 64;
  if (wave >= ngroups) return;

  const size_t seq0 = PAGED ? 0 : static_cast<size_t>(b) * n_max;  // row of entry 0
  const uint8_t* kb = keys + seq0 * KROW + g * (MX ? 16 : 32);
  const float* sb = kscale + seq0;
  const uint32_t* swb = reinterpret_cast<const uint32_t*>(sb);  // MXFP4 scale bytes
  ST* srow = scores + static_cast<size_t>(b * nq + t0 + c16) * sstride;
  const bool row_ok = t0 + c16 < nq;
  // A operands of group G: entry G*64 + 16blk + c16 (clamped into the visible range), bytes
  // 32g..32g+31; entry scales of the 4 entries G*64 + 16blk + 4g + i this lane's D holds
  auto load = [&](int G, i32x8 (&a)[4], f32x4 (&ks)[4], int (&sa)[4]) {
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) {
      // entry of this lane and pool row of entry 0 of its 16-entry block (the block's clamped
      // entries, scale loads included, stay in the block holding nv_max - 1)
      const int el = min(G * 64 + blk * 16 + c16, nv_max - 1);
      long long r0 = 0;
      int e = el;
      if constexpr (PAGED) {
        const int tb = min(G * 64 + blk * 16, (nv_max - 1) & ~15);
        r0 = static_cast<long long>(block_base_uniform(pm, b, tb >> pm.shift)) +
             (tb & ((1 << pm.shift) - 1)) - tb;
        e = static_cast<int>(r0 + el);
      }
      if constexpr (MX) {  // 16 bytes of codes and this lane's block scale; no entry scale
        const u32x4 v = *reinterpret_cast<const u32x4*>(kb + static_cast<size_t>(e) * KROW);
        a[blk] = i32x8{static_cast<int>(v[0]), static_cast<int>(v[1]), static_cast<int>(v[2]),
                       static_cast<int>(v[3]), 0, 0, 0, 0};
        sa[blk] = static_cast<int>((swb[e] >> (8 * g)) & 0xffu);
        ks[blk] = f32x4{1.f, 1.f, 1.f, 1.f};
        continue;
      }
      sa[blk] = 127;
      const u32x4* src = reinterpret_cast<const u32x4*>(kb + static_cast<size_t>(e) * DI);
      const u32x4 lo = src[0], hi = src[1];
      a[blk] = i32x8{static_cast<int>(lo[0]), static_cast<int>(lo[1]), static_cast<int>(lo[2]),
                     static_cast<int>(lo[3]), static_cast<int>(hi[0]), static_cast<int>(hi[1]),
                     static_cast<int>(hi[2]), static_cast<int>(hi[3])};
#pragma unroll
      for (int i = 0; i < 4; ++i)
        ks[blk][i] = sb[r0 + min(G * 64 + blk * 16 + 4 * g + i, nv_max - 1)];
    }
  };
  const uint8_t* qb = s_q + c16 * DI;
  const int ch0 = ((MX ? g : 2 * g) ^ qswz(c16)) << 4;
  const int ch1 = ((MX ? 4 + g : 2 * g + 1) ^ qswz(c16)) << 4;
  i32x8 a[4], an[4];
  f32x4 ks[4], ksn[4];
  int sa[4], san[4];
  load(wave, a, ks, sa);
  for (int G = wave; G < ngroups; G += kGemmWaves) {
    load(min(G + kGemmWaves, ngroups - 1), an, ksn, san);  // always issued: same order
    f32x4 acc[4];
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) acc[blk] = f32x4{0.f, 0.f, 0.f, 0.f};
    // heads are software-pipelined: the four MFMAs of head h+1 are issued before the epilogue
    // of head h reads its results, and each head's query codes are read from LDS one step
    // before its MFMAs
    // head h's B operand (and, FP4 queries, this lane's block scale in bq[4])
    auto readq = [&](int h, i32x8& bq, float& ch) {
      const uint8_t* qh = qb + min(h, H_I - 1) * kGemmQ * DI;
      const u32x4 lo = *reinterpret_cast<const u32x4*>(qh + ch0);
      if constexpr (QX) {
        const uint32_t sw = s_qs[min(h, H_I - 1) * kGemmQ + c16];
        bq = i32x8{static_cast<int>(lo[0]), static_cast<int>(lo[1]), static_cast<int>(lo[2]),
                   static_cast<int>(lo[3]), static_cast<int>((sw >> (8 * g)) & 0xffu), 0, 0, 0};
      } else {
        const u32x4 hi = *reinterpret_cast<const u32x4*>(qh + ch1);
        bq = i32x8{static_cast<int>(lo[0]), static_cast<int>(lo[1]), static_cast<int>(lo[2]),
                   static_cast<int>(lo[3]), static_cast<int>(hi[0]), static_cast<int>(hi[1]),
                   static_cast<int>(hi[2]), static_cast<int>(hi[3])};
      }
      ch = s_c[min(h, H_I - 1) * kGemmQ + c16];
    };
    auto issue = [&](const i32x8& bq, f32x4 (&d)[4]) {
#pragma unroll
      for (int blk = 0; blk < 4; ++blk) {
        if constexpr (QX) {
          const i32x8 b4 = i32x8{bq[0], bq[1], bq[2], bq[3], 0, 0, 0, 0};
          d[blk] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              a[blk], b4, f32x4{0.f, 0.f, 0.f, 0.f}, 4, 4, 0, sa[blk], 0, bq[4]);
        } else if constexpr (MX) {
          d[blk] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              a[blk], bq, f32x4{0.f, 0.f, 0.f, 0.f}, 4, 0, 0, sa[blk], 0, 127);
        } else {
          d[blk] = mfma_fp8_16x16x128(a[blk], bq, f32x4{0.f, 0.f, 0.f, 0.f});
        }
      }
    };
    // acc += max(d, 0) * ch; the ReLU is a signed integer max of the float's bits with 0
    // (negative floats have negative integer patterns), one instruction
    auto epi = [&](const f32x4 (&d)[4], float ch) {
#pragma unroll
      for (int blk = 0; blk < 4; ++blk)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          acc[blk][i] = fmaf(__int_as_float(max(__float_as_int(d[blk][i]), 0)), ch, acc[blk][i]);
    };
    f32x4 dA[4], dB[4];
    float cA, cB, cc, cn;
    i32x8 bc, bn;
    readq(0, bc, cc);
    issue(bc, dA);
    cA = cc;
    readq(1, bc, cc);
    int h = 1;
    for (; h + 1 < H_I; h += 2) {
      readq(h + 1, bn, cn);
      issue(bc, dB);  // head h
      cB = cc;
      epi(dA, cA);
      readq(h + 2, bc, cc);
      issue(bn, dA);  // head h + 1
      cA = cn;
      epi(dB, cB);
    }
    if (h < H_I) {
      issue(bc, dB);
      epi(dA, cA);
      epi(dB, cc);
    } else {
      epi(dA, cA);
    }
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) {
      const int e = G * 64 + blk * 16 + 4 * g;
      if (row_ok && e < my_nv)
        Scores<ST>::put4(srow, e,
                         f32x4{acc[blk][0] * ks[blk][0], acc[blk][1] * ks[blk][1],
                               acc[blk][2] * ks[blk][2], acc[blk][3] * ks[blk][3]});
      a[blk] = an[blk];
      ks[blk] = ksn[blk];
      sa[blk] = san[blk];
    }
  }
}

// ============================================================================ block helpers
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
  uint32_t later = 0;
  for (int w2 = wave + 1; w2 < NWAVE; ++w2) later += s_tmp[w2];
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

template <typename T, bool kDescending, int THREADS>
__device__ void bitonic_sort(T* a, int n) {  // n power of two
  for (int k2 = 2; k2 <= n; k2 <<= 1) {
    for (int j = k2 >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < n; i += THREADS) {
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
  int eq_seen = 0, slot_base = 0;
  for (int w2 = 0; w2 < wave; ++w2) {
    const int eqb = eq_seen;
    int take_eq = need_eq - eqb;
    take_eq = take_eq < 0 ? 0 : (take_eq > static_cast<int>(s_eq[w2]) ? static_cast<int>(s_eq[w2]) : take_eq);
    slot_base += static_cast<int>(s_gt[w2]) + take_eq;
    eq_seen += static_cast<int>(s_eq[w2]);
  }
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

// Exact kk-th largest key (T) among n keys that all lie in [lo, hi], and how many keys equal
// to T are taken (need_eq).  One 12-bit histogram over the bits just below the common prefix of
// lo and hi (so the bins split the keys' actual range); if the crossing bin holds at most 64
// keys they are gathered into a small list and ranked by pairwise comparison in one wave,
// otherwise the full radix select runs.
template <int THREADS, typename KeyFn>
__device__ void select_kth(KeyFn key, int n, int kk, uint32_t lo, uint32_t hi,
                           uint32_t* hist /*4096*/, uint32_t* s_tmp, int* s_res, uint32_t& T,
                           int& need_eq, bool zeroed = false) {
  __shared__ uint32_t s_bin[64];
  __shared__ uint32_t s_nb;
  const int tid = threadIdx.x;
  const uint32_t diff = lo ^ hi;
  const int top = diff ? 32 - __clz(diff) : 0;  // bits below the common prefix
  const int shift = top > 12 ? top - 12 : 0;
  const uint32_t pmask = top >= 32 ? 0u : ~((1u << top) - 1u);
  const uint32_t prefix = lo & pmask;
  const uint32_t c1 = radix_pass<THREADS>(key, n, prefix, pmask, shift, 4096,
                                          static_cast<uint32_t>(kk), hist, s_tmp, s_res, zeroed);
  const uint32_t d1 = static_cast<uint32_t>(s_res[0]);
  const uint32_t r1 = static_cast<uint32_t>(s_res[1]);
  __syncthreads();
  if (c1 > 64) {
    radix_select<THREADS>(key, n, kk, hist, s_tmp, s_res, T, need_eq);
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
    for (int j = 0; j < nbk; ++j) {
      const uint32_t o = s_bin[j];
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
template <int THREADS, int PER, typename ST>
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
  // keys; every chunk load is issued (clamped into the row) and masked, the row's last partial
  // chunk is read element by element
  uint32_t kr[PER];
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int base = (i * THREADS + tid) * 4;
    // the address depends only on the row length, not on n_vis, so the loads need not wait for
    // the row's position and entry count
    float f[4];
    Scores<ST>::four(srow, min(base, sstride - 4), f);
#pragma unroll
    for (int j = 0; j < 4; ++j) kr[i * 4 + j] = (base + j < n_vis) ? order_key(f[j]) : 0u;
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
  // candidates (visible keys >= T_lo) per chunk column, packed two columns to a word, and the
  // largest candidate key
  uint32_t cw[CW], kmax = 0;
#pragma unroll
  for (int w = 0; w < CW; ++w) cw[w] = 0u;
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    uint32_t c = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool in = (i * THREADS + tid) * 4 + j < n_vis && kr[i * 4 + j] >= Tlo;
      c += in ? 1u : 0u;
      kmax = in ? max(kmax, kr[i * 4 + j]) : kmax;
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
        const int e = (i * THREADS + tid) * 4 + j;
        if (e < n_vis && kr[i * 4 + j] >= Tlo) {
          s_ckey[sl] = kr[i * 4 + j];
          s_cidx[sl] = e;
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
  ProfScope ps("fill_u32", s);
  fill_u32_kernel<<<grid, 256, 0, s>>>(p, v, n);
  return hipGetLastError();
}

// ============================================================================ multi-WG top-k
// For rows longer than one workgroup's register file (decode at long context).  A row is cut
// into chunks of kCollectChunk entries, one 1024-thread workgroup each.  A workgroup selects its
// chunk's candidates with a threshold of its own: T_c, the lower edge of the 12-bit bin (refined
// by 12 more bits when crowded) holding its r-th largest key, r = the chunk's expected share of
// the row's top kk plus four standard deviations.  It writes the (key, index) pairs >= T_c in
// ascending index order into its own region (block prefix sum, no global atomics) with the
// count and T_c.  A finalize workgroup per row (a second launch: a device-scope handoff inside
// one launch costs an L2 write-back per workgroup on this multi-XCD part) concatenates the
// regions (a list in ascending index order), finds the kk-th key T of the list with one
// histogram pass over its actual range and emits the keys above it plus the first ties in index
// order.  The list holds every key >= T of the row exactly when T >= every chunk's T_c (a key
// >= T is then >= its chunk's threshold); otherwise (a chunk holding far more than its share
// of the top keys), and on a region overflow or too few candidates, the exact streaming select
// of the row runs instead.
constexpr int kCollectChunk = 4096;
constexpr int kCandPerChunk = 1024;
constexpr int kSCandCap = 8192;  // candidates of a row held by its finalize workgroup
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
  const int row = blockIdx.x / nchunks;
  const int chunk = blockIdx.x % nchunks;
  const int tid = threadIdx.x;
  const int n_vis = visible(n_entries, pos, row, nq, m, n_max);
  const int kk = min(k, n_vis);
  const ST* srow = scores + static_cast<size_t>(row) * sstride;
  if (n_vis <= k) return;  // everything is selected; finalize does not read the regions
  const int used = (n_vis + kCollectChunk - 1) / kCollectChunk;  // chunks holding visible keys
  if (chunk >= used) return;
  const size_t rc = static_cast<size_t>(row) * nchunks + chunk;
  const int e0 = chunk * kCollectChunk;
  const int len = min(kCollectChunk, n_vis - e0);

  // this chunk's keys (one 16-byte load per thread, clamped into the row), also to LDS for the
  // histogram pass; the histogram is cleared while the loads are in flight
  uint32_t key[PER];
  {
    const int base = e0 + tid * PER;
    float f[4];
    Scores<ST>::four(srow, min(base, sstride - 4), f);
#pragma unroll
    for (int j = 0; j < 4; ++j) key[j] = base + j < n_vis ? order_key(f[j]) : 0u;
  }
  for (int i = tid; i < kHistBins; i += THREADS) hist[i] = 0u;
#pragma unroll
  for (int j = 0; j < PER; ++j) s_key[tid * PER + j] = key[j];
  __syncthreads();
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
  uint64_t* cdst = cand + rc * kCandPerChunk;
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
    ccount[2 * rc] = total;
    ccount[2 * rc + 1] = Tc;
  }
}

template <typename ST>
__global__ __launch_bounds__(1024) void topk_finalize_kernel(
    const ST* __restrict__ scores, int sstride, const int32_t* __restrict__ n_entries,
    const int32_t* __restrict__ pos, int nq, int m, int k, int n_max, int nchunks,
    const uint32_t* __restrict__ ccount, const uint64_t* __restrict__ cand,
    int32_t* __restrict__ idx_out, float* __restrict__ score_out) {
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
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
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
  const int used = (n_vis + kCollectChunk - 1) / kCollectChunk;  // <= nchunks
  if (tid == 0) {
    s_flag = used > THREADS ? 1 : 0;  // 1 = take the exact fallback
    s_lo = 0xffffffffu;
    s_hi = 0u;
    s_tmax = 0u;
  }
  __syncthreads();
  if (!s_flag) {
    const size_t rc = static_cast<size_t>(row) * nchunks + tid;
    const uint32_t c = tid < used ? ccount[2 * rc] : 0u;
    const uint32_t tc = wave_max_u32(tid < used ? ccount[2 * rc + 1] : 0u);
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
  // 16 threads per region, each region's pairs to its place in the concatenated list
  for (int c = tid >> 4; c < used; c += THREADS / 16) {
    const uint32_t o = s_off[c], n = s_off[c + 1] - o;
    const uint64_t* src = cand + (static_cast<size_t>(row) * nchunks + c) * kCandPerChunk;
    for (uint32_t j = tid & 15; j < n; j += 16) {
      const uint64_t v = src[j];
      const uint32_t kv = static_cast<uint32_t>(v >> 32);
      ckey[o + j] = kv;
      cidx[o + j] = static_cast<int32_t>(v & 0xffffffffu);
      lo = min(lo, kv);
      hi = max(hi, kv);
    }
  }
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
  if (T < s_tmax) {  // some chunk's threshold cut keys that reach T: exact streaming select
    auto kf = [&](int e) { return order_key(Scores<ST>::at(srow, e)); };
    radix_select<THREADS>(kf, n_vis, kk, hist, s_tmp, s_res, T, need_eq);
    ordered_emit<THREADS>(kf, n_vis, T, need_eq, kk, k, srow, out, sout, s_tmp);
    return;
  }
  // the candidate list is in ascending index order
  ordered_emit_fn<THREADS>(ck, nc, T, need_eq, k, [&](int slot, int j) {
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

static int score_stride(int n_max) { return (n_max + 63) & ~63; }

// Rows longer than the 1024-thread sampled select holds (and not too many of them) use the
// multi-workgroup select (measured slower than the one-workgroup select at 32K entries).
bool index_use_multi(int rows, int n_max) {
  return n_max > kRowTopkBigN && rows <= kMultiMaxRows;
}

static int collect_chunks(int n_max) { return (n_max + kCollectChunk - 1) / kCollectChunk; }

size_t index_topk_workspace(int rows, int n_max, int k, bool score_bf16) {
  const size_t sb = score_bf16 ? 2 : 4;
  size_t b = align256(static_cast<size_t>(rows) * score_stride(n_max) * sb);
  if (index_use_multi(rows, n_max)) {
    const size_t rc = static_cast<size_t>(rows) * collect_chunks(n_max);
    b += align256(rc * 8);  // (count, threshold) per chunk
    b += align256(rc * kCandPerChunk * 8);
  }
  (void)k;
  return b;
}

void index_topk_layout(IndexArgs& a, void* ws, int rows) {
  unsigned char* p = static_cast<unsigned char*>(ws);
  a.sstride = score_stride(a.n_max);
  a.scores = p;
  p += align256(static_cast<size_t>(rows) * a.sstride * (a.score_bf16 ? 2 : 4));
  a.counters = nullptr;
  a.cand = nullptr;
  if (index_use_multi(rows, a.n_max)) {
    const size_t rc = static_cast<size_t>(rows) * collect_chunks(a.n_max);
    a.counters = reinterpret_cast<uint32_t*>(p);
    p += align256(rc * 8);
    a.cand = reinterpret_cast<uint64_t*>(p);
  }
}

#ifndef CSA_SCORE_TPW
#define CSA_SCORE_TPW 32
#endif
constexpr int kScoreTPW = CSA_SCORE_TPW;       // tiles of 16 entries per wave
constexpr int kScoreChunk = 4 * kScoreTPW * 16;  // entries per workgroup

template <int DI, int HT, bool MX, bool PAGED, bool QX, typename ST>
static void launch_scores_k(const IndexArgs& a, int chunk, int nchunks, hipStream_t s) {
  const unsigned grid = static_cast<unsigned>(nchunks) * static_cast<unsigned>(a.B * a.nq);
  index_score_kernel<DI, HT, kScoreTPW, MX, PAGED, QX, ST><<<grid, 256, 0, s>>>(
      a.qi, a.qi_scale, a.wi, a.keys, a.kscale, a.n_entries, a.pos, a.nq, a.n_max, a.H_I, a.m,
      chunk, static_cast<ST*>(a.scores), a.sstride, nchunks, a.pages);
}
template <int DI, int HT, bool MX, bool QX, typename ST>
static void launch_scores_p(const IndexArgs& a, int chunk, int nchunks, hipStream_t s) {
  if (a.pages.table != nullptr)
    launch_scores_k<DI, HT, MX, true, QX, ST>(a, chunk, nchunks, s);
  else
    launch_scores_k<DI, HT, MX, false, QX, ST>(a, chunk, nchunks, s);
}
template <int DI, int HT, typename ST>
static void launch_scores_t(const IndexArgs& a, int chunk, int nchunks, hipStream_t s) {
  ProfScope ps("index_score", s);
  if (a.key_fmt == 1) {
    if (a.q_fmt == 1)
      launch_scores_p<DI, HT, true, true, ST>(a, chunk, nchunks, s);
    else
      launch_scores_p<DI, HT, true, false, ST>(a, chunk, nchunks, s);
  } else {
    launch_scores_p<DI, HT, false, false, ST>(a, chunk, nchunks, s);
  }
}

template <typename ST>
static hipError_t launch_scores(const IndexArgs& a, int chunk, hipStream_t s) {
  const int nchunks = (a.n_max + chunk - 1) / chunk;
  const int ht = (a.H_I + 15) / 16;
#define CSA_SCORE_CASE(DI_, HT_)                            \
  if (a.d_I == DI_ && ht == HT_) {                         \
    launch_scores_t<DI_, HT_, ST>(a, chunk, nchunks, s);    \
    return hipGetLastError();                              \
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

// Rows scored as a product over heads (16 query rows of a sequence per workgroup) when every
// sequence brings at least 16 query rows and the heads fit the LDS tile.
static bool use_gemm_scores(const IndexArgs& a) {
  return a.nq >= kGemmQ && a.d_I == kGemmDI && a.H_I <= kGemmH;
}

template <bool MX, bool PAGED, bool QX, typename ST>
static hipError_t launch_gemm_scores_t(const IndexArgs& a, hipStream_t s) {
  if (hipError_t e = ensure_max_lds(
          reinterpret_cast<const void*>(index_gemm_kernel<MX, PAGED, QX, ST>), kGemmLds))
    return e;
  const int qtiles = (a.nq + kGemmQ - 1) / kGemmQ;
  ProfScope ps("index_score", s);
  index_gemm_kernel<MX, PAGED, QX, ST>
      <<<static_cast<unsigned>(a.B) * qtiles, kGemmThreads, kGemmLds, s>>>(
          a.qi, a.qi_scale, a.wi, a.keys, a.kscale, a.n_entries, a.pos, a.nq, a.n_max, a.H_I,
          a.m, qtiles, static_cast<ST*>(a.scores), a.sstride, a.pages);
  return hipGetLastError();
}

template <bool MX, bool QX, typename ST>
static hipError_t launch_gemm_scores_p(const IndexArgs& a, hipStream_t s) {
  return a.pages.table ? launch_gemm_scores_t<MX, true, QX, ST>(a, s)
                       : launch_gemm_scores_t<MX, false, QX, ST>(a, s);
}

template <typename ST>
static hipError_t launch_gemm_scores(const IndexArgs& a, hipStream_t s) {
  if (a.key_fmt != 1) return launch_gemm_scores_p<false, false, ST>(a, s);
  return a.q_fmt == 1 ? launch_gemm_scores_p<true, true, ST>(a, s)
                      : launch_gemm_scores_p<true, false, ST>(a, s);
}

template <typename ST>
static hipError_t launch_index_topk_t(const IndexArgs& a, hipStream_t s) {
  const int rows = a.B * a.nq;
  const bool multi = index_use_multi(rows, a.n_max);
  hipError_t e = (!multi && use_gemm_scores(a)) ? launch_gemm_scores<ST>(a, s)
                                                : launch_scores<ST>(a, kScoreChunk, s);
  if (e != hipSuccess) return e;
  const ST* sc = static_cast<const ST*>(a.scores);
  if (!multi) {
    if (a.n_max <= 4096) return launch_row_topk<256, kRowTopkMaxN, ST>(a, rows, s);
    if (a.n_max <= 16384) {
      ProfScope ps("topk_sample", s);
      // 512 threads x 32 keys (measured 1.83 ms against 2.89 ms for 256 x 64 and 3.68 ms for
      // 1024 x 32 on the 64K-token prefill rows)
      topk_sample_kernel<512, 32, ST><<<rows, 512, 0, s>>>(sc, a.sstride, a.n_entries, a.pos,
                                                          a.nq, a.m, a.k, a.n_max, a.idx_out,
                                                          a.score_out);
      return hipGetLastError();
    }
    ProfScope ps("topk_sample", s);
    topk_sample_kernel<1024, 32, ST><<<rows, 1024, 0, s>>>(sc, a.sstride, a.n_entries, a.pos,
                                                          a.nq, a.m, a.k, a.n_max, a.idx_out,
                                                          a.score_out);
    return hipGetLastError();
  }
  const int ncc = collect_chunks(a.n_max);
  {
    ProfScope ps("topk_collect", s);
    topk_collect_kernel<ST><<<static_cast<unsigned>(ncc) * rows, 1024, 0, s>>>(
        sc, a.sstride, a.n_entries, a.pos, a.nq, a.m, a.k, a.n_max, ncc, a.counters, a.cand);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if ((e = ensure_max_lds(reinterpret_cast<const void*>(topk_finalize_kernel<ST>), kMultiLds)))
    return e;
  ProfScope ps("topk_finalize", s);
  topk_finalize_kernel<ST><<<rows, 1024, kMultiLds, s>>>(sc, a.sstride, a.n_entries, a.pos,
                                                         a.nq, a.m, a.k, a.n_max, ncc,
                                                         a.counters, a.cand, a.idx_out,
                                                         a.score_out);
  return hipGetLastError();
}

hipError_t launch_index_topk(const IndexArgs& a, hipStream_t s) {
  return a.score_bf16 ? launch_index_topk_t<uint16_t>(a, s) : launch_index_topk_t<float>(a, s);
}

}  // namespace csa
