// Lightning indexer scoring for gfx950.
//
// Method: "DeepSeek V4 模型技术大全", chapter "Attention", section "CSA 的完整路径":
//   I_{t,s} = sum_h w^I_{t,h} ReLU(q^I_{t,h} . K^IComp_s)  for s < floor((t+1)/m).
// Operands are E4M3 codes with float32 scales; since the scales are positive,
//   w_h ReLU(sq_h sk_s x) = sk_s (w_h sq_h) ReLU(x),
// so the MFMA works on raw codes and the epilogue applies (w_h sq_h) per head and sk_s per entry.
//
// The indexer query may be MXFP4 too (both operands FP4: E2M1 codes with an E8M0 scale per 32
// dims on each side, applied inside the scaled MFMA).  Scores may be stored as fp32 or, rounded
// to nearest even, as bf16 ("index scores FP32 -> BF16"); the top-k (topk.hip) then ranks the
// bf16 values.
#include "topk_common.h"

#ifndef CSA_STREAM_LOAD
#define CSA_STREAM_LOAD(p) __builtin_nontemporal_load(p)
#endif

namespace csa {

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
// COL: the workgroup also selects its chunk's top-k candidates for the multi-workgroup select
// (the order keys of the scores it stores, kept in LDS; collect_candidates): region and (count,
// threshold) of chunk `blockIdx.x % nchunks` of the row in cand / ccount, as the selection's
// collect kernel writes them for its own chunks.  Chunks with no visible entry, and rows of no
// more than k visible entries, write nothing (the finalize does not read them).
template <int DI, int HT, int TPW, bool MX = false, bool PAGED = false, bool QX = false,
          typename ST = float, bool COL = false>
__global__ __launch_bounds__(256) void index_score_kernel(
    const uint8_t* __restrict__ qi, const float* __restrict__ qi_scale,
    const float* __restrict__ wi, const uint8_t* __restrict__ keys,
    const float* __restrict__ kscale, const int32_t* __restrict__ n_entries,
    const int32_t* __restrict__ pos, int nq, int n_max, int H_I, int m, int chunk,
    ST* __restrict__ scores, int sstride, int nchunks, PageMap pm, int k,
    uint32_t* __restrict__ ccount, uint64_t* __restrict__ cand) {
  static_assert(!QX || MX, "an FP4 query is paired with FP4 keys");
  constexpr int KB = DI / 4;   // key bytes per lane (its lane group's K slice)
  constexpr int KK = DI / 32;  // 8-byte MFMA steps per slice
  constexpr int CH = 4 * TPW * 16;  // entries per workgroup (the launch's chunk)
  __shared__ uint32_t s_key[COL ? CH : 1];          // COL: order keys of the chunk's scores
  __shared__ uint32_t s_hist[COL ? kHistBins : 1];  // COL: histogram of the collect passes
  __shared__ uint32_t s_tmp[4];
  __shared__ int s_res[2];

  // every launch parameter is requested at once (scalar loads complete out of order, so each
  // later batch the compiler would issue on demand costs a full wait on all of them)
  asm volatile("" ::"s"(qi), "s"(qi_scale), "s"(wi), "s"(keys), "s"(kscale), "s"(n_entries),
               "s"(pos), "s"(nq), "s"(n_max), "s"(H_I), "s"(m), "s"(chunk), "s"(scores),
               "s"(sstride), "s"(nchunks), "s"(pm.table), "s"(pm.stride), "s"(pm.shift));
  if constexpr (COL) asm volatile("" ::"s"(k), "s"(ccount), "s"(cand));
  const int row = blockIdx.x / nchunks;
  const int b = row / nq;
  const int e0 = (blockIdx.x % nchunks) * chunk;
  const int tid = threadIdx.x;
  const int l = lane_id(), g = l >> 4, c16 = l & 15, wave = tid >> 6;
  // position and entry count of the row through the vector path, first: one round trip,
  // waited for only where the visible length is needed
  int rv = pos ? row : b, bv = b;
  asm volatile("" : "+v"(rv), "+v"(bv));
  int t_vec = (pos ? pos : n_entries)[rv];
  int ne_vec = n_entries[bv];

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
        const float wv = wi[static_cast<size_t>(row) * H_I + (hh < H_I ? hh : 0)];
        wq[ht][i] = hh < H_I ? wv : 0.f;  // the query scale acts inside the MFMA
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
    // (loads unconditional, from a clamped head, then selected: guarded loads went out one
    // pair at a time, each behind a wait)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hh = ht * 16 + g * 4 + i;
      const size_t hi = static_cast<size_t>(row) * H_I + (hh < H_I ? hh : 0);
      const float wv = wi[hi], sv = qi_scale[hi];
      wq[ht][i] = hh < H_I ? wv * sv : 0.f;
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
      if constexpr (COL) s_key[e - e0] = order_key(Scores<ST>::stored(sc));
    }
  };
  // The first tiles are loaded before the row's visible length is known (clamped to the
  // allocated entries; scores past the visible end are never stored), so no wave waits for
  // the position and entry-count loads before its first key loads.
  constexpr int PD = 3, NB = PD + 1;  // a spare buffer: tile t+PD's loads go out before tile t
  KeyTile kb[NB];                      // is computed
#pragma unroll
  for (int t = 0; t < PD; ++t) load(t, kb[t], n_max - 1);
  asm volatile("" : "+v"(t_vec), "+v"(ne_vec) : : "memory");  // after the first tiles' loads
  int n_vis;
  {
    const long tt = pos ? __builtin_amdgcn_readfirstlane(t_vec) : (row % nq);
    long v = (tt + 1) / m;
    const int n = min(__builtin_amdgcn_readfirstlane(ne_vec), n_max);
    if (v > n) v = n;
    n_vis = static_cast<int>(v < 0 ? 0 : v);  // as visible(): min(n_entries, (t+1)/m) in [0, n_max]
  }
  const int e1 = min(n_vis, e0 + chunk);
  if (e0 < e1) {
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      if (t + PD < TPW) load(t + PD, kb[(t + PD) % NB], e1 - 1);
      compute(t, kb[t % NB], e1);
    }
  }
  if constexpr (COL) {
    // (e0, e1 and n_vis are uniform over the workgroup)
    if (e0 >= e1 || n_vis <= k) return;
    constexpr int PER = CH / 256;
    for (int i = tid; i < kHistBins; i += 256) s_hist[i] = 0u;
    __syncthreads();  // every stored key in s_key, s_hist cleared
    const int len = e1 - e0;
    uint32_t key[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) key[i] = tid * PER + i < len ? s_key[tid * PER + i] : 0u;
    const size_t rc = static_cast<size_t>(row) * nchunks + blockIdx.x % nchunks;
    collect_candidates<256, PER>(key, s_key, e0, len, n_vis, k, s_hist, s_tmp, s_res,
                                 cand + rc * kCandPerChunk, ccount + 2 * rc);
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
constexpr int kGemmFillTiles = 256;   // workgroups that fill the device (one per CU)
constexpr int kGemmPartGroups = 64;   // 64-entry groups of an entry part at the least
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
    const int32_t* __restrict__ pos, int nq, int n_max, int H_I, int m, int qtiles, int gpp,
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
  // this workgroup's part of the entry groups (blockIdx.y of gridDim.y parts of gpp groups:
  // few query tiles over a long cache still fill the device)
  const int g0 = static_cast<int>(blockIdx.y) * gpp;
  const int ngroups = min((nv_max + 63) / 64, g0 + gpp);
  if (g0 + wave >= ngroups) return;

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
  load(g0 + wave, a, ks, sa);
  for (int G = g0 + wave; G < ngroups; G += kGemmWaves) {
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

// ============================================================================ launchers
#ifndef CSA_SCORE_TPW
#define CSA_SCORE_TPW 32
#endif
constexpr int kScoreTPW = CSA_SCORE_TPW;       // tiles of 16 entries per wave
constexpr int kScoreChunk = 4 * kScoreTPW * 16;  // entries per workgroup

template <int DI, int HT, bool MX, bool PAGED, bool QX, typename ST, bool COL>
static void launch_scores_k(const IndexArgs& a, int chunk, int nchunks, hipStream_t s) {
  const unsigned grid = static_cast<unsigned>(nchunks) * static_cast<unsigned>(a.B * a.nq);
  index_score_kernel<DI, HT, kScoreTPW, MX, PAGED, QX, ST, COL><<<grid, 256, 0, s>>>(
      a.qi, a.qi_scale, a.wi, a.keys, a.kscale, a.n_entries, a.pos, a.nq, a.n_max, a.H_I, a.m,
      chunk, static_cast<ST*>(a.scores), a.sstride, nchunks, a.pages, a.k, a.counters, a.cand);
}
template <int DI, int HT, bool MX, bool QX, typename ST, bool COL>
static void launch_scores_p(const IndexArgs& a, int chunk, int nchunks, hipStream_t s) {
  if (a.pages.table != nullptr)
    launch_scores_k<DI, HT, MX, true, QX, ST, COL>(a, chunk, nchunks, s);
  else
    launch_scores_k<DI, HT, MX, false, QX, ST, COL>(a, chunk, nchunks, s);
}
template <int DI, int HT, typename ST, bool COL>
static void launch_scores_t(const IndexArgs& a, int chunk, int nchunks, hipStream_t s) {
  ProfScope ps("index_score", s);
  if (a.key_fmt == 1) {
    if (a.q_fmt == 1)
      launch_scores_p<DI, HT, true, true, ST, COL>(a, chunk, nchunks, s);
    else
      launch_scores_p<DI, HT, true, false, ST, COL>(a, chunk, nchunks, s);
  } else {
    launch_scores_p<DI, HT, false, false, ST, COL>(a, chunk, nchunks, s);
  }
}

// COL: the scorer also collects its chunks' candidates (index_fused_collect: d_I = 128 only)
template <typename ST, bool COL = false>
static hipError_t launch_scores(const IndexArgs& a, int chunk, hipStream_t s) {
  const int nchunks = (a.n_max + chunk - 1) / chunk;
  const int ht = (a.H_I + 15) / 16;
#define CSA_SCORE_CASE(DI_, HT_)                                 \
  if (a.d_I == DI_ && ht == HT_) {                              \
    launch_scores_t<DI_, HT_, ST, COL>(a, chunk, nchunks, s);    \
    return hipGetLastError();                                   \
  }
  CSA_SCORE_CASE(128, 4)
  CSA_SCORE_CASE(128, 3)
  CSA_SCORE_CASE(128, 2)
  CSA_SCORE_CASE(128, 1)
  if constexpr (!COL) {
    CSA_SCORE_CASE(64, 4)
    CSA_SCORE_CASE(64, 3)
    CSA_SCORE_CASE(64, 2)
    CSA_SCORE_CASE(64, 1)
    CSA_SCORE_CASE(32, 4)
    CSA_SCORE_CASE(32, 3)
    CSA_SCORE_CASE(32, 2)
    CSA_SCORE_CASE(32, 1)
  }
#undef CSA_SCORE_CASE
  return hipErrorInvalidValue;
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
  // entry parts: enough workgroups to fill the device when there are few query tiles (a
  // 4096-entry part at the least)
  const int tiles = a.B * qtiles;
  const int groups = (a.n_max + 63) / 64;
  const int parts = std::max(1, std::min((kGemmFillTiles + tiles - 1) / tiles,
                                         (groups + kGemmPartGroups - 1) / kGemmPartGroups));
  const int gpp = (groups + parts - 1) / parts;
  ProfScope ps("index_score", s);
  index_gemm_kernel<MX, PAGED, QX, ST>
      <<<dim3(static_cast<unsigned>(tiles), static_cast<unsigned>(parts)), kGemmThreads,
         kGemmLds, s>>>(
          a.qi, a.qi_scale, a.wi, a.keys, a.kscale, a.n_entries, a.pos, a.nq, a.n_max, a.H_I,
          a.m, qtiles, gpp, static_cast<ST*>(a.scores), a.sstride, a.pages);
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

// (Both scorers write the same score rows, so either selection path reads them: rows of a
// cache over 32768 entries -- the chunks of a long prompt -- are scored as a product too.)
template <typename ST>
static hipError_t launch_index_scores_t(const IndexArgs& a, hipStream_t s) {
  return use_gemm_scores(a) ? launch_gemm_scores<ST>(a, s) : launch_scores<ST>(a, kScoreChunk, s);
}

hipError_t launch_index_scores(const IndexArgs& a, hipStream_t s) {
  return a.score_bf16 ? launch_index_scores_t<uint16_t>(a, s) : launch_index_scores_t<float>(a, s);
}

// Rows over caches of more than kFusedMinN entries that the decode scorer takes (fewer than 16
// query rows a sequence, or more heads than the product's LDS tile) and d_I = 128: the scorer
// collects each chunk's candidates itself, in the workgroup that has just scored the chunk, and
// the selection is the finalize alone (no second read of the scores, one launch fewer).  The
// collection adds about 3 us to the scorer on MI355X: at 1M entries (4 rows) that is less than
// the collect launch it replaces (decode step 70.0 -> 66.4 us); at 32768 entries (32 rows) the
// one-workgroup row select is as fast (60 us either way), and rows that short keep it.
constexpr int kFusedMinN = 32768;
bool index_fused_collect(int nq, int d_I, int H_I, int rows, int n_max) {
  const bool gemm = nq >= kGemmQ && d_I == kGemmDI && H_I <= kGemmH;
  return !gemm && d_I == 128 && n_max > kFusedMinN && rows <= kMultiMaxRows;
}
int index_score_chunk() { return kScoreChunk; }

hipError_t launch_index_scores_collect(const IndexArgs& a, hipStream_t s) {
  return a.score_bf16 ? launch_scores<uint16_t, true>(a, kScoreChunk, s)
                      : launch_scores<float, true>(a, kScoreChunk, s);
}

}  // namespace csa
