// Token-level compressor of CSA / HCA for gfx950.
//
// Method: "DeepSeek V4 模型技术大全", chapter "Attention".
//  - section "CSA 的完整路径": C^a = H W^a_KV, C^b = H W^b_KV, Z^a = H W^a_Z, Z^b = H W^b_Z;
//    block i's weights are a softmax over the 2m rows [Z^a_{mi..m(i+1)-1} + B^a;
//    Z^b_{m(i-1)..mi-1} + B^b], taken per channel, and C^Comp_i = sum S^a (.) C^a + sum S^b (.) C^b.
//    The indexer keys K^IComp come from the same operation with their own weights.
//  - section "HCA 的完整路径": m'-row blocks, C^Comp_i = sum S (.) C with S = softmax(Z + B).
//  - section "注意力实现细节": compressed entries are RMS-normalised and carry partial RoPE.
// Block 0 of the overlapping compressor has no b-rows.  Entry i sits at position m*i; the
// window KV of token u is RMSNorm(h_u W_win) * gamma_win with RoPE at u.  Indexer keys are not
// normalised or rotated and are stored as E4M3 with one fp32 scale (max|x|/448) per entry.
//
// Pipeline: one bf16 MFMA GEMM computes every projection of the new tokens into an fp32
// staging buffer (projections of tokens from earlier calls come from the per-sequence tail
// ring); a pooling kernel per closed block; a window kernel per token; a tail-ring update.
#include "common.h"
#include "kernels.h"

namespace csa {

// ============================================================================ GEMM
// Cst[M, N] (fp32) = A[M, K] (bf16, row-major) . Bw[N, K]^T (bf16, row-major), K % 32 == 0.
// 128x128 tile per workgroup, 4 waves each owning 64x64 (4x4 MFMA 16x16x32 tiles).
constexpr int GBM = 128, GBN = 128, GBK = 32, GLD = GBK + 8;

__global__ __launch_bounds__(256) void gemm_tn_bf16_kernel(const uint16_t* __restrict__ A,
                                                          const uint16_t* __restrict__ Bw,
                                                          float* __restrict__ Cst, int M, int N,
                                                          int K, int tiles_n) {
  __shared__ __align__(16) uint16_t sa[2][GBM * GLD];
  __shared__ __align__(16) uint16_t sb[2][GBN * GLD];
  const int tid = threadIdx.x;
  const int l = lane_id(), g = l >> 4, c16 = l & 15, wave = tid >> 6;
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
  const int m0 = tm * GBM, n0 = tn * GBN;
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;

  // each thread stages 2 x 16 bytes of A and of B per K step
  u32x4 ra[2], rb[2];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int ch = tid + i * 256;      // 512 chunks = 128 rows x 4 chunks of 8 bf16
      const int rr = ch >> 2, cc = (ch & 3) * 8;
      const int am = m0 + rr, bn = n0 + rr;
      ra[i] = am < M ? *reinterpret_cast<const u32x4*>(A + static_cast<size_t>(am) * K + k0 + cc)
                     : u32x4{0, 0, 0, 0};
      rb[i] = bn < N ? *reinterpret_cast<const u32x4*>(Bw + static_cast<size_t>(bn) * K + k0 + cc)
                     : u32x4{0, 0, 0, 0};
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int ch = tid + i * 256;
      const int rr = ch >> 2, cc = (ch & 3) * 8;
      *reinterpret_cast<u32x4*>(&sa[buf][rr * GLD + cc]) = ra[i];
      *reinterpret_cast<u32x4*>(&sb[buf][rr * GLD + cc]) = rb[i];
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = K / GBK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * GBK);
    bf16x8 af[4], bfr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      af[i] = as_bf16x8(*reinterpret_cast<const u32x4*>(&sa[buf][(wm + i * 16 + c16) * GLD + g * 8]));
      bfr[i] = as_bf16x8(*reinterpret_cast<const u32x4*>(&sb[buf][(wn + i * 16 + c16) * GLD + g * 8]));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma_bf16_16x16x32(af[i], bfr[j], acc[i][j]);
    if (kt + 1 < nk) sstore(buf ^ 1);
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + wn + j * 16 + c16;
      if (n >= N) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = m0 + wm + i * 16 + g * 4 + e;
        if (m < M) Cst[static_cast<size_t>(m) * N + n] = acc[i][j][e];
      }
    }
}

// Large-tile variant for K % 64 == 0: 256x256 tile per workgroup of 8 waves (two per SIMD),
// wave (wm, wn) owning rows wm*128.. and columns wn*64.. with 4x2 MFMA 32x32x16 tiles (128
// accumulator VGPRs).  K advances 64 at a time through two LDS stages of A and B panels
// (2 x 64 KiB) filled by direct global->LDS 16-byte loads: one load instruction writes 1 KiB
// (8 rows of 128 bytes); which chunk a lane fetches sets the layout, so chunk c of row r sits at
// 16-byte position c ^ g(r), g(r) = (r & 7) ^ ((r >> 3) & 1), which keeps the fragment reads
// (lane -> row l%32, chunk pair) free of bank conflicts for 8- and 16-lane bank groups.  Tiles
// are numbered in groups of 8 M-tiles and the numbering is laid out XCD by XCD (workgroup b runs
// on XCD b % 8), so the 32 workgroups resident on an XCD share 8 A panels and 4 B panels
// through its L2.
constexpr int G2M = 256, G2N = 256, G2K = 64, G2_THREADS = 512;
constexpr int kEpiPitch = G2N + 8;  // fp32 row pitch of the epilogue staging (64 rows: 66 KiB)
constexpr size_t kGemm2Lds = 2 * (G2M + G2N) * G2K * sizeof(uint16_t);  // 128 KiB

__device__ __forceinline__ int g2_swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// C[m, n] = sum_k A[m, k] W[n, k] with row strides lda, ldw, ldc (elements); OutT = float, or
// uint16_t for a bf16 result (round to nearest even).
template <typename OutT>
__global__ __launch_bounds__(G2_THREADS) void gemm_tn_bf16_256_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ Bw, OutT* __restrict__ Cst,
    int M, int N, int K, int lda, int ldw, int ldc, int tiles_m, int tiles_n, int per_xcd,
    bool vec_ok) {
  extern __shared__ __align__(16) unsigned char smem[];
  typedef __attribute__((address_space(3))) void lds_void;
  const int bid = blockIdx.x;
  const int t = (bid & 7) * per_xcd + (bid >> 3);
  if (t >= tiles_m * tiles_n) return;
  // grouped order: 8 M-tiles (fewer in the last group) per column sweep
  const int group = t / (8 * tiles_n);
  const int gm0 = group * 8;
  const int gsize = min(8, tiles_m - gm0);
  const int within = t - group * 8 * tiles_n;
  const int tm = gm0 + within % gsize, tn = within / gsize;
  const int m0 = tm * G2M, n0 = tn * G2N;

  const int tid = threadIdx.x, l = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int h = l >> 5, n32 = l & 31;

  // direct loads: instruction q of wave w covers panel rows (4w + q)*8 .. +7; lane i takes row
  // +i/8, LDS position i%8, global chunk (i%8) ^ g(row)
  const uint16_t* asrc[4];
  const uint16_t* bsrc[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = (4 * wave + q) * 8 + (l >> 3);
    const int c = (l & 7) ^ g2_swz(r);
    asrc[q] = A + static_cast<size_t>(min(m0 + r, M - 1)) * lda + c * 8;
    bsrc[q] = Bw + static_cast<size_t>(min(n0 + r, N - 1)) * ldw + c * 8;
  }
  auto issue = [&](int kt, int stage) {
    unsigned char* sa = smem + stage * 65536 + (4 * wave) * 8 * 128;
    unsigned char* sb = sa + 32768;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      __builtin_amdgcn_global_load_lds(asrc[q] + kt * G2K, (lds_void*)(sa + q * 1024),
                                       16, 0, 0);
      __builtin_amdgcn_global_load_lds(bsrc[q] + kt * G2K, (lds_void*)(sb + q * 1024),
                                       16, 0, 0);
    }
  };
  // fragment offsets: row l%32 of a 32-row block (g depends on l only), chunk 2ks + h
  const int gr = g2_swz(n32);
  uint32_t aoff[4], boff[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const uint32_t pos = static_cast<uint32_t>((2 * ks + h) ^ gr) * 16u;
    aoff[ks] = static_cast<uint32_t>(wm * 128 + n32) * 128u + pos;
    boff[ks] = 32768u + static_cast<uint32_t>(wn * 64 + n32) * 128u + pos;
  }

  f32x16 acc[4][2];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) acc[mi][ni] = f32x16{};

  const int nk = K / G2K;
  issue(0, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int stage = kt & 1;
    if (kt + 1 < nk) issue(kt + 1, stage ^ 1);
    const unsigned char* base = smem + stage * 65536;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      u32x4 af[4], bf[2];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
        af[mi] = *reinterpret_cast<const u32x4*>(base + aoff[ks] + mi * 4096);
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
        bf[ni] = *reinterpret_cast<const u32x4*>(base + boff[ks] + ni * 4096);
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(af[mi]),
                                                                as_bf16x8(bf[ni]), acc[mi][ni], 0, 0, 0);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the next stage has landed
    __syncthreads();                                   // and every wave is done with this one
  }
  // Epilogue through LDS (free after the last barrier), 64 tile rows per pass: the waves that
  // own them write their accumulators as fp32 rows (pitch kEpiPitch: rows 4 apart land 32 banks
  // apart, so the two half-waves' rows do not collide), then every wave reads whole rows back,
  // 32 bytes per lane, and stores them as full-width row segments.
  // D of a 32x32 tile: lane l holds column l%32, rows 8*(i/4) + 4h + i%4.
  float* stage = reinterpret_cast<float*>(smem);
  const bool full_n = vec_ok && n0 + G2N <= N;
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    if (wm == (pass >> 1)) {
#pragma unroll
      for (int mh = 0; mh < 2; ++mh) {
        const int mi = 2 * (pass & 1) + mh;
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int r = mh * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
            stage[r * kEpiPitch + wn * 64 + ni * 32 + n32] = acc[mi][ni][i];
          }
      }
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int r = it * 16 + wave * 2 + (l >> 5);  // tile row within the pass
      const int c = (l & 31) * 8;                    // first of 8 columns
      const f32x4 v0 = *reinterpret_cast<const f32x4*>(stage + r * kEpiPitch + c);
      const f32x4 v1 = *reinterpret_cast<const f32x4*>(stage + r * kEpiPitch + c + 4);
      const int m = m0 + pass * 64 + r;
      if (m < M) {
        OutT* dst = Cst + static_cast<size_t>(m) * ldc + n0 + c;
        if (full_n) {
          if constexpr (sizeof(OutT) == 2) {
            u32x4 o;
            o[0] = pack_bf16x2(v0[0], v0[1]);
            o[1] = pack_bf16x2(v0[2], v0[3]);
            o[2] = pack_bf16x2(v1[0], v1[1]);
            o[3] = pack_bf16x2(v1[2], v1[3]);
            *reinterpret_cast<u32x4*>(dst) = o;
          } else {
            reinterpret_cast<f32x4*>(dst)[0] = v0;
            reinterpret_cast<f32x4*>(dst)[1] = v1;
          }
        } else {
          const float vv[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            if (n0 + c + j < N) {
              if constexpr (sizeof(OutT) == 2)
                dst[j] = f32_to_bf16(vv[j]);
              else
                dst[j] = vv[j];
            }
          }
        }
      }
    }
    __syncthreads();
  }
}

// One launch of the large-tile GEMM (K % 64 == 0): tiles in XCD order, LDS attribute set once
// per output type.
template <typename OutT>
static hipError_t launch_gemm_256(const uint16_t* A, int lda, const uint16_t* W, int ldw, OutT* C,
                                  int ldc, int M, int N, int K, hipStream_t s) {
  if (hipError_t e = ensure_max_lds(
          reinterpret_cast<const void*>(gemm_tn_bf16_256_kernel<OutT>), kGemm2Lds))
    return e;
  const int tm2 = (M + G2M - 1) / G2M, tn2 = (N + G2N - 1) / G2N;
  const int per_xcd = (tm2 * tn2 + 7) / 8;
  // full-row vector stores need 8-element aligned rows (16 or 32 bytes)
  const bool vec_ok = ldc % 8 == 0 && reinterpret_cast<uintptr_t>(C) % (8 * sizeof(OutT)) == 0;
  gemm_tn_bf16_256_kernel<OutT><<<8 * per_xcd, G2_THREADS, kGemm2Lds, s>>>(
      A, W, C, M, N, K, lda, ldw, ldc, tm2, tn2, per_xcd, vec_ok);
  return hipGetLastError();
}

hipError_t launch_gemm_tn(const GemmArgs& g, hipStream_t s) {
  if (g.K % G2K != 0 || g.M < 1 || g.N < 1) return hipErrorInvalidValue;
  ProfScope ps(g.name, s);
  if (g.bf16_out)
    return launch_gemm_256(g.A, g.lda, g.W, g.ldw, static_cast<uint16_t*>(g.C), g.ldc, g.M, g.N,
                           g.K, s);
  return launch_gemm_256(g.A, g.lda, g.W, g.ldw, static_cast<float*>(g.C), g.ldc, g.M, g.N, g.K,
                         s);
}


// ============================================================================ helpers
__device__ float block_sum(float v, float* s_red) {
  const int tid = threadIdx.x;
  v = wave_sum_xor(v, 48);
#pragma unroll
  for (int off = 8; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  if ((tid & 63) == 0) s_red[tid >> 6] = v;
  __syncthreads();
  float t = 0.f;
  for (int w = 0; w < static_cast<int>(blockDim.x >> 6); ++w) t += s_red[w];
  __syncthreads();
  return t;
}
__device__ float block_max(float v, float* s_red) {
  const int tid = threadIdx.x;
  v = wave_max_xor(v, 48);
#pragma unroll
  for (int off = 8; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  if ((tid & 63) == 0) s_red[tid >> 6] = v;
  __syncthreads();
  float t = -INFINITY;
  for (int w = 0; w < static_cast<int>(blockDim.x >> 6); ++w) t = fmaxf(t, s_red[w]);
  __syncthreads();
  return t;
}

struct PoolParams {
  int mode, B, T, c, d_I, m, r, n_cols, tail_rows, tail_cols, n_max, nblk;
  int key_fmt;  // 0 E4M3 + per-entry scale, 1 MXFP4
  const int32_t* pos0;
  const float* proj;
  const float* tail;
  const float *bias_a, *bias_b, *bias_ia, *bias_ib, *gamma;
  const float* inv_freq;
  float eps;
  uint16_t* entries;
  uint8_t* ikeys;
  float* iscale;
  PageMap pages;               // layout of entries, ikeys and iscale
  const int32_t* n_keep;       // [B] entries already in the cache, kept as they are (or null)
  bool entry_mixed;            // entries as [c-r E4M3 codes | r bf16] rows (c + r bytes)
};

__device__ __forceinline__ const float* proj_row(const PoolParams& p, int b, int p0, int u) {
  if (u >= p0) return p.proj + (static_cast<size_t>(b) * p.T + (u - p0)) * p.n_cols;
  return p.tail + (static_cast<size_t>(b) * p.tail_rows + (u % p.tail_rows)) * p.tail_cols;
}

// Softmax-weighted pooling of one channel over the block's rows.  a-rows: tokens ma..ma+m-1
// using value column cv_a, logit column cz_a and bias ba; b-rows (if has_b): tokens mb..mb+m-1.
__device__ float pool_channel(const PoolParams& p, int b, int p0, int ma, int mb, bool has_b,
                              int cv_a, int cz_a, const float* ba, int cv_b, int cz_b,
                              const float* bb, int width, int ch) {
  float mx = -INFINITY;
  for (int r = 0; r < p.m; ++r) mx = fmaxf(mx, proj_row(p, b, p0, ma + r)[cz_a + ch] + ba[r * width + ch]);
  if (has_b)
    for (int r = 0; r < p.m; ++r)
      mx = fmaxf(mx, proj_row(p, b, p0, mb + r)[cz_b + ch] + bb[r * width + ch]);
  float den = 0.f, num = 0.f;
  for (int r = 0; r < p.m; ++r) {
    const float* rowp = proj_row(p, b, p0, ma + r);
    const float w = expf(rowp[cz_a + ch] + ba[r * width + ch] - mx);
    den += w;
    num += w * rowp[cv_a + ch];
  }
  if (has_b)
    for (int r = 0; r < p.m; ++r) {
      const float* rowp = proj_row(p, b, p0, mb + r);
      const float w = expf(rowp[cz_b + ch] + bb[r * width + ch] - mx);
      den += w;
      num += w * rowp[cv_b + ch];
    }
  return num / den;
}

__global__ __launch_bounds__(256) void pool_kernel(PoolParams p) {
  __shared__ float s_val[512];
  __shared__ float s_red[8];
  const int b = blockIdx.x / p.nblk;
  const int p0 = p.pos0 ? p.pos0[b] : 0;
  const int i = p0 / p.m + blockIdx.x % p.nblk;
  if (i > (p0 + p.T) / p.m - 1) return;  // block does not close in this call
  if (i >= p.n_max) return;               // never write past the cache
  if (p.n_keep && i < p.n_keep[b]) return;  // already in the cache (rebuilding state only)
  const size_t erow = entry_row(p.pages, p.n_max, b, i);
  const int tid = threadIdx.x;
  const int c = p.c;
  const bool csa = p.mode == 0;
  const int ma = p.m * i, mb = p.m * (i - 1);
  const bool has_b = csa && i >= 1;
  float ss = 0.f;
  for (int ch = tid; ch < c; ch += 256) {
    float v;
    if (csa)
      v = pool_channel(p, b, p0, ma, mb, has_b, 0, 2 * c, p.bias_a, c, 3 * c, p.bias_b, c, ch);
    else
      v = pool_channel(p, b, p0, ma, mb, false, 0, c, p.bias_a, 0, 0, nullptr, c, ch);
    s_val[ch] = v;
    ss += v * v;
  }
  const float tot = block_sum(ss, s_red);  // includes the barrier that publishes s_val
  const float inv_rms = rsqrtf(tot / c + p.eps);
  // bf16 row of c values, or (mixed) c - r E4M3 codes of the unrotated dims then r bf16
  unsigned char* dst = reinterpret_cast<unsigned char*>(p.entries) +
                       erow * static_cast<size_t>(p.entry_mixed ? c + p.r : 2 * c);
  const int pos = p.m * i;
  for (int pp = tid; pp < c / 2; pp += 256) {
    const int d = 2 * pp;
    float x0 = s_val[d] * inv_rms * p.gamma[d];
    float x1 = s_val[d + 1] * inv_rms * p.gamma[d + 1];
    if (d >= c - p.r) {
      float cs, sn;
      rope_cos_sin(pos, p.inv_freq[(d - (c - p.r)) >> 1], cs, sn);
      const float y0 = x0 * cs - x1 * sn, y1 = x0 * sn + x1 * cs;
      x0 = y0;
      x1 = y1;
    }
    if (!p.entry_mixed)
      *reinterpret_cast<uint32_t*>(dst + 2 * d) = pack_bf16x2(x0, x1);
    else if (d < c - p.r)
      *reinterpret_cast<uint16_t*>(dst + d) =
          static_cast<uint16_t>(e4m3_rne(x0) | (static_cast<uint32_t>(e4m3_rne(x1)) << 8));
    else
      *reinterpret_cast<uint32_t*>(dst + (c - p.r) + 2 * (d - (c - p.r))) = pack_bf16x2(x0, x1);
  }
  if (!csa) return;
  // indexer keys: same pooling on their own streams, then per-entry E4M3 quantisation or
  // MXFP4 blocks
  const int dI = p.d_I;
  const int base = 4 * c;
  float amax = 0.f;
  __syncthreads();
  for (int ch = tid; ch < dI; ch += 256) {
    const float v = pool_channel(p, b, p0, ma, mb, has_b, base, base + 2 * dI, p.bias_ia,
                                 base + dI, base + 3 * dI, p.bias_ib, dI, ch);
    s_val[ch] = v;
    amax = fmaxf(amax, fabsf(v));
  }
  if (p.key_fmt == 1) {
    // MXFP4: thread ch < dI (<= 128) holds channel ch; the 32 lanes of a half-wave form one
    // block: shared exponent floor(log2 max|v|) - 2 (frexp: max = f 2^ex, f in [0.5, 1)),
    // E8M0 byte exponent + 127, elements v / 2^exponent to E2M1, two per byte (even channel in
    // the low nibble).  Blocks past dI (dI < 128) get the unit scale byte.
    const bool has = tid < dI;
    const float v = has ? s_val[tid] : 0.f;
    float am = fabsf(v);
#pragma unroll
    for (int off = 16; off > 0; off >>= 1) am = fmaxf(am, __shfl_xor(am, off, 64));
    int ex;
    (void)frexpf(am, &ex);
    const int se = am > 0.f ? min(max(ex - 3, -127), 127) : -127;
    const uint32_t code = e2m1_rne(ldexpf(v, -se));
    const uint32_t hi = static_cast<uint32_t>(__shfl_down(static_cast<int>(code), 1, 64));
    uint8_t* kd = p.ikeys + erow * (dI / 2);
    if (has && (tid & 1) == 0) kd[tid >> 1] = static_cast<uint8_t>(code | (hi << 4));
    uint8_t* sd = reinterpret_cast<uint8_t*>(p.iscale) + erow * 4;
    if (tid < 128 && (tid & 31) == 0) sd[tid >> 5] = static_cast<uint8_t>(has ? se + 127 : 127);
    return;
  }
  amax = block_max(amax, s_red);
  const float scale = amax > 0.f ? amax / 448.f : 1.f;
  uint8_t* kd = p.ikeys + erow * dI;
  for (int ch = tid; ch < dI; ch += 256) kd[ch] = e4m3_rne(s_val[ch] / scale);
  if (tid == 0) p.iscale[erow] = scale;
}

// Window KV of every new token: RMSNorm(h_u W_win) * gamma_win, RoPE at u.
__global__ __launch_bounds__(256) void window_kernel(const float* __restrict__ proj, int T,
                                                     int n_cols, int c, int r, const int32_t* pos0,
                                                     const float* __restrict__ gamma_win,
                                                     const float* __restrict__ inv_freq, float eps,
                                                     uint16_t* __restrict__ window,
                                                     int win_slots) {
  __shared__ float s_red[8];
  const int bt = blockIdx.x;
  const int b = bt / T, tt = bt % T;
  const int u = (pos0 ? pos0[b] : 0) + tt;
  const float* src = proj + static_cast<size_t>(bt) * n_cols + (n_cols - c);
  const int tid = threadIdx.x;
  float x[4];  // c <= 512: two pairs per thread at most
  float ss = 0.f;
  int np = 0;
  for (int pp = tid; pp < c / 2; pp += 256, ++np) {
    x[2 * np] = src[2 * pp];
    x[2 * np + 1] = src[2 * pp + 1];
    ss += x[2 * np] * x[2 * np] + x[2 * np + 1] * x[2 * np + 1];
  }
  const float inv_rms = rsqrtf(block_sum(ss, s_red) / c + eps);
  uint16_t* dst = window + (static_cast<size_t>(b) * win_slots + (u % win_slots)) * c;
  np = 0;
  for (int pp = tid; pp < c / 2; pp += 256, ++np) {
    const int d = 2 * pp;
    float x0 = x[2 * np] * inv_rms * gamma_win[d];
    float x1 = x[2 * np + 1] * inv_rms * gamma_win[d + 1];
    if (d >= c - r) {
      float cs, sn;
      rope_cos_sin(u, inv_freq[(d - (c - r)) >> 1], cs, sn);
      const float y0 = x0 * cs - x1 * sn, y1 = x0 * sn + x1 * cs;
      x0 = y0;
      x1 = y1;
    }
    *reinterpret_cast<uint32_t*>(dst + d) = pack_bf16x2(x0, x1);
  }
}

// Copy the projections of the last tail_rows new tokens into the tail ring; update n_entries.
__global__ __launch_bounds__(256) void tail_kernel(const float* __restrict__ proj, int T, int n_cols,
                                                   int tail_rows, int tail_cols, int m,
                                                   const int32_t* pos0, float* __restrict__ tail,
                                                   int32_t* __restrict__ n_entries, int nrows) {
  const int b = blockIdx.x / nrows;
  const int j = blockIdx.x % nrows;
  const int p0 = pos0 ? pos0[b] : 0;
  const int tt = T - nrows + j;  // new-token index
  const int u = p0 + tt;
  const float* src = proj + (static_cast<size_t>(b) * T + tt) * n_cols;
  float* dst = tail + (static_cast<size_t>(b) * tail_rows + (u % tail_rows)) * tail_cols;
  for (int cc = threadIdx.x; cc < tail_cols; cc += 256) dst[cc] = src[cc];
  if (j == 0 && threadIdx.x == 0) n_entries[b] = (p0 + T) / m;
}

// ============================================================================ launch
size_t compress_workspace(int B, int T, int n_cols) {
  return (static_cast<size_t>(B) * T * n_cols * sizeof(float) + 255) & ~static_cast<size_t>(255);
}

hipError_t launch_compress(const CompressArgs& a, hipStream_t s) {
  const int M = a.B * a.T;
  const int tiles_m = (M + GBM - 1) / GBM, tiles_n = (a.n_cols + GBN - 1) / GBN;
  if (a.D % G2K == 0) {
    GemmArgs g;
    g.A = a.H;
    g.lda = a.D;
    g.W = a.W;
    g.ldw = a.D;
    g.C = a.proj;
    g.ldc = a.n_cols;
    g.M = M;
    g.N = a.n_cols;
    g.K = a.D;
    g.bf16_out = false;
    g.name = "compress_gemm";
    hipError_t e = launch_gemm_tn(g, s);
    if (e != hipSuccess) return e;
  } else {
    ProfScope ps("compress_gemm", s);
    gemm_tn_bf16_kernel<<<tiles_m * tiles_n, 256, 0, s>>>(a.H, a.W, a.proj, M, a.n_cols, a.D,
                                                          tiles_n);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  PoolParams p;
  p.mode = a.mode;
  p.B = a.B;
  p.T = a.T;
  p.c = a.c;
  p.d_I = a.d_I;
  p.m = a.m;
  p.r = a.r;
  p.n_cols = a.n_cols;
  p.tail_rows = a.tail_rows;
  p.tail_cols = a.tail_cols;
  p.n_max = a.n_max;
  p.nblk = a.T / a.m + 1;
  p.pos0 = a.pos0;
  p.proj = a.proj;
  p.tail = a.tail;
  p.bias_a = a.bias_a;
  p.bias_b = a.bias_b;
  p.bias_ia = a.bias_ia;
  p.bias_ib = a.bias_ib;
  p.gamma = a.gamma;
  p.inv_freq = a.inv_freq;
  p.eps = a.eps;
  p.entries = a.entries;
  p.ikeys = a.ikeys;
  p.iscale = a.iscale;
  p.key_fmt = a.key_fmt;
  p.pages = a.pages;
  p.n_keep = a.keep_existing ? a.n_entries : nullptr;
  p.entry_mixed = a.entry_mixed;
  {
    ProfScope ps("compress_pool", s);
    pool_kernel<<<a.B * p.nblk, 256, 0, s>>>(p);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    ProfScope ps("compress_window", s);
    window_kernel<<<M, 256, 0, s>>>(a.proj, a.T, a.n_cols, a.c, a.r, a.pos0, a.gamma_win,
                                    a.inv_freq, a.eps, a.window, a.win_slots);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nrows = a.T < a.tail_rows ? a.T : a.tail_rows;
  ProfScope ps("compress_tail", s);
  tail_kernel<<<a.B * nrows, 256, 0, s>>>(a.proj, a.T, a.n_cols, a.tail_rows, a.tail_cols, a.m,
                                          a.pos0, a.tail, a.n_entries, nrows);
  return hipGetLastError();
}

}  // namespace csa
