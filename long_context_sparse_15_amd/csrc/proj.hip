// Query-side projections and the grouped output projection for gfx950: the dense steps on
// either side of the attention path.
//
// Method: "DeepSeek V4 模型技术大全", chapter "Attention": section "CSA 的完整路径" gives
//   c^Q_t = h_t W^DQ,  q^I_t = c^Q_t W^IUQ (split into n_h^I heads),  w^I_t = h_t W_w;
// section "注意力实现细节" says queries are RMS-normalised and the output projection is grouped:
//   O = Concat_u O^[u],  z^[u] = O^[u] W^[u]_down (rank r_o),  y = Proj(Concat_u z^[u]).
// The attention query is c^Q W^UQ normalised per head.  Intermediates: c^Q and z are stored in
// bf16; q in bf16 (unrotated; RoPE happens in the attention kernels); q^I as E4M3 codes with one
// fp32 scale per (token, head), max|x| / 448, or (FP4 indexer query) as MXFP4: E2M1 codes with
// one E8M0 scale per 32 dims, shared exponent floor(log2 max|x|) - 2; w^I in fp32.
//
// Every product is the large-tile bf16 MFMA GEMM (launch_gemm_tn, fp32 accumulation).  The
// query up-projection writes its bf16 result straight into q (the attention-query heads) and a
// small bf16 buffer (the indexer-query heads); one pass then finishes them: a wave per head
// reads the head's row, normalises it in place (or takes its max for the E4M3 scale) with
// wave-wide reductions.  The normalisation thus reads the product rounded to bf16 (one bf16
// rounding more than a normalisation of the fp32 product; an fp32 buffer of the product cost
// 10.7 GB of extra traffic at 64K tokens).
#include <cmath>

#include "common.h"
#include "kernels.h"

namespace csa {

namespace {

constexpr size_t kProjChunkBytes = size_t{256} << 20;  // fp32 / bf16 chunk buffers

int chunk_rows(int BT, size_t row_bytes) {
  size_t r = kProjChunkBytes / row_bytes;
  r = r / 256 * 256;
  if (r < 256) r = 256;
  return static_cast<int>(r < static_cast<size_t>(BT) ? r : static_cast<size_t>(BT));
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// v summed over the wave: quad permutes, the mirrored half-row and row (DPP), then l^16 and l^32
// (lane swaps).
__device__ __forceinline__ float wave_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xb1, 0xf, 0xf, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4e, 0xf, 0xf, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xf, 0xf, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xf, 0xf, false));
  return wave_sum_xor16_32(v);
}

template <int N>
struct alignas(4 * N) Words {
  uint32_t v[N];
};

// One workgroup (4 waves) per token row.  Attention-query heads (c values of q each, normalised
// in place with gain gamma): a wave takes a head per pass, lane l the c/64 consecutive values
// from c/64*l, loaded as one vector; each wave keeps UNR heads' loads in flight before it
// reduces.  Indexer-query heads (d_I values of P each, E4M3 with max|x|/448 scale): d_I/8 lanes
// per head, 8 values (16 bytes) per lane, 64/(d_I/8) heads per wave pass.  MX: MXFP4 instead,
// four lanes per 32-dim block: the block's max from two lane swaps, E8M0 byte from its binary
// exponent, 8 E2M1 codes (one dword) per lane.
template <int C, int DI, bool MX>
__global__ __launch_bounds__(256) void query_finish_kernel(
    const uint16_t* __restrict__ P, int ldp, int n_h, int H_I, const float* __restrict__ gamma,
    float eps, uint16_t* __restrict__ q, uint8_t* __restrict__ qi, float* __restrict__ qi_scale) {
  constexpr int V = C / 64, QW = V / 2, UNR = 4;
  constexpr int LPH = DI / 8, HPW = 64 / LPH;
  static_assert(C % 128 == 0 && DI % 8 == 0 && LPH <= 64, "head widths");
  const int row = blockIdx.x;
  const int l = lane_id(), wave = threadIdx.x >> 6;
  float g[V];
#pragma unroll
  for (int i = 0; i < V; ++i) g[i] = gamma[l * V + i];
  uint16_t* qrow = q + static_cast<size_t>(row) * n_h * C + l * V;
  for (int h0 = wave * UNR; h0 < n_h; h0 += 4 * UNR) {
    Words<QW> w[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int hd = h0 + u < n_h ? h0 + u : n_h - 1;
      w[u] = *reinterpret_cast<const Words<QW>*>(qrow + static_cast<size_t>(hd) * C);
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      float x[V];
      float ss = 0.f;
#pragma unroll
      for (int j = 0; j < QW; ++j) {
        x[2 * j] = __uint_as_float(w[u].v[j] << 16);
        x[2 * j + 1] = __uint_as_float(w[u].v[j] & 0xffff0000u);
        ss += x[2 * j] * x[2 * j] + x[2 * j + 1] * x[2 * j + 1];
      }
      const float inv = rsqrtf(wave_sum(ss) / C + eps);
      Words<QW> o;
#pragma unroll
      for (int j = 0; j < QW; ++j)
        o.v[j] = pack_bf16x2(x[2 * j] * inv * g[2 * j], x[2 * j + 1] * inv * g[2 * j + 1]);
      if (h0 + u < n_h)
        *reinterpret_cast<Words<QW>*>(qrow + static_cast<size_t>(h0 + u) * C) = o;
    }
  }
  const int sub = l % LPH;
  for (int pass = wave; pass * HPW < H_I; pass += 4) {
    const int h = pass * HPW + l / LPH;
    if (h >= H_I) continue;
    const u32x4 w = *reinterpret_cast<const u32x4*>(P + static_cast<size_t>(row) * ldp + h * DI +
                                                    sub * 8);
    float x[8];
    float am = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[2 * j] = __uint_as_float(w[j] << 16);
      x[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
      am = fmaxf(am, fmaxf(fabsf(x[2 * j]), fabsf(x[2 * j + 1])));
    }
    if constexpr (MX) {
      am = fmaxf(am, __shfl_xor(am, 1, 64));
      am = fmaxf(am, __shfl_xor(am, 2, 64));
      int ex;
      (void)frexpf(am, &ex);  // am = f 2^ex, f in [0.5, 1): floor(log2 am) = ex - 1
      const int se = am > 0.f ? min(max(ex - 3, -127), 127) : -127;
      uint32_t code = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) code |= e2m1_rne(ldexpf(x[j], -se)) << (4 * j);
      const size_t rh = static_cast<size_t>(row) * H_I + h;
      *reinterpret_cast<uint32_t*>(qi + rh * (DI / 2) + sub * 4) = code;
      if ((sub & 3) == 0)
        reinterpret_cast<uint8_t*>(qi_scale)[rh * 4 + (sub >> 2)] = static_cast<uint8_t>(se + 127);
      continue;
    }
#pragma unroll
    for (int off = LPH / 2; off > 0; off >>= 1) am = fmaxf(am, __shfl_xor(am, off, 64));
    const float scale = am > 0.f ? am / 448.f : 1.f;
    uint32_t c[2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
      c[j] = static_cast<uint32_t>(e4m3_rne(x[4 * j] / scale)) |
             (static_cast<uint32_t>(e4m3_rne(x[4 * j + 1] / scale)) << 8) |
             (static_cast<uint32_t>(e4m3_rne(x[4 * j + 2] / scale)) << 16) |
             (static_cast<uint32_t>(e4m3_rne(x[4 * j + 3] / scale)) << 24);
    uint8_t* dst = qi + (static_cast<size_t>(row) * H_I + h) * DI + sub * 8;
    *reinterpret_cast<uint2*>(dst) = make_uint2(c[0], c[1]);
    if (sub == 0) qi_scale[static_cast<size_t>(row) * H_I + h] = scale;
  }
}

template <int C, int DI>
hipError_t launch_finish(const uint16_t* P, int ldp, const QueryProjArgs& a, hipStream_t s) {
  ProfScope ps("qproj_finish", s);
  if (a.qi_mx)
    query_finish_kernel<C, DI, true><<<a.BT, 256, 0, s>>>(P, ldp, a.n_h, a.qi ? a.H_I : 0,
                                                          a.gamma_q, a.eps, a.q, a.qi,
                                                          a.qi_scale);
  else
    query_finish_kernel<C, DI, false><<<a.BT, 256, 0, s>>>(P, ldp, a.n_h, a.qi ? a.H_I : 0,
                                                           a.gamma_q, a.eps, a.q, a.qi,
                                                           a.qi_scale);
  return hipGetLastError();
}

}  // namespace

size_t query_proj_workspace(int BT, int r_q, int n_h, int c, int H_I, int d_I) {
  (void)n_h;
  (void)c;
  return align256(static_cast<size_t>(BT) * r_q * sizeof(uint16_t)) +
         align256(static_cast<size_t>(BT) * H_I * d_I * sizeof(uint16_t));
}

hipError_t launch_query_proj(const QueryProjArgs& a, hipStream_t s) {
  const bool idx = a.qi != nullptr;
  const int H_I = idx ? a.H_I : 0;
  const int iw = H_I * a.d_I;  // indexer-query width
  unsigned char* p = static_cast<unsigned char*>(a.ws);
  uint16_t* cq = reinterpret_cast<uint16_t*>(p);
  uint16_t* qib = reinterpret_cast<uint16_t*>(p + align256(static_cast<size_t>(a.BT) * a.r_q * 2));
  GemmArgs g;
  // c^Q = h W^DQ (bf16) and w^I = h W_w (fp32, straight into the output)
  g = GemmArgs{a.H, a.D, a.w_dq, a.D, cq, a.r_q, a.BT, a.r_q, a.D, true, "qproj_down"};
  hipError_t e = launch_gemm_tn(g, s);
  if (e != hipSuccess) return e;
  if (idx) {
    g = GemmArgs{a.H, a.D, a.w_w, a.D, a.wi, H_I, a.BT, H_I, a.D, false, "qproj_w"};
    e = launch_gemm_tn(g, s);
    if (e != hipSuccess) return e;
  }
  // c^Q W^UQ into q (bf16, normalised below) and c^Q W^IUQ into the indexer-query buffer
  g = GemmArgs{cq, a.r_q, a.w_uq, a.r_q, a.q, a.n_h * a.c, a.BT, a.n_h * a.c, a.r_q, true,
               "qproj_up"};
  e = launch_gemm_tn(g, s);
  if (e != hipSuccess) return e;
  if (idx) {
    g = GemmArgs{cq, a.r_q, a.w_iuq, a.r_q, qib, iw, a.BT, iw, a.r_q, true, "qproj_up"};
    e = launch_gemm_tn(g, s);
    if (e != hipSuccess) return e;
  }
#define CSA_FINISH_CASE(C_, DI_) \
  if (a.c == C_ && (!idx || a.d_I == DI_)) return launch_finish<C_, DI_>(qib, iw, a, s);
  CSA_FINISH_CASE(512, 128)
  CSA_FINISH_CASE(512, 64)
  CSA_FINISH_CASE(512, 32)
  CSA_FINISH_CASE(256, 128)
  CSA_FINISH_CASE(256, 64)
  CSA_FINISH_CASE(256, 32)
  CSA_FINISH_CASE(128, 128)
  CSA_FINISH_CASE(128, 64)
  CSA_FINISH_CASE(128, 32)
#undef CSA_FINISH_CASE
  return hipErrorInvalidValue;
}

size_t output_proj_workspace(int BT, int g, int r_o) {
  const size_t width = static_cast<size_t>(g) * r_o;
  return align256(static_cast<size_t>(chunk_rows(BT, width * 2)) * width * sizeof(uint16_t));
}

hipError_t launch_output_proj(const OutputProjArgs& a, hipStream_t s) {
  const int zw = a.g * a.r_o;                 // width of Concat_u z^[u]
  const int gw = a.n_h / a.g * a.c;           // input width of one group
  const int ow = a.n_h * a.c;                 // row width of O
  uint16_t* z = static_cast<uint16_t*>(a.ws);
  const int rows = chunk_rows(a.BT, static_cast<size_t>(zw) * 2);
  for (int r0 = 0; r0 < a.BT; r0 += rows) {
    const int m = a.BT - r0 < rows ? a.BT - r0 : rows;
    for (int u = 0; u < a.g; ++u) {
      const GemmArgs g{a.O + static_cast<size_t>(r0) * ow + static_cast<size_t>(u) * gw, ow,
                       a.w_down + static_cast<size_t>(u) * a.r_o * gw, gw, z + u * a.r_o, zw,
                       m, a.r_o, gw, true, "oproj_down"};
      hipError_t e = launch_gemm_tn(g, s);
      if (e != hipSuccess) return e;
    }
    const GemmArgs g{z, zw, a.w_proj, zw, a.y + static_cast<size_t>(r0) * a.D, a.D, m, a.D, zw,
                     true, "oproj_up"};
    hipError_t e = launch_gemm_tn(g, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace csa
