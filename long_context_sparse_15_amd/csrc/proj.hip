// Query-side projections and the grouped output projection for gfx950: the dense steps on
// either side of the attention path.
//
// Method: "DeepSeek V4 模型技术大全", chapter "Attention": section "CSA 的完整路径" gives
//   c^Q_t = h_t W^DQ,  q^I_t = c^Q_t W^IUQ (split into n_h^I heads),  w^I_t = h_t W_w;
// section "注意力实现细节" says queries are RMS-normalised and the output projection is grouped:
//   O = Concat_u O^[u],  z^[u] = O^[u] W^[u]_down (rank r_o),  y = Proj(Concat_u z^[u]).
// The attention query is c^Q W^UQ normalised per head.  Intermediates: c^Q and z are stored in
// bf16; q in bf16 (unrotated; RoPE happens in the attention kernels); q^I as E4M3 codes with one
// fp32 scale per (token, head), max|x| / 448; w^I in fp32.
//
// Every product is the large-tile bf16 MFMA GEMM (launch_gemm_tn, fp32 accumulation).  The
// fp32 results of the query up-projection are produced in row chunks sized to a bounded
// workspace and finished by one pass: a wave per head reads the head's row, normalises it (or
// takes its max for the E4M3 scale) with wave-wide reductions and stores the result.
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

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

// One workgroup (4 waves) per token row of the chunk; wave w takes "heads" w, w+4, ... of the
// row: the first n_h are attention-query heads (c floats each: RMSNorm with gain gamma, bf16),
// the next H_I are indexer-query heads (d_I floats each: E4M3 with max|x|/448 scale).
template <int C, int DI>
__global__ __launch_bounds__(256) void query_finish_kernel(
    const float* __restrict__ P, int ldp, int n_h, int H_I, const float* __restrict__ gamma,
    float eps, uint16_t* __restrict__ q, uint8_t* __restrict__ qi, float* __restrict__ qi_scale) {
  constexpr int PERQ = C / 64, PERI = DI / 64 > 0 ? DI / 64 : 1;
  const int row = blockIdx.x;
  const int l = lane_id(), wave = threadIdx.x >> 6;
  const float* src = P + static_cast<size_t>(row) * ldp;
  for (int hd = wave; hd < n_h + H_I; hd += 4) {
    if (hd < n_h) {
      float x[PERQ];
      float ss = 0.f;
#pragma unroll
      for (int i = 0; i < PERQ; ++i) {
        x[i] = src[hd * C + i * 64 + l];
        ss += x[i] * x[i];
      }
      const float inv = rsqrtf(wave_sum(ss) / C + eps);
      uint16_t* dst = q + (static_cast<size_t>(row) * n_h + hd) * C;
#pragma unroll
      for (int i = 0; i < PERQ; ++i) dst[i * 64 + l] = f32_to_bf16(x[i] * inv * gamma[i * 64 + l]);
    } else {
      const int h = hd - n_h;
      const float* s2 = src + n_h * C + h * DI;
      float x[PERI];
      float am = 0.f;
#pragma unroll
      for (int i = 0; i < PERI; ++i) {
        const int d = i * 64 + l;
        x[i] = d < DI ? s2[d] : 0.f;
        am = fmaxf(am, fabsf(x[i]));
      }
      am = wave_max(am);
      const float scale = am > 0.f ? am / 448.f : 1.f;
      uint8_t* dst = qi + (static_cast<size_t>(row) * H_I + h) * DI;
#pragma unroll
      for (int i = 0; i < PERI; ++i) {
        const int d = i * 64 + l;
        if (d < DI) dst[d] = e4m3_rne(x[i] / scale);
      }
      if (l == 0) qi_scale[static_cast<size_t>(row) * H_I + h] = scale;
    }
  }
}

template <int C, int DI>
hipError_t launch_finish(const float* P, int ldp, int rows, const QueryProjArgs& a, int r0,
                         hipStream_t s) {
  ProfScope ps("qproj_finish", s);
  query_finish_kernel<C, DI><<<rows, 256, 0, s>>>(
      P, ldp, a.n_h, a.qi ? a.H_I : 0, a.gamma_q, a.eps,
      a.q + static_cast<size_t>(r0) * a.n_h * a.c,
      a.qi ? a.qi + static_cast<size_t>(r0) * a.H_I * a.d_I : nullptr,
      a.qi ? a.qi_scale + static_cast<size_t>(r0) * a.H_I : nullptr);
  return hipGetLastError();
}

}  // namespace

size_t query_proj_workspace(int BT, int r_q, int n_h, int c, int H_I, int d_I) {
  const size_t width = static_cast<size_t>(n_h) * c + static_cast<size_t>(H_I) * d_I;
  const int rows = chunk_rows(BT, width * sizeof(float));
  return align256(static_cast<size_t>(BT) * r_q * sizeof(uint16_t)) +
         align256(static_cast<size_t>(rows) * width * sizeof(float));
}

hipError_t launch_query_proj(const QueryProjArgs& a, hipStream_t s) {
  const bool idx = a.qi != nullptr;
  const int H_I = idx ? a.H_I : 0;
  const int width = a.n_h * a.c + H_I * a.d_I;
  unsigned char* p = static_cast<unsigned char*>(a.ws);
  uint16_t* cq = reinterpret_cast<uint16_t*>(p);
  float* buf = reinterpret_cast<float*>(p + align256(static_cast<size_t>(a.BT) * a.r_q * 2));
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
  const int rows = chunk_rows(a.BT, static_cast<size_t>(width) * sizeof(float));
  for (int r0 = 0; r0 < a.BT; r0 += rows) {
    const int m = a.BT - r0 < rows ? a.BT - r0 : rows;
    const uint16_t* A = cq + static_cast<size_t>(r0) * a.r_q;
    g = GemmArgs{A, a.r_q, a.w_uq, a.r_q, buf, width, m, a.n_h * a.c, a.r_q, false, "qproj_up"};
    e = launch_gemm_tn(g, s);
    if (e != hipSuccess) return e;
    if (idx) {
      g = GemmArgs{A, a.r_q, a.w_iuq, a.r_q, buf + a.n_h * a.c, width, m, H_I * a.d_I, a.r_q,
                   false, "qproj_up"};
      e = launch_gemm_tn(g, s);
      if (e != hipSuccess) return e;
    }
#define CSA_FINISH_CASE(C_, DI_)                                         \
    if (a.c == C_ && (!idx || a.d_I == DI_)) {                           \
      e = launch_finish<C_, DI_>(buf, width, m, a, r0, s);               \
      if (e != hipSuccess) return e;                                     \
      continue;                                                          \
    }
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
  return hipSuccess;
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
