// C ABI of libcsa.so: argument validation, workspace layout and kernel sequencing.
// The operations and their definitions are documented in include/csa.h.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <initializer_list>
#include <mutex>
#include <string>

#include "../../include/csa.h"

#include "kernels.h"

namespace {

thread_local std::string g_last_error;

int vfail(int code, const char* fmt, va_list ap) {
  char buf[512];
  vsnprintf(buf, sizeof(buf), fmt, ap);
  g_last_error = buf;
  return code;
}

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  const int rc = vfail(code, fmt, ap);
  va_end(ap);
  return rc;
}

}  // namespace

namespace csa {
// Records the calling thread's last error (csa_last_error) and returns `code`; for the other
// host-side parts of the library.
int api_fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  const int rc = vfail(code, fmt, ap);
  va_end(ap);
  return rc;
}
}  // namespace csa

// Static scratch of csa_decode_noalloc (see scratch_of_current_device below).
static __device__ __align__(256) unsigned char scratch[CSA_NOALLOC_SCRATCH_BYTES];

namespace {

// Positions of a chunk's queries: pos[b][i] = pos0[b] + i.
__global__ __launch_bounds__(256) void chunk_positions_kernel(const int32_t* __restrict__ pos0,
                                                              int T, int32_t* __restrict__ pos) {
  const int b = blockIdx.y;
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < T) pos[static_cast<size_t>(b) * T + i] = pos0[b] + i;
}

hipError_t launch_chunk_positions(const int32_t* pos0, int B, int T, int32_t* pos,
                                  hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((T + 255) / 256), static_cast<unsigned>(B));
  chunk_positions_kernel<<<grid, 256, 0, s>>>(pos0, T, pos);
  return hipGetLastError();
}

int hip_fail(hipError_t e, const char* where) {
  return fail(CSA_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

bool is_csa(const csa_config_t* c) { return c->mode == CSA_MODE_CSA; }

int check_config(const csa_config_t* c, bool need_compressor) {
  if (!c) return fail(CSA_ERR_INVALID_ARG, "cfg is NULL");
  if (c->mode != CSA_MODE_CSA && c->mode != CSA_MODE_HCA)
    return fail(CSA_ERR_INVALID_ARG, "mode %d is neither CSA nor HCA", c->mode);
  if (c->m < 1) return fail(CSA_ERR_INVALID_ARG, "m=%d < 1", c->m);
  if (c->head_dim != 128 && c->head_dim != 256 && c->head_dim != 512)
    return fail(CSA_ERR_INVALID_ARG, "head_dim=%d not in {128, 256, 512}", c->head_dim);
  if (c->rope_dim < 2 || (c->rope_dim & 1) || c->rope_dim > c->head_dim || c->rope_dim > 128)
    return fail(CSA_ERR_INVALID_ARG, "rope_dim=%d must be even, 2..min(head_dim,128)",
                c->rope_dim);
  if (c->n_heads < 1 || c->n_heads > 128)
    return fail(CSA_ERR_INVALID_ARG, "n_heads=%d not in 1..128", c->n_heads);
  if (c->n_win < 1 || c->n_win > 1024)
    return fail(CSA_ERR_INVALID_ARG, "n_win=%d not in 1..1024", c->n_win);
  if (!(c->softmax_scale > 0.f) || !std::isfinite(c->softmax_scale))
    return fail(CSA_ERR_INVALID_ARG, "softmax_scale must be finite and > 0");
  if (!(c->rms_eps >= 0.f)) return fail(CSA_ERR_INVALID_ARG, "rms_eps must be >= 0");
  if (!c->rope_inv_freq) return fail(CSA_ERR_INVALID_ARG, "rope_inv_freq is NULL");
  if (is_csa(c)) {
    if (c->idx_dim != 32 && c->idx_dim != 64 && c->idx_dim != 128)
      return fail(CSA_ERR_INVALID_ARG, "idx_dim=%d not in {32, 64, 128}", c->idx_dim);
    if (c->idx_heads < 1 || c->idx_heads > 64)
      return fail(CSA_ERR_INVALID_ARG, "idx_heads=%d not in 1..64", c->idx_heads);
    if (c->top_k < 1 || c->top_k > csa::kMaxTopK)
      return fail(CSA_ERR_INVALID_ARG, "top_k=%d not in 1..%d", c->top_k, csa::kMaxTopK);
    if (c->idx_key_format != CSA_IDX_E4M3 && c->idx_key_format != CSA_IDX_MXFP4)
      return fail(CSA_ERR_INVALID_ARG, "idx_key_format=%d is neither E4M3 nor MXFP4",
                  c->idx_key_format);
    if (c->idx_query_format != CSA_IDX_E4M3 && c->idx_query_format != CSA_IDX_MXFP4)
      return fail(CSA_ERR_INVALID_ARG, "idx_query_format=%d is neither E4M3 nor MXFP4",
                  c->idx_query_format);
    if (c->idx_query_format == CSA_IDX_MXFP4 && c->idx_key_format != CSA_IDX_MXFP4)
      return fail(CSA_ERR_UNSUPPORTED, "an MXFP4 indexer query needs MXFP4 keys");
    if (c->score_format != CSA_SCORE_FP32 && c->score_format != CSA_SCORE_BF16)
      return fail(CSA_ERR_INVALID_ARG, "score_format=%d is neither FP32 nor BF16",
                  c->score_format);
  }
  if (c->entry_format != CSA_ENT_BF16 && c->entry_format != CSA_ENT_MIXED)
    return fail(CSA_ERR_INVALID_ARG, "entry_format=%d is neither BF16 nor MIXED",
                c->entry_format);
  if (c->entry_format == CSA_ENT_MIXED && (c->head_dim != 512 || c->rope_dim % 16))
    return fail(CSA_ERR_UNSUPPORTED, "mixed entries need head_dim 512 and rope_dim a multiple "
                "of 16 (head_dim=%d, rope_dim=%d)", c->head_dim, c->rope_dim);
  if (need_compressor) {
    if (c->hidden < 32 || (c->hidden % 32))
      return fail(CSA_ERR_INVALID_ARG, "hidden=%d must be a positive multiple of 32", c->hidden);
  }
  return CSA_OK;
}

int weight_cols(const csa_config_t* c) {
  return is_csa(c) ? 5 * c->head_dim + 4 * c->idx_dim : 3 * c->head_dim;
}
void tail_shape(const csa_config_t* c, int* rows, int* cols) {
  if (is_csa(c)) {
    *rows = 2 * c->m;
    *cols = 4 * c->head_dim + 4 * c->idx_dim;
  } else {
    *rows = c->m;
    *cols = 2 * c->head_dim;
  }
}

// CSA_ERR_INVALID_ARG unless every non-NULL pointer is 16-byte aligned.
int check_aligned(std::initializer_list<const void*> ptrs) {
  for (const void* p : ptrs)
    if (reinterpret_cast<uintptr_t>(p) & 15)
      return fail(CSA_ERR_INVALID_ARG, "device pointer %p is not 16-byte aligned", p);
  return CSA_OK;
}

// The caller's workspace: at least `need` bytes (CSA_ERR_WORKSPACE) and 256-byte aligned as
// documented (the kernels move scores and partials in 16-byte vectors from 256-byte aligned
// sub-buffers).  A NULL workspace is accepted when the operation needs none.
int check_workspace(const void* ws, size_t ws_bytes, size_t need) {
  if (need && (!ws || ws_bytes < need))
    return fail(CSA_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  if (reinterpret_cast<uintptr_t>(ws) & 255)
    return fail(CSA_ERR_INVALID_ARG, "workspace %p is not 256-byte aligned", ws);
  return CSA_OK;
}

int check_cache(const csa_config_t* c, const csa_cache_t* k, bool need_keys, bool need_tail) {
  if (!k) return fail(CSA_ERR_INVALID_ARG, "cache is NULL");
  if (k->n_max < 1) return fail(CSA_ERR_INVALID_ARG, "cache n_max=%d < 1", k->n_max);
  if (k->win_slots < c->n_win)
    return fail(CSA_ERR_INVALID_ARG, "cache win_slots=%d < n_win=%d", k->win_slots, c->n_win);
  if (!k->entries || !k->window || !k->n_entries)
    return fail(CSA_ERR_INVALID_ARG, "cache entries/window/n_entries is NULL");
  if (need_keys && (!k->idx_keys || !k->idx_scale))
    return fail(CSA_ERR_INVALID_ARG, "cache idx_keys/idx_scale is NULL");
  if (need_tail && !k->tail) return fail(CSA_ERR_INVALID_ARG, "cache tail is NULL");
  if (int rc = check_aligned({k->entries, k->idx_keys, k->window, k->tail})) return rc;
  if (k->block_entries != 0) {
    const int be = k->block_entries;
    if (be < 0 || (be & (be - 1)))
      return fail(CSA_ERR_INVALID_ARG, "block_entries=%d must be 0 or a power of two", be);
    if (is_csa(c) && be < 16)
      return fail(CSA_ERR_INVALID_ARG, "CSA caches need block_entries >= 16 (got %d)", be);
    if (!k->block_table || k->blocks_per_seq < 1 || k->n_blocks < 1)
      return fail(CSA_ERR_INVALID_ARG, "paged cache needs block_table, blocks_per_seq >= 1 "
                  "and n_blocks >= 1");
    if (static_cast<long long>(k->blocks_per_seq) * be != k->n_max)
      return fail(CSA_ERR_INVALID_ARG, "n_max=%d != blocks_per_seq*block_entries=%lld",
                  k->n_max, static_cast<long long>(k->blocks_per_seq) * be);
    if (static_cast<long long>(k->n_blocks) * be >= (1LL << 31))
      return fail(CSA_ERR_INVALID_ARG, "pool of %d blocks x %d entries exceeds 2^31 rows",
                  k->n_blocks, be);
  }
  return CSA_OK;
}

csa::PageMap page_map(const csa_cache_t* k) {
  csa::PageMap pm;
  if (k->block_entries > 0) {
    pm.table = k->block_table;
    pm.stride = k->blocks_per_seq;
    int sh = 0;
    while ((1 << sh) < k->block_entries) ++sh;
    pm.shift = sh;
    pm.n_blocks = k->n_blocks;
  }
  return pm;
}

int check_weights(const csa_config_t* c, const csa_weights_t* w) {
  if (!w) return fail(CSA_ERR_INVALID_ARG, "weights are NULL");
  if (!w->w_cat || !w->bias_a || !w->gamma || !w->gamma_win)
    return fail(CSA_ERR_INVALID_ARG, "w_cat/bias_a/gamma/gamma_win is NULL");
  if (is_csa(c) && (!w->bias_b || !w->bias_ia || !w->bias_ib))
    return fail(CSA_ERR_INVALID_ARG, "CSA needs bias_b, bias_ia and bias_ib");
  return CSA_OK;
}

// Selection over rows longer than kRowTopkBigN entries runs on the multi-workgroup path, whose
// per-call row count is bounded; longer rows in bigger batches are refused, not truncated.
int check_index_rows(const csa_config_t* c, long long rows, int n_max) {
  if (is_csa(c) && n_max > csa::kRowTopkBigN && rows > csa::kMultiMaxRows)
    return fail(CSA_ERR_UNSUPPORTED, "%lld query rows over caches of n_max=%d > %d entries: "
                "call with at most %d query rows at a time", rows, n_max, csa::kRowTopkBigN,
                csa::kMultiMaxRows);
  return CSA_OK;
}

// --- workspace layouts ----------------------------------------------------------------------
size_t ws_compress(const csa_config_t* c, int B, int T) {
  return csa::compress_workspace(B, T, weight_cols(c));
}
size_t ws_index(const csa_config_t* c, int B, int nq, int n_max) {
  return csa::index_topk_workspace(B * nq, nq, n_max, c->idx_dim, c->idx_heads,
                                   c->score_format == CSA_SCORE_BF16);
}
size_t ws_mqa(const csa_config_t* c, int B, int nq, int max_list) {
  const csa::MqaPlan p = csa::plan_mqa(nq, c->n_heads, c->head_dim, max_list, c->entry_format == CSA_ENT_MIXED);
  return csa::mqa_workspace(p, B * nq, c->n_heads, c->head_dim);
}
int max_list_sparse(const csa_config_t* c) { return c->top_k + c->n_win; }
int max_list_dense(const csa_config_t* c, int n_max) { return n_max + c->n_win; }

size_t ws_attend(const csa_config_t* c, int B, int nq, int n_max) {
  return is_csa(c) ? ws_mqa(c, B, nq, max_list_sparse(c))
                   : ws_mqa(c, B, nq, max_list_dense(c, n_max));
}

// decode / prefill: [idx buffer (CSA)] + [query positions (prefill)] + union(compress, index,
// attend)
size_t ws_layer(const csa_config_t* c, int B, int T, int n_max, bool prefill, bool compress) {
  const int rows = B * T;
  size_t idx = is_csa(c) ? align256(static_cast<size_t>(rows) * c->top_k * 4) : 0;
  if (prefill) idx += align256(static_cast<size_t>(rows) * 4);  // query positions (chunked)
  size_t u = ws_attend(c, B, T, n_max);
  if (is_csa(c)) u = std::max(u, ws_index(c, B, T, n_max));
  if (compress) u = std::max(u, ws_compress(c, B, prefill ? T : 1));
  return idx + u;
}

void fill_index_args(csa::IndexArgs& a, const csa_config_t* c, int B, int nq, const uint8_t* qi,
                     const float* qi_scale, const float* wi, const csa_cache_t* k,
                     const int32_t* pos, int32_t* idx_out, float* score_out, void* ws) {
  a.qi = qi;
  a.qi_scale = qi_scale;
  a.wi = wi;
  a.keys = k->idx_keys;
  a.kscale = k->idx_scale;
  a.n_entries = k->n_entries;
  a.pos = pos;
  a.B = B;
  a.nq = nq;
  a.n_max = k->n_max;
  a.H_I = c->idx_heads;
  a.d_I = c->idx_dim;
  a.m = c->m;
  a.k = c->top_k;
  a.key_fmt = c->idx_key_format;
  a.q_fmt = c->idx_query_format;
  a.score_bf16 = c->score_format == CSA_SCORE_BF16;
  a.pages = page_map(k);
  a.idx_out = idx_out;
  a.score_out = score_out;
  csa::index_topk_layout(a, ws, B * nq);
}

void fill_mqa_args(csa::MqaArgs& a, const csa_config_t* c, int B, int nq, const uint16_t* q,
                   const csa_cache_t* k, const int32_t* idx, const int32_t* pos,
                   const float* sink, uint16_t* out, float* lse_out, void* ws) {
  a.q = q;
  a.entries = k->entries;
  a.window = k->window;
  a.idx = idx;
  a.n_entries = k->n_entries;
  a.pos = pos;
  a.sink = sink;
  a.inv_freq = c->rope_inv_freq;
  a.B = B;
  a.nq = nq;
  a.n_heads = c->n_heads;
  a.c = c->head_dim;
  a.r = c->rope_dim;
  a.k = c->top_k;
  a.m = c->m;
  a.n_win = c->n_win;
  a.win_slots = k->win_slots;
  a.n_max = k->n_max;
  a.pages = page_map(k);
  a.entry_mixed = c->entry_format == CSA_ENT_MIXED;
  a.scale = c->softmax_scale;
  a.out = out;
  a.lse_out = lse_out;
  a.part = static_cast<float*>(ws);
}

int run_compress(const csa_config_t* c, int B, int T, const uint16_t* H, const int32_t* pos0,
                 const csa_weights_t* w, const csa_cache_t* k, void* ws, hipStream_t s,
                 bool keep_existing = true) {
  csa::CompressArgs a;
  a.mode = c->mode;
  a.B = B;
  a.T = T;
  a.D = c->hidden;
  a.c = c->head_dim;
  a.d_I = is_csa(c) ? c->idx_dim : 0;
  a.key_fmt = is_csa(c) ? c->idx_key_format : 0;
  a.m = c->m;
  a.r = c->rope_dim;
  a.n_cols = weight_cols(c);
  tail_shape(c, &a.tail_rows, &a.tail_cols);
  a.win_slots = k->win_slots;
  a.n_max = k->n_max;
  a.H = H;
  a.pos0 = pos0;
  a.W = w->w_cat;
  a.bias_a = w->bias_a;
  a.bias_b = w->bias_b;
  a.bias_ia = w->bias_ia;
  a.bias_ib = w->bias_ib;
  a.gamma = w->gamma;
  a.gamma_win = w->gamma_win;
  a.inv_freq = c->rope_inv_freq;
  a.eps = c->rms_eps;
  a.entries = k->entries;
  a.ikeys = k->idx_keys;
  a.iscale = k->idx_scale;
  a.window = k->window;
  a.tail = k->tail;
  a.n_entries = k->n_entries;
  a.pages = page_map(k);
  a.keep_existing = keep_existing;
  a.entry_mixed = c->entry_format == CSA_ENT_MIXED;
  a.proj = static_cast<float*>(ws);
  hipError_t e = csa::launch_compress(a, s);
  return e == hipSuccess ? CSA_OK : hip_fail(e, "compress launch");
}

int run_index(const csa_config_t* c, int B, int nq, const uint8_t* qi, const float* qi_scale,
              const float* wi, const csa_cache_t* k, const int32_t* pos, int32_t* idx_out,
              float* score_out, void* ws, hipStream_t s) {
  csa::IndexArgs a;
  fill_index_args(a, c, B, nq, qi, qi_scale, wi, k, pos, idx_out, score_out, ws);
  hipError_t e = csa::launch_index_topk(a, s);
  return e == hipSuccess ? CSA_OK : hip_fail(e, "index_topk launch");
}

int run_attend(const csa_config_t* c, int B, int nq, const uint16_t* q, const csa_cache_t* k,
               const int32_t* idx, const int32_t* pos, const float* sink, uint16_t* out,
               float* lse_out, void* ws, hipStream_t s) {
  csa::MqaArgs a;
  fill_mqa_args(a, c, B, nq, q, k, idx, pos, sink, out, lse_out, ws);
  const int max_list = idx ? max_list_sparse(c) : max_list_dense(c, k->n_max);
  const csa::MqaPlan p = csa::plan_mqa(nq, c->n_heads, c->head_dim, max_list, c->entry_format == CSA_ENT_MIXED);
  hipError_t e = csa::launch_mqa(a, p, s);
  return e == hipSuccess ? CSA_OK : hip_fail(e, "attention launch");
}

int check_qproj_config(const csa_config_t* c) {
  if (c->hidden < 64 || c->hidden % 64)
    return fail(CSA_ERR_INVALID_ARG, "hidden=%d must be a positive multiple of 64", c->hidden);
  if (c->q_rank < 64 || c->q_rank % 64)
    return fail(CSA_ERR_INVALID_ARG, "q_rank=%d must be a positive multiple of 64", c->q_rank);
  return CSA_OK;
}

int check_oproj_config(const csa_config_t* c) {
  if (c->hidden < 1) return fail(CSA_ERR_INVALID_ARG, "hidden=%d < 1", c->hidden);
  if (c->out_groups < 1 || c->n_heads % c->out_groups)
    return fail(CSA_ERR_INVALID_ARG, "out_groups=%d must divide n_heads=%d", c->out_groups,
                c->n_heads);
  if ((c->n_heads / c->out_groups * c->head_dim) % 64)
    return fail(CSA_ERR_INVALID_ARG, "a group's width (n_heads/out_groups*head_dim) must be a "
                "multiple of 64");
  if (c->out_rank < 1 || (c->out_groups * c->out_rank) % 64)
    return fail(CSA_ERR_INVALID_ARG, "out_groups*out_rank=%d must be a positive multiple of 64",
                c->out_groups * c->out_rank);
  return CSA_OK;
}

// Validation shared by csa_decode and csa_decode_noalloc; *need receives the scratch bytes the
// step uses (index buffer, then the union of the compressor, scorer and attention buffers).
int decode_check(const csa_config_t* cfg, int32_t B, const uint16_t* h_new,
                 const csa_weights_t* w, const csa_cache_t* cache, const int32_t* pos,
                 const uint16_t* q, const uint8_t* qi, const float* qi_scale, const float* wi,
                 const float* sink, const uint16_t* out, size_t* need) {
  const bool comp = h_new != nullptr;
  int rc = check_config(cfg, comp);
  if (rc) return rc;
  if ((rc = check_cache(cfg, cache, is_csa(cfg), comp))) return rc;
  if (comp && (rc = check_weights(cfg, w))) return rc;
  if (B < 1) return fail(CSA_ERR_INVALID_ARG, "B=%d must be >= 1", B);
  if ((rc = check_index_rows(cfg, B, cache->n_max))) return rc;
  if (!pos || !q || !sink || !out) return fail(CSA_ERR_INVALID_ARG, "pos/q/sink/out is NULL");
  if ((rc = check_aligned({h_new, q, qi, out, w ? w->w_cat : nullptr}))) return rc;
  if (is_csa(cfg) && (!qi || !qi_scale || !wi))
    return fail(CSA_ERR_INVALID_ARG, "CSA decode needs qi, qi_scale and wi");
  *need = ws_layer(cfg, B, 1, cache->n_max, false, comp);
  return CSA_OK;
}

// One decode step on already validated arguments, with scratch ws.
int decode_run(const csa_config_t* cfg, int32_t B, const uint16_t* h_new,
               const csa_weights_t* w, const csa_cache_t* cache, const int32_t* pos,
               const uint16_t* q, const uint8_t* qi, const float* qi_scale, const float* wi,
               const float* sink, uint16_t* out, int32_t* idx_out, void* ws, hipStream_t s) {
  int rc = CSA_OK;
  unsigned char* p = static_cast<unsigned char*>(ws);
  int32_t* idx = nullptr;
  if (is_csa(cfg)) {
    idx = idx_out ? idx_out : reinterpret_cast<int32_t*>(p);
    p += align256(static_cast<size_t>(B) * cfg->top_k * 4);
  }
  if (h_new && (rc = run_compress(cfg, B, 1, h_new, pos, w, cache, p, s))) return rc;
  if (is_csa(cfg)) {
    if ((rc = run_index(cfg, B, 1, qi, qi_scale, wi, cache, pos, idx, nullptr, p, s))) return rc;
    return run_attend(cfg, B, 1, q, cache, idx, pos, sink, out, nullptr, p, s);
  }
  return run_attend(cfg, B, 1, q, cache, nullptr, pos, sink, out, nullptr, p, s);
}

// ---- static scratch of csa_decode_noalloc ---------------------------------------------------
// One file-scope device array: every GPU the library runs on holds its own copy, at its own
// address, until the process ends.  Host code never passes the array's name to a kernel (on the
// host it only names the symbol); it takes each device's address once, with that device current,
// through hipGetSymbolAddress and uses that pointer.  No decode buffer has to start zeroed:
// every scratch byte a kernel reads was written earlier in the same call.
constexpr size_t kScratchBytes = CSA_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

int scratch_of_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxScratchDevices)
    return fail(CSA_ERR_UNSUPPORTED, "device %d is beyond the %d devices the static scratch "
                "tracks", dev, kMaxScratchDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(CSA_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return CSA_OK;
}

}  // namespace

extern "C" {

int csa_version(void) { return 1 * 10000 + 3 * 100 + 0; }

int csa_profile_start(void) {
  csa::profile_start();
  return CSA_OK;
}

int csa_profile_stop(csa_kernel_time_t* out, int32_t max_out, int32_t* n_out) {
  if (!out || !n_out || max_out < 0) return fail(CSA_ERR_INVALID_ARG, "out/n_out is NULL");
  static_assert(sizeof(csa_kernel_time_t) == sizeof(csa::ProfTotal), "layout");
  int n = 0;
  const int rc = csa::profile_stop(reinterpret_cast<csa::ProfTotal*>(out), max_out, &n);
  *n_out = n;
  return rc == 0 ? CSA_OK : fail(CSA_ERR_HIP, "waiting for timing events failed");
}

const char* csa_last_error(void) { return g_last_error.c_str(); }

int csa_weight_cols(const csa_config_t* cfg, int32_t* n_cols) {
  int rc = check_config(cfg, false);
  if (rc) return rc;
  if (!n_cols) return fail(CSA_ERR_INVALID_ARG, "n_cols is NULL");
  *n_cols = weight_cols(cfg);
  return CSA_OK;
}

int csa_tail_shape(const csa_config_t* cfg, int32_t* rows, int32_t* cols) {
  int rc = check_config(cfg, false);
  if (rc) return rc;
  if (!rows || !cols) return fail(CSA_ERR_INVALID_ARG, "rows/cols is NULL");
  int r, c;
  tail_shape(cfg, &r, &c);
  *rows = r;
  *cols = c;
  return CSA_OK;
}

int csa_workspace_size(const csa_config_t* cfg, int32_t op, int32_t B, int32_t nq, int32_t n_max,
                       size_t* bytes) {
  int rc = check_config(cfg, op == CSA_OP_COMPRESS || op == CSA_OP_PREFILL);
  if (rc) return rc;
  if (!bytes) return fail(CSA_ERR_INVALID_ARG, "bytes is NULL");
  if (B < 1 || nq < 1 || n_max < 1) return fail(CSA_ERR_INVALID_ARG, "B, nq, n_max must be >= 1");
  if (op == CSA_OP_INDEX_TOPK || op == CSA_OP_PREFILL || op == CSA_OP_DECODE) {
    if ((rc = check_index_rows(cfg, op == CSA_OP_DECODE ? static_cast<long long>(B)
                                                        : static_cast<long long>(B) * nq,
                               n_max)))
      return rc;
  }
  switch (op) {
    case CSA_OP_COMPRESS: *bytes = ws_compress(cfg, B, nq); break;
    case CSA_OP_INDEX_TOPK:
      if (!is_csa(cfg)) return fail(CSA_ERR_INVALID_ARG, "index_topk needs CSA mode");
      *bytes = ws_index(cfg, B, nq, n_max);
      break;
    case CSA_OP_SPARSE_MQA: *bytes = ws_mqa(cfg, B, nq, max_list_sparse(cfg)); break;
    case CSA_OP_HCA_MQA: *bytes = ws_mqa(cfg, B, nq, max_list_dense(cfg, n_max)); break;
    case CSA_OP_DECODE: *bytes = ws_layer(cfg, B, 1, n_max, false, true); break;
    case CSA_OP_PREFILL: *bytes = ws_layer(cfg, B, nq, n_max, true, true); break;
    case CSA_OP_QUERY_PROJ:
      if ((rc = check_qproj_config(cfg))) return rc;
      *bytes = csa::query_proj_workspace(B * nq, cfg->q_rank, cfg->n_heads, cfg->head_dim,
                                         is_csa(cfg) ? cfg->idx_heads : 0, cfg->idx_dim);
      break;
    case CSA_OP_OUTPUT_PROJ:
      if ((rc = check_oproj_config(cfg))) return rc;
      *bytes = csa::output_proj_workspace(B * nq, cfg->out_groups, cfg->out_rank);
      break;
    default: return fail(CSA_ERR_INVALID_ARG, "unknown op %d", op);
  }
  return CSA_OK;
}

int csa_compress(const csa_config_t* cfg, int32_t B, int32_t T, const uint16_t* H,
                 const int32_t* pos0, const csa_weights_t* w, const csa_cache_t* cache,
                 void* workspace, size_t ws_bytes, void* stream) {
  int rc = check_config(cfg, true);
  if (rc) return rc;
  if ((rc = check_cache(cfg, cache, is_csa(cfg), true))) return rc;
  if ((rc = check_weights(cfg, w))) return rc;
  if (B < 1 || T < 1) return fail(CSA_ERR_INVALID_ARG, "B=%d, T=%d must be >= 1", B, T);
  if (!H || !pos0) return fail(CSA_ERR_INVALID_ARG, "H or pos0 is NULL");
  if ((rc = check_aligned({H, w ? w->w_cat : nullptr}))) return rc;
  const size_t need = ws_compress(cfg, B, T);
  if ((rc = check_workspace(workspace, ws_bytes, need))) return rc;
  return run_compress(cfg, B, T, H, pos0, w, cache, workspace,
                      reinterpret_cast<hipStream_t>(stream));
}

int csa_index_topk(const csa_config_t* cfg, int32_t B, int32_t nq, const uint8_t* qi,
                   const float* qi_scale, const float* wi, const csa_cache_t* cache,
                   const int32_t* pos, int32_t* idx_out, float* score_out, void* workspace,
                   size_t ws_bytes, void* stream) {
  int rc = check_config(cfg, false);
  if (rc) return rc;
  if (!is_csa(cfg)) return fail(CSA_ERR_INVALID_ARG, "csa_index_topk needs CSA mode");
  if ((rc = check_cache(cfg, cache, true, false))) return rc;
  if (B < 1 || nq < 1) return fail(CSA_ERR_INVALID_ARG, "B=%d, nq=%d must be >= 1", B, nq);
  if (!qi || !qi_scale || !wi || !pos || !idx_out)
    return fail(CSA_ERR_INVALID_ARG, "qi/qi_scale/wi/pos/idx_out is NULL");
  if ((rc = check_aligned({qi}))) return rc;
  if ((rc = check_index_rows(cfg, static_cast<long long>(B) * nq, cache->n_max))) return rc;
  const size_t need = ws_index(cfg, B, nq, cache->n_max);
  if ((rc = check_workspace(workspace, ws_bytes, need))) return rc;
  return run_index(cfg, B, nq, qi, qi_scale, wi, cache, pos, idx_out, score_out, workspace,
                   reinterpret_cast<hipStream_t>(stream));
}

int csa_sparse_mqa(const csa_config_t* cfg, int32_t B, int32_t nq, const uint16_t* q,
                   const csa_cache_t* cache, const int32_t* idx, const int32_t* pos,
                   const float* sink, uint16_t* out, float* lse_out, void* workspace,
                   size_t ws_bytes, void* stream) {
  int rc = check_config(cfg, false);
  if (rc) return rc;
  if ((rc = check_cache(cfg, cache, false, false))) return rc;
  if (B < 1 || nq < 1) return fail(CSA_ERR_INVALID_ARG, "B=%d, nq=%d must be >= 1", B, nq);
  if (!q || !idx || !pos || !sink || !out)
    return fail(CSA_ERR_INVALID_ARG, "q/idx/pos/sink/out is NULL");
  if ((rc = check_aligned({q, out}))) return rc;
  if (cfg->top_k < 1 || cfg->top_k > csa::kMaxTopK)
    return fail(CSA_ERR_INVALID_ARG, "top_k=%d not in 1..%d", cfg->top_k, csa::kMaxTopK);
  const size_t need = ws_mqa(cfg, B, nq, max_list_sparse(cfg));
  if ((rc = check_workspace(workspace, ws_bytes, need))) return rc;
  return run_attend(cfg, B, nq, q, cache, idx, pos, sink, out, lse_out, workspace,
                    reinterpret_cast<hipStream_t>(stream));
}

int hca_dense_mqa(const csa_config_t* cfg, int32_t B, int32_t nq, const uint16_t* q,
                  const csa_cache_t* cache, const int32_t* pos, const float* sink, uint16_t* out,
                  float* lse_out, void* workspace, size_t ws_bytes, void* stream) {
  int rc = check_config(cfg, false);
  if (rc) return rc;
  if ((rc = check_cache(cfg, cache, false, false))) return rc;
  if (B < 1 || nq < 1) return fail(CSA_ERR_INVALID_ARG, "B=%d, nq=%d must be >= 1", B, nq);
  if (!q || !pos || !sink || !out) return fail(CSA_ERR_INVALID_ARG, "q/pos/sink/out is NULL");
  if ((rc = check_aligned({q, out}))) return rc;
  const size_t need = ws_mqa(cfg, B, nq, max_list_dense(cfg, cache->n_max));
  if ((rc = check_workspace(workspace, ws_bytes, need))) return rc;
  return run_attend(cfg, B, nq, q, cache, nullptr, pos, sink, out, lse_out, workspace,
                    reinterpret_cast<hipStream_t>(stream));
}

int csa_decode(const csa_config_t* cfg, int32_t B, const uint16_t* h_new, const csa_weights_t* w,
               const csa_cache_t* cache, const int32_t* pos, const uint16_t* q, const uint8_t* qi,
               const float* qi_scale, const float* wi, const float* sink, uint16_t* out,
               int32_t* idx_out, void* workspace, size_t ws_bytes, void* stream) {
  size_t need = 0;
  int rc = decode_check(cfg, B, h_new, w, cache, pos, q, qi, qi_scale, wi, sink, out, &need);
  if (rc) return rc;
  if ((rc = check_workspace(workspace, ws_bytes, need))) return rc;
  return decode_run(cfg, B, h_new, w, cache, pos, q, qi, qi_scale, wi, sink, out, idx_out,
                    workspace, reinterpret_cast<hipStream_t>(stream));
}

int csa_decode_noalloc(const csa_config_t* cfg, int32_t B, const uint16_t* h_new,
                       const csa_weights_t* w, const csa_cache_t* cache, const int32_t* pos,
                       const uint16_t* q, const uint8_t* qi, const float* qi_scale,
                       const float* wi, const float* sink, uint16_t* out, int32_t* idx_out,
                       void* stream) {
  size_t need = 0;
  int rc = decode_check(cfg, B, h_new, w, cache, pos, q, qi, qi_scale, wi, sink, out, &need);
  if (rc) return rc;
  if (need > kScratchBytes)
    return fail(CSA_ERR_UNSUPPORTED, "this decode needs %zu bytes of scratch, more than the %zu "
                "bytes of csa_decode_noalloc's static scratch (use csa_decode with a workspace)",
                need, kScratchBytes);
  void* ws = nullptr;
  if ((rc = scratch_of_current_device(&ws))) return rc;
  return decode_run(cfg, B, h_new, w, cache, pos, q, qi, qi_scale, wi, sink, out, idx_out, ws,
                    reinterpret_cast<hipStream_t>(stream));
}

int csa_prefill(const csa_config_t* cfg, int32_t B, int32_t T, const uint16_t* H,
                const int32_t* pos0, const csa_weights_t* w, const csa_cache_t* cache,
                const uint16_t* q, const uint8_t* qi, const float* qi_scale, const float* wi,
                const float* sink, uint16_t* out, int32_t* idx_out, void* workspace,
                size_t ws_bytes, void* stream) {
  int rc = check_config(cfg, true);
  if (rc) return rc;
  if ((rc = check_cache(cfg, cache, is_csa(cfg), true))) return rc;
  if ((rc = check_weights(cfg, w))) return rc;
  if (B < 1 || T < 1) return fail(CSA_ERR_INVALID_ARG, "B=%d, T=%d must be >= 1", B, T);
  if (!H || !q || !sink || !out) return fail(CSA_ERR_INVALID_ARG, "H/q/sink/out is NULL");
  if ((rc = check_aligned({H, q, qi, out, w ? w->w_cat : nullptr}))) return rc;
  if (is_csa(cfg) && (!qi || !qi_scale || !wi))
    return fail(CSA_ERR_INVALID_ARG, "CSA prefill needs qi, qi_scale and wi");
  if (!pos0 && cache->win_slots < T)
    return fail(CSA_ERR_INVALID_ARG, "prefill needs win_slots=%d >= T=%d", cache->win_slots, T);
  if (pos0 && cache->win_slots < static_cast<long long>(T) + cfg->n_win - 1)
    return fail(CSA_ERR_INVALID_ARG, "chunked prefill needs win_slots=%d >= T + n_win - 1 = %d",
                cache->win_slots, T + cfg->n_win - 1);
  if (!pos0 && T / cfg->m > cache->n_max)
    return fail(CSA_ERR_INVALID_ARG, "T/m=%d entries exceed n_max=%d", T / cfg->m, cache->n_max);
  if ((rc = check_index_rows(cfg, static_cast<long long>(B) * T, cache->n_max))) return rc;
  const size_t need = ws_layer(cfg, B, T, cache->n_max, true, true);
  if ((rc = check_workspace(workspace, ws_bytes, need))) return rc;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  unsigned char* p = static_cast<unsigned char*>(workspace);
  int32_t* idx = nullptr;
  if (is_csa(cfg)) {
    idx = idx_out ? idx_out : reinterpret_cast<int32_t*>(p);
    p += align256(static_cast<size_t>(B) * T * cfg->top_k * 4);
  }
  // chunked prefill: the queries' positions pos0[b] + i, written once for the scorer, the
  // selection and the attention
  int32_t* qpos = nullptr;
  if (pos0) {
    qpos = reinterpret_cast<int32_t*>(p);
    const hipError_t e = launch_chunk_positions(pos0, B, T, qpos, s);
    if (e != hipSuccess) return hip_fail(e, "chunk positions launch");
  }
  p += align256(static_cast<size_t>(B) * T * 4);
  if ((rc = run_compress(cfg, B, T, H, pos0, w, cache, p, s, pos0 != nullptr))) return rc;
  if (is_csa(cfg)) {
    if ((rc = run_index(cfg, B, T, qi, qi_scale, wi, cache, qpos, idx, nullptr, p, s)))
      return rc;
    return run_attend(cfg, B, T, q, cache, idx, qpos, sink, out, nullptr, p, s);
  }
  return run_attend(cfg, B, T, q, cache, nullptr, qpos, sink, out, nullptr, p, s);
}

int csa_query_proj(const csa_config_t* cfg, int32_t B, int32_t T, const uint16_t* H,
                   const csa_qproj_weights_t* w, uint16_t* q_out, uint8_t* qi_out,
                   float* qi_scale_out, float* wi_out, void* workspace, size_t ws_bytes,
                   void* stream) {
  int rc = check_config(cfg, false);
  if (rc) return rc;
  if ((rc = check_qproj_config(cfg))) return rc;
  if (B < 1 || T < 1) return fail(CSA_ERR_INVALID_ARG, "B=%d, T=%d must be >= 1", B, T);
  if (!H || !w || !w->w_dq || !w->w_uq || !w->gamma_q || !q_out)
    return fail(CSA_ERR_INVALID_ARG, "H, weights (w_dq, w_uq, gamma_q) or q_out is NULL");
  const bool csa_mode = is_csa(cfg);
  if (csa_mode && (!w->w_w || !w->w_iuq || !qi_out || !qi_scale_out || !wi_out))
    return fail(CSA_ERR_INVALID_ARG, "CSA needs w_w, w_iuq, qi_out, qi_scale_out and wi_out");
  if ((rc = check_aligned({H, w->w_dq, w->w_w, w->w_uq, w->w_iuq, w->gamma_q, q_out, qi_out,
                           qi_scale_out, wi_out})))
    return rc;
  const int BT = B * T;
  const size_t need = csa::query_proj_workspace(BT, cfg->q_rank, cfg->n_heads, cfg->head_dim,
                                                csa_mode ? cfg->idx_heads : 0, cfg->idx_dim);
  if ((rc = check_workspace(workspace, ws_bytes, need))) return rc;
  csa::QueryProjArgs a;
  a.BT = BT;
  a.D = cfg->hidden;
  a.r_q = cfg->q_rank;
  a.n_h = cfg->n_heads;
  a.c = cfg->head_dim;
  a.H_I = csa_mode ? cfg->idx_heads : 0;
  a.d_I = csa_mode ? cfg->idx_dim : 0;
  a.eps = cfg->rms_eps;
  a.H = H;
  a.w_dq = w->w_dq;
  a.w_w = csa_mode ? w->w_w : nullptr;
  a.w_uq = w->w_uq;
  a.w_iuq = csa_mode ? w->w_iuq : nullptr;
  a.gamma_q = w->gamma_q;
  a.q = q_out;
  a.qi = csa_mode ? qi_out : nullptr;
  a.qi_scale = csa_mode ? qi_scale_out : nullptr;
  a.qi_mx = csa_mode && cfg->idx_query_format == CSA_IDX_MXFP4;
  a.wi = csa_mode ? wi_out : nullptr;
  a.ws = workspace;
  const hipError_t e = csa::launch_query_proj(a, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? CSA_OK : hip_fail(e, "csa_query_proj");
}

int csa_output_proj(const csa_config_t* cfg, int32_t B, int32_t T, const uint16_t* O,
                    const csa_oproj_weights_t* w, uint16_t* y_out, void* workspace,
                    size_t ws_bytes, void* stream) {
  int rc = check_config(cfg, false);
  if (rc) return rc;
  if ((rc = check_oproj_config(cfg))) return rc;
  if (B < 1 || T < 1) return fail(CSA_ERR_INVALID_ARG, "B=%d, T=%d must be >= 1", B, T);
  if (!O || !w || !w->w_down || !w->w_proj || !y_out)
    return fail(CSA_ERR_INVALID_ARG, "O, w_down, w_proj or y_out is NULL");
  if ((rc = check_aligned({O, w->w_down, w->w_proj, y_out}))) return rc;
  const int BT = B * T;
  const size_t need = csa::output_proj_workspace(BT, cfg->out_groups, cfg->out_rank);
  if ((rc = check_workspace(workspace, ws_bytes, need))) return rc;
  csa::OutputProjArgs a;
  a.BT = BT;
  a.D = cfg->hidden;
  a.n_h = cfg->n_heads;
  a.c = cfg->head_dim;
  a.g = cfg->out_groups;
  a.r_o = cfg->out_rank;
  a.O = O;
  a.w_down = w->w_down;
  a.w_proj = w->w_proj;
  a.y = y_out;
  a.ws = workspace;
  const hipError_t e = csa::launch_output_proj(a, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? CSA_OK : hip_fail(e, "csa_output_proj");
}

}  // extern "C"
