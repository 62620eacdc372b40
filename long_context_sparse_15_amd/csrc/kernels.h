// Internal launcher interface between the C ABI layer (api.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace csa {

constexpr int kHistBins = 4096;     // first-level top-k histogram: top 12 bits of the key
constexpr int kCandCap = 4096;      // candidates kept for the exact refinement of one row
constexpr int kMaxTopK = 4096;
constexpr int kRowTopkMaxN = 16384; // row select with 256 threads holds this many keys in LDS
constexpr int kRowTopkBigN = 32768; // row select with 1024 threads holds this many keys

// ---------------------------------------------------------------- cache layout
// Where the per-sequence entry arrays (compressed entries, indexer keys, key scales) keep
// logical entry e of sequence b.  table == nullptr: contiguous, row b * n_max + e.  Otherwise
// the arrays are pools of n_blocks physical blocks of 2^shift entries each, and e lives in row
// e & (2^shift - 1) of block table[b * stride + (e >> shift)] (clamped into the pool, so a bad
// table entry gives wrong values, never an access outside the pool).  Callers keep e < n_max.
struct PageMap {
  const int32_t* table = nullptr;
  int stride = 0;    // table entries per sequence
  int shift = 0;     // log2(entries per block)
  int n_blocks = 0;  // physical blocks in the pools
};
__device__ __forceinline__ size_t entry_row(const PageMap& pm, int n_max, int b, int e) {
  if (!pm.table) return static_cast<size_t>(b) * n_max + e;
  int blk = pm.table[static_cast<size_t>(b) * pm.stride + (e >> pm.shift)];
  blk = blk < 0 ? 0 : (blk >= pm.n_blocks ? pm.n_blocks - 1 : blk);
  return (static_cast<size_t>(blk) << pm.shift) + (e & ((1 << pm.shift) - 1));
}
// First row of the physical block of logical block j of sequence b, for wave-uniform b and j:
// one scalar-cache load (counted apart from the vector loads, so waiting for it never waits
// for key loads in flight).
__device__ __forceinline__ size_t block_base_uniform(const PageMap& pm, int b, int j) {
  const int i = __builtin_amdgcn_readfirstlane(b * pm.stride + j);
  typedef const __attribute__((address_space(4))) int32_t* ctab;
  int blk = reinterpret_cast<ctab>(reinterpret_cast<uintptr_t>(pm.table))[i];
  blk = blk < 0 ? 0 : (blk >= pm.n_blocks ? pm.n_blocks - 1 : blk);
  return static_cast<size_t>(blk) << pm.shift;
}

// ---------------------------------------------------------------- indexer + top-k
struct IndexArgs {
  const uint8_t* qi;      // [rows, H_I, d_I]
  const float* qi_scale;  // [rows, H_I]
  const float* wi;        // [rows, H_I]
  const uint8_t* keys;    // [B, n_max, d_I] e4m3, or [B, n_max, d_I/2] packed MXFP4
  const float* kscale;    // [B, n_max] fp32, or 4 E8M0 block-scale bytes per entry (MXFP4)
  const int32_t* n_entries;  // [B]
  const int32_t* pos;     // [rows] or nullptr (t = query index within its sequence)
  int B, nq, n_max, H_I, d_I, m, k;
  int key_fmt;            // 0 e4m3 + fp32 scale, 1 MXFP4
  int q_fmt;              // 0 e4m3 + fp32 scale per head, 1 MXFP4 (qi [rows, H_I, d_I/2], qi_scale
                          // 4 E8M0 bytes per head); 1 needs key_fmt 1
  bool score_bf16;        // scores stored as bf16 (nearest even) instead of fp32
  PageMap pages;          // layout of keys and kscale (paged: blocks of >= 16 entries)
  void* scores;           // workspace [rows, sstride] fp32 or bf16
  int sstride;
  uint32_t* counters;     // workspace [rows, chunks, 2]: candidates and threshold of each chunk
  uint64_t* cand;         // workspace [rows, chunks, candidates per chunk]: (key, index)
  int32_t* idx_out;       // [rows, k]
  float* score_out;       // [rows, k] or nullptr
};
// Rows longer than kRowTopkBigN (and not too many) use the multi-workgroup select: chunks of a
// row take candidates of their own (regions of kCandPerChunk pairs), a finalize workgroup per
// row selects among them.  The chunks are kCollectChunk entries when a selection kernel collects
// them, or the decode scorer's chunks when it collects its own (index_fused_collect).
constexpr int kMultiMaxRows = 4096;
constexpr int kCollectChunk = 4096;
constexpr int kCandPerChunk = 1024;
bool index_use_multi(int rows, int n_max);
// decode-scorer rows whose chunks' candidates the scorer collects (index.hip)
bool index_fused_collect(int nq, int d_I, int H_I, int rows, int n_max);
int index_score_chunk();  // entries a decode-scorer workgroup scores (and collects)
size_t index_topk_workspace(int rows, int nq, int n_max, int d_I, int H_I, bool score_bf16);
void index_topk_layout(IndexArgs& a, void* ws, int rows);  // needs a.n_max, nq, d_I, H_I set
hipError_t launch_index_scores(const IndexArgs& a, hipStream_t s);  // a.scores only
// the decode scorer with candidate collection (index_fused_collect rows): a.scores, a.counters
// and a.cand
hipError_t launch_index_scores_collect(const IndexArgs& a, hipStream_t s);
hipError_t launch_index_topk(const IndexArgs& a, hipStream_t s);    // scores, then selection

// ---------------------------------------------------------------- attention
struct MqaArgs {
  const uint16_t* q;        // [rows, n_heads, c]
  const uint16_t* entries;  // [B, n_max, c]
  const uint16_t* window;   // [B, win_slots, c]
  const int32_t* idx;       // [rows, k] (sparse) or nullptr (dense: all visible entries)
  const int32_t* n_entries; // [B]
  const int32_t* pos;       // [rows] or nullptr
  const float* sink;        // [n_heads]
  const float* inv_freq;    // [r/2]
  int B, nq, n_heads, c, r, k, m, n_win, win_slots, n_max;
  PageMap pages;            // layout of entries
  bool entry_mixed;         // entries as [c-r E4M3 codes | r bf16] rows (c + r bytes)
  float scale;
  uint16_t* out;            // [rows, n_heads, c]
  float* lse_out;           // [rows, n_heads] or nullptr
  float* part;              // workspace partials
};
struct MqaPlan {
  int kind;           // kMqaSliced (mqa.hip) or kMqaHeadBlock (mqa_hb.hip)
  int head_pairs;     // 32-head groups per workgroup (one wave each per dim slice)
  int slices;         // dim slices (waves) per head pair
  int heads_per_wg;   // 32 * head_pairs
  int head_groups;
  int split_rows;     // rows of the key list per workgroup (multiple of 32)
  int n_splits;
};
constexpr int kMqaSliced = 0;     // waves own 32 heads x a dim slice, logits summed through LDS
constexpr int kMqaHeadBlock = 1;  // waves own 32 heads x all 512 dims, 128 heads a workgroup
constexpr int kMqaHeadBlockQ = 2; // the same per wave, two queries of 64 heads a workgroup
// nq = queries per sequence in the call; the batch size is deliberately not an input (the plan
// fixes the order of every query's softmax sums, see mqa.hip)
MqaPlan plan_mqa(int nq, int n_heads, int c, int max_list, bool mixed);
size_t mqa_workspace(const MqaPlan& p, int rows, int n_heads, int c);
hipError_t launch_mqa(const MqaArgs& a, const MqaPlan& p, hipStream_t s);

// ---------------------------------------------------------------- compressor
struct CompressArgs {
  int mode;                 // 0 CSA, 1 HCA
  int B, T, D, c, d_I, m, r, n_cols, tail_rows, tail_cols, win_slots, n_max;
  int key_fmt;              // indexer keys: 0 e4m3 + fp32 scale, 1 MXFP4
  PageMap pages;            // layout of entries, ikeys and iscale
  bool keep_existing;       // blocks below n_entries[b] (on entry) are not written
  bool entry_mixed;         // entries as [c-r E4M3 codes | r bf16] rows (c + r bytes)
  const uint16_t* H;        // [B, T, D]
  const int32_t* pos0;      // [B] or nullptr (all 0)
  const uint16_t* W;        // [n_cols, D]
  const float *bias_a, *bias_b, *bias_ia, *bias_ib, *gamma, *gamma_win;
  const float* inv_freq;
  float eps;
  uint16_t* entries;
  uint8_t* ikeys;
  float* iscale;
  uint16_t* window;
  float* tail;
  int32_t* n_entries;
  float* proj;              // workspace [B*T, n_cols]
};
size_t compress_workspace(int B, int T, int n_cols);
hipError_t launch_compress(const CompressArgs& a, hipStream_t s);

// ---------------------------------------------------------------- dense projections
// C[M, N] = A[M, K] W[N, K]^T, bf16 operands, fp32 accumulation, K % 64 == 0.
struct GemmArgs {
  const uint16_t* A;
  int lda;
  const uint16_t* W;
  int ldw;
  void* C;          // fp32, or bf16 when bf16_out
  int ldc;
  int M, N, K;
  bool bf16_out;
  const char* name;  // label for launch timing
};
hipError_t launch_gemm_tn(const GemmArgs& g, hipStream_t s);

struct QueryProjArgs {
  int BT, D, r_q, n_h, c, H_I, d_I;
  float eps;
  const uint16_t* H;      // [BT, D]
  const uint16_t* w_dq;   // [r_q, D]
  const uint16_t* w_w;    // [H_I, D] or nullptr
  const uint16_t* w_uq;   // [n_h * c, r_q]
  const uint16_t* w_iuq;  // [H_I * d_I, r_q] or nullptr
  const float* gamma_q;   // [c]
  uint16_t* q;            // [BT, n_h, c]
  uint8_t* qi;            // [BT, H_I, d_I] (MXFP4: [BT, H_I, d_I/2]) or nullptr
  float* qi_scale;        // [BT, H_I] fp32 (MXFP4: 4 E8M0 bytes per head) or nullptr
  bool qi_mx;             // indexer query as MXFP4
  float* wi;              // [BT, H_I] or nullptr
  void* ws;
};
size_t query_proj_workspace(int BT, int r_q, int n_h, int c, int H_I, int d_I);
hipError_t launch_query_proj(const QueryProjArgs& a, hipStream_t s);

struct OutputProjArgs {
  int BT, D, n_h, c, g, r_o;
  const uint16_t* O;       // [BT, n_h, c]
  const uint16_t* w_down;  // [g, r_o, (n_h / g) * c]
  const uint16_t* w_proj;  // [D, g * r_o]
  uint16_t* y;             // [BT, D]
  void* ws;
};
size_t output_proj_workspace(int BT, int g, int r_o);
hipError_t launch_output_proj(const OutputProjArgs& a, hipStream_t s);

// ---------------------------------------------------------------- misc
// Raises kernel fn's dynamic-LDS limit to at least `bytes` (never lowers it).  Thread-safe: the
// limits already set are kept per function under one lock, so concurrent first launches from
// several threads each see the attribute in place before they launch.
hipError_t ensure_max_lds(const void* fn, size_t bytes);

// ---------------------------------------------------------------- launch timing (opt-in)
struct ProfTotal {
  char name[40];
  int32_t launches;
  double total_ms;
};
class ProfScope {  // brackets one kernel launch with hipEvents when timing is on
 public:
  ProfScope(const char* name, hipStream_t s);
  ~ProfScope();
  ProfScope(const ProfScope&) = delete;
  ProfScope& operator=(const ProfScope&) = delete;

 private:
  const char* name_;
  hipStream_t stream_;
  void* a_;
};
int profile_start();
int profile_stop(ProfTotal* out, int max, int* n);

}  // namespace csa
