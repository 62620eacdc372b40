/*
 * csa.h - C ABI of the MI355X (gfx950) Compressed Sparse Attention / Heavily Compressed
 * Attention library (libcsa.so).
 *
 * The method is DeepSeek-V4's long-context attention as described in
 * "DeepSeek V4 模型技术大全" (wineandchord.com book), chapter "Attention", sections
 * "CSA 的完整路径", "HCA 的完整路径" and "注意力实现细节", and in
 * "DeepSeek-V4 技术报告深度解读" (chang-wenbin.github.io), sections 2.1-2.3.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every call returns an int status: CSA_OK (0) or a negative CSA_ERR_* code.  On error
 *    nothing has been enqueued and csa_last_error() (per calling thread) describes why.
 *  - No call allocates device memory and no call synchronizes: work is enqueued on the HIP
 *    stream passed as `stream` (a hipStream_t, NULL = the default stream) and the call returns.
 *  - Every tensor argument is a caller-owned DEVICE pointer to contiguous row-major memory,
 *    unless marked "host".  Tensors the kernels move as 16-byte vectors must be 16-byte aligned
 *    (CSA_ERR_INVALID_ARG otherwise): hidden states, weights, queries, indexer queries,
 *    outputs, and the cache's entries, keys, window and tail.  The library keeps no pointer
 *    after a call returns.
 *  - Scratch memory comes from the caller's `workspace` (device, 256-byte aligned) of
 *    `ws_bytes` bytes; csa_workspace_size() returns the bytes an operation needs.  Workspace
 *    contents on entry are irrelevant and are clobbered.
 *  - Element types: bf16 = uint16_t bit patterns, e4m3 = uint8_t OCP FP8 E4M3 ("fn": bias 7,
 *    no infinities, max 448), fp32 = float, indices and positions = int32_t.
 *  - Token positions are 0-based.  Token u's window row lives in row (u % win_slots) of the
 *    window buffer; compressed entry i (covering tokens m*i .. m*i+m-1) lives in row i.
 *  - Calls on the same stream are ordered; calls that share a cache or workspace must not
 *    overlap on different streams.
 */
#ifndef CSA_H_
#define CSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSA_OK 0
#define CSA_ERR_INVALID_ARG (-1) /* NULL pointer, bad shape or unsupported parameter */
#define CSA_ERR_UNSUPPORTED (-2) /* valid request outside what the kernels implement */
#define CSA_ERR_WORKSPACE (-3)   /* ws_bytes smaller than csa_workspace_size() */
#define CSA_ERR_HIP (-4)         /* a HIP runtime call failed (message in csa_last_error) */

#define CSA_MODE_CSA 0 /* overlapping m-token compressor + lightning indexer + top-k */
#define CSA_MODE_HCA 1 /* non-overlapping m'-token compressor, dense over closed entries */

/* Storage of the indexer keys K^IComp (csa_config_t.idx_key_format).  The pages give the
 * indexer's QK path in FP8 and, for V4's indexer, FP4 ("DeepSeek V4 模型技术大全", chapter
 * "Attention", section "注意力实现细节"); the bit layouts are the public OCP formats. */
#define CSA_IDX_E4M3 0  /* e4m3 codes [idx_dim] + one fp32 scale per entry (max|k|/448) */
#define CSA_IDX_MXFP4 1 /* OCP MXFP4: E2M1 codes packed two per byte [idx_dim/2] (dim 2i in the
                           low nibble of byte i) + one E8M0 scale byte per 32 dims (shared
                           exponent floor(log2 max|k|) - 2) */

/* Index-score storage before the top-k (csa_config_t.score_format).  The pages store the
 * indexer's scores in BF16 for a faster selector (Deep dive "论文专题讲解：DeepSeek-V4", section
 * "FP4 QAT", table row "index scores": FP32 -> BF16). */
#define CSA_SCORE_FP32 0 /* fp32 scores; selection exact on them */
#define CSA_SCORE_BF16 1 /* each score rounded to bf16 (nearest even), top-k on the bf16 values,
                            the lower index winning the ties this creates */

/* Storage of the compressed entries (csa_config_t.entry_format). */
#define CSA_ENT_BF16 0  /* head_dim bf16 values per entry */
#define CSA_ENT_MIXED 1 /* head_dim - rope_dim E4M3 codes of the unrotated dims (no scale), then
                           rope_dim bf16 rotated dims: head_dim + rope_dim bytes per entry.  The
                           pages keep the RoPE dims in BF16 and the rest in FP8 ("DeepSeek V4
                           模型技术大全", chapter "Attention", section "注意力实现细节").  Requires
                           head_dim 512 and rope_dim a multiple of 16; window rows stay bf16. */

/* Operation ids for csa_workspace_size(). */
#define CSA_OP_COMPRESS 0
#define CSA_OP_INDEX_TOPK 1
#define CSA_OP_SPARSE_MQA 2
#define CSA_OP_HCA_MQA 3
#define CSA_OP_DECODE 4
#define CSA_OP_PREFILL 5
#define CSA_OP_QUERY_PROJ 6  /* csa_query_proj over B*nq tokens (n_max ignored) */
#define CSA_OP_OUTPUT_PROJ 7 /* csa_output_proj over B*nq tokens (n_max ignored) */

/* Layer configuration, passed by pointer (read during the call only).
 * Supported set (CSA_ERR_INVALID_ARG otherwise):
 *   head_dim in {128, 256, 512};
 *   rope_dim even, 2 <= rope_dim <= min(head_dim, 128);
 *   1 <= n_heads <= 128;  n_win in 1..1024;
 *   CSA: idx_dim in {32, 64, 128}, 1 <= idx_heads <= 64, 1 <= top_k <= 4096, m >= 1,
 *        idx_key_format CSA_IDX_E4M3 or CSA_IDX_MXFP4; idx_query_format CSA_IDX_E4M3 or
 *        CSA_IDX_MXFP4, the latter only with MXFP4 keys (CSA_ERR_UNSUPPORTED otherwise);
 *        score_format CSA_SCORE_FP32 or CSA_SCORE_BF16;
 *   HCA: m >= 1;  hidden (compressor only) a positive multiple of 32;
 *   entry_format CSA_ENT_BF16 or CSA_ENT_MIXED (the latter: head_dim 512 and rope_dim a multiple
 *   of 16, CSA_ERR_UNSUPPORTED otherwise);
 *   projections only: hidden and q_rank multiples of 64; out_groups dividing n_heads with
 *   (n_heads/out_groups)*head_dim and out_groups*out_rank multiples of 64. */
typedef struct csa_config {
  int32_t mode;       /* CSA_MODE_CSA or CSA_MODE_HCA */
  int32_t m;          /* compression ratio: 4 in CSA layers, 128 (m') in HCA layers */
  int32_t top_k;      /* k: compressed entries selected per query (CSA) */
  int32_t n_win;      /* sliding-window length n_win (128) */
  int32_t n_heads;    /* query heads n_h sharing the single K=V head */
  int32_t head_dim;   /* entry / head width c = d_h */
  int32_t rope_dim;   /* r: trailing dims that carry RoPE */
  int32_t idx_heads;  /* indexer heads n_h^I (CSA) */
  int32_t idx_dim;    /* indexer dim d_I (CSA) */
  int32_t hidden;     /* hidden size D of the compressor input */
  float softmax_scale; /* logit scale (1/sqrt(d_h)) */
  float rms_eps;       /* RMSNorm epsilon (1e-6) */
  const float* rope_inv_freq; /* device fp32 [rope_dim/2]: angle of pair i at position p is
                                 p * rope_inv_freq[i] (base 160000 for compressed layers; any
                                 table, e.g. YaRN-scaled, may be passed) */
  int32_t idx_key_format;     /* CSA_IDX_E4M3 (0) or CSA_IDX_MXFP4 (1); CSA only */
  /* Projections on either side of attention (csa_query_proj / csa_output_proj only):
   * query LoRA rank r_q (1024 Flash, 1536 Pro), output groups g (8 / 16), output rank r_o
   * (1024).  Book, chapter "Attention": configuration table and section "注意力实现细节". */
  int32_t q_rank;
  int32_t out_groups;
  int32_t out_rank;
  int32_t entry_format; /* CSA_ENT_BF16 (0) or CSA_ENT_MIXED (1) */
  /* Format of the indexer query q^I (CSA).  CSA_IDX_E4M3: qi e4m3 [.., idx_heads, idx_dim] with
   * qi_scale fp32 [.., idx_heads] (max|q|/448).  CSA_IDX_MXFP4 (the pages' FP4 QK path: query
   * and keys both FP4, Deep dive "论文专题讲解：DeepSeek-V4", section "FP4 QAT", table row "CSA
   * indexer QK path"): qi uint8 [.., idx_heads, idx_dim/2] packed E2M1 codes as the keys', and
   * qi_scale the same 4 bytes per (token, head) holding its idx_dim/32 E8M0 block scales, block
   * b in byte b (unused bytes are ignored). */
  int32_t idx_query_format;
  int32_t score_format;  /* CSA_SCORE_FP32 (0) or CSA_SCORE_BF16 (1); CSA only */
} csa_config_t;

/* Caller-owned per-sequence attention state for B sequences (all device pointers).
 *  entries   bf16 [B, n_max, head_dim]  compressed entries, RMS-normalised and rotated; with
 *            CSA_ENT_MIXED uint8 [B, n_max, head_dim + rope_dim] (see CSA_ENT_MIXED)
 *  idx_keys  e4m3 [B, n_max, idx_dim]   indexer keys K^IComp (CSA; NULL for HCA); with
 *            CSA_IDX_MXFP4: uint8 [B, n_max, idx_dim/2] packed E2M1 codes
 *  idx_scale fp32 [B, n_max]            per-entry scale of idx_keys (CSA; NULL for HCA); with
 *            CSA_IDX_MXFP4 the same 4 bytes per entry hold the idx_dim/32 E8M0 block scales,
 *            block b in byte b (unused bytes are ignored)
 *  window    bf16 [B, win_slots, head_dim]  uncompressed window KV, token u in row u%win_slots
 *  tail      fp32 [B, tail_rows, tail_cols] compressor projections of the last tail_rows tokens
 *            (row u % tail_rows); only used by the compressor (csa_tail_shape gives the shape)
 *  n_entries int32 [B]                   closed entries per sequence (read; the compressor
 *                                        updates it)
 *
 * Block layout (the hybrid cache of Book "DeepSeek V4 模型技术大全", chapter "Attention":
 * compressed entries in fixed-size blocks of lcm(m, 128) tokens, i.e. 128/m entries for m = 4
 * and one entry for m' = 128; the window ring and compressor tail stay per-sequence state).
 * block_entries = 0 selects the contiguous layout above.  block_entries > 0 (a power of two;
 * CSA: >= 16) makes entries, idx_keys and idx_scale pools of n_blocks physical blocks of
 * block_entries entries ([n_blocks, block_entries, ...], same per-entry widths), and puts
 * logical entry i of sequence b in row i % block_entries of physical block
 * block_table[b * blocks_per_seq + i / block_entries].  Requires n_max = blocks_per_seq *
 * block_entries and n_blocks * block_entries < 2^31.  Table values outside 0..n_blocks-1 are
 * clamped into the pool (wrong results, never an access outside it).  Sequences may map the
 * same physical blocks (a shared prefix): readers never write entries, and csa_compress writes
 * only blocks i >= n_entries[b]. */
typedef struct csa_cache {
  int32_t n_max;
  int32_t win_slots;
  uint16_t* entries;
  uint8_t* idx_keys;
  float* idx_scale;
  uint16_t* window;
  float* tail;
  int32_t* n_entries;
  int32_t block_entries;       /* 0: contiguous; else entries per block */
  int32_t blocks_per_seq;      /* block_table row length */
  int32_t n_blocks;            /* physical blocks in each pool */
  const int32_t* block_table;  /* device int32 [B, blocks_per_seq] */
} csa_cache_t;

/* Compressor parameters (device pointers).
 *  w_cat  bf16 [n_cols, hidden], one row per projection output column (csa_weight_cols):
 *         CSA: [W^a_KV c | W^b_KV c | W^a_Z c | W^b_Z c | W^a_I dI | W^b_I dI | W^a_IZ dI |
 *               W^b_IZ dI | W_win c];   HCA: [W_KV c | W_Z c | W_win c]
 *  bias_a fp32 [m, c]   B^a (CSA) or B (HCA), the compressor's position bias
 *  bias_b fp32 [m, c]   B^b (CSA; NULL for HCA)
 *  bias_ia, bias_ib fp32 [m, dI]  position biases of the indexer-key compressor (CSA)
 *  gamma, gamma_win fp32 [c]      RMSNorm gains of compressed entries and of window KV */
typedef struct csa_weights {
  const uint16_t* w_cat;
  const float* bias_a;
  const float* bias_b;
  const float* bias_ia;
  const float* bias_ib;
  const float* gamma;
  const float* gamma_win;
} csa_weights_t;

/* Library version: major*10000 + minor*100 + patch. */
int csa_version(void);

/* Message describing the last error returned on the calling thread ("" if none). */
const char* csa_last_error(void);

/* Opt-in launch timing, for measurement tools.  Between csa_profile_start() and
 * csa_profile_stop() every kernel the library launches is bracketed by two hipEvents recorded on
 * its launch stream.  csa_profile_stop() waits for those events and fills out[0..*n_out) with
 * one record per kernel name: launches and summed event time in milliseconds.  Not for use while
 * another thread is launching through the library. */
typedef struct csa_kernel_time {
  char name[40];
  int32_t launches;
  double total_ms;
} csa_kernel_time_t;
int csa_profile_start(void);
int csa_profile_stop(csa_kernel_time_t* out /* host */, int32_t max_out,
                     int32_t* n_out /* host */);

/* Host-side shape helpers (no device work). */
int csa_weight_cols(const csa_config_t* cfg, int32_t* n_cols /* host out */);
int csa_tail_shape(const csa_config_t* cfg, int32_t* rows /* host out */,
                   int32_t* cols /* host out */);

/* Bytes of workspace operation `op` (CSA_OP_*) needs for B sequences, nq queries (or tokens)
 * per sequence and caches of n_max entries.  *bytes is a host pointer. */
int csa_workspace_size(const csa_config_t* cfg, int32_t op, int32_t B, int32_t nq,
                       int32_t n_max, size_t* bytes);

/* csa_compress - token-level compressor (CSA: overlapping 2m-token windows with streams
 * C^a/C^b weighted by a per-channel softmax of Z^a+B^a / Z^b+B^b, plus the indexer keys
 * K^IComp from the same operation; HCA: m'-token windows of C weighted by softmax(Z+B)).
 * Book "DeepSeek V4 模型技术大全", chapter "Attention", section "CSA 的完整路径" (first three
 * equations and the K^IComp sentence) and section "HCA 的完整路径" (first two equations);
 * entries are RMS-normalised and carry partial RoPE at position m*i (section "注意力实现细节").
 *
 *  H     bf16 [B, T, hidden]: T new tokens of each sequence, sequence b's at positions
 *        pos0[b] .. pos0[b]+T-1.
 *  pos0  int32 [B] device: first new position per sequence, with floor(pos0[b]/m) <=
 *        n_entries[b] <= floor((pos0[b]+T)/m); the tail ring must hold the projections of the
 *        tokens before pos0[b] that the first new block reads (none for a fresh sequence).
 *        n_entries[b] > floor(pos0[b]/m) rebuilds state only: with entries 0..n_entries[b]-1
 *        already in the cache (e.g. blocks shared with another sequence), re-running the last
 *        max(n_win, 2m) tokens before position m*n_entries[b] refills the window ring and the
 *        tail ring and writes no entry (prefix reuse with tail recompute).
 *  Effects per sequence: every block i >= n_entries[b] that closes inside the call
 *  (m(i+1)-1 within the new tokens) is written to entries[b,i] (bf16, RMSNorm*gamma, RoPE at
 *  m*i) and, for CSA, to
 *  idx_keys/idx_scale[b,i] (E4M3 with per-entry scale max|x|/448, no norm, no RoPE);
 *  window rows of the new tokens (RMSNorm(h W_win)*gamma_win, RoPE at u); the tail ring;
 *  n_entries[b] = floor((pos0[b]+T)/m).  Requires floor((pos0[b]+T)/m) <= n_max.
 */
int csa_compress(const csa_config_t* cfg, int32_t B, int32_t T, const uint16_t* H,
                 const int32_t* pos0, const csa_weights_t* w, const csa_cache_t* cache,
                 void* workspace, size_t ws_bytes, void* stream);

/* csa_index_topk - lightning-indexer scores I_{t,s} = sum_h w_{t,h} ReLU(q^I_{t,h} . K^I_s)
 * over the closed entries s < min(n_entries[b], floor((t+1)/m)), then TopK_k.
 * Book "DeepSeek V4 模型技术大全", chapter "Attention", section "CSA 的完整路径" (indexer
 * score and TopK equations).
 *
 *  qi        e4m3 [B, nq, idx_heads, idx_dim]   indexer queries
 *  qi_scale  fp32 [B, nq, idx_heads]            per-(token, head) scale of qi
 *  wi        fp32 [B, nq, idx_heads]            head weights w^I
 *  pos       int32 [B, nq]                      query positions t
 *  idx_out   int32 [B, nq, top_k]  selected entry indices in ascending order; when fewer
 *            than top_k entries are visible all of them are selected and the rest is -1.
 *            Ties at the k-th score go to the lower index.
 *  score_out fp32 [B, nq, top_k] or NULL: I_{t,s} of each selected index (-inf for -1 pads);
 *            with CSA_SCORE_BF16 the bf16 value the selection ranked, widened to fp32.
 * Caches of more than 32768 entries (n_max) take at most 4096 query rows (B*nq) per call
 * (CSA_ERR_UNSUPPORTED otherwise; the same holds for csa_decode's B and csa_prefill's B*T).
 */
int csa_index_topk(const csa_config_t* cfg, int32_t B, int32_t nq, const uint8_t* qi,
                   const float* qi_scale, const float* wi, const csa_cache_t* cache,
                   const int32_t* pos, int32_t* idx_out, float* score_out, void* workspace,
                   size_t ws_bytes, void* stream);

/* csa_sparse_mqa - shared-KV multi-query attention of each query over its selected entries
 * plus its sliding window, with a per-head sink logit in the softmax denominator:
 * p_j = exp(z_j) / (exp(a_h) + sum_u exp(z_u)), z_j = scale * RoPE(q_h, t) . e_j, o_h =
 * sum_j p_j e_j, whose last rope_dim dims are rotated back by -t.
 * Book "DeepSeek V4 模型技术大全", chapter "Attention": component table (shared K=V MQA,
 * attention sink, window W_t = {t-n_win+1..t}), section "注意力实现细节" (partial RoPE with
 * reverse rotation of the core-attention output).
 *
 *  q       bf16 [B, nq, n_heads, head_dim]  RMS-normalised queries, not rotated
 *  idx     int32 [B, nq, top_k]             entry indices (any order; -1 entries skipped)
 *  pos     int32 [B, nq]                    query positions t (window = max(0,t-n_win+1)..t;
 *                                           those rows must be present in cache->window)
 *  sink    fp32 [n_heads]                   sink logits a_h
 *  out     bf16 [B, nq, n_heads, head_dim]
 *  lse_out fp32 [B, nq, n_heads] or NULL:   log sum_j exp(z_j) without the sink
 */
int csa_sparse_mqa(const csa_config_t* cfg, int32_t B, int32_t nq, const uint16_t* q,
                   const csa_cache_t* cache, const int32_t* idx, const int32_t* pos,
                   const float* sink, uint16_t* out, float* lse_out, void* workspace,
                   size_t ws_bytes, void* stream);

/* hca_dense_mqa - as csa_sparse_mqa but over every closed entry j < min(n_entries[b],
 * floor((t+1)/m')) (no indexer), plus the window and the sink.
 * Book "DeepSeek V4 模型技术大全", chapter "Attention", section "HCA 的完整路径" (visible set
 * J_t and K_attn(t) = entries[J_t] U window).  Arguments as csa_sparse_mqa without idx. */
int hca_dense_mqa(const csa_config_t* cfg, int32_t B, int32_t nq, const uint16_t* q,
                  const csa_cache_t* cache, const int32_t* pos, const float* sink, uint16_t* out,
                  float* lse_out, void* workspace, size_t ws_bytes, void* stream);

/* csa_decode - one decode step for B sequences at positions pos[b]:
 *  1. if h_new != NULL: csa_compress of the new token (T=1, pos0=pos) with weights w;
 *  2. CSA mode: csa_index_topk (nq=1) then csa_sparse_mqa; HCA mode: hca_dense_mqa.
 *  h_new bf16 [B, hidden] or NULL (then w may be NULL and the cache must already hold the
 *  token's window row); q bf16 [B, n_heads, head_dim]; qi/qi_scale/wi as csa_index_topk
 *  with nq=1 (ignored in HCA mode); out bf16 [B, n_heads, head_dim];
 *  idx_out int32 [B, top_k] or NULL (CSA: the selected indices). */
int csa_decode(const csa_config_t* cfg, int32_t B, const uint16_t* h_new,
               const csa_weights_t* w, const csa_cache_t* cache, const int32_t* pos,
               const uint16_t* q, const uint8_t* qi, const float* qi_scale, const float* wi,
               const float* sink, uint16_t* out, int32_t* idx_out, void* workspace,
               size_t ws_bytes, void* stream);

/* csa_decode_noalloc - csa_decode without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Same arguments, effects and errors as csa_decode, minus workspace/ws_bytes.  Scratch comes from
 * a static device array of CSA_NOALLOC_SCRATCH_BYTES inside the library: each GPU the library
 * runs on holds its own copy until the process ends, and its address is looked up once per
 * device, on the first call with that device current.  A step needing more scratch than that
 * (csa_workspace_size(cfg, CSA_OP_DECODE, B, 1, n_max, ...)) returns CSA_ERR_UNSUPPORTED and
 * launches nothing; the configured workloads need at most about 17 MiB (1M-context HCA, B=16).
 * The call allocates nothing: no hipMalloc, hipFree or allocating library routine (with the
 * opt-in launch timer off).  All calls on one GPU share its array, so calls that overlap on one
 * GPU (different streams or threads without ordering between them) race: serialise them. */
#define CSA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int csa_decode_noalloc(const csa_config_t* cfg, int32_t B, const uint16_t* h_new,
                       const csa_weights_t* w, const csa_cache_t* cache, const int32_t* pos,
                       const uint16_t* q, const uint8_t* qi, const float* qi_scale,
                       const float* wi, const float* sink, uint16_t* out, int32_t* idx_out,
                       void* stream);

/* csa_prefill - causal layer over T new tokens of each of B sequences: csa_compress, then for
 * every new token t as a query the causal csa_index_topk and csa_sparse_mqa (HCA mode:
 * hca_dense_mqa).
 *  pos0  NULL: every sequence starts at position 0 (tokens 0..T-1); every block is written
 *        whatever n_entries holds on entry, and n_entries ends as floor(T/m).  Requires
 *        cache->win_slots >= T.
 *        int32 [B] device: chunked prefill.  Sequence b continues at pos0[b] (tokens
 *        pos0[b]..pos0[b]+T-1) on a cache that holds its earlier chunks: the compressor
 *        continues exactly as csa_compress with the same pos0 (n_entries[b] = floor(pos0[b]/m)
 *        on entry, the tail ring holding the earlier tokens' projections), and query i of
 *        sequence b sits at position pos0[b]+i.  The window ring must keep the last n_win-1
 *        rows of the earlier chunks while this chunk's rows are written: requires
 *        cache->win_slots >= T + n_win - 1, the same ring size for every chunk of a sequence
 *        (row u lives in slot u % win_slots).  Book "DeepSeek V4 模型技术大全", section "1M
 *        context 推理策略", row "chunked prefill" (a long prompt enters in chunks that write the
 *        cache as they go; closed compressed entries advance at each chunk's end, the window
 *        rolls, and causality, positions and the compressor's state carry across the
 *        boundary).  A sequence prefilled in chunks of 16 or more tokens gets the bits of a
 *        single call over the whole prompt.
 * q bf16 [B, T, n_heads, head_dim]; qi/qi_scale/wi as csa_index_topk with nq=T; out bf16
 * [B, T, n_heads, head_dim]; idx_out int32 [B, T, top_k] or NULL. */
int csa_prefill(const csa_config_t* cfg, int32_t B, int32_t T, const uint16_t* H,
                const int32_t* pos0, const csa_weights_t* w, const csa_cache_t* cache,
                const uint16_t* q, const uint8_t* qi, const float* qi_scale, const float* wi,
                const float* sink, uint16_t* out, int32_t* idx_out, void* workspace,
                size_t ws_bytes, void* stream);

/* Weights of the query-side projections (device, bf16 unless noted; one row per output
 * column, like w_cat):
 *  w_dq  [q_rank, hidden]            W^DQ  (c^Q = h W^DQ)
 *  w_w   [idx_heads, hidden]         W_w   (w^I = h W_w; CSA, NULL for HCA)
 *  w_uq  [n_heads*head_dim, q_rank]  W^UQ  (attention query before its per-head RMSNorm)
 *  w_iuq [idx_heads*idx_dim, q_rank] W^IUQ (q^I = c^Q W^IUQ; CSA, NULL for HCA)
 *  gamma_q fp32 [head_dim]           RMSNorm gain of every attention-query head */
typedef struct csa_qproj_weights {
  const uint16_t* w_dq;
  const uint16_t* w_w;
  const uint16_t* w_uq;
  const uint16_t* w_iuq;
  const float* gamma_q;
} csa_qproj_weights_t;

/* Weights of the grouped output projection (device, bf16, one row per output column):
 *  w_down [out_groups, out_rank, (n_heads/out_groups)*head_dim]  W^[u]_down of group u
 *  w_proj [hidden, out_groups*out_rank]                         Proj */
typedef struct csa_oproj_weights {
  const uint16_t* w_down;
  const uint16_t* w_proj;
} csa_oproj_weights_t;

/* csa_query_proj - the queries of T tokens of B sequences from their hidden states.
 * Book, chapter "Attention", section "CSA 的完整路径": c^Q = h W^DQ, q^I = c^Q W^IUQ split
 * into idx_heads heads, w^I = h W_w; section "注意力实现细节": queries are RMS-normalised.
 *  H bf16 [B, T, hidden];
 *  q_out bf16 [B, T, n_heads, head_dim]: c^Q W^UQ, each head RMS-normalised over head_dim with
 *        gain gamma_q (eps = rms_eps), not rotated (the attention calls rotate it at t);
 *  qi_out e4m3 [B, T, idx_heads, idx_dim], qi_scale_out fp32 [B, T, idx_heads] (max|x|/448 per
 *        head), wi_out fp32 [B, T, idx_heads]: the csa_index_topk inputs (CSA; NULL for HCA);
 *        with idx_query_format CSA_IDX_MXFP4, qi_out packed MXFP4 [B, T, idx_heads, idx_dim/2]
 *        and qi_scale_out its E8M0 block-scale bytes, 4 per head (as csa_config_t describes).
 * c^Q is kept in bf16 between the two products; all products accumulate in fp32.
 * Requires hidden and q_rank multiples of 64. */
int csa_query_proj(const csa_config_t* cfg, int32_t B, int32_t T, const uint16_t* H,
                   const csa_qproj_weights_t* w, uint16_t* q_out, uint8_t* qi_out,
                   float* qi_scale_out, float* wi_out, void* workspace, size_t ws_bytes,
                   void* stream);

/* csa_output_proj - grouped output projection of T tokens of B sequences.
 * Book, chapter "Attention", section "注意力实现细节" and its component table:
 * O = Concat_u O^[u] (group u = heads u*n_heads/g .. (u+1)*n_heads/g-1), z^[u] = O^[u] W^[u]_down,
 * y = Proj(Concat_u z^[u]).
 *  O bf16 [B, T, n_heads, head_dim] (the attention output); y_out bf16 [B, T, hidden].
 * z is kept in bf16 between the two products.  Requires out_groups dividing n_heads and
 * (n_heads/out_groups)*head_dim, out_groups*out_rank multiples of 64. */
int csa_output_proj(const csa_config_t* cfg, int32_t B, int32_t T, const uint16_t* O,
                    const csa_oproj_weights_t* w, uint16_t* y_out, void* workspace,
                    size_t ws_bytes, void* stream);

/* ---- Block manager (host only; no device work) ------------------------------------------
 * Book "DeepSeek V4 模型技术大全", chapter "Attention": the hybrid cache keeps compressed entries
 * in blocks of lcm(m, 128) = 128 tokens and reuses the blocks of a shared token prefix.  One
 * block id names the same 128 tokens in every pool of the block layout (CSA entries, indexer
 * keys and scales, HCA entries), so one manager serves all of a model's CSA and HCA layers when
 * their pools hold the same n_blocks.
 *
 * The manager tracks, per block id 0..n_blocks-1, a reference count (sequences whose table maps
 * it) and a registry of full blocks under a 64-bit key naming the token prefix they end
 * (csa_blocks_chain_keys).  A registered block whose count reaches zero stays registered
 * ("idle") until a lookup takes it back or an allocation finds no never-registered block free;
 * allocation then recycles the least recently released idle block and unregisters it.
 * A manager is used by one thread at a time.  Errors: CSA_ERR_INVALID_ARG (NULL, out-of-range
 * or unreferenced block, over-release; nothing changes), CSA_ERR_UNSUPPORTED (not enough free
 * blocks; nothing allocated). */
typedef struct csa_block_manager csa_block_manager_t;
int csa_blocks_create(int32_t n_blocks, csa_block_manager_t** out /* host */);
int csa_blocks_destroy(csa_block_manager_t* m);
/* *n_free = blocks allocatable now (free + idle), *n_idle = idle registered blocks (either
 * pointer may be NULL). */
int csa_blocks_counts(const csa_block_manager_t* m, int32_t* n_free, int32_t* n_idle);
int csa_blocks_refcount(const csa_block_manager_t* m, int32_t block, int32_t* count);
/* n fresh blocks into blocks[0..n) (host), each with count 1; all or nothing. */
int csa_blocks_alloc(csa_block_manager_t* m, int32_t n, int32_t* blocks);
/* One more reference to each listed block (a sequence mapping another's blocks). */
int csa_blocks_share(csa_block_manager_t* m, int32_t n, const int32_t* blocks);
/* One reference less per listing; a block reaching zero becomes free (idle if registered). */
int csa_blocks_release(csa_block_manager_t* m, int32_t n, const int32_t* blocks);
/* Register a block in use, now holding the entries of the whole prefix named by key.  A key
 * already registered keeps its first block (the call succeeds and changes nothing). */
int csa_blocks_publish(csa_block_manager_t* m, uint64_t key, int32_t block);
/* Longest run of leading keys[0..n_keys) that are registered: their blocks go to
 * blocks[0..*n_hit) (host) with one more reference each (idle blocks come back into use).  The
 * caller then maps them, rebuilds the sequence's window and compressor tail from the last
 * max(n_win, 2m) prefix tokens (csa_compress with n_entries preset) and continues. */
int csa_blocks_lookup(csa_block_manager_t* m, int32_t n_keys, const uint64_t* keys,
                      int32_t* blocks, int32_t* n_hit);
/* Prefix keys of the floor(n_tokens / block_tokens) whole blocks of a token-id sequence (host
 * arrays): key j depends on seed and on tokens 0 .. (j+1)*block_tokens-1 only, through a chain
 * of 64-bit mixes (the splitmix64 finaliser).  Equal prefixes give equal keys; any differing
 * token changes its block's key and every later one. */
int csa_blocks_chain_keys(const int32_t* tokens, int32_t n_tokens, int32_t block_tokens,
                          uint64_t seed, uint64_t* keys);

#ifdef __cplusplus
}
#endif

#endif /* CSA_H_ */
