"""CPU oracle for Compressed Sparse Attention (CSA) and Heavily Compressed Attention (HCA).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and its Python
binding) may import, call or link this package; only the test suite, the smoke check and
the benchmark's CPU-baseline leg use it.

It is a plain, slow, float64 numpy execution of the method as the pages define it, with no
tiling, fusion or reordering beyond what the definitions state.  Sources, cited by page title
and section:

* "DeepSeek V4 模型技术大全" (wineandchord.com book), chapter "Attention", section
  "CSA 的完整路径" (compressor, indexer and top-k equations), section "HCA 的完整路径"
  (heavy compressor and visibility set), section "注意力实现细节" (RMSNorm of entries,
  partial RoPE on the last 64 dims with reverse rotation of the output), and the component
  table (attention-sink probability, the window set W_t, lcm(4,128)=128 block alignment).
* "DeepSeek-V4 技术报告深度解读" (chang-wenbin.github.io), sections 2.1-2.3 (the five CSA
  components in words; partial RoPE; learnable sink logit).

Every function states the passage it follows.  Where the pages are silent the reading taken
is named in the function's docstring (R1..R25); the same list is in the design notes.

Parity pins: every public function is pinned by tests that do not reuse its own formula
(closed forms, textbook special cases computed with torch, hand-computed fixtures under
tests/golden/, brute force on tiny inputs).  No function here is "parity unpinned".
"""
from .numerics import (bf16_bits_to_f64, f64_to_bf16_bits, e4m3_table, e4m3_decode,
                       e4m3_encode, quantize_rows_e4m3, e2m1_decode, e2m1_encode,
                       mx_shared_exponent, quantize_rows_mxfp4, mxfp4_decode)
from .csa import (project, pool_overlap, pool_plain, rms_norm, rope_rotate, split_columns,
                  compress_tokens, index_scores, index_scores_mxfp4, index_scores_fp4,
                  round_scores_bf16, score_function, topk_select,
                  visible_entries, window_tokens, attend, csa_query, hca_query, csa_layer,
                  hca_layer, query_projections, grouped_output_projection,
                  quantize_entries_mixed, decode_entries_mixed)

__all__ = [
    "bf16_bits_to_f64", "f64_to_bf16_bits", "e4m3_table", "e4m3_decode", "e4m3_encode",
    "quantize_rows_e4m3", "e2m1_decode", "e2m1_encode", "mx_shared_exponent",
    "quantize_rows_mxfp4", "mxfp4_decode", "index_scores_mxfp4", "index_scores_fp4",
    "round_scores_bf16", "score_function", "project", "pool_overlap",
    "pool_plain", "rms_norm", "rope_rotate", "split_columns", "compress_tokens", "index_scores", "topk_select", "visible_entries",
    "window_tokens", "attend", "csa_query", "hca_query", "csa_layer", "hca_layer",
    "query_projections", "grouped_output_projection", "quantize_entries_mixed",
    "decode_entries_mixed",
]
