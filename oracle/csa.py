"""CSA / HCA, step by step, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Notation follows "DeepSeek V4 模型技术大全" (wineandchord.com), chapter "Attention":
H = hidden states [T, D]; m = CSA compression ratio (4); m' = HCA ratio (128); c = d_h = entry
width (512); r = RoPE dims (64, the last r of c); H_I, d_I = indexer heads / dim; n_h = query
heads; k = top-k; n_win = 128.  Token indices are 0-based, as the book states for both the CSA
and the HCA visibility sets.

Readings taken where the pages are silent (also listed in the design notes):
  R1  the compressor's Softmax_row runs per channel over the 2m (HCA: m') token rows;
  R2  block 0 of the overlapping compressor has no b-rows (tokens -m..-1 do not exist);
  R3  Z has the same width as C; B^a, B^b are [m, width] (HCA B is [m', width]);
  R4  a trailing incomplete block is never emitted;
  R5  indexer keys: the compressor output with no RMSNorm and no RoPE, E4M3 with a per-entry
      float32 scale; the indexer query is E4M3 with a per-(token, head) float32 scale;
  R6  partial RoPE on the last r dims in interleaved pairs (2i, 2i+1) with the caller's
      inverse-frequency table; an entry's position is m*i (HCA m'*i), a token's is its index;
  R7  the index score I_{t,s} carries no extra scale;
  R8  top-k ties: the lower entry index wins; fewer than k visible entries -> all of them;
      the selected set is returned in ascending index order;
  R9  the window of query t is tokens max(0, t-n_win+1) .. t, inclusive of t;
  R10 the window's uncompressed KV of token u is RMSNorm(h_u W_win) (own gain) with RoPE at u;
  R11 the sparse (or dense-compressed) branch, the window branch and the sink share ONE
      softmax over the union of their keys;
  R12 logits are scaled by the caller's softmax scale (1/sqrt(d_h) in the workloads);
  R13 the sink only adds exp(a_h) to the denominator;
  R14 the attention output's last r dims are rotated back by -t;
  R18 the query arrives RMS-normalised (its projection and norm are upstream) but not
      rotated: the attention step applies RoPE at the query position t;
  R19 optional FP4 indexer keys are OCP MXFP4: 32 consecutive dims share one E8M0 scale
      (shared exponent floor(log2 max|v|) - 2, all-zero block -127), elements E2M1 with ties to
      even and saturation.  Paired with an E4M3 query this is a labelled variant of this
      library (index_scores_mxfp4), not the pages' path, which R24 gives;
  R24 the pages' FP4 indexer QK path: the indexer query is FP4 too, quantised like the keys
      (MXFP4, blocks of 32 dims of one (token, head) row, one E8M0 scale per block), so both
      operands of every q^I . K dot product are MXFP4 values (index_scores_fp4);
  R25 optional BF16 index scores: each score I_{t,s} is rounded to bf16 (nearest, ties to even)
      before TopK, and TopK runs on the rounded values with the lower index winning the (now
      frequent) ties (round_scores_bf16); index sets are then compared outside a band of one
      bf16 ulp of the k-th score instead of 1e-3;
  R20 query side: c^Q = h W^DQ is stored in bf16 between the two projections; the attention
      query is c^Q W^UQ RMS-normalised over each head's c dims with one gain vector shared by
      the heads, stored bf16 and not rotated (R18); q^I = c^Q W^IUQ is stored as R5; w^I = h W_w
      stays fp32;
  R21 grouped output projection: group u holds the consecutive heads u*n_h/g .. (u+1)*n_h/g-1,
      z^[u] is stored in bf16, Proj is a plain linear map from g*r_o to D (no bias), y in bf16;
  R22 mixed-precision entries (optional): the pages keep the RoPE dims of a KV entry in BF16 and
      the other dims in FP8 without naming a scale: dims 0..c-r-1 are stored as E4M3 codes of
      the normalised, gain-scaled value itself (RNE, saturating at 448, no scale: RMS-normalised
      entries stay far inside E4M3's range), dims c-r..c-1 (rotated) as bf16; window rows stay
      bf16.  E4M3 values are exact in bf16, so a decoded entry is a bf16 row.
"""
import numpy as np

from .numerics import (bf16_bits_to_f64, f64_to_bf16_bits, e4m3_decode, e4m3_encode,
                       quantize_rows_e4m3,
                       quantize_rows_mxfp4, mxfp4_decode)


# ----------------------------------------------------------------------------- a1 projections

def project(h_bits, w_bits):
    """C = H W for every projection at once (CSA: C^a, C^b, Z^a, Z^b and the indexer's own four,
    plus the window projection; HCA: C, Z and the window projection).

    Book, chapter "Attention", section "CSA 的完整路径", first equation (C^a = H W^a_KV, ...);
    section "HCA 的完整路径", first equation.  h_bits [T, D] and w_bits [cols, D] (one row per
    output column) are bf16; products and sums in float64.  Returns [T, cols].
    """
    H = bf16_bits_to_f64(h_bits)
    W = bf16_bits_to_f64(w_bits)
    return H @ W.T


def split_columns(P, mode, c, d_i):
    """Split the concatenated projection columns into named streams.

    Column order of the concatenated weight (a layout choice of this library):
      CSA: [Wa_KV c | Wb_KV c | Wa_Z c | Wb_Z c | Wa_I dI | Wb_I dI | Wa_IZ dI | Wb_IZ dI | W_win c]
      HCA: [W_KV c | W_Z c | W_win c]
    """
    if mode == "csa":
        o = 0
        out = {}
        for name, w in (("Ca", c), ("Cb", c), ("Za", c), ("Zb", c), ("Ia", d_i), ("Ib", d_i),
                        ("IZa", d_i), ("IZb", d_i), ("Win", c)):
            out[name] = P[..., o:o + w]
            o += w
        assert o == P.shape[-1]
        return out
    if mode == "hca":
        assert P.shape[-1] == 3 * c
        return {"C": P[..., :c], "Z": P[..., c:2 * c], "Win": P[..., 2 * c:]}
    raise ValueError(mode)


# ----------------------------------------------------------------------------- a2 pooling

def _softmax_over_rows(logits):
    """Softmax over axis 0 (the token rows), independently per channel (reading R1)."""
    mx = np.max(logits, axis=0, keepdims=True)
    e = np.exp(logits - mx)
    return e / np.sum(e, axis=0, keepdims=True)


def pool_overlap(Ca, Cb, Za, Zb, Ba, Bb, m, n_blocks):
    """Overlapping 2m-token compressor.

    Book, chapter "Attention", section "CSA 的完整路径", second and third equations: for block i
    the weights [S^a_{mi..m(i+1)-1}; S^b_{m(i-1)..mi-1}] are a row-softmax of
    [Z^a_{mi..m(i+1)-1} + B^a; Z^b_{m(i-1)..mi-1} + B^b] and the entry is
    sum_j S^a_j (.) C^a_j + sum_j S^b_j (.) C^b_j.  Block 0 has no b-rows (R2).
    Ca, Cb, Za, Zb: [T, w]; Ba, Bb: [m, w].  Returns [n_blocks, w].
    """
    w = Ca.shape[1]
    out = np.zeros((n_blocks, w), dtype=np.float64)
    for i in range(n_blocks):
        a_rows = slice(m * i, m * (i + 1))
        logits = [Za[a_rows] + Ba]
        values = [Ca[a_rows]]
        if i >= 1:
            b_rows = slice(m * (i - 1), m * i)
            logits.append(Zb[b_rows] + Bb)
            values.append(Cb[b_rows])
        S = _softmax_over_rows(np.concatenate(logits, axis=0))
        out[i] = np.sum(S * np.concatenate(values, axis=0), axis=0)
    return out


def pool_plain(C, Z, Bias, m, n_blocks):
    """Non-overlapping m'-token compressor of HCA.

    Book, chapter "Attention", section "HCA 的完整路径", second equation:
    S_{m'i..m'(i+1)-1} = Softmax_row(Z_{m'i..m'(i+1)-1} + B), entry = sum_j S_j (.) C_j.
    """
    w = C.shape[1]
    out = np.zeros((n_blocks, w), dtype=np.float64)
    for i in range(n_blocks):
        rows = slice(m * i, m * (i + 1))
        S = _softmax_over_rows(Z[rows] + Bias)
        out[i] = np.sum(S * C[rows], axis=0)
    return out


def rms_norm(x, gamma, eps):
    """RMSNorm over the last axis: x / sqrt(mean(x^2) + eps) * gamma.

    Book, chapter "Attention", component table row "RMSNorm for query / compressed entries" and
    section "注意力实现细节" (queries and compressed entries are RMS-normalised); eps 1e-6 is
    the book's configuration table value.
    """
    x = np.asarray(x, dtype=np.float64)
    rms = np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return x / rms * np.asarray(gamma, dtype=np.float64)


def rope_rotate(x, positions, inv_freq, sign=1.0):
    """Partial RoPE on the last r = 2*len(inv_freq) dims, interleaved pairs (reading R6).

    Book, chapter "Attention", section "注意力实现细节": RoPE only on the last 64 dims, and the
    core-attention output is rotated back (sign = -1, reading R14).  Pair i of the RoPE slice
    (x0, x1) at position p turns by angle sign * p * inv_freq[i]:
    (x0 cos - x1 sin, x0 sin + x1 cos).  x: [..., c]; positions broadcast against x[..., 0].
    """
    x = np.array(x, dtype=np.float64, copy=True)
    f = np.asarray(inv_freq, dtype=np.float64)
    r = 2 * f.shape[0]
    c = x.shape[-1]
    p = np.asarray(positions, dtype=np.float64)[..., None]
    ang = sign * p * f  # [..., r/2]
    cs, sn = np.cos(ang), np.sin(ang)
    x0 = x[..., c - r + 0::2].copy()
    x1 = x[..., c - r + 1::2].copy()
    x[..., c - r + 0::2] = x0 * cs - x1 * sn
    x[..., c - r + 1::2] = x0 * sn + x1 * cs
    return x


def quantize_entries_mixed(values, r):
    """Mixed-precision storage of compressed entries (reading R22; Book, chapter "Attention",
    section "注意力实现细节": RoPE dims in BF16, the rest in FP8).  values float64 [n, c]
    (normalised and rotated).  Returns (codes uint8 [n, c-r]: E4M3 of dims 0..c-r-1, rope
    uint16 [n, r]: bf16 bits of dims c-r..c-1)."""
    values = np.asarray(values, np.float64)
    c = values.shape[1]
    return e4m3_encode(values[:, :c - r]), f64_to_bf16_bits(values[:, c - r:])


def decode_entries_mixed(codes, rope_bits):
    """bf16 bits [n, c] of the real values of mixed-precision entries (reading R22): the E4M3
    dims decoded (exactly representable in bf16), then the bf16 RoPE dims."""
    vals = np.concatenate([e4m3_decode(codes), bf16_bits_to_f64(rope_bits)], axis=1)
    return f64_to_bf16_bits(vals)


def compress_tokens(h_bits, w_bits, params, mode, m, c, d_i, inv_freq, eps, idx_format="e4m3",
                    entry_format="bf16"):
    """Run the compressor on a whole token prefix H[0:T] (a1 + a2 + epilogue).

    Returns a dict with
      entries  uint16 [floor(T/m), c]  bf16 bits of RoPE(RMSNorm(C^Comp_i) * gamma, m*i)
      pre      float64 [floor(T/m), c] C^Comp before the norm (for stage-wise tests)
      ikeys    uint8 [floor(T/m), d_I] E4M3 codes of K^IComp (CSA only; reading R5), or with
               idx_format "mxfp4" uint8 [floor(T/m), d_I/2] packed MXFP4 codes (reading R19)
      iscale   float32 [floor(T/m)], or uint8 [floor(T/m), d_I/32] E8M0 block scales (mxfp4)
      ipre     float64 [floor(T/m), d_I]
      win      uint16 [T, c] bf16 bits of RoPE(RMSNorm(h_u W_win) * gamma_win, u) (reading R10)
      ecodes, erope  (entry_format "mixed") quantize_entries_mixed of the same values (R22)
    params: dict with Ba, Bb, BIa, BIb (CSA) or B (HCA), gamma, gamma_win.
    Book, chapter "Attention": "CSA 的完整路径" (compressor; K^IComp from the same
    compression operation), "HCA 的完整路径" (m' compressor), "注意力实现细节" (RMSNorm and
    partial RoPE of compressed entries).
    """
    P = project(h_bits, w_bits)
    T = P.shape[0]
    n = T // m  # reading R4
    s = split_columns(P, mode, c, d_i)
    out = {}
    if mode == "csa":
        pre = pool_overlap(s["Ca"], s["Cb"], s["Za"], s["Zb"], params["Ba"], params["Bb"], m, n)
        ipre = pool_overlap(s["Ia"], s["Ib"], s["IZa"], s["IZb"], params["BIa"], params["BIb"],
                            m, n)
        if idx_format == "mxfp4":
            codes, scale = quantize_rows_mxfp4(ipre)
        else:
            codes, scale = quantize_rows_e4m3(ipre)
        out.update(ikeys=codes, iscale=scale, ipre=ipre)
    else:
        pre = pool_plain(s["C"], s["Z"], params["B"], m, n)
    normed = rms_norm(pre, params["gamma"], eps)
    rotated = rope_rotate(normed, m * np.arange(n), inv_freq)
    out["entries"] = f64_to_bf16_bits(rotated)
    if entry_format == "mixed":
        out["ecodes"], out["erope"] = quantize_entries_mixed(rotated, 2 * len(inv_freq))
    out["pre"] = pre
    win = rope_rotate(rms_norm(s["Win"], params["gamma_win"], eps), np.arange(T), inv_freq)
    out["win"] = f64_to_bf16_bits(win)
    return out


# ----------------------------------------------------------------------------- a3/a4 indexer

def visible_entries(t, m, n_entries):
    """Number of closed compressed blocks visible to the query at token t: floor((t+1)/m),
    capped by the number of entries that exist.  Book, chapter "Attention": the CSA score set
    s < floor((t+1)/m) and the HCA set j < floor((t+1)/m') (0-based tokens)."""
    return int(min(n_entries, (t + 1) // m))


def window_tokens(t, n_win):
    """Token indices of the sliding window of query t: max(0, t-n_win+1) .. t (reading R9;
    book component table, W_t = {u | t - n_win + 1 <= u <= t})."""
    return np.arange(max(0, t - n_win + 1), t + 1)


def index_scores(qi_codes, qi_scale, wi, ki_codes, ki_scale, n_vis):
    """Lightning-indexer scores I_{t,s} for one query token over entries s < n_vis.

    Book, chapter "Attention", section "CSA 的完整路径":
    I_{t,s} = sum_h w^I_{t,h} ReLU(q^I_{t,h} . K^IComp_s), with no extra scale (R7).  The
    stored operands are E4M3 codes with float32 scales (R5); each is decoded to its real
    value (code value times scale) and the sums run in float64.
    qi_codes [H_I, d_I] u8, qi_scale [H_I] f32, wi [H_I] f32, ki_codes [N, d_I] u8,
    ki_scale [N] f32.  Returns float64 [n_vis].
    """
    q = e4m3_decode(qi_codes) * np.asarray(qi_scale, np.float64)[:, None]   # [H_I, d_I]
    k = e4m3_decode(ki_codes[:n_vis]) * np.asarray(ki_scale[:n_vis], np.float64)[:, None]
    dots = k @ q.T                                                           # [n_vis, H_I]
    return np.maximum(dots, 0.0) @ np.asarray(wi, np.float64)


def index_scores_mxfp4(qi_codes, qi_scale, wi, ki_packed, ki_scales, n_vis):
    """index_scores with the keys in MXFP4 (reading R19: the pages' FP4 indexer keys, the
    "FP4 indexer" of the V4 model card, stored as OCP MXFP4; the query stays E4M3 with a
    per-head scale).  Same formula as index_scores; each key is decoded to its real value
    (E2M1 code times its block's power-of-two scale) and the sums run in float64.
    ki_packed [N, d_I/2] u8, ki_scales [N, d_I/32] u8 (E8M0).  Returns float64 [n_vis]."""
    q = e4m3_decode(qi_codes) * np.asarray(qi_scale, np.float64)[:, None]   # [H_I, d_I]
    k = mxfp4_decode(ki_packed[:n_vis], ki_scales[:n_vis])                 # [n_vis, d_I]
    dots = k @ q.T
    return np.maximum(dots, 0.0) @ np.asarray(wi, np.float64)


def index_scores_fp4(qi_packed, qi_scales, wi, ki_packed, ki_scales, n_vis):
    """index_scores with both indexer operands FP4 (reading R24: the pages run the indexer's QK
    product in FP4, query and keys alike - Deep dive "论文专题讲解：DeepSeek-V4", section "FP4
    QAT", table row "CSA indexer QK path"; Analysis "DeepSeek-V4 技术报告深度解读" §5.4).  The query
    of each head is one MXFP4 row: its real values are E2M1 codes times the power-of-two scale
    of their 32-dim block, as are the keys', and the dot products, ReLU and the head sum run in
    float64 on those values.  qi_packed [H_I, d_I/2] u8, qi_scales [H_I, d_I/32] u8 (E8M0),
    wi [H_I] f32, ki_packed [N, d_I/2] u8, ki_scales [N, d_I/32] u8.  Returns float64 [n_vis]."""
    q = mxfp4_decode(qi_packed, qi_scales)                                  # [H_I, d_I]
    k = mxfp4_decode(ki_packed[:n_vis], ki_scales[:n_vis])                 # [n_vis, d_I]
    dots = k @ q.T
    return np.maximum(dots, 0.0) @ np.asarray(wi, np.float64)


def round_scores_bf16(scores):
    """Index scores stored in BF16 before the top-k (reading R25; Deep dive "论文专题讲解：
    DeepSeek-V4", section "FP4 QAT", table row "index scores": FP32 -> BF16, which the pages
    credit with a 2x faster top-k selector).  Each score is rounded to the nearest bf16 number
    (ties to even); returns the float64 values of those numbers."""
    return bf16_bits_to_f64(f64_to_bf16_bits(scores))


def topk_select(scores, k):
    """TopK_k over the visible scores (book, chapter "Attention", section "CSA 的完整路径",
    I_t = TopK_k{I_{t,s} | s < floor((t+1)/m)}).  Ties: lower index wins; fewer than k
    candidates: all of them (R8).  Returns the selected indices in ascending order (int64)."""
    scores = np.asarray(scores, dtype=np.float64)
    kk = min(k, scores.shape[0])
    order = np.argsort(-scores, kind="stable")
    return np.sort(order[:kk])


# ----------------------------------------------------------------------------- a5-a7 attention

def attend(q_bits, rows_bits, sink, scale, t, inv_freq):
    """Shared-KV multi-query attention of one query token over a set of key rows, with sink.

    q_bits [n_h, c] bf16 (normalised, not rotated: R18); rows_bits [n, c] bf16 — every row is
    both key and value (book component table "Shared K=V MQA"); sink [n_h] logits a_h.
    For head h: z_j = scale * RoPE(q_h, t) . e_j (R12), and
    p_j = exp(z_j) / (exp(a_h) + sum_u exp(z_u))  (book component table, attention sink),
    o_h = sum_j p_j e_j, then the last r dims of o_h are rotated back by -t (R14).
    All key sources share this one softmax (R11).  Returns (out [n_h, c] float64,
    lse [n_h] = log sum_j exp(z_j) without the sink, or -inf for an empty row set).
    """
    q = rope_rotate(bf16_bits_to_f64(q_bits), t, inv_freq)
    E = bf16_bits_to_f64(rows_bits)
    a = np.asarray(sink, dtype=np.float64)
    n_h = q.shape[0]
    if E.shape[0] == 0:
        return np.zeros_like(q), np.full(n_h, -np.inf)
    z = scale * (q @ E.T)                               # [n_h, n]
    M = np.maximum(np.max(z, axis=1), a)                # stabiliser
    ez = np.exp(z - M[:, None])
    denom = np.exp(a - M) + np.sum(ez, axis=1)
    p = ez / denom[:, None]
    o = p @ E
    lse = M + np.log(np.sum(ez, axis=1))
    return rope_rotate(o, t, inv_freq, sign=-1.0), lse


def score_function(idx_format="e4m3", qi_format="e4m3"):
    """The index-score function of a key format (idx_format "e4m3" or "mxfp4") and query format
    (qi_format "e4m3" or "mxfp4"; an MXFP4 query needs MXFP4 keys, reading R24)."""
    if qi_format == "mxfp4":
        assert idx_format == "mxfp4", "an FP4 query is paired with FP4 keys"
        return index_scores_fp4
    return index_scores_mxfp4 if idx_format == "mxfp4" else index_scores


def csa_query(t, q_bits, qi_codes, qi_scale, wi, sink, entries, ikeys, iscale, n_entries, win,
              win_pos_to_row, m, k, n_win, scale, inv_freq, idx_format="e4m3", qi_format="e4m3",
              score_format="fp32"):
    """One CSA query token t: score the visible entries, select the top-k, attend over the
    selected entries plus the sliding window plus the sink.

    entries [N, c] bf16 bits, ikeys [N, d_I], iscale [N]; win: bf16 rows of uncompressed KV and
    win_pos_to_row(u) -> row index into win for token u.  score_format "bf16" rounds the scores
    to bf16 before the top-k (reading R25).
    Returns dict(sel, scores, out, lse).
    """
    n_vis = visible_entries(t, m, n_entries)
    score_fn = score_function(idx_format, qi_format)
    scores = score_fn(qi_codes, qi_scale, wi, ikeys, iscale, n_vis)
    if score_format == "bf16":
        scores = round_scores_bf16(scores)
    sel = topk_select(scores, k)
    rows = [entries[sel]]
    wt = window_tokens(t, n_win)
    rows.append(win[[win_pos_to_row(u) for u in wt]])
    out, lse = attend(q_bits, np.concatenate(rows, axis=0), sink, scale, t, inv_freq)
    return {"sel": sel, "scores": scores, "out": out, "lse": lse}


def hca_query(t, q_bits, sink, entries, n_entries, win, win_pos_to_row, m, n_win, scale,
              inv_freq):
    """One HCA query token t: dense attention over every closed entry j < floor((t+1)/m') plus
    the window and the sink (book, chapter "Attention", section "HCA 的完整路径",
    K_attn(t) = K_HCA[J_t] U K_window)."""
    n_vis = visible_entries(t, m, n_entries)
    wt = window_tokens(t, n_win)
    rows = np.concatenate([entries[:n_vis], win[[win_pos_to_row(u) for u in wt]]], axis=0)
    out, lse = attend(q_bits, rows, sink, scale, t, inv_freq)
    return {"out": out, "lse": lse}


def csa_layer(h_bits, w_bits, params, q_bits, qi_codes, qi_scale, wi, sink, m, c, d_i, k,
              n_win, scale, inv_freq, eps, queries, idx_format="e4m3", qi_format="e4m3",
              score_format="fp32"):
    """Whole CSA layer from hidden states, for the listed query tokens (prefill rows or decode
    steps alike: a decode step at position t is the prefill row t of the longer prefix, since
    every quantity depends only on tokens <= t).  q_bits etc. are indexed by token.
    Returns (compressed dict, {t: csa_query result})."""
    comp = compress_tokens(h_bits, w_bits, params, "csa", m, c, d_i, inv_freq, eps, idx_format)
    res = {}
    for t in queries:
        # entries closed by token t only depend on tokens <= t (causality); the oracle computes
        # them from the whole prefix once and lets visibility mask the rest.
        res[t] = csa_query(t, q_bits[t], qi_codes[t], qi_scale[t], wi[t], sink, comp["entries"],
                           comp["ikeys"], comp["iscale"], comp["entries"].shape[0], comp["win"],
                           lambda u: u, m, k, n_win, scale, inv_freq, idx_format, qi_format,
                           score_format)
    return comp, res


def hca_layer(h_bits, w_bits, params, q_bits, sink, m, c, n_win, scale, inv_freq, eps, queries):
    """Whole HCA layer from hidden states for the listed query tokens."""
    comp = compress_tokens(h_bits, w_bits, params, "hca", m, c, 0, inv_freq, eps)
    res = {}
    for t in queries:
        res[t] = hca_query(t, q_bits[t], sink, comp["entries"], comp["entries"].shape[0],
                           comp["win"], lambda u: u, m, n_win, scale, inv_freq)
    return comp, res


# ----------------------------------------------------------------------------- query and output
# projections (the steps on either side of the attention path)

def query_projections(h_bits, w_dq_bits, w_w_bits, w_uq_bits, w_iuq_bits, gamma_q, n_h, c,
                      H_I, d_I, eps, qi_format="e4m3"):
    """Indexer query, indexer head weights and attention query of every token.

    Book, chapter "Attention", section "CSA 的完整路径": c^Q_t = h_t W^DQ,
    q^I_t = c^Q_t W^IUQ split into n_h^I heads, w^I_t = h_t W_w; section "注意力实现细节":
    queries are RMS-normalised; readings R5, R18, R20.
    h_bits [T, D] bf16; weights bf16, one row per output column: w_dq [r_q, D], w_w [H_I, D],
    w_uq [n_h*c, r_q], w_iuq [H_I*d_I, r_q]; gamma_q [c].
    Returns dict(cq bf16 [T, r_q], q bf16 [T, n_h, c], qi u8 [T, H_I, d_I], qi_scale f32
    [T, H_I], wi f32 [T, H_I], qpre f64 [T, n_h, c], qi_pre f64 [T, H_I, d_I]); with qi_format
    "mxfp4" (reading R24) qi is u8 [T, H_I, d_I/2] packed MXFP4 and qi_scale u8 [T, H_I, d_I/32]
    its E8M0 block scales.
    """
    H = bf16_bits_to_f64(h_bits)
    T = H.shape[0]
    cq = f64_to_bf16_bits(H @ bf16_bits_to_f64(w_dq_bits).T)
    CQ = bf16_bits_to_f64(cq)
    wi = (H @ bf16_bits_to_f64(w_w_bits).T).astype(np.float32)
    qi_pre = (CQ @ bf16_bits_to_f64(w_iuq_bits).T).reshape(T, H_I, d_I)
    if qi_format == "mxfp4":
        qi, qi_scale = quantize_rows_mxfp4(qi_pre)
    else:
        qi, qi_scale = quantize_rows_e4m3(qi_pre)
    qpre = (CQ @ bf16_bits_to_f64(w_uq_bits).T).reshape(T, n_h, c)
    q = f64_to_bf16_bits(rms_norm(qpre, gamma_q, eps))
    return {"cq": cq, "q": q, "qi": qi, "qi_scale": qi_scale, "wi": wi, "qpre": qpre,
            "qi_pre": qi_pre}


def grouped_output_projection(o_bits, w_down_bits, w_proj_bits, g):
    """Layer output from the attention output of every token.

    Book, chapter "Attention", section "注意力实现细节" and the component table row "Grouped
    output projection": O = Concat_u O^[u], z^[u] = O^[u] W^[u]_down with
    W^[u]_down in R^{(n_h/g) d_h x r_o}, y = Proj(Concat_u z^[u]); reading R21.
    o_bits [T, n_h, c] bf16; w_down_bits [g, r_o, (n_h/g)*c] bf16 (row = output column);
    w_proj_bits [D, g*r_o] bf16.  Returns (z bf16 [T, g*r_o], y bf16 [T, D]).
    """
    O = bf16_bits_to_f64(o_bits)
    T = O.shape[0]
    O = O.reshape(T, -1)
    width = O.shape[1] // g
    zs = [O[:, u * width:(u + 1) * width] @ bf16_bits_to_f64(w_down_bits[u]).T for u in range(g)]
    z = f64_to_bf16_bits(np.concatenate(zs, axis=1))
    y = f64_to_bf16_bits(bf16_bits_to_f64(z) @ bf16_bits_to_f64(w_proj_bits).T)
    return z, y
