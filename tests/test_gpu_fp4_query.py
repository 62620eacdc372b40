"""GPU parity of the indexer's FP4 query path (reading R24: query and keys both MXFP4, the
scaled fp4 x fp4 MFMA) and of BF16 index scores (reading R25: scores rounded to bf16 before the
top-k) against the oracle: decode scoring and selection over seeded caches (several chunks,
ragged tails, the multi-workgroup select, two MXFP4 blocks per head, exact ties), the full-size
128K and 1M decodes in the benchmark's launch configuration, the query projection writing an
MXFP4 indexer query, and a whole tiny layer whose compressor writes the MXFP4 keys."""
import numpy as np
import pytest
import torch

import long_context_sparse_15_amd as csa
import oracle as O
from synth import inputs as S
from synth import gpu as G
from gpu_common import (DEV, bf16_f64, check_close, check_scores_bf16, check_selection,
                        check_selection_bf16, config_for, dev, host_bits, say, window_rows_ring,
                        workspace)

pytestmark = pytest.mark.gpu

FMT = {"e4m3": csa.IDX_E4M3, "mxfp4": csa.IDX_MXFP4}


def _ref_scores(x, b, w, key_fmt, qi_fmt, n_vis, ikeys=None, iscale=None):
    ik = x["ikeys"][b] if ikeys is None else ikeys
    isc = x["iscale"][b] if iscale is None else iscale
    fn = O.score_function(key_fmt, qi_fmt)
    qs = x["qi_scale"][b, 0]
    if qi_fmt == "mxfp4":
        qs = qs[:, :w.d_I // 32]
    if key_fmt == "mxfp4":
        isc = isc[:, :w.d_I // 32]
    return fn(x["qi"][b, 0], qs, x["wi"][b, 0], ik, isc, n_vis)


def _check_row(idx_row, sc_row, ref, k, bf16, what):
    kk = min(k, ref.shape[0])
    sel = idx_row[:kk]
    if bf16:
        check_selection_bf16(idx_row, ref, k, what + " selection")
        check_scores_bf16(sc_row[:kk], ref[sel], what + " scores", full_ref=ref)
    else:
        check_selection(idx_row, ref, k, what + " selection")
        check_close(sc_row[:kk], ref[sel], what + " scores",
                    atol=1e-5 * max(1.0, np.abs(ref).max(initial=0.0)), rtol=1e-5)
    assert np.all(np.isneginf(sc_row[kk:])), what + " padding scores"
    return sel


def _decode_case(w, B, N, positions, key_fmt, qi_fmt, score_fmt, ties=False, prep=None):
    x = S.decode_cache_inputs(w, B=B, N=N, key_fmt=key_fmt, qi_fmt=qi_fmt)
    x["pos"] = np.array(positions, dtype=np.int32)
    if ties:  # a block of identical keys: exactly equal scores on both sides
        x["ikeys"][:, 100:] = x["ikeys"][:, 100:101]
        x["iscale"][:, 100:] = x["iscale"][:, 100:101]
    if prep:
        prep(x)
    d = {k: dev(x[k]) for k in ("entries", "window", "pos", "n_entries", "q", "sink", "inv_freq",
                                "ikeys", "iscale", "qi", "qi_scale", "wi")}
    bf16 = score_fmt == "bf16"
    cfg = config_for(w, d["inv_freq"], idx_key_format=FMT[key_fmt],
                     idx_query_format=FMT[qi_fmt],
                     score_format=csa.SCORE_BF16 if bf16 else csa.SCORE_FP32)
    cache = csa.make_cache(N, x["window"].shape[1], d["entries"], d["window"], d["n_entries"],
                           idx_keys=d["ikeys"], idx_scale=d["iscale"])
    ws = workspace(csa.workspace_size(cfg, csa.OP_DECODE, B, 1, N))
    idx = torch.empty((B, 1, w.k), dtype=torch.int32, device=DEV)
    sc = torch.empty((B, 1, w.k), dtype=torch.float32, device=DEV)
    csa.index_topk(cfg, d["qi"], d["qi_scale"], d["wi"], cache, d["pos"], idx, ws, score_out=sc)
    out = torch.empty((B, w.n_h, w.c), dtype=torch.bfloat16, device=DEV)
    idx2 = torch.empty((B, w.k), dtype=torch.int32, device=DEV)
    csa.decode(cfg, cache, d["pos"], d["q"][:, 0].contiguous(), d["sink"], out, ws,
               qi=d["qi"], qi_scale=d["qi_scale"], wi=d["wi"], idx_out=idx2)
    torch.cuda.synchronize()
    idx_h, sc_h = idx.cpu().numpy()[:, 0], sc.cpu().numpy()[:, 0]
    assert np.array_equal(idx2.cpu().numpy(), idx_h), "fused decode selection differs"
    out_h = bf16_f64(out.view(torch.int16))
    slots = x["window"].shape[1]
    for b in range(B):
        t = int(x["pos"][b])
        n_vis = O.visible_entries(t, w.m, x["n_entries"][b])
        ref = _ref_scores(x, b, w, key_fmt, qi_fmt, n_vis)
        sel = _check_row(idx_h[b], sc_h[b], ref, w.k, bf16, "seq %d" % b)
        if ties:
            rr = O.round_scores_bf16(ref) if bf16 else ref
            assert np.array_equal(sel, O.topk_select(rr, w.k)), "tie order"
        rows = np.concatenate([x["entries"][b][sel], window_rows_ring(x["window"][b], t, w.n_win,
                                                                      slots)])
        o_ref, _ = O.attend(x["q"][b, 0], rows, x["sink"], w.scale, t, x["inv_freq"])
        check_close(out_h[b], o_ref, "seq %d output" % b)


CASES = [
    # (workload, B, N, positions): several chunks and a ragged tail; n_vis < k; no entry visible
    ("csa_decode_128k", 3, 5000, [4 * 5000 + 3, 4 * 3000 + 1, 10]),
    ("csa_decode_128k", 2, 20000, [4 * 20000, 4 * 17000 + 3]),   # 1024-thread row select
    ("csa_decode_1m", 2, 40000, [4 * 40000 + 1, 4 * 33000]),     # multi-workgroup select
    ("tiny_csa", 2, 700, [2063, 2]),                              # d_I = 64: two blocks
]


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("score_fmt", ["fp32", "bf16"])
def test_fp4_query_decode_parity(case, score_fmt):
    name, B, N, positions = case
    say("fp4 x fp4 decode", score_fmt, case)
    _decode_case(S.shrink(S.WORKLOADS[name]), B, N, positions, "mxfp4", "mxfp4", score_fmt)


@pytest.mark.parametrize("case", CASES)
def test_bf16_scores_e4m3_decode_parity(case):
    name, B, N, positions = case
    say("bf16 scores, e4m3 decode", case)
    _decode_case(S.shrink(S.WORKLOADS[name]), B, N, positions, "e4m3", "e4m3", "bf16")


@pytest.mark.parametrize("key_fmt,qi_fmt", [("e4m3", "e4m3"), ("mxfp4", "mxfp4")])
def test_bf16_scores_exact_ties_lower_index_wins(key_fmt, qi_fmt):
    say("bf16 scores, exact ties", key_fmt, qi_fmt)
    w = S.shrink(S.WORKLOADS["tiny_csa"])
    _decode_case(w, 2, 900, [4 * 900, 4 * 500], key_fmt, qi_fmt, "bf16", ties=True)


@pytest.mark.parametrize("key_fmt,qi_fmt", [("e4m3", "e4m3"), ("mxfp4", "mxfp4")])
def test_bf16_scores_exact_ties_multi_workgroup(key_fmt, qi_fmt):
    """bf16 scores over 40000 entries (the scorer's per-chunk candidates and the finalize), every
    key from entry 100 on identical: each chunk's candidates overflow its region and the exact
    select decides; the lowest indices win the ties."""
    say("bf16 scores, exact ties, multi-workgroup select", key_fmt, qi_fmt)
    w = S.shrink(S.WORKLOADS["csa_decode_1m"])
    _decode_case(w, 2, 40000, [4 * 40000, 4 * 35000 + 2], key_fmt, qi_fmt, "bf16", ties=True)


def test_bf16_scores_clustered_top_keys_multi_workgroup():
    """bf16 scores over 40000 entries whose top keys all sit in entries 8192..12287 (two of the
    scorer's chunks): those chunks' own thresholds cut keys above the k-th key and the finalize
    re-reads them through the bf16 score rows (the keys it compares are those the scorer ranked)."""
    say("bf16 scores, clustered top keys, multi-workgroup select")
    w = S.shrink(S.WORKLOADS["csa_decode_1m"])

    def prep(x):
        x["iscale"][:, 8192:12288] *= 16.0

    _decode_case(w, 2, 40000, [4 * 40000, 4 * 39000 + 2], "e4m3", "e4m3", "bf16", prep=prep)


def _full(name, score_fmt, sample):
    w = S.WORKLOADS[name]
    say("full-size fp4 x fp4 decode", name, score_fmt)
    x = G.decode_cache_inputs(w, DEV, key_fmt="mxfp4", qi_fmt="mxfp4")
    bf16 = score_fmt == "bf16"
    cfg = csa.make_config(csa.MODE_CSA, w.m, w.n_h, w.c, w.r, x["inv_freq"], top_k=w.k,
                          n_win=w.n_win, idx_heads=w.H_I, idx_dim=w.d_I, softmax_scale=w.scale,
                          idx_key_format=csa.IDX_MXFP4, idx_query_format=csa.IDX_MXFP4,
                          score_format=csa.SCORE_BF16 if bf16 else csa.SCORE_FP32)
    cache = csa.make_cache(w.N, w.n_win, x["entries"], x["window"], x["n_entries"],
                           idx_keys=x["ikeys"], idx_scale=x["iscale"])
    ws = workspace(csa.workspace_size(cfg, csa.OP_DECODE, w.B, 1, w.N))
    out = torch.empty((w.B, w.n_h, w.c), dtype=torch.bfloat16, device=DEV)
    idx = torch.full((w.B, w.k), -7, dtype=torch.int32, device=DEV)
    csa.decode(cfg, cache, x["pos"], x["q"][:, 0].contiguous(), x["sink"], out, ws, qi=x["qi"],
               qi_scale=x["qi_scale"], wi=x["wi"], idx_out=idx)
    torch.cuda.synchronize()
    out_h = bf16_f64(out.view(torch.int16))
    idx_h = idx.cpu().numpy()
    inv, sink = x["inv_freq"].cpu().numpy(), x["sink"].cpu().numpy()
    for b in sample:
        t = int(w.t)
        n_vis = O.visible_entries(t, w.m, w.N)
        ref = O.index_scores_fp4(x["qi"][b, 0].cpu().numpy(),
                                 x["qi_scale"][b, 0].cpu().numpy()[:, :w.d_I // 32],
                                 x["wi"][b, 0].cpu().numpy(), x["ikeys"][b].cpu().numpy(),
                                 x["iscale"][b].cpu().numpy()[:, :w.d_I // 32], n_vis)
        (check_selection_bf16 if bf16 else check_selection)(idx_h[b], ref, w.k,
                                                            "%s seq %d selection" % (name, b))
        ent = x["entries"][b].cpu().numpy().view(np.uint16)
        win = x["window"][b].cpu().numpy().view(np.uint16)
        rows = np.concatenate([ent[idx_h[b][:min(w.k, n_vis)]],
                               win[[u % w.n_win for u in O.window_tokens(t, w.n_win)]]])
        o_ref, _ = O.attend(x["q"][b, 0].cpu().numpy().view(np.uint16), rows, sink, w.scale, t,
                            inv)
        check_close(out_h[b], o_ref, "%s seq %d output" % (name, b))


@pytest.mark.parametrize("score_fmt", ["fp32", "bf16"])
def test_full_fp4_query_decode_128k(score_fmt):
    _full("csa_decode_128k", score_fmt, [0, 19, 31])


@pytest.mark.parametrize("score_fmt", ["fp32", "bf16"])
def test_full_fp4_query_decode_1m(score_fmt):
    _full("csa_decode_1m", score_fmt, [0, 3])


def test_query_projection_writes_mxfp4_indexer_query():
    """csa_query_proj with an MXFP4 indexer query against the oracle's projections: block scale
    bytes equal except where the block's largest value sits within 2^-8 (the bf16 rounding of
    the product) of a power of two, codes within one E2M1 step, w^I and q as with E4M3."""
    rng = np.random.default_rng(7)
    T, D, r_q, n_h, c, H_I, d_I = 40, 256, 128, 4, 128, 8, 128
    say("query projection, mxfp4 indexer query", T, D)
    bf = lambda a: O.f64_to_bf16_bits(a)
    h = bf(rng.standard_normal((T, D)))
    w_dq = bf(rng.standard_normal((r_q, D)) / np.sqrt(D))
    w_w = bf(rng.standard_normal((H_I, D)) / np.sqrt(D))
    w_uq = bf(rng.standard_normal((n_h * c, r_q)) / np.sqrt(r_q))
    w_iuq = bf(rng.standard_normal((H_I * d_I, r_q)) / np.sqrt(r_q))
    gq = (1.0 + 0.1 * rng.standard_normal(c)).astype(np.float32)
    ref = O.query_projections(h, w_dq, w_w, w_uq, w_iuq, gq, n_h, c, H_I, d_I, 1e-6,
                              qi_format="mxfp4")
    inv = dev(S.rope_inv_freq(64, 160000.0))
    cfg = csa.make_config(csa.MODE_CSA, 4, n_h, c, 64, inv, top_k=16, idx_heads=H_I, idx_dim=d_I,
                          hidden=D, q_rank=r_q, idx_key_format=csa.IDX_MXFP4,
                          idx_query_format=csa.IDX_MXFP4)
    wq = csa.make_qproj_weights(dev(w_dq), dev(w_uq), dev(gq), w_w=dev(w_w), w_iuq=dev(w_iuq))
    q = torch.empty((1, T, n_h, c), dtype=torch.int16, device=DEV)
    qi = torch.empty((1, T, H_I, d_I // 2), dtype=torch.uint8, device=DEV)
    qs = torch.full((1, T, H_I, 4), 0, dtype=torch.uint8, device=DEV)
    wi = torch.empty((1, T, H_I), dtype=torch.float32, device=DEV)
    ws = workspace(csa.workspace_size(cfg, csa.OP_QUERY_PROJ, 1, T, 1))
    csa.query_proj(cfg, dev(h)[None], wq, q, ws, qi_out=qi, qi_scale_out=qs, wi_out=wi)
    torch.cuda.synchronize()
    nb = d_I // 32
    got_s = qs[0].cpu().numpy()[..., :nb]
    got_c = qi[0].cpu().numpy()
    amax = np.max(np.abs(ref["qi_pre"].reshape(T, H_I, nb, 32)), axis=-1)
    near = np.abs(amax / np.exp2(np.round(np.log2(np.maximum(amax, 1e-300)))) - 1.0) < 2.0 ** -8
    same = got_s == ref["qi_scale"]
    assert np.all(same | near), "block scale bytes differ away from a power-of-two boundary"
    assert same.mean() > 0.9

    def codes(p):
        cc = np.empty(p.shape[:-1] + (2 * p.shape[-1],), np.int32)
        cc[..., 0::2], cc[..., 1::2] = p & 0xF, p >> 4
        return np.where(cc & 8, -(cc & 7), cc & 7).reshape(T, H_I, nb, 32)
    diff = np.abs(codes(got_c) - codes(ref["qi"]))
    assert np.all(diff[same] <= 1), "codes differ by more than one E2M1 step"
    check_close(wi[0].cpu().numpy(), ref["wi"], "w^I", atol=1e-4, rtol=1e-3)
    check_close(O.bf16_bits_to_f64(host_bits(q[0])), O.bf16_bits_to_f64(ref["q"]), "q")


def test_fp4_query_layer_prefill_then_decode():
    """Tiny CSA layer, FP4 query and keys (the compressor writes the MXFP4 keys), BF16 scores:
    prefill of 2048 tokens, then the 16 decode steps; selection and attention stage-wise on the
    GPU's stored keys and rows."""
    w = S.WORKLOADS["tiny_csa"]
    T = 2048
    say("fp4 x fp4 layer, bf16 scores", T)
    x = S.layer_inputs(w, T=T, qi_fmt="mxfp4")
    TT = x["T_total"]
    d = {k: dev(x[k]) for k in x if isinstance(x[k], np.ndarray)}
    cfg = config_for(w, d["inv_freq"], idx_key_format=csa.IDX_MXFP4,
                     idx_query_format=csa.IDX_MXFP4, score_format=csa.SCORE_BF16)
    n_max = TT // w.m + 1
    slots = 1 << (TT - 1).bit_length()
    tr, tc = csa.tail_shape(cfg)
    ct = dict(entries=torch.zeros((1, n_max, w.c), dtype=torch.int16, device=DEV),
              window=torch.zeros((1, slots, w.c), dtype=torch.int16, device=DEV),
              n_entries=torch.zeros(1, dtype=torch.int32, device=DEV),
              tail=torch.zeros((1, tr, tc), dtype=torch.float32, device=DEV),
              idx_keys=torch.zeros((1, n_max, w.d_I // 2), dtype=torch.uint8, device=DEV),
              idx_scale=torch.zeros((1, n_max, 4), dtype=torch.uint8, device=DEV))
    weights = csa.make_weights(d["W"], d["Ba"], d["gamma"], d["gamma_win"], bias_b=d["Bb"],
                               bias_ia=d["BIa"], bias_ib=d["BIb"])
    cache = csa.make_cache(n_max, slots, **ct)
    ws = workspace(max(csa.workspace_size(cfg, csa.OP_PREFILL, 1, T, n_max),
                       csa.workspace_size(cfg, csa.OP_DECODE, 1, 1, n_max)))
    out = torch.empty((1, TT, w.n_h, w.c), dtype=torch.bfloat16, device=DEV)
    idx = torch.full((1, TT, w.k), -7, dtype=torch.int32, device=DEV)
    csa.prefill(cfg, d["H"][:, :T].contiguous(), weights, cache, d["q"][:, :T].contiguous(),
                d["sink"], out[:, :T], ws, qi=d["qi"][:, :T].contiguous(),
                qi_scale=d["qi_scale"][:, :T].contiguous(), wi=d["wi"][:, :T].contiguous(),
                idx_out=idx[:, :T])
    pos = torch.zeros(1, dtype=torch.int32, device=DEV)
    for t in range(T, TT):
        pos.fill_(t)
        csa.decode(cfg, cache, pos, d["q"][:, t].contiguous(), d["sink"], out[:, t], ws,
                   h_new=d["H"][:, t].contiguous(), weights=weights, qi=d["qi"][:, t].contiguous(),
                   qi_scale=d["qi_scale"][:, t].contiguous(), wi=d["wi"][:, t].contiguous(),
                   idx_out=idx[:, t])
    torch.cuda.synchronize()
    n_ent = TT // w.m
    nb = w.d_I // 32
    keys = ct["idx_keys"][0].cpu().numpy()[:n_ent]
    scl = ct["idx_scale"][0].cpu().numpy()[:n_ent, :nb]
    ent = host_bits(ct["entries"][0])
    win = host_bits(ct["window"][0])
    rng = np.random.default_rng(0)
    qs = sorted(set([0, 3, 4, 5, 127, 128, 129, T - 1] + list(range(T, TT)) +
                    list(rng.integers(0, T, 24))))
    out_h = bf16_f64(out.view(torch.int16)[0])
    idx_h = idx[0].cpu().numpy()
    for t in qs:
        n_vis = O.visible_entries(t, w.m, n_ent)
        sc = O.index_scores_fp4(x["qi"][0, t], x["qi_scale"][0, t][:, :nb], x["wi"][0, t], keys,
                                scl, n_vis)
        check_selection_bf16(idx_h[t], sc, w.k, "query %d selection" % t)
        sel = idx_h[t][:min(w.k, n_vis)]
        rows = np.concatenate([ent[sel], win[O.window_tokens(t, w.n_win) % slots]])
        ref, _ = O.attend(x["q"][0, t], rows, x["sink"], w.scale, t, x["inv_freq"])
        check_close(out_h[t], ref, "query %d output" % t)
