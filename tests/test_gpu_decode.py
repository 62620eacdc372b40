"""GPU parity of the decode path (csa_index_topk, csa_sparse_mqa, hca_dense_mqa, csa_decode)
against the CPU oracle on seeded inputs: several tiles, ragged tails, n_vis < k, no visible
entry, exact ties and massive ties."""
import numpy as np
import pytest
import torch

import long_context_sparse_15_amd as csa
import oracle as O
from synth import inputs as S
from gpu_common import (DEV, bf16_f64, check_close, check_selection, config_for, dev, say,
                        window_rows_ring, workspace)

pytestmark = pytest.mark.gpu


def _setup(w, x, ring=None):
    B, N = x["B"], x["N"]
    d = {k: dev(x[k]) for k in ("entries", "window", "pos", "n_entries", "q", "sink",
                                 "inv_freq")}
    if w.mode == "csa":
        for k in ("ikeys", "iscale", "qi", "qi_scale", "wi"):
            d[k] = dev(x[k])
    cfg = config_for(w, d["inv_freq"])
    cache = csa.make_cache(N, x["window"].shape[1], d["entries"], d["window"], d["n_entries"],
                           idx_keys=d.get("ikeys"), idx_scale=d.get("iscale"))
    return cfg, cache, d


def _oracle_row(w, x, b, t, sel=None):
    """Oracle attention of sequence b's decode query at position t over sel (CSA) or all
    visible entries (HCA), plus the ring window."""
    slots = x["window"].shape[1]
    win = window_rows_ring(x["window"][b], t, w.n_win, slots)
    if sel is None:
        n_vis = O.visible_entries(t, w.m, x["n_entries"][b])
        rows = np.concatenate([x["entries"][b][:n_vis], win])
    else:
        rows = np.concatenate([x["entries"][b][sel], win])
    return O.attend(x["q"][b, 0], rows, x["sink"], w.scale, t, x["inv_freq"])


def run_csa_case(w, x, exact_ties=False, score_atol_mult=1.0):
    B, N = x["B"], x["N"]
    cfg, cache, d = _setup(w, x)
    idx = torch.empty((B, 1, w.k), dtype=torch.int32, device=DEV)
    sc = torch.empty((B, 1, w.k), dtype=torch.float32, device=DEV)
    ws = workspace(csa.workspace_size(cfg, csa.OP_DECODE, B, 1, N))
    csa.index_topk(cfg, d["qi"], d["qi_scale"], d["wi"], cache, d["pos"], idx, ws, score_out=sc)
    out = torch.empty((B, 1, w.n_h, w.c), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, 1, w.n_h), dtype=torch.float32, device=DEV)
    csa.sparse_mqa(cfg, d["q"], cache, idx, d["pos"], d["sink"], out, ws, lse_out=lse)
    out2 = torch.empty_like(out)
    idx2 = torch.empty((B, w.k), dtype=torch.int32, device=DEV)
    csa.decode(cfg, cache, d["pos"], d["q"][:, 0].contiguous(), d["sink"], out2, ws,
               qi=d["qi"], qi_scale=d["qi_scale"], wi=d["wi"], idx_out=idx2)
    torch.cuda.synchronize()
    idx_h, sc_h = idx.cpu().numpy(), sc.cpu().numpy()
    out_h = bf16_f64(out.view(torch.int16))
    lse_h = lse.cpu().numpy()
    assert np.array_equal(idx2.cpu().numpy(), idx_h[:, 0]), "fused decode selection differs"
    assert torch.equal(out2.view(torch.int16), out.view(torch.int16)), "fused decode output differs"
    for b in range(B):
        t = int(x["pos"][b])
        n_vis = O.visible_entries(t, w.m, x["n_entries"][b])
        ref_scores = O.index_scores(x["qi"][b, 0], x["qi_scale"][b, 0], x["wi"][b, 0],
                                    x["ikeys"][b], x["iscale"][b], n_vis)
        check_selection(idx_h[b, 0], ref_scores, w.k, "seq %d selection" % b)
        kk = min(w.k, n_vis)
        sel = idx_h[b, 0, :kk]
        if exact_ties:
            assert np.array_equal(sel, O.topk_select(ref_scores, w.k)), "tie order"
        check_close(sc_h[b, 0, :kk], ref_scores[sel], "seq %d scores" % b,
                    atol=1e-5 * score_atol_mult * max(1.0, np.abs(ref_scores).max(initial=0.0)),
                    rtol=1e-5)
        assert np.all(np.isneginf(sc_h[b, 0, kk:]))
        ref, ref_lse = _oracle_row(w, x, b, t, sel=sel)
        check_close(out_h[b, 0], ref, "seq %d output" % b)
        check_close(lse_h[b, 0], ref_lse, "seq %d lse" % b, atol=2e-3, rtol=1e-4)


def _w(name, **kw):
    return S.shrink(S.WORKLOADS[name], **kw)


@pytest.mark.parametrize("case", [
    # (workload, B, N, positions): several chunks and a ragged tail; n_vis < k; no entry visible
    ("csa_decode_128k", 3, 5000, [4 * 5000 + 3, 4 * 3000 + 1, 10]),
    ("csa_decode_128k", 2, 2177, [4 * 2177, 4 * 700 + 2]),
    ("csa_decode_1m", 2, 9000, [4 * 9000 + 7, 4 * 4500]),
    ("tiny_csa", 2, 700, [2063, 2]),
    ("tiny_csa", 1, 64, [300]),
    # one 1024-thread workgroup per row with every key in LDS (16K < n_vis <= 32K)
    ("csa_decode_128k", 2, 20000, [4 * 20000, 4 * 17000 + 3]),
    # multi-workgroup select (n_vis > 32K): the scorer's per-chunk thresholds and regions, finalize
    ("csa_decode_1m", 2, 40000, [4 * 40000 + 1, 4 * 33000]),
    # the same cache with rows of n_vis <= k (no regions written: everything selected), k + 1
    # and one visible entry past a chunk boundary
    ("csa_decode_1m", 4, 40000, [4 * 1500 + 3, 4 * 2049, 4 * 2048 * 3 + 4, 4 * 40000]),
])
def test_csa_decode_parity(case):
    name, B, N, positions = case
    say("csa decode", case)
    w = _w(name)
    x = S.decode_cache_inputs(w, B=B, N=N)
    x["pos"] = np.array(positions, dtype=np.int32)
    run_csa_case(w, x)


def test_csa_decode_exact_ties_lower_index_wins():
    say("csa decode exact ties")
    w = _w("tiny_csa")
    x = S.decode_cache_inputs(w, B=2, N=900)
    # blocks of identical keys -> exactly equal scores on both sides
    x["ikeys"][:, 100:900] = x["ikeys"][:, 100:101]
    x["iscale"][:, 100:900] = x["iscale"][:, 100:101]
    x["pos"] = np.array([4 * 900, 4 * 500], dtype=np.int32)
    run_csa_case(w, x, exact_ties=True)


def test_csa_decode_massive_ties_exact_fallback():
    say("csa decode massive ties (candidate overflow)")
    w = _w("tiny_csa")
    x = S.decode_cache_inputs(w, B=1, N=6000)
    x["ikeys"][:] = x["ikeys"][:, :1]
    x["iscale"][:] = x["iscale"][:, :1]
    x["pos"] = np.array([4 * 6000], dtype=np.int32)
    run_csa_case(w, x, exact_ties=True)


def test_csa_decode_massive_ties_multi_workgroup_fallback():
    say("csa decode massive ties, multi-workgroup select")
    w = _w("csa_decode_128k")
    x = S.decode_cache_inputs(w, B=1, N=40000)
    x["ikeys"][:, 5000:] = x["ikeys"][:, 5000:5001]
    x["iscale"][:, 5000:] = x["iscale"][:, 5000:5001]
    x["pos"] = np.array([4 * 40000], dtype=np.int32)
    run_csa_case(w, x, exact_ties=True)


def test_csa_decode_clustered_top_keys_multi_workgroup_fallback():
    """The top keys of a long row all sit in its first 4096 entries (two of the decode scorer's
    2048-entry chunks, whose candidates it collects itself): those chunks' own thresholds cut
    keys above the k-th key; the finalize sees it and reads the chunks again for every key at or
    above the list's k-th key."""
    say("csa decode clustered top keys, multi-workgroup select")
    w = _w("csa_decode_1m")
    x = S.decode_cache_inputs(w, B=1, N=40000)
    x["iscale"][:, :4096] *= 16.0
    x["pos"] = np.array([4 * 40000], dtype=np.int32)
    # the fp32 sums' rounding scales with their 16x larger terms
    run_csa_case(w, x, score_atol_mult=16.0)


@pytest.mark.parametrize("chunks", [(1, 4, 9), (9,)])
def test_csa_decode_top_keys_in_several_chunks(chunks):
    """The top keys of two long rows sit in a few 4096-entry spans (each two of the decode
    scorer's 2048-entry chunks; the last one partial, as the newest entries of a prompt would):
    each such chunk's threshold cuts keys above the k-th key, and the finalize re-reads exactly
    those chunks; the second row's top keys are spread evenly (no chunk re-read)."""
    say("csa decode top keys in chunks", chunks)
    w = _w("csa_decode_1m")
    x = S.decode_cache_inputs(w, B=2, N=40000)
    for c in chunks:
        x["iscale"][0, 4096 * c:4096 * (c + 1)] *= 16.0
    x["pos"] = np.array([4 * 40000, 4 * 39000 + 2], dtype=np.int32)
    run_csa_case(w, x, score_atol_mult=16.0)


@pytest.mark.parametrize("case", [
    ("hca_decode_1m", 3, 300, [128 * 300 + 5, 128 * 100 + 127, 60]),
    ("tiny_hca", 2, 40, [128 * 40, 127]),
    # lists longer than 4096 rows with 128 heads: the head-block kernel, sixteen spans; positions
    # that fill the list, leave a ragged last tile, leave most spans empty, and leave no entry
    ("hca_decode_1m", 4, 4500, [128 * 4500 + 5, 128 * 3001 + 77, 128 * 40, 1000]),
    # 96 heads: the last 32-head block of the workgroup is empty
    ("hca_decode_1m", 2, 4200, [128 * 4200 + 127, 128 * 2222], 96),
])
def test_hca_dense_parity(case):
    name, B, N, positions = case[:4]
    say("hca dense", case)
    w = _w(name, **({"n_h": case[4]} if len(case) > 4 else {}))
    x = S.decode_cache_inputs(w, B=B, N=N)
    x["pos"] = np.array(positions, dtype=np.int32)
    cfg, cache, d = _setup(w, x)
    ws = workspace(csa.workspace_size(cfg, csa.OP_DECODE, B, 1, N))
    out = torch.empty((B, 1, w.n_h, w.c), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, 1, w.n_h), dtype=torch.float32, device=DEV)
    csa.hca_dense_mqa(cfg, d["q"], cache, d["pos"], d["sink"], out, ws, lse_out=lse)
    out2 = torch.empty((B, w.n_h, w.c), dtype=torch.bfloat16, device=DEV)
    csa.decode(cfg, cache, d["pos"], d["q"][:, 0].contiguous(), d["sink"], out2, ws)
    torch.cuda.synchronize()
    assert torch.equal(out2.view(torch.int16), out[:, 0].view(torch.int16))
    out_h = bf16_f64(out.view(torch.int16))
    lse_h = lse.cpu().numpy()
    for b in range(B):
        t = int(x["pos"][b])
        ref, ref_lse = _oracle_row(w, x, b, t)
        check_close(out_h[b, 0], ref, "seq %d output" % b)
        check_close(lse_h[b, 0], ref_lse, "seq %d lse" % b, atol=2e-3, rtol=1e-4)
