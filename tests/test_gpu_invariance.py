"""Batch invariance of the decode path, and span partials at extreme entry magnitudes.

Batch-invariant decoding (Analysis "DeepSeek-V4 技术报告深度解读" §5.3; Book "DeepSeek V4 模型技术大
全", section "推理系统深拆", row "avoid split-KV"): a sequence's decode output must not depend on
which other sequences share the call or on its slot in the batch.  Each case decodes one
sequence of a full-size workload alone, inside a batch of 5 at another slot, and inside the
workload's own batch, and requires identical bits for the output and the selected indices.

The magnitude cases scale entries and window rows by 2^17 (beyond fp16's range) and by 2^-20
(below its normal range), and the query by the inverse power of two so that the logits stay
exactly those of the unscaled rows, and check both a one-span plan (a run of 16 queries per sequence) and
the split plan (one query per sequence, several spans merged by the combine kernel) against
the oracle, with the tolerance scaled by the magnitude, for 64 and 128 heads; and the same for
an HCA decode over a list longer than 4096 rows with 128 heads (the head-block kernel)."""
import numpy as np
import pytest
import torch

import long_context_sparse_15_amd as csa
import oracle as O
from synth import inputs as S
from synth import gpu as G
from gpu_common import DEV, check_close, config_for, dev, say, window_rows_ring, workspace

pytestmark = pytest.mark.gpu


def _decode_subset(w, x, seqs, cfg):
    """csa_decode over the sequences `seqs` of x (in that order, as a new batch)."""
    sl = torch.tensor(seqs, dtype=torch.long, device=DEV)
    y = {}
    for k in ("entries", "window", "pos", "n_entries", "ikeys", "iscale", "q", "qi", "qi_scale",
              "wi"):
        if k in x:
            y[k] = x[k].index_select(0, sl).contiguous()
    B = len(seqs)
    cache = csa.make_cache(w.N, w.n_win, y["entries"], y["window"], y["n_entries"],
                           idx_keys=y.get("ikeys"), idx_scale=y.get("iscale"))
    ws = workspace(csa.workspace_size(cfg, csa.OP_DECODE, B, 1, w.N))
    out = torch.empty((B, w.n_h, w.c), dtype=torch.bfloat16, device=DEV)
    q = y["q"][:, 0].contiguous()
    if w.mode == "csa":
        idx = torch.empty((B, w.k), dtype=torch.int32, device=DEV)
        csa.decode(cfg, cache, y["pos"], q, x["sink"], out, ws, qi=y["qi"],
                   qi_scale=y["qi_scale"], wi=y["wi"], idx_out=idx)
    else:
        idx = None
        csa.decode(cfg, cache, y["pos"], q, x["sink"], out, ws)
    torch.cuda.synchronize()
    return out.view(torch.int16).cpu(), (idx.cpu() if idx is not None else None)


@pytest.mark.parametrize("name,seq,others", [
    ("csa_decode_128k", 7, [3, 30, 12, 0]),
    ("csa_decode_1m", 2, [0, 1, 3, 3]),
    ("hca_decode_1m", 9, [15, 1, 4, 0]),
])
def test_decode_batch_invariant(name, seq, others):
    w = S.WORKLOADS[name]
    say("batch invariance", name, "sequence", seq)
    x = G.decode_cache_inputs(w, DEV)
    # a different position for every sequence, so the batch mixes rows of different lengths
    pos = x["pos"].clone()
    n_ent = x["n_entries"].clone()
    step = w.m * 37
    for b in range(w.B):
        pos[b] = w.t - step * b
        n_ent[b] = min(w.N, (int(pos[b]) + 1) // w.m)
    x["pos"], x["n_entries"] = pos, n_ent
    cfg = csa.make_config(csa.MODE_CSA if w.mode == "csa" else csa.MODE_HCA, w.m, w.n_h, w.c,
                          w.r, x["inv_freq"], top_k=w.k, n_win=w.n_win, idx_heads=w.H_I,
                          idx_dim=w.d_I, softmax_scale=w.scale)
    full_out, full_idx = _decode_subset(w, x, list(range(w.B)), cfg)
    alone_out, alone_idx = _decode_subset(w, x, [seq], cfg)
    five = others[:2] + [seq] + others[2:]
    five_out, five_idx = _decode_subset(w, x, five, cfg)
    for label, o, i, slot in (("alone", alone_out, alone_idx, 0), ("batch of 5", five_out,
                                                                  five_idx, 2)):
        assert torch.equal(o[slot], full_out[seq]), "%s: output bits differ %s" % (name, label)
        if i is not None:
            assert torch.equal(i[slot], full_idx[seq]), "%s: selection differs %s" % (name, label)


def _scaled_bits(bits, e):
    """bf16 bit patterns times 2^e (exact: only the exponent changes)."""
    return O.f64_to_bf16_bits(O.bf16_bits_to_f64(bits) * 2.0 ** e)


@pytest.mark.parametrize("e,n_h", [(17, 64), (-20, 64), (17, 128), (-20, 128)])
def test_span_partials_extreme_magnitudes(e, n_h):
    w = S.shrink(S.WORKLOADS["csa_decode_128k"], n_h=n_h)
    B, N = 16, 3000
    say("span partials at magnitude 2^%d, %d heads" % (e, n_h))
    x = S.decode_cache_inputs(w, B=B, N=N)
    x["pos"] = (4 * N - 37 * np.arange(B)).astype(np.int32)
    x["entries"] = _scaled_bits(x["entries"], e)
    x["window"] = _scaled_bits(x["window"], e)
    # the query takes the inverse power of two: logits (and so the softmax weights) are exactly
    # those of the unscaled rows, only the values the partials carry change magnitude
    x["q"] = _scaled_bits(x["q"], -e)
    d = {k: dev(x[k]) for k in ("entries", "window", "pos", "n_entries", "q", "sink", "inv_freq",
                                 "ikeys", "iscale", "qi", "qi_scale", "wi")}
    cfg = config_for(w, d["inv_freq"])
    cache = csa.make_cache(N, w.n_win, d["entries"], d["window"], d["n_entries"],
                           idx_keys=d["ikeys"], idx_scale=d["iscale"])
    ws = workspace(csa.workspace_size(cfg, csa.OP_DECODE, B, 16, N))
    idx = torch.empty((B, 1, w.k), dtype=torch.int32, device=DEV)
    csa.index_topk(cfg, d["qi"], d["qi_scale"], d["wi"], cache, d["pos"], idx, ws)
    # split plan: one query per sequence, several spans merged by the combine kernel
    out_split = torch.empty((B, 1, w.n_h, w.c), dtype=torch.bfloat16, device=DEV)
    csa.sparse_mqa(cfg, d["q"], cache, idx, d["pos"], d["sink"], out_split, ws)
    # one-span plan: the same 16 queries as one sequence's run of 16 (nq = 16), over a cache
    # of that sequence's rows repeated: row j of the run is sequence j's query
    one = {}
    for k in ("entries", "window"):
        one[k] = d[k][:1].contiguous()
    out_one = torch.empty((1, B, w.n_h, w.c), dtype=torch.bfloat16, device=DEV)
    q16 = d["q"][:, 0].reshape(1, B, w.n_h, w.c).contiguous()
    idx16 = idx[:, 0].reshape(1, B, w.k).contiguous()
    pos16 = d["pos"].reshape(1, B).contiguous()
    n1 = d["n_entries"][:1].contiguous()
    cache1 = csa.make_cache(N, w.n_win, one["entries"], one["window"], n1)
    ws1 = workspace(csa.workspace_size(cfg, csa.OP_SPARSE_MQA, 1, B, N))
    csa.sparse_mqa(cfg, q16, cache1, idx16, pos16, d["sink"], out_one, ws1)
    torch.cuda.synchronize()
    idx_h = idx.cpu().numpy()
    got_split = O.bf16_bits_to_f64(out_split.view(torch.int16).cpu().numpy().view(np.uint16))
    got_one = O.bf16_bits_to_f64(out_one.view(torch.int16).cpu().numpy().view(np.uint16))
    mag = 2.0 ** e
    for b in range(B):
        t = int(x["pos"][b])
        n_vis = O.visible_entries(t, w.m, N)
        sel = idx_h[b, 0, :min(w.k, n_vis)]
        win = window_rows_ring(x["window"][b], t, w.n_win, w.n_win)
        ref, _ = O.attend(x["q"][b, 0], np.concatenate([x["entries"][b][sel], win]), x["sink"],
                          w.scale, t, x["inv_freq"])
        check_close(got_split[b, 0], ref, "2^%d split, seq %d" % (e, b), atol=1e-2 * mag)
        # the one-span run reads sequence 0's rows for every query
        win0 = window_rows_ring(x["window"][0], t, w.n_win, w.n_win)
        ref0, _ = O.attend(x["q"][b, 0], np.concatenate([x["entries"][0][sel], win0]),
                           x["sink"], w.scale, t, x["inv_freq"])
        check_close(got_one[0, b], ref0, "2^%d one span, query %d" % (e, b), atol=1e-2 * mag)


@pytest.mark.parametrize("e", [17, -20])
def test_head_block_partials_extreme_magnitudes(e):
    w = S.shrink(S.WORKLOADS["hca_decode_1m"])
    B, N = 3, 4300
    say("head-block span partials at magnitude 2^%d" % e)
    x = S.decode_cache_inputs(w, B=B, N=N)
    x["pos"] = np.array([128 * N + 3, 128 * 2500 + 9, 128 * 4100], dtype=np.int32)
    x["entries"] = _scaled_bits(x["entries"], e)
    x["window"] = _scaled_bits(x["window"], e)
    x["q"] = _scaled_bits(x["q"], -e)
    d = {k: dev(x[k]) for k in ("entries", "window", "pos", "n_entries", "q", "sink", "inv_freq")}
    cfg = config_for(w, d["inv_freq"])
    cache = csa.make_cache(N, w.n_win, d["entries"], d["window"], d["n_entries"])
    ws = workspace(csa.workspace_size(cfg, csa.OP_DECODE, B, 1, N))
    out = torch.empty((B, 1, w.n_h, w.c), dtype=torch.bfloat16, device=DEV)
    csa.hca_dense_mqa(cfg, d["q"], cache, d["pos"], d["sink"], out, ws)
    torch.cuda.synchronize()
    got = O.bf16_bits_to_f64(out.view(torch.int16).cpu().numpy().view(np.uint16))
    mag = 2.0 ** e
    for b in range(B):
        t = int(x["pos"][b])
        n_vis = O.visible_entries(t, w.m, N)
        win = window_rows_ring(x["window"][b], t, w.n_win, w.n_win)
        ref, _ = O.attend(x["q"][b, 0], np.concatenate([x["entries"][b][:n_vis], win]), x["sink"],
                          w.scale, t, x["inv_freq"])
        check_close(got[b, 0], ref, "2^%d seq %d" % (e, b), atol=1e-2 * mag)
