"""GPU checks of chunked prefill (csa_prefill with per-sequence start positions pos0): a prompt
entered in chunks leaves the same cache (entries, indexer keys and scales, window rows, tail,
entry counts) and gives the same selections and outputs, bit for bit, as one call over the whole
prompt when every chunk has 16 or more tokens; chunk boundaries fall inside compression blocks
(the compressor's tail ring carries the open block) and the window ring carries the last
n_win - 1 rows across them.  Shorter chunks (decode-sized runs of queries take the decode span
plan) and a batch whose sequences sit at different positions are checked against the oracle,
stage-wise on the GPU's stored state; chunks written into the block cache layout leave the bits
of one contiguous call."""
import dataclasses

import numpy as np
import pytest
import torch

import long_context_sparse_15_amd as csa
import oracle as O
from synth import inputs as S
from gpu_common import (DEV, bf16_f64, check_close, check_selection, config_for, dev, host_bits,
                        say, workspace)
from test_gpu_layer import _build

pytestmark = pytest.mark.gpu


def _wide():
    # the production head shape: head dim 512, 64 heads, indexer 64 x 128 (the two-query
    # head-block attention and the many-row scorer)
    return dataclasses.replace(S.WORKLOADS["tiny_csa"], name="tiny_csa_wide", c=512, n_h=64,
                               H_I=64, d_I=128, T=1024)


def _workload(name):
    return _wide() if name == "wide" else S.WORKLOADS[name]


def _prefill(w, x, cfg, cache, weights, d, ws, out, idx, t0, T, pos0=None):
    """csa_prefill over tokens t0..t0+T-1 of every sequence into out/idx[:, t0:t0+T]."""
    kw = {}
    if w.mode == "csa":
        kw = dict(qi=d["qi"][:, t0:t0 + T].contiguous(),
                  qi_scale=d["qi_scale"][:, t0:t0 + T].contiguous(),
                  wi=d["wi"][:, t0:t0 + T].contiguous())
    o = torch.empty((w.B, T, w.n_h, w.c), dtype=torch.bfloat16, device=DEV)
    ix = torch.full((w.B, T, max(w.k, 1)), -7, dtype=torch.int32, device=DEV)
    if w.mode == "csa":
        kw["idx_out"] = ix
    csa.prefill(cfg, d["H"][:, t0:t0 + T].contiguous(), weights, cache,
                d["q"][:, t0:t0 + T].contiguous(), d["sink"], o, ws, pos0=pos0, **kw)
    out[:, t0:t0 + T] = o
    idx[:, t0:t0 + T] = ix


def _check_oracle(w, x, ct, out, idx, slots, n_ent, b, ts, what):
    """Selections and outputs of sequence b's queries ts against the oracle on the GPU's stored
    entries, keys and window rows (x holds sequence b's inputs at index b)."""
    ent = host_bits(ct["entries"][b])
    win = host_bits(ct["window"][b])
    out_h = bf16_f64(out.view(torch.int16)[b])
    idx_h = idx[b].cpu().numpy()
    if w.mode == "csa":
        keys = ct["idx_keys"][b].cpu().numpy()
        ksc = ct["idx_scale"][b].cpu().numpy()
    for t in ts:
        n_vis = O.visible_entries(t, w.m, n_ent)
        if w.mode == "csa":
            sc = O.index_scores(x["qi"][b, t], x["qi_scale"][b, t], x["wi"][b, t], keys, ksc,
                                n_vis)
            check_selection(idx_h[t], sc, w.k, "%s query %d selection" % (what, t))
            sel = idx_h[t][:min(w.k, n_vis)]
        else:
            sel = np.arange(n_vis)
        rows = np.concatenate([ent[sel], win[O.window_tokens(t, w.n_win) % slots]])
        ref, _ = O.attend(x["q"][b, t], rows, x["sink"], w.scale, t, x["inv_freq"])
        check_close(out_h[t], ref, "%s query %d output" % (what, t))


@pytest.mark.parametrize("name,T,chunks,n_max", [
    ("tiny_csa", 2048, [700, 1000, 348], None),
    ("tiny_csa", 2046, [16, 17, 1013, 1000], None),
    ("tiny_hca", 2040, [1000, 1040], None),
    ("wide", 1024, [333, 500, 191], None),
    # a cache of more than 32768 entries, as the chunks of a long prompt see: the selection
    # takes the multi-workgroup path
    ("wide", 1024, [333, 500, 191], 40000),
])
def test_chunked_prefill_equals_one_call(name, T, chunks, n_max):
    assert sum(chunks) == T and min(chunks) >= 16
    w = _workload(name)
    say("chunked prefill", name, T, chunks, n_max)
    x = S.layer_inputs(w, T=T)
    # one cache filled by a single call, one by the chunks (same ring size: row u in slot
    # u % slots)
    cfg, cache1, ct1, weights, d, n_max, slots = _build(w, x, x["T_total"], n_max)
    _, cache2, ct2, _, _, _, _ = _build(w, x, x["T_total"], n_max)
    assert slots >= max(chunks) + w.n_win - 1
    ws = workspace(csa.workspace_size(cfg, csa.OP_PREFILL, w.B, T, n_max))
    shape = (w.B, T, w.n_h, w.c)
    out1 = torch.empty(shape, dtype=torch.bfloat16, device=DEV)
    out2 = torch.empty(shape, dtype=torch.bfloat16, device=DEV)
    idx1 = torch.full((w.B, T, max(w.k, 1)), -7, dtype=torch.int32, device=DEV)
    idx2 = idx1.clone()
    _prefill(w, x, cfg, cache1, weights, d, ws, out1, idx1, 0, T)
    t0 = 0
    for n in chunks:
        pos0 = torch.full((w.B,), t0, dtype=torch.int32, device=DEV)
        _prefill(w, x, cfg, cache2, weights, d, ws, out2, idx2, t0, n, pos0=pos0)
        t0 += n
    torch.cuda.synchronize()
    n_ent = T // w.m
    assert int(ct2["n_entries"][0]) == n_ent
    for k in ct1:
        if k == "window":  # rows of tokens 0..T-1 (the rest of the ring is never written)
            assert torch.equal(ct1[k][:, :T], ct2[k][:, :T]), k
        else:
            assert torch.equal(ct1[k], ct2[k]), k
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))
    if w.mode == "csa":
        assert torch.equal(idx1, idx2)
    # the chunked run against the oracle around the chunk boundaries
    ts, t0 = [0, T - 1], 0
    for n in chunks[:-1]:
        t0 += n
        ts += [t0 - 1, t0, t0 + 1]
    _check_oracle(w, x, ct2, out2, idx2, slots, n_ent, 0, sorted(set(ts)), name)


def test_chunked_prefill_short_chunks_and_ragged_positions():
    """Chunks of 1, 3 and 9 tokens (decode-sized runs of queries) and a batch of two sequences
    at different positions in one call: sequence 0 continues its prompt while sequence 1 starts
    a new one from position 0 over its old cache rows.  Checked against the oracle."""
    w = S.shrink(S.WORKLOADS["tiny_csa"], B=2)
    say("chunked prefill, short chunks and ragged positions")
    x = S.layer_inputs(w, T=700)
    cfg, cache, ct, weights, d, n_max, slots = _build(w, x, x["T_total"])
    ws = workspace(max(csa.workspace_size(cfg, csa.OP_PREFILL, 2, n, n_max)
                       for n in (1, 3, 9, 174, 500)))
    out = torch.empty((2, 700, w.n_h, w.c), dtype=torch.bfloat16, device=DEV)
    idx = torch.full((2, 700, w.k), -7, dtype=torch.int32, device=DEV)
    # both sequences: tokens 0..186 in chunks 1, 3, 9, 174
    t0 = 0
    for n in (1, 3, 9, 174):
        pos0 = torch.full((2,), t0, dtype=torch.int32, device=DEV)
        _prefill(w, x, cfg, cache, weights, d, ws, out, idx, t0, n, pos0=pos0)
        t0 += n
    torch.cuda.synchronize()
    for b in range(2):
        _check_oracle(w, x, ct, out, idx, slots, 187 // w.m, b, [0, 1, 3, 4, 12, 13, 100, 186],
                      "seq %d" % b)
    # sequence 0 continues at 187 with its tokens 187..686; sequence 1 restarts at 0 with new
    # tokens (its tokens 187..686 of the inputs, as a fresh prompt)
    ct["n_entries"][1] = 0
    pos0 = torch.tensor([187, 0], dtype=torch.int32, device=DEV)
    o = torch.empty((2, 500, w.n_h, w.c), dtype=torch.bfloat16, device=DEV)
    ix = torch.full((2, 500, w.k), -7, dtype=torch.int32, device=DEV)
    sl = slice(187, 687)
    csa.prefill(cfg, d["H"][:, sl].contiguous(), weights, cache, d["q"][:, sl].contiguous(),
                d["sink"], o, ws, qi=d["qi"][:, sl].contiguous(),
                qi_scale=d["qi_scale"][:, sl].contiguous(), wi=d["wi"][:, sl].contiguous(),
                idx_out=ix, pos0=pos0)
    torch.cuda.synchronize()
    assert int(ct["n_entries"][0]) == 687 // w.m and int(ct["n_entries"][1]) == 500 // w.m
    # sequence 0: positions 187..686 of its own prompt
    out0 = torch.zeros((1, 700, w.n_h, w.c), dtype=torch.bfloat16, device=DEV)
    idx0 = torch.full((1, 700, w.k), -7, dtype=torch.int32, device=DEV)
    out0[:, sl] = o[:1]
    idx0[:, sl] = ix[:1]
    _check_oracle(w, x, {k: v[:1] for k, v in ct.items()}, out0, idx0, slots, 687 // w.m, 0,
                  [187, 188, 190, 191, 400, 686], "seq 0 continued")
    # sequence 1: a fresh prompt made of the inputs' tokens 187..686 at positions 0..499
    x1 = {k: (v[1:2, sl] if k in ("H", "q", "qi", "qi_scale", "wi") else v)
          for k, v in x.items()}
    _check_oracle(w, x1, {k: v[1:2] for k, v in ct.items()}, o[1:2], ix[1:2], slots,
                  500 // w.m, 0, [0, 1, 2, 3, 127, 128, 129, 499], "seq 1 restarted")
    # its entries against the oracle's compressor over the new prompt
    params = {k: x[k] for k in ("Ba", "Bb", "BIa", "BIb", "gamma", "gamma_win")}
    comp = O.compress_tokens(x["H"][1, sl], x["W"], params, w.mode, w.m, w.c, w.d_I,
                             x["inv_freq"], 1e-6)
    ent = host_bits(ct["entries"][1])[:500 // w.m]
    check_close(O.bf16_bits_to_f64(ent), O.bf16_bits_to_f64(comp["entries"]), "seq 1 entries")


@pytest.mark.parametrize("name,T,chunks", [
    ("tiny_csa", 2048, [700, 1000, 348]),
    ("tiny_hca", 2040, [1000, 1040]),
    ("wide", 1024, [333, 500, 191]),
])
def test_chunked_prefill_on_block_cache_equals_one_call(name, T, chunks):
    """Chunked prefill on the block cache layout (entries, keys and scales in randomly placed
    pool blocks) leaves the bits of one contiguous call: entries and keys read back through the
    block table, window rows, selections and outputs."""
    from test_gpu_paged import _block_entries, _from_pool, _layer_cache, _perm_table, _weights
    w = _workload(name)
    say("chunked prefill, block cache", name, T, chunks)
    x = S.layer_inputs(w, T=T)
    d = {k: dev(x[k]) for k in x if isinstance(x[k], np.ndarray)}
    cfg = config_for(w, d["inv_freq"])
    be = _block_entries(w)
    bps = (x["T_total"] // w.m + 1 + be - 1) // be
    n_max = bps * be
    slots = 1 << (x["T_total"] - 1).bit_length()
    assert slots >= max(chunks) + w.n_win - 1
    table, n_blocks = _perm_table(1, bps, 3, seed=T + 7)
    weights = _weights(w, d)
    cache_c, ct_c = _layer_cache(w, cfg, n_max, slots, False)
    cache_p, ct_p = _layer_cache(w, cfg, n_max, slots, False, table, n_blocks)
    ws = workspace(csa.workspace_size(cfg, csa.OP_PREFILL, 1, T, n_max))
    shape = (1, T, w.n_h, w.c)
    out1 = torch.empty(shape, dtype=torch.bfloat16, device=DEV)
    out2 = torch.empty(shape, dtype=torch.bfloat16, device=DEV)
    idx1 = torch.full((1, T, max(w.k, 1)), -7, dtype=torch.int32, device=DEV)
    idx2 = idx1.clone()
    _prefill(w, x, cfg, cache_c, weights, d, ws, out1, idx1, 0, T)
    t0 = 0
    for n in chunks:
        pos0 = torch.full((1,), t0, dtype=torch.int32, device=DEV)
        _prefill(w, x, cfg, cache_p, weights, d, ws, out2, idx2, t0, n, pos0=pos0)
        t0 += n
    torch.cuda.synchronize()
    n_ent = T // w.m
    assert int(ct_p["n_entries"][0]) == n_ent
    assert torch.equal(_from_pool(ct_p["entries"], table, be)[0, :n_ent],
                       ct_c["entries"][0, :n_ent]), "entries differ"
    assert torch.equal(ct_p["window"][:, :T], ct_c["window"][:, :T]), "window rows differ"
    if w.mode == "csa":
        assert torch.equal(_from_pool(ct_p["idx_keys"], table, be)[0, :n_ent],
                           ct_c["idx_keys"][0, :n_ent]), "indexer keys differ"
        assert torch.equal(_from_pool(ct_p["idx_scale"], table, be)[0, :n_ent].view(torch.int32),
                           ct_c["idx_scale"][0, :n_ent].view(torch.int32)), "key scales differ"
        assert torch.equal(idx1, idx2), "selections differ"
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16)), "outputs differ"
