"""GPU parity of the block (paged) cache layout: compressed entries, indexer keys and key scales
in pools of fixed-size blocks addressed through a per-sequence block table (blocks of 128 tokens:
128/m entries, i.e. 32 for CSA and 1 for HCA), with the window ring and compressor tail as
per-sequence state.

* The same layer (prefill, then decode steps through the compressor) run on a contiguous cache
  and on a paged cache whose blocks are a random permutation of a larger pool gives identical
  bits: outputs, selected indices, and every entry, key and scale (read back through the table);
  the paged run is also checked stage-wise against the oracle.
* Full-size decodes (128K CSA with E4M3 and MXFP4 keys, 1M CSA, 1M HCA; bf16 and mixed-precision
  entries) on paged copies of the cache give the contiguous run's bits, with sequences of
  different lengths.
* Prefix reuse: a second sequence maps the first sequence's leading blocks, rebuilds its window
  and compressor tail by re-running the last 128 prefix tokens (no entry is written, the shared
  blocks keep their bits), then continues with tokens of its own; its entries match a
  from-scratch run of the same tokens bit for bit and its outputs match the oracle."""
import dataclasses

import numpy as np
import pytest
import torch

import long_context_sparse_15_amd as csa
import oracle as O
from synth import inputs as S
from synth import gpu as G
from gpu_common import (DEV, bf16_f64, check_close, check_selection, config_for, dev, host_bits,
                        say, workspace)

pytestmark = pytest.mark.gpu


def _block_entries(w):
    return 128 // w.m  # blocks of lcm(m, 128) = 128 tokens


def _perm_table(B, bps, extra, seed):
    """Each sequence's logical blocks mapped to distinct, randomly placed pool blocks; the pool
    holds `extra` blocks more than the table uses."""
    n_blocks = B * bps + extra
    perm = np.random.default_rng(seed).permutation(n_blocks)[:B * bps]
    return perm.reshape(B, bps).astype(np.int32), n_blocks


def _rows(table, be):
    t = torch.from_numpy(np.ascontiguousarray(table)).to(DEV).long()
    return (t[:, :, None] * be + torch.arange(be, device=DEV)[None, None, :]).reshape(
        table.shape[0], -1)


def _to_pool(x, table, n_blocks, be):
    """Contiguous [B, n_max, ...] -> pool [n_blocks * be, ...] through the table."""
    B, n_max = x.shape[0], x.shape[1]
    pool = torch.zeros((n_blocks * be,) + tuple(x.shape[2:]), dtype=x.dtype, device=DEV)
    pool[_rows(table, be).reshape(-1)] = x.reshape((B * n_max,) + tuple(x.shape[2:]))
    return pool


def _from_pool(pool, table, be):
    """Pool -> logical [B, blocks_per_seq * be, ...] through the table."""
    r = _rows(table, be)
    return pool[r.reshape(-1)].reshape(tuple(r.shape) + tuple(pool.shape[1:]))


def _wide(w):
    """The tiny CSA layer at the production head shape (64 heads x 512, indexer 64 x 128): the
    eight-wave attention kernel and the many-row indexer product run."""
    return dataclasses.replace(w, name="tiny_csa_wide", c=512, n_h=64, H_I=64, d_I=128, T=1024)


def _layer_cache(w, cfg, n_max, slots, mx, table=None, n_blocks=0):
    """Zeroed cache of one sequence: contiguous, or pools of n_blocks blocks with `table`."""
    be = _block_entries(w)
    lead = (n_blocks * be,) if table is not None else (1, n_max)
    tr, tc = csa.tail_shape(cfg)
    ct = dict(entries=torch.zeros(lead + (w.c,), dtype=torch.int16, device=DEV),
              window=torch.zeros((1, slots, w.c), dtype=torch.int16, device=DEV),
              n_entries=torch.zeros(1, dtype=torch.int32, device=DEV),
              tail=torch.zeros((1, tr, tc), dtype=torch.float32, device=DEV))
    if w.mode == "csa":
        ct["idx_keys"] = torch.zeros(lead + (w.d_I // 2 if mx else w.d_I,), dtype=torch.uint8,
                                     device=DEV)
        ct["idx_scale"] = torch.zeros(lead, dtype=torch.float32, device=DEV)
    kw = {}
    if table is not None:
        kw = dict(block_table=dev(table), block_entries=be, n_blocks=n_blocks)
    return csa.make_cache(n_max, slots, **ct, **kw), ct


def _weights(w, d):
    if w.mode == "csa":
        return csa.make_weights(d["W"], d["Ba"], d["gamma"], d["gamma_win"], bias_b=d["Bb"],
                                bias_ia=d["BIa"], bias_ib=d["BIb"])
    return csa.make_weights(d["W"], d["B"], d["gamma"], d["gamma_win"])


def _run_layer(w, x, d, cfg, cache, n_max):
    T, TT = x["T"], x["T_total"]
    csa_mode = w.mode == "csa"
    weights = _weights(w, d)
    ws = workspace(max(csa.workspace_size(cfg, csa.OP_PREFILL, 1, T, n_max),
                       csa.workspace_size(cfg, csa.OP_DECODE, 1, 1, n_max)))
    out = torch.empty((1, TT, w.n_h, w.c), dtype=torch.bfloat16, device=DEV)
    idx = torch.full((1, TT, max(w.k, 1)), -7, dtype=torch.int32, device=DEV)
    kw = {}
    if csa_mode:
        kw = dict(qi=d["qi"][:, :T].contiguous(), qi_scale=d["qi_scale"][:, :T].contiguous(),
                  wi=d["wi"][:, :T].contiguous(), idx_out=idx[:, :T])
    csa.prefill(cfg, d["H"][:, :T].contiguous(), weights, cache, d["q"][:, :T].contiguous(),
                d["sink"], out[:, :T], ws, **kw)
    pos = torch.zeros(1, dtype=torch.int32, device=DEV)
    for t in range(T, TT):
        pos.fill_(t)
        dk = {}
        if csa_mode:
            dk = dict(qi=d["qi"][:, t].contiguous(), qi_scale=d["qi_scale"][:, t].contiguous(),
                      wi=d["wi"][:, t].contiguous(), idx_out=idx[:, t])
        csa.decode(cfg, cache, pos, d["q"][:, t].contiguous(), d["sink"], out[:, t], ws,
                   h_new=d["H"][:, t].contiguous(), weights=weights, **dk)
    torch.cuda.synchronize()
    return out, idx


def _check_against_oracle(w, x, T, n_ent, ent, win, slots, keys, ksc, mx, out, idx, qs):
    """Stage-wise: each sampled query's selection against the oracle's scores on the stored keys,
    its output against the oracle's attention over the stored rows."""
    out_h = bf16_f64(out.view(torch.int16)[0])
    idx_h = idx[0].cpu().numpy()
    for t in qs:
        n_vis = O.visible_entries(t, w.m, n_ent)
        if w.mode == "csa":
            if mx:
                sc = O.index_scores_mxfp4(x["qi"][0, t], x["qi_scale"][0, t], x["wi"][0, t],
                                          keys, ksc, n_vis)
            else:
                sc = O.index_scores(x["qi"][0, t], x["qi_scale"][0, t], x["wi"][0, t], keys,
                                    ksc, n_vis)
            check_selection(idx_h[t], sc, w.k, "query %d selection" % t)
            sel = idx_h[t][:min(w.k, n_vis)]
        else:
            sel = np.arange(n_vis)
        rows = np.concatenate([ent[sel], win[O.window_tokens(t, w.n_win) % slots]])
        ref, _ = O.attend(x["q"][0, t], rows, x["sink"], w.scale, t, x["inv_freq"])
        check_close(out_h[t], ref, "query %d output" % t)


def _key_views(ct_keys, ct_scale, n_ent, w, mx):
    keys = ct_keys.cpu().numpy()[:n_ent]
    if mx:
        ksc = ct_scale.contiguous().view(torch.uint8).cpu().numpy().reshape(-1, 4)[:n_ent]
        return keys, ksc[:, :w.d_I // 32]
    return keys, ct_scale.cpu().numpy()[:n_ent]


@pytest.mark.parametrize("name,key_fmt,T", [("tiny_csa", "e4m3", 2046), ("tiny_csa", "mxfp4", 2048),
                                            ("tiny_hca", None, 2040), ("wide", "e4m3", 1024),
                                            ("wide", "mxfp4", 1022)])
def test_paged_layer_matches_contiguous(name, key_fmt, T):
    w = _wide(S.WORKLOADS["tiny_csa"]) if name == "wide" else S.WORKLOADS[name]
    say("paged layer", w.name, key_fmt, "T", T)
    mx = key_fmt == "mxfp4"
    x = S.layer_inputs(w, T=T)
    TT = x["T_total"]
    d = {k: dev(x[k]) for k in x if isinstance(x[k], np.ndarray)}
    cfg = config_for(w, d["inv_freq"],
                     **({"idx_key_format": csa.IDX_MXFP4} if mx else {}))
    be = _block_entries(w)
    bps = (TT // w.m + 1 + be - 1) // be
    n_max = bps * be
    slots = 1 << (TT - 1).bit_length()
    table, n_blocks = _perm_table(1, bps, 5, seed=T)

    cache_c, ct_c = _layer_cache(w, cfg, n_max, slots, mx)
    out_c, idx_c = _run_layer(w, x, d, cfg, cache_c, n_max)
    cache_p, ct_p = _layer_cache(w, cfg, n_max, slots, mx, table, n_blocks)
    out_p, idx_p = _run_layer(w, x, d, cfg, cache_p, n_max)

    n_ent = TT // w.m
    assert int(ct_p["n_entries"][0]) == n_ent
    assert torch.equal(out_p.view(torch.int16), out_c.view(torch.int16)), "outputs differ"
    if w.mode == "csa":
        assert torch.equal(idx_p, idx_c), "selections differ"
    ent_p = _from_pool(ct_p["entries"], table, be)[0]
    assert torch.equal(ent_p[:n_ent], ct_c["entries"][0, :n_ent]), "entries differ"
    assert torch.equal(ct_p["window"], ct_c["window"]), "window rows differ"
    keys = ksc = None
    if w.mode == "csa":
        kp = _from_pool(ct_p["idx_keys"], table, be)[0]
        sp = _from_pool(ct_p["idx_scale"], table, be)[0]
        assert torch.equal(kp[:n_ent], ct_c["idx_keys"][0, :n_ent]), "indexer keys differ"
        assert torch.equal(sp[:n_ent].view(torch.int32),
                           ct_c["idx_scale"][0, :n_ent].view(torch.int32)), "key scales differ"
        keys, ksc = _key_views(kp, sp, n_ent, w, mx)
    rng = np.random.default_rng(1)
    qs = sorted(set([0, 4, 127, 128, 129, T - 1] + list(range(T, TT)) +
                    list(rng.integers(0, T, 12))))
    _check_against_oracle(w, x, T, n_ent, host_bits(ent_p), host_bits(ct_p["window"][0]), slots,
                          keys, ksc, mx, out_p, idx_p, qs)


@pytest.mark.parametrize("name,key_fmt,B,ent", [("csa_decode_128k", "e4m3", 4, "bf16"),
                                                ("csa_decode_128k", "mxfp4", 4, "bf16"),
                                                ("csa_decode_1m", "e4m3", 1, "bf16"),
                                                ("csa_decode_1m", "mxfp4", 1, "bf16"),
                                                ("hca_decode_1m", None, 4, "bf16"),
                                                ("csa_decode_128k", "e4m3", 4, "mixed"),
                                                ("hca_decode_1m", None, 4, "mixed")])
def test_paged_decode_matches_contiguous(name, key_fmt, B, ent):
    w = dataclasses.replace(S.WORKLOADS[name], B=B)
    say("paged decode", name, key_fmt, ent, "B=%d N=%d" % (B, w.N))
    mx = key_fmt == "mxfp4"
    x = G.decode_cache_inputs(w, DEV, key_fmt=key_fmt or "e4m3", entry_fmt=ent)
    # sequences of different lengths, not multiples of the block size
    x["n_entries"] = torch.tensor([w.N - 37 * b - (5 if b else 0) for b in range(B)],
                                  dtype=torch.int32, device=DEV)
    csa_mode = w.mode == "csa"
    be = _block_entries(w)
    bps = w.N // be
    table, n_blocks = _perm_table(B, bps, 3, seed=B)
    cfg = csa.make_config(csa.MODE_CSA if csa_mode else csa.MODE_HCA, w.m, w.n_h, w.c, w.r,
                          x["inv_freq"], top_k=w.k, n_win=w.n_win, idx_heads=w.H_I,
                          idx_dim=w.d_I, softmax_scale=w.scale,
                          idx_key_format=csa.IDX_MXFP4 if mx else csa.IDX_E4M3,
                          entry_format=csa.ENT_MIXED if ent == "mixed" else csa.ENT_BF16)
    ws = workspace(csa.workspace_size(cfg, csa.OP_DECODE, B, 1, w.N))
    q = x["q"][:, 0].contiguous()

    def run(cache):
        out = torch.empty((B, w.n_h, w.c), dtype=torch.bfloat16, device=DEV)
        idx = torch.full((B, max(w.k, 1)), -7, dtype=torch.int32, device=DEV)
        if csa_mode:
            csa.decode(cfg, cache, x["pos"], q, x["sink"], out, ws, qi=x["qi"],
                       qi_scale=x["qi_scale"], wi=x["wi"], idx_out=idx)
        else:
            csa.decode(cfg, cache, x["pos"], q, x["sink"], out, ws)
        torch.cuda.synchronize()
        return out, idx

    cache_c = csa.make_cache(w.N, w.n_win, x["entries"], x["window"], x["n_entries"],
                             idx_keys=x.get("ikeys"), idx_scale=x.get("iscale"))
    out_c, idx_c = run(cache_c)
    pools = {"entries": _to_pool(x["entries"], table, n_blocks, be)}
    if csa_mode:
        pools["idx_keys"] = _to_pool(x["ikeys"], table, n_blocks, be)
        pools["idx_scale"] = _to_pool(x["iscale"], table, n_blocks, be)
    cache_p = csa.make_cache(w.N, w.n_win, pools["entries"], x["window"], x["n_entries"],
                             idx_keys=pools.get("idx_keys"), idx_scale=pools.get("idx_scale"),
                             block_table=dev(table), block_entries=be, n_blocks=n_blocks)
    out_p, idx_p = run(cache_p)
    assert torch.equal(out_p.view(torch.int16), out_c.view(torch.int16)), "outputs differ"
    if csa_mode:
        assert torch.equal(idx_p, idx_c), "selections differ"


@pytest.mark.parametrize("name", ["tiny_csa", "wide"])
def test_prefix_reuse_with_tail_recompute(name):
    w = _wide(S.WORKLOADS["tiny_csa"]) if name == "wide" else S.WORKLOADS[name]
    P, TA, TB = 512, 1024, 812  # shared prefix, first sequence, second sequence (P + 300 own)
    say("prefix reuse", w.name, "P", P, "A", TA, "B", TB)
    xa = S.layer_inputs(w, T=TA)
    xb = S.layer_inputs(w, seed=w.seed + 7, T=TB)
    # the second sequence's first P tokens are the first sequence's (hidden states and queries)
    for k in ("H", "q", "qi", "qi_scale", "wi"):
        xb[k][:, :P] = xa[k][:, :P]
    for k in ("W", "Ba", "Bb", "BIa", "BIb", "gamma", "gamma_win", "inv_freq", "sink"):
        xb[k] = xa[k]
    da = {k: dev(xa[k]) for k in xa if isinstance(xa[k], np.ndarray)}
    db = {k: dev(xb[k]) for k in xb if isinstance(xb[k], np.ndarray)}
    cfg = config_for(w, da["inv_freq"])
    be = _block_entries(w)
    bps = (TA // w.m + be - 1) // be + 1
    n_max = bps * be
    slots = 2048
    pb = P // w.m // be  # shared blocks
    n_blocks = 2 * bps + 3
    perm = np.random.default_rng(5).permutation(n_blocks).astype(np.int32)
    ta = perm[:bps].reshape(1, bps)
    tb = np.concatenate([ta[0, :pb], perm[bps:2 * bps - pb]]).reshape(1, bps).astype(np.int32)
    weights = _weights(w, da)
    ws = workspace(max(csa.workspace_size(cfg, csa.OP_PREFILL, 1, TB, n_max),
                       csa.workspace_size(cfg, csa.OP_PREFILL, 1, TA, n_max),
                       csa.workspace_size(cfg, csa.OP_COMPRESS, 1, TB - P, n_max),
                       csa.workspace_size(cfg, csa.OP_INDEX_TOPK, 1, TB - P, n_max),
                       csa.workspace_size(cfg, csa.OP_SPARSE_MQA, 1, TB - P, n_max)))

    # sequence A: prefill of TA tokens into the shared pools
    cache_a, ct_a = _layer_cache(w, cfg, n_max, slots, False, ta, n_blocks)
    out_a = torch.empty((1, TA, w.n_h, w.c), dtype=torch.bfloat16, device=DEV)
    csa.prefill(cfg, da["H"][:, :TA].contiguous(), weights, cache_a, da["q"][:, :TA].contiguous(),
                da["sink"], out_a, ws, qi=da["qi"][:, :TA].contiguous(),
                qi_scale=da["qi_scale"][:, :TA].contiguous(), wi=da["wi"][:, :TA].contiguous())
    torch.cuda.synchronize()
    shared_rows = _rows(ta[:, :pb], be).reshape(-1)
    before = [ct_a[k][shared_rows].clone() for k in ("entries", "idx_keys", "idx_scale")]

    # sequence B: same pools, its own table, window, tail and entry count
    tr, tc = csa.tail_shape(cfg)
    ct_b = dict(entries=ct_a["entries"], idx_keys=ct_a["idx_keys"], idx_scale=ct_a["idx_scale"],
                window=torch.zeros((1, slots, w.c), dtype=torch.int16, device=DEV),
                n_entries=torch.full((1,), P // w.m, dtype=torch.int32, device=DEV),
                tail=torch.zeros((1, tr, tc), dtype=torch.float32, device=DEV))
    cache_b = csa.make_cache(n_max, slots, **ct_b, block_table=dev(tb), block_entries=be,
                             n_blocks=n_blocks)
    R = 128  # max(n_win, 2m): the window and the overlapping compressor's tail
    pos0 = torch.full((1,), P - R, dtype=torch.int32, device=DEV)
    csa.compress(cfg, db["H"][:, P - R:P].contiguous(), pos0, weights, cache_b, ws)
    torch.cuda.synchronize()
    assert int(ct_b["n_entries"][0]) == P // w.m
    for k, b0 in zip(("entries", "idx_keys", "idx_scale"), before):
        assert torch.equal(ct_a[k][shared_rows], b0), "a shared block was written: " + k
    # B's own tokens as one chunk: compressor, causal selection, sparse attention
    n_own = TB - P
    pos0.fill_(P)
    csa.compress(cfg, db["H"][:, P:TB].contiguous(), pos0, weights, cache_b, ws)
    pos = torch.arange(P, TB, dtype=torch.int32, device=DEV).view(1, n_own)
    idx_b = torch.full((1, n_own, w.k), -7, dtype=torch.int32, device=DEV)
    csa.index_topk(cfg, db["qi"][:, P:TB].contiguous(), db["qi_scale"][:, P:TB].contiguous(),
                   db["wi"][:, P:TB].contiguous(), cache_b, pos, idx_b, ws)
    out_b = torch.empty((1, n_own, w.n_h, w.c), dtype=torch.bfloat16, device=DEV)
    csa.sparse_mqa(cfg, db["q"][:, P:TB].contiguous(), cache_b, idx_b, pos, db["sink"], out_b,
                   ws)
    torch.cuda.synchronize()
    n_ent = TB // w.m
    assert int(ct_b["n_entries"][0]) == n_ent

    # from scratch: B's whole token sequence through a contiguous cache
    cache_r, ct_r = _layer_cache(w, cfg, n_max, slots, False)
    out_r = torch.empty((1, TB, w.n_h, w.c), dtype=torch.bfloat16, device=DEV)
    csa.prefill(cfg, db["H"][:, :TB].contiguous(), weights, cache_r, db["q"][:, :TB].contiguous(),
                db["sink"], out_r, ws, qi=db["qi"][:, :TB].contiguous(),
                qi_scale=db["qi_scale"][:, :TB].contiguous(), wi=db["wi"][:, :TB].contiguous())
    torch.cuda.synchronize()
    ent_b = _from_pool(ct_b["entries"], tb, be)[0]
    keys_b = _from_pool(ct_b["idx_keys"], tb, be)[0]
    sc_b = _from_pool(ct_b["idx_scale"], tb, be)[0]
    assert torch.equal(ent_b[:n_ent], ct_r["entries"][0, :n_ent]), "entries differ"
    assert torch.equal(keys_b[:n_ent], ct_r["idx_keys"][0, :n_ent]), "indexer keys differ"
    assert torch.equal(sc_b[:n_ent].view(torch.int32),
                       ct_r["idx_scale"][0, :n_ent].view(torch.int32)), "key scales differ"
    wins = torch.arange(TB - w.n_win, TB, device=DEV) % slots
    assert torch.equal(ct_b["window"][0, wins], ct_r["window"][0, wins]), "window rows differ"
    check_close(bf16_f64(out_b.view(torch.int16)[0]),
                bf16_f64(out_r.view(torch.int16)[0, P:]), "outputs vs from-scratch run")

    # stage-wise oracle check of B's own queries on B's stored state
    full_idx = torch.full((1, TB, w.k), -1, dtype=torch.int32, device=DEV)
    full_idx[:, P:] = idx_b
    full_out = torch.zeros((1, TB, w.n_h, w.c), dtype=torch.bfloat16, device=DEV)
    full_out[:, P:] = out_b
    keys, ksc = _key_views(keys_b, sc_b, n_ent, w, False)
    rng = np.random.default_rng(2)
    qs = sorted(set([P, P + 1, TB - 1] + list(rng.integers(P, TB, 10))))
    _check_against_oracle(w, xb, TB, n_ent, host_bits(ent_b), host_bits(ct_b["window"][0]),
                          slots, keys, ksc, False, full_out, full_idx, qs)


def test_paged_ragged_batch_matches_contiguous():
    """Three sequences on one block table, appended by csa_compress at different positions (one
    restarting from 0), then one csa_decode step each at its own position: the paged cache
    gives the contiguous cache's entries, keys, scales, window rows and outputs bit for bit."""
    w = S.shrink(S.WORKLOADS["tiny_csa"], B=3)
    say("paged ragged batch", w.name)
    x = S.layer_inputs(w, T=200)
    d = {k: dev(x[k]) for k in x if isinstance(x[k], np.ndarray)}
    cfg = config_for(w, d["inv_freq"])
    be = _block_entries(w)
    bps = (216 // w.m + be) // be + 1
    n_max = bps * be
    slots = 256
    table, n_blocks = _perm_table(3, bps, 4, seed=9)
    tr, tc = csa.tail_shape(cfg)

    def make(paged):
        lead = (n_blocks * be,) if paged else (3, n_max)
        ct = dict(entries=torch.zeros(lead + (w.c,), dtype=torch.int16, device=DEV),
                  window=torch.zeros((3, slots, w.c), dtype=torch.int16, device=DEV),
                  n_entries=torch.zeros(3, dtype=torch.int32, device=DEV),
                  tail=torch.zeros((3, tr, tc), dtype=torch.float32, device=DEV),
                  idx_keys=torch.zeros(lead + (w.d_I,), dtype=torch.uint8, device=DEV),
                  idx_scale=torch.zeros(lead, dtype=torch.float32, device=DEV))
        kw = dict(block_table=dev(table), block_entries=be, n_blocks=n_blocks) if paged else {}
        return csa.make_cache(n_max, slots, **ct, **kw), ct

    weights = _weights(w, d)
    ws = workspace(max(csa.workspace_size(cfg, csa.OP_COMPRESS, 3, 120, n_max),
                       csa.workspace_size(cfg, csa.OP_DECODE, 3, 1, n_max)))
    runs = []
    for paged in (False, True):
        cache, ct = make(paged)
        pos0 = torch.zeros(3, dtype=torch.int32, device=DEV)
        csa.compress(cfg, d["H"][:, :120].contiguous(), pos0, weights, cache, ws)
        ct["n_entries"][1] = 0                       # sequence 1 restarts from position 0
        pos0 = torch.tensor([120, 0, 120], dtype=torch.int32, device=DEV)
        csa.compress(cfg, d["H"][:, 120:200].contiguous(), pos0, weights, cache, ws)
        pos = torch.tensor([199, 79, 199], dtype=torch.int32, device=DEV)
        out = torch.empty((3, w.n_h, w.c), dtype=torch.bfloat16, device=DEV)
        idx = torch.full((3, w.k), -7, dtype=torch.int32, device=DEV)
        csa.decode(cfg, cache, pos, d["q"][:, 199].contiguous(), d["sink"], out, ws,
                   qi=d["qi"][:, 199].contiguous(), qi_scale=d["qi_scale"][:, 199].contiguous(),
                   wi=d["wi"][:, 199].contiguous(), idx_out=idx)
        torch.cuda.synchronize()
        runs.append((ct, out, idx))
    (cc, oc, ic), (cp, op, ip) = runs
    assert torch.equal(cp["n_entries"], cc["n_entries"])
    for k in ("entries", "idx_keys", "idx_scale"):
        logical = _from_pool(cp[k], table, be)
        for b in range(3):
            n = int(cc["n_entries"][b])
            got, ref = logical[b, :n], cc[k][b, :n]
            if k == "idx_scale":
                got, ref = got.view(torch.int32), ref.view(torch.int32)
            assert torch.equal(got, ref), (k, b)
    assert torch.equal(cp["window"], cc["window"])
    assert torch.equal(op.view(torch.int16), oc.view(torch.int16))
    assert torch.equal(ip, ic)


@pytest.mark.parametrize("name", ["csa_decode_128k", "hca_decode_1m"])
def test_paged_decode_short_and_empty_sequences(name):
    """Sequences with no closed entry, fewer visible entries than k, a partial last block and a
    full cache, decoded from a paged cache: bit-equal to the contiguous cache."""
    w = dataclasses.replace(S.WORKLOADS[name], B=4, N=4096)
    say("paged short/empty sequences", name)
    x = G.decode_cache_inputs(w, DEV)
    x["n_entries"] = torch.tensor([0, 5, 300, w.N], dtype=torch.int32, device=DEV)
    csa_mode = w.mode == "csa"
    be = _block_entries(w)
    table, n_blocks = _perm_table(4, w.N // be, 2, seed=21)
    cfg = csa.make_config(csa.MODE_CSA if csa_mode else csa.MODE_HCA, w.m, w.n_h, w.c, w.r,
                          x["inv_freq"], top_k=w.k, n_win=w.n_win, idx_heads=w.H_I,
                          idx_dim=w.d_I, softmax_scale=w.scale)
    ws = workspace(csa.workspace_size(cfg, csa.OP_DECODE, 4, 1, w.N))
    q = x["q"][:, 0].contiguous()
    pools = {"entries": _to_pool(x["entries"], table, n_blocks, be)}
    if csa_mode:
        pools["idx_keys"] = _to_pool(x["ikeys"], table, n_blocks, be)
        pools["idx_scale"] = _to_pool(x["iscale"], table, n_blocks, be)
    caches = [csa.make_cache(w.N, w.n_win, x["entries"], x["window"], x["n_entries"],
                             idx_keys=x.get("ikeys"), idx_scale=x.get("iscale")),
              csa.make_cache(w.N, w.n_win, pools["entries"], x["window"], x["n_entries"],
                             idx_keys=pools.get("idx_keys"), idx_scale=pools.get("idx_scale"),
                             block_table=dev(table), block_entries=be, n_blocks=n_blocks)]
    res = []
    for cache in caches:
        out = torch.empty((4, w.n_h, w.c), dtype=torch.bfloat16, device=DEV)
        idx = torch.full((4, max(w.k, 1)), -7, dtype=torch.int32, device=DEV)
        if csa_mode:
            csa.decode(cfg, cache, x["pos"], q, x["sink"], out, ws, qi=x["qi"],
                       qi_scale=x["qi_scale"], wi=x["wi"], idx_out=idx)
        else:
            csa.decode(cfg, cache, x["pos"], q, x["sink"], out, ws)
        torch.cuda.synchronize()
        res.append((out, idx))
    (oc, ic), (op, ip) = res
    assert torch.equal(op.view(torch.int16), oc.view(torch.int16))
    if csa_mode:
        assert torch.equal(ip, ic)
        ih = ic.cpu().numpy()
        assert np.all(ih[0] == -1)                                  # nothing visible
        assert np.array_equal(ih[1, :5], np.arange(5)) and np.all(ih[1, 5:] == -1)
        assert np.array_equal(ih[2, :300], np.arange(300)) and np.all(ih[2, 300:] == -1)
    assert torch.isfinite(oc.float()).all()
