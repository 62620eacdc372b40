"""GPU parity of mixed-precision entries (CSA_ENT_MIXED: the unrotated dims as E4M3 codes without
a scale, the RoPE dims in bf16; reading R22) against the oracle:

* the compressor writes mixed rows: codes within one E4M3 step of the oracle's quantisation of
  its own float64 values, RoPE dims within the bf16 bound;
* a whole layer (prefill, then decode steps) at the production head shape, checked stage-wise:
  each query's selection against the oracle's scores, its output against the oracle's attention
  over the GPU's stored rows decoded by the oracle; the same layer on the block layout gives the
  same bits;
* full-size decodes (128K CSA, 1M HCA) over synthetic mixed caches, sampled sequences against
  the oracle."""
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


def _wide():
    return dataclasses.replace(S.WORKLOADS["tiny_csa"], name="tiny_csa_wide", c=512, n_h=64,
                               H_I=64, d_I=128, T=1024)


def _e4m3_steps(a, b):
    a = a.astype(np.int32)
    b = b.astype(np.int32)
    mag = lambda c: np.where(c & 0x80, -(c & 0x7F), c & 0x7F)
    return np.abs(mag(a) - mag(b))


def _run(w, x, d, cfg, n_max, slots, table=None, n_blocks=0):
    T, TT = x["T"], x["T_total"]
    eb = w.c + w.r
    be = 128 // w.m
    lead = (n_blocks * be,) if table is not None else (1, n_max)
    tr, tc = csa.tail_shape(cfg)
    ct = dict(entries=torch.zeros(lead + (eb,), dtype=torch.uint8, device=DEV),
              window=torch.zeros((1, slots, w.c), dtype=torch.int16, device=DEV),
              n_entries=torch.zeros(1, dtype=torch.int32, device=DEV),
              tail=torch.zeros((1, tr, tc), dtype=torch.float32, device=DEV),
              idx_keys=torch.zeros(lead + (w.d_I,), dtype=torch.uint8, device=DEV),
              idx_scale=torch.zeros(lead, dtype=torch.float32, device=DEV))
    kw = {}
    if table is not None:
        kw = dict(block_table=dev(table), block_entries=be, n_blocks=n_blocks)
    cache = csa.make_cache(n_max, slots, **ct, **kw)
    weights = csa.make_weights(d["W"], d["Ba"], d["gamma"], d["gamma_win"], bias_b=d["Bb"],
                               bias_ia=d["BIa"], bias_ib=d["BIb"])
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
                   h_new=d["H"][:, t].contiguous(), weights=weights,
                   qi=d["qi"][:, t].contiguous(), qi_scale=d["qi_scale"][:, t].contiguous(),
                   wi=d["wi"][:, t].contiguous(), idx_out=idx[:, t])
    torch.cuda.synchronize()
    return out, idx, ct


@pytest.mark.parametrize("T", [1024, 1022])
def test_mixed_layer_against_oracle(T):
    w = _wide()
    say("mixed layer", w.name, "T", T)
    x = S.layer_inputs(w, T=T)
    TT = x["T_total"]
    d = {k: dev(x[k]) for k in x if isinstance(x[k], np.ndarray)}
    cfg = config_for(w, d["inv_freq"], entry_format=csa.ENT_MIXED)
    be = 128 // w.m
    bps = (TT // w.m + 1 + be - 1) // be
    n_max = bps * be
    slots = 1 << (TT - 1).bit_length()
    out, idx, ct = _run(w, x, d, cfg, n_max, slots)
    n_ent = TT // w.m
    assert int(ct["n_entries"][0]) == n_ent
    k = w.c - w.r
    rows = ct["entries"][0, :n_ent].cpu().numpy()
    codes = rows[:, :k]
    rope = np.ascontiguousarray(rows[:, k:]).view(np.uint16)

    # compressor: the oracle's own mixed quantisation of its float64 entries
    params = {kk: x[kk] for kk in ("Ba", "Bb", "BIa", "BIb", "gamma", "gamma_win")}
    comp = O.compress_tokens(x["H"][0], x["W"], params, "csa", w.m, w.c, w.d_I, x["inv_freq"],
                             1e-6, entry_format="mixed")
    assert _e4m3_steps(codes, comp["ecodes"]).max() <= 1, "entry codes differ by > one step"
    check_close(O.bf16_bits_to_f64(rope), O.bf16_bits_to_f64(comp["erope"]), "RoPE dims")

    # stage-wise selection and attention on the stored state
    ent = O.decode_entries_mixed(codes, rope)
    win = host_bits(ct["window"][0])
    keys = ct["idx_keys"][0].cpu().numpy()[:n_ent]
    ksc = ct["idx_scale"][0].cpu().numpy()[:n_ent]
    out_h = bf16_f64(out.view(torch.int16)[0])
    idx_h = idx[0].cpu().numpy()
    rng = np.random.default_rng(4)
    for t in sorted(set([0, 4, 127, 128, 129, T - 1] + list(range(T, TT)) +
                        list(rng.integers(0, T, 12)))):
        n_vis = O.visible_entries(t, w.m, n_ent)
        sc = O.index_scores(x["qi"][0, t], x["qi_scale"][0, t], x["wi"][0, t], keys, ksc, n_vis)
        check_selection(idx_h[t], sc, w.k, "query %d selection" % t)
        sel = idx_h[t][:min(w.k, n_vis)]
        rws = np.concatenate([ent[sel], win[O.window_tokens(t, w.n_win) % slots]])
        ref, _ = O.attend(x["q"][0, t], rws, x["sink"], w.scale, t, x["inv_freq"])
        check_close(out_h[t], ref, "query %d output" % t)

    # the same layer on the block layout: identical bits
    n_blocks = bps + 3
    table = np.random.default_rng(T).permutation(n_blocks)[:bps].reshape(1, bps).astype(np.int32)
    out_p, idx_p, ct_p = _run(w, x, d, cfg, n_max, slots, table, n_blocks)
    assert torch.equal(out_p.view(torch.int16), out.view(torch.int16)), "paged outputs differ"
    assert torch.equal(idx_p, idx)
    r = (torch.from_numpy(table).to(DEV).long()[:, :, None] * be +
         torch.arange(be, device=DEV)).reshape(-1)
    assert torch.equal(ct_p["entries"][r][:n_ent], ct["entries"][0, :n_ent])


@pytest.mark.parametrize("name,B", [("csa_decode_128k", 8), ("hca_decode_1m", 4)])
def test_mixed_decode_full_size(name, B):
    w = dataclasses.replace(S.WORKLOADS[name], B=B)
    say("mixed decode", name, "B=%d N=%d" % (B, w.N))
    x = G.decode_cache_inputs(w, DEV, entry_fmt="mixed")
    csa_mode = w.mode == "csa"
    cfg = csa.make_config(csa.MODE_CSA if csa_mode else csa.MODE_HCA, w.m, w.n_h, w.c, w.r,
                          x["inv_freq"], top_k=w.k, n_win=w.n_win, idx_heads=w.H_I,
                          idx_dim=w.d_I, softmax_scale=w.scale, entry_format=csa.ENT_MIXED)
    cache = csa.make_cache(w.N, w.n_win, x["entries"], x["window"], x["n_entries"],
                           idx_keys=x.get("ikeys"), idx_scale=x.get("iscale"))
    ws = workspace(csa.workspace_size(cfg, csa.OP_DECODE, B, 1, w.N))
    out = torch.empty((B, w.n_h, w.c), dtype=torch.bfloat16, device=DEV)
    idx = torch.full((B, max(w.k, 1)), -7, dtype=torch.int32, device=DEV)
    q = x["q"][:, 0].contiguous()
    if csa_mode:
        csa.decode(cfg, cache, x["pos"], q, x["sink"], out, ws, qi=x["qi"],
                   qi_scale=x["qi_scale"], wi=x["wi"], idx_out=idx)
    else:
        csa.decode(cfg, cache, x["pos"], q, x["sink"], out, ws)
    torch.cuda.synchronize()
    out_h = bf16_f64(out.view(torch.int16))
    inv = x["inv_freq"].cpu().numpy()
    sink = x["sink"].cpu().numpy()
    t = int(w.t)
    n_vis = O.visible_entries(t, w.m, w.N)
    k = w.c - w.r
    for b in (0, B - 1):
        rows = x["entries"][b].cpu().numpy()
        ent = O.decode_entries_mixed(rows[:, :k], np.ascontiguousarray(rows[:, k:]).view(np.uint16))
        win = host_bits(x["window"][b])
        if csa_mode:
            sc = O.index_scores(x["qi"][b, 0].cpu().numpy(), x["qi_scale"][b, 0].cpu().numpy(),
                                x["wi"][b, 0].cpu().numpy(), x["ikeys"][b].cpu().numpy(),
                                x["iscale"][b].cpu().numpy(), n_vis)
            ih = idx[b].cpu().numpy()
            check_selection(ih, sc, w.k, "sequence %d selection" % b)
            sel = ih[:min(w.k, n_vis)]
        else:
            sel = np.arange(n_vis)
        rws = np.concatenate([ent[sel], win[O.window_tokens(t, w.n_win) % w.n_win]])
        qb = host_bits(x["q"][b, 0])
        ref, _ = O.attend(qb, rws, sink, w.scale, t, inv)
        check_close(out_h[b], ref, "sequence %d output" % b)
