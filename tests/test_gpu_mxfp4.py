"""GPU parity of the MXFP4 indexer-key path (OCP MXFP4: E2M1 codes with an E8M0 scale per 32
dims; the query stays E4M3) against the oracle: decode scoring, top-k and attention on seeded
MXFP4 caches, and a whole tiny layer whose compressor writes the MXFP4 keys itself."""
import numpy as np
import pytest
import torch

import long_context_sparse_15_amd as csa
import oracle as O
from synth import inputs as S
from gpu_common import (DEV, bf16_f64, check_close, check_selection, config_for, dev, host_bits,
                        say, window_rows_ring, workspace)

pytestmark = pytest.mark.gpu


def _decode_case(w, B, N, positions):
    x = S.decode_cache_inputs(w, B=B, N=N, key_fmt="mxfp4")
    x["pos"] = np.array(positions, dtype=np.int32)
    d = {k: dev(x[k]) for k in ("entries", "window", "pos", "n_entries", "q", "sink", "inv_freq",
                                "ikeys", "iscale", "qi", "qi_scale", "wi")}
    cfg = config_for(w, d["inv_freq"], idx_key_format=csa.IDX_MXFP4)
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
        ref = O.index_scores_mxfp4(x["qi"][b, 0], x["qi_scale"][b, 0], x["wi"][b, 0],
                                   x["ikeys"][b], x["iscale"][b][:, :w.d_I // 32], n_vis)
        check_selection(idx_h[b], ref, w.k, "seq %d selection" % b)
        kk = min(w.k, n_vis)
        sel = idx_h[b, :kk]
        check_close(sc_h[b, :kk], ref[sel], "seq %d scores" % b,
                    atol=1e-5 * max(1.0, np.abs(ref).max(initial=0.0)), rtol=1e-5)
        assert np.all(np.isneginf(sc_h[b, kk:]))
        rows = np.concatenate([x["entries"][b][sel], window_rows_ring(x["window"][b], t, w.n_win,
                                                                      slots)])
        o_ref, _ = O.attend(x["q"][b, 0], rows, x["sink"], w.scale, t, x["inv_freq"])
        check_close(out_h[b], o_ref, "seq %d output" % b)


@pytest.mark.parametrize("case", [
    # (workload, B, N, positions): several chunks and a ragged tail; n_vis < k; no entry visible
    ("csa_decode_128k", 3, 5000, [4 * 5000 + 3, 4 * 3000 + 1, 10]),
    ("csa_decode_1m", 2, 40000, [4 * 40000 + 1, 4 * 33000]),   # multi-workgroup select
    ("tiny_csa", 2, 700, [2063, 2]),                            # d_I = 64: two blocks
])
def test_mxfp4_decode_parity(case):
    name, B, N, positions = case
    say("mxfp4 decode", case)
    _decode_case(S.shrink(S.WORKLOADS[name]), B, N, positions)


def _mx_codes(packed):
    c = np.empty(packed.shape[:-1] + (2 * packed.shape[-1],), dtype=np.int32)
    c[..., 0::2] = packed & 0xF
    c[..., 1::2] = packed >> 4
    return c


def test_mxfp4_layer_prefill_then_decode():
    """Tiny CSA layer with MXFP4 keys written by the compressor: prefill of 2048 tokens, then the
    16 decode steps.  Key scale bytes equal the oracle's except in blocks whose largest pooled
    magnitude lies within 1e-5 of a power of two; codes within one E2M1 step; then selection and
    attention stage-wise on the GPU's stored keys and rows."""
    w = S.WORKLOADS["tiny_csa"]
    T = 2048
    say("mxfp4 layer", T)
    x = S.layer_inputs(w, T=T)
    TT = x["T_total"]
    d = {k: dev(x[k]) for k in x if isinstance(x[k], np.ndarray)}
    cfg = config_for(w, d["inv_freq"], idx_key_format=csa.IDX_MXFP4)
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
    params = {k: x[k] for k in ("Ba", "Bb", "BIa", "BIb", "gamma", "gamma_win")}
    comp = O.compress_tokens(x["H"][0], x["W"], params, "csa", w.m, w.c, w.d_I, x["inv_freq"],
                             1e-6, idx_format="mxfp4")
    keys = ct["idx_keys"][0].cpu().numpy()[:n_ent]
    scl = ct["idx_scale"][0].cpu().numpy()[:n_ent]
    nb = w.d_I // 32
    assert np.all(scl[:, nb:] == 127), "unused scale bytes"
    amax = np.max(np.abs(comp["ipre"].reshape(n_ent, nb, 32)), axis=2)
    near = np.abs(amax / np.exp2(np.round(np.log2(np.maximum(amax, 1e-300)))) - 1.0) < 1e-5
    same = scl[:, :nb] == comp["iscale"]
    assert np.all(same | near), "block scale bytes differ away from a power-of-two boundary"
    gc, oc = _mx_codes(keys), _mx_codes(comp["ikeys"])
    mag = lambda c: np.where(c & 8, -(c & 7), c & 7)
    diff = np.abs(mag(gc) - mag(oc)).reshape(n_ent, nb, 32)
    assert np.all(diff[same] <= 1), "key codes differ by more than one E2M1 step"
    ent = host_bits(ct["entries"][0])
    win = host_bits(ct["window"][0])
    check_close(O.bf16_bits_to_f64(ent[:n_ent]), O.bf16_bits_to_f64(comp["entries"]), "entries")
    rng = np.random.default_rng(0)
    qs = sorted(set([0, 3, 4, 5, 127, 128, 129, T - 1] + list(range(T, TT)) +
                    list(rng.integers(0, T, 24))))
    out_h = bf16_f64(out.view(torch.int16)[0])
    idx_h = idx[0].cpu().numpy()
    for t in qs:
        n_vis = O.visible_entries(t, w.m, n_ent)
        sc = O.index_scores_mxfp4(x["qi"][0, t], x["qi_scale"][0, t], x["wi"][0, t], keys,
                                  scl[:, :nb], n_vis)
        check_selection(idx_h[t], sc, w.k, "query %d selection" % t)
        sel = idx_h[t][:min(w.k, n_vis)]
        rows = np.concatenate([ent[sel], win[O.window_tokens(t, w.n_win) % slots]])
        ref, _ = O.attend(x["q"][0, t], rows, x["sink"], w.scale, t, x["inv_freq"])
        check_close(out_h[t], ref, "query %d output" % t)
