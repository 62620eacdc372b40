"""GPU parity of csa_sparse_mqa with many query rows (the prefill shape: more rows than
workgroups resident at once) against the oracle's float64 attention on sampled rows: early rows
with short windows, lists padded with -1 as top-k pads them, indices past the sequence's
entries, and rows on both sides of multiples of the CU count."""
import numpy as np
import pytest
import torch

import long_context_sparse_15_amd as csa
import oracle as O
from synth import inputs as S
from gpu_common import DEV, bf16_f64, check_close, dev, say, workspace

pytestmark = pytest.mark.gpu


def _case(seed, nq, k, N, n_ent, n_h=64, c=512, r=64, n_win=128):
    rng = np.random.Generator(np.random.PCG64(seed))
    B, slots = 1, nq + 8
    entries = S.bf16_normal(rng, (B, N, c))
    window = S.bf16_normal(rng, (B, slots, c))
    q = S.bf16_normal(rng, (B, nq, n_h, c))
    sink = rng.standard_normal(n_h).astype(np.float32)
    pos = np.arange(nq, dtype=np.int32).reshape(B, nq)
    idx = np.full((B, nq, k), -1, dtype=np.int32)
    for i in range(nq):
        nv = int(rng.integers(k - 24, k + 1))
        sel = np.sort(rng.choice(N, size=nv, replace=False))  # some beyond n_ent: masked
        idx[0, i, :nv] = sel
    inv = S.rope_inv_freq(r, 160000.0)
    scale = 1.0 / np.sqrt(c)
    cfg = csa.make_config(csa.MODE_CSA, 4, n_h, c, r, dev(inv), top_k=k, n_win=n_win,
                          idx_heads=64, idx_dim=128, softmax_scale=scale)
    ne = np.array([n_ent], dtype=np.int32)
    cache = csa.make_cache(N, slots, dev(entries), dev(window), dev(ne))
    out = torch.empty((B, nq, n_h, c), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, nq, n_h), dtype=torch.float32, device=DEV)
    ws = workspace(csa.workspace_size(cfg, csa.OP_SPARSE_MQA, B, nq, N))
    csa.sparse_mqa(cfg, dev(q), cache, dev(idx), dev(pos), dev(sink), out, ws, lse_out=lse)
    torch.cuda.synchronize()
    out_h = bf16_f64(out.view(torch.int16))
    lse_h = lse.cpu().numpy()
    G = 256  # CU count of the device: check rows around its multiples
    picks = sorted(set([0, 1, 2, 3, 100, G - 1, G, G + 1, 2 * G - 1, 2 * G, 3 * G, 4 * G - 1,
                        4 * G, nq - 2, nq - 1] + list(rng.integers(0, nq, size=12))))
    for i in picks:
        if i >= nq:
            continue
        t = int(pos[0, i])
        sel = idx[0, i][(idx[0, i] >= 0) & (idx[0, i] < n_ent)]
        win = window[0][[u % slots for u in O.window_tokens(t, n_win)]]
        rows = np.concatenate([entries[0][sel], win])
        ref, ref_lse = O.attend(q[0, i], rows, sink, scale, t, inv)
        check_close(out_h[0, i], ref, "row %d output" % i)
        check_close(lse_h[0, i], ref_lse, "row %d lse" % i, atol=2e-3, rtol=1e-4)


@pytest.mark.parametrize("case", [
    # (seed, rows, k, entries, visible entries, heads)
    (21, 1100, 160, 600, 560, 64),
    # 512-entry lists (the prefill top-k)
    (22, 1309, 512, 1500, 1500, 64),
    # more than 64 heads: two 64-head groups of workgroups, also with a head count that leaves
    # part of the last group empty
    (23, 300, 512, 1500, 1400, 128),
    (24, 270, 160, 600, 560, 96),
])
def test_many_row_sparse_attention_parity(case):
    say("many-row attention", case)
    seed, nq, k, N, n_ent, n_h = case
    _case(seed, nq, k, N, n_ent, n_h=n_h)
