"""Helpers shared by the GPU parity tests: device copies of the seeded inputs, cache and config
construction through the binding, and the comparison rules against the oracle."""
import sys

import numpy as np
import torch

import long_context_sparse_15_amd as csa
import oracle as O

DEV = "cuda"

# floating-point outputs: |gpu - ref| <= ATOL + RTOL * |ref|  (bf16 outputs, fp32 accumulation)
ATOL, RTOL = 1e-2, 2e-2
# index sets: elements may differ only where the oracle score is within this band of the k-th
TIE_REL = 1e-3
# fp32 index scores: |gpu - oracle| <= FP32_SCORE_ATOL * max(1, max|score of the row|) + 1e-5 |score|
FP32_SCORE_ATOL = 1e-5


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def dev(x):
    """numpy -> torch on the GPU; uint16 bf16 bit patterns travel as int16."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        x = x.view(np.int16)
    return torch.from_numpy(x).to(DEV)


def host_bits(t):
    """GPU bf16 (int16) tensor -> numpy uint16 bit patterns."""
    return t.cpu().numpy().view(np.uint16)


def bf16_f64(t):
    return O.bf16_bits_to_f64(host_bits(t))


def config_for(w, inv_freq_dev, **over):
    kw = dict(mode=csa.MODE_CSA if w.mode == "csa" else csa.MODE_HCA, m=w.m, n_heads=w.n_h,
              head_dim=w.c, rope_dim=w.r, inv_freq=inv_freq_dev, top_k=w.k, n_win=w.n_win,
              idx_heads=w.H_I, idx_dim=w.d_I, hidden=w.D, softmax_scale=w.scale, rms_eps=1e-6)
    kw.update(over)
    return csa.make_config(**kw)


def workspace(nbytes):
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=DEV)


def check_close(got, ref, what, atol=ATOL, rtol=RTOL):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    err = np.abs(got - ref)
    bad = err > atol + rtol * np.abs(ref)
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError("%s: %d/%d outside tolerance; first at %s got %r ref %r" %
                             (what, int(bad.sum()), bad.size, tuple(i), got[tuple(i)],
                              ref[tuple(i)]))


def check_selection(idx_row, scores_ref, k, what):
    """GPU index row (ascending, -1 padded) against the oracle's float64 scores: same size,
    ascending, unique, visible, and equal to the oracle's set except where a score lies within
    the tie band of the k-th score."""
    n_vis = scores_ref.shape[0]
    kk = min(k, n_vis)
    idx_row = np.asarray(idx_row)
    assert np.all(idx_row[kk:] == -1), what + ": padding"
    sel = idx_row[:kk]
    assert np.all(sel >= 0) and np.all(sel < n_vis), what + ": out of range"
    assert np.all(np.diff(sel) > 0), what + ": not strictly ascending"
    ref = O.topk_select(scores_ref, k)
    if kk == 0:
        return
    kth = np.sort(scores_ref)[::-1][kk - 1]
    band = TIE_REL * max(1.0, abs(kth))
    diff = np.setxor1d(sel, ref)
    if diff.size:
        far = diff[np.abs(scores_ref[diff] - kth) > band]
        assert far.size == 0, "%s: %d indices differ outside the tie band (e.g. %d: %r vs kth %r)" % (
            what, far.size, far[0], scores_ref[far[0]], kth)


def window_rows_ring(win_bits_b, t, n_win, slots):
    """Rows of a ring window buffer for query t (token u in row u % slots)."""
    return win_bits_b[[u % slots for u in O.window_tokens(t, n_win)]]


def bf16_ulp(v):
    """Spacing of bf16 numbers at |v| (8 significant bits): 2^(floor(log2|v|) - 7)."""
    a = abs(float(v))
    if a == 0.0:
        return 2.0 ** -133
    return 2.0 ** (np.floor(np.log2(a)) - 7)


def check_selection_bf16(idx_row, scores_ref, k, what):
    """As check_selection for BF16 index scores (reading R25): the oracle's float64 scores are
    rounded to bf16 and ranked with the lower index winning ties; the GPU rounds its fp32 score,
    which can land one bf16 step away, so indices may differ only where the oracle's bf16 score
    lies within one bf16 ulp of the k-th one."""
    n_vis = scores_ref.shape[0]
    kk = min(k, n_vis)
    idx_row = np.asarray(idx_row)
    assert np.all(idx_row[kk:] == -1), what + ": padding"
    sel = idx_row[:kk]
    assert np.all(sel >= 0) and np.all(sel < n_vis), what + ": out of range"
    assert np.all(np.diff(sel) > 0), what + ": not strictly ascending"
    if kk == 0:
        return
    rb = O.round_scores_bf16(scores_ref)
    ref = O.topk_select(rb, k)
    kth = np.sort(rb)[::-1][kk - 1]
    # one bf16 step, plus the fp32 score's own error (as the fp32 score check allows it)
    band = bf16_ulp(kth) * (1 + 1e-9) + FP32_SCORE_ATOL * max(1.0, np.abs(scores_ref).max())
    diff = np.setxor1d(sel, ref)
    if diff.size:
        far = diff[np.abs(rb[diff] - kth) > band]
        assert far.size == 0, "%s: %d indices differ outside one bf16 ulp of the k-th score " \
            "(e.g. %d: %r vs kth %r)" % (what, far.size, far[0], rb[far[0]], kth)


def check_scores_bf16(got, scores_ref, what, full_ref=None):
    """GPU bf16 scores (widened to fp32) against the oracle's float64 scores: bf16 values within
    one bf16 step of the oracle's score plus the fp32 sum's own error (the GPU rounds an fp32
    sum whose error the fp32 score check bounds by FP32_SCORE_ATOL * max(1, max|score|) absolute
    and 1e-5 relative; head weights of both signs can make a small score out of large terms)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(scores_ref, np.float64)
    assert np.array_equal(O.round_scores_bf16(got), got), what + ": not bf16 values"
    scale = max(1.0, np.abs(ref if full_ref is None else full_ref).max(initial=0.0))
    ulp = np.array([bf16_ulp(v) for v in ref])
    bad = np.abs(got - ref) > ulp * (1 + 1e-9) + FP32_SCORE_ATOL * scale + 1e-5 * np.abs(ref)
    assert not bad.any(), "%s: %d scores more than one bf16 step off" % (what, int(bad.sum()))
