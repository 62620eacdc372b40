"""Pins for the CPU oracle: each test checks the oracle against something other than its own
formula - hand-computed fixtures (tests/golden), closed forms, textbook special cases computed
with torch, and brute force on tiny inputs.  CPU only."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O
from synth import inputs as S

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _num(v):
    if isinstance(v, str):
        if v.startswith("ln"):
            return math.log(float(v[2:]))
        if "/" in v:
            a, b = v.split("/")
            return float(a) / float(b)
        return float(v)
    return float(v)


def _col(xs):
    return np.array([_num(v) for v in xs], dtype=np.float64)[:, None]


# ----------------------------------------------------------------------------- formats

def test_e4m3_table_spec_points():
    g = _gold("e4m3_points.json")
    tab = O.e4m3_table()
    for code, val in g["points"]:
        assert tab[code] == val and math.copysign(1, tab[code]) == math.copysign(1, val), code
    for code in g["nan_codes"]:
        assert math.isnan(tab[code])
    assert np.sum(np.isnan(tab)) == 2


def test_e4m3_table_matches_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).double().numpy()
    tab = O.e4m3_table()
    fin = ~np.isnan(ref)
    assert np.array_equal(np.isnan(ref), np.isnan(tab))
    assert np.array_equal(ref[fin], tab[fin])


def test_e4m3_encode_matches_torch_rne():
    rng = np.random.default_rng(11)
    tab = O.e4m3_table()
    fin = tab[~np.isnan(tab)]
    # all representable values, all midpoints between neighbours (ties), random values
    pos = np.unique(np.abs(fin))
    mids = (pos[1:] + pos[:-1]) / 2
    x = np.concatenate([fin, mids, -mids, rng.uniform(-460, 460, 20000),
                        rng.standard_normal(20000) * 0.01])
    x = x[np.abs(x) < 464]  # torch gives NaN from the midpoint 464 upward; the oracle saturates
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8)
    got = O.e4m3_encode(x.astype(np.float32).astype(np.float64))
    assert np.array_equal(ref.numpy(), got)
    assert np.all(O.e4m3_encode(np.array([500.0, 1e6, -1e9])) == np.array([0x7E, 0x7E, 0xFE]))


def test_e2m1_table_spec_points():
    g = _gold("mxfp4_points.json")
    for code, val in g["e2m1"]:
        got = float(O.e2m1_decode(np.array([code]))[0])
        assert got == val and math.copysign(1, got) == math.copysign(1, val), code


def test_e2m1_encode_spec_examples():
    g = _gold("mxfp4_points.json")
    for x, code in g["encode"]:
        assert int(O.e2m1_encode(np.array([x]))[0]) == code, x


def test_e2m1_encode_is_nearest_with_even_ties_brute_force():
    mags = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    xs = np.concatenate([np.linspace(-8, 8, 4001), np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5,
                                                             5.0, -0.25, -5.0])])
    got = O.e2m1_encode(xs)
    for x, c in zip(xs, got):
        a = min(abs(x), 6.0)
        d = np.abs(mags - a)
        best = np.flatnonzero(d == d.min())
        want = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
        assert (int(c) & 7) == want and (int(c) >> 3) == int(np.signbit(x)), x


def test_mx_shared_exponent_fixture_and_torch_e8m0():
    g = _gold("mxfp4_points.json")
    for b in g["blocks"]:
        assert int(O.mx_shared_exponent(np.array([b["amax"]]))[0]) + 127 == b["scale_byte"], b
    # floor(log2(x)) of a normal binary32 is its biased exponent field minus 127; the shared
    # exponent is that minus 2 (the largest E2M1 exponent), clamped to E8M0's range
    rng = np.random.default_rng(21)
    a = np.exp2(rng.uniform(-125, 125, 4000)).astype(np.float32)
    field = ((a.view(np.uint32) >> np.uint32(23)) & np.uint32(0xFF)).astype(np.int64)
    want = np.clip(field - 127 - 2, -127, 127)
    assert np.array_equal(O.mx_shared_exponent(a.astype(np.float64)), want)


def test_quantize_rows_mxfp4_packing_hand_example():
    x = np.zeros((1, 64))
    x[0, :4] = [1.0, 2.0, 3.0, 4.0]      # block 0: amax 4 -> exponent 0, codes 2, 4, 5, 6
    x[0, 32:34] = [-0.75, 0.1875]        # block 1: amax 0.75 -> exponent -3, scaled -6, 1.5
    packed, scales = O.quantize_rows_mxfp4(x)
    assert list(scales[0]) == [127, 124]
    assert list(packed[0, :2]) == [0x42, 0x65] and np.all(packed[0, 2:16] == 0)
    assert list(packed[0, 16:17]) == [0x3F] and np.all(packed[0, 17:] == 0)
    assert np.array_equal(O.mxfp4_decode(packed, scales), x)


def test_quantize_rows_mxfp4_roundtrip_and_error_bound():
    rng = np.random.default_rng(22)
    # values already on the grid round-trip exactly
    codes = rng.integers(0, 16, (8, 128)).astype(np.uint8)
    codes[:, ::32] = 7                   # every block reaches magnitude 6: exponent = block's
    se = rng.integers(-10, 10, (8, 4))
    x = O.e2m1_decode(codes) * np.repeat(np.exp2(se.astype(np.float64)), 32, axis=1)
    p, s = O.quantize_rows_mxfp4(x)
    assert np.array_equal(O.mxfp4_decode(p, s), x)
    # random rows: each element within half a grid step of its scaled value (or clamped to 6)
    y = rng.standard_normal((64, 128)) * np.exp2(rng.integers(-8, 8, (64, 1)))
    p, s = O.quantize_rows_mxfp4(y)
    d = O.mxfp4_decode(p, s)
    X = np.repeat(np.exp2(s.astype(np.float64) - 127), 32, axis=1)
    a = np.abs(y) / X
    step = np.where(a < 2, 0.5, np.where(a < 4, 1.0, 2.0))
    err = np.abs(d - y) / X
    clamp = np.maximum(a - 6.0, 0.0)
    assert np.all(err <= 0.5 * step + clamp + 1e-12)
    assert np.all(np.max(np.abs(d), axis=1) > 0)


def test_index_scores_mxfp4_equals_e4m3_path_on_shared_values():
    # keys whose real values are exact in both formats (E2M1 magnitudes x 2^e, |.| <= 448):
    # the MXFP4 scorer must give exactly the E4M3 scorer's scores
    rng = np.random.default_rng(23)
    H, d, N = 4, 64, 50
    codes = rng.integers(0, 16, (N, d)).astype(np.uint8)
    codes[:, ::32] = 7
    se = rng.integers(-3, 5, (N, d // 32))
    kv = O.e2m1_decode(codes) * np.repeat(np.exp2(se.astype(np.float64)), 32, axis=1)
    kp, ks = O.quantize_rows_mxfp4(kv)
    ke = O.e4m3_encode(kv)
    assert np.array_equal(O.e4m3_decode(ke), kv)
    qc = S.e4m3_normalish(rng, (H, d))
    qs = rng.uniform(0.5, 2.0, H).astype(np.float32)
    wi = rng.standard_normal(H).astype(np.float32)
    a = O.index_scores(qc, qs, wi, ke, np.ones(N, np.float32), N - 3)
    b = O.index_scores_mxfp4(qc, qs, wi, kp, ks, N - 3)
    assert a.shape == (N - 3,) and np.array_equal(a, b)


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(12)
    x = np.concatenate([rng.standard_normal(50000) * 10.0 ** rng.integers(-30, 30, 50000),
                        1.0 + np.arange(1, 512) * 2.0 ** -9, [0.0, -0.0, 1e-40, -3e-39]])
    # float32-representable inputs: torch converts float64 through float32 (a double rounding
    # the oracle does not do), so compare where both are a single RNE step
    x = x.astype(np.float32).astype(np.float64)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = O.f64_to_bf16_bits(x)
    assert np.array_equal(ref, got)
    back = O.bf16_bits_to_f64(got)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).double().numpy())


def test_quantize_rows_e4m3_scale_and_range():
    rng = np.random.default_rng(13)
    x = rng.standard_normal((64, 128)) * rng.uniform(0.01, 100, (64, 1))
    codes, scale = O.quantize_rows_e4m3(x)
    dec = O.e4m3_decode(codes) * scale[:, None].astype(np.float64)
    # the largest magnitude maps to the largest finite code; relative error <= half an ulp (2^-4)
    assert np.all(np.max(np.abs(O.e4m3_decode(codes)), axis=1) == 448.0)
    big = np.abs(x) > scale[:, None] * 2.0 ** -6
    assert np.all(np.abs(dec - x)[big] <= np.abs(x)[big] * 2.0 ** -4 * (1 + 1e-6))
    z, zs = O.quantize_rows_e4m3(np.zeros((2, 8)))
    assert np.all(O.e4m3_decode(z) == 0) and np.all(zs == 1.0)


# ----------------------------------------------------------------------------- compressor

def test_pool_overlap_hand_fixture():
    g = _gold("pool_overlap_m2.json")
    m = g["m"]
    Ca, Cb, Za, Zb = (_col(g[k]) for k in ("Ca", "Cb", "Za", "Zb"))
    for case in g["cases"]:
        got = O.pool_overlap(Ca, Cb, Za, Zb, _col(case["Ba"]), _col(case["Bb"]), m, 2)
        assert np.allclose(got[:, 0], [_num(v) for v in case["expect"]], rtol=1e-13, atol=0)


def test_pool_plain_hand_fixture():
    g = _gold("pool_plain_m3.json")
    C, Z = _col(g["C"]), _col(g["Z"])
    got = O.pool_plain(C, Z, np.zeros((3, 1)), 3, 2)
    assert abs(got[0, 0] - _num(g["expect_block0_nobias"])) < 1e-12
    got = O.pool_plain(C, np.zeros((6, 1)), _col(g["B"]), 3, 2)
    assert abs(got[1, 0] - _num(g["expect_block1_bias"])) < 1e-12


def test_pool_constant_logits_is_mean():
    """Closed form: with Z constant per channel and zero bias every weight is equal, so block i
    is the mean of its 2m rows (m rows for block 0 of the overlapping compressor, m' for HCA)."""
    rng = np.random.default_rng(1)
    m, T, w = 4, 32, 5
    Ca, Cb = rng.standard_normal((T, w)), rng.standard_normal((T, w))
    Z = np.tile(rng.standard_normal((1, w)), (T, 1))
    got = O.pool_overlap(Ca, Cb, Z, Z, np.zeros((m, w)), np.zeros((m, w)), m, T // m)
    assert np.allclose(got[0], Ca[0:m].mean(0), atol=1e-14)
    for i in range(1, T // m):
        ref = (Ca[m * i:m * i + m].sum(0) + Cb[m * i - m:m * i].sum(0)) / (2 * m)
        assert np.allclose(got[i], ref, atol=1e-14)
    got = O.pool_plain(Ca, Z, np.zeros((8, w)), 8, T // 8)
    assert np.allclose(got, Ca.reshape(T // 8, 8, w).mean(1), atol=1e-14)


def test_pool_weights_are_a_convex_combination():
    """Weights are non-negative and sum to 1 per channel: with C = 1 every entry is exactly 1,
    and every entry lies within [min, max] of its rows."""
    rng = np.random.default_rng(2)
    m, T, w = 4, 40, 7
    Z1, Z2 = rng.standard_normal((T, w)) * 5, rng.standard_normal((T, w)) * 5
    B1, B2 = rng.standard_normal((m, w)), rng.standard_normal((m, w))
    ones = np.ones((T, w))
    assert np.allclose(O.pool_overlap(ones, ones, Z1, Z2, B1, B2, m, T // m), 1.0, atol=1e-14)
    Ca, Cb = rng.standard_normal((T, w)), rng.standard_normal((T, w))
    got = O.pool_overlap(Ca, Cb, Z1, Z2, B1, B2, m, T // m)
    for i in range(1, T // m):
        rows = np.concatenate([Ca[m * i:m * i + m], Cb[m * i - m:m * i]])
        assert np.all(got[i] <= rows.max(0) + 1e-12) and np.all(got[i] >= rows.min(0) - 1e-12)


def test_pool_overlap_swap_symmetry():
    """Brute force on the definition's structure: dropping the b-stream (B^b -> -inf) leaves a
    plain m-row pooling of the a-stream (the HCA operator with m' = m)."""
    rng = np.random.default_rng(3)
    m, T, w = 4, 24, 3
    Ca, Cb, Za, Zb = (rng.standard_normal((T, w)) for _ in range(4))
    Ba = rng.standard_normal((m, w))
    got = O.pool_overlap(Ca, Cb, Za, Zb, Ba, np.full((m, w), -1e300), m, T // m)
    ref = O.pool_plain(Ca, Za, Ba, m, T // m)
    assert np.allclose(got, ref, atol=1e-14)


def test_entry_counts_match_the_pages():
    """floor(T/m) closed entries: 2048 tokens -> 512 CSA entries; 2^20 tokens -> 262144 CSA and
    8192 HCA entries; a 128-token block (lcm(4,128)) gives 32 CSA + 1 HCA entries."""
    assert O.visible_entries(2047, 4, 10 ** 9) == 512
    assert O.visible_entries((1 << 20) - 1, 4, 10 ** 9) == 262144
    assert O.visible_entries((1 << 20) - 1, 128, 10 ** 9) == 8192
    assert O.visible_entries(127, 4, 10 ** 9) == 32 and O.visible_entries(127, 128, 10 ** 9) == 1
    # entry s becomes visible exactly at token t = m(s+1) - 1 (closed block, 0-based tokens)
    for m in (1, 4, 128):
        for s in range(5):
            t = m * (s + 1) - 1
            assert O.visible_entries(t, m, 10 ** 9) == s + 1
            assert O.visible_entries(t - 1, m, 10 ** 9) == s
    assert list(O.window_tokens(2, 128)) == [0, 1, 2]
    assert list(O.window_tokens(300, 128)) == list(range(173, 301))


def test_rms_norm_closed_forms():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((10, 512)) * 7
    y = O.rms_norm(x, np.ones(512), 0.0)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=1)), 1.0, atol=1e-12)
    assert np.allclose(O.rms_norm(3.5 * x, np.ones(512), 0.0), y, atol=1e-12)
    g = rng.standard_normal(512)
    assert np.allclose(O.rms_norm(x, g, 1e-6), O.rms_norm(x, np.ones(512), 1e-6) * g)
    # eps: an all-equal row of value v has rms |v|, result v/sqrt(v^2+eps)
    v = 1e-3
    assert np.allclose(O.rms_norm(np.full((1, 4), v), np.ones(4), 1e-6), v / math.sqrt(v * v + 1e-6))


def test_rope_matches_complex_multiplication():
    rng = np.random.default_rng(5)
    c, r = 16, 8
    f = S.rope_inv_freq(r, 160000.0)
    x = rng.standard_normal((3, c))
    pos = np.array([0, 7, 1 << 20])
    y = O.rope_rotate(x, pos, f)
    assert np.array_equal(y[:, :c - r], x[:, :c - r])
    z = (x[:, c - r::2] + 1j * x[:, c - r + 1::2]) * np.exp(1j * pos[:, None] * f.astype(np.float64))
    assert np.allclose(y[:, c - r::2], z.real, atol=1e-12)
    assert np.allclose(y[:, c - r + 1::2], z.imag, atol=1e-12)
    # quarter turn of a single pair: (x0, x1) -> (-x1, x0)
    q = O.rope_rotate(np.array([[2.0, 3.0]]), np.pi / 2, np.array([1.0]))
    assert np.allclose(q, [[-3.0, 2.0]], atol=1e-15)


def test_rope_inverse_norm_and_relative_position():
    rng = np.random.default_rng(6)
    c, r = 64, 32
    f = S.rope_inv_freq(r, 160000.0)
    x, y = rng.standard_normal(c), rng.standard_normal(c)
    for p in (0, 5, 131072, 1 << 20):
        xr = O.rope_rotate(x, p, f)
        assert np.allclose(np.linalg.norm(xr), np.linalg.norm(x))
        assert np.allclose(O.rope_rotate(xr, p, f, sign=-1.0), x, atol=1e-12)
    d = [O.rope_rotate(x, p + 37, f) @ O.rope_rotate(y, p, f) for p in (0, 1000, 99999)]
    assert np.allclose(d, d[0], atol=1e-10)


# ----------------------------------------------------------------------------- indexer, top-k

def test_index_score_hand_fixture():
    g = _gold("index_score_hand.json")
    got = O.index_scores(np.array(g["qi_codes"], np.uint8), np.array(g["qi_scale"], np.float32),
                         np.array(g["wi"], np.float32), np.array(g["ki_codes"], np.uint8),
                         np.array(g["ki_scale"], np.float32), 2)
    assert np.array_equal(got, np.array(g["expect"]))
    got1 = O.index_scores(np.array(g["qi_codes"], np.uint8), np.array(g["qi_scale"], np.float32),
                          np.array(g["wi"], np.float32), np.array(g["ki_codes"], np.uint8),
                          np.array(g["ki_scale"], np.float32), 1)
    assert got1.shape == (1,) and got1[0] == 6.0


def test_index_score_brute_force_loops():
    """Brute force: Python loops over heads and dims on decoded E4M3 values."""
    rng = np.random.default_rng(7)
    HI, dI, N = 3, 8, 9
    qc = S.e4m3_normalish(rng, (HI, dI))
    kc = S.e4m3_normalish(rng, (N, dI))
    qs = rng.uniform(0.5, 2, HI).astype(np.float32)
    ks = rng.uniform(0.5, 2, N).astype(np.float32)
    w = rng.standard_normal(HI).astype(np.float32)
    tab = O.e4m3_table()
    got = O.index_scores(qc, qs, w, kc, ks, 7)
    for s in range(7):
        tot = 0.0
        for h in range(HI):
            dot = sum(float(tab[qc[h, d]]) * float(qs[h]) * float(tab[kc[s, d]]) * float(ks[s])
                      for d in range(dI))
            tot += float(w[h]) * max(dot, 0.0)
        assert abs(got[s] - tot) <= 1e-12 * (1 + abs(tot))


def test_index_score_relu_scale_folding():
    """ReLU(a x) = a ReLU(x) for a > 0: doubling a key's scale doubles its score; all-negative
    dots give exactly 0."""
    rng = np.random.default_rng(8)
    qc = S.e4m3_normalish(rng, (4, 16))
    kc = S.e4m3_normalish(rng, (20, 16))
    qs, w = np.ones(4, np.float32), rng.standard_normal(4).astype(np.float32)
    ks = np.ones(20, np.float32)
    a = O.index_scores(qc, qs, w, kc, ks, 20)
    b = O.index_scores(qc, qs, w, kc, 2 * ks, 20)
    assert np.allclose(b, 2 * a, rtol=1e-14, atol=0)
    q_pos = np.full((1, 4), 0x38, np.uint8)      # all +1
    k_neg = np.full((3, 4), 0xB8, np.uint8)      # all -1
    z = O.index_scores(q_pos, np.ones(1, np.float32), np.ones(1, np.float32), k_neg,
                       np.ones(3, np.float32), 3)
    assert np.all(z == 0.0)


def test_topk_against_sorted_with_ties():
    rng = np.random.default_rng(9)
    for n, k in ((50, 10), (10, 64), (300, 64), (1000, 999)):
        sc = rng.integers(0, 20, n).astype(np.float64)  # many ties
        got = O.topk_select(sc, k)
        ref = sorted(sorted(range(n), key=lambda i: (-sc[i], i))[:min(k, n)])
        assert list(got) == ref
    assert list(O.topk_select(np.array([]), 5)) == []
    assert list(O.topk_select(np.array([1.0, 1.0, 1.0]), 2)) == [0, 1]


# ----------------------------------------------------------------------------- attention

def _bits(x):
    return O.f64_to_bf16_bits(x)


def test_attend_without_sink_is_textbook_sdpa():
    """a_h -> -inf gives plain softmax attention: compare with torch's SDPA on the rotated
    query (float64), then the output's reverse rotation."""
    rng = np.random.default_rng(10)
    nh, c, r, n, t = 4, 64, 16, 37, 1234
    f = S.rope_inv_freq(r, 160000.0)
    qb, eb = _bits(rng.standard_normal((nh, c))), _bits(rng.standard_normal((n, c)))
    out, lse = O.attend(qb, eb, np.full(nh, -np.inf), 0.125, t, f)
    q = torch.from_numpy(O.rope_rotate(O.bf16_bits_to_f64(qb), t, f))
    e = torch.from_numpy(O.bf16_bits_to_f64(eb))
    ref = torch.nn.functional.scaled_dot_product_attention(q[None, :, None, :].transpose(1, 2)
                                                           .reshape(1, 1, nh, c),
                                                           e[None, None], e[None, None],
                                                           scale=0.125)[0, 0]
    ref = O.rope_rotate(ref.numpy(), t, f, sign=-1.0)
    assert np.allclose(out, ref, atol=1e-12)
    ref_lse = torch.logsumexp(0.125 * q @ e.T, dim=1).numpy()
    assert np.allclose(lse, ref_lse, atol=1e-12)


def test_attend_sink_closed_forms():
    """With a sink: the probabilities sum to sigma(lse - a) < 1; the output equals the sink-free
    output times that mass; a single row gets p = sigma(z - a); an explicit extra key column
    with logit a and a zero value gives the same result."""
    rng = np.random.default_rng(14)
    nh, c, r, n, t = 3, 32, 8, 11, 77
    f = S.rope_inv_freq(r, 160000.0)
    qb, eb = _bits(rng.standard_normal((nh, c))), _bits(rng.standard_normal((n, c)))
    a = rng.standard_normal(nh)
    o_s, lse = O.attend(qb, eb, a, 0.2, t, f)
    o_n, lse_n = O.attend(qb, eb, np.full(nh, -np.inf), 0.2, t, f)
    mass = 1.0 / (1.0 + np.exp(a - lse))
    assert np.all(mass < 1) and np.allclose(lse, lse_n)
    assert np.allclose(o_s, o_n * mass[:, None], atol=1e-12)
    # explicit sink column in torch
    q = torch.from_numpy(O.rope_rotate(O.bf16_bits_to_f64(qb), t, f))
    e = torch.from_numpy(O.bf16_bits_to_f64(eb))
    z = torch.cat([0.2 * q @ e.T, torch.from_numpy(a)[:, None]], dim=1)
    p = torch.softmax(z, dim=1)[:, :-1]
    ref = O.rope_rotate((p @ e).numpy(), t, f, sign=-1.0)
    assert np.allclose(o_s, ref, atol=1e-12)
    # single row: output = sigma(z - a) * row (then un-rotated)
    o1, l1 = O.attend(qb, eb[:1], a, 0.2, t, f)
    assert np.allclose(o1, O.rope_rotate(np.outer(1 / (1 + np.exp(a - l1)),
                                                  O.bf16_bits_to_f64(eb[0])), t, f, sign=-1.0))
    # empty row set: zero output (all mass on the sink)
    o0, l0 = O.attend(qb, eb[:0], a, 0.2, t, f)
    assert np.all(o0 == 0) and np.all(np.isneginf(l0))


def _dense_reference(h, W, p, q, sink, t, m, c, d_i, n_win, scale, f, eps):
    """Independent torch construction of the m=1 reading: with B^b -> -inf and m = 1 each entry
    s is RMSNorm(h_s W^a_KV) * gamma rotated at s, and CSA with k >= #entries attends over all
    entries s <= t plus the window tokens, plus the sink column."""
    H = torch.from_numpy(O.bf16_bits_to_f64(h))
    Wt = torch.from_numpy(O.bf16_bits_to_f64(W))
    P = H @ Wt.T
    Ca = P[:, :c]
    Win = P[:, 4 * c + 4 * d_i:]

    def norm_rot(x, g, pos):
        y = x / torch.sqrt((x * x).mean(-1, keepdim=True) + eps) * torch.from_numpy(g).double()
        ang = torch.from_numpy(pos).double()[:, None] * torch.from_numpy(f).double()[None]
        zc = torch.complex(y[:, c - 2 * len(f)::2], y[:, c - 2 * len(f) + 1::2]) * torch.polar(
            torch.ones_like(ang), ang)
        y = y.clone()
        y[:, c - 2 * len(f)::2] = zc.real
        y[:, c - 2 * len(f) + 1::2] = zc.imag
        return y

    T = H.shape[0]
    ent = norm_rot(Ca, p["gamma"], np.arange(T))
    win = norm_rot(Win, p["gamma_win"], np.arange(T))
    bf = lambda x: x.to(torch.bfloat16).double()
    keys = torch.cat([bf(ent[:t + 1]), bf(win[max(0, t - n_win + 1):t + 1])])
    # the query is taken as given (normalised upstream) and only rotated at t
    qq = torch.from_numpy(O.rope_rotate(O.bf16_bits_to_f64(q), t, f))
    z = torch.cat([scale * qq @ keys.T, torch.from_numpy(sink).double()[:, None]], dim=1)
    pr = torch.softmax(z, dim=1)[:, :-1]
    return O.rope_rotate((pr @ keys).numpy(), t, f, sign=-1.0)


def test_csa_layer_m1_reduces_to_dense_mqa():
    """Reading R15: m = 1, B^b -> -inf (the b-stream gets zero weight) and k >= #entries turn CSA
    into dense shared-KV MQA over every token <= t plus the 128-token window plus the sink."""
    w = S.shrink(S.WORKLOADS["tiny_csa"], m=1, c=32, r=16, n_h=4, H_I=2, d_I=16, D=48, T=40,
                 decode_steps=0, k=1000)
    x = S.layer_inputs(w)
    x["Bb"] = np.full_like(x["Bb"], -1e30)
    params = {k: x[k] for k in ("Ba", "Bb", "BIa", "BIb", "gamma", "gamma_win")}
    n_win = 8
    qs = [0, 5, 17, 39]
    comp, res = O.csa_layer(x["H"][0], x["W"], params, x["q"][0], x["qi"][0], x["qi_scale"][0],
                            x["wi"][0], x["sink"], 1, w.c, w.d_I, w.k, n_win, w.scale,
                            x["inv_freq"], 1e-6, qs)
    for t in qs:
        ref = _dense_reference(x["H"][0], x["W"], params, x["q"][0, t], x["sink"], t, 1, w.c,
                               w.d_I, n_win, w.scale, x["inv_freq"], 1e-6)
        assert len(res[t]["sel"]) == t + 1
        assert np.allclose(res[t]["out"], ref, atol=1e-10)


def test_csa_decode_rows_are_prefill_rows_and_causal():
    """Every quantity for query t depends only on tokens <= t: running the layer on a prefix
    ending at t gives the same selection and output as on the longer sequence."""
    w = S.shrink(S.WORKLOADS["tiny_csa"], c=32, r=16, n_h=2, H_I=2, d_I=16, D=32, T=60,
                 decode_steps=4, k=5)
    x = S.layer_inputs(w)
    params = {k: x[k] for k in ("Ba", "Bb", "BIa", "BIb", "gamma", "gamma_win")}
    args = lambda T: (x["H"][0, :T], x["W"], params, x["q"][0], x["qi"][0], x["qi_scale"][0],
                      x["wi"][0], x["sink"], w.m, w.c, w.d_I, w.k, 16, w.scale, x["inv_freq"],
                      1e-6)
    _, full = O.csa_layer(*args(64), queries=[30, 47, 63])
    for t in (30, 47, 63):
        _, part = O.csa_layer(*args(t + 1), queries=[t])
        assert np.array_equal(full[t]["sel"], part[t]["sel"])
        assert np.allclose(full[t]["out"], part[t]["out"], atol=1e-13)
    # early queries: t < 3 sees no closed entry, only the window and the sink
    _, early = O.csa_layer(*args(64), queries=[0, 2, 3])
    assert len(early[0]["sel"]) == 0 and len(early[2]["sel"]) == 0 and len(early[3]["sel"]) == 1


def test_hca_layer_m1_is_dense_over_tokens():
    """HCA with m' = 1 and B -> any value: each entry is the token's own normalised C row, so the
    layer is dense attention over all tokens <= t plus the window (checked against the explicit
    construction used for the CSA reduction, with the HCA column layout)."""
    w = S.shrink(S.WORKLOADS["tiny_hca"], m=1, c=32, r=16, n_h=3, D=40, T=24, decode_steps=0)
    x = S.layer_inputs(w)
    params = {k: x[k] for k in ("B", "gamma", "gamma_win")}
    comp, res = O.hca_layer(x["H"][0], x["W"], params, x["q"][0], x["sink"], 1, w.c, 6, w.scale,
                            x["inv_freq"], 1e-6, [0, 11, 23])
    P = O.project(x["H"][0], x["W"])
    ent = O.rope_rotate(O.rms_norm(P[:, :w.c], x["gamma"], 1e-6), np.arange(24), x["inv_freq"])
    win = O.rope_rotate(O.rms_norm(P[:, 2 * w.c:], x["gamma_win"], 1e-6), np.arange(24),
                        x["inv_freq"])
    for t in (0, 11, 23):
        keys = np.concatenate([ent[:t + 1], win[max(0, t - 5):t + 1]])
        keys = O.bf16_bits_to_f64(O.f64_to_bf16_bits(keys))
        q = torch.from_numpy(O.rope_rotate(O.bf16_bits_to_f64(x["q"][0, t]), t, x["inv_freq"]))
        z = torch.cat([w.scale * q @ torch.from_numpy(keys).T,
                       torch.from_numpy(x["sink"]).double()[:, None]], 1)
        ref = O.rope_rotate((torch.softmax(z, 1)[:, :-1] @ torch.from_numpy(keys)).numpy(), t,
                            x["inv_freq"], sign=-1.0)
        assert np.allclose(res[t]["out"], ref, atol=1e-10)


def test_compress_epilogue_closed_forms():
    """Entries: with gamma = 1 the un-rotated part has RMS ~1 (bf16 rounding aside) and the
    rotation preserves the norm of the RoPE slice; indexer keys decode to the pooled values
    within half an E4M3 ulp."""
    w = S.shrink(S.WORKLOADS["tiny_csa"], T=64, decode_steps=0)
    x = S.layer_inputs(w)
    params = {k: x[k] for k in ("Ba", "Bb", "BIa", "BIb", "gamma_win")}
    params["gamma"] = np.ones(w.c, np.float32)
    comp = O.compress_tokens(x["H"][0], x["W"], params, "csa", w.m, w.c, w.d_I, x["inv_freq"],
                             1e-6)
    e = O.bf16_bits_to_f64(comp["entries"])
    assert e.shape == (16, w.c)
    assert np.allclose(np.sqrt(np.mean(e * e, axis=1)), 1.0, atol=2e-3)
    pre_n = O.rms_norm(comp["pre"], np.ones(w.c), 1e-6)
    assert np.allclose(np.linalg.norm(e[:, -w.r:], axis=1), np.linalg.norm(pre_n[:, -w.r:], axis=1),
                       rtol=1e-2)
    dec = O.e4m3_decode(comp["ikeys"]) * comp["iscale"][:, None].astype(np.float64)
    big = np.abs(comp["ipre"]) > comp["iscale"][:, None] * 2.0 ** -6
    assert np.all(np.abs(dec - comp["ipre"])[big] <= np.abs(comp["ipre"])[big] * 2.0 ** -4 + 1e-12)
    # the same layer with MXFP4 keys: identical entries and pooled keys; every key element within
    # half an E2M1 step of its block-scaled value (or clamped at 6)
    c4 = O.compress_tokens(x["H"][0], x["W"], params, "csa", w.m, w.c, w.d_I, x["inv_freq"],
                           1e-6, idx_format="mxfp4")
    assert np.array_equal(c4["entries"], comp["entries"]) and np.array_equal(c4["ipre"],
                                                                             comp["ipre"])
    assert c4["ikeys"].shape == (16, w.d_I // 2) and c4["iscale"].shape == (16, w.d_I // 32)
    X = np.repeat(np.exp2(c4["iscale"].astype(np.float64) - 127), 32, axis=1)
    a = np.abs(c4["ipre"]) / X
    step = np.where(a < 2, 0.5, np.where(a < 4, 1.0, 2.0))
    err = np.abs(O.mxfp4_decode(c4["ikeys"], c4["iscale"]) - c4["ipre"]) / X
    assert np.all(err <= 0.5 * step + np.maximum(a - 6.0, 0.0) + 1e-12)


# ----------------------------------------------------------------------------- query / output
# projections: closed forms with identity and one-hot weights, exact scaling, group isolation

def _bf16(x):
    return O.f64_to_bf16_bits(np.asarray(x, dtype=np.float64))


def test_query_projections_closed_forms():
    rng = np.random.default_rng(31)
    T, D, n_h, c, H_I, d_I = 5, 64, 2, 32, 2, 32
    r_q = n_h * c                       # = 64 = D: identity down-projection possible
    h = _bf16(rng.standard_normal((T, D)))
    eye = _bf16(np.eye(D))
    w_w = _bf16(np.eye(D)[[3, 40]])    # w^I_j = h[:, 3], h[:, 40]
    w_uq = _bf16(np.eye(r_q))           # qpre = c^Q split into heads
    w_iuq = _bf16(rng.standard_normal((H_I * d_I, r_q)) / 8)
    ones = np.ones(c)
    r = O.query_projections(h, eye, w_w, w_uq, w_iuq, ones, n_h, c, H_I, d_I, 1e-6)
    hf = O.bf16_bits_to_f64(h)
    assert np.array_equal(r["cq"], h)                                   # identity W^DQ
    assert np.array_equal(r["wi"].astype(np.float64), hf[:, [3, 40]])   # one-hot W_w
    assert np.array_equal(r["qpre"], hf.reshape(T, n_h, c))             # heads in order
    q = O.bf16_bits_to_f64(r["q"])
    rms = np.sqrt(np.mean(q * q, axis=-1))
    assert np.allclose(rms, 1.0, atol=4e-3)                              # gain 1: unit RMS
    cos = np.sum(q * r["qpre"], -1) / np.linalg.norm(q, axis=-1) / np.linalg.norm(r["qpre"], axis=-1)
    assert np.all(cos > 1 - 1e-4)                                       # direction kept
    dec = O.e4m3_decode(r["qi"]) * r["qi_scale"][..., None].astype(np.float64)
    big = np.abs(r["qi_pre"]) > r["qi_scale"][..., None] * 2.0 ** -6
    assert np.all(np.abs(dec - r["qi_pre"])[big] <= np.abs(r["qi_pre"])[big] * 2.0 ** -4)
    # doubling h (exact in bf16) doubles c^Q, q^I's scales and w^I, keeps the codes and q
    r2 = O.query_projections(_bf16(2 * hf), eye, w_w, w_uq, w_iuq, ones, n_h, c, H_I, d_I, 0.0)
    r1 = O.query_projections(h, eye, w_w, w_uq, w_iuq, ones, n_h, c, H_I, d_I, 0.0)
    assert np.array_equal(O.bf16_bits_to_f64(r2["cq"]), 2 * O.bf16_bits_to_f64(r1["cq"]))
    assert np.array_equal(r2["qi"], r1["qi"]) and np.array_equal(r2["qi_scale"], 2 * r1["qi_scale"])
    assert np.array_equal(r2["q"], r1["q"]) and np.array_equal(r2["wi"], 2 * r1["wi"])


def test_grouped_output_projection_closed_forms():
    rng = np.random.default_rng(32)
    T, n_h, c, g = 3, 4, 16, 2
    width = n_h // g * c                 # 32 dims per group
    o = _bf16(rng.standard_normal((T, n_h, c)))
    of = O.bf16_bits_to_f64(o).reshape(T, -1)
    # identity blocks (r_o = width): z is O itself, concatenated in head order
    w_down = np.stack([_bf16(np.eye(width))] * g)
    w_proj = _bf16(np.eye(g * width)[[5, 40, 63]])   # y picks z columns 5, 40, 63
    z, y = O.grouped_output_projection(o, w_down, w_proj, g)
    assert np.array_equal(z, o.reshape(T, -1))
    assert np.array_equal(O.bf16_bits_to_f64(y), of[:, [5, 40, 63]])
    # random blocks: group u's z depends only on its own heads
    w_down = _bf16(rng.standard_normal((g, 8, width)) / 4)
    w_proj = _bf16(rng.standard_normal((6, g * 8)) / 4)
    z, y = O.grouped_output_projection(o, w_down, w_proj, g)
    o0 = O.bf16_bits_to_f64(o).copy()
    o0[:, n_h // g:, :] = 0.0           # silence group 1's heads
    z0, _ = O.grouped_output_projection(_bf16(o0), w_down, w_proj, g)
    assert np.array_equal(z0[:, :8], z[:, :8])
    assert np.all(O.bf16_bits_to_f64(z0[:, 8:]) == 0.0)
    # one group with identity weights is a plain projection
    z1, y1 = O.grouped_output_projection(o, _bf16(np.eye(n_h * c))[None], _bf16(np.eye(n_h * c)), 1)
    assert np.array_equal(z1, o.reshape(T, -1)) and np.array_equal(y1, z1)


# ---------------------------------------------------------------- mixed-precision entries (R22)

def test_mixed_entries_split_and_hand_values():
    """One-hot rows put their value on the right side of the split at c - r: 1.0 in the last
    non-RoPE dim is E4M3 0x38 (exponent field 7, bias 7); 1.0 in the first RoPE dim is bf16
    0x3F80.  Values past the E4M3 range saturate at 448 (0x7E), signs are kept."""
    c, r = 16, 8
    x = np.zeros((4, c))
    x[0, c - r - 1] = 1.0
    x[1, c - r] = 1.0
    x[2, 0] = 1000.0
    x[3, 1] = -0.5
    codes, rope = O.quantize_entries_mixed(x, r)
    assert codes.shape == (4, c - r) and rope.shape == (4, r)
    assert codes[0, c - r - 1] == 0x38 and np.all(rope[0] == 0)
    assert np.all(codes[1] == 0) and rope[1, 0] == 0x3F80 and np.all(rope[1, 1:] == 0)
    assert codes[2, 0] == 0x7E
    assert codes[3, 1] == 0xB0  # -0.5: sign, exponent field 6, mantissa 0


def test_mixed_entries_round_trip_on_representable_values():
    """Values that E4M3 (first dims) and bf16 (RoPE dims) hold exactly come back exactly; the
    E4M3 values are taken from the OCP point table, not from the oracle's own decoder."""
    g = _gold("e4m3_points.json")
    pts = np.array([v for _, v in g["points"]], dtype=np.float64)
    rng = np.random.default_rng(3)
    c, r = 64, 16
    x = np.empty((5, c))
    x[:, :c - r] = rng.choice(np.concatenate([pts, -pts]), size=(5, c - r))
    x[:, c - r:] = rng.integers(-128, 128, size=(5, r)) / 16.0   # 7 significant bits: exact in bf16
    codes, rope = O.quantize_entries_mixed(x, r)
    back = O.bf16_bits_to_f64(O.decode_entries_mixed(codes, rope))
    assert np.array_equal(back, x)


def test_mixed_entries_error_bound_and_compressor():
    """The compressor's mixed entries (reading R22) decode to within half an E4M3 step of the
    bf16 entries' values on the non-RoPE dims (relative 2^-4, or 2^-10 absolute below the
    normal range) and equal them on the RoPE dims."""
    w = S.WORKLOADS["tiny_csa"]
    x = S.layer_inputs(w, T=256)
    params = {k: x[k] for k in ("Ba", "Bb", "BIa", "BIb", "gamma", "gamma_win")}
    comp = O.compress_tokens(x["H"][0], x["W"], params, "csa", w.m, w.c, w.d_I, x["inv_freq"],
                             1e-6, entry_format="mixed")
    dec = O.bf16_bits_to_f64(O.decode_entries_mixed(comp["ecodes"], comp["erope"]))
    ref = O.bf16_bits_to_f64(comp["entries"])
    k = w.c - w.r
    assert np.array_equal(dec[:, k:], ref[:, k:])
    err = np.abs(dec[:, :k] - ref[:, :k])
    assert np.all(err <= np.maximum(2.0 ** -4 * np.abs(ref[:, :k]), 2.0 ** -10) * 1.01)
    assert err.max() > 0  # the quantisation is not a no-op


# ----------------------------------------------------------------------------- FP4 query, BF16 scores

def _fp4_row(byte0, d=32):
    """A packed MXFP4 row of d dims with only byte 0 (dims 0 and 1) non-zero."""
    r = np.zeros(d // 2, np.uint8)
    r[0] = byte0
    return r


def test_index_score_fp4_hand_fixture():
    g = _gold("index_score_fp4_hand.json")
    qp = np.stack([_fp4_row(b) for b in g["qi_byte0"]])
    kp = np.stack([_fp4_row(b) for b in g["ki_byte0"]])
    qs = np.array(g["qi_scale"], np.uint8)[:, None]
    ks = np.array(g["ki_scale"], np.uint8)[:, None]
    got = O.index_scores_fp4(qp, qs, np.array(g["wi"], np.float32), kp, ks, 2)
    assert np.array_equal(got, np.array(g["expect"]))


def test_index_score_fp4_brute_force_loops():
    """Brute force with an E2M1 magnitude table written out here and E8M0 scales 2^(byte-127)."""
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    rng = np.random.default_rng(41)
    HI, dI, N = 3, 64, 7
    qcodes = rng.integers(0, 16, (HI, dI))
    kcodes = rng.integers(0, 16, (N, dI))
    qsb = rng.integers(120, 132, (HI, dI // 32)).astype(np.uint8)
    ksb = rng.integers(120, 132, (N, dI // 32)).astype(np.uint8)
    pack = lambda c: (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)
    w = rng.standard_normal(HI).astype(np.float32)
    got = O.index_scores_fp4(pack(qcodes), qsb, w, pack(kcodes), ksb, 6)

    def val(code, sb):
        v = mags[code & 7] * 2.0 ** (int(sb) - 127)
        return -v if code & 8 else v
    for s in range(6):
        tot = 0.0
        for h in range(HI):
            dot = sum(val(qcodes[h, d], qsb[h, d // 32]) * val(kcodes[s, d], ksb[s, d // 32])
                      for d in range(dI))
            tot += float(w[h]) * max(dot, 0.0)
        assert abs(got[s] - tot) <= 1e-12 * (1 + abs(tot))


def test_index_scores_fp4_equals_e4m3_path_on_shared_values():
    """Queries and keys whose real values both formats hold exactly (E2M1 magnitudes times a
    power of two per 32-dim block): the FP4 x FP4 scorer, the E4M3 x MXFP4 variant and the E4M3
    scorer give identical scores."""
    rng = np.random.default_rng(42)
    H, d, N = 4, 128, 40

    def shared(rows):
        codes = rng.integers(0, 16, (rows, d)).astype(np.uint8)
        codes[:, ::32] = 7  # every block holds its largest magnitude, 6 x 2^e
        se = rng.integers(-3, 5, (rows, d // 32))
        return O.e2m1_decode(codes) * np.repeat(np.exp2(se.astype(np.float64)), 32, axis=1)
    qv, kv = shared(H), shared(N)
    qp, qs = O.quantize_rows_mxfp4(qv)
    kp, ks = O.quantize_rows_mxfp4(kv)
    assert np.array_equal(O.mxfp4_decode(qp, qs), qv) and np.array_equal(O.mxfp4_decode(kp, ks), kv)
    qe, ke = O.e4m3_encode(qv), O.e4m3_encode(kv)
    assert np.array_equal(O.e4m3_decode(qe), qv) and np.array_equal(O.e4m3_decode(ke), kv)
    wi = rng.standard_normal(H).astype(np.float32)
    one_q, one_k = np.ones(H, np.float32), np.ones(N, np.float32)
    a = O.index_scores(qe, one_q, wi, ke, one_k, N - 5)
    b = O.index_scores_mxfp4(qe, one_q, wi, kp, ks, N - 5)
    c = O.index_scores_fp4(qp, qs, wi, kp, ks, N - 5)
    assert np.array_equal(a, b) and np.array_equal(a, c)
    assert O.score_function("mxfp4", "mxfp4") is O.index_scores_fp4
    assert O.score_function("mxfp4", "e4m3") is O.index_scores_mxfp4
    assert O.score_function() is O.index_scores


def test_round_scores_bf16_hand_fixture_and_topk():
    g = _gold("bf16_scores_topk_hand.json")
    sc = np.array(g["scores"])
    r = O.round_scores_bf16(sc)
    assert np.array_equal(r, np.array(g["rounded"]))
    assert list(O.topk_select(r, g["k"])) == g["expect_bf16"]
    assert list(O.topk_select(sc, g["k"])) == g["expect_full"]


def test_round_scores_bf16_against_torch_and_order():
    """float32 inputs (one rounding step, so torch's conversion is a single RNE too), exact
    bf16 values kept, monotone non-decreasing."""
    rng = np.random.default_rng(43)
    x = (rng.standard_normal(20000) * 10.0 ** rng.integers(-6, 6, 20000)).astype(np.float32)
    got = O.round_scores_bf16(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(got, ref)
    assert np.array_equal(O.round_scores_bf16(got), got)
    srt = np.sort(x.astype(np.float64))
    assert np.all(np.diff(O.round_scores_bf16(srt)) >= 0)


def test_csa_query_bf16_scores_select_on_rounded_values():
    """csa_query with BF16 scores: the selection is the top-k of the rounded scores with the
    lower index winning ties (brute force with Python's sorted)."""
    rng = np.random.default_rng(44)
    w = S.shrink(S.WORKLOADS["tiny_csa"])
    x = S.decode_cache_inputs(w, B=1, N=400)
    t = 4 * 400
    r = O.csa_query(t, x["q"][0, 0], x["qi"][0, 0], x["qi_scale"][0, 0], x["wi"][0, 0], x["sink"],
                    x["entries"][0], x["ikeys"][0], x["iscale"][0], 400, x["window"][0],
                    lambda u: u % w.n_win, w.m, w.k, w.n_win, w.scale, x["inv_freq"],
                    score_format="bf16")
    full = O.index_scores(x["qi"][0, 0], x["qi_scale"][0, 0], x["wi"][0, 0], x["ikeys"][0],
                          x["iscale"][0], 400)
    rounded = O.round_scores_bf16(full)
    assert np.array_equal(r["scores"], rounded)
    ref = sorted(sorted(range(400), key=lambda i: (-rounded[i], i))[:w.k])
    assert list(r["sel"]) == ref
    assert len(np.unique(rounded)) < 400  # bf16 rounding does create ties here
    del rng


def test_query_projections_mxfp4_query():
    """qi_format "mxfp4": the indexer query is the MXFP4 quantisation of the same pre-quantised
    values, each element within half an E2M1 step (times its block scale) of them, or clamped
    at 6 times the block scale."""
    rng = np.random.default_rng(45)
    T, D, n_h, c, H_I, d_I = 4, 64, 2, 32, 2, 64
    r_q = 64
    bf = lambda a: O.f64_to_bf16_bits(a)
    h = bf(rng.standard_normal((T, D)))
    w_dq = bf(rng.standard_normal((r_q, D)) / 8)
    w_w = bf(rng.standard_normal((H_I, D)) / 8)
    w_uq = bf(rng.standard_normal((n_h * c, r_q)) / 8)
    w_iuq = bf(rng.standard_normal((H_I * d_I, r_q)) / 8)
    a = O.query_projections(h, w_dq, w_w, w_uq, w_iuq, np.ones(c), n_h, c, H_I, d_I, 1e-6)
    b = O.query_projections(h, w_dq, w_w, w_uq, w_iuq, np.ones(c), n_h, c, H_I, d_I, 1e-6,
                            qi_format="mxfp4")
    assert np.array_equal(a["qi_pre"], b["qi_pre"]) and np.array_equal(a["q"], b["q"])
    assert b["qi"].shape == (T, H_I, d_I // 2) and b["qi_scale"].shape == (T, H_I, d_I // 32)
    p, sc = O.quantize_rows_mxfp4(b["qi_pre"])
    assert np.array_equal(p, b["qi"]) and np.array_equal(sc, b["qi_scale"])
    dec = O.mxfp4_decode(b["qi"], b["qi_scale"])
    X = np.repeat(np.exp2(b["qi_scale"].astype(np.float64) - 127), 32, axis=-1)
    y = b["qi_pre"] / X
    step = np.where(np.abs(y) < 2, 0.5, np.where(np.abs(y) < 4, 1.0, 2.0))
    clamp = np.maximum(np.abs(y) - 6.0, 0.0)  # a block's largest values may saturate at 6
    assert np.all(np.abs(dec - b["qi_pre"]) / X <= 0.5 * step + clamp + 1e-12)
