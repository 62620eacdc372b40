"""Workload shapes and seeded input generators (see the package docstring)."""
from dataclasses import dataclass, replace

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    mode: str              # "csa" or "hca"
    B: int                 # sequences
    m: int                 # compression ratio (4 CSA, 128 HCA)
    c: int                 # entry width d_h
    r: int                 # RoPE dims (trailing)
    n_h: int               # query heads
    n_win: int = 128
    k: int = 0             # top-k (CSA)
    H_I: int = 0           # indexer heads
    d_I: int = 0           # indexer dim
    D: int = 0             # hidden size (compressor input), 0 = no compressor in the workload
    T: int = 0             # prefill tokens (layer workloads)
    decode_steps: int = 0  # decode steps after the prefill (layer workloads)
    N: int = 0             # resident entries per sequence (decode-cache workloads)
    t: int = 0             # query position of the decode step (decode-cache workloads)
    sink: float = None     # constant sink logit; None = N(0,1) per head
    rope_base: float = 160000.0
    seed: int = 0

    @property
    def scale(self):
        return float(1.0 / np.sqrt(self.c))


# The five workloads: a tiny whole layer (prefill 2048 + 16 decode steps), CSA decode at 128K
# and 1M context, HCA dense decode at 1M context, and a 64K-token CSA prefill; and a chunk of a
# 1M-token prompt's chunked prefill.
WORKLOADS = {
    "tiny_csa": Workload("tiny_csa", "csa", B=1, m=4, c=128, r=64, n_h=8, k=64, H_I=4, d_I=64,
                         D=512, T=2048, decode_steps=16, sink=0.5, seed=0),
    "tiny_hca": Workload("tiny_hca", "hca", B=1, m=128, c=128, r=64, n_h=8, D=512, T=2048,
                         decode_steps=16, sink=0.5, seed=1),
    "csa_decode_128k": Workload("csa_decode_128k", "csa", B=32, m=4, c=512, r=64, n_h=64, k=512,
                                H_I=64, d_I=128, N=32768, t=131072, seed=2),
    "csa_decode_1m": Workload("csa_decode_1m", "csa", B=4, m=4, c=512, r=64, n_h=128, k=2048,
                              H_I=64, d_I=128, N=262144, t=1 << 20, seed=3),
    "hca_decode_1m": Workload("hca_decode_1m", "hca", B=16, m=128, c=512, r=64, n_h=128,
                              N=8192, t=1 << 20, seed=4),
    "csa_prefill_64k": Workload("csa_prefill_64k", "csa", B=1, m=4, c=512, r=64, n_h=64, k=512,
                                H_I=64, d_I=128, D=4096, T=65536, seed=5),
    # one chunk of a long prompt's chunked prefill: T = 4096 new tokens at positions t..t+T-1
    # (t = 2^20 - 4096, the last chunk of a 1M-token prompt) over a cache of N = 262144 entries
    # of which the first t/m are closed
    "csa_prefill_1m_chunk": Workload("csa_prefill_1m_chunk", "csa", B=1, m=4, c=512, r=64,
                                     n_h=64, k=512, H_I=64, d_I=128, D=4096, T=4096, N=262144,
                                     t=(1 << 20) - 4096, seed=6),
}


def shrink(w, **kw):
    """A smaller variant of a workload (same structure), for parity tests."""
    return replace(w, **kw)


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def bf16_normal(rng, shape, std=1.0, chunk=1 << 24):
    """bf16 bit patterns of N(0, std^2) draws (float32 draw, upper 16 bits kept)."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        x = rng.standard_normal(e - s, dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        out[s:e] = (x.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    return out.reshape(shape)


def e4m3_normalish(rng, shape, chunk=1 << 24):
    """E4M3 code bytes whose magnitudes follow N(0,1) to within a binade.

    sign = sign of a normal draw x; exponent field = clip(E + 6, 0, 14) where |x| lies in
    [2^(E-1), 2^E); mantissa = 3 uniform random bits.
    """
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint8)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        x = rng.standard_normal(e - s, dtype=np.float32)
        _, ex = np.frexp(x)
        field = np.clip(ex.astype(np.int32) + 6, 0, 14).astype(np.uint8)
        mant = rng.integers(0, 8, size=e - s, dtype=np.uint8)
        sign = (x < 0).astype(np.uint8)
        out[s:e] = (sign << 7) | (field << 3) | mant
    return out.reshape(shape)


def rope_inv_freq(r, base):
    """The RoPE inverse-frequency table base^(-2i/r), i < r/2, as float32."""
    return (base ** (-(np.arange(0, r, 2, dtype=np.float64) / r))).astype(np.float32)


def weight_cols(w):
    """Columns of the concatenated compressor weight (see the ABI header for the order)."""
    if w.mode == "csa":
        return 5 * w.c + 4 * w.d_I
    return 3 * w.c


def tail_shape(w):
    """(rows, cols) of the per-sequence compressor tail ring."""
    if w.mode == "csa":
        return 2 * w.m, 4 * w.c + 4 * w.d_I
    return w.m, 2 * w.c


def _queries(rng, w, nq, out, qi_fmt="e4m3"):
    out["q"] = bf16_normal(rng, (w.B, nq, w.n_h, w.c))
    if w.mode == "csa":
        if qi_fmt == "mxfp4":  # packed codes [.., H_I, d_I/2] and 4 E8M0 bytes per head
            out["qi"], out["qi_scale"] = mxfp4_normalish(rng, (w.B, nq, w.H_I), w.d_I)
        else:
            out["qi"] = e4m3_normalish(rng, (w.B, nq, w.H_I, w.d_I))
            out["qi_scale"] = rng.uniform(0.5, 1.5, size=(w.B, nq, w.H_I)).astype(np.float32) / 16
        out["wi"] = (rng.standard_normal((w.B, nq, w.H_I), dtype=np.float32) / 8)
    if w.sink is None:
        out["sink"] = rng.standard_normal(w.n_h, dtype=np.float32)
    else:
        out["sink"] = np.full(w.n_h, w.sink, dtype=np.float32)


def layer_inputs(w, seed=None, T=None, qi_fmt="e4m3"):
    """Inputs of a whole layer run from hidden states: prefill of T tokens (default w.T) plus
    w.decode_steps decode tokens.  Arrays are indexed [B, token, ...]; the compressor weight is
    [cols, D] (one row per output column)."""
    rng = _rng(w.seed if seed is None else seed)
    T = w.T if T is None else T
    tt = T + w.decode_steps
    out = {"T": T, "T_total": tt}
    out["H"] = bf16_normal(rng, (w.B, tt, w.D))
    out["W"] = bf16_normal(rng, (weight_cols(w), w.D), std=1.0 / np.sqrt(w.D))
    if w.mode == "csa":
        out["Ba"] = rng.standard_normal((w.m, w.c), dtype=np.float32)
        out["Bb"] = rng.standard_normal((w.m, w.c), dtype=np.float32)
        out["BIa"] = rng.standard_normal((w.m, w.d_I), dtype=np.float32)
        out["BIb"] = rng.standard_normal((w.m, w.d_I), dtype=np.float32)
    else:
        out["B"] = rng.standard_normal((w.m, w.c), dtype=np.float32)
    out["gamma"] = (1.0 + 0.1 * rng.standard_normal(w.c)).astype(np.float32)
    out["gamma_win"] = (1.0 + 0.1 * rng.standard_normal(w.c)).astype(np.float32)
    out["inv_freq"] = rope_inv_freq(w.r, w.rope_base)
    _queries(rng, w, tt, out, qi_fmt)
    return out


# E2M1 magnitude codes 0..7 in the proportions an N(0,1) block quantised with its shared
# exponent would show (small magnitudes likelier, 6 rare)
MXFP4_MAG_P = np.array([0.10, 0.19, 0.17, 0.15, 0.17, 0.13, 0.07, 0.02])


def mxfp4_normalish(rng, rows_shape, d):
    """Packed MXFP4 rows of d dims: E2M1 codes (sign uniform, magnitude code drawn from
    MXFP4_MAG_P), two per byte with the even dim in the low nibble -> uint8 [..., d/2]; and
    4 E8M0 scale bytes per row, uniform in 121..125 for the d/32 blocks, 127 for unused bytes
    -> uint8 [..., 4].  No value is quantised here: the codes are drawn directly."""
    n = int(np.prod(rows_shape))
    mag = rng.choice(8, size=(n, d), p=MXFP4_MAG_P).astype(np.uint8)
    sign = rng.integers(0, 2, size=(n, d), dtype=np.uint8) << np.uint8(3)
    codes = mag | sign
    packed = (codes[:, 0::2] | (codes[:, 1::2] << np.uint8(4))).astype(np.uint8)
    scales = np.full((n, 4), 127, dtype=np.uint8)
    scales[:, :d // 32] = rng.integers(121, 126, size=(n, d // 32), dtype=np.uint8)
    return packed.reshape(tuple(rows_shape) + (d // 2,)), scales.reshape(tuple(rows_shape) + (4,))


def decode_cache_inputs(w, seed=None, B=None, N=None, key_fmt="e4m3", qi_fmt="e4m3"):
    """Inputs of one decode step over a resident cache: N entries per sequence (bf16 ~N(0,1)),
    indexer keys (CSA: E4M3 with per-entry scales, or MXFP4 with key_fmt "mxfp4"), a 128-row
    window ring (token u in row u mod 128) and one query per sequence at position w.t (the
    indexer query E4M3 with a scale per head, or MXFP4 with qi_fmt "mxfp4")."""
    rng = _rng(w.seed if seed is None else seed)
    B = w.B if B is None else B
    N = w.N if N is None else N
    w = replace(w, B=B, N=N)
    out = {"N": N, "B": B}
    out["entries"] = bf16_normal(rng, (B, N, w.c))
    if w.mode == "csa" and key_fmt == "mxfp4":
        out["ikeys"], out["iscale"] = mxfp4_normalish(rng, (B, N), w.d_I)
    elif w.mode == "csa":
        out["ikeys"] = e4m3_normalish(rng, (B, N, w.d_I))
        out["iscale"] = rng.uniform(0.5, 1.5, size=(B, N)).astype(np.float32) / 16
    out["window"] = bf16_normal(rng, (B, w.n_win, w.c))
    out["inv_freq"] = rope_inv_freq(w.r, w.rope_base)
    out["pos"] = np.full(B, w.t, dtype=np.int32)
    out["n_entries"] = np.full(B, N, dtype=np.int32)
    _queries(rng, w, 1, out, qi_fmt)
    return out
