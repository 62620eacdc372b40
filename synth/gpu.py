"""Full-size seeded inputs generated on the GPU with torch, for timing runs.

Same recipe as synth.inputs (bf16 = normal draws truncated to their upper 16 bits; E4M3 codes
assembled from sign/exponent of a normal draw plus uniform mantissa bits; uniform scales),
drawn from torch's device generator instead of numpy PCG64 so that gigabyte-sized workloads
are produced in milliseconds: the benchmark times them, and the full-size parity tests check
the kernels on them against the oracle (fed host copies of the same tensors).
"""
import torch

from .inputs import MXFP4_MAG_P, rope_inv_freq, weight_cols


def _gen(seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def bf16_normal(g, shape, device, std=1.0, chunk=1 << 26):
    n = 1
    for s in shape:
        n *= s
    out = torch.empty(n, dtype=torch.int16, device=device)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        x = torch.randn(e - s, generator=g, device=device, dtype=torch.float32)
        if std != 1.0:
            x *= std
        out[s:e] = (x.view(torch.int32) >> 16).to(torch.int16)
    return out.view(*shape)


def e4m3_normalish(g, shape, device, chunk=1 << 26):
    n = 1
    for s in shape:
        n *= s
    out = torch.empty(n, dtype=torch.uint8, device=device)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        x = torch.randn(e - s, generator=g, device=device, dtype=torch.float32)
        _, ex = torch.frexp(x)
        field = torch.clamp(ex + 6, 0, 14).to(torch.int32)
        mant = torch.randint(0, 8, (e - s,), generator=g, device=device, dtype=torch.int32)
        sign = (x < 0).to(torch.int32)
        out[s:e] = ((sign << 7) | (field << 3) | mant).to(torch.uint8)
    return out.view(*shape)


def _uniform(g, shape, device, lo, hi):
    return torch.rand(*shape, generator=g, device=device) * (hi - lo) + lo


def mxfp4_normalish(g, rows_shape, d, device, chunk=1 << 24):
    """As synth.inputs.mxfp4_normalish, on the device (magnitude codes by inverse CDF)."""
    n = 1
    for s in rows_shape:
        n *= s
    cdf = torch.cumsum(torch.tensor(MXFP4_MAG_P, dtype=torch.float32, device=device), 0)
    packed = torch.empty((n, d // 2), dtype=torch.uint8, device=device)
    for s in range(0, n, chunk // d):
        e = min(n, s + chunk // d)
        u = torch.rand((e - s, d), generator=g, device=device)
        mag = torch.clamp(torch.searchsorted(cdf, u), max=7).to(torch.int32)
        sign = torch.randint(0, 2, (e - s, d), generator=g, device=device, dtype=torch.int32)
        codes = mag | (sign << 3)
        packed[s:e] = (codes[:, 0::2] | (codes[:, 1::2] << 4)).to(torch.uint8)
    scales = torch.full((n, 4), 127, dtype=torch.uint8, device=device)
    scales[:, :d // 32] = torch.randint(121, 126, (n, d // 32), generator=g, device=device,
                                        dtype=torch.int32).to(torch.uint8)
    return packed.view(*rows_shape, d // 2), scales.view(*rows_shape, 4)


def mixed_entries(g, shape, c, r, device):
    """Entry rows of c + r bytes: c - r E4M3 codes (as e4m3_normalish) then r bf16 values
    (N(0,1)), the mixed-precision entry layout."""
    codes = e4m3_normalish(g, tuple(shape) + (c - r,), device)
    rope = bf16_normal(g, tuple(shape) + (r,), device).contiguous().view(torch.uint8)
    return torch.cat([codes, rope], dim=-1).contiguous()


def decode_cache_inputs(w, device="cuda", seed=None, key_fmt="e4m3", entry_fmt="bf16",
                        qi_fmt="e4m3"):
    """As synth.inputs.decode_cache_inputs, on the device (entry_fmt "mixed": entries as
    mixed_entries rows)."""
    g = _gen(w.seed if seed is None else seed, device)
    B, N = w.B, w.N
    out = {"B": B, "N": N}
    if entry_fmt == "mixed":
        out["entries"] = mixed_entries(g, (B, N), w.c, w.r, device)
    else:
        out["entries"] = bf16_normal(g, (B, N, w.c), device)
    if w.mode == "csa" and key_fmt == "mxfp4":
        out["ikeys"], out["iscale"] = mxfp4_normalish(g, (B, N), w.d_I, device)
    elif w.mode == "csa":
        out["ikeys"] = e4m3_normalish(g, (B, N, w.d_I), device)
        out["iscale"] = _uniform(g, (B, N), device, 0.5, 1.5) / 16
    out["window"] = bf16_normal(g, (B, w.n_win, w.c), device)
    out["inv_freq"] = torch.from_numpy(rope_inv_freq(w.r, w.rope_base)).to(device)
    out["pos"] = torch.full((B,), w.t, dtype=torch.int32, device=device)
    out["n_entries"] = torch.full((B,), N, dtype=torch.int32, device=device)
    _queries(g, w, 1, out, device, qi_fmt)
    return out


def _queries(g, w, nq, out, device, qi_fmt="e4m3"):
    out["q"] = bf16_normal(g, (w.B, nq, w.n_h, w.c), device)
    if w.mode == "csa":
        if qi_fmt == "mxfp4":
            out["qi"], out["qi_scale"] = mxfp4_normalish(g, (w.B, nq, w.H_I), w.d_I, device)
        else:
            out["qi"] = e4m3_normalish(g, (w.B, nq, w.H_I, w.d_I), device)
            out["qi_scale"] = _uniform(g, (w.B, nq, w.H_I), device, 0.5, 1.5) / 16
        out["wi"] = torch.randn(w.B, nq, w.H_I, generator=g, device=device) / 8
    if w.sink is None:
        out["sink"] = torch.randn(w.n_h, generator=g, device=device)
    else:
        out["sink"] = torch.full((w.n_h,), w.sink, device=device)


def layer_inputs(w, device="cuda", seed=None, qi_fmt="e4m3"):
    """As synth.inputs.layer_inputs (prefill of w.T tokens, no decode tokens), on the device."""
    g = _gen(w.seed if seed is None else seed, device)
    T = w.T
    out = {"T": T, "T_total": T}
    out["H"] = bf16_normal(g, (w.B, T, w.D), device)
    out["W"] = bf16_normal(g, (weight_cols(w), w.D), device, std=1.0 / w.D ** 0.5)
    if w.mode == "csa":
        for k, width in (("Ba", w.c), ("Bb", w.c), ("BIa", w.d_I), ("BIb", w.d_I)):
            out[k] = torch.randn(w.m, width, generator=g, device=device)
    else:
        out["B"] = torch.randn(w.m, w.c, generator=g, device=device)
    out["gamma"] = 1.0 + 0.1 * torch.randn(w.c, generator=g, device=device)
    out["gamma_win"] = 1.0 + 0.1 * torch.randn(w.c, generator=g, device=device)
    out["inv_freq"] = torch.from_numpy(rope_inv_freq(w.r, w.rope_base)).to(device)
    _queries(g, w, T, out, device, qi_fmt)
    return out
