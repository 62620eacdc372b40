#!/usr/bin/env python3
"""Benchmark of the CSA/HCA hot path on one MI355X.

Default workload (the metric's headline): CSA decode, batch 32, 128K context (32768 compressed
bf16 entries of 512 dims per sequence, last 64 rotated), 64 query heads sharing one K=V head,
indexer 64 heads x 128 dims with E4M3 keys, top-k 512, 128-token window, per-head sink.  A step
is one csa_decode call (indexer scoring + exact top-k + sparse MQA over the selected entries and
the window, with the sink) for all 32 sequences, inputs resident in HBM.

Timing: W untimed warm-up steps, then exactly K steps between two HIP events on the stream the
library launches on, synchronised on both sides (their mean gives the value); then K more steps
with an event before each, for the median, p10 and p90 of single steps.  Consecutive steps
cycle through --rotate independent copies of the cache so that no step finds its working set
(~164 MB) in the 256 MB Infinity Cache.  A further, profiled pass of K steps brackets every
kernel launch with HIP events (csa_profile_start/stop) to get the dominant kernel's average
duration for the roofline.

Also measured (one entry each under "also"): CSA decode at 1M context (B=4, 262144 entries, 128
heads, k=2048), HCA dense decode at 1M context (B=16, 8192 entries, 128 heads), the 64K-token
CSA prefill, variants of these with MXFP4 indexer keys ("_mxfp4": E4M3 query), with the pages'
FP4 indexer QK path ("_fp4q": MXFP4 query and keys), with BF16 index scores ("_bf16s"), with
the block cache layout ("_paged") and with mixed-precision entries ("_mixed"), and the
query-side and grouped output projections of the 64K-token prefill.  Each line carries the CPU
oracle timed on a bounded sample of its own workload.

Prints ONE JSON line.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "CSA decode tokens/s & HBM GB/s at 128K-1M ctx; prefill tokens/s (1 GPU)"
HBM_PEAK_GBS = 8000.0         # MI355X HBM3E, GB/s
FP8_PEAK_TFLOPS = 5000.0      # MI355X dense fp8 MFMA
FP4_PEAK_TFLOPS = 10100.0     # MI355X dense fp4 MFMA
BF16_PEAK_TFLOPS = 2500.0     # MI355X dense bf16 MFMA

DEFAULT_EXTRA = ",".join([
    "csa_decode_1m", "hca_decode_1m", "csa_prefill_64k",
    "csa_decode_128k_fp4q", "csa_decode_1m_fp4q", "csa_prefill_64k_fp4q",
    "csa_decode_128k_bf16s", "csa_decode_1m_fp4q_bf16s", "csa_prefill_64k_fp4q_bf16s",
    "csa_decode_128k_mxfp4", "csa_decode_1m_mxfp4", "csa_prefill_64k_mxfp4",
    "qo_proj_64k",
    "csa_decode_128k_paged", "csa_decode_1m_paged", "hca_decode_1m_paged",
    "csa_decode_128k_mixed", "csa_decode_1m_mixed", "hca_decode_1m_mixed",
    "csa_prefill_64k_chunk8k", "csa_prefill_1m_chunk",
])
FLAGS = ("mxfp4", "fp4q", "bf16s", "paged", "mixed", "chunk8k")

# source files whose hash a committed counter summary records, per kernel
KERNEL_SOURCES = {"index_score": ("index.hip", "index_common.h", "common.h", "kernels.h"),
                  "mqa_dense": ("mqa.hip", "mqa_hb.hip", "mqa_common.h", "common.h",
                                "kernels.h"),
                  "mqa_sparse": ("mqa.hip", "mqa_hb.hip", "mqa_common.h", "common.h",
                                 "kernels.h"),
                  "all_projections": ("proj.hip", "compress.hip", "common.h", "kernels.h")}


def parse_name(name):
    """Workload name -> (base workload, set of variant flags)."""
    from synth import inputs as S
    for base in sorted(S.WORKLOADS, key=len, reverse=True):
        if name == base or name.startswith(base + "_"):
            flags = set(f for f in name[len(base):].split("_") if f)
            bad = flags - set(FLAGS)
            if bad:
                raise SystemExit("unknown workload variant(s) %s in %s" % (sorted(bad), name))
            return base, flags
    if name.startswith("qo_proj"):
        return name, set()
    raise SystemExit("unknown workload %s" % name)


def formats(flags):
    """(key format, query format, bf16 scores) of a variant."""
    key = "mxfp4" if ("mxfp4" in flags or "fp4q" in flags) else "e4m3"
    q = "mxfp4" if "fp4q" in flags else "e4m3"
    return key, q, "bf16s" in flags


def _key_bytes(w, key_fmt):
    """Indexer-key bytes per entry: E4M3 codes + an fp32 scale, or MXFP4 codes (two per byte)
    + the 4-byte word of E8M0 block scales."""
    return (w.d_I // 2 if key_fmt == "mxfp4" else w.d_I) + 4


def _query_bytes(w, q_fmt):
    """Indexer-query bytes per token: codes + the 4-byte scale word + the fp32 head weight."""
    return w.H_I * ((w.d_I // 2 if q_fmt == "mxfp4" else w.d_I) + 8)


def _decode_bytes(w, n_vis, key_fmt="e4m3", q_fmt="e4m3", mixed=False):
    """Algorithmic HBM bytes of one decode token (what the method must move): indexer keys and
    their scales over the visible entries, the top-k gathered entries (CSA) or every visible
    entry (HCA), the window rows, the query and the output, the indexer query.  Mixed entries
    take c + r bytes (E4M3 unrotated dims, bf16 RoPE dims) instead of 2c."""
    c2 = w.c * 2
    e2 = w.c + w.r if mixed else c2
    b = w.n_win * c2 + 2 * w.n_h * c2
    if w.mode == "csa":
        b += n_vis * _key_bytes(w, key_fmt) + min(w.k, n_vis) * e2 + _query_bytes(w, q_fmt)
    else:
        b += n_vis * e2
    return b


def _score_kernel_bytes(w, n_vis, key_fmt="e4m3", q_fmt="e4m3"):
    """Algorithmic bytes of one indexer-scoring launch per sequence: keys + scales + query."""
    return n_vis * _key_bytes(w, key_fmt) + _query_bytes(w, q_fmt)


def _source_hash(kernel):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "long_context_sparse_15_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _profiled_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter summary
    (profiles/<kernel>_<workload>_counters.md: FETCH_SIZE and WRITE_SIZE scaled by a plain-copy
    calibration), or None when there is none or the kernel sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", "%s_%s_counters.md" % (kernel, workload))
    if not os.path.exists(path) or kernel not in KERNEL_SOURCES:
        return None
    vals = {}
    for line in open(path):
        if ":" in line and line.startswith("    "):
            k, v = line.strip().split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("source_sha256") != _source_hash(kernel) or vals.get("kernel") != kernel:
        return None
    return int(vals["traffic_bytes_per_launch"])


def _pct(xs, q):
    s = sorted(xs)
    i = min(len(s) - 1, max(0, int(round(q * (len(s) - 1)))))
    return s[i]


def _time_steps(step, K, W, stream):
    """W warm-up steps; then exactly K steps between two events (synchronised on both sides),
    whose mean is the measurement; then K more steps with an event before each and one after
    the last, for the spread of single steps (the events between steps add a little time of
    their own, so these are kept apart from the mean).
    Returns (mean ms per step of the first K, [ms of each step of the second K])."""
    import torch
    for i in range(W):
        step(i)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(K):
        step(W + i)
    t1.record(stream)
    torch.cuda.synchronize()
    mean = t0.elapsed_time(t1) / K
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    for i in range(K):
        ev[i].record(stream)
        step(W + K + i)
    ev[K].record(stream)
    torch.cuda.synchronize()
    return mean, [ev[i].elapsed_time(ev[i + 1]) for i in range(K)]


def _step_stats(per):
    return {"median": _pct(per, 0.5), "p10": _pct(per, 0.1), "p90": _pct(per, 0.9),
            "min": min(per), "max": max(per)}


def _profiled(step, K, W):
    import torch
    import long_context_sparse_15_amd as csa
    torch.cuda.synchronize()
    csa.profile_start()
    for i in range(K):
        step(W + 2 * K + i)
    torch.cuda.synchronize()
    return csa.profile_stop()


def _kernel_roofline(prof, kname, work, bound, peak, unit, workload):
    """Roofline entry of kernel kname: algorithmic work per launch / its average event-timed
    launch duration, against `peak`; traffic from the committed counter summary (or None)."""
    launches, tot = prof[kname]
    kdur = tot / launches
    ach = work / (kdur / 1e3) / (1e9 if unit == "GB/s" else 1e12)
    r = {"kernel": kname, "bound": bound, "achieved": ach, "peak": peak, "unit": unit,
         "frac": ach / peak, "traffic": _profiled_traffic(kname, workload),
         "avg_launch_ms": kdur}
    r["bytes_per_launch" if unit == "GB/s" else "flops_per_launch"] = work
    return r


def decode_workload(name, K, W, rotate):
    """One decode step per iteration of a named decode workload and its variants."""
    import torch
    import long_context_sparse_15_amd as csa
    from synth import inputs as S
    from synth import gpu as G

    base, flags = parse_name(name)
    key_fmt, q_fmt, bf16s = formats(flags)
    paged, mixed = "paged" in flags, "mixed" in flags
    w = S.WORKLOADS[base]
    dev = "cuda"
    x = G.decode_cache_inputs(w, dev, key_fmt=key_fmt, qi_fmt=q_fmt,
                              entry_fmt="mixed" if mixed else "bf16")
    heavy = ["entries", "window"] + (["ikeys", "iscale"] if w.mode == "csa" else [])
    copies = [x]
    for r in range(1, rotate):
        y = dict(x)
        for k in heavy:
            y[k] = x[k].clone()
        copies.append(y)
    fmt = {"e4m3": csa.IDX_E4M3, "mxfp4": csa.IDX_MXFP4}
    cfg = csa.make_config(csa.MODE_CSA if w.mode == "csa" else csa.MODE_HCA, w.m, w.n_h, w.c,
                          w.r, x["inv_freq"], top_k=w.k, n_win=w.n_win, idx_heads=w.H_I,
                          idx_dim=w.d_I, softmax_scale=w.scale, idx_key_format=fmt[key_fmt],
                          idx_query_format=fmt[q_fmt],
                          score_format=csa.SCORE_BF16 if bf16s else csa.SCORE_FP32,
                          entry_format=csa.ENT_MIXED if mixed else csa.ENT_BF16)
    pg = {}
    if paged:
        be = 128 // w.m
        n_blocks = w.B * (w.N // be)
        gen = torch.Generator().manual_seed(w.seed)
        table = torch.randperm(n_blocks, generator=gen).view(w.B, w.N // be).to(torch.int32)
        table = table.to(dev)
        rows = (table.long()[:, :, None] * be + torch.arange(be, device=dev)).reshape(-1)
        for y in copies:
            for k in ("entries", "ikeys", "iscale"):
                if k in y:
                    pool = torch.empty((n_blocks * be,) + tuple(y[k].shape[2:]), dtype=y[k].dtype,
                                       device=dev)
                    pool[rows] = y[k].reshape((-1,) + tuple(y[k].shape[2:]))
                    y[k] = pool
        pg = dict(block_table=table, block_entries=be, n_blocks=n_blocks)
    caches = [csa.make_cache(w.N, w.n_win, y["entries"], y["window"], y["n_entries"],
                             idx_keys=y.get("ikeys"), idx_scale=y.get("iscale"), **pg)
              for y in copies]
    ws = torch.empty(csa.workspace_size(cfg, csa.OP_DECODE, w.B, 1, w.N), dtype=torch.uint8,
                     device=dev)
    out = torch.empty((w.B, w.n_h, w.c), dtype=torch.bfloat16, device=dev)
    q = x["q"][:, 0].contiguous()
    stream = torch.cuda.current_stream()

    def step(i):
        y = copies[i % rotate]
        if w.mode == "csa":
            csa.decode(cfg, caches[i % rotate], y["pos"], q, y["sink"], out, ws, qi=y["qi"],
                       qi_scale=y["qi_scale"], wi=y["wi"])
        else:
            csa.decode(cfg, caches[i % rotate], y["pos"], q, y["sink"], out, ws)

    ms, per = _time_steps(step, K, W, stream)
    prof = _profiled(step, K, W)
    n_vis = min(w.N, (w.t + 1) // w.m)
    step_bytes = w.B * _decode_bytes(w, n_vis, key_fmt, q_fmt, mixed)
    res = {"workload": name, "value": w.B / (ms / 1e3), "unit": "tokens/s", "ms_per_step": ms,
           "step_ms": _step_stats(per),
           "hbm_gbs": step_bytes / (ms / 1e3) / 1e9,
           "hbm_frac": step_bytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS,
           "kernels_ms_per_step": {k: v[1] / K for k, v in prof.items()}}
    if w.mode == "csa":
        kname, kbytes = "index_score", w.B * _score_kernel_bytes(w, n_vis, key_fmt, q_fmt)
    else:
        kname = "mqa_dense"
        kbytes = w.B * (n_vis * (w.c + w.r if mixed else 2 * w.c) + w.n_win * w.c * 2 +
                        2 * w.n_h * w.c * 2)
    res["roofline"] = _kernel_roofline(prof, kname, kbytes, "hbm", HBM_PEAK_GBS, "GB/s", name)
    del copies, caches, ws
    torch.cuda.empty_cache()
    return res


def prefill_flops(w):
    """Algorithmic FLOPs of the 64K prefill: compressor projections, causal indexer, sparse +
    window attention."""
    T, B = w.T, w.B
    n_max = T // w.m
    n_cols = 5 * w.c + 4 * w.d_I
    f_comp = 2.0 * B * T * w.D * n_cols
    pairs = sum(min(n_max, (t + 1) // w.m) for t in range(T))
    f_idx = 2.0 * B * pairs * w.H_I * w.d_I
    visits = sum(min(w.k, min(n_max, (t + 1) // w.m)) + min(w.n_win, t + 1) for t in range(T))
    f_mqa = 4.0 * B * visits * w.n_h * w.c
    return f_comp, f_idx, f_mqa


def prefill_workload(name, K, W):
    """The whole prefill (compressor, causal indexer, top-k, sparse MQA) of a named workload and
    its key/query/score-format variants."""
    import torch
    import long_context_sparse_15_amd as csa
    from synth import inputs as S
    from synth import gpu as G

    base, flags = parse_name(name)
    key_fmt, q_fmt, bf16s = formats(flags)
    w = S.WORKLOADS[base]
    dev = "cuda"
    x = G.layer_inputs(w, dev, qi_fmt=q_fmt)
    T, B = w.T, w.B
    n_max = T // w.m
    fmt = {"e4m3": csa.IDX_E4M3, "mxfp4": csa.IDX_MXFP4}
    cfg = csa.make_config(csa.MODE_CSA, w.m, w.n_h, w.c, w.r, x["inv_freq"], top_k=w.k,
                          n_win=w.n_win, idx_heads=w.H_I, idx_dim=w.d_I, hidden=w.D,
                          softmax_scale=w.scale, idx_key_format=fmt[key_fmt],
                          idx_query_format=fmt[q_fmt],
                          score_format=csa.SCORE_BF16 if bf16s else csa.SCORE_FP32)
    tr, tc = csa.tail_shape(cfg)
    mx = key_fmt == "mxfp4"
    ct = dict(entries=torch.zeros((B, n_max, w.c), dtype=torch.int16, device=dev),
              window=torch.zeros((B, T, w.c), dtype=torch.int16, device=dev),
              n_entries=torch.zeros(B, dtype=torch.int32, device=dev),
              tail=torch.zeros((B, tr, tc), dtype=torch.float32, device=dev),
              idx_keys=torch.zeros((B, n_max, w.d_I // 2 if mx else w.d_I), dtype=torch.uint8,
                                   device=dev),
              idx_scale=torch.zeros((B, n_max), dtype=torch.float32, device=dev))
    cache = csa.make_cache(n_max, T, **ct)
    weights = csa.make_weights(x["W"], x["Ba"], x["gamma"], x["gamma_win"], bias_b=x["Bb"],
                               bias_ia=x["BIa"], bias_ib=x["BIb"])
    ws = torch.empty(csa.workspace_size(cfg, csa.OP_PREFILL, B, T, n_max), dtype=torch.uint8,
                     device=dev)
    out = torch.empty((B, T, w.n_h, w.c), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()
    # "chunk8k": the same prompt as consecutive csa_prefill calls of 8192 tokens, each chunk
    # continuing the cache at its start position (the first from position 0)
    chunk = 8192 if "chunk8k" in flags else T
    parts = []
    for c0 in range(0, T, chunk):
        sl = slice(c0, c0 + chunk)
        parts.append(dict(H=x["H"][:, sl].contiguous(), q=x["q"][:, sl].contiguous(),
                          out=out[:, sl], qi=x["qi"][:, sl].contiguous(),
                          qi_scale=x["qi_scale"][:, sl].contiguous(),
                          wi=x["wi"][:, sl].contiguous(),
                          pos0=None if c0 == 0 else
                          torch.full((B,), c0, dtype=torch.int32, device=dev)))

    def step(i):
        for pt in parts:
            csa.prefill(cfg, pt["H"], weights, cache, pt["q"], x["sink"], pt["out"], ws,
                        qi=pt["qi"], qi_scale=pt["qi_scale"], wi=pt["wi"], pos0=pt["pos0"])

    ms, per = _time_steps(step, K, W, stream)
    prof = _profiled(step, K, W)
    f_comp, f_idx, f_mqa = prefill_flops(w)
    idx_peak = FP4_PEAK_TFLOPS if q_fmt == "mxfp4" else FP8_PEAK_TFLOPS
    ideal_ms = (f_comp / (BF16_PEAK_TFLOPS * 1e12) + f_idx / (idx_peak * 1e12) +
                f_mqa / (BF16_PEAK_TFLOPS * 1e12)) * 1e3
    res = {"workload": name, "value": B * T / (ms / 1e3), "unit": "tokens/s", "ms_per_step": ms,
           "step_ms": _step_stats(per), "mfma_roofline_frac": ideal_ms / ms,
           "kernels_ms_per_step": {k: v[1] / K for k, v in prof.items()},
           # the dominant kernel: sparse + window attention, a bf16 MFMA contraction
           "roofline": _kernel_roofline(prof, "mqa_sparse", f_mqa / len(parts), "mfma",
                                        BF16_PEAK_TFLOPS, "TFLOP/s", name),
           # the indexer against its own MFMA peak (fp8, or fp4 for the FP4 query path)
           "indexer_roofline": _kernel_roofline(prof, "index_score", f_idx / len(parts), "mfma",
                                                idx_peak, "TFLOP/s", name)}
    if len(parts) > 1:
        res["chunks"] = {"tokens": chunk, "calls_per_step": len(parts),
                         "work_per_launch": "the step's flops / calls (an average chunk)"}
    del x, ws, out, ct, cache, parts
    torch.cuda.empty_cache()
    return res


def chunk_flops(w):
    """Algorithmic FLOPs of one chunk of a chunked prefill (T tokens at positions t..t+T-1):
    compressor projections of the chunk, the indexer of every chunk query over its visible
    entries, sparse + window attention."""
    n_cols = 5 * w.c + 4 * w.d_I
    f_comp = 2.0 * w.B * w.T * w.D * n_cols
    vis = [min(w.N, (u + 1) // w.m) for u in range(w.t, w.t + w.T)]
    f_idx = 2.0 * w.B * sum(vis) * w.H_I * w.d_I
    f_mqa = 4.0 * w.B * sum(min(w.k, v) + w.n_win for v in vis) * w.n_h * w.c
    return f_comp, f_idx, f_mqa


def chunk_workload(name, K, W):
    """One chunk of a long prompt's chunked prefill: csa_prefill of T tokens continuing a
    sequence at position t over a cache whose first t/m entries are closed (synthetic entries,
    keys, window rows and compressor tail stand for the earlier chunks).  Each step first
    restores the entry count to t/m (a one-element fill) so that every step writes the chunk's
    entries anew."""
    import torch
    import long_context_sparse_15_amd as csa
    from synth import inputs as S
    from synth import gpu as G

    base, flags = parse_name(name)
    w = S.WORKLOADS[base]
    dev = "cuda"
    x = G.layer_inputs(w, dev)
    xc = G.decode_cache_inputs(S.shrink(w, B=1), dev)
    B, T, N = w.B, w.T, w.N
    cfg = csa.make_config(csa.MODE_CSA, w.m, w.n_h, w.c, w.r, x["inv_freq"], top_k=w.k,
                          n_win=w.n_win, idx_heads=w.H_I, idx_dim=w.d_I, hidden=w.D,
                          softmax_scale=w.scale)
    tr, tc = csa.tail_shape(cfg)
    slots = 1 << (T + w.n_win - 1 - 1).bit_length()  # >= T + n_win - 1
    g = torch.Generator(device=dev)
    g.manual_seed(w.seed + 100)
    n_pre = w.t // w.m
    ne = torch.full((B,), n_pre, dtype=torch.int32, device=dev)
    ct = dict(entries=xc["entries"], idx_keys=xc["ikeys"], idx_scale=xc["iscale"],
              window=G.bf16_normal(g, (B, slots, w.c), dev), n_entries=ne,
              tail=torch.randn((B, tr, tc), generator=g, device=dev))
    cache = csa.make_cache(N, slots, **ct)
    weights = csa.make_weights(x["W"], x["Ba"], x["gamma"], x["gamma_win"], bias_b=x["Bb"],
                               bias_ia=x["BIa"], bias_ib=x["BIb"])
    ws = torch.empty(csa.workspace_size(cfg, csa.OP_PREFILL, B, T, N), dtype=torch.uint8,
                     device=dev)
    out = torch.empty((B, T, w.n_h, w.c), dtype=torch.bfloat16, device=dev)
    pos0 = torch.full((B,), w.t, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()

    def step(i):
        ne.fill_(n_pre)
        csa.prefill(cfg, x["H"], weights, cache, x["q"], x["sink"], out, ws, qi=x["qi"],
                    qi_scale=x["qi_scale"], wi=x["wi"], pos0=pos0)

    ms, per = _time_steps(step, K, W, stream)
    prof = _profiled(step, K, W)
    f_comp, f_idx, f_mqa = chunk_flops(w)
    res = {"workload": name, "value": B * T / (ms / 1e3), "unit": "tokens/s", "ms_per_step": ms,
           "step_ms": _step_stats(per), "context": w.t + T,
           "kernels_ms_per_step": {k: v[1] / K for k, v in prof.items()},
           # the dominant kernel at this context: the indexer over every visible entry
           "roofline": _kernel_roofline(prof, "index_score", f_idx, "mfma", FP8_PEAK_TFLOPS,
                                        "TFLOP/s", name),
           "attention_roofline": _kernel_roofline(prof, "mqa_sparse", f_mqa, "mfma",
                                                  BF16_PEAK_TFLOPS, "TFLOP/s", name)}
    del x, xc, ws, out, ct, cache
    torch.cuda.empty_cache()
    return res


def proj_workload(name, K, W):
    """Query-side projections and grouped output projection of the 64K-token prefill at the
    V4-Flash shape (hidden 4096, r_q 1024, 64 heads x 512, indexer 64 x 128, 8 groups of rank
    1024): one csa_query_proj and one csa_output_proj per step."""
    import torch
    import long_context_sparse_15_amd as csa
    from synth import inputs as S
    from synth import gpu as G

    w = S.WORKLOADS["csa_prefill_64k"]
    dev = "cuda"
    T, D, n_h, c, H_I, d_I, r_q, g, r_o = w.T, w.D, w.n_h, w.c, w.H_I, w.d_I, 1024, 8, 1024
    gen = G._gen(w.seed + 100, dev)
    H = G.bf16_normal(gen, (1, T, D), dev)
    Oatt = G.bf16_normal(gen, (1, T, n_h, c), dev)
    wq = csa.make_qproj_weights(G.bf16_normal(gen, (r_q, D), dev, std=D ** -0.5),
                                G.bf16_normal(gen, (n_h * c, r_q), dev, std=r_q ** -0.5),
                                torch.ones(c, device=dev),
                                w_w=G.bf16_normal(gen, (H_I, D), dev, std=D ** -0.5),
                                w_iuq=G.bf16_normal(gen, (H_I * d_I, r_q), dev, std=r_q ** -0.5))
    width = n_h // g * c
    wo = csa.make_oproj_weights(G.bf16_normal(gen, (g, r_o, width), dev, std=width ** -0.5),
                                G.bf16_normal(gen, (D, g * r_o), dev, std=(g * r_o) ** -0.5))
    inv = torch.from_numpy(S.rope_inv_freq(w.r, w.rope_base)).to(dev)
    cfg = csa.make_config(csa.MODE_CSA, w.m, n_h, c, w.r, inv, top_k=w.k, idx_heads=H_I,
                          idx_dim=d_I, hidden=D, q_rank=r_q, out_groups=g, out_rank=r_o)
    q = torch.empty((1, T, n_h, c), dtype=torch.int16, device=dev)
    qi = torch.empty((1, T, H_I, d_I), dtype=torch.uint8, device=dev)
    qs = torch.empty((1, T, H_I), dtype=torch.float32, device=dev)
    wi = torch.empty((1, T, H_I), dtype=torch.float32, device=dev)
    y = torch.empty((1, T, D), dtype=torch.int16, device=dev)
    ws = torch.empty(max(csa.workspace_size(cfg, csa.OP_QUERY_PROJ, 1, T, 1),
                         csa.workspace_size(cfg, csa.OP_OUTPUT_PROJ, 1, T, 1)),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step(i):
        csa.query_proj(cfg, H, wq, q, ws, qi_out=qi, qi_scale_out=qs, wi_out=wi)
        csa.output_proj(cfg, Oatt, wo, y, ws)

    ms, per = _time_steps(step, K, W, stream)
    prof = _profiled(step, K, W)
    flops = proj_flops(T, D, r_q, H_I, n_h, c, d_I, g, r_o)
    ach = flops / (ms / 1e3) / 1e12
    res = {"workload": name, "value": T / (ms / 1e3), "unit": "tokens/s", "ms_per_step": ms,
           "step_ms": _step_stats(per),
           "kernels_ms_per_step": {k: v[1] / K for k, v in prof.items()},
           # every launch of the step together (six GEMM shapes and the finish pass); traffic is
           # the step's HBM bytes
           "roofline": {"kernel": "all_projections", "bound": "mfma", "achieved": ach,
                        "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                        "frac": ach / BF16_PEAK_TFLOPS,
                        "traffic": _profiled_traffic("all_projections", name),
                        "flops_per_step": flops}}
    del H, Oatt, q, qi, qs, wi, y, ws, wq, wo
    torch.cuda.empty_cache()
    return res


def proj_flops(T, D, r_q, H_I, n_h, c, d_I, g, r_o):
    return 2.0 * T * (D * (r_q + H_I) + r_q * (n_h * c + H_I * d_I) + n_h * c * r_o + g * r_o * D)


# ----------------------------------------------------------------------------- CPU oracle

def _host_info():
    import numpy as np  # noqa: F401  (BLAS pools exist once numpy is loaded)
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return threads, model


def _cpu_decode(name, budget_s):
    """Oracle decode steps of the workload: a step is B tokens (the GPU step's batch) over two
    distinct sampled sequences of the workload, alternately; median of 3 steps (fewer when one
    step exceeds the budget)."""
    import numpy as np
    import oracle as O
    from synth import inputs as S
    base, flags = parse_name(name)
    key_fmt, q_fmt, bf16s = formats(flags)
    w = S.WORKLOADS[base]
    x = S.decode_cache_inputs(w, B=2, key_fmt=key_fmt, qi_fmt=q_fmt)
    nb = w.d_I // 32 if w.mode == "csa" else 0
    steps = []
    for _ in range(3):
        t0 = time.time()
        for j in range(w.B):
            b = j % 2
            t = int(x["pos"][b])
            if w.mode == "csa":
                qs = x["qi_scale"][b, 0][:, :nb] if q_fmt == "mxfp4" else x["qi_scale"][b, 0]
                ks = x["iscale"][b][:, :nb] if key_fmt == "mxfp4" else x["iscale"][b]
                O.csa_query(t, x["q"][b, 0], x["qi"][b, 0], qs, x["wi"][b, 0], x["sink"],
                            x["entries"][b], x["ikeys"][b], ks, w.N, x["window"][b],
                            lambda u: u % w.n_win, w.m, w.k, w.n_win, w.scale, x["inv_freq"],
                            idx_format=key_fmt, qi_format=q_fmt,
                            score_format="bf16" if bf16s else "fp32")
            else:
                O.hca_query(t, x["q"][b, 0], x["sink"], x["entries"][b], w.N, x["window"][b],
                            lambda u: u % w.n_win, w.m, w.n_win, w.scale, x["inv_freq"])
        steps.append(time.time() - t0)
        if sum(steps) > budget_s:
            break
    med = float(np.median(steps))
    return {"value": w.B / med, "unit": "tokens/s", "kind": "oracle",
            "sample": "median of %d oracle decode steps of %d tokens (2 distinct sequences of the "
                      "%s workload, %s keys, %s query, %s scores): %s s"
                      % (len(steps), w.B, base, key_fmt, q_fmt, "bf16" if bf16s else "fp32",
                         ", ".join("%.2f" % s for s in steps))}


def _cpu_prefill(name):
    """The 64K prefill, extrapolated from bounded samples: the compressor on 1024 tokens
    (x T/1024), and indexer + top-k + attention on 32 query positions spread evenly over 0..T-1
    over a resident synthetic cache of the T/m entries (x T/32, the cost of a query growing with
    its position)."""
    import numpy as np
    import oracle as O
    from synth import inputs as S
    base, flags = parse_name(name)
    key_fmt, q_fmt, bf16s = formats(flags)
    w = S.WORKLOADS[base]
    Tc = 1024
    xl = S.layer_inputs(S.shrink(w, decode_steps=0), T=Tc, qi_fmt=q_fmt)
    params = {k: xl[k] for k in ("Ba", "Bb", "BIa", "BIb", "gamma", "gamma_win")}
    t0 = time.time()
    O.compress_tokens(xl["H"][0], xl["W"], params, "csa", w.m, w.c, w.d_I, xl["inv_freq"], 1e-6,
                      idx_format=key_fmt)
    t_comp = (time.time() - t0) * (w.T / Tc)
    n_max = w.T // w.m
    x = S.decode_cache_inputs(S.shrink(w, N=n_max, t=w.T - 1), B=1, key_fmt=key_fmt,
                              qi_fmt=q_fmt)
    win = S.bf16_normal(np.random.default_rng(1), (w.T, w.c))
    nb = w.d_I // 32
    qs = x["qi_scale"][0, 0][:, :nb] if q_fmt == "mxfp4" else x["qi_scale"][0, 0]
    ks = x["iscale"][0][:, :nb] if key_fmt == "mxfp4" else x["iscale"][0]
    n_q = 32
    t0 = time.time()
    for t in np.linspace(0, w.T - 1, n_q).astype(int):
        O.csa_query(int(t), x["q"][0, 0], x["qi"][0, 0], qs, x["wi"][0, 0], x["sink"],
                    x["entries"][0], x["ikeys"][0], ks, n_max, win, lambda u: u, w.m, w.k,
                    w.n_win, w.scale, x["inv_freq"], idx_format=key_fmt, qi_format=q_fmt,
                    score_format="bf16" if bf16s else "fp32")
    t_q = (time.time() - t0) * (w.T / n_q)
    total = t_comp + t_q
    return {"value": w.B * w.T / total, "unit": "tokens/s", "kind": "oracle",
            "sample": "extrapolated, not run whole: compressor timed on %d tokens (x%d: %.1f s), "
                      "indexer + top-k + attention on %d query positions spread over 0..%d "
                      "(x%d: %.1f s); %s keys, %s query, %s scores"
                      % (Tc, w.T // Tc, t_comp, n_q, w.T - 1, w.T // n_q, t_q, key_fmt, q_fmt,
                         "bf16" if bf16s else "fp32")}


def _cpu_chunk(name):
    """A chunk of a 1M-token prompt, extrapolated from bounded samples: the compressor on 1024
    of its tokens (x T/1024), indexer + top-k + attention on 4 of its query positions over a
    synthetic cache of N entries (x T/4; every query of the chunk sees about the same number of
    entries)."""
    import numpy as np
    import oracle as O
    from synth import inputs as S
    base, _ = parse_name(name)
    w = S.WORKLOADS[base]
    Tc = 1024
    xl = S.layer_inputs(S.shrink(w, decode_steps=0), T=Tc)
    params = {k: xl[k] for k in ("Ba", "Bb", "BIa", "BIb", "gamma", "gamma_win")}
    t0 = time.time()
    O.compress_tokens(xl["H"][0], xl["W"], params, "csa", w.m, w.c, w.d_I, xl["inv_freq"], 1e-6)
    t_comp = (time.time() - t0) * (w.T / Tc)
    x = S.decode_cache_inputs(S.shrink(w, t=w.t + w.T - 1), B=1)
    win = S.bf16_normal(np.random.default_rng(1), (w.n_win, w.c))
    n_q = 4
    t0 = time.time()
    for t in np.linspace(w.t, w.t + w.T - 1, n_q).astype(int):
        O.csa_query(int(t), x["q"][0, 0], x["qi"][0, 0], x["qi_scale"][0, 0], x["wi"][0, 0],
                    x["sink"], x["entries"][0], x["ikeys"][0], x["iscale"][0], w.N, win,
                    lambda u: u % w.n_win, w.m, w.k, w.n_win, w.scale, x["inv_freq"])
    t_q = (time.time() - t0) * (w.T / n_q)
    total = t_comp + t_q
    return {"value": w.B * w.T / total, "unit": "tokens/s", "kind": "oracle",
            "sample": "extrapolated, not run whole: compressor timed on %d tokens (x%d: %.1f s), "
                      "indexer + top-k + attention on %d query positions of the chunk over %d "
                      "entries (x%d: %.1f s)" % (Tc, w.T // Tc, t_comp, n_q, w.N, w.T // n_q, t_q)}


def _cpu_proj():
    """Query-side and output projections at the 64K prefill's shape, timed on 512 tokens and
    extrapolated (x128): every product is per token."""
    import numpy as np
    import oracle as O
    from synth import inputs as S
    w = S.WORKLOADS["csa_prefill_64k"]
    T, D, n_h, c, H_I, d_I, r_q, g, r_o = 512, w.D, w.n_h, w.c, w.H_I, w.d_I, 1024, 8, 1024
    rng = np.random.default_rng(3)
    bf = lambda shape, std: S.bf16_normal(rng, shape, std)
    h = bf((T, D), 1.0)
    t0 = time.time()
    O.query_projections(h, bf((r_q, D), D ** -0.5), bf((H_I, D), D ** -0.5),
                        bf((n_h * c, r_q), r_q ** -0.5), bf((H_I * d_I, r_q), r_q ** -0.5),
                        np.ones(c), n_h, c, H_I, d_I, 1e-6)
    width = n_h // g * c
    O.grouped_output_projection(bf((T, n_h, c), 1.0), bf((g, r_o, width), width ** -0.5),
                                bf((D, g * r_o), (g * r_o) ** -0.5), g)
    el = (time.time() - t0) * (w.T / T)
    return {"value": w.T / el, "unit": "tokens/s", "kind": "oracle",
            "sample": "extrapolated: query and output projections timed on %d tokens (x%d)"
                      % (T, w.T // T)}


_CPU_CACHE = {}


def cpu_baseline(name, budget_s=12.0):
    """The CPU oracle as it stands, on a bounded sample of the workload `name` (host cores; the
    thread count is what the BLAS pool actually uses).  The block layout and the mixed entry
    format are invisible to the oracle, which computes the same attention on the same values:
    those lines reuse their base workload's oracle timing, as does a prefill taken in chunks."""
    threads, model = _host_info()
    base, flags = parse_name(name)
    layout_only = flags & {"paged", "mixed", "chunk8k"}
    key = base + "".join("_" + f for f in sorted(flags - {"paged", "mixed", "chunk8k"}))
    if key not in _CPU_CACHE:
        if base.startswith("qo_proj"):
            r = _cpu_proj()
        elif base.startswith("csa_prefill_1m_chunk"):
            r = _cpu_chunk(key)
        elif base.startswith("csa_prefill"):
            r = _cpu_prefill(key)
        else:
            r = _cpu_decode(key, budget_s)
        _CPU_CACHE[key] = r
    r = dict(_CPU_CACHE[key])
    if layout_only:
        names = {"paged": "block layout", "mixed": "mixed entry format",
                 "chunk8k": "chunking (the same tokens in one pass)"}
        r["sample"] = "the %s oracle timing (the oracle has no %s): %s" % (
            key, " / ".join(names[f] for f in sorted(layout_only)), r["sample"])
    r["cores"] = threads
    r["cpu_model"] = model
    return r


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="csa_decode_128k")
    ap.add_argument("--extra", default=DEFAULT_EXTRA,
                    help="comma-separated extra workloads ('' for none)")
    ap.add_argument("--prefill-steps", type=int, default=10)
    ap.add_argument("--rotate", type=int, default=4)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--calib-copy", type=int, default=0,
                    help="also run N plain 1 GiB device copies (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import long_context_sparse_15_amd as csa
    csa.lib()  # fails loudly if the HIP library is missing
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(3)

    def run(name, head=False):
        print("[bench] %s%s" % ("" if head else "extra ", name), file=sys.stderr, flush=True)
        if name.startswith("csa_prefill_1m_chunk"):
            return chunk_workload(name, args.prefill_steps, max(1, args.prefill_steps // 5))
        if name.startswith("csa_prefill"):
            return prefill_workload(name, args.prefill_steps, max(1, args.prefill_steps // 5))
        if name.startswith("qo_proj"):
            return proj_workload(name, args.prefill_steps, max(1, args.prefill_steps // 5))
        return decode_workload(name, args.steps, args.warmup, args.rotate)

    head = run(args.workload, head=True)
    also = [run(n) for n in args.extra.split(",") if n]
    if args.calib_copy:
        src = torch.empty(1 << 29, dtype=torch.int16, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(args.calib_copy):
            dst.copy_(src)
        torch.cuda.synchronize()
    cpu = None
    if not args.no_cpu:
        print("[bench] cpu oracle baselines", file=sys.stderr, flush=True)
        cpu = cpu_baseline(args.workload)
        for a in also:
            print("[bench] cpu oracle %s" % a["workload"], file=sys.stderr, flush=True)
            a["cpu_baseline"] = cpu_baseline(a["workload"])

    from synth import inputs as S
    base, flags = parse_name(args.workload)
    w = S.WORKLOADS.get(base, S.WORKLOADS["csa_prefill_64k"])  # the projections: that shape
    key_fmt, q_fmt, bf16s = formats(flags)
    line = {
        "metric": METRIC, "value": head["value"], "unit": head["unit"], "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": head["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8+bf16", "data": "synthetic",
        "config": {"workload": args.workload, "batch": w.B, "context": w.t, "entries": w.N,
                   "heads": w.n_h, "head_dim": w.c,
                   "indexer": "%dx%d %s keys, %s query, %s scores" % (
                       w.H_I, w.d_I, key_fmt, q_fmt, "bf16" if bf16s else "fp32"),
                   "top_k": w.k, "window": w.n_win},
        "step_ms": head.get("step_ms"),
        "hbm_gbs": head.get("hbm_gbs"), "hbm_frac": head.get("hbm_frac"),
        "roofline": head["roofline"], "cpu_baseline": cpu,
        "kernels_ms_per_step": head["kernels_ms_per_step"], "also": also,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
