#!/usr/bin/env python3
"""Benchmark of the CSA/HCA hot path on one MI355X.

Default workload (the metric's headline): CSA decode, batch 32, 128K context (32768 compressed
bf16 entries of 512 dims per sequence, last 64 rotated), 64 query heads sharing one K=V head,
indexer 64 heads x 128 dims with E4M3 keys, top-k 512, 128-token window, per-head sink.  A step
is one csa_decode call (indexer scoring + exact top-k + sparse MQA over the selected entries and
the window, with the sink) for all 32 sequences, inputs resident in HBM.

Timing: W untimed warm-up steps, then exactly K steps between two HIP events on the stream the
library launches on, synchronised on both sides.  Consecutive steps cycle through --rotate
independent copies of the cache so that no step finds its working set (~164 MB) in the 256 MB
Infinity Cache.  A second, profiled pass of K steps brackets every kernel launch with HIP events
(csa_profile_start/stop) to get the dominant kernel's average duration for the roofline.

Also measured (one line, under "also"): CSA decode at 1M context (B=4, 262144 entries, 128
heads, k=2048), HCA dense decode at 1M context (B=16, 8192 entries, 128 heads), the 64K-token
CSA prefill, the 128K / 1M decodes and the prefill again with MXFP4 indexer keys (E2M1 codes
with an E8M0 scale per 32 dims instead of E4M3 codes with a per-entry fp32 scale), and the
query-side and grouped output projections of the 64K-token prefill.  The CPU oracle is timed on
a bounded sample of the headline workload.

Prints ONE JSON line.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "CSA decode tokens/s & HBM GB/s at 128K-1M ctx; prefill tokens/s (1 GPU)"
HBM_PEAK_GBS = 8000.0         # MI355X HBM3E, GB/s
FP8_PEAK_TFLOPS = 5000.0      # MI355X dense fp8 MFMA
BF16_PEAK_TFLOPS = 2500.0     # MI355X dense bf16 MFMA


def _key_bytes(w, key_fmt):
    """Indexer-key bytes per entry: E4M3 codes + an fp32 scale, or MXFP4 codes (two per byte)
    + the 4-byte word of E8M0 block scales."""
    return (w.d_I // 2 if key_fmt == "mxfp4" else w.d_I) + 4


def _decode_bytes(w, n_vis, key_fmt="e4m3", mixed=False):
    """Algorithmic HBM bytes of one decode token (what the method must move): indexer keys and
    their scales over the visible entries, the top-k gathered entries (CSA) or every visible
    entry (HCA), the window rows, the query and the output, the indexer query.  Mixed entries
    take c + r bytes (E4M3 unrotated dims, bf16 RoPE dims) instead of 2c."""
    c2 = w.c * 2
    e2 = w.c + w.r if mixed else c2
    b = w.n_win * c2 + 2 * w.n_h * c2
    if w.mode == "csa":
        b += n_vis * _key_bytes(w, key_fmt) + min(w.k, n_vis) * e2 + w.H_I * (w.d_I + 8)
    else:
        b += n_vis * e2
    return b


def _score_kernel_bytes(w, n_vis, key_fmt="e4m3"):
    """Algorithmic bytes of one indexer-scoring launch per sequence: keys + scales + query."""
    return n_vis * _key_bytes(w, key_fmt) + w.H_I * (w.d_I + 8)


def _profiled_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter summary
    (profiles/<kernel>_<workload>_counters.txt: FETCH_SIZE and WRITE_SIZE scaled by a plain-copy
    calibration), or None when there is none or the kernel sources changed since it was taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "%s_%s_counters.txt" % (kernel, workload))
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line:
            k, v = line.strip().split(":", 1)
            vals[k.strip()] = v.strip()
    h = hashlib.sha256()
    for f in ("index.hip", "common.h", "kernels.h"):
        with open(os.path.join(ROOT, "long_context_sparse_15_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    if vals.get("source_sha256") != h.hexdigest() or vals.get("kernel") != kernel:
        return None
    return int(vals["traffic_bytes_per_launch"])


def _time_steps(step, K, W, stream):
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
    return t0.elapsed_time(t1) / K


def _profiled(step, K, W):
    import torch
    import long_context_sparse_15_amd as csa
    torch.cuda.synchronize()
    csa.profile_start()
    for i in range(K):
        step(W + K + i)
    torch.cuda.synchronize()
    return csa.profile_stop()


def decode_workload(name, K, W, rotate):
    """One decode step per iteration of a named workload; a "_mxfp4" suffix runs the same
    workload with MXFP4 indexer keys (the E4M3 keys are the configured default), a "_paged"
    suffix with the entries, keys and scales in block pools (blocks of 128 tokens, 128/m
    entries) placed in a random order and addressed through a block table."""
    import torch
    import long_context_sparse_15_amd as csa
    from synth import inputs as S
    from synth import gpu as G

    key_fmt = "mxfp4" if "_mxfp4" in name else "e4m3"
    paged = "_paged" in name
    mixed = "_mixed" in name
    base = name.replace("_paged", "").replace("_mxfp4", "").replace("_mixed", "")
    w = S.WORKLOADS[base]
    dev = "cuda"
    x = G.decode_cache_inputs(w, dev, key_fmt=key_fmt, entry_fmt="mixed" if mixed else "bf16")
    heavy = ["entries", "window"] + (["ikeys", "iscale"] if w.mode == "csa" else [])
    copies = [x]
    for r in range(1, rotate):
        y = dict(x)
        for k in heavy:
            y[k] = x[k].clone()
        copies.append(y)
    cfg = csa.make_config(csa.MODE_CSA if w.mode == "csa" else csa.MODE_HCA, w.m, w.n_h, w.c,
                          w.r, x["inv_freq"], top_k=w.k, n_win=w.n_win, idx_heads=w.H_I,
                          idx_dim=w.d_I, softmax_scale=w.scale,
                          idx_key_format=csa.IDX_MXFP4 if key_fmt == "mxfp4" else csa.IDX_E4M3,
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

    ms = _time_steps(step, K, W, stream)
    prof = _profiled(step, K, W)
    n_vis = min(w.N, (w.t + 1) // w.m)
    step_bytes = w.B * _decode_bytes(w, n_vis, key_fmt, mixed)
    res = {"workload": name, "value": w.B / (ms / 1e3), "unit": "tokens/s", "ms_per_step": ms,
           "hbm_gbs": step_bytes / (ms / 1e3) / 1e9,
           "hbm_frac": step_bytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS,
           "kernels_ms_per_step": {k: v[1] / K for k, v in prof.items()}}
    if w.mode == "csa":
        kname = "index_score"
        kbytes = w.B * _score_kernel_bytes(w, n_vis, key_fmt)
    else:
        kname = "mqa_dense"
        kbytes = w.B * (n_vis * (w.c + w.r if mixed else 2 * w.c) + w.n_win * w.c * 2 +
                        2 * w.n_h * w.c * 2)
    launches, tot = prof[kname]
    kdur = tot / launches
    ach = kbytes / (kdur / 1e3) / 1e9
    traffic = (_profiled_traffic(kname, name) if kname == "index_score" and key_fmt == "e4m3"
               else None)
    res["roofline"] = {"kernel": kname, "bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS,
                       "unit": "GB/s", "frac": ach / HBM_PEAK_GBS, "traffic": traffic,
                       "bytes_per_launch": kbytes, "avg_launch_ms": kdur}
    del copies, caches, ws
    torch.cuda.empty_cache()
    return res


def prefill_workload(name, K, W):
    """The whole prefill (compressor, causal indexer, top-k, sparse MQA) of a named workload; a
    "_mxfp4" suffix has the compressor write MXFP4 indexer keys."""
    import torch
    import long_context_sparse_15_amd as csa
    from synth import inputs as S
    from synth import gpu as G

    mx = name.endswith("_mxfp4")
    w = S.WORKLOADS[name[:-len("_mxfp4")] if mx else name]
    dev = "cuda"
    x = G.layer_inputs(w, dev)
    T, B = w.T, w.B
    n_max = T // w.m
    cfg = csa.make_config(csa.MODE_CSA, w.m, w.n_h, w.c, w.r, x["inv_freq"], top_k=w.k,
                          n_win=w.n_win, idx_heads=w.H_I, idx_dim=w.d_I, hidden=w.D,
                          softmax_scale=w.scale,
                          idx_key_format=csa.IDX_MXFP4 if mx else csa.IDX_E4M3)
    tr, tc = csa.tail_shape(cfg)
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

    def step(i):
        csa.prefill(cfg, x["H"], weights, cache, x["q"], x["sink"], out, ws, qi=x["qi"],
                    qi_scale=x["qi_scale"], wi=x["wi"])

    ms = _time_steps(step, K, W, stream)
    prof = _profiled(step, K, W)
    # algorithmic FLOPs: compressor projections, causal indexer, sparse + window attention
    n_cols = 5 * w.c + 4 * w.d_I
    f_comp = 2.0 * B * T * w.D * n_cols
    pairs = sum(min(n_max, (t + 1) // w.m) for t in range(T))
    f_idx = 2.0 * B * pairs * w.H_I * w.d_I
    visits = sum(min(w.k, min(n_max, (t + 1) // w.m)) + min(w.n_win, t + 1) for t in range(T))
    f_mqa = 4.0 * B * visits * w.n_h * w.c
    ideal_ms = (f_comp / (BF16_PEAK_TFLOPS * 1e12) + f_idx / (FP8_PEAK_TFLOPS * 1e12) +
                f_mqa / (BF16_PEAK_TFLOPS * 1e12)) * 1e3
    k_idx = prof.get("index_score", (1, float("nan")))
    idx_ms = k_idx[1] / k_idx[0]
    ach = f_idx / (idx_ms / 1e3) / 1e12
    res = {"workload": name, "value": B * T / (ms / 1e3), "unit": "tokens/s", "ms_per_step": ms,
           "mfma_roofline_frac": ideal_ms / ms,
           "kernels_ms_per_step": {k: v[1] / K for k, v in prof.items()},
           "roofline": {"kernel": "index_score", "bound": "mfma", "achieved": ach,
                        "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                        "frac": ach / FP8_PEAK_TFLOPS, "traffic": None,
                        "flops_per_launch": f_idx, "avg_launch_ms": idx_ms}}
    del x, ws, out, ct, cache
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

    ms = _time_steps(step, K, W, stream)
    prof = _profiled(step, K, W)
    flops = 2.0 * T * (D * (r_q + H_I) + r_q * (n_h * c + H_I * d_I) + n_h * c * r_o +
                       g * r_o * D)
    ach = flops / (ms / 1e3) / 1e12
    res = {"workload": name, "value": T / (ms / 1e3), "unit": "tokens/s", "ms_per_step": ms,
           "kernels_ms_per_step": {k: v[1] / K for k, v in prof.items()},
           "roofline": {"kernel": "all projections", "bound": "mfma", "achieved": ach,
                        "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                        "frac": ach / BF16_PEAK_TFLOPS, "traffic": None, "flops_per_step": flops}}
    del H, Oatt, q, qi, qs, wi, y, ws, wq, wo
    torch.cuda.empty_cache()
    return res


def cpu_baseline(name, budget_s=10.0):
    """The CPU oracle on a bounded sample of the same workload: decode steps of sampled
    sequences (same shapes and recipe, numpy generator), timed on the host cores."""
    import numpy as np
    import oracle as O
    from synth import inputs as S
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    w = S.WORKLOADS[name]
    sample_b = 2
    x = S.decode_cache_inputs(w, B=sample_b)
    done = 0
    t0 = time.time()
    while True:
        b = done % sample_b
        t = int(x["pos"][b])
        if w.mode == "csa":
            O.csa_query(t, x["q"][b, 0], x["qi"][b, 0], x["qi_scale"][b, 0], x["wi"][b, 0],
                        x["sink"], x["entries"][b], x["ikeys"][b], x["iscale"][b], w.N,
                        x["window"][b], lambda u: u % w.n_win, w.m, w.k, w.n_win, w.scale,
                        x["inv_freq"])
        else:
            O.hca_query(t, x["q"][b, 0], x["sink"], x["entries"][b], w.N, x["window"][b],
                        lambda u: u % w.n_win, w.m, w.n_win, w.scale, x["inv_freq"])
        done += 1
        el = time.time() - t0
        if el > budget_s or done >= 4096:
            break
    return {"value": done / el, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "%d decode tokens (sequences of the %s workload, %d distinct) in %.1f s"
                      % (done, name, sample_b, el)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="csa_decode_128k")
    ap.add_argument("--extra", default="csa_decode_1m,hca_decode_1m,csa_prefill_64k,"
                    "csa_decode_128k_mxfp4,csa_decode_1m_mxfp4,csa_prefill_64k_mxfp4,"
                    "qo_proj_64k,csa_decode_128k_paged,csa_decode_1m_paged,hca_decode_1m_paged,"
                    "csa_decode_128k_mixed,csa_decode_1m_mixed,hca_decode_1m_mixed",
                    help="comma-separated extra workloads ('' for none)")
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

    print("[bench] %s: %d warm-up + %d timed steps" % (args.workload, args.warmup, args.steps),
          file=sys.stderr, flush=True)
    head = decode_workload(args.workload, args.steps, args.warmup, args.rotate)
    also = []
    for name in [n for n in args.extra.split(",") if n]:
        print("[bench] extra %s" % name, file=sys.stderr, flush=True)
        if name.startswith("csa_prefill"):
            also.append(prefill_workload(name, max(2, args.steps // 10), 1))
        elif name.startswith("qo_proj"):
            also.append(proj_workload(name, max(2, args.steps // 10), 1))
        else:
            also.append(decode_workload(name, args.steps, args.warmup, args.rotate))
    if args.calib_copy:
        src = torch.empty(1 << 29, dtype=torch.int16, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(args.calib_copy):
            dst.copy_(src)
        torch.cuda.synchronize()
    cpu = None
    if not args.no_cpu:
        print("[bench] cpu oracle baseline", file=sys.stderr, flush=True)
        cpu = cpu_baseline(args.workload)

    from synth import inputs as S
    w = S.WORKLOADS[args.workload]
    line = {
        "metric": METRIC, "value": head["value"], "unit": head["unit"], "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": head["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8+bf16", "data": "synthetic",
        "config": {"workload": args.workload, "batch": w.B, "context": w.t, "entries": w.N,
                   "heads": w.n_h, "head_dim": w.c, "indexer": "%dx%d e4m3" % (w.H_I, w.d_I),
                   "top_k": w.k, "window": w.n_win},
        "hbm_gbs": head["hbm_gbs"], "hbm_frac": head["hbm_frac"],
        "roofline": head["roofline"], "cpu_baseline": cpu,
        "kernels_ms_per_step": head["kernels_ms_per_step"], "also": also,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
