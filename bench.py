"""Benchmark of the AWQ hot path on one MI355X.

One step = the whole path on one synthetic layer resident in HBM: activation statistic ->
20-candidate scale search (scale table, group ranges, fused quantize + error GEMM + squared
error, reduction and argmin) -> exact quantization and packing at the winning scales.

Default workload: the attention-projection-shaped layer, X bf16 [4096 x 4096], W bf16
[4096 x 4096] (N x K), group 128, 20 candidates.  Prints one JSON line.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--config attn] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "AWQ α-search layers/sec + effective TFLOP/s (% MFMA peak), K=N=4096, M=4096"
PEAK_BF16_TFLOPS = 2516.6  # MI355X dense bf16 matrix peak (AMD spec, 2.5 PF class)
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E


def cpu_baseline(config: str, n_sample: int, min_seconds: float = 10.0, max_reps: int = 3):
    """The oracle as it stands, on a bounded column sample of the same layer (all M tokens,
    all K channels, the first n_sample output channels), scaled to layer-searches/s.  The
    sample is repeated until at least min_seconds of CPU work (at most max_reps times)."""
    import numpy as np
    from oracle import awq_oracle as o
    from post_weight_quantization_mean_amd import synth
    affinity = len(os.sched_getaffinity(0))
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        infos = [i for i in threadpool_info() if i.get("user_api") == "blas"] or threadpool_info()
        threads = max([i.get("num_threads", 1) for i in infos] or [1])
        if infos:
            i = infos[0]
            blas = f"{i.get('internal_api', '?')} {i.get('version', '?')} ({i.get('threading_layer', '?')}, " \
                   f"{i.get('num_threads', '?')} threads)"
    except Exception:  # threadpoolctl missing: report the affinity set
        threads = affinity
    spec = synth.CONFIGS[config].layers[0]
    cfg_id = synth.CONFIGS[config].cfg_id
    X = synth.make_x(spec, 0, cfg_id, 0)
    W = synth.make_w(spec, 0, cfg_id, 0, rows=n_sample)
    X64, W32 = synth.to_f64(X), synth.to_f32(W)
    times = []
    while not times or (sum(times) < min_seconds and len(times) < max_reps):
        t0 = time.perf_counter()
        a32 = o.activation_stat(X64).astype(np.float32)
        res = o.search(X64, W32, a32)
        o.pack(W32, res["s_best"])
        times.append(time.perf_counter() - t0)
    dt = statistics.mean(times)
    frac = n_sample / spec.N
    return {"value": frac / dt, "unit": "layer-searches/s", "cores": int(threads), "affinity_cores": affinity,
            "blas": blas, "kind": "oracle",
            "sample": f"{config} layer, all {spec.M} tokens and {spec.K} channels, first {n_sample} of "
                      f"{spec.N} output channels (statistic over the full X), stats + 20-candidate search "
                      f"+ pack; {len(times)} run(s), mean {dt:.2f} s, scaled by N/{n_sample}"}


def search_traffic(config: str):
    """HBM bytes per launch of the fused search kernel, from the FETCH_SIZE / WRITE_SIZE counter
    summary committed under profiles/, or None when that summary was taken on another version
    of the kernel source (its sha256 is recorded there) or for another workload."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"search_fused_{config}_traffic.txt")
    src = os.path.join(ROOT, "post_weight_quantization_mean_amd", "csrc", "search.hip")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith(" "):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    if fields.get("search.hip sha256") != sha or "traffic bytes per launch" not in fields:
        return None
    return float(fields["traffic bytes per launch"])


def hbm_kernels(torch, awq, dev, reps: int = 10):
    """The two bandwidth-bound kernels at the largest shapes of the decoder-block workload:
    awq_stats on the MLP down-projection input X bf16 [16384 x 14336] (2 bytes per element
    read) and awq_pack on the fused gate+up weight W bf16 [28672 x 4096] (2 bytes read, 0.53125
    written per weight).  Two timings, both with every input in HBM:
      * ms / frac: back to back over eight distinct inputs of that shape (3.8 GB of X, 1.9 GB of
        W: far more than the 256 MB last-level cache, so no call finds its input cached), as a
        model's layers are quantized one after another; events around each pass of eight calls;
      * ms_single_call / frac_single_call: one call after a 512 MiB read that evicts the cache,
        events around it (this adds the launch's own start and end, 2-3 us).
    Seeded random values; the kernels' cost does not depend on them."""
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    res = {}
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)  # 2x the 256 MB last-level cache
    fl = torch.zeros(1, dtype=torch.int32, device=dev)
    nb = 8

    def entry(shape, nbytes, fn_one, fns):
        ms1 = _time_reps(torch, fn_one, reps, flush)
        ms = _back_to_back_ms(torch, fns, max(3, reps // 2))
        gbs, gbs1 = nbytes / (ms * 1e-3) / 1e9, nbytes / (ms1 * 1e-3) / 1e9
        return {"shape": shape, "bytes": nbytes, "ms": ms, "gbs": gbs, "frac": gbs / PEAK_HBM_GBS,
                "ms_single_call": ms1, "frac_single_call": gbs1 / PEAK_HBM_GBS, "inputs": nb}

    M, K = 16384, 14336
    Xs = [torch.randn((M, K), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16) for _ in range(nb)]
    a = torch.empty(K, dtype=torch.float32, device=dev)
    ws = torch.empty(awq.stats_workspace_bytes(M, K), dtype=torch.uint8, device=dev)
    res["stats"] = entry([M, K], 2.0 * M * K + 4.0 * K,
                         lambda: awq.stats(Xs[0], out=a, workspace=ws, flags=fl, check=False),
                         [lambda X=X: awq.stats(X, out=a, workspace=ws, flags=fl, check=False) for X in Xs])
    del Xs, ws
    N, K = 28672, 4096
    Ws = [torch.randn((N, K), generator=g, device=dev, dtype=torch.float32).mul_(K ** -0.5).to(torch.bfloat16)
          for _ in range(nb)]
    # per-channel scales spread like the search's a^alpha (log-normal, sigma 0.25); s = 1, the
    # alpha = 0 candidate, is slower on bf16 weights (exact fp32 quotient ties take the exact path)
    sv = torch.exp(0.25 * torch.randn(K, generator=g, device=dev, dtype=torch.float32))
    out = (torch.empty((N, K // 8), dtype=torch.int32, device=dev),
           torch.empty((N, K // 128), dtype=torch.float16, device=dev),
           torch.empty((N, K // 128), dtype=torch.float16, device=dev))
    res["pack"] = entry([N, K], 2.53125 * N * K + 4.0 * K,
                        lambda: awq.pack(Ws[0], sv, flags=fl, out=out, check=False),
                        [lambda W=W: awq.pack(W, sv, flags=fl, out=out, check=False) for W in Ws])
    del Ws
    awq.raise_for_flags(fl)
    return res


def _back_to_back_ms(torch, fns, reps):
    """Per-call time of the calls fns issued back to back: median over reps passes, events
    around each pass (after one untimed pass)."""
    for f in fns:
        f()
    torch.cuda.synchronize()
    t = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for f in fns:
            f()
        e1.record()
        torch.cuda.synchronize()
        t.append(e0.elapsed_time(e1) / len(fns))
    return statistics.median(t)


def clip_search(torch, awq, Xd, Wd, s_best, stride: int = 8, reps: int = 10):
    """The clipping search that follows the scale search, on the same layer at its winning
    scales, scoring every ``stride``-th token (a strided view, no copy): 10 thresholds per
    (output channel, group).  Reported beside the step, not inside it: work 10 x 2*Ms*K*N
    flop on the matrix cores (Ms sampled tokens), plus the range and select launches."""
    Xs = Xd[::stride]
    Ms, K = Xs.shape
    N = Wd.shape[0]
    ws = torch.empty(awq.clip_workspace_bytes(Ms, K, N), dtype=torch.uint8, device=Xd.device)
    fl = torch.zeros(1, dtype=torch.int32, device=Xd.device)
    ms = _time_reps(torch, lambda: awq.clip(Xs, Wd, s_best, workspace=ws, flags=fl, check=False), reps)
    awq.raise_for_flags(fl)
    flops = 10 * 2.0 * Ms * K * N
    tf = flops / (ms * 1e-3) / 1e12
    return {"tokens": Ms, "token_stride": stride, "n_clip": 10, "ms": ms, "flop": flops,
            "tflops": tf, "frac_mfma_peak": tf / PEAK_BF16_TFLOPS,
            "note": "whole awq_clip call (range pre-pass, clipped qdq + bf16 MFMA product, select)"}


GELU_VALU_PER_ELEMENT = 38  # scale_kernel<2, true, 4>: VALU instructions per element, from its assembly


def fold_ops(torch, awq, dev, reps: int = 10):
    """Applying the scales, at the decoder block's largest shapes: awq_scale_cols in place on the
    fused gate+up weight bf16 [28672 x 4096] and awq_scaled_act (GELU) from the MLP activation
    bf16 [16384 x 14336] into a second buffer; 2 bytes read + 2 written per element (plus s).
    The last-level cache is flushed between calls.  Seeded random values."""
    g = torch.Generator(device=dev)
    g.manual_seed(2)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    fl = torch.zeros(1, dtype=torch.int32, device=dev)
    res = {}
    N, K = 28672, 4096
    W = torch.randn((N, K), generator=g, device=dev, dtype=torch.float32).mul_(K ** -0.5).to(torch.bfloat16)
    s = torch.exp(0.25 * torch.randn(K, generator=g, device=dev, dtype=torch.float32))
    ms = _time_reps(torch, lambda: awq.scale_cols(W, s, flags=fl, check=False), reps, flush)
    nbytes = 4.0 * N * K + 4.0 * K
    res["scale_cols"] = {"shape": [N, K], "bytes": nbytes, "ms": ms, "gbs": nbytes / (ms * 1e-3) / 1e9,
                         "frac": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS}
    del W
    M, K = 16384, 14336
    X = torch.randn((M, K), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    Y = torch.empty_like(X)
    s = torch.exp(0.25 * torch.randn(K, generator=g, device=dev, dtype=torch.float32))
    ms = _time_reps(torch, lambda: awq.scaled_act(X, s, "gelu", out=Y, flags=fl, check=False), reps, flush)
    nbytes = 4.0 * M * K + 4.0 * K
    # the GELU is bound by ALU issue: its compiled loop spends about 38 VALU instructions per
    # element (the library erfcf about 25); the ALU roof at the 2.4 GHz spec clock is that count
    # over 256 CUs x 64 lanes per clock
    alu_ms = M * K * GELU_VALU_PER_ELEMENT / (256 * 64 * 2.4e9) * 1e3
    res["scaled_act_gelu"] = {"shape": [M, K], "bytes": nbytes, "ms": ms, "gbs": nbytes / (ms * 1e-3) / 1e9,
                              "frac": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, "bound": "alu",
                              "valu_per_element": GELU_VALU_PER_ELEMENT, "alu_roof_ms_at_2_4ghz": alu_ms,
                              "frac_alu_at_2_4ghz": alu_ms / ms}
    awq.raise_for_flags(fl)
    return res


def w4a16_products(torch, awq, dev, reps: int = 10):
    """The W4A16 product over a packed artefact of the decoder block's fused gate+up weight
    (N = 28672, K = 4096): decode with one token (HBM-bound: 0.53125 bytes per weight, the
    last-level cache flushed between calls), decode with 1, 2, 4 and 8 tokens back to back over
    eight such artefacts in one HIP graph, and prefill with 4096 tokens (MFMA-bound, 2 M K N
    flop).  The artefacts are packed on the GPU from seeded bf16 weights."""
    g = torch.Generator(device=dev)
    g.manual_seed(1)
    N, K = 28672, 4096
    W = torch.randn((N, K), generator=g, device=dev, dtype=torch.float32).mul_(K ** -0.5).to(torch.bfloat16)
    s = torch.exp(0.25 * torch.randn(K, generator=g, device=dev, dtype=torch.float32))
    q, sc, zz = awq.pack(W, s)
    del W
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    x1 = torch.randn((1, K), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    y1 = torch.empty((1, N), dtype=torch.float32, device=dev)
    ms_d = _time_reps(torch, lambda: awq.w4a16(x1, q, sc, zz, out=y1), reps, flush)
    bytes_d = N * K * 0.5 + N * (K // 128) * 4.0 + K * 2.0 + N * 4.0
    # back to back, as consecutive layers of a model decode: eight artefacts (8 x 62.5 MB, more
    # than the last-level cache), 32 calls captured in one HIP graph, so that neither a launch's
    # host cost nor the fixed cost of timing one short launch with events is in the figure
    arts = [(q, sc, zz)]
    for _ in range(7):
        Wi = torch.randn((N, K), generator=g, device=dev, dtype=torch.float32).mul_(K ** -0.5).to(torch.bfloat16)
        arts.append(awq.pack(Wi, s))
        del Wi
    graph = {}
    for m in (1, 2, 4, 8):
        xm = torch.randn((m, K), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
        ys = [torch.empty((m, N), dtype=torch.float32, device=dev) for _ in arts]
        eager = [awq.w4a16(xm, *a) for a in arts]
        ms = _graph_ms_per_call(torch, lambda: [awq.w4a16(xm, *a, out=y) for _ in range(4) for a, y in zip(arts, ys)],
                                4 * len(arts), reps)
        if not all(torch.equal(y, e) for y, e in zip(ys, eager)):
            raise RuntimeError("w4a16 decode: graph replay differs from the eager call")
        b = N * K * 0.5 + N * (K // 128) * 4.0 + m * K * 2.0 + m * N * 4.0
        graph[str(m)] = {"ms": ms, "gbs": b / (ms * 1e-3) / 1e9, "frac_hbm": b / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS}
    del arts
    M = 4096
    xp = torch.randn((M, K), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    yp = torch.empty((M, N), dtype=torch.float32, device=dev)
    wsp = torch.empty(awq.w4a16_workspace_bytes(M, K), dtype=torch.uint8, device=dev)  # the copy of X
    ms_p = _time_reps(torch, lambda: awq.w4a16(xp, q, sc, zz, out=yp, workspace=wsp), max(3, reps // 2))
    flop = 2.0 * M * K * N
    return {"decode": {"tokens": 1, "shape": [N, K], "ms": ms_d, "bytes": bytes_d,
                       "gbs": bytes_d / (ms_d * 1e-3) / 1e9, "frac_hbm": bytes_d / (ms_d * 1e-3) / 1e9 / PEAK_HBM_GBS,
                       "note": "ms: one call, events around it, last-level cache flushed before it"},
            "decode_in_graph": {"tokens": graph, "artefacts": 8, "calls": 32,
                                "note": "per-call time of 32 back-to-back calls over 8 different artefacts, one HIP graph"},
            "prefill": {"tokens": M, "shape": [N, K], "ms": ms_p, "flop": flop,
                        "note": "one flushed call: the copy of X in operand order (xfrag) and the product",
                        "tflops": flop / (ms_p * 1e-3) / 1e12,
                        "frac_mfma_peak": flop / (ms_p * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}}


# Layer-searches/s (blocks/s for the block) at 50 % of the bf16 peak for the search's own
# flop: the targets the configurations are quoted against (context, not part of `value`).
TARGET_HALF_PEAK = {"attn": 457.8, "down": 170.3, "gate_up": 27.1, "block": 8.8}


def layer_step(torch, awq, synth, spec, dev, reps, gram=False):
    """One full-size layer through the whole path (statistic -> search -> pack), inputs drawn on
    the GPU with the synthetic recipe: median of reps event-timed steps, each split into its
    stages, with the fused kernel timed alone by the events awq_search_timed records.  gram: the
    Gram-form search of the same layer as well (whole call)."""
    X, W = synth.make_layer_device(spec, dev)
    M, K, N = spec.M, spec.K, spec.N
    a = torch.empty(K, dtype=torch.float32, device=dev)
    ws_st = torch.empty(awq.stats_workspace_bytes(M, K), dtype=torch.uint8, device=dev)
    ws_se = torch.empty(awq.search_workspace_bytes(M, K, N), dtype=torch.uint8, device=dev)
    fl = torch.zeros(1, dtype=torch.int32, device=dev)
    out = (torch.empty((N, K // 8), dtype=torch.int32, device=dev),
           torch.empty((N, K // 128), dtype=torch.float16, device=dev),
           torch.empty((N, K // 128), dtype=torch.float16, device=dev))
    stream = torch.cuda.current_stream(dev)

    def one(ev):
        ev[0].record(stream)
        awq.stats(X, out=a, workspace=ws_st, flags=fl, check=False)
        ev[1].record(stream)
        r = awq.search(X, W, a, workspace=ws_se, flags=fl, check=False, fused_events=(ev[4], ev[5]))
        ev[2].record(stream)
        awq.pack(W, r.s_best, flags=fl, out=out, check=False)
        ev[3].record(stream)
        return r

    def events():
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
        for e in evs:
            e.record(stream)
        return evs

    one(events())
    torch.cuda.synchronize()
    evs = [events() for _ in range(reps)]
    for ev in evs:
        res = one(ev)
    torch.cuda.synchronize()
    awq.raise_for_flags(fl)
    med = lambda i, j: statistics.median(ev[i].elapsed_time(ev[j]) for ev in evs)
    step, fused = med(0, 3), med(4, 5)
    flop = 20 * 2.0 * M * K * N
    row = {"shape": [M, K, N], "dtype": spec.dtype, "step_ms": step, "stats_ms": med(0, 1),
           "search_ms": med(1, 2), "fused_ms": fused, "pack_ms": med(2, 3),
           "layer_searches_per_s": 1000.0 / step, "fused_tflops": flop / (fused * 1e-3) / 1e12,
           "fused_frac": flop / (fused * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
           "step_tflops": flop / (step * 1e-3) / 1e12, "best_alpha": res.best_index / 20.0}
    if gram:
        ws_g = torch.empty(awq.search_workspace_bytes(M, K, N, gram=True), dtype=torch.uint8, device=dev)
        call = lambda: awq.search(X, W, a, workspace=ws_g, flags=fl, check=False, gram=True)
        g_ms = _time_reps(torch, call, reps)
        awq.raise_for_flags(fl)
        row["gram_search_ms"] = g_ms
        row["gram_direct_equiv_tflops"] = flop / (g_ms * 1e-3) / 1e12
        row["gram_speedup_vs_direct_search"] = row["search_ms"] / g_ms
        row["step_ms_with_gram"] = row["stats_ms"] + g_ms + row["pack_ms"]
        row["layer_searches_per_s_with_gram"] = 1000.0 / row["step_ms_with_gram"]
        del ws_g
    del X, W, ws_se, ws_st, out
    torch.cuda.empty_cache()
    return row


def gram_pays(spec) -> bool:
    """The Gram form does less work than the direct one when M > K + 512 (its triangular
    candidate product costs about 2 K (K + 512) N flop against 2 M K N; bf16 only)."""
    return spec.dtype == "bf16" and spec.M > spec.K + 512


def per_config(torch, awq, dev):
    """Every configuration's throughput beside the headline: tiny, attn, down and gate+up as one
    layer each, and the decoder block as its four layers searched in turn (blocks/s), with the
    Gram form as well for every layer where M > K + 512 (gate+up; the block's four layers)."""
    from post_weight_quantization_mean_amd import synth
    reps = {"tiny": 20, "attn": 10, "down": 5, "gate_up": 3}
    res = {}
    for name in ("tiny", "attn", "down", "gate_up"):
        spec = synth.CONFIGS[name].layers[0]
        res[name] = layer_step(torch, awq, synth, spec, dev, reps[name], gram=gram_pays(spec))
        if name in TARGET_HALF_PEAK:
            res[name]["target_at_half_peak"] = TARGET_HALF_PEAK[name]
    layers = {}
    for spec in synth.CONFIGS["block"].layers:
        layers[spec.name] = layer_step(torch, awq, synth, spec, dev, 3, gram=gram_pays(spec))
    total = sum(r["step_ms"] for r in layers.values())
    best = sum(r["stats_ms"] + r["pack_ms"] + min(r["search_ms"], r.get("gram_search_ms", float("inf")))
               for r in layers.values())
    flop = sum(20 * 2.0 * r["shape"][0] * r["shape"][1] * r["shape"][2] for r in layers.values())
    res["block"] = {"layers": layers, "block_ms": total, "blocks_per_s": 1000.0 / total,
                    "block_ms_with_gram": best, "blocks_per_s_with_gram": 1000.0 / best,
                    "effective_tflops": flop / (total * 1e-3) / 1e12,
                    "target_at_half_peak": TARGET_HALF_PEAK["block"]}
    res["note"] = ("inputs drawn on the GPU with the synthetic recipe (dense-kernel cost does not depend on the "
                   "values); step = stats + search + pack, medians of event-timed steps; fused_* is the fused "
                   "search kernel alone; *_with_gram takes the Gram-form search where it is faster")
    return res


def clock_sample(torch, awq, dev, seconds=2.0, samples=3):
    """The GPU clock while the fused search runs back to back: amd-smi's per-XCD gfx clocks,
    sampled from a second thread during seconds of queued attn-layer searches."""
    import subprocess
    import threading
    from post_weight_quantization_mean_amd import synth
    spec = synth.CONFIGS["attn"].layers[0]
    X, W = synth.make_layer_device(spec, dev)
    a = awq.stats(X)
    ws = torch.empty(awq.search_workspace_bytes(spec.M, spec.K, spec.N), dtype=torch.uint8, device=dev)
    fl = torch.zeros(1, dtype=torch.int32, device=dev)
    awq.search(X, W, a, workspace=ws, flags=fl, check=False)
    torch.cuda.synchronize()
    found, errors = [], []

    def sampler():
        time.sleep(0.3)
        for _ in range(samples):
            try:
                out = subprocess.run(["amd-smi", "metric", "-g", "0", "--clock", "--json"], capture_output=True,
                                     text=True, timeout=20)
                found.extend(_gfx_clocks(json.loads(out.stdout)))
            except Exception as e:  # amd-smi missing or its output changed: report, do not fail
                errors.append(repr(e)[:200])
            time.sleep(0.1)

    t = threading.Thread(target=sampler)
    t0 = time.perf_counter()
    t.start()
    n = 0
    while time.perf_counter() - t0 < seconds or t.is_alive():
        for _ in range(50):
            awq.search(X, W, a, workspace=ws, flags=fl, check=False)
        n += 50
        torch.cuda.synchronize()
        if n > 20000:
            break
    t.join()
    del X, W, ws
    torch.cuda.empty_cache()
    if not found:
        return {"mhz": None, "source": "amd-smi", "errors": errors}
    return {"mhz": statistics.median(found), "min_mhz": min(found), "max_mhz": max(found), "samples": len(found),
            "source": "amd-smi metric --clock (median of the per-XCD gfx clocks) during back-to-back attn searches"}


def _gfx_clocks(obj):
    """Every gfx_<i>.clk value (MHz) in amd-smi's JSON, wherever it sits."""
    vals = []
    if isinstance(obj, dict):
        for k, v in obj.items():
            if k.startswith("gfx_") and isinstance(v, dict) and isinstance(v.get("clk"), dict):
                val = v["clk"].get("value")
                if isinstance(val, (int, float)):
                    vals.append(float(val))
            else:
                vals.extend(_gfx_clocks(v))
    elif isinstance(obj, list):
        for v in obj:
            vals.extend(_gfx_clocks(v))
    return vals


def _time_reps(torch, fn, reps, flush=None):
    """Median of reps event-timed calls.  flush, when given, is a buffer larger than the
    last-level cache that is read between calls (outside the timed intervals), so that every
    call reads its input from HBM.  It is read, not overwritten: a fill leaves the cache full
    of dirty lines, and the next call would pay for writing them back (a 28672 x 4096 pack
    measured 59 us after a fill and 55 us after a read; a device copy 4.4 TB/s against 5.7)."""
    fn()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    words = flush.view(torch.int32) if flush is not None else None
    for e0, e1 in evs:
        if words is not None:
            words.amax()
        e0.record()
        fn()
        e1.record()
    torch.cuda.synchronize()
    return statistics.median(e0.elapsed_time(e1) for e0, e1 in evs)


def _graph_ms_per_call(torch, fn, calls, reps):
    """Median over reps replays of one HIP graph that holds fn's launches, per launch (calls of
    them in fn).  fn runs once on a side stream before the capture (first-call set-up)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        fn()
    gr.replay()
    torch.cuda.synchronize()
    t = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        gr.replay()
        e1.record()
        torch.cuda.synchronize()
        t.append(e0.elapsed_time(e1) / calls)
    return statistics.median(t)


def copy_probe(mib: int, reps: int):
    """A plain device-to-device copy of a known size, the calibration run for the HBM byte
    counters (FETCH_SIZE / WRITE_SIZE per dispatch against 2 x mib MiB moved)."""
    import torch
    dev = torch.device("cuda:0")
    n = mib * (1 << 20) // 4
    src = torch.arange(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    assert torch.equal(dst[-4:], src[-4:])
    print(json.dumps({"copy_probe_mib": mib, "reps": reps, "bytes_read": n * 4, "bytes_written": n * 4}),
          flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="attn")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=4096, help="output channels of the oracle sample")
    ap.add_argument("--no-hbm", action="store_true", help="skip the large-input stats / pack timing")
    ap.add_argument("--no-clip", action="store_true", help="skip the clipping-search timing")
    ap.add_argument("--no-w4a16", action="store_true", help="skip the W4A16 product timing")
    ap.add_argument("--no-fold", action="store_true", help="skip the scale-application timing")
    ap.add_argument("--no-configs", action="store_true", help="skip the per-configuration throughput")
    ap.add_argument("--no-clock", action="store_true", help="skip the GPU clock sample")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain copy of MIB MiB (counter calibration) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "the library runs the path on one GPU; --gpus must be 1 "
                                   "(the path would shard along N with one 160-byte loss all-reduce)"}))
        sys.exit(2)

    if args.copy_probe:
        copy_probe(args.copy_probe, max(args.steps, 1))
        return

    import torch
    from post_weight_quantization_mean_amd import awq, synth
    if not os.path.exists(awq._LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()

    dev = torch.device("cuda:0")
    spec, X, W = synth.make_layer(args.config)
    M, K, N = spec.M, spec.K, spec.N
    Xd, Wd = X.to(dev), W.to(dev)
    del X, W
    a = torch.empty(K, dtype=torch.float32, device=dev)
    ws_stats = torch.empty(awq.stats_workspace_bytes(M, K), dtype=torch.uint8, device=dev)
    ws_search = torch.empty(awq.search_workspace_bytes(M, K, N), dtype=torch.uint8, device=dev)
    flags = torch.zeros(1, dtype=torch.int32, device=dev)
    qweight = torch.empty((N, K // 8), dtype=torch.int32, device=dev)
    scales = torch.empty((N, K // 128), dtype=torch.float16, device=dev)
    zeros = torch.empty_like(scales)

    stream = torch.cuda.current_stream(dev)

    def events():
        # [0..3]: stage boundaries on the call stream; [4], [5]: recorded by the library right
        # before and after the fused search kernel, on the same stream
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
        for e in evs:
            e.record(stream)  # creates the HIP event outside the timed region
        return evs

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        awq.stats(Xd, out=a, workspace=ws_stats, flags=flags, check=False)
        if ev:
            ev[1].record(stream)
        res = awq.search(Xd, Wd, a, workspace=ws_search, flags=flags, check=False,
                         fused_events=(ev[4], ev[5]) if ev else None)
        if ev:
            ev[2].record(stream)
        awq.pack(Wd, res.s_best, flags=flags, out=(qweight, scales, zeros), check=False)
        if ev:
            ev[3].record(stream)
        return res

    for _ in range(args.warmup):
        res = step()
    torch.cuda.synchronize()
    awq.raise_for_flags(flags)

    # All events are created up front and read after the loop: no host sync inside the
    # timed region, every launch queued back to back on the one stream.
    evs = [events() for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    wall0 = time.perf_counter()
    for k in range(args.steps):
        res = step(evs[k])
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    awq.raise_for_flags(flags)
    per_step = [(e[0].elapsed_time(e[1]), e[1].elapsed_time(e[2]), e[2].elapsed_time(e[3]),
                 e[4].elapsed_time(e[5])) for e in evs]

    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / args.steps
    st_ms = statistics.mean(p[0] for p in per_step)
    se_ms = statistics.mean(p[1] for p in per_step)
    pk_ms = statistics.mean(p[2] for p in per_step)
    fu_ms = statistics.mean(p[3] for p in per_step)
    flops = 20 * 2.0 * M * K * N
    achieved = flops / (fu_ms * 1e-3) / 1e12
    traffic = search_traffic(args.config)
    out = {
        "metric": METRIC,
        "value": 1000.0 / ms_per_step,
        "unit": "layer-searches/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{args.config}: X bf16 [{M} x {K}], W bf16 [{N} x {K}], group 128, "
                               f"20 candidates, stats + search + pack", "M": M, "K": K, "N": N,
                   "group": 128, "n_grid": 20},
        "effective_tflops": flops / (ms_per_step * 1e-3) / 1e12,
        "pct_mfma_peak": 100.0 * flops / (ms_per_step * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "stage_ms": {"stats": st_ms, "search": se_ms, "search_fused_kernel": fu_ms, "pack": pk_ms},
        # the attn layer's X (32 MiB) and W fit in the 256 MB last-level cache: these rates are
        # cache-resident; the `hbm` field times both kernels on larger inputs streamed from HBM
        "stats_gbs_cache_resident": 2.0 * M * K / (st_ms * 1e-3) / 1e9,
        "pack_gbs_cache_resident": 2.53125 * K * N / (pk_ms * 1e-3) / 1e9,
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS, "traffic": traffic,
                     "kernel": "search_persistent_kernel (fused quantize + bf16 MFMA error product + "
                               "squared error, all 20 candidates in one launch)",
                     "work_per_launch": f"20 x 2*M*K*N = {flops:.4g} flop",
                     "ms_per_launch": fu_ms},
        "best_alpha": res.best_index / 20.0,
        "wall_s": wall,
    }
    if not args.no_clip:
        out["clip"] = clip_search(torch, awq, Xd, Wd, res.s_best)
    if not args.no_hbm:
        out["hbm"] = hbm_kernels(torch, awq, dev)
    if not args.no_w4a16:
        out["w4a16"] = w4a16_products(torch, awq, dev)
    if not args.no_fold:
        out["fold"] = fold_ops(torch, awq, dev)
    if not args.no_configs:
        out["configs"] = per_config(torch, awq, dev)
    if not args.no_clock:
        clk = clock_sample(torch, awq, dev)
        out["gpu_clock"] = clk
        if clk.get("mhz"):
            out["roofline"]["frac_at_measured_clock"] = achieved / (PEAK_BF16_TFLOPS * clk["mhz"] / 2400.0)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.config, args.cpu_sample)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
