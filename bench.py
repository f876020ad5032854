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
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # threadpoolctl missing: report the affinity set
        threads = len(os.sched_getaffinity(0))
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
    return {"value": frac / dt, "unit": "layer-searches/s", "cores": int(threads), "kind": "oracle",
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
    written per weight).  Each call streams from HBM: a 512 MiB buffer is overwritten between
    calls, so no input is left in the 256 MB last-level cache.  Seeded random values; the
    kernels' cost does not depend on them."""
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    res = {}
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)  # 2x the 256 MB last-level cache
    M, K = 16384, 14336
    X = torch.randn((M, K), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    a = torch.empty(K, dtype=torch.float32, device=dev)
    ws = torch.empty(awq.stats_workspace_bytes(M, K), dtype=torch.uint8, device=dev)
    fl = torch.zeros(1, dtype=torch.int32, device=dev)
    ms = _time_reps(torch, lambda: awq.stats(X, out=a, workspace=ws, flags=fl, check=False), reps, flush)
    nbytes = 2.0 * M * K + 4.0 * K
    res["stats"] = {"shape": [M, K], "bytes": nbytes, "ms": ms, "gbs": nbytes / (ms * 1e-3) / 1e9,
                    "frac": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS}
    del X, ws
    N, K = 28672, 4096
    W = torch.randn((N, K), generator=g, device=dev, dtype=torch.float32).mul_(K ** -0.5).to(torch.bfloat16)
    # per-channel scales spread like the search's a^alpha (log-normal, sigma 0.25); s = 1, the
    # alpha = 0 candidate, is slower on bf16 weights (exact fp32 quotient ties take the exact path)
    sv = torch.exp(0.25 * torch.randn(K, generator=g, device=dev, dtype=torch.float32))
    out = (torch.empty((N, K // 8), dtype=torch.int32, device=dev),
           torch.empty((N, K // 128), dtype=torch.float16, device=dev),
           torch.empty((N, K // 128), dtype=torch.float16, device=dev))
    ms = _time_reps(torch, lambda: awq.pack(W, sv, flags=fl, out=out, check=False), reps, flush)
    nbytes = 2.53125 * N * K + 4.0 * K
    res["pack"] = {"shape": [N, K], "bytes": nbytes, "ms": ms, "gbs": nbytes / (ms * 1e-3) / 1e9,
                   "frac": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS}
    awq.raise_for_flags(fl)
    return res


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


def gram_form(torch, awq, dev, reps: int = 3):
    """The scale search in both loss forms on the decoder block's qkv layer (M = 16384 tokens,
    K = 4096, N = 6144, bf16): the direct form (20 x 2 M K N flop on the matrix cores) and the
    Gram form (G = X^T X once, 2 M K^2 flop, then 20 x 2 (2K) K N flop for the [G_hi; G_lo]
    stack).  Whole calls, event-timed; seeded random values with the workload's shapes."""
    g = torch.Generator(device=dev)
    g.manual_seed(3)
    M, K, N = 16384, 4096, 6144
    c = torch.exp(0.5 * torch.randn(K, generator=g, device=dev))
    X = (torch.randn((M, K), generator=g, device=dev) * c).to(torch.bfloat16)
    W = torch.randn((N, K), generator=g, device=dev).mul_(K ** -0.5).to(torch.bfloat16)
    a = awq.stats(X)
    ws = torch.empty(max(awq.search_workspace_bytes(M, K, N), awq.search_workspace_bytes(M, K, N, gram=True)),
                     dtype=torch.uint8, device=dev)
    fl = torch.zeros(1, dtype=torch.int32, device=dev)
    res = {}
    out = {}
    for name, gram in (("direct", False), ("gram", True)):
        out[name] = awq.search(X, W, a, workspace=ws, flags=fl, check=False, gram=gram)
        ms = _time_reps(torch, lambda: awq.search(X, W, a, workspace=ws, flags=fl, check=False, gram=gram), reps)
        flop = 20 * 2.0 * (2 * K if gram else M) * K * N + (2.0 * M * K * K if gram else 0.0)
        res[name] = {"ms": ms, "flop": flop, "tflops": flop / (ms * 1e-3) / 1e12,
                     "best": out[name].best_index}
    awq.raise_for_flags(fl)
    Ld, Lg = out["direct"].losses.double(), out["gram"].losses.double()
    res["shape"] = [M, K, N]
    res["speedup"] = res["direct"]["ms"] / res["gram"]["ms"]
    res["max_rel_loss_diff"] = float(((Lg - Ld).abs() / Ld).max())
    res["direct_equiv_tflops"] = res["direct"]["flop"] / (res["gram"]["ms"] * 1e-3) / 1e12
    res["note"] = "whole awq_search / awq_search_gram calls; direct_equiv_tflops = direct-form flop / gram time"
    return res


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
    res["scaled_act_gelu"] = {"shape": [M, K], "bytes": nbytes, "ms": ms, "gbs": nbytes / (ms * 1e-3) / 1e9,
                              "frac": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS}
    awq.raise_for_flags(fl)
    return res


def w4a16_products(torch, awq, dev, reps: int = 10):
    """The W4A16 product over a packed artefact of the decoder block's fused gate+up weight
    (N = 28672, K = 4096): decode with one token (HBM-bound: 0.53125 bytes per weight, the
    last-level cache flushed between calls) and prefill with 4096 tokens (MFMA-bound,
    2 M K N flop).  The artefact is packed on the GPU from a seeded bf16 weight."""
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
    M = 4096
    xp = torch.randn((M, K), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    yp = torch.empty((M, N), dtype=torch.float32, device=dev)
    ms_p = _time_reps(torch, lambda: awq.w4a16(xp, q, sc, zz, out=yp), max(3, reps // 2))
    flop = 2.0 * M * K * N
    return {"decode": {"tokens": 1, "shape": [N, K], "ms": ms_d, "bytes": bytes_d,
                       "gbs": bytes_d / (ms_d * 1e-3) / 1e9, "frac_hbm": bytes_d / (ms_d * 1e-3) / 1e9 / PEAK_HBM_GBS},
            "prefill": {"tokens": M, "shape": [N, K], "ms": ms_p, "flop": flop,
                        "tflops": flop / (ms_p * 1e-3) / 1e12,
                        "frac_mfma_peak": flop / (ms_p * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}}


def _time_reps(torch, fn, reps, flush=None):
    """Median of reps event-timed calls.  flush, when given, is a buffer larger than the
    last-level cache that is overwritten between calls (outside the timed intervals), so that
    every call reads its input from HBM."""
    fn()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for e0, e1 in evs:
        if flush is not None:
            flush.zero_()
        e0.record()
        fn()
        e1.record()
    torch.cuda.synchronize()
    return statistics.median(e0.elapsed_time(e1) for e0, e1 in evs)


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
    ap.add_argument("--no-gram", action="store_true", help="skip the Gram-form search timing")
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
        "stats_gbs": 2.0 * M * K / (st_ms * 1e-3) / 1e9,
        "pack_gbs": 2.53125 * K * N / (pk_ms * 1e-3) / 1e9,
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS, "traffic": traffic,
                     "kernel": "search_pipelined_kernel (fused quantize + bf16 MFMA error product + "
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
    if not args.no_gram:
        out["gram"] = gram_form(torch, awq, dev)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.config, args.cpu_sample)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
