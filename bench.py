"""Benchmark of the lightning-indexer hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-extra]

A step is one forward of the V4 lightning indexer on the 32K workload
(batch 1, seqlen 32768, seqlen_kv 8192, 64 heads, index_dim 128,
compress_ratio 4, topk 2048): causally masked scoring of every valid
(query, key) pair plus the per-query top-k.  Two routes compute it and both
are timed on the same inputs: lix_topk's fused path (no logits in HBM) and
the materialized path (lix_indexer_logits, then lix_topk over the logits);
the step is the faster one, named in config.path.  The same run also times
the gather lix_topk_scores at the selected indices, the direct scoring at
those indices (lix_indexer_scores_at), the backward of those scores
(lix_indexer_backward, seeded upstream gradient), lix_indexer_scores_v41 and a top-512 of its
bf16 scores (lix_topk_bf16) on the V4.1 workload (batch 1, 16384 queries, 4096
keys, packed documents), a 1 GiB device copy (achievable HBM bandwidth), the
4K workload cold (L2 and MALL flushed by a 1 GiB write before each call) and
warm, the fused step on the 131K workload, and a bf16 8192^3 GEMM through
torch (hipBLASLt) as the achievable dense MFMA rate beside the published one.

Prints one JSON line.  `value` is causally valid TFLOP/s (2*H*D per visible
pair) over the whole step; queries/s are reported beside it.  Kernel
durations come from HIP events on the stream the library launches on.
Inputs are resident in HBM before timing starts.
"""

import argparse
import json
import os
import platform
import sys
import time

import numpy as np
import torch

import synth
import sparse_attention_lightning_bf16_amd as lx

METRIC = "indexer TFLOP/s (causal-valid) + queries/s incl. top-k, 32K ctx, 1 MI355X"
PEAK_BF16_TFLOPS = 2500.0        # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0            # MI355X HBM3E, published


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def causal_valid_pairs(S, Skv, c):
    p = np.arange(S, dtype=np.int64)
    return int(np.minimum((p + 1) // c, Skv).sum())


class EventTimer:
    """Average duration of a repeated launch, measured with HIP events on the current stream."""

    def __init__(self):
        self.pairs = []

    def __enter__(self):
        self.start = torch.cuda.Event(enable_timing=True)
        self.end = torch.cuda.Event(enable_timing=True)
        self.start.record()
        return self

    def __exit__(self, *exc):
        self.end.record()
        self.pairs.append((self.start, self.end))

    def mean_ms(self):
        torch.cuda.synchronize()
        return float(np.mean([s.elapsed_time(e) for s, e in self.pairs]))


def time_loop(fn, steps, warmup):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t = EventTimer()
    wall0 = time.perf_counter()
    for _ in range(steps):
        with t:
            fn()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - wall0) * 1e3 / steps
    return t.mean_ms(), wall


def time_each(fn, steps, warmup, between=None):
    """Mean per-call time with HIP events around each call; `between` runs untimed before each call."""
    for _ in range(warmup):
        if between is not None:
            between()
        fn()
    torch.cuda.synchronize()
    t = EventTimer()
    for _ in range(steps):
        if between is not None:
            between()
        with t:
            fn()
    return t.mean_ms()


def extra_parts(dev, steps, warmup):
    """Achievable copy bandwidth, the 4K materialized step cold and warm, the 131K fused step."""
    out = {}
    # achievable dense bf16 rate on this machine: a large library GEMM (hipBLASLt through torch)
    a = torch.randn(8192, 8192, device=dev, dtype=torch.bfloat16)
    bm = torch.randn(8192, 8192, device=dev, dtype=torch.bfloat16)
    gemm_ms = time_each(lambda: torch.matmul(a, bm), steps, warmup)
    out["gemm_bf16_8192_ms"] = gemm_ms
    out["gemm_bf16_tflops"] = 2.0 * 8192 ** 3 / gemm_ms / 1e9
    del a, bm
    src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    copy_ms = time_each(lambda: dst.copy_(src), steps, warmup)
    out["copy_1gib_ms"] = copy_ms
    out["copy_gbs"] = 2.0 * src.numel() * 4 / copy_ms / 1e6             # read + write
    flush = lambda: dst.fill_(0.0)                                        # 1 GiB write: evicts L2 and MALL
    del src

    cfg = synth.WORKLOADS["4k"]
    inp = synth.v4_inputs(**cfg)
    q, k, w = (inp[x].to(dev) for x in "qkw")
    c, tk = cfg["compress_ratio"], cfg["topk"]
    logits = torch.empty(cfg["batch"], cfg["seqlen"], cfg["seqlen_kv"], dtype=torch.float32, device=dev)
    def step4k():
        lx.indexer_logits(q, k, w, c, out=logits)
        return lx.topk_from_logits(logits, c, tk)
    out["4k_materialized_warm_ms"] = time_each(step4k, steps, warmup)
    out["4k_materialized_cold_ms"] = time_each(step4k, steps, warmup, between=flush)
    out["4k_fused_warm_ms"] = time_each(lambda: lx.topk(q, k, w, c, tk), steps, warmup)
    out["4k_fused_cold_ms"] = time_each(lambda: lx.topk(q, k, w, c, tk), steps, warmup, between=flush)
    del q, k, w, logits, dst

    log("timing the 131K fused step")
    cfg = synth.WORKLOADS["131k"]
    inp = synth.v4_inputs(**cfg)
    q, k, w = (inp[x].to(dev) for x in "qkw")
    del inp
    c, tk = cfg["compress_ratio"], cfg["topk"]
    ms = time_each(lambda: lx.topk(q, k, w, c, tk), max(3, steps // 4), 2)
    pairs = cfg["batch"] * causal_valid_pairs(cfg["seqlen"], cfg["seqlen_kv"], c)
    out["131k_fused_ms"] = ms
    out["131k_fused_tflops"] = 2.0 * cfg["heads"] * cfg["index_dim"] * pairs / ms / 1e9
    out["131k_queries_per_s"] = cfg["batch"] * cfg["seqlen"] / (ms * 1e-3)
    return out


def source_digest():
    """sha256 over the library's kernel and ABI sources (csrc/*)."""
    import hashlib
    root = os.path.join(os.path.dirname(os.path.abspath(__file__)), "sparse_attention_lightning_bf16_amd", "csrc")
    h = hashlib.sha256()
    for name in sorted(os.listdir(root)):
        if name.endswith((".hip", ".h", ".cpp")):
            with open(os.path.join(root, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def recorded_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed FETCH_SIZE/WRITE_SIZE summary, or None when
    that summary was taken on other kernel sources than the ones built here."""
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", "indexer_32k_hbm_traffic.md")
    try:
        lines = open(path).read().splitlines()
    except OSError:
        return None
    for line in lines:
        if line.startswith("traffic-record: "):
            rec = json.loads(line[len("traffic-record: "):])
            if rec.get("source_sha256") != source_digest():
                return None
            k = rec.get("kernels", {}).get(kernel)
            if k is None:
                return None
            return {"read_bytes": k["read_bytes"], "written_bytes": k["written_bytes"],
                    "total_bytes": k["read_bytes"] + k["written_bytes"],
                    "algorithmic_bytes": k.get("algorithmic_bytes"), "source": "profiles/indexer_32k_hbm_traffic.md"}
    return None


def cpu_baseline(inp, cfg, sample_every):
    """The float64 oracle on a stratified sample of the workload's query rows."""
    import oracle
    from threadpoolctl import threadpool_info
    S, Skv, c, tk = cfg["seqlen"], cfg["seqlen_kv"], cfg["compress_ratio"], cfg["topk"]
    H, D = cfg["heads"], cfg["index_dim"]
    nb = {x: synth.bits(inp[x]) for x in "qkw"}
    ks, ke = oracle.causal_ranges(S, Skv, c)
    rows = np.arange(sample_every - 1, S, sample_every)
    t0 = time.perf_counter()
    lg = oracle.indexer_logits_rows(nb["q"], nb["k"], nb["w"], 0, rows, ks, ke)
    oracle.topk_select(lg, ks[rows], ke[rows], tk)
    dt = time.perf_counter() - t0
    flop = 2.0 * H * D * float(ke[rows].sum())
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {
        "value": flop / dt / 1e12,
        "unit": "TFLOP/s",
        "queries_per_s": len(rows) / dt,
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"{len(rows)} query rows (every {sample_every}th of {S}) of the 32K workload: "
                   f"float64 logits of each visible key, then top-{tk}; {dt:.1f} s"),
        "host_cpu": platform.processor() or platform.machine(),
        "os_cpu_count": os.cpu_count(),
    }


def profile_part(args, dev, q, k, w, cfg):
    """Launch one kernel only, for profiler runs; prints its mean duration."""
    c, tk = cfg["compress_ratio"], cfg["topk"]
    B, S, Skv = cfg["batch"], cfg["seqlen"], cfg["seqlen_kv"]
    if args.part == "copy":
        # plain device copy of a known size: the reference for scaling HBM counters
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        ms, _ = time_loop(lambda: dst.copy_(src), args.steps, args.warmup)
    elif args.part == "v41":
        vin = synth.v41_inputs(**synth.WORKLOADS["v41"])
        vq, vk, vw, va = (vin[x].to(dev) for x in ("queries", "keys", "weights", "allowed"))
        ms, _ = time_loop(lambda: lx.indexer_scores_v41(vq, vk, vw, va), args.steps, args.warmup)
    else:
        logits = torch.empty(B, S, Skv, dtype=torch.float32, device=dev)
        lx.indexer_logits(q, k, w, c, out=logits)
        if args.part == "logits":
            ms, _ = time_loop(lambda: lx.indexer_logits(q, k, w, c, out=logits), args.steps, args.warmup)
        else:
            ms, _ = time_loop(lambda: lx.topk_from_logits(logits, c, tk), args.steps, args.warmup)
    print(json.dumps({"part": args.part, "ms": ms, "steps": args.steps, "warmup": args.warmup}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the copy-bandwidth, 4K cold/warm and 131K fused parts")
    ap.add_argument("--cpu-sample-every", type=int, default=3)
    ap.add_argument("--part", choices=["all", "fused", "logits", "topk", "v41", "copy"], default="all",
                    help="time one kernel only (for profiler runs); the JSON line then covers that part")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the indexer's multi-GPU sharding is not built.", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    lx.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    cfg = synth.WORKLOADS["32k"]
    B, S, Skv, H, D = cfg["batch"], cfg["seqlen"], cfg["seqlen_kv"], cfg["heads"], cfg["index_dim"]
    c, tk = cfg["compress_ratio"], cfg["topk"]
    log("generating the 32K workload")
    inp = synth.v4_inputs(**cfg)
    q, k, w = (inp[x].to(dev) for x in "qkw")
    torch.cuda.synchronize()
    pairs = B * causal_valid_pairs(S, Skv, c)
    flop = 2.0 * H * D * pairs

    # ---- the step: fused scoring + top-k
    if args.part in ("logits", "topk", "v41", "copy"):
        profile_part(args, dev, q, k, w, cfg)
        return
    log("timing the fused step")
    fused_ms, _ = time_loop(lambda: lx.topk(q, k, w, c, tk), args.steps, args.warmup)
    sc_f, ix_f = lx.topk(q, k, w, c, tk)

    parts = {"fused_topk_ms": fused_ms}
    roof_kernel = {"name": "v4_fused_topk_kernel", "ms": fused_ms}
    if args.part == "all":
        log("timing the materialized path")
        logits = torch.empty(B, S, Skv, dtype=torch.float32, device=dev)
        def materialized_step():
            lx.indexer_logits(q, k, w, c, out=logits)
            return lx.topk_from_logits(logits, c, tk)
        step_m_ms, _ = time_loop(materialized_step, args.steps, args.warmup)
        score_ms, _ = time_loop(lambda: lx.indexer_logits(q, k, w, c, out=logits), args.steps, args.warmup)
        topk_ms, _ = time_loop(lambda: lx.topk_from_logits(logits, c, tk), args.steps, args.warmup)
        sc_m, ix_m = lx.topk_from_logits(logits, c, tk)
        same = bool(torch.equal(ix_m, ix_f) and torch.equal(sc_m, sc_f))
        gather_ms, _ = time_loop(lambda: lx.topk_scores(logits, ix_f), args.steps, args.warmup)
        # scores at given indices straight from q, k, w (the topk_indices branch of the pages' entry point)
        at_ms, _ = time_loop(lambda: lx.indexer_scores_at(q, k, w, c, ix_f), args.steps, args.warmup)
        at_same = bool(torch.equal(lx.indexer_scores_at(q, k, w, c, ix_f), sc_f))
        at_pairs = int((ix_f >= 0).sum())
        # algorithmic bytes of the row top-k: read the visible logits, write scores+indices
        topk_bytes = 4.0 * pairs + 8.0 * B * S * tk
        logits_bytes = 4.0 * B * S * Skv + 2.0 * B * S * H * D + 4.0 * B * S * H
        gather_bytes = 4.0 * 2 * B * S * tk + 4.0 * B * S * tk          # idx + value read, scores write
        parts.update({
            "materialized_logits_ms": score_ms,
            "materialized_topk_ms": topk_ms,
            "materialized_step_ms": step_m_ms,
            "materialized_sum_of_parts_ms": score_ms + topk_ms,
            "materialized_scoring_tflops": flop / score_ms / 1e9,
            "materialized_logits_store_gbs": logits_bytes / score_ms / 1e6,
            "topk_from_logits_gbs": topk_bytes / topk_ms / 1e6,
            "topk_from_logits_hbm_frac": topk_bytes / topk_ms / 1e6 / PEAK_HBM_GBS,
            "topk_bytes": topk_bytes,
            "gather_ms": gather_ms,
            "gather_gbs": gather_bytes / gather_ms / 1e6,
            "fused_equals_materialized": same,
            "scores_at_ms": at_ms,
            "scores_at_tflops": 2.0 * H * D * at_pairs / at_ms / 1e9,
            "scores_at_equals_topk_scores": at_same,
            "logits_then_gather_ms": score_ms + gather_ms,
        })
        del logits

        # backward of the selected scores (lix_indexer_backward) with a seeded upstream gradient
        log("timing the backward")
        g_up = synth.upstream_gradient(B, S, tk, 346).to(dev)
        bw_ms, _ = time_loop(lambda: lx.indexer_backward(q, k, w, c, ix_f, g_up), max(3, args.steps // 4), 2)
        parts.update({
            "backward_ms": bw_ms,
            # algorithmic work: four GEMM passes over the selected entries (d twice, dq, dk)
            "backward_gemm_tflops": 4 * 2.0 * H * D * at_pairs / bw_ms / 1e9,
        })
        del g_up

        log("timing the V4.1 workload")
        vcfg = synth.WORKLOADS["v41"]
        vin = synth.v41_inputs(**vcfg)
        vq, vk, vw, va = (vin[x].to(dev) for x in ("queries", "keys", "weights", "allowed"))
        v41_ms, _ = time_loop(lambda: lx.indexer_scores_v41(vq, vk, vw, va), args.steps, args.warmup)
        v41_scores = lx.indexer_scores_v41(vq, vk, vw, va)
        v41_topk_ms, _ = time_loop(lambda: lx.topk_bf16(v41_scores, 512), args.steps, args.warmup)
        Lq, G = vcfg["local_sequence"], vcfg["global_compressed"]
        v41_bytes = (2.0 * Lq * H * D + 2.0 * G * D + 2.0 * Lq * H + 1.0 * Lq * G + 2.0 * Lq * G)
        allowed_pairs = int(vin["allowed"].sum())
        parts.update({
            "v41_ms": v41_ms,
            "v41_gbs": v41_bytes / v41_ms / 1e6,
            "v41_hbm_frac": v41_bytes / v41_ms / 1e6 / PEAK_HBM_GBS,
            "v41_allowed_fraction": allowed_pairs / (Lq * G),
            "v41_allowed_tflops": 2.0 * H * D * allowed_pairs / v41_ms / 1e9,
            "v41_topk512_ms": v41_topk_ms,
            "v41_topk512_gbs": (2.0 * Lq * G + 6.0 * Lq * 512) / v41_topk_ms / 1e6,
        })

        if not args.no_extra:
            log("timing a library GEMM, copy bandwidth and the 4K workload")
            parts.update(extra_parts(dev, args.steps, args.warmup))
            parts["topk_frac_of_copy"] = topk_bytes / topk_ms / 1e6 / parts["copy_gbs"]

    # The step is the faster of the two routes to the same forward; both are reported.
    if args.part == "all" and parts["materialized_step_ms"] < fused_ms:
        step_ms = parts["materialized_step_ms"]
        path = "materialized: lix_indexer_logits then lix_topk over the logits"
        roof_kernel = {"name": "v4_logits_kernel", "ms": parts["materialized_logits_ms"]}
    else:
        step_ms = fused_ms
        path = "fused: lix_topk scoring and selecting on chip"
    value = flop / step_ms / 1e9
    achieved = flop / roof_kernel["ms"] / 1e9
    traffic = recorded_traffic(roof_kernel["name"])
    measured = {}
    if "gemm_bf16_tflops" in parts:
        measured = {"gemm_bf16_tflops": parts["gemm_bf16_tflops"], "copy_gbs": parts["copy_gbs"],
                    "frac_of_gemm": achieved / parts["gemm_bf16_tflops"]}
    result = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "32k lightning-indexer forward (scoring + top-k)", "path": path, "batch": B,
                   "seqlen": S, "seqlen_kv": Skv, "heads": H, "index_dim": D, "compress_ratio": c,
                   "topk": tk, "causal_valid_pairs": pairs},
        "queries_per_s": B * S / (step_ms * 1e-3),
        "roofline": {"bound": "mfma", "kernel": roof_kernel["name"], "achieved": achieved,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                     "traffic": traffic, "measured_peaks": measured},
        "parts": parts,
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle sample")
        result["cpu_baseline"] = cpu_baseline(inp, cfg, args.cpu_sample_every)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
