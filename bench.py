"""Benchmark of the packed indexer step (score + block top-k) on one MI355X.

One step is one call of the hot path over one batch: the NVFP4 store of the
step's new keys (each request's last packed_queries tokens; NVFP4 workload
only), the packed block scoring and the forced top-k, for every request of
one layer.  The NVFP4 pool itself is quantized once before timing, and that
whole-pool store is timed and reported on its own.  By default the workload is 32 requests x 4 draft
rows x 4 index heads, fp8 e4m3 keys, contexts U[491520, 524285], 3 graph-pad
requests (about 2.08 GB of K per step, eight times the 256 MB Infinity Cache,
so back-to-back steps stream K from HBM).

Prints one JSON line: the metric (us per index step, wall clock over the
timed steps), the dominant kernel's roofline against the 8 TB/s HBM peak
(algorithmic bytes over its mean duration, from HIP events on its launch
stream in a separate pass of at least 20 steps), the rate at which the part
reads the same K pages with nothing else to do (``idx_probe_read``), the
CPU oracle timed on the host as a reported baseline (all cores, and one
thread on a sixteenth of that sample), and, in the default run, every other
workload's step, kernels and score roofline under ``other_workloads``.

    python bench.py [--gpus 1] [--steps 100] [--warmup 10] [--config 3] [--k-format fp8]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

METRIC = "index step µs (score+top-k) and achieved HBM GB/s vs peak, 1 MI355X"
HBM_PEAK_GBPS = 8000.0
MFMA_PEAK_TFLOPS = 2500.0   # dense bf16 / f16 MFMA (fp8 keys are widened to bf16, NVFP4 to f16)


def parse() -> argparse.Namespace:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=3,
                    help="workload index 0..5 (default 3; 5 is the prefill scorer)")
    ap.add_argument("--local-blocks", type=int, default=None)
    ap.add_argument("--k-format", choices=("bf16", "fp8", "nvfp4"), default=None,
                    help="store the workload's keys in this format instead (same shape)")
    ap.add_argument("--event-steps", type=int, default=None,
                    help="steps of the event-timed kernel pass (default max(20, min(steps, 100)))")
    ap.add_argument("--no-read-ceiling", action="store_true",
                    help="skip the plain-read measurement of the step's K pages")
    ap.add_argument("--attn-q-per-kv", type=int, default=4,
                    help="query heads per KV head of the sparse attention measured after the step "
                         "(0: skip it; packed_queries * this must be <= 64)")
    ap.add_argument("--attn-kv-format", choices=("bf16", "fp8", "both"), default="both",
                    help="K/V format(s) of the sparse attention measured after the step")
    ap.add_argument("--score-mode", choices=("max", "lse"), default="max",
                    help="block reduction: max (default) or lse")
    ap.add_argument("--sm-scale", type=float, default=1 / 128 ** 0.5,
                    help="softmax scale of the lse mode (default 1/sqrt(128))")
    ap.add_argument("--other-workloads", dest="other_workloads", action="store_true", default=None,
                    help="also time the other decode workloads, the ~150K shape with fp8 keys and the "
                         "prefill workload (default: on for the headline run)")
    ap.add_argument("--no-other-workloads", dest="other_workloads", action="store_false")
    ap.add_argument("--other-first", action="store_true",
                    help="time the other workloads before the headline one instead of after it")
    ap.add_argument("--other-pause", type=float, default=10.0,
                    help="seconds of idle GPU between the headline workload and the others")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-requests", type=int, default=None,
                    help="requests in the CPU-oracle sample (default: all real requests)")
    ap.add_argument("--cpu-rows", type=int, default=512,
                    help="packed rows of the first request in the CPU-oracle sample when a request "
                         "packs more than 16 rows (default 512)")
    ap.add_argument("--calibration-copy", type=int, default=0, metavar="MiB",
                    help="first run a plain device copy of this many MiB three times (a kernel of "
                         "known traffic, to scale hardware byte counters)")
    return ap.parse_args()


# The sources each measured kernel is built from (under csrc/).
KERNEL_SOURCES = {
    "score_kernel": ("device.h", "tile.h", "score.hip"),
    "rows_kernel": ("device.h", "tile.h", "score_rows.hip"),
    "attn_partial_kernel": ("device.h", "attn.hip"),
    "fp4_store_wide_kernel": ("device.h", "fp4_store.hip"),
}


def source_digest(kernel: str) -> str:
    """First 16 hex digits of the sha256 of a kernel's sources and the C
    header: a counter summary taken on other sources is stale."""
    h = hashlib.sha256()
    csrc = ROOT / "sparse_attention_lightning_amd" / "csrc"
    for f in [csrc / n for n in KERNEL_SOURCES[kernel]] + [ROOT / "include" / "idx.h"]:
        h.update(f.read_bytes())
    return h.hexdigest()[:16]


def traffic_from_profiles(kernel: str, fmt: str, workload: str):
    """HBM bytes per launch from a committed counter summary, if it was taken
    on the kernel's current sources (else None)."""
    digest = source_digest(kernel)
    f = ROOT / "profiles" / f"{kernel}_{fmt}_{workload}_traffic.md"
    if not f.exists():
        return None
    text = f.read_text()
    m_src = re.search(r"source digest:\s*([0-9a-f]+)", text)
    m_b = re.search(r"hbm bytes per launch:\s*([0-9.eE+]+)", text)
    if not m_src or not m_b or m_src.group(1) != digest:
        return None
    return float(m_b.group(1))


def main() -> int:
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU: the indexer step has no multi-GPU path in this build; "
              "requests shard across GPUs with no exchange, so one GPU's share is this same step "
              "on fewer requests", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from sparse_attention_lightning_amd import idx as I
    from sparse_attention_lightning_amd import workloads as W

    torch.cuda.set_device(0)
    dev = "cuda"
    if args.calibration_copy:
        src = torch.ones(args.calibration_copy << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.other_workloads is None:
        args.other_workloads = args.config == 3 and args.k_format is None and args.score_mode == "max"
    others = None
    if args.other_workloads and args.other_first:
        others = bench_other_workloads(n_ev=max(20, min(args.steps, 50)), warmup=min(args.warmup, 5))
        torch.cuda.empty_cache()
        time.sleep(args.other_pause)
    kf = {None: None, "bf16": W.K_BF16, "fp8": W.K_FP8_E4M3, "nvfp4": W.K_NVFP4}[args.k_format]
    w = W.config(args.config, device=dev, local_blocks=args.local_blocks, k_format=kf)
    mode = ({"score_mode": I.IDX_SCORE_LSE, "sm_scale": args.sm_scale} if args.score_mode == "lse"
            else {"score_mode": I.IDX_SCORE_MAX})
    st = Step(w, mode, dev, time_pool=True)
    rows, K, MB = w.rows, w.topk, w.max_blocks
    outs, p, fp4, pool_store = st.outs, st.p, st.fp4, st.pool_store
    P, H = w.packed_queries, w.gqa
    k_bytes, score_bytes, step_bytes = st.k_bytes, st.score_bytes, st.step_bytes
    flush = st.flush
    stream = torch.cuda.current_stream()

    def one_step(ev=None):
        st.run(stream, ev)

    for _ in range(args.warmup):
        if flush is not None:
            flush.sum()
        one_step()
    torch.cuda.synchronize()

    # 1. wall clock over the timed steps, with no event inside
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        if flush is not None:
            flush.sum()
        one_step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # 2. kernel durations from HIP events on the launch stream, in a pass of
    # its own (an event between two launches costs a few microseconds, which
    # the wall-clock pass must not carry).  When the cache is flushed between
    # steps the step time is the mean of the event-timed kernels, since the
    # wall clock then includes the flush.
    n_ev = args.event_steps if args.event_steps else max(20, min(args.steps, 100))
    t_ev = st.event_pass(stream, n_ev)
    store_ms, score_ms, topk_ms = t_ev["store"], t_ev["score"], t_ev["topk"]
    step_ms = [a + b + c for a, b, c in zip(store_ms, score_ms, topk_ms)]
    ms_per_step = wall * 1e3 / args.steps if flush is None else float(np.mean(step_ms))
    score_mean_s = float(np.mean(score_ms)) / 1e3
    achieved = score_bytes / score_mean_s / 1e9
    fmt_name = {W.K_BF16: "bf16", W.K_FP8_E4M3: "fp8", W.K_NVFP4: "nvfp4"}[w.k_format]
    # the committed counter profiles are of the max reduction
    kname = "score_kernel" if P * H <= 16 else "rows_kernel"
    traffic = traffic_from_profiles(kname, fmt_name, w.name) if args.score_mode == "max" else None

    if P * H <= 16:
        roofline = {"kernel": "score_kernel", "bound": "hbm", "achieved": round(achieved, 1),
                    "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                    "traffic": traffic, "algorithmic_bytes": score_bytes}
    else:
        # many rows a request (prefill): 256 flop per (row, visible token);
        # K crosses HBM once, so the matrix cores bound the kernel
        rl = w.row_len.cpu().numpy().astype(np.int64).reshape(w.n_req, P)[: w.n_real]
        flops = int(rl.sum()) * H * 2 * 128
        tflops = flops / score_mean_s / 1e12
        roofline = {"kernel": "rows_kernel", "bound": "mfma", "achieved": round(tflops, 1),
                    "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(tflops / MFMA_PEAK_TFLOPS, 4),
                    "traffic": traffic, "algorithmic_flops": flops, "algorithmic_bytes": score_bytes}
    line = {
        "metric": METRIC,
        "value": round(ms_per_step * 1e3, 2),
        "unit": "us",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {W.K_BF16: "bf16", W.K_FP8_E4M3: "fp8_e4m3->bf16", W.K_NVFP4: "nvfp4->f16"}[w.k_format],
        "data": "synthetic",
        "config": {
            "workload": w.name, "requests": w.n_real, "graph_pads": w.n_req - w.n_real,
            "block_score": args.score_mode,
            **({"sm_scale": args.sm_scale} if args.score_mode == "lse" else {}),
            "packed_queries": P, "gqa": H, "head_dim": 128, "block": 128,
            "k_format": W.FORMAT_NAMES[w.k_format], "q": "bf16",
            "context_tokens": [int(w.req_len.min()), int(w.req_len.max() + P - 1)],
            "topk": K, "init_blocks": w.init_blocks, "local_blocks": w.local_blocks,
            "k_bytes_per_step": k_bytes, "parallelism": "single GPU",
            "cache": ("flushed between steps" if flush is not None
                      else f"K is {k_bytes / (256 << 20):.1f}x the 256 MB MALL"),
        },
        "achieved_GBps": round(step_bytes / (ms_per_step / 1e3) / 1e9, 1),
        "kernels_us": {"score": round(score_mean_s * 1e6, 2),
                       "topk": round(float(np.mean(topk_ms)) * 1e3, 2),
                       },
        "kernel_samples": n_ev,
        # spread of the event-timed score kernel over the event pass
        "score_us_p10_p50_p90": [round(float(x) * 1e3, 2) for x in np.percentile(score_ms, [10, 50, 90])],
        "roofline": roofline,
        "cpu_baseline": None,
    }
    if fp4:
        line["fp4_store_step_tokens"] = int(st.step_staging.shape[0])
        line["fp4_store_step"] = "in the score launch (idx_score_packed_fp4)"
        line["fp4_store_pool"] = pool_store
    if args.attn_q_per_kv and P <= 16 and P * args.attn_q_per_kv <= 64:
        for kvf in ("bf16", "fp8"):
            if args.attn_kv_format in (kvf, "both"):
                key = "sparse_attn" if kvf == "bf16" else "sparse_attn_fp8kv"
                line[key] = bench_attn(w, outs["topk_ids"], args.attn_q_per_kv, kvf, flush, stream,
                                       n_ev=max(10, min(args.steps, 50)))
    if not args.no_read_ceiling and P * H <= 16:
        line["hbm_read_ceiling"] = read_ceiling(w, flush, stream)
        line["score_frac_of_page_gather"] = round(achieved / line["hbm_read_ceiling"]["page_gather_GBps"], 4)

    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_requests, args.cpu_rows, mode)
    if others is None and args.other_workloads:
        del st, outs, p, w, flush, one_step
        torch.cuda.empty_cache()
        time.sleep(args.other_pause)
        others = bench_other_workloads(n_ev=max(20, min(args.steps, 50)), warmup=min(args.warmup, 5))
    if others is not None:
        line["other_workloads"] = others
    print(json.dumps(line), flush=True)
    return 0


class Step:
    """One workload's step: its parameters and outputs, the NVFP4 store of the
    step's new keys (each request's last packed_queries tokens; the whole pool
    is stored once first, and that store is timed when ``time_pool``), the
    algorithmic byte counts, and the 1 GiB read that leaves the caches without
    K between steps when the 256 MB MALL could hold it."""

    def __init__(self, w, mode: dict, dev: str, time_pool: bool = False):
        import numpy as np
        import torch

        from sparse_attention_lightning_amd import idx as I
        from sparse_attention_lightning_amd import workloads as W

        self.w = w
        rows, K, MB = w.rows, w.topk, w.max_blocks
        self.outs = {"block_scores": torch.empty((rows, MB), dtype=torch.float32, device=dev),
                     "topk_ids": torch.empty((rows, K), dtype=torch.int32, device=dev),
                     "topk_scores": torch.empty((rows, K), dtype=torch.float32, device=dev)}
        self.fp4 = w.k_format == W.K_NVFP4
        self.pool_store = None
        self.step_staging = self.step_slots = None
        if self.fp4:
            I.idx_fp4_store(w.staging, w.slot_mapping, w.k, w.k_scale)
            if time_pool:
                # median of 5 calls, each after a 1 GiB read that leaves the
                # caches without its data
                evict = torch.ones(1 << 28, dtype=torch.int32, device=dev)
                pool_ms = []
                for _ in range(5):
                    evict.sum()
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record()
                    I.idx_fp4_store(w.staging, w.slot_mapping, w.k, w.k_scale)
                    e1.record()
                    torch.cuda.synchronize()
                    pool_ms.append(e0.elapsed_time(e1))
                del evict
                n_pool = w.staging.shape[0]
                pool_us = float(np.median(pool_ms)) * 1e3
                self.pool_store = {"tokens": n_pool, "us": round(pool_us, 2), "calls": 5,
                                   "GBps": round(n_pool * (256 + 72 + 8) / (pool_us / 1e6) / 1e9, 1),
                                   "algorithmic_bytes": n_pool * (256 + 72 + 8),
                                   "traffic": traffic_from_profiles("fp4_store_wide_kernel", "nvfp4", w.name)}
            ends = np.cumsum(w.group_len()[: w.n_real].astype(np.int64))
            new_rows = np.concatenate([np.arange(e - w.packed_queries, e) for e in ends])
            sel = torch.as_tensor(new_rows, device=dev)
            self.step_staging = w.staging.index_select(0, sel).contiguous()
            self.step_slots = w.slot_mapping.index_select(0, sel).contiguous()
            # the step's keys go in through the score launch (idx_score_packed_fp4)
            self.keys = I.make_new_keys(self.step_staging, self.step_slots)
        self.p = I.make_params(k_format=w.k_format, q=w.q, k=w.k, k_scale=w.k_scale, req_slot=w.req_slot,
                               block_table=w.block_table, row_len=w.row_len, packed_queries=w.packed_queries,
                               gqa=w.gqa, topk=K, init_blocks=w.init_blocks, local_blocks=w.local_blocks,
                               max_blocks=MB, n_slot_rows=w.n_slot_rows, n_pages=w.n_pages, **mode,
                               **self.outs)
        # algorithmic bytes (token-exact K of each real request's longest row)
        P, H = w.packed_queries, w.gqa
        self.k_bytes = w.k_tokens() * W.BYTES_PER_TOKEN[w.k_format]
        real_rows = w.n_real * P * H
        self.score_bytes = (self.k_bytes + real_rows * 256 + w.pool_pages_used() * 4
                            + (w.n_req * P + w.n_req) * 4)
        if self.fp4:  # the step's keys: staging and slot in, payload and scales out
            self.score_bytes += self.step_staging.shape[0] * (256 + 8 + 72)
        self.step_bytes = self.score_bytes + rows * K * 8
        # reads leave clean lines, so the step pays no write-back
        self.flush = torch.ones(1 << 28, dtype=torch.int32, device=dev) if self.k_bytes < (1 << 30) else None

    def run(self, stream, ev=None):
        """One step on ``stream``; ``ev``: events ev[1..3] around the
        scoring (with the NVFP4 store of the step's new keys, which the score
        launch makes itself) and the selection."""
        from sparse_attention_lightning_amd import idx as I

        if ev is not None:
            ev[1].record(stream)
        if self.fp4:
            I.idx_score_packed_fp4(self.p, self.keys, stream)  # the NVFP4 store of the step's keys included
        else:
            I.idx_score_packed(self.p, stream)
        if ev is not None:
            ev[2].record(stream)
        I.idx_block_topk(self.p, stream)
        if ev is not None:
            ev[3].record(stream)

    def step_pass(self, stream, n: int) -> list:
        """Whole-step durations (ms) over ``n`` steps, one event pair around
        each step (the gaps between its launches included), each after the
        cache-clearing read when there is one."""
        import torch

        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n)]
        for e in ev:
            if self.flush is not None:
                self.flush.sum()
            e[0].record(stream)
            self.run(stream)
            e[1].record(stream)
        torch.cuda.synchronize()
        return [e[0].elapsed_time(e[1]) for e in ev]

    def event_pass(self, stream, n: int) -> dict:
        """Kernel durations (ms lists) from HIP events on ``stream`` over
        ``n`` steps, each after the cache-clearing read when there is one."""
        import torch

        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(n)]
        for e in ev:
            if self.flush is not None:
                self.flush.sum()
            self.run(stream, e)
        torch.cuda.synchronize()
        return {"store": [0.0] * n,  # no launch of its own (NVFP4: inside the score launch)
                "score": [e[1].elapsed_time(e[2]) for e in ev],
                "topk": [e[2].elapsed_time(e[3]) for e in ev]}


# The other workloads measured after the headline one, with the keys' format
# override of the ~150K shape (fp8 beside NVFP4, the comparison the pages make).
OTHER_WORKLOADS = ((1, None), (2, None), (4, None), (4, "fp8"), (5, None), (0, None))


def bench_other_workloads(n_ev: int, warmup: int) -> dict:
    """Each other workload's step in max mode, ``n_ev`` steps after
    ``warmup``, a 1 GiB read before each step when K fits the MALL: the step
    from one event pair around each step (launch gaps included), the
    kernels from the four-event pass, the score kernel's roofline fraction,
    and the step against the 70 %-of-HBM-peak time of its K bytes."""
    import numpy as np
    import torch

    from sparse_attention_lightning_amd import idx as I
    from sparse_attention_lightning_amd import workloads as W

    stream = torch.cuda.current_stream()
    res = {}
    for cfg, kfname in OTHER_WORKLOADS:
        kf = {None: None, "fp8": W.K_FP8_E4M3}[kfname]
        w = W.config(cfg, device="cuda", k_format=kf)
        st = Step(w, {"score_mode": I.IDX_SCORE_MAX}, "cuda")
        for _ in range(warmup):
            if st.flush is not None:
                st.flush.sum()
            st.run(stream)
        torch.cuda.synchronize()
        step_us = float(np.mean(st.step_pass(stream, n_ev))) * 1e3
        t = st.event_pass(stream, n_ev)
        score_s = float(np.mean(t["score"])) / 1e3
        P, H = w.packed_queries, w.gqa
        entry = {"k_format": W.FORMAT_NAMES[w.k_format], "step_us": round(step_us, 2),
                 "kernels_us": {"score": round(score_s * 1e6, 2), "topk": round(float(np.mean(t["topk"])) * 1e3, 2),
                                },
                 "k_bytes_per_step": st.k_bytes}
        if P * H <= 16:
            gbps = st.score_bytes / score_s / 1e9
            entry["score_roofline"] = {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS,
                                       "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4)}
            if w.n_real > 2:  # the tiny workload is launch-bound: no bar
                bar = st.k_bytes / (0.7 * HBM_PEAK_GBPS * 1e9) * 1e6
                entry["step_bar_us_70pct_hbm"] = round(bar, 1)
                entry["step_frac_of_hbm_peak"] = round(st.k_bytes / (step_us / 1e6) / 1e9 / HBM_PEAK_GBPS, 4)
        else:
            rl = w.row_len.cpu().numpy().astype(np.int64).reshape(w.n_req, P)[: w.n_real]
            tflops = int(rl.sum()) * H * 2 * 128 / score_s / 1e12
            entry["score_roofline"] = {"bound": "mfma", "achieved": round(tflops, 1), "peak": MFMA_PEAK_TFLOPS,
                                       "unit": "TFLOP/s", "frac": round(tflops / MFMA_PEAK_TFLOPS, 4)}
        entry["steps"] = n_ev
        entry["timing"] = "step: one event pair a step; kernels: an event pair each, in a pass of their own"
        res[w.name] = entry
        del st, w
        torch.cuda.empty_cache()
    a, b = res.get("64req_150k_nvfp4"), res.get("64req_150k_fp8")
    if a and b:
        res["nvfp4_over_fp8_step"] = round(a["step_us"] / b["step_us"], 3)
    return res


def bench_attn(w, topk_ids, G: int, kvf: str, flush, stream, n_ev: int) -> dict:
    """The sparse attention over the blocks the step just selected: K and V
    pools (bf16 or fp8 e4m3, ``kvf``) of the workload's page count, G query
    heads per KV head, softmax scale 1/sqrt(128).  Timed with HIP events
    around each call (one or two launches), mean of ``n_ev`` calls after 3
    warm-ups.  Algorithmic bytes: for every (request, KV head), the K and V
    of each block in the union of its draft rows' selections, up to the
    longest of those rows' visible tokens in it (2 x 256 B a token in bf16,
    2 x 128 B in fp8), plus queries, ids and outputs."""
    import numpy as np
    import torch

    from sparse_attention_lightning_amd import idx as I
    from sparse_attention_lightning_amd import workloads as W

    at = W.make_attn(w, G, kv_format=W.K_BF16 if kvf == "bf16" else W.K_FP8_E4M3)
    P, H, R = w.packed_queries, w.gqa, w.n_req
    out = torch.empty_like(at.q)
    lse = torch.empty(at.q.shape[:3], dtype=torch.float32, device=at.q.device)
    p = I.make_attn_params(q=at.q, k=at.k, v=at.v, req_slot=w.req_slot, block_table=w.block_table,
                           row_len=w.row_len, topk_ids=topk_ids, out=out, lse=lse, sm_scale=128 ** -0.5)
    for _ in range(3):
        I.idx_sparse_attn(p, stream)
    torch.cuda.synchronize()
    ms = []
    for _ in range(n_ev):
        if flush is not None:
            flush.sum()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        I.idx_sparse_attn(p, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
    # algorithmic bytes from the selection
    ids = topk_ids.cpu().numpy().reshape(R, P, H, -1)
    lens = w.row_len.cpu().numpy().reshape(R, P).astype(np.int64)
    slots = w.req_slot.cpu().numpy()
    tokens = union = selected = 0
    for r in range(R):
        if not (0 <= slots[r] < w.n_slot_rows):
            continue
        nb = (lens[r] + 127) // 128
        for h in range(H):
            best = {}
            for j in range(P):
                for b in ids[r, j, h]:
                    if 0 <= b < nb[j]:
                        selected += 1
                        best[int(b)] = max(best.get(int(b), 0), int(min(128, lens[r, j] - 128 * b)))
            union += len(best)
            tokens += sum(best.values())
    rows = R * P * H * G
    kv_token = 512 if kvf == "bf16" else 256
    nbytes = tokens * kv_token + rows * 256 * 2 + rows * 4 + ids.size * 4
    us = float(np.mean(ms)) * 1e3
    gbps = nbytes / (us / 1e6) / 1e9
    del at, out, lse, p
    torch.cuda.empty_cache()
    traffic = traffic_from_profiles("attn_partial_kernel", kvf, w.name)
    return {"us": round(us, 2), "us_p10_p50_p90": [round(float(x) * 1e3, 2) for x in np.percentile(ms, [10, 50, 90])],
            "kv_format": kvf, "q_per_kv": G, "kv_heads": H, "query_heads": rows, "selected_blocks": int(selected),
            "union_blocks": int(union), "kv_bytes": int(tokens * kv_token), "algorithmic_bytes": int(nbytes),
            "achieved_GBps": round(gbps, 1), "frac_of_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4),
            "roofline": {"kernel": "attn_partial_kernel + attn_combine_kernel (one call)", "bound": "hbm",
                         "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": traffic},
            "calls": n_ev}


def read_ceiling(w, flush, stream, reps: int = 10) -> dict:
    """How fast the part reads the step's K pages with nothing else to do.

    ``idx_probe_read`` streams the pages the score kernel reads (each real
    request's blocks up to its longest row, in step order, every workgroup
    an equal contiguous share) and, for comparison, the whole K pool in
    address order; median of ``reps`` event-timed launches each, with
    ordinary and with non-temporal loads.  NVFP4 pages are measured on the
    payload plane (8 KB a page; the score kernel also reads 1 KB of scales)."""
    import numpy as np
    import torch

    from sparse_attention_lightning_amd import idx as I
    from sparse_attention_lightning_amd import workloads as W

    page_bytes = {W.K_BF16: 32768, W.K_FP8_E4M3: 16384, W.K_NVFP4: 8192}[w.k_format]
    bt = w.block_table.cpu().numpy()
    slots = w.req_slot.cpu().numpy()
    nbg = (w.group_len()[: w.n_real].astype(np.int64) + 127) // 128
    units = np.concatenate([bt[slots[r], : nbg[r]] for r in range(w.n_real)]).astype(np.int32)
    units_t = torch.as_tensor(units, device=w.k.device)
    base = w.k.view(torch.uint8)
    sink = torch.empty(4096, dtype=torch.int32, device=w.k.device)
    out = {"unit": "GB/s"}
    for name, u, n in (("page_gather", units_t, len(units)), ("contiguous", None, w.n_pages)):
        best = 0.0
        for nt in (False, True):
            ms = []
            for _ in range(reps):
                if flush is not None:
                    flush.sum()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                I.idx_probe_read(base, page_bytes, u, n_units=n, nt=nt, sink=sink, stream=stream)
                e1.record(stream)
                torch.cuda.synchronize()
                ms.append(e0.elapsed_time(e1))
            gbps = n * page_bytes / (float(np.median(ms)) / 1e3) / 1e9
            out[f"{name}{'_nt' if nt else ''}_GBps"] = round(gbps, 1)
            best = max(best, gbps)
        out[f"{name}_GBps"] = round(best, 1)
    out["bytes"] = {"page_gather": int(len(units)) * page_bytes, "contiguous": int(w.n_pages) * page_bytes}
    out["method"] = ("idx_probe_read: 16-byte loads only, 16 a thread in flight, a resident grid of "
                     "512-thread workgroups each on an equal contiguous share of the units; "
                     "page_gather = the step's K pages in step order, contiguous = the whole K pool in "
                     "address order; median of %d event-timed launches; best of ordinary and "
                     "non-temporal loads" % reps)
    return out


def cpu_info() -> dict:
    model = "unknown"
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                model = ln.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count()
    return {"cpu_model": model, "nproc": usable, "cpu_count": os.cpu_count()}


def cpu_baseline(w, n_sample, n_rows, mode) -> dict:
    """The oracle, untuned, on the host cores, scaled to one full step.

    Up to 16 rows a request: the step over the first ``n_sample`` real
    requests (default all), scaled by request-tokens.  More rows a request
    (prefill): the first ``n_rows`` packed rows of the first request, scaled
    by the summed row lengths (the scoring work is linear in them)."""
    import numpy as np

    from oracle.binding import Oracle
    from sparse_attention_lightning_amd import workloads as W

    o = Oracle()
    P, H = w.packed_queries, w.gqa
    if w.k_format == W.K_NVFP4:
        a = w.oracle_args(w.k.cpu().numpy(), w.k_scale.cpu().numpy())
    else:
        a = w.oracle_args()
    R = a["n_req"]
    q_all = a["q"].reshape(R, P * H, 128)
    len_all = a["row_len"].reshape(R, P)
    if P * H > 16:
        n, p = 1, max(1, min(n_rows, P))
        lw = len_all[: w.n_real].astype(np.int64)
        frac = lw[0, :p].sum() / lw.sum()
        what = f"score+top-k of the first {p} of {P} packed rows of request 0 ({w.n_real} requests)"
        scale = "scaled by summed row lengths"
    else:
        n = w.n_real if n_sample is None else min(n_sample, w.n_real)
        p = P
        lmax = w.group_len()[: w.n_real].astype(np.int64)
        frac = lmax[:n].sum() / lmax.sum()
        what = (f"score+top-k of the first {n} of {w.n_real} requests "
                f"({int(lmax[:n].sum())} request-tokens)")
        scale = "scaled by token count"
    q = q_all[:n, : p * H].reshape(-1, H, 128)
    sub = dict(a, **mode, n_req=n, packed_queries=p, q=np.ascontiguousarray(q),
               req_slot=np.ascontiguousarray(a["req_slot"][:n]),
               row_len=np.ascontiguousarray(len_all[:n, :p].reshape(-1)))
    times = []
    for _ in range(3):
        t0 = time.perf_counter()
        o.step(**sub)
        times.append(time.perf_counter() - t0)
    t = float(np.median(times))
    out = {"value": round(float(t / frac) * 1e6, 1), "unit": "us", "cores": o.threads(),
           "kind": "oracle", "sample": f"{what}, median of 3, {scale}", **cpu_info()}
    # one thread, on a sixteenth of that sample (median of 3), scaled the same way
    if P * H > 16:
        p1 = max(1, p // 16)
        frac1 = lw[0, :p1].sum() / lw.sum()
        sub1 = dict(sub, packed_queries=p1, q=np.ascontiguousarray(q_all[:1, : p1 * H].reshape(-1, H, 128)),
                    row_len=np.ascontiguousarray(len_all[:1, :p1].reshape(-1)))
        what1 = f"the first {p1} packed rows of request 0"
    else:
        n1 = max(1, n // 16)
        frac1 = lmax[:n1].sum() / lmax.sum()
        sub1 = dict(sub, n_req=n1, q=np.ascontiguousarray(q_all[:n1].reshape(-1, H, 128)),
                    req_slot=np.ascontiguousarray(a["req_slot"][:n1]),
                    row_len=np.ascontiguousarray(len_all[:n1].reshape(-1)))
        what1 = f"the first {n1} requests"
    before = o.set_threads(1)
    try:
        t1s = []
        for _ in range(3):
            t0 = time.perf_counter()
            o.step(**sub1)
            t1s.append(time.perf_counter() - t0)
    finally:
        o.set_threads(before)
    t1 = float(np.median(t1s))
    out["value_1thread"] = round(float(t1 / frac1) * 1e6, 1)
    out["sample_1thread"] = f"{what1}, median of 3, {scale}"
    return out


if __name__ == "__main__":
    sys.exit(main())
