"""Benchmark: one decode-verify step of block-verify attention on MI355X.

Workload: 1 request, context 32768 tokens, a block of 16 drafted tokens, 24
query heads / 4 kv heads, head dim 256, 16-token pages placed at random in a
65536-page int8 pool (the long-context single-stream case; the pages measure
decode on prompts up to 32K tokens -- Splash community summary on
discuss.pytorch.kr, section "benchmark method").

One step = the whole hot path on one batch: append the drafted block's K/V
(quantise to int8 into the paged pools) and run block-verify attention over the
full context, as one call (splash_verify_attn_append: the workgroups holding
the block's pages quantise it, attend to it and store it).  The same work as
two calls, the append and then the verify call, is reported beside it.
Inputs are resident in HBM before timing.  Steps rotate over R
disjoint replicas of the request's pages (identical values, R * 68 MB >= 1 GiB)
so that the 256 MB Infinity Cache cannot serve the context from one step to
the next.

Timing.  Calls are captured in HIP graphs of C consecutive calls (C = the
largest divisor of --steps up to 16), as a serving loop captures the calls of
several layers in one graph; a graph launch costs several microseconds of idle
GPU that a per-call graph would charge to every call.  There are enough graphs,
each on its own window of replicas, that consecutive replays cycle through all
R replicas whatever --steps is.  The timed replays are queued behind a
device-side sleep, so the GPU runs them back to back whatever the host's
launch rate; events on the launch stream bracket exactly --steps calls, and
every figure is the median over 5 such batches.

The other workloads (tiny latency case, 4K context, four requests sharing a
prefix, 16 requests of 32K with ragged drafts) are timed the same way, each
over replicas that together exceed 1 GiB (the 16 x 32K batch is 1.09 GB by
itself).

Prints one JSON line.  `value` is the step's algorithmic HBM bytes (int8 K and
V plus fp16 scales per context token and kv head, q in, out, block table and
lengths, and the append's source rows, codes and scales) over the step time.
`roofline` is the verify call at 32K: its algorithmic bytes over its time.
`roofline.traffic` is the measured HBM bytes per call, taken from the
committed counter summary when that summary was made from the kernel source
now in the tree (else null).  `cpu_baseline` times the CPU oracle on the host
cores.

Host-only helper modes (no GPU) turn rocprofv3 CSV output into the short text
summaries kept under profiles/:
    python bench.py --summarize-stats DIR PHASE_LOG CMD...
    python bench.py --summarize-traffic FETCH_DIR WRITE_DIR PHASE_LOG CMD...
    python bench.py --summarize-counters DIR PHASE_LOG CMD...
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import math
import os
import sys
import time
from pathlib import Path

import numpy as np

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0                            # dense fp16/bf16 MFMA, MI355X
METRIC = "verify-attn µs/call + achieved HBM GB/s (% of peak) at 32K ctx, T=16"
WORKLOAD = "verify 1 req x ctx 32768, T=16 drafts, 24q/4kv heads, D=256, int8 KV in 16-token pages"
PART_KERNEL = "verify_partition_kernel<256, 6, 0>"        # the causal instantiation at D = 256, G = 6
TRAFFIC_SUMMARY = ROOT / "profiles" / "verify_d256_ctx32k_hbm_traffic.md"
# sources the verify kernels are compiled from (their hash stamps counter summaries)
KERNEL_SOURCES = ["speculative_decode_attention_amd/csrc/verify_attn.hip",
                  "speculative_decode_attention_amd/csrc/device.h",
                  "speculative_decode_attention_amd/csrc/launch.h"]
CALIB_MIB = 512
DEFAULT_STEPS = 200
BATCHES = 5
ROTATE_BYTES = 1 << 30                                    # replicas rotated per timed leg: >= 1 GiB


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=DEFAULT_STEPS)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--splits", type=int, default=0, help="0 = the library's preset")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="repeat whole oracle calls until this much wall time has passed")
    ap.add_argument("--copy-calibration", action="store_true",
                    help=f"also run a plain {CALIB_MIB} MiB device copy (for counter calibration)")
    ap.add_argument("--legs", default="all",
                    help="comma list of extra legs (configs,accept,prefill,scaling,ceiling) or all / none")
    ap.add_argument("--phase-log", metavar="FILE",
                    help="write the kernel launches of each phase (for the rocprofv3 summaries)")
    ap.add_argument("--summarize-stats", nargs="+", metavar="ARG")
    ap.add_argument("--summarize-traffic", nargs="+", metavar="ARG")
    ap.add_argument("--summarize-counters", nargs="+", metavar="ARG")
    ap.add_argument("--oracle-one-thread", metavar="DIR", help=argparse.SUPPRESS)
    return ap.parse_args()


def verify_bytes(ctx, Hkv, D, T, Hq, B=1, P=16):
    """Algorithmic bytes of one verify call (per (token, kv head): int8 K + V, fp16 scales)."""
    kv = B * ctx * Hkv * (2 * D + 4)
    qo = B * T * Hq * D * 2 * 2
    bt = B * (-(-ctx // P)) * 4
    return kv + qo + bt + 8 * B


def batch_bytes(context_lens, draft_lens, Hkv, D, Hq, P=16, distinct_tokens=None):
    """Algorithmic bytes of one verify call over a batch: every request's context
    pages (shared pages once when distinct_tokens is given), q in and out for the
    drafted rows, block-table entries and lengths."""
    ctx = [int(c) for c in context_lens]
    d = [int(x) for x in draft_lens]
    tokens = sum(ctx) if distinct_tokens is None else distinct_tokens
    return (tokens * Hkv * (2 * D + 4) + sum(d) * Hq * D * 2 * 2
            + sum(-(-c // P) for c in ctx) * 4 + 8 * len(ctx))


def batch_flops(context_lens, draft_lens, Hq, D):
    """QK^T and PV over each drafted row's visible keys: 4 D per (row, key)."""
    return sum(4 * D * Hq * sum(c - dd + t + 1 for t in range(dd))
               for c, dd in zip((int(x) for x in context_lens), (int(x) for x in draft_lens)))


def append_bytes(T, Hkv, D, B=1):
    """Algorithmic bytes of appending T tokens: fp32 source rows in, codes and scales out."""
    return B * T * Hkv * (2 * D * 4 + 2 * D + 2 * 2) + 8 * B


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        h.update((ROOT / rel).read_bytes())
    return h.hexdigest()[:16]


def stored_traffic():
    """Measured HBM bytes per verify call from the committed counter summary, if it
    was made from the kernel source now in the tree."""
    if not TRAFFIC_SUMMARY.exists():
        return None
    for line in TRAFFIC_SUMMARY.read_text().splitlines():
        if line.startswith("{") and '"source_hash"' in line:
            rec = json.loads(line)
            if rec.get("source_hash") == kernel_source_hash():
                return rec
    return None


class Phases:
    """Launches of the causal D = 256 partition kernel made by each phase, in order:
    the rocprofv3 summaries slice the kernel trace with them."""

    def __init__(self):
        self.items = []

    def add(self, name, launches):
        self.items.append({"phase": name, "launches": int(launches)})

    def write(self, path):
        Path(path).write_text(json.dumps(self.items, indent=1))


PHASES = Phases()


def progress(msg):
    """A progress line on stderr (stdout carries only the JSON line)."""
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def _torch_up(dev):
    import torch

    def up(a):
        a = np.ascontiguousarray(a)
        return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(dev)
    return up


def sleep_ahead(n_items, us_each=40.0):
    """Keep the GPU busy while the host queues n_items launches."""
    import torch
    torch.cuda._sleep(int(max(n_items, 1) * us_each * 1e-6 * 2.0e9))


class Rotation:
    """HIP graphs of C consecutive calls over R replicas, enough graphs (each on
    its own window of replicas) that consecutive replays cycle through all R."""

    def __init__(self, calls, steps, stream):
        import torch
        if len(calls) < 16:                                   # a graph of one call would time its launch
            calls = list(calls) * -(-16 // len(calls))
        R = len(calls)
        self.C = max(d for d in range(1, min(R, 16) + 1) if steps % d == 0)
        ng = R // math.gcd(R, self.C)
        self.graphs = []
        for i in range(ng):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for j in range(self.C):
                    calls[(i * self.C + j) % R]()
            self.graphs.append(g)
        self.next = 0
        self.replayed = 0

    def replay(self, n):
        for _ in range(n):
            self.graphs[self.next % len(self.graphs)].replay()
            self.next += 1
        self.replayed += n

    def time(self, steps, warmup, batches=BATCHES):
        """Median µs per call over `batches` batches of exactly `steps` calls (and the batches)."""
        import torch
        self.replay(max(len(self.graphs), -(-warmup // self.C)))
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        per = []
        for _ in range(batches):
            sleep_ahead(steps // self.C)
            e0.record()
            self.replay(steps // self.C)
            e1.record()
            torch.cuda.synchronize()
            per.append(e0.elapsed_time(e1) * 1e3 / steps)
        return float(np.median(per)), per

    @property
    def calls(self):
        return self.replayed * self.C


def page_replicas(pools, tables, R, num_pages, seed):
    """Copy the pages `tables` (int32 [B][n]) name into R - 1 fresh disjoint page
    sets of the same pools; returns the R block tables (replica 0 is the original)."""
    import torch
    dev = pools[0].device
    used = np.unique(tables)
    free = np.setdiff1d(np.arange(num_pages), used)
    rng = np.random.default_rng(seed)
    extra = rng.choice(free, size=(R - 1) * used.size, replace=False).astype(np.int32)
    src = torch.from_numpy(used.astype(np.int64)).to(dev)
    out = [tables.astype(np.int32)]
    for r in range(1, R):
        fresh = extra[(r - 1) * used.size:r * used.size]
        dst = torch.from_numpy(fresh.astype(np.int64)).to(dev)
        for pool in pools:
            pool[dst] = pool[src]
        remap = np.zeros(num_pages, np.int32)
        remap[used] = fresh
        out.append(remap[tables])
    return out


def main():
    args = parse()
    if args.summarize_stats:
        return summarize_stats(*args.summarize_stats[:2], args.summarize_stats[2:])
    if args.summarize_traffic:
        return summarize_traffic(*args.summarize_traffic[:3], args.summarize_traffic[3:])
    if args.summarize_counters:
        return summarize_counters(*args.summarize_counters[:2], args.summarize_counters[2:])
    if args.oracle_one_thread:
        return oracle_one_thread_child(args.oracle_one_thread)
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(sharding by request, kv head or context is described in DESIGN.md).", file=sys.stderr)
        sys.exit(2)
    legs = set() if args.legs == "none" else (
        {"configs", "accept", "prefill", "scaling", "ceiling"} if args.legs == "all" else set(args.legs.split(",")))
    import torch

    import speculative_decode_attention_amd as sda
    from speculative_decode_attention_amd import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    up = _torch_up(dev)
    progress("32K workload: building")
    wl = synth.make_config(3)
    B, T, Hq, Hkv, D, P = wl.B, wl.T_max, wl.Hq, wl.Hkv, wl.D, wl.P
    ctx = int(wl.context_lens[0])
    n_pages = -(-ctx // P)
    call_bytes = verify_bytes(ctx, Hkv, D, T, Hq)
    R = -(-ROTATE_BYTES // call_bytes)                   # 16 replicas of 68 MB

    # pools and the context, appended by the library itself
    pools = [up(a) for a in (wl.k_pool, wl.v_pool, wl.k_scale, wl.v_scale)]
    for ph in wl.appends:
        sda.splash_kv_append_int8(up(ph.k_src), up(ph.v_src), *pools, up(ph.block_table),
                                  up(ph.context_lens), up(ph.draft_lens))
    tables = page_replicas(pools, wl.block_table[:, :n_pages], R, wl.num_pages, 1234)
    bts = [up(t) for t in tables]
    draft = wl.appends[-1]
    k_new, v_new = up(draft.k_src), up(draft.v_src)
    ctx_t, dl_t = up(wl.context_lens), up(wl.draft_lens)
    q = up(wl.q)
    out = torch.empty_like(q)
    S_req = args.splits or sda.splash_verify_attn_default_splits(B, Hkv, ctx, P, D)
    S = sda.effective_splits(ctx, P, S_req)
    ws = torch.zeros(max(sda.splash_verify_attn_workspace_bytes(B, T, Hq, D, S), 16), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def verify(r):
        sda.splash_verify_attn(q, out, *pools, bts[r], ctx_t, dl_t, ctx, wl.sm_scale, num_splits=S_req, workspace=ws)

    def step_seq(r):
        sda.splash_kv_append_int8(k_new, v_new, *pools, bts[r], ctx_t, dl_t)
        verify(r)

    # the step as one launch: the verify call appends the block itself
    def step(r):
        sda.splash_verify_attn_append(k_new, v_new, q, out, *pools, bts[r], ctx_t, dl_t, ctx, wl.sm_scale,
                                      num_splits=S_req, workspace=ws)

    # the same call with a tree-shaped block mask (random candidate tree)
    tree = torch.from_numpy(synth.tree_block_masks(77, wl.draft_lens, T).view(np.int32)).to(dev)

    def verify_tree(r):
        sda.splash_verify_attn_masked(q, out, *pools, bts[r], ctx_t, dl_t, tree, ctx, wl.sm_scale,
                                      num_splits=S_req, workspace=ws)

    # the same call for a sliding-window drafter: only the last W keys per draft
    W = 4096

    def verify_window(r):
        sda.splash_verify_attn_window(q, out, *pools, bts[r], ctx_t, dl_t, W, ctx, wl.sm_scale, workspace=ws)

    cap = torch.cuda.Stream()
    # eager calls first (every lazy init done), then the graphs
    for r in range(R):
        step_seq(r)
        step(r)
    verify_tree(0)
    verify_window(0)
    torch.cuda.synchronize()
    PHASES.add("eager warm-up, 32K", R)
    rot = {name: Rotation([(lambda r=r, f=fn: f(r)) for r in range(R)], args.steps, cap)
           for name, fn in (("verify", verify), ("step", step), ("step_seq", step_seq), ("verify_tree", verify_tree),
                            ("verify_window", verify_window))}
    torch.cuda.synchronize()

    progress("32K workload: timing")
    us_verify, per_verify = rot["verify"].time(args.steps, args.warmup)
    PHASES.add("verify call, 32K, rotating replicas (roofline)", rot["verify"].calls)
    us_step, per_step = rot["step"].time(args.steps, args.warmup)
    us_step_seq, _ = rot["step_seq"].time(args.steps, args.warmup)
    PHASES.add("append + verify steps, 32K", rot["step_seq"].calls)
    us_tree, _ = rot["verify_tree"].time(args.steps, args.warmup)
    us_window, _ = rot["verify_window"].time(args.steps, args.warmup)
    ms_step = us_step * 1e-3
    step_bytes = call_bytes + append_bytes(T, Hkv, D)
    value = step_bytes / (ms_step * 1e-3) / 1e9
    window_bytes = verify_bytes(min(ctx, W + T - 1), Hkv, D, T, Hq)
    achieved = call_bytes / (us_verify * 1e-6) / 1e9

    # the same calls on one replica only: its pages stay in the 256 MB Infinity Cache
    warm = Rotation([lambda: verify(0)], args.steps, cap)
    us_warm, _ = warm.time(args.steps, args.warmup)
    PHASES.add("verify call, 32K, one replica (MALL-warm)", warm.calls)
    del rot, warm
    del pools, bts, ws, q, out
    torch.cuda.empty_cache()

    progress(f"32K verify {us_verify:.2f} us/call, step {us_step:.2f} us")
    configs = config_legs(dev, args.steps, args.warmup) if "configs" in legs else None
    stream_gbs = read_ceiling_gbs(dev) if "ceiling" in legs else None
    accept = accept_leg(dev, args.steps) if "accept" in legs else None
    prefill = prefill_leg(dev, args.steps) if "prefill" in legs else None
    scaling = context_scaling_leg(dev, args.steps, args.warmup) if "scaling" in legs else None

    if args.copy_calibration:
        n = CALIB_MIB * 2 ** 20 // 4
        a = torch.ones(n, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            torch.neg(a, out=b)
        torch.cuda.synchronize()
        del a, b

    cpu = None
    if not args.no_cpu_baseline:
        progress("CPU oracle baseline")
        cpu = cpu_baseline(wl, args.cpu_seconds)
    if args.phase_log:
        PHASES.write(args.phase_log)

    trec = stored_traffic()
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",                                  # MFMA operands (fp32 accumulation); q/out are bf16
        "data": "synthetic",
        "config": {"workload": WORKLOAD, "global_batch": B, "seq_len": ctx, "draft_block": T,
                   "q_heads": Hq, "kv_heads": Hkv, "head_dim": D, "page_tokens": P, "kv_dtype": "int8", "io_dtype": "bf16",
                   "splits": S, "replicas": R, "rotated_bytes": R * call_bytes, "step_bytes": step_bytes,
                   "batches": BATCHES, "step_us_batches": [round(x, 2) for x in per_step],
                   "step": "splash_verify_attn_append: the block appended and verified in one call",
                   "step_sequential_us": round(us_step_seq, 2),
                   "verify_us_per_call": round(us_verify, 2),
                   "verify_us_batches": [round(x, 2) for x in per_verify],
                   "verify_gbs": round(achieved, 1),
                   "verify_pct_of_hbm_peak": round(100 * achieved / HBM_PEAK_GBS, 1),
                   "verify_us_mall_warm": round(us_warm, 2),
                   "verify_tree_mask_us_per_call": round(us_tree, 2),
                   "verify_window_4096": {"us_per_call": round(us_window, 2),
                                          "gbs": round(window_bytes / (us_window * 1e-6) / 1e9, 1)},
                   "hbm_read_ceiling_pages_gbs": stream_gbs and round(stream_gbs, 1)},
        "roofline": {"bound": "hbm", "kernel": "verify call (" + PART_KERNEL + " and its merge)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": trec["hbm_bytes_per_call"] if trec else None,
                     "bytes_per_launch": call_bytes, "mean_launch_us": round(us_verify, 3),
                     "page_read_ceiling_gbs": stream_gbs and round(stream_gbs, 1),
                     "frac_of_page_read_ceiling": stream_gbs and round(achieved / stream_gbs, 4)},
        "cpu_baseline": cpu,
        "configs": configs,
        "accept": accept,
        "prefill": prefill,
        "context_scaling": scaling,
    }
    print(json.dumps(line), flush=True)


def config_legs(dev, steps, warmup) -> dict:
    """The other named workloads through splash_verify_attn, each over page
    replicas that together exceed 1 GiB (config 5 is 1.09 GB by itself), in the
    rotating graphs of the 32K leg: µs per call (median of 5 batches), GB/s of
    algorithmic bytes and its fraction of 8 TB/s; for the shared-prefix batch
    (bytes of shared pages once) also the fp16 MFMA bound."""
    import torch
    import speculative_decode_attention_amd as sda
    from speculative_decode_attention_amd import synth
    up = _torch_up(dev)
    res = {}
    cap = torch.cuda.Stream()
    for cfg in (1, 2, 4, 5):
        progress(f"config {cfg}: building")
        wl = synth.make_config(cfg)
        pools = [up(a) for a in (wl.k_pool, wl.v_pool, wl.k_scale, wl.v_scale)]
        for ph in wl.appends:
            sda.splash_kv_append_int8(up(ph.k_src), up(ph.v_src), *pools, up(ph.block_table),
                                      up(ph.context_lens), up(ph.draft_lens))
        wl.appends = None
        mp = -(-wl.max_context_len // wl.P)
        used_tokens = len(np.unique(wl.block_table[:, :mp])) * wl.P
        nbytes = batch_bytes(wl.context_lens, wl.draft_lens, wl.Hkv, wl.D, wl.Hq, wl.P,
                             distinct_tokens=used_tokens if cfg == 4 else None)
        per_replica = used_tokens * wl.Hkv * (2 * wl.D + 4)
        R = 1 if cfg == 1 else max(1, -(-ROTATE_BYTES // per_replica))
        tables = page_replicas(pools, wl.block_table[:, :mp], R, wl.num_pages, 100 + cfg)
        bts = [up(t) for t in tables]
        q, cl, dl = up(wl.q), up(wl.context_lens), up(wl.draft_lens)
        out = torch.empty_like(q)
        ctx = wl.max_context_len
        S = sda.effective_splits(ctx, wl.P, sda.splash_verify_attn_default_splits(wl.B, wl.Hkv, ctx, wl.P, wl.D))
        ws = torch.zeros(max(sda.splash_verify_attn_workspace_bytes(wl.B, wl.T_max, wl.Hq, wl.D, S), 16),
                         dtype=torch.uint8, device=dev)

        def call(r):
            sda.splash_verify_attn(q, out, *pools, bts[r], cl, dl, ctx, wl.sm_scale, workspace=ws)

        for r in range(R):
            call(r)
        torch.cuda.synchronize()
        rot = Rotation([(lambda r=r: call(r)) for r in range(R)], steps, cap)
        us, per = rot.time(steps, warmup)
        if wl.D == 256:
            PHASES.add(f"config {cfg}", R + rot.calls)
        flops = batch_flops(wl.context_lens, wl.draft_lens, wl.Hq, wl.D)
        hbm_us = nbytes / (HBM_PEAK_GBS * 1e3)
        mfma_us = flops / (MFMA_F16_PEAK_TFLOPS * 1e6)
        progress(f"config {cfg}: {us:.2f} us/call")
        res[f"config_{cfg}"] = {
            "workload": synth.CONFIG_NAMES[cfg], "splits": S, "replicas": R,
            "us_per_call": round(us, 2), "us_batches": [round(x, 2) for x in per],
            "bytes": nbytes, "gbs": round(nbytes / (us * 1e-6) / 1e9, 1),
            "frac_of_hbm_peak": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "hbm_bound_us": round(hbm_us, 2), "flops": flops, "mfma_bound_us": round(mfma_us, 2),
            "frac_of_fp16_mfma_peak": round(mfma_us / us, 4)}
        if cfg == 1:
            res["config_1"]["note"] = "latency: one request of 256 tokens, 76 KB"
        del rot, pools, bts, q, out, ws
        torch.cuda.empty_cache()
    return res


def accept_leg(dev, steps: int) -> dict:
    """The step after verify: greedy acceptance over the target's logits (bf16,
    151,936-token vocabulary) for the verify workloads' block shapes.  Calls go
    back to back on logits replicas that together exceed the 256 MB Infinity
    Cache, so the logits come from HBM; bytes are the logits of the rows read."""
    import torch
    import speculative_decode_attention_amd as sda
    from speculative_decode_attention_amd import synth
    progress("acceptance leg")
    res = {}
    for name, B, dls in (("one_request_T16", 1, [16]), ("sixteen_requests_ragged_T16", 16, None)):
        case = synth.make_accept_case(21, B=B, T_max=16, draft_lens=dls)
        V = case.V
        row_bytes = V * 2
        R = max(2, -(-(768 << 20) // case.logits.nbytes))
        base = torch.from_numpy(case.logits.view(np.int16)).to(dev)
        logits = base.unsqueeze(0).repeat(R, 1, 1, 1).contiguous()
        bt = torch.from_numpy(case.block_tokens).to(dev)
        dl = torch.from_numpy(case.draft_lens).to(dev)
        ctx = torch.from_numpy(case.context_lens).to(dev)
        acc = torch.empty(B, dtype=torch.int32, device=dev)
        nxt = torch.empty(B, dtype=torch.int32, device=dev)
        ws = torch.zeros(max(sda.splash_verify_accept_workspace_bytes(B, 16, V), 16), dtype=torch.uint8, device=dev)

        def call(r):
            # each call rolls context_lens back in place; nothing else reads it
            # here, so it is left to drift rather than reset by an extra launch
            sda.splash_verify_accept(logits[r], bt, dl, ctx, acc, nxt, workspace=ws)

        for r in range(min(R, 8)):
            call(r)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(int(max(steps, 1) * 60e-6 * 2.0e9))
        e0.record()
        for i in range(steps):
            call(i % R)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / steps * 1e3
        nbytes = int(case.draft_lens.sum()) * row_bytes + int(case.draft_lens.sum()) * 4 + B * 16
        res[name] = {"B": B, "vocab": V, "rows": int(case.draft_lens.sum()), "logit_bytes": nbytes,
                     "us_per_call": round(us, 2), "gbs": round(nbytes / (us * 1e-6) / 1e9, 1)}
        del logits, base
    return res


def prefill_leg(dev, steps: int) -> dict:
    """Chunked prefill on the same cache layout: a 512-token chunk closing a
    32,768-token context (24 q / 4 kv heads, D = 256), its K/V already appended.
    FLOPs count QK^T and PV over each token's visible keys (4 * D per key and
    q head); bytes are the distinct K/V pages and scales of the context plus
    the chunk's q and out, each read or written once."""
    import torch
    import speculative_decode_attention_amd as sda
    from speculative_decode_attention_amd import synth
    ctx, chunk, Hq, Hkv, D, P = 32768, 512, 24, 4, 256, 16
    progress("prefill leg")
    wl = synth.make_workload("prefill", 31, B=1, context_lens=[ctx], T_max=chunk, draft_lens=[chunk],
                             Hq=Hq, Hkv=Hkv, D=D, num_pages=ctx // P + 8)

    def up(a):
        a = np.ascontiguousarray(a)
        return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(dev)

    pools = [up(a) for a in (wl.k_pool, wl.v_pool, wl.k_scale, wl.v_scale)]
    for ph in wl.appends:
        sda.splash_kv_append_int8(up(ph.k_src), up(ph.v_src), *pools, up(ph.block_table),
                                  up(ph.context_lens), up(ph.draft_lens))
    q, bt, cl, dl = up(wl.q), up(wl.block_table), up(wl.context_lens), up(wl.draft_lens)
    out = torch.empty_like(q)
    ws = torch.empty(max(sda.splash_prefill_attn_workspace_bytes(1, chunk, Hq, Hkv, D, ctx), 16),
                     dtype=torch.uint8, device=dev)

    def call():
        sda.splash_prefill_attn(q, out, *pools, bt, cl, dl, ctx, wl.sm_scale, workspace=ws)

    for _ in range(3):
        call()
    torch.cuda.synchronize()
    n = max(steps // 10, 5)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    per = []
    for _ in range(BATCHES):
        sleep_ahead(n, 60.0)
        e0.record()
        for _ in range(n):
            call()
        e1.record()
        torch.cuda.synchronize()
        per.append(e0.elapsed_time(e1) / n * 1e3)
    us = float(np.median(per))
    keys = sum(ctx - chunk + t + 1 for t in range(chunk))
    flops = 4 * D * Hq * keys
    kv_bytes = verify_bytes(ctx, Hkv, D, chunk, Hq)
    del pools, q, out, ws
    return {"workload": "512-token chunk at the end of a 32768-token context", "chunk": chunk,
            "context": ctx, "us_per_call": round(us, 1), "us_batches": [round(x, 1) for x in per], "flops": flops,
            "tflops": round(flops / (us * 1e-6) / 1e12, 1),
            "frac_of_fp16_mfma_peak": round(flops / (us * 1e-6) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4),
            "distinct_bytes": kv_bytes, "distinct_gbs": round(kv_bytes / (us * 1e-6) / 1e9, 1),
            "tokens_per_s": round(chunk / (us * 1e-6), 0)}


SCALING_CONTEXTS = (8192, 32768, 131072)


def scaling_replicas(ctx: int) -> int:
    """Page replicas the context-scaling leg rotates over at this context (>= 1 GiB)."""
    num_pages = ctx // 16 + 8
    pool_bytes = num_pages * 4 * 16 * (2 * 256 + 2 * 2)
    return max(2, -(-ROTATE_BYTES // pool_bytes))


def context_scaling_leg(dev, steps: int, warmup: int) -> dict:
    """The verify call (one request, T = 16, 24 q / 4 kv heads, D = 256) at 8K,
    32K and 128K tokens of context.  The per-launch costs (launch, start-up,
    pipeline fill and drain, the split merge) are fixed, so the rate rises with
    the context.  Each context's pages are repeated until the calls rotate over
    more than 1 GiB, so the pages come from HBM.  The cache holds the library's
    quantisation of Gaussian rows, as in the 32K workload above."""
    import torch
    import speculative_decode_attention_amd as sda
    from speculative_decode_attention_amd import synth
    res = {}
    cap = torch.cuda.Stream()
    for ctx in SCALING_CONTEXTS:
        progress(f"context scaling {ctx}")
        wl = synth.make_workload("scaling", 61, B=1, context_lens=[ctx], T_max=16, Hq=24, Hkv=4, D=256,
                                 num_pages=ctx // 16 + 8)
        host = (wl.k_pool, wl.v_pool, wl.k_scale.view(np.int16), wl.v_scale.view(np.int16))
        one = [torch.from_numpy(np.ascontiguousarray(a)).to(dev) for a in host]
        for ph in wl.appends:
            sda.splash_kv_append_int8(torch.from_numpy(ph.k_src).to(dev), torch.from_numpy(ph.v_src).to(dev), *one,
                                      torch.from_numpy(ph.block_table).to(dev), torch.from_numpy(ph.context_lens).to(dev),
                                      torch.from_numpy(ph.draft_lens).to(dev))
        wl.appends = None                                     # the source rows are no longer needed
        R = scaling_replicas(ctx)
        pools = [a.repeat((R,) + (1,) * (a.dim() - 1)) for a in one]
        del one
        bts = [torch.from_numpy(wl.block_table + r * wl.num_pages).to(dev) for r in range(R)]
        q = torch.from_numpy(wl.q.view(np.int16)).to(dev)
        cl, dl = torch.from_numpy(wl.context_lens).to(dev), torch.from_numpy(wl.draft_lens).to(dev)
        out = torch.empty_like(q)
        S = sda.splash_verify_attn_default_splits(1, 4, ctx, 16, 256)
        ws = torch.zeros(max(sda.splash_verify_attn_workspace_bytes(1, 16, 24, 256, S), 16), dtype=torch.uint8,
                         device=dev)

        def call(r):
            sda.splash_verify_attn(q, out, *pools, bts[r], cl, dl, ctx, wl.sm_scale, workspace=ws)

        for r in range(R):
            call(r)
        torch.cuda.synchronize()
        rot = Rotation([(lambda r=r: call(r)) for r in range(R)], steps, cap)
        us, per = rot.time(steps, warmup)
        PHASES.add(f"context scaling {ctx}", R + rot.calls)
        nbytes = verify_bytes(ctx, 4, 256, 16, 24)
        res[f"ctx_{ctx}"] = {"us_per_call": round(us, 2), "us_batches": [round(x, 2) for x in per],
                             "bytes": nbytes, "splits": S, "replicas": R,
                             "gbs": round(nbytes / (us * 1e-6) / 1e9, 1),
                             "frac_of_hbm_peak": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
        del rot, pools, bts, q, out, ws
        torch.cuda.empty_cache()
    return res


def read_ceiling_gbs(dev) -> float:
    """GB/s of a pure copy of the partition kernel's page stream (the probe library)."""
    progress("page-read ceiling")
    import ctypes
    import torch
    from speculative_decode_attention_amd import build as hip_build
    if not hip_build.PROBE_LIB.exists():
        raise SystemExit(f"{hip_build.PROBE_LIB} is missing: run __graft_entry__.build() first")
    lib = ctypes.CDLL(str(hip_build.PROBE_LIB))
    fn = lib.splash_probe_read_pages
    fn.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    fn.restype = ctypes.c_int
    npages = 1 << 20                                          # 4 GiB, far beyond the 256 MB Infinity Cache
    pool = torch.ones(npages * 4096, dtype=torch.uint8, device=dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    perm = torch.randperm(npages, generator=gen, device=dev, dtype=torch.int32)
    grid = 4 * torch.cuda.get_device_properties(dev).multi_processor_count
    sink = torch.empty(grid, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream

    def once():
        rc = fn(pool.data_ptr(), perm.data_ptr(), npages, sink.data_ptr(), grid, stream)
        if rc != 0:
            raise RuntimeError(f"splash_probe_read_pages failed ({rc})")

    once()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 5
    e0.record()
    for _ in range(reps):
        once()
    e1.record()
    torch.cuda.synchronize()
    gbs = reps * npages * 4096 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del pool, perm, sink
    return gbs


def cpu_baseline(wl, seconds):
    """The oracle as it stands, on this host's cores: whole verify calls of the
    same workload, repeated until `seconds` of wall time have passed."""
    import oracle
    orc = oracle.load()
    pools = [a.copy() for a in (wl.k_pool, wl.v_pool, wl.k_scale, wl.v_scale)]
    for ph in wl.appends:
        orc.kv_append_int8(ph.k_src, ph.v_src, *pools, ph.block_table, ph.context_lens, ph.draft_lens)
    rows = np.array([(0, t, h) for t in range(int(wl.draft_lens[0])) for h in range(wl.Hq)], np.int32)
    calls = 0
    t0 = time.perf_counter()
    while True:
        orc.verify_attn_rows(wl.q, *pools, wl.block_table, wl.context_lens, wl.draft_lens, wl.Hkv,
                             wl.sm_scale, rows)
        calls += 1
        sec = time.perf_counter() - t0
        if sec >= seconds:
            break
    sec_per_call = sec / calls
    call_bytes = verify_bytes(int(wl.context_lens[0]), wl.Hkv, wl.D, wl.T_max, wl.Hq)
    one = oracle_one_thread(wl, pools, rows)
    return {"value": round(call_bytes / sec_per_call / 1e9, 3), "unit": "GB/s", "cores": orc.num_threads(),
            "kind": "oracle",
            "sample": f"{calls} whole verify calls of the benchmark workload ({len(rows)} output rows "
                      f"each, fp64 C oracle, OpenMP) in {sec:.1f} s: {sec_per_call * 1e3:.0f} ms/call "
                      f"on {cpu_model()}",
            "one_thread": one and {"value": round(call_bytes / one["sec_per_call"] / 1e9, 4), "unit": "GB/s",
                                   "cores": one["threads"],
                                   "sample": f"{one['calls']} whole call(s) in a child process with "
                                             f"OMP_NUM_THREADS=1: {one['sec_per_call'] * 1e3:.0f} ms/call"}}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown CPU"


def oracle_one_thread(wl, pools, rows, seconds=4.0):
    """The same oracle call on one host thread, in a child process (OpenMP reads
    its thread count at start-up); the inputs travel as .npy files."""
    import subprocess
    import tempfile
    # only the pages the request reads travel, renumbered 0..n-1 (the oracle reads
    # the pools through the block table alone)
    n_pages = -(-int(wl.context_lens[0]) // wl.P)
    used = wl.block_table[0, :n_pages]
    with tempfile.TemporaryDirectory() as d:
        arrays = {"q": wl.q, "k_pool": pools[0][used], "v_pool": pools[1][used], "k_scale": pools[2][used],
                  "v_scale": pools[3][used], "block_table": np.arange(n_pages, dtype=np.int32)[None, :],
                  "context_lens": wl.context_lens[:1], "draft_lens": wl.draft_lens[:1], "rows": rows}
        for k, a in arrays.items():
            np.save(Path(d) / f"{k}.npy", np.ascontiguousarray(a))
        (Path(d) / "meta.json").write_text(json.dumps({"Hkv": wl.Hkv, "sm_scale": wl.sm_scale, "seconds": seconds}))
        env = dict(os.environ, OMP_NUM_THREADS="1")
        try:
            proc = subprocess.run([sys.executable, str(Path(__file__).resolve()), "--oracle-one-thread", d],
                                  env=env, capture_output=True, text=True, timeout=300)
        except subprocess.TimeoutExpired:
            return None
        if proc.returncode != 0 or not proc.stdout.strip():
            return None
        return json.loads(proc.stdout.strip().splitlines()[-1])


def oracle_one_thread_child(d):
    import oracle
    orc = oracle.load()
    a = {k: np.load(Path(d) / f"{k}.npy") for k in ("q", "k_pool", "v_pool", "k_scale", "v_scale", "block_table",
                                                    "context_lens", "draft_lens", "rows")}
    meta = json.loads((Path(d) / "meta.json").read_text())
    calls, t0 = 0, time.perf_counter()
    while True:
        orc.verify_attn_rows(a["q"], a["k_pool"], a["v_pool"], a["k_scale"], a["v_scale"], a["block_table"],
                             a["context_lens"], a["draft_lens"], meta["Hkv"], meta["sm_scale"], a["rows"])
        calls += 1
        sec = time.perf_counter() - t0
        if sec >= meta["seconds"]:
            break
    print(json.dumps({"sec_per_call": sec / calls, "calls": calls, "threads": orc.num_threads()}), flush=True)


# ---------------------------------------------------------------------------
# rocprofv3 summaries (host only)
# ---------------------------------------------------------------------------

def _short(name: str) -> str:
    name = name.replace("void ", "").replace("(anonymous namespace)::", "")
    if "splash::" in name:
        return name.split("(")[0].replace("splash::", "")
    return name[:60]


def _find(d: str, suffix: str) -> Path:
    hits = sorted(Path(d).rglob(f"*{suffix}"))
    if not hits:
        raise SystemExit(f"no *{suffix} under {d}")
    return hits[0]


def _phase_slices(phase_log, n_launches):
    """(phase, start, end) index ranges into the causal D = 256 partition
    kernel's launches, in dispatch order, from the phase log bench.py wrote."""
    items = json.loads(Path(phase_log).read_text())
    out, i = [], 0
    for it in items:
        out.append((it["phase"], i, i + it["launches"]))
        i += it["launches"]
    if i != n_launches:
        raise SystemExit(f"the phase log counts {i} partition launches, the trace holds {n_launches}")
    return out


HEADLINE = "verify call, 32K, rotating replicas (roofline)"


def summarize_stats(d, phase_log, cmd):
    """Markdown summary of a `rocprofv3 --kernel-trace --stats` run of bench.py."""
    rows = list(csv.DictReader(open(_find(d, "kernel_stats.csv"))))
    print("# Kernel time: verify path, 32K context, T=16, 24q/4kv heads, D=256\n")
    print("Command (from the repository root on an MI355X):\n")
    print("```\n" + " ".join(cmd) + "\n```\n")
    print(f"Verify kernel source hash: `{kernel_source_hash()}`\n")
    print("| kernel | calls | mean µs | min µs | max µs | share % |")
    print("|---|---:|---:|---:|---:|---:|")
    for r in rows:
        print(f"| `{_short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
              f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f} |")
    trace = sorted(csv.DictReader(open(_find(d, "kernel_trace.csv"))), key=lambda r: int(r["Start_Timestamp"]))
    part = [r for r in trace if PART_KERNEL in r["Kernel_Name"]]
    dur = np.array([(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in part])
    print(f"\nThe `{_short(PART_KERNEL)}` launches by phase of the run (kernel trace, phase log "
          "written by the same run):\n")
    print("| phase | launches | mean µs | median µs |")
    print("|---|---:|---:|---:|")
    for name, i0, i1 in _phase_slices(phase_log, len(dur)):
        if i1 > i0:
            print(f"| {name} | {i1 - i0} | {dur[i0:i1].mean():.2f} | {np.median(dur[i0:i1]):.2f} |")
    # kernels launched between two partition launches of the headline phase: the rest of each call
    for name, i0, i1 in _phase_slices(phase_log, len(dur)):
        if name != HEADLINE:
            continue
        t0, t1 = int(part[i0]["Start_Timestamp"]), int(part[i1 - 1]["End_Timestamp"])
        inside = [r for r in trace if t0 <= int(r["Start_Timestamp"]) <= t1 and "splash::" in r["Kernel_Name"]]
        per = {}
        for r in inside:
            per.setdefault(_short(r["Kernel_Name"]), []).append(
                (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        print(f"\nKernels of the headline phase ({name}): one verify call is each of these once.\n")
        print("| kernel | launches | mean µs |")
        print("|---|---:|---:|")
        for k, v in per.items():
            print(f"| `{k}` | {len(v)} | {np.mean(v):.2f} |")
        span = (t1 - t0) / 1e3 / (i1 - i0)
        print(f"\nFirst partition start to last partition end, over the phase's calls: {span:.2f} µs per call.")


def _dispatches(d, counter):
    """(dispatch id, kernel name, value) of one counter, in dispatch order."""
    rows = sorted(csv.DictReader(open(_find(d, "counter_collection.csv"))), key=lambda r: int(r["Dispatch_Id"]))
    return [(int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"]))
            for r in rows if r["Counter_Name"] == counter]


def _headline_window(disp, phase_log):
    """Per kernel, the counter values of the library's kernels launched during the
    headline phase (from its first partition dispatch to the dispatch after its
    last one, which is that call's merge when there is one), and the call count."""
    part = [x for x in disp if PART_KERNEL in x[1]]
    sl = {name: (i0, i1) for name, i0, i1 in _phase_slices(phase_log, len(part))}
    i0, i1 = sl[HEADLINE]
    lo, hi = part[i0][0], part[i1 - 1][0] + 1
    per = {}
    for did, name, val in disp:
        if lo <= did <= hi and "splash::" in name:
            per.setdefault(name, []).append(val)
    return per, i1 - i0


def summarize_traffic(fetch_dir, write_dir, phase_log, cmd):
    """HBM bytes per verify call from FETCH_SIZE and WRITE_SIZE (KiB) passes, each
    scaled by what the same counter reads for a plain copy of known size."""
    fetch, write = _dispatches(fetch_dir, "FETCH_SIZE"), _dispatches(write_dir, "WRITE_SIZE")
    calib_bytes = CALIB_MIB * 2 ** 20

    def calib(disp):
        vals = [v for _, k, v in disp if "neg" in k.lower()]
        if not vals:
            raise SystemExit("no copy-calibration (neg) kernel in the counter output")
        return calib_bytes / (float(np.median(vals)) * 1024.0)

    f_fac, w_fac = calib(fetch), calib(write)
    fper, calls = _headline_window(fetch, phase_log)
    wper, _ = _headline_window(write, phase_log)
    print("# HBM traffic: verify path, 32K context, T=16, 24q/4kv heads, D=256\n")
    print("Commands (from the repository root on an MI355X), one counter per run:\n")
    print("```\n" + " ".join(cmd) + "\n```\n")
    print(f"Calibration: a plain {CALIB_MIB} MiB device copy (torch.neg, {calib_bytes} bytes read and "
          f"{calib_bytes} written) reads FETCH_SIZE x {f_fac:.3f} and WRITE_SIZE x {w_fac:.3f} "
          "of the true bytes; the figures below are scaled by these factors.\n")
    print(f"The library's kernels during the headline phase ({HEADLINE}, {calls} calls):\n")
    print("| kernel | dispatches | mean FETCH_SIZE KiB | mean WRITE_SIZE KiB | fetched MB per call | written MB per call |")
    print("|---|---:|---:|---:|---:|---:|")
    fb_call = wb_call = 0.0
    for k in sorted(fper):
        fv, wv = fper[k], wper.get(k, [0.0])
        fb = float(np.sum(fv)) * 1024 * f_fac / calls
        wb = float(np.sum(wv)) * 1024 * w_fac / calls
        fb_call, wb_call = fb_call + fb, wb_call + wb
        print(f"| `{_short(k)}` | {len(fv)} | {np.mean(fv):.0f} | {np.mean(wv):.0f} | {fb / 1e6:.2f} | {wb / 1e6:.2f} |")
    rec = {"kernels": "verify call", "calls": calls, "source_hash": kernel_source_hash(),
           "fetch_bytes_per_call": round(fb_call), "write_bytes_per_call": round(wb_call),
           "hbm_bytes_per_call": round(fb_call + wb_call), "fetch_factor": round(f_fac, 4),
           "write_factor": round(w_fac, 4)}
    print(f"\nPer call: {fb_call / 1e6:.2f} MB fetched + {wb_call / 1e6:.2f} MB written = "
          f"{(fb_call + wb_call) / 1e6:.2f} MB against {verify_bytes(32768, 4, 256, 16, 24) / 1e6:.2f} MB "
          "algorithmic.")
    # the partition kernel by phase of the run (every workload the run timed)
    pf = [v for _, k, v in fetch if PART_KERNEL in k]
    pw = [v for _, k, v in write if PART_KERNEL in k]
    print(f"\nThe `{_short(PART_KERNEL)}` launches by phase of the run (scaled as above):\n")
    print("| phase | launches | fetched MB per launch | written MB per launch |")
    print("|---|---:|---:|---:|")
    for name, i0, i1 in _phase_slices(phase_log, len(pf)):
        if i1 > i0:
            print(f"| {name} | {i1 - i0} | {np.mean(pf[i0:i1]) * 1024 * f_fac / 1e6:.2f} | "
                  f"{np.mean(pw[i0:i1]) * 1024 * w_fac / 1e6:.2f} |")
    # every library kernel of the run, whatever workload launched it (the
    # prefill leg's chunked partition and merge, the D = 64 kernels of config 1)
    fall, wall = {}, {}
    for _, k, v in fetch:
        if "splash::" in k:
            fall.setdefault(_short(k), []).append(v)
    for _, k, v in write:
        if "splash::" in k:
            wall.setdefault(_short(k), []).append(v)
    print("\nEvery library kernel of the run, per dispatch (scaled as above):\n")
    print("| kernel | dispatches | fetched MB per dispatch | written MB per dispatch |")
    print("|---|---:|---:|---:|")
    for k in sorted(fall):
        print(f"| `{k}` | {len(fall[k])} | {np.mean(fall[k]) * 1024 * f_fac / 1e6:.2f} | "
              f"{np.mean(wall.get(k, [0.0])) * 1024 * w_fac / 1e6:.2f} |")
    print("\nRecord read by bench.py (`roofline.traffic`, only while the source hash matches):\n")
    print(json.dumps(rec))


SQ_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CU_CYCLES", "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE",
               "SQ_INSTS_VALU_MFMA_MOPS_F16", "SQ_INSTS_LDS", "SQ_WAVE_CYCLES", "GRBM_GUI_ACTIVE")


def summarize_counters(d, phase_log, cmd, n_cu=256, n_xcd=8):
    """Markdown summary of one `rocprofv3 --pmc` pass of SQ counters over the
    partition kernel's launches of the headline phase."""
    rows = sorted(csv.DictReader(open(_find(d, "counter_collection.csv"))), key=lambda r: int(r["Dispatch_Id"]))
    per = {}
    for r in rows:
        if PART_KERNEL in r["Kernel_Name"]:
            per.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    n_all = len(next(iter(per.values())))
    sl = {name: (i0, i1) for name, i0, i1 in _phase_slices(phase_log, n_all)}
    i0, i1 = sl[HEADLINE]
    mean = {k: float(np.mean(v[i0:i1])) for k, v in per.items()}
    print("# SQ counters: verify partition kernel, 32K context, T=16, 24q/4kv heads, D=256\n")
    print("Command (from the repository root on an MI355X), one pass:\n")
    print("```\n" + " ".join(cmd) + "\n```\n")
    print(f"Verify kernel source hash: `{kernel_source_hash()}`; {i1 - i0} launches of the headline phase "
          "(mean per dispatch, summed over the device).\n")
    print("| counter | mean per launch |")
    print("|---|---:|")
    for k in SQ_COUNTERS:
        if k in mean:
            print(f"| `{k}` | {mean[k]:.4g} |")
    gui = mean.get("GRBM_GUI_ACTIVE")
    mfma = mean.get("SQ_VALU_MFMA_BUSY_CYCLES")
    conf, lds = mean.get("SQ_LDS_BANK_CONFLICT"), mean.get("SQ_LDS_IDX_ACTIVE")
    print("\nDerived:\n")
    if gui and mfma is not None:
        cyc = gui / n_xcd                                 # GRBM_GUI_ACTIVE is summed over the XCDs
        print(f"- launch length: `GRBM_GUI_ACTIVE / {n_xcd} XCDs` = {cyc:.4g} cycles")
        print(f"- MFMA busy: `SQ_VALU_MFMA_BUSY_CYCLES / (launch length x {n_cu} CUs x 4 SIMDs)` = "
              f"{100 * mfma / (cyc * n_cu * 4):.1f}% of the launch's SIMD-cycles")
    mops = mean.get("SQ_INSTS_VALU_MFMA_MOPS_F16")
    if mops is not None:
        print(f"- fp16 MFMA work: `SQ_INSTS_VALU_MFMA_MOPS_F16 x 512` = {mops * 512 / 1e9:.2f} GFLOP per launch "
              "(the algorithmic 12.9 GFLOP plus the padded rows and the bias products)")
    if lds:
        print(f"- LDS bank conflicts: `SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE` = {100 * conf / lds:.2f}% of the LDS "
              "active cycles")


if __name__ == "__main__":
    main()
