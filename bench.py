"""Benchmark: one decode-verify step of block-verify attention on MI355X.

Workload: 1 request, context 32768 tokens, a block of 16 drafted tokens, 24
query heads / 4 kv heads, head dim 256, 16-token pages placed at random in a
65536-page int8 pool (the long-context single-stream case; the pages measure
decode on prompts up to 32K tokens -- Splash community summary on
discuss.pytorch.kr, section "benchmark method").

One step = the whole hot path on one batch: append the drafted block's K/V
(quantise to int8 into the paged pools) and run block-verify attention over the
full context (split-K partition + log-sum-exp merge).  Inputs are resident in
HBM before timing.  Steps rotate over R disjoint replicas of the request's
pages (identical values, R * 67 MB >= 1 GiB) so that the 256 MB Infinity
Cache cannot serve the context from one step to the next.

Timing.  Steps are captured in one HIP graph that runs C consecutive steps,
one per replica (C = the largest divisor of K that is at most R), as a serving
loop captures the calls of several layers in one graph; a graph launch costs
several microseconds of idle GPU that a per-call graph would charge to every
step.  The timed replays are queued behind a device-side sleep, so the GPU
runs them back to back whatever the host's launch rate; events on the launch
stream bracket exactly K steps (K / C replays).  The partition kernel is also timed alone, K launches back to
back between one event pair (queued the same way): its algorithmic bytes over
its mean launch duration give `roofline.achieved`.

Prints one JSON line.  `value` is the step's algorithmic HBM bytes (int8 K and
V plus fp16 scales per context token and kv head, q in, out, block table and
lengths, and the append's source rows, codes and scales) over the step time.
`roofline.traffic` is the partition kernel's measured HBM bytes per launch,
taken from the committed counter summary when that summary was made from the
kernel source now in the tree (else null).  `cpu_baseline` times the CPU
oracle on the host cores.

Host-only helper modes (no GPU) turn rocprofv3 CSV output into the short text
summaries kept under profiles/:
    python bench.py --summarize-stats DIR CMD...
    python bench.py --summarize-traffic FETCH_DIR WRITE_DIR CMD...
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
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
TRAFFIC_SUMMARY = ROOT / "profiles" / "verify_partition_d256_ctx32k_hbm_traffic.md"
# sources the partition kernel is compiled from (their hash stamps counter summaries)
KERNEL_SOURCES = ["speculative_decode_attention_amd/csrc/verify_attn.hip",
                  "speculative_decode_attention_amd/csrc/device.h",
                  "speculative_decode_attention_amd/csrc/launch.h"]
CALIB_MIB = 512
PMC_STEPS = 20                                            # --steps of the counter runs
DEFAULT_STEPS = 200


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=DEFAULT_STEPS)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--replicas", type=int, default=16)
    ap.add_argument("--splits", type=int, default=0, help="0 = the library's preset")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="repeat whole oracle calls until this much wall time has passed")
    ap.add_argument("--copy-calibration", action="store_true",
                    help=f"also run a plain {CALIB_MIB} MiB device copy (for counter calibration)")
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


def append_bytes(T, Hkv, D, B=1):
    """Algorithmic bytes of appending T tokens: fp32 source rows in, codes and scales out."""
    return B * T * Hkv * (2 * D * 4 + 2 * D + 2 * 2) + 8 * B


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        h.update((ROOT / rel).read_bytes())
    return h.hexdigest()[:16]


def stored_traffic():
    """Measured HBM bytes per partition launch from the committed counter summary,
    if it was made from the kernel source now in the tree."""
    if not TRAFFIC_SUMMARY.exists():
        return None
    for line in TRAFFIC_SUMMARY.read_text().splitlines():
        if line.startswith("{") and '"source_hash"' in line:
            rec = json.loads(line)
            if rec.get("source_hash") == kernel_source_hash():
                return rec
    return None


def main():
    args = parse()
    if args.summarize_stats:
        return summarize_stats(args.summarize_stats[0], args.summarize_stats[1:])
    if args.summarize_traffic:
        return summarize_traffic(*args.summarize_traffic[:2], args.summarize_traffic[2:])
    if args.summarize_counters:
        return summarize_counters(args.summarize_counters[0], args.summarize_counters[1:])
    if args.oracle_one_thread:
        return oracle_one_thread_child(args.oracle_one_thread)
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(sharding by request, kv head or context is described in DESIGN.md).", file=sys.stderr)
        sys.exit(2)
    import torch

    import speculative_decode_attention_amd as sda
    from speculative_decode_attention_amd import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    R = args.replicas
    wl = synth.make_config(3)
    B, T, Hq, Hkv, D, P = wl.B, wl.T_max, wl.Hq, wl.Hkv, wl.D, wl.P
    ctx = int(wl.context_lens[0])
    n_pages = -(-ctx // P)

    def up(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(a).to(dev)

    # pools and the context, appended by the library itself
    k_pool, v_pool, k_scale, v_scale = (up(a) for a in (wl.k_pool, wl.v_pool, wl.k_scale, wl.v_scale))
    for ph in wl.appends:
        sda.splash_kv_append_int8(up(ph.k_src), up(ph.v_src), k_pool, v_pool, k_scale, v_scale,
                                  up(ph.block_table), up(ph.context_lens), up(ph.draft_lens))
    # R disjoint replicas of the request's pages (replica 0 is the workload's own placement)
    used = np.zeros(wl.num_pages, bool)
    used[wl.block_table[0, :n_pages]] = True
    free = np.flatnonzero(~used)
    rng = np.random.default_rng(1234)
    extra = rng.choice(free, size=(R - 1) * n_pages, replace=False).astype(np.int32)
    tables = [wl.block_table[0, :n_pages].astype(np.int32)] + [extra[i * n_pages:(i + 1) * n_pages] for i in range(R - 1)]
    src = torch.from_numpy(tables[0].astype(np.int64)).to(dev)
    for r in range(1, R):
        dst = torch.from_numpy(tables[r].astype(np.int64)).to(dev)
        for pool in (k_pool, v_pool, k_scale, v_scale):
            pool[dst] = pool[src]
    bts = [up(t[None, :]) for t in tables]
    draft = wl.appends[-1]
    k_new, v_new = up(draft.k_src), up(draft.v_src)
    ctx_t, dl_t = up(wl.context_lens), up(wl.draft_lens)
    q = up(wl.q)
    out = torch.empty_like(q)
    S_req = args.splits or sda.splash_verify_attn_default_splits(B, Hkv, ctx, P, D)
    S = sda.effective_splits(ctx, P, S_req)
    ws = torch.empty(max(sda.splash_verify_attn_workspace_bytes(B, T, Hq, D, S), 16), dtype=torch.uint8, device=dev)
    po_shape, pl_shape = sda.partial_shapes(B, Hq, wl.Hkv, D, S)
    part_o = torch.empty(po_shape, dtype=torch.float16, device=dev)
    part_lse = torch.empty(pl_shape, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    def step(r):
        sda.splash_kv_append_int8(k_new, v_new, k_pool, v_pool, k_scale, v_scale, bts[r], ctx_t, dl_t)
        sda.splash_verify_attn(q, out, k_pool, v_pool, k_scale, v_scale, bts[r], ctx_t, dl_t, ctx,
                               wl.sm_scale, num_splits=S_req, workspace=ws)

    def verify(r):
        sda.splash_verify_attn(q, out, k_pool, v_pool, k_scale, v_scale, bts[r], ctx_t, dl_t, ctx,
                               wl.sm_scale, num_splits=S_req, workspace=ws)

    # the same call with a tree-shaped block mask (random candidate tree)
    tree = torch.from_numpy(synth.tree_block_masks(77, wl.draft_lens, T).view(np.int32)).to(dev)

    def verify_tree(r):
        sda.splash_verify_attn_masked(q, out, k_pool, v_pool, k_scale, v_scale, bts[r], ctx_t, dl_t, tree, ctx,
                                      wl.sm_scale, num_splits=S_req, workspace=ws)

    # the same call for a sliding-window drafter: only the last W keys per draft
    W = 4096

    def verify_window(r):
        sda.splash_verify_attn_window(q, out, k_pool, v_pool, k_scale, v_scale, bts[r], ctx_t, dl_t, W, ctx,
                                      wl.sm_scale, workspace=ws)

    def partition(r):
        sda.splash_verify_attn_partition(q, k_pool, v_pool, k_scale, v_scale, bts[r], ctx_t, dl_t,
                                         ctx, wl.sm_scale, S, part_o, part_lse)

    # one captured graph per replica; eager calls first so every lazy init is done
    for r in range(R):
        step(r)
    torch.cuda.synchronize()
    cap = torch.cuda.Stream()
    # one graph of C consecutive calls on replicas 0..C-1
    C = max(d for d in range(1, R + 1) if args.steps % d == 0)
    graphs = {}
    verify_tree(0)
    verify_window(0)
    for name, fn in (("step", step), ("verify", verify), ("verify_tree", verify_tree),
                     ("verify_window", verify_window)):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            for r in range(C):
                fn(r)
        graphs[name] = g
    torch.cuda.synchronize()

    def sleep_ahead(n_items):
        # keep the GPU busy while the host queues n_items (about 40 us of host time each)
        torch.cuda._sleep(int(max(n_items, 1) * 40e-6 * 2.0e9))

    def timed_replays(g, n, warm):
        """Mean time of one call over n calls (n / C replays)."""
        for _ in range(-(-warm // C)):
            g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        sleep_ahead(n // C)
        e0.record()
        for _ in range(n // C):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    ms_step = timed_replays(graphs["step"], args.steps, args.warmup)
    step_bytes = verify_bytes(ctx, Hkv, D, T, Hq) + append_bytes(T, Hkv, D)
    value = step_bytes / (ms_step * 1e-3) / 1e9
    us_verify = timed_replays(graphs["verify"], args.steps, args.warmup) * 1e3
    us_tree = timed_replays(graphs["verify_tree"], args.steps, args.warmup) * 1e3
    us_window = timed_replays(graphs["verify_window"], args.steps, args.warmup) * 1e3
    window_bytes = verify_bytes(min(ctx, W + T - 1), Hkv, D, T, Hq)

    # the partition kernel alone, launched back to back on its stream: one event
    # pair brackets the launches (queued behind a sleep, so the host's launch
    # rate does not show); also an event pair around each single launch
    for i in range(args.warmup):
        partition(i % R)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    sleep_ahead(args.steps)
    e0.record()
    for i in range(args.steps):
        partition(i % R)
    e1.record()
    torch.cuda.synchronize()
    part_us = e0.elapsed_time(e1) / args.steps * 1e3
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    sleep_ahead(args.steps)
    for i in range(args.steps):
        starts[i].record()
        partition(i % R)
        ends[i].record()
    torch.cuda.synchronize()
    part_us_single = float(np.mean([s.elapsed_time(e) for s, e in zip(starts, ends)])) * 1e3
    # the same launches on one replica only: its pages stay in the 256 MB Infinity Cache
    sleep_ahead(args.steps)
    e0.record()
    for i in range(args.steps):
        partition(0)
    e1.record()
    torch.cuda.synchronize()
    part_us_warm = e0.elapsed_time(e1) / args.steps * 1e3
    # practical HBM read ceiling for the same access pattern: 4 KB pages at
    # permuted positions of a 4 GiB pool, 16-byte direct-to-LDS loads, no compute
    stream_gbs = read_ceiling_gbs(dev)
    accept = accept_leg(dev, args.steps)
    prefill = prefill_leg(dev, args.steps)
    scaling = context_scaling_leg(dev, args.steps)
    shared = shared_prefix_leg(dev, args.steps)
    part_bytes = verify_bytes(ctx, Hkv, D, T, Hq)
    achieved = part_bytes / (part_us * 1e-6) / 1e9

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
        cpu = cpu_baseline(wl, args.cpu_seconds)

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
                   "splits": S, "replicas": R, "calls_per_graph": C, "step_bytes": step_bytes,
                   "verify_us_per_call": round(us_verify, 2),
                   "verify_tree_mask_us_per_call": round(us_tree, 2),
                   "verify_window_4096": {"us_per_call": round(us_window, 2),
                                          "gbs": round(window_bytes / (us_window * 1e-6) / 1e9, 1)},
                   "partition_us_mall_warm": round(part_us_warm, 3),
                   "hbm_read_ceiling_pages_gbs": round(stream_gbs, 1),
                   "verify_pct_of_hbm_peak": round(100 * part_bytes / (us_verify * 1e-6) / 1e9 / HBM_PEAK_GBS, 1)},
        "roofline": {"bound": "hbm", "kernel": PART_KERNEL,
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": trec["hbm_bytes_per_launch"] if trec else None,
                     "bytes_per_launch": part_bytes, "mean_launch_us": round(part_us, 3),
                     "single_launch_event_us": round(part_us_single, 3),
                     "page_read_ceiling_gbs": round(stream_gbs, 1),
                     "frac_of_page_read_ceiling": round(achieved / stream_gbs, 4)},
        "cpu_baseline": cpu,
        "accept": accept,
        "prefill": prefill,
        "shared_prefix": shared,
        "context_scaling": scaling,
    }
    print(json.dumps(line), flush=True)


def accept_leg(dev, steps: int) -> dict:
    """The step after verify: greedy acceptance over the target's logits (bf16,
    151,936-token vocabulary) for the verify workloads' block shapes.  Calls go
    back to back on logits replicas that together exceed the 256 MB Infinity
    Cache, so the logits come from HBM; bytes are the logits of the rows read."""
    import torch
    import speculative_decode_attention_amd as sda
    from speculative_decode_attention_amd import synth
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
    torch.cuda._sleep(int(n * 60e-6 * 2.0e9))
    e0.record()
    for _ in range(n):
        call()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / n * 1e3
    keys = sum(ctx - chunk + t + 1 for t in range(chunk))
    flops = 4 * D * Hq * keys
    kv_bytes = verify_bytes(ctx, Hkv, D, chunk, Hq)
    del pools, q, out, ws
    return {"workload": "512-token chunk at the end of a 32768-token context", "chunk": chunk,
            "context": ctx, "us_per_call": round(us, 1), "flops": flops,
            "tflops": round(flops / (us * 1e-6) / 1e12, 1),
            "frac_of_fp16_mfma_peak": round(flops / (us * 1e-6) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4),
            "distinct_bytes": kv_bytes, "distinct_gbs": round(kv_bytes / (us * 1e-6) / 1e9, 1),
            "tokens_per_s": round(chunk / (us * 1e-6), 0)}


SCALING_CONTEXTS = (8192, 32768, 131072)


def scaling_replicas(ctx: int) -> int:
    """Page replicas the context-scaling leg rotates over at this context."""
    num_pages = ctx // 16 + 8
    pool_bytes = num_pages * 4 * 16 * (2 * 256 + 2 * 2)
    return max(2, -(-(512 << 20) // pool_bytes))


def scaling_leg_launches(steps: int) -> int:
    """Partition launches the context-scaling leg makes (eager warm-up, one warm
    replay of every graph, the timed replays; all contexts)."""
    return sum(R + R + max(1, max(steps // 2, 2 * R) // R) * R for R in map(scaling_replicas, SCALING_CONTEXTS))


def context_scaling_leg(dev, steps: int) -> dict:
    """The verify call (one request, T = 16, 24 q / 4 kv heads, D = 256) at 8K,
    32K and 128K tokens of context.  The per-launch costs (launch, start-up,
    pipeline fill and drain, partial stores, merge) are fixed, so the rate
    rises with the context.  Each context's pages are repeated until the calls
    rotate over more than 512 MB (twice the Infinity Cache), so the pages come
    from HBM.  The cache holds the library's quantisation of Gaussian rows, as
    in the 32K workload above (the value distribution matters: widely spread
    scores move the softmax reference more often)."""
    import torch
    import speculative_decode_attention_amd as sda
    from speculative_decode_attention_amd import synth
    res = {}
    for ctx in SCALING_CONTEXTS:
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
        assert R * sum(a.nbytes for a in host) >= 512 << 20
        pools = [a.repeat((R,) + (1,) * (a.dim() - 1)) for a in one]
        del one
        bts = [torch.from_numpy(wl.block_table + r * wl.num_pages).to(dev) for r in range(R)]
        q = torch.from_numpy(wl.q.view(np.int16)).to(dev)
        cl, dl = torch.from_numpy(wl.context_lens).to(dev), torch.from_numpy(wl.draft_lens).to(dev)
        out = torch.empty_like(q)
        S = sda.splash_verify_attn_default_splits(1, 4, ctx, 16, 256)
        ws = torch.empty(max(sda.splash_verify_attn_workspace_bytes(1, 16, 24, 256, S), 16), dtype=torch.uint8,
                         device=dev)

        def call(r):
            sda.splash_verify_attn(q, out, *pools, bts[r], cl, dl, ctx, wl.sm_scale, workspace=ws)

        for r in range(R):
            call(r)
        torch.cuda.synchronize()
        # graphs of C consecutive calls on different replicas (host launch rate does not show)
        C = min(R, 16)
        graphs = []
        for g0 in range(0, R, C):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=torch.cuda.Stream()):
                for r in range(g0, min(g0 + C, R)):
                    call(r)
            graphs.append(g)
        reps = max(1, max(steps // 2, 2 * R) // R)
        for g in graphs:
            g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(int(reps * len(graphs) * 20e-6 * 2.0e9))
        e0.record()
        for _ in range(reps):
            for g in graphs:
                g.replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / (reps * R) * 1e3
        nbytes = verify_bytes(ctx, 4, 256, 16, 24)
        res[f"ctx_{ctx}"] = {"us_per_call": round(us, 2), "bytes": nbytes, "splits": S,
                             "gbs": round(nbytes / (us * 1e-6) / 1e9, 1),
                             "frac_of_hbm_peak": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
        del graphs, pools, bts, q, out, ws
    return res


def shared_leg_launches(steps: int) -> int:
    """Partition launches the shared-prefix leg makes (it runs last): warm-up + timed."""
    return 5 + max(steps // 2, 10)


def shared_prefix_leg(dev, steps: int) -> dict:
    """Four concurrent requests sharing one 24,576-token prefix through identical
    block-table entries, plus 2,048 private tokens each (T = 16, 24 q / 4 kv
    heads, D = 256).  Bounds: HBM over the distinct bytes (shared pages once)
    and the fp16 MFMA peak over the FLOPs (4 * D per valid row and visible key)."""
    import torch
    import speculative_decode_attention_amd as sda
    from speculative_decode_attention_amd import synth
    wl = synth.make_config(4)

    def up(a):
        a = np.ascontiguousarray(a)
        return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(dev)

    pools = [up(a) for a in (wl.k_pool, wl.v_pool, wl.k_scale, wl.v_scale)]
    for ph in wl.appends:
        sda.splash_kv_append_int8(up(ph.k_src), up(ph.v_src), *pools, up(ph.block_table),
                                  up(ph.context_lens), up(ph.draft_lens))
    q, bt, cl, dl = up(wl.q), up(wl.block_table), up(wl.context_lens), up(wl.draft_lens)
    out = torch.empty_like(q)
    ctx = int(wl.max_context_len)
    S = sda.splash_verify_attn_default_splits(wl.B, wl.Hkv, ctx, wl.P, wl.D)
    ws = torch.empty(max(sda.splash_verify_attn_workspace_bytes(wl.B, wl.T_max, wl.Hq, wl.D, S), 16),
                     dtype=torch.uint8, device=dev)

    def call():
        sda.splash_verify_attn(q, out, *pools, bt, cl, dl, ctx, wl.sm_scale, workspace=ws)

    n = shared_leg_launches(steps) - 5
    for _ in range(5):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(int(n * 40e-6 * 2.0e9))
    e0.record()
    for _ in range(n):
        call()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / n * 1e3
    d = [int(x) for x in wl.draft_lens]
    ctxs = [int(x) for x in wl.context_lens]
    distinct_tokens = len(np.unique(wl.block_table[:, :-(-ctx // wl.P)])) * wl.P
    nbytes = (distinct_tokens * wl.Hkv * (2 * wl.D + 4) + sum(d) * wl.Hq * wl.D * 4
              + wl.block_table[:, :-(-ctx // wl.P)].size * 4 + 8 * wl.B)
    flops = sum(4 * wl.D * wl.Hq * sum(c - dd + t + 1 for t in range(dd)) for c, dd in zip(ctxs, d))
    hbm_us = nbytes / (HBM_PEAK_GBS * 1e3)
    mfma_us = flops / (MFMA_F16_PEAK_TFLOPS * 1e6)
    del pools, q, out, ws
    return {"workload": "4 requests sharing a 24576-token prefix + 2048 private tokens each, T=16",
            "us_per_call": round(us, 2), "splits": S, "distinct_bytes": nbytes, "flops": flops,
            "hbm_bound_us": round(hbm_us, 2), "mfma_bound_us": round(mfma_us, 2),
            "tflops": round(flops / (us * 1e-6) / 1e12, 1),
            "frac_of_fp16_mfma_peak": round(mfma_us / us, 4),
            "distinct_gbs": round(nbytes / (us * 1e-6) / 1e9, 1)}


def read_ceiling_gbs(dev) -> float:
    """GB/s of a pure copy of the partition kernel's page stream (the probe library)."""
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


def summarize_stats(d, cmd):
    """Markdown summary of a `rocprofv3 --kernel-trace --stats` run."""
    rows = list(csv.DictReader(open(_find(d, "kernel_stats.csv"))))
    print("# Kernel time: verify path, 32K context, T=16, 24q/4kv heads, D=256\n")
    print("Command (from the repository root on an MI355X):\n")
    print("```\n" + " ".join(cmd) + "\n```\n")
    print(f"Partition kernel source hash: `{kernel_source_hash()}`\n")
    print("| kernel | calls | mean µs | min µs | max µs | share % |")
    print("|---|---:|---:|---:|---:|---:|")
    for r in rows:
        print(f"| `{_short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
              f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f} |")
    # the partition launches in the order bench.py makes them (default --steps):
    # graph replays, then three runs of `steps` launches each
    trace = sorted(csv.DictReader(open(_find(d, "kernel_trace.csv"))), key=lambda r: int(r["Start_Timestamp"]))
    us = np.array([(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
                   for r in trace if PART_KERNEL in r["Kernel_Name"]])
    n = DEFAULT_STEPS
    n_shared, n_scaling = shared_leg_launches(n), scaling_leg_launches(n)
    us, us_shared = us[:-n_shared], us[-n_shared:]
    us = us[:-n_scaling]                                  # the context-scaling leg (other contexts)
    print(f"\nThe table's `{_short(PART_KERNEL)}` row also holds the launches of the shared-prefix and "
          f"context-scaling legs (other workloads); over the {len(us)} launches of the 32K workload alone "
          f"the mean is {us.mean():.2f} µs.")
    if len(us) > 3 * n:
        print("\nPartition launches by phase of the run (kernel trace):\n")
        print("| phase | launches | mean µs |")
        print("|---|---:|---:|")
        for name, seg in (("verify graphs (with the merge)", us[:-3 * n]),
                          ("back to back, 16 rotating cache replicas (`roofline.mean_launch_us`)", us[-3 * n:-2 * n]),
                          ("one event pair per launch", us[-2 * n:-n]),
                          ("back to back, one replica (MALL-warm)", us[-n:]),
                          ("shared-prefix leg: 4 requests, 24,576 shared + 2,048 private tokens each",
                           us_shared)):
            print(f"| {name} | {len(seg)} | {seg.mean():.2f} |")


def _per_dispatch(d, counter):
    """Counter value per dispatch, per kernel name, in dispatch order."""
    per = {}
    rows = sorted(csv.DictReader(open(_find(d, "counter_collection.csv"))), key=lambda r: int(r["Dispatch_Id"]))
    for r in rows:
        if r["Counter_Name"] != counter:
            continue
        per.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return per


def summarize_traffic(fetch_dir, write_dir, cmd):
    """HBM bytes per dispatch from FETCH_SIZE and WRITE_SIZE (KiB) passes, each
    scaled by what the same counter reads for a plain copy of known size."""
    fetch, write = _per_dispatch(fetch_dir, "FETCH_SIZE"), _per_dispatch(write_dir, "WRITE_SIZE")
    calib_bytes = CALIB_MIB * 2 ** 20

    def calib(per):
        cands = [(k, v) for k, v in per.items() if "neg" in k.lower()]
        if not cands:
            raise SystemExit("no copy-calibration (neg) kernel in the counter output")
        vals = max(cands, key=lambda kv: np.mean(kv[1]))[1]
        return calib_bytes / (float(np.median(vals)) * 1024.0)

    f_fac, w_fac = calib(fetch), calib(write)
    # the shared-prefix leg runs last: its partition launches are reported on their own
    n_shared, n_scaling = shared_leg_launches(PMC_STEPS), scaling_leg_launches(PMC_STEPS)
    shared = {}
    for per, key in ((fetch, "f"), (write, "w")):
        for k in list(per):
            if PART_KERNEL in k:
                shared[key] = per[k][-n_shared:]
                per[k] = per[k][:-(n_shared + n_scaling)]     # the context-scaling leg's are other contexts
    part = [k for k in fetch if PART_KERNEL in k]
    if not part:
        raise SystemExit("no partition kernel in the counter output")
    print("# HBM traffic: verify path, 32K context, T=16, 24q/4kv heads, D=256\n")
    print("Commands (from the repository root on an MI355X), one counter per run:\n")
    print("```\n" + " ".join(cmd) + "\n```\n")
    print(f"Calibration: a plain {CALIB_MIB} MiB device copy (torch.neg, {calib_bytes} bytes read and "
          f"{calib_bytes} written) reads FETCH_SIZE x {f_fac:.3f} and WRITE_SIZE x {w_fac:.3f} "
          "of the true bytes; the figures below are scaled by these factors.\n")
    print("| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | fetched MB | written MB |")
    print("|---|---:|---:|---:|---:|---:|")
    rec = None
    for k in sorted(fetch):
        if "splash::" not in k:
            continue
        fk, wk = float(np.mean(fetch[k])), float(np.mean(write.get(k, [0.0])))
        fb, wb = fk * 1024 * f_fac, wk * 1024 * w_fac
        print(f"| `{_short(k)}` | {len(fetch[k])} | {fk:.0f} | {wk:.0f} | {fb / 1e6:.2f} | {wb / 1e6:.2f} |")
        if PART_KERNEL in k:
            rec = {"kernel": _short(k), "source_hash": kernel_source_hash(),
                   "fetch_bytes_per_launch": round(fb), "write_bytes_per_launch": round(wb),
                   "hbm_bytes_per_launch": round(fb + wb), "fetch_factor": round(f_fac, 4),
                   "write_factor": round(w_fac, 4)}
    if shared:
        fb, wb = float(np.mean(shared["f"])) * 1024 * f_fac, float(np.mean(shared["w"])) * 1024 * w_fac
        print(f"| `{_short(PART_KERNEL)}`, shared-prefix leg (4 requests, 24,576 shared + 2,048 private "
              f"tokens each) | {len(shared['f'])} | {np.mean(shared['f']):.0f} | {np.mean(shared['w']):.0f} | "
              f"{fb / 1e6:.2f} | {wb / 1e6:.2f} |")
    print("\nRecord read by bench.py (`roofline.traffic`, only while the source hash matches):\n")
    print(json.dumps(rec))


SQ_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CU_CYCLES", "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE",
               "SQ_INSTS_VALU_MFMA_MOPS_F16", "SQ_INSTS_LDS", "SQ_WAVE_CYCLES", "GRBM_GUI_ACTIVE")


def summarize_counters(d, cmd, n_cu=256, n_xcd=8):
    """Markdown summary of one `rocprofv3 --pmc` pass of SQ counters over the
    partition kernel's launches of the 32K workload (the shared-prefix and
    context-scaling legs, which run last, are left out)."""
    rows = sorted(csv.DictReader(open(_find(d, "counter_collection.csv"))), key=lambda r: int(r["Dispatch_Id"]))
    per = {}
    for r in rows:
        if PART_KERNEL in r["Kernel_Name"]:
            per.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    drop = shared_leg_launches(PMC_STEPS) + scaling_leg_launches(PMC_STEPS)
    mean = {k: float(np.mean(v[:-drop])) for k, v in per.items()}
    n = len(next(iter(per.values()))) - drop
    print("# SQ counters: verify partition kernel, 32K context, T=16, 24q/4kv heads, D=256\n")
    print("Command (from the repository root on an MI355X), one pass:\n")
    print("```\n" + " ".join(cmd) + "\n```\n")
    print(f"Partition kernel source hash: `{kernel_source_hash()}`; {n} launches of the 32K workload "
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
