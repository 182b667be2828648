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

Prints one JSON line.  `value` is the step's algorithmic HBM bytes (int8 K and
V plus fp16 scales per context token and kv head, q in, out, block table and
lengths, and the append's source rows, codes and scales) over the step time.
`roofline` is the verify partition kernel alone: its algorithmic bytes over its
mean launch duration measured with HIP events on the launch stream.
`cpu_baseline` times the CPU oracle on the host cores on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time
from pathlib import Path

import numpy as np

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

HBM_PEAK_GBS = 8000.0
METRIC = "verify-attn µs/call + achieved HBM GB/s (% of peak) at 32K ctx, T=16"
WORKLOAD = "verify 1 req x ctx 32768, T=16 drafts, 24q/4kv heads, D=256, int8 KV in 16-token pages"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--replicas", type=int, default=16)
    ap.add_argument("--splits", type=int, default=0, help="0 = the library's preset")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=384, help="oracle rows timed for the CPU baseline")
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


def main():
    args = parse()
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
    torch.cuda.synchronize()

    def step(i):
        bt = bts[i % R]
        sda.splash_kv_append_int8(k_new, v_new, k_pool, v_pool, k_scale, v_scale, bt, ctx_t, dl_t)
        sda.splash_verify_attn(q, out, k_pool, v_pool, k_scale, v_scale, bt, ctx_t, dl_t, ctx,
                               wl.sm_scale, num_splits=S_req, workspace=ws)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(args.steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / args.steps
    step_bytes = verify_bytes(ctx, Hkv, D, T, Hq) + append_bytes(T, Hkv, D)
    value = step_bytes / (ms_step * 1e-3) / 1e9

    # the verify call alone (partition + merge), rotating replicas
    e0.record()
    for i in range(args.steps):
        bt = bts[i % R]
        sda.splash_verify_attn(q, out, k_pool, v_pool, k_scale, v_scale, bt, ctx_t, dl_t, ctx,
                               wl.sm_scale, num_splits=S_req, workspace=ws)
    e1.record()
    torch.cuda.synchronize()
    us_verify = e0.elapsed_time(e1) / args.steps * 1e3

    # the partition kernel alone: HIP events around each launch on its stream
    part_o = torch.empty((B, Hq, T, S, D), dtype=torch.float32, device=dev)
    part_lse = torch.empty((B, Hq, T, S), dtype=torch.float32, device=dev)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    for i in range(args.warmup):
        sda.splash_verify_attn_partition(q, k_pool, v_pool, k_scale, v_scale, bts[i % R], ctx_t, dl_t,
                                         ctx, wl.sm_scale, S, part_o, part_lse)
    for i in range(args.steps):
        starts[i].record()
        sda.splash_verify_attn_partition(q, k_pool, v_pool, k_scale, v_scale, bts[i % R], ctx_t, dl_t,
                                         ctx, wl.sm_scale, S, part_o, part_lse)
        ends[i].record()
    torch.cuda.synchronize()
    part_us = float(np.mean([s.elapsed_time(e) for s, e in zip(starts, ends)])) * 1e3
    part_bytes = verify_bytes(ctx, Hkv, D, T, Hq)
    achieved = part_bytes / (part_us * 1e-6) / 1e9

    # MALL-warm reference: the same call on one page set
    e0.record()
    for i in range(args.steps):
        sda.splash_verify_attn(q, out, k_pool, v_pool, k_scale, v_scale, bts[0], ctx_t, dl_t, ctx,
                               wl.sm_scale, num_splits=S_req, workspace=ws)
    e1.record()
    torch.cuda.synchronize()
    us_warm = e0.elapsed_time(e1) / args.steps * 1e3

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, args.cpu_rows)

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
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": WORKLOAD, "global_batch": B, "seq_len": ctx, "draft_block": T,
                   "q_heads": Hq, "kv_heads": Hkv, "head_dim": D, "page_tokens": P, "kv_dtype": "int8",
                   "splits": S, "replicas": R, "step_bytes": step_bytes,
                   "verify_us_per_call": round(us_verify, 2),
                   "verify_pct_of_hbm_peak": round(100 * part_bytes / (us_verify * 1e-6) / 1e9 / HBM_PEAK_GBS, 1),
                   "verify_us_per_call_mall_warm": round(us_warm, 2)},
        "roofline": {"bound": "hbm", "kernel": "verify_partition_kernel<256,6>",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "bytes_per_launch": part_bytes, "mean_launch_us": round(part_us, 3)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def cpu_baseline(wl, n_rows):
    """The oracle as it stands, on this host's cores, over a bounded sample of rows."""
    import oracle
    orc = oracle.load()
    pools = [a.copy() for a in (wl.k_pool, wl.v_pool, wl.k_scale, wl.v_scale)]
    for ph in wl.appends:
        orc.kv_append_int8(ph.k_src, ph.v_src, *pools, ph.block_table, ph.context_lens, ph.draft_lens)
    rows = np.array([(0, t, h) for t in range(int(wl.draft_lens[0])) for h in range(wl.Hq)], np.int32)
    rows = rows[:n_rows]
    t0 = time.perf_counter()
    orc.verify_attn_rows(wl.q, *pools, wl.block_table, wl.context_lens, wl.draft_lens, wl.Hkv,
                         wl.sm_scale, rows)
    sec = time.perf_counter() - t0
    total_rows = int(wl.draft_lens.sum()) * wl.Hq
    call_bytes = verify_bytes(int(wl.context_lens[0]), wl.Hkv, wl.D, wl.T_max, wl.Hq)
    sec_per_call = sec * total_rows / len(rows)
    threads = int(os.environ.get("OMP_NUM_THREADS") or os.cpu_count() or 1)
    return {"value": round(call_bytes / sec_per_call / 1e9, 3), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{len(rows)} of {total_rows} output rows of one verify call (fp64 C oracle, "
                      f"OpenMP), {sec:.2f} s; scaled to a whole call: {sec_per_call * 1e3:.0f} ms/call"}


if __name__ == "__main__":
    main()
