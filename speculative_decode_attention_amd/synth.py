"""Seeded synthetic inputs for block-verify attention over an int8 paged KV cache.

This module holds none of the method's arithmetic.  It draws random numbers,
places given token rows at the pool positions a block table names (plain
indexing in the documented layouts), and fills unused memory with poison.
The HIP library's tests and benchmark and the CPU oracle both read what it
returns; it imports neither of them.

Workloads.  The pages measure on coding prompts up to 32K tokens, with 4
concurrent requests and with 16 requests of 32K each (Splash community summary
on discuss.pytorch.kr, sections "benchmark method", "concurrency"); the five
named workloads below take those shapes with synthetic values, since attention
cost depends on shapes and lengths, not on token content.

Draw order for a seed (fixed): q, K source, V source, scales (direct-value
workloads only), page placement, draft lengths (when drawn).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

# Poison for memory no request owns: codes 127 with scale 8.0, so that a read
# of the wrong page moves a softmax by a large amount instead of a little.
POISON_CODE = 127
POISON_SCALE_F16 = np.uint16(0x4800)   # binary16 bits of 8.0


def _bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (the input's dtype)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


@dataclass
class AppendPhase:
    """One call of the append entry point: tokens land at ctx - d + t."""
    block_table: np.ndarray      # int32 [B][max_pages_per_seq]
    context_lens: np.ndarray     # int32 [B]
    draft_lens: np.ndarray       # int32 [B]
    k_src: np.ndarray            # float32 [B][T][Hkv][D]
    v_src: np.ndarray            # float32 [B][T][Hkv][D]


@dataclass
class Workload:
    name: str
    B: int
    T_max: int
    Hq: int
    Hkv: int
    D: int
    P: int
    num_pages: int
    sm_scale: float
    q: np.ndarray                # bf16 bits uint16 [B][T_max][Hq][D]
    block_table: np.ndarray      # int32 [B][max_pages_per_seq]
    context_lens: np.ndarray     # int32 [B]
    draft_lens: np.ndarray       # int32 [B]
    # initial pool contents: poison everywhere except directly placed tokens
    k_pool: np.ndarray           # int8 [num_pages][Hkv][P][D]
    v_pool: np.ndarray           # int8 [num_pages][Hkv][P/8][D][8]
    k_scale: np.ndarray          # fp16 bits uint16 [num_pages][Hkv][P]
    v_scale: np.ndarray          # fp16 bits uint16 [num_pages][Hkv][P]
    appends: list = field(default_factory=list)   # AppendPhase, applied in order
    # token-major views of what each request's context holds (for dense checks)
    direct_tokens: list | None = None   # per request (k int8 [N][Hkv][D], v, ks [N][Hkv], vs)
    poison_page: int = -1
    pages_used: np.ndarray | None = None

    @property
    def max_pages_per_seq(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.B else 0

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv


def empty_pools(num_pages: int, Hkv: int, P: int, D: int):
    k_pool = np.full((num_pages, Hkv, P, D), POISON_CODE, dtype=np.int8)
    v_pool = np.full((num_pages, Hkv, P // 8, D, 8), POISON_CODE, dtype=np.int8)
    k_scale = np.full((num_pages, Hkv, P), POISON_SCALE_F16, dtype=np.uint16)
    v_scale = np.full((num_pages, Hkv, P), POISON_SCALE_F16, dtype=np.uint16)
    return k_pool, v_pool, k_scale, v_scale


def place_tokens(k_pool, v_pool, k_scale, v_scale, bt_row, first_pos, k, v, ks, vs):
    """Store token rows first_pos.. at the (page, slot) the block-table row names.

    k, v: int8 [n][Hkv][D]; ks, vs: fp16 bits [n][Hkv].  K pages are
    [Hkv][P][D] (token rows); V pages are [Hkv][P/8][D][8] (two d-major tiles of
    8 tokens each).
    """
    P = k_pool.shape[2]
    pos = first_pos + np.arange(k.shape[0])
    pages = np.asarray(bt_row)[pos // P]
    slots = pos % P
    for g in range(k_pool.shape[1]):
        k_pool[pages, g, slots, :] = k[:, g, :]
        v_pool[pages, g, slots // 8, :, slots % 8] = v[:, g, :]
        k_scale[pages, g, slots] = ks[:, g]
        v_scale[pages, g, slots] = vs[:, g]


def make_workload(name: str, seed: int, *, B: int, context_lens, T_max: int, Hq: int, Hkv: int,
                  D: int, num_pages: int, P: int = 16, draft_lens=None, values: str = "quantized",
                  placement: str = "random", shared_prefix: int = 0, nan_pad_q: bool = False,
                  sm_scale: float | None = None, extra_pages: int = 0, k_mag: float = 1.0,
                  v_mag: float = 1.0, k_spike=None, v_gain=None) -> Workload:
    """Build one seeded workload.

    values: "quantized" -> fp32 N(0,1) K/V source rows appended through the
    append entry point; "direct" -> int8 codes uniform in [-127, 127] and fp16
    scales uniform in [0.01, 0.05] placed in the pools as given.
    draft_lens: a list, or "random" for uniform draws in 1..T_max.
    k_mag, v_mag: standard deviations of the "quantized" K and V source rows
    (large values give peaked scores; large or small V values give V scales far
    from 1).
    k_spike: None, or a function amp(pos, ctx) -> float array giving, for the
    context positions pos of a request whose context holds ctx tokens, an
    amplitude a; the K source row at pos gets a * w added, with w one N(0,1)
    vector per kv head (drawn last, after the draft lengths).  Rising amplitudes
    put a row's largest score late in the context ("quantized" values, no
    shared prefix).
    v_gain: None, or a function gain(pos, ctx) -> float array multiplying the V
    source row at each context position of a request (V scales that grow or
    shrink along the context; "quantized" values, no shared prefix).
    shared_prefix: tokens (a whole number of pages) that every request shares
    through identical block-table entries.
    """
    rng = np.random.default_rng(seed)
    ctx = np.asarray(context_lens, dtype=np.int64).reshape(-1)
    if ctx.size == 1 and B > 1:
        ctx = np.full(B, int(ctx[0]), dtype=np.int64)
    assert ctx.size == B
    assert shared_prefix % P == 0 and all(shared_prefix <= c for c in ctx)
    if sm_scale is None:
        sm_scale = 1.0 / float(np.sqrt(D))

    # 1. q
    q32 = rng.standard_normal((B, T_max, Hq, D), dtype=np.float32)
    # 2-3. K and V source rows (shared prefix once, then each request's own tokens)
    own = [int(c) - shared_prefix for c in ctx]
    n_unique = shared_prefix + sum(own)
    if values == "quantized":
        k_all = rng.standard_normal((n_unique, Hkv, D), dtype=np.float32) * np.float32(k_mag)
        v_all = rng.standard_normal((n_unique, Hkv, D), dtype=np.float32) * np.float32(v_mag)
    elif values == "direct":
        k_all = rng.integers(-127, 128, size=(n_unique, Hkv, D)).astype(np.int8)
        v_all = rng.integers(-127, 128, size=(n_unique, Hkv, D)).astype(np.int8)
        # 4. scales
        ks_all = rng.uniform(0.01, 0.05, size=(n_unique, Hkv)).astype(np.float32)
        vs_all = rng.uniform(0.01, 0.05, size=(n_unique, Hkv)).astype(np.float32)
        ks_all = ks_all.astype(np.float16).view(np.uint16)
        vs_all = vs_all.astype(np.float16).view(np.uint16)
    else:
        raise ValueError(values)

    # 5. page placement
    prefix_pages = shared_prefix // P
    own_pages = [-(-o // P) for o in own]           # ceil
    n_pages_needed = prefix_pages + sum(own_pages) + extra_pages
    assert n_pages_needed <= num_pages, "pool too small"
    if placement == "random":
        ids = rng.choice(num_pages, size=n_pages_needed, replace=False).astype(np.int32)
    elif placement == "contiguous":
        ids = np.arange(n_pages_needed, dtype=np.int32)
    else:
        raise ValueError(placement)
    used = np.zeros(num_pages, dtype=bool)
    used[ids] = True
    free = np.flatnonzero(~used)
    poison_page = int(free[0]) if free.size else -1

    max_pages_per_seq = max(prefix_pages + op for op in own_pages) if B else 0
    block_table = np.full((B, max(max_pages_per_seq, 1)), max(poison_page, 0), dtype=np.int32)
    cursor = prefix_pages
    for b in range(B):
        block_table[b, :prefix_pages] = ids[:prefix_pages]
        block_table[b, prefix_pages:prefix_pages + own_pages[b]] = ids[cursor:cursor + own_pages[b]]
        cursor += own_pages[b]

    # 6. draft lengths
    if draft_lens is None:
        dl = np.full(B, T_max, dtype=np.int32)
    elif isinstance(draft_lens, str) and draft_lens == "random":
        dl = rng.integers(1, T_max + 1, size=B).astype(np.int32)
    else:
        dl = np.asarray(draft_lens, dtype=np.int32).reshape(-1)
        if dl.size == 1 and B > 1:
            dl = np.full(B, int(dl[0]), dtype=np.int32)
    assert all(0 <= d <= T_max and d <= c for d, c in zip(dl, ctx))

    if k_spike is not None:
        assert values == "quantized" and shared_prefix == 0, "K spikes take private quantised contexts"
        w = rng.standard_normal((Hkv, D), dtype=np.float32)
        for b in range(B):
            start = sum(own[:b])
            amp = np.asarray(k_spike(np.arange(own[b]), int(ctx[b])), dtype=np.float32)
            k_all[start:start + own[b]] += amp[:, None, None] * w[None]
    if v_gain is not None:
        assert values == "quantized" and shared_prefix == 0, "V gains take private quantised contexts"
        for b in range(B):
            start = sum(own[:b])
            gain = np.asarray(v_gain(np.arange(own[b]), int(ctx[b])), dtype=np.float32)
            v_all[start:start + own[b]] *= gain[:, None, None]

    if nan_pad_q:
        for b in range(B):
            q32[b, dl[b]:] = np.nan
    q = _bf16_bits(q32)

    k_pool, v_pool, k_scale, v_scale = empty_pools(num_pages, Hkv, P, D)
    wl = Workload(name=name, B=B, T_max=T_max, Hq=Hq, Hkv=Hkv, D=D, P=P, num_pages=num_pages,
                  sm_scale=float(sm_scale), q=q, block_table=block_table,
                  context_lens=ctx.astype(np.int32), draft_lens=dl, k_pool=k_pool, v_pool=v_pool,
                  k_scale=k_scale, v_scale=v_scale, poison_page=poison_page, pages_used=ids)

    # token ranges of each request inside the unique-token arrays
    def token_rows(arr, b):
        start = shared_prefix + sum(own[:b])
        return np.concatenate([arr[:shared_prefix], arr[start:start + own[b]]], axis=0)

    if values == "direct":
        wl.direct_tokens = []
        if shared_prefix:
            place_tokens(k_pool, v_pool, k_scale, v_scale, block_table[0], 0,
                         k_all[:shared_prefix], v_all[:shared_prefix],
                         ks_all[:shared_prefix], vs_all[:shared_prefix])
        for b in range(B):
            start = shared_prefix + sum(own[:b])
            sl = slice(start, start + own[b])
            place_tokens(k_pool, v_pool, k_scale, v_scale, block_table[b], shared_prefix,
                         k_all[sl], v_all[sl], ks_all[sl], vs_all[sl])
            wl.direct_tokens.append((token_rows(k_all, b), token_rows(v_all, b),
                                     token_rows(ks_all, b), token_rows(vs_all, b)))
        return wl

    # quantized values: the pools are filled by append calls, in three phases
    # (shared prefix once; each request's own context before its drafts; the
    # draft block itself, which is what a decode step appends)
    if shared_prefix:
        bt0 = block_table[:1].copy()
        wl.appends.append(AppendPhase(
            block_table=bt0, context_lens=np.array([shared_prefix], np.int32),
            draft_lens=np.array([shared_prefix], np.int32),
            k_src=np.ascontiguousarray(k_all[None, :shared_prefix]),
            v_src=np.ascontiguousarray(v_all[None, :shared_prefix])))
    body = [int(ctx[b]) - int(dl[b]) - shared_prefix for b in range(B)]
    Tb = max(body) if B else 0
    if Tb > 0:
        ksrc = np.zeros((B, Tb, Hkv, D), np.float32)
        vsrc = np.zeros((B, Tb, Hkv, D), np.float32)
        for b in range(B):
            start = shared_prefix + sum(own[:b])
            ksrc[b, :body[b]] = k_all[start:start + body[b]]
            vsrc[b, :body[b]] = v_all[start:start + body[b]]
        wl.appends.append(AppendPhase(
            block_table=block_table, context_lens=(ctx - dl).astype(np.int32),
            draft_lens=np.asarray(body, np.int32), k_src=ksrc, v_src=vsrc))
    ksrc = np.zeros((B, T_max, Hkv, D), np.float32)
    vsrc = np.zeros((B, T_max, Hkv, D), np.float32)
    for b in range(B):
        start = shared_prefix + sum(own[:b]) + body[b]
        ksrc[b, :dl[b]] = k_all[start:start + dl[b]]
        vsrc[b, :dl[b]] = v_all[start:start + dl[b]]
    wl.appends.append(AppendPhase(block_table=block_table, context_lens=ctx.astype(np.int32),
                                  draft_lens=dl.copy(), k_src=ksrc, v_src=vsrc))
    return wl


# --------------------------------------------------------------------------
# The five named workloads.
# --------------------------------------------------------------------------
CONFIG_NAMES = {
    1: "tiny: 1 req, ctx 256, T=4, 8q/2kv, D=64, contiguous pages, direct int8 values",
    2: "1 req, ctx 4096, T=16, 24q/4kv, D=256, 256 pages shuffled in a 65536-page pool",
    3: "1 req, ctx 32768, T=16, 24q/4kv, D=256, 2048 pages shuffled in a 65536-page pool",
    4: "4 req sharing a 24576-token prefix + 2048 own tokens, T=16, 24q/4kv, D=256",
    5: "16 req x ctx 32768, ragged T in 1..16, 24q/4kv, D=256, 40960-page pool",
}


def make_config(cfg: int, seed: int | None = None, **over) -> Workload:
    """The named workload `cfg` (1..5) with its default seed (cfg - 1)."""
    seed = cfg - 1 if seed is None else seed
    if cfg == 1:
        kw = dict(B=1, context_lens=[256], T_max=4, Hq=8, Hkv=2, D=64, num_pages=16,
                  values="direct", placement="contiguous", sm_scale=1.0 / 8.0)
    elif cfg == 2:
        kw = dict(B=1, context_lens=[4096], T_max=16, Hq=24, Hkv=4, D=256, num_pages=65536)
    elif cfg == 3:
        kw = dict(B=1, context_lens=[32768], T_max=16, Hq=24, Hkv=4, D=256, num_pages=65536)
    elif cfg == 4:
        kw = dict(B=4, context_lens=[26624] * 4, T_max=16, Hq=24, Hkv=4, D=256,
                  num_pages=65536, shared_prefix=24576)
    elif cfg == 5:
        kw = dict(B=16, context_lens=[32768] * 16, T_max=16, Hq=24, Hkv=4, D=256,
                  num_pages=40960, draft_lens="random", nan_pad_q=True)
    else:
        raise ValueError(cfg)
    kw.update(over)
    return make_workload(f"config{cfg}", seed, **kw)


# --------------------------------------------------------------------------
# Acceptance of a verified block: synthetic target logits.  The pages name the
# step (the target checks the drafted block in one pass and the output equals
# autoregressive decoding) but no vocabulary; 151,936 is the vocabulary of the
# Qwen tokenizer family the engine ships models of.  Logits are N(0, 1) * spread
# clipped to [-32, 32], rounded to bf16; every read row gets a spike of 64.0 at a
# drawn token, so each row's greedy token is known by construction (with
# `ties`, a second equal spike at a higher id, so the lower id must win), and the
# drafts copy those tokens up to a drawn acceptance point and differ there.
# --------------------------------------------------------------------------
VOCAB = 151936
SPIKE = 64.0


@dataclass
class AcceptCase:
    logits: np.ndarray           # bf16 bits uint16 [B][T_max][V]
    block_tokens: np.ndarray     # int32 [B][T_max]: [last committed token, drafts...]
    draft_lens: np.ndarray       # int32 [B]
    context_lens: np.ndarray     # int32 [B], cache length after the block
    planted_tokens: np.ndarray   # int32 [B][T_max]: the spike's token of each read row (-1 elsewhere)
    planted_accept: np.ndarray   # int32 [B]: block tokens kept, by construction

    @property
    def B(self) -> int:
        return self.logits.shape[0]

    @property
    def T_max(self) -> int:
        return self.logits.shape[1]

    @property
    def V(self) -> int:
        return self.logits.shape[2]


def make_accept_case(seed: int, *, B: int, T_max: int, V: int = VOCAB, draft_lens=None, accept_lens=None,
                     context_base: int = 4096, ties: bool = False, spread: float = 2.0) -> AcceptCase:
    """Draw order: logits, draft lengths (if not given), planted tokens, tie tokens,
    acceptance points (if not given), first block tokens, rejected drafts, trailing drafts."""
    rng = np.random.default_rng(seed)
    x = np.clip(rng.standard_normal((B, T_max, V), dtype=np.float32) * np.float32(spread), -32.0, 32.0)
    if draft_lens is None:
        draft_lens = rng.integers(1, T_max + 1, size=B)
    dl = np.asarray(draft_lens, dtype=np.int32).reshape(B)
    planted = rng.integers(0, V, size=(B, T_max)).astype(np.int32)
    second = rng.integers(0, V, size=(B, T_max)).astype(np.int32)
    if accept_lens is None:
        accept_lens = np.array([rng.integers(1, d + 1) if d > 0 else 0 for d in dl])
    acc = np.asarray(accept_lens, dtype=np.int32).reshape(B)
    first = rng.integers(0, V, size=B).astype(np.int32)
    wrong = rng.integers(1, V, size=(B, T_max)).astype(np.int32)
    tail = rng.integers(0, V, size=(B, T_max)).astype(np.int32)
    bt = np.zeros((B, T_max), dtype=np.int32)
    for b in range(B):
        d = int(dl[b])
        if d == 0:
            planted[b, :] = -1
            continue
        for t in range(d):
            y = int(planted[b, t])
            if ties and V > 1:
                lo, hi = sorted((y, int(second[b, t])))
                if lo == hi:
                    hi = (lo + 1) % V
                    lo, hi = min(lo, hi), max(lo, hi)
                x[b, t, hi] = SPIKE
                planted[b, t] = y = lo
            x[b, t, y] = SPIKE
        planted[b, d:] = -1
        a = int(acc[b])
        assert 1 <= a <= d, "acceptance point must lie in [1, d]"
        bt[b, 0] = first[b]
        for i in range(d - 1):                     # draft at block position i + 1 vs row i
            if i < a - 1:
                bt[b, i + 1] = planted[b, i]
            elif i == a - 1:
                bt[b, i + 1] = (planted[b, i] + wrong[b, i]) % V     # any token but the greedy one
            else:
                bt[b, i + 1] = tail[b, i]
    ctx = np.full(B, context_base, dtype=np.int32) + dl
    return AcceptCase(logits=_bf16_bits(x), block_tokens=bt, draft_lens=dl, context_lens=ctx,
                      planted_tokens=planted, planted_accept=acc)


def tree_block_masks(seed: int, draft_lens, T_max: int) -> np.ndarray:
    """Random candidate trees over each request's block: draft t > 0 hangs under a
    drawn earlier draft; bit u of mask[b][t] is set for t itself and each
    ancestor u (the drafts a tree-verify pass lets draft t see).  uint32 [B][T_max]."""
    rng = np.random.default_rng(seed)
    dl = np.asarray(draft_lens, dtype=np.int64)
    masks = np.zeros((len(dl), T_max), dtype=np.uint32)
    for b, d in enumerate(dl):
        parent = [-1] + [int(rng.integers(0, t)) for t in range(1, int(d))]
        for t in range(int(d)):
            m, u = 0, t
            while u >= 0:
                m |= 1 << u
                u = parent[u]
            masks[b, t] = m
    return masks


def chain_block_masks(draft_lens, T_max: int) -> np.ndarray:
    """The causal chain as block masks: draft t sees drafts 0..t."""
    dl = np.asarray(draft_lens, dtype=np.int64)
    masks = np.zeros((len(dl), T_max), dtype=np.uint32)
    for b, d in enumerate(dl):
        for t in range(int(d)):
            masks[b, t] = (1 << (t + 1)) - 1
    return masks
