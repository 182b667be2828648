"""Helpers shared by the GPU tests: uploads, bf16 decoding, the attention
tolerance, and workloads prepared once per session (oracle pools and GPU pools
built from the same seeded source rows)."""
from __future__ import annotations

import sys

import numpy as np

import oracle
import speculative_decode_attention_amd as sda
from speculative_decode_attention_amd import synth

BF16_NAN = 0x7FC0

# tolerance: relative L2 <= 2e-3 over the valid rows, and every element within
# 1e-2 plus half a bf16 ulp of the reference (rounding even the exact fp64
# answer to bf16 moves an element by up to half an ulp, which exceeds 1e-2 when
# |o| >= 2.56)
REL_L2 = 2e-3
ABS = 1e-2
# per element, beside the above: |got - ref| <= half an ulp of bf16(ref) + MAG_REL * mag + floor,
# where mag = sum_j w_j |v_j| / sum_j w_j is the attention of |V| (the size of the row before
# the signs of V cancel).  The kernel rounds P' = p 2^jv s_v and the split partials to fp16,
# each a relative 2^-11 of that size; 2^-8 leaves a margin of 2 over their sum.  A P' below
# binary16's normal range is rounded to an absolute 2^-25 instead: in output units at most
# 2^-25 * 127 / 2^jv per key, with 2^jv >= 64 / s_max and the row sum >= 1, i.e. under
# 2^-24 N s_max over N visible keys (s_max the request's largest V scale); the floor takes
# 2^-23 N s_max.
MAG_REL = 2.0 ** -8
FLOOR_REL = 2.0 ** -23


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def torch_mod():
    import torch
    return torch


def up(a):
    torch = torch_mod()
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to("cuda")


def bf16_to_f64(bits):
    bits = np.asarray(bits).view(np.uint16).astype(np.uint32) << 16
    return bits.view(np.float32).astype(np.float64)


def half_ulp_bf16(ref):
    a = np.abs(ref)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, 2.0 ** (e - 8), 0.0)


def attn_error(got, ref, v_scale=1.0):
    """got, ref: fp64 arrays of the same shape (valid rows only).  v_scale: the
    magnitude V was drawn at (attention is linear in V, so the absolute slack
    of 1e-2, stated for unit-scale V, scales with it)."""
    diff = got - ref
    rel = float(np.linalg.norm(diff) / max(np.linalg.norm(ref), 1e-300))
    bound = ABS * v_scale + half_ulp_bf16(ref)
    excess = float(np.max(np.abs(diff) - bound)) if diff.size else -1.0
    ref_bf16 = bf16_to_f64(_round_bf16(ref))
    ulps = float(np.max(np.abs(got - ref_bf16) / np.maximum(2 * half_ulp_bf16(ref), 1e-300))) if diff.size else 0.0
    return dict(rel_l2=rel, max_abs=float(np.max(np.abs(diff))) if diff.size else 0.0,
                bound_excess=excess, max_ulps_vs_bf16_ref=ulps,
                finite=bool(np.all(np.isfinite(got))))


def _round_bf16(x):
    import torch
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy()


def assert_attn_ok(got, ref, where, mag=None, v_scale=1.0, floor=None):
    """mag: the attention of |V| for the same rows (enables the per-element bound);
    floor: per row, the binary16 underflow term of that bound (0 if None);
    v_scale: the magnitude V was drawn at (scales the absolute slack)."""
    e = attn_error(got, ref, v_scale)
    log(f"  {where}: rel_l2={e['rel_l2']:.3e} max|err|={e['max_abs']:.3e} "
        f"bound_excess={e['bound_excess']:.2e} ulps_vs_bf16(ref)={e['max_ulps_vs_bf16_ref']:.2f}")
    assert e["finite"], f"{where}: non-finite output"
    assert e["rel_l2"] <= REL_L2, f"{where}: relative L2 {e['rel_l2']:.3e}"
    assert e["bound_excess"] <= 0, f"{where}: an element exceeds {ABS * v_scale:.0e} + half a bf16 ulp"
    if mag is not None:
        fl = 0.0 if floor is None else np.asarray(floor, np.float64).reshape(-1, *([1] * (got.ndim - 1)))
        ratio = (np.abs(got - ref) - half_ulp_bf16(ref) - fl) / np.maximum(mag, 1e-300)
        worst = float(ratio.max()) if ratio.size else 0.0
        log(f"    per element: max (|err| - half ulp) / mag = {worst:.2e} (bound {MAG_REL:.2e})")
        assert worst <= MAG_REL, f"{where}: an element exceeds half a bf16 ulp + {MAG_REL:.2e} * mag"
    return e


class Prepared:
    """One workload with oracle pools (host) and GPU pools built by the GPU append."""

    def __init__(self, wl: synth.Workload):
        self.wl = wl
        orc = oracle.load()
        self.pools = [a.copy() for a in (wl.k_pool, wl.v_pool, wl.k_scale, wl.v_scale)]
        for ph in wl.appends:
            orc.kv_append_int8(ph.k_src, ph.v_src, *self.pools, ph.block_table, ph.context_lens,
                               ph.draft_lens)
        self.g_pools = [up(a) for a in (wl.k_pool, wl.v_pool, wl.k_scale, wl.v_scale)]
        for ph in wl.appends:
            sda.splash_kv_append_int8(up(ph.k_src), up(ph.v_src), *self.g_pools, up(ph.block_table),
                                      up(ph.context_lens), up(ph.draft_lens))
        torch_mod().cuda.synchronize()
        self._abs_pools = None
        self.q = up(wl.q)
        self.bt = up(wl.block_table)
        self.ctx = up(wl.context_lens)
        self.dl = up(wl.draft_lens)

    def pools_equal(self):
        names = ("k_pool", "v_pool", "k_scale", "v_scale")
        for name, host, dev in zip(names, self.pools, self.g_pools):
            got = dev.cpu().numpy()
            if host.dtype == np.uint16:
                got = got.view(np.uint16)
            if not np.array_equal(got, host):
                bad = np.flatnonzero(got.ravel() != host.ravel())
                return f"{name}: {bad.size} bytes differ, first at flat index {bad[0]}"
        return None

    def run(self, num_splits=0, out=None):
        torch = torch_mod()
        wl = self.wl
        if out is None:
            out = torch.full(tuple(wl.q.shape), BF16_NAN, dtype=torch.int16, device="cuda")
        sda.splash_verify_attn(self.q, out, *self.g_pools, self.bt, self.ctx, self.dl,
                               wl.max_context_len, wl.sm_scale, num_splits=num_splits)
        torch.cuda.synchronize()
        return out

    def valid_rows(self):
        wl = self.wl
        return np.array([(b, t, h) for b in range(wl.B) for t in range(int(wl.draft_lens[b]))
                         for h in range(wl.Hq)], dtype=np.int32)

    @property
    def abs_pools(self):
        """The oracle's pools with every V code replaced by its absolute value (codes are
        never -128): the attention over them is sum_j w_j |v_j| / sum_j w_j."""
        if self._abs_pools is None:
            kp, vp, ks, vs = self.pools
            self._abs_pools = [kp, np.abs(vp.astype(np.int16)).astype(np.int8), ks, vs]
        return self._abs_pools

    def p_floor(self, rows):
        """Per row (b, t, h): FLOOR_REL * (keys the row sees) * (request b's largest V scale)."""
        wl = self.wl
        if not hasattr(self, "_smax"):
            vs = self.pools[3].view(np.float16).astype(np.float64)
            self._smax = np.zeros(wl.B)
            for b in range(wl.B):
                pos = np.arange(int(wl.context_lens[b]))
                if pos.size:
                    self._smax[b] = vs[wl.block_table[b, pos // wl.P], :, pos % wl.P].max()
        rows = np.asarray(rows)
        b, t = rows[:, 0], rows[:, 1]
        n = wl.context_lens[b].astype(np.float64) - wl.draft_lens[b] + t + 1
        return FLOOR_REL * n * self._smax[b]

    def oracle_rows(self, rows, abs_v=False):
        wl = self.wl
        return oracle.load().verify_attn_rows(wl.q, *(self.abs_pools if abs_v else self.pools), wl.block_table,
                                              wl.context_lens, wl.draft_lens, wl.Hkv, wl.sm_scale, rows)


_cache = {}


def prepared_config(cfg: int) -> Prepared:
    if cfg not in _cache:
        log(f"[prepare] config {cfg}: {synth.CONFIG_NAMES[cfg]}")
        _cache.clear()                      # one large workload resident at a time
        _cache[cfg] = Prepared(synth.make_config(cfg))
    return _cache[cfg]
