"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Append/quantise: whole pools byte-identical (poison bytes included).
Attention: bf16 rows against the unrounded fp64 oracle on every valid row of
all five configurations, in the launch configuration the benchmark times (the
split preset): relative L2 <= 2e-3, every element within 1e-2 plus half a bf16
ulp, and every element within half a bf16 ulp plus 2^-8 of the attention of
|V|.  The exported partition and merge are checked element by element in the
oracle's own split layout.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

import oracle  # noqa: E402
import speculative_decode_attention_amd as sda  # noqa: E402
from speculative_decode_attention_amd import synth  # noqa: E402
from gpu_util import (BF16_NAN, MAG_REL, Prepared, assert_attn_ok, bf16_to_f64, log,  # noqa: E402
                      prepared_config, up)


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_append_pools_bit_exact(cfg):
    prep = prepared_config(cfg)
    bad = prep.pools_equal()
    assert bad is None, bad


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_verify_matches_oracle(cfg):
    prep = prepared_config(cfg) if cfg != 1 else Prepared(synth.make_config(1))
    wl = prep.wl
    S = sda.effective_splits(wl.max_context_len, wl.P,
                             sda.splash_verify_attn_default_splits(wl.B, wl.Hkv, wl.max_context_len, wl.P, wl.D))
    log(f"  config {cfg}: preset splits {S}")
    out = prep.run(num_splits=0).cpu().numpy()
    rows = prep.valid_rows()                                # every row of every request
    ref = prep.oracle_rows(rows)
    got = bf16_to_f64(out[rows[:, 0], rows[:, 1], rows[:, 2]])
    assert_attn_ok(got, ref, f"config {cfg} ({len(rows)} rows)", mag=prep.oracle_rows(rows, abs_v=True), floor=prep.p_floor(rows))
    # rows past each request's draft are never written
    for b in range(wl.B):
        assert np.all(out[b, int(wl.draft_lens[b]):].view(np.uint16) == BF16_NAN)


@pytest.mark.parametrize("S", [1, 2, 3, 7, 16, 64, 100])
def test_split_count_sweep(S):
    prep = prepared_config(2)
    out = prep.run(num_splits=S).cpu().numpy()
    rows = prep.valid_rows()
    got = bf16_to_f64(out[rows[:, 0], rows[:, 1], rows[:, 2]])
    ref = prep.oracle_rows(rows)
    assert_attn_ok(got, ref, f"config 2, {S} splits", mag=prep.oracle_rows(rows, abs_v=True), floor=prep.p_floor(rows))


def split_reference(prep, S):
    """The oracle's split path on the prepared pools (and on pools of |V| for the
    per-element size), with the documented split length."""
    wl = prep.wl
    cdiv = lambda a, b: -(-a // b)
    L = 4 * cdiv(cdiv(cdiv(wl.max_context_len, wl.P), S), 4)
    assert sda.splash_verify_attn_split_pages(wl.max_context_len, wl.P, S) == L
    orc = oracle.load()
    args = (wl.block_table, wl.context_lens, wl.draft_lens, wl.Hkv, wl.sm_scale, S, L)
    ro, rl = orc.verify_attn_split(wl.q, *prep.pools, *args)
    mo, _ = orc.verify_attn_split(wl.q, *prep.abs_pools, *args)
    return ro, rl, mo


def run_partition(prep, S):
    wl = prep.wl
    po_shape, pl_shape = sda.partial_shapes(wl.B, wl.Hq, wl.T_max, wl.D, S)
    part_o = torch.full(po_shape, float("nan"), device="cuda")
    part_lse = torch.full(pl_shape, float("nan"), device="cuda")
    sda.splash_verify_attn_partition(prep.q, *prep.g_pools, prep.bt, prep.ctx, prep.dl,
                                     wl.max_context_len, wl.sm_scale, S, part_o, part_lse)
    torch.cuda.synchronize()
    return part_o, part_lse


@pytest.mark.parametrize("v_mag", [1.0, 3e4, 1e-4])
def test_partition_partials_match_oracle_split(v_mag):
    """fp32 partial rows and log-sum-exps of each split, element by element,
    including empty splits (lse -inf, zero row); then the exported merge of
    these partials against the oracle's whole call."""
    wl = synth.make_workload("part", 31, B=2, context_lens=[700, 130], T_max=16, draft_lens=[16, 9],
                             Hq=24, Hkv=4, D=256, num_pages=128, v_mag=v_mag)
    prep = Prepared(wl)
    S = 13                                                  # 4 pages a split: splits 11, 12 empty
    part_o, part_lse = run_partition(prep, S)
    ro, rl, mo = split_reference(prep, S)
    go, gl = part_o.cpu().numpy().astype(np.float64), part_lse.cpu().numpy().astype(np.float64)
    worst_o, worst_l = 0.0, 0.0
    for b in range(wl.B):
        d = int(wl.draft_lens[b])
        r_l, g_l = rl[b, :, :d], gl[b, :, :d]
        assert np.array_equal(np.isneginf(r_l), np.isneginf(g_l)), "empty splits differ"
        assert np.all(np.isnan(gl[b, :, d:])) and np.all(np.isnan(go[b, :, d:])), "rows past the draft written"
        live = ~np.isneginf(r_l)
        assert np.all(go[b, :, :d][~live] == 0.0), "a split with no visible key has a non-zero row"
        err_l = np.abs(g_l[live] - r_l[live])
        # l sums p rounded to fp16 (each a relative 2^-11 at most): |d lse| <= 2^-11 + score rounding
        assert err_l.max() <= 1e-3, f"lse error {err_l.max():.2e}"
        r_o, g_o, m_o = ro[b, :, :d][live], go[b, :, :d][live], mo[b, :, :d][live]
        assert np.all(np.isfinite(g_o))
        # the binary16 underflow floor of each row, over its split's keys at most
        fl = prep.p_floor(np.array([(b, t, 0) for t in range(d)]))            # [d]
        fl = np.broadcast_to(fl[None, :, None], live.shape)[live][:, None]
        ratio = (np.abs(g_o - r_o) - fl) / np.maximum(m_o, 1e-300)
        worst_o, worst_l = max(worst_o, float(ratio.max())), max(worst_l, float(err_l.max()))
        assert ratio.max() <= MAG_REL, f"request {b}: partial element off by {ratio.max():.2e} of its size"
    log(f"  partials (v_mag {v_mag}): max |err| / mag {worst_o:.2e}, max |d lse| {worst_l:.2e}")
    # the exported merge over the kernel's own partials = the whole call
    out = torch.full(tuple(wl.q.shape), BF16_NAN, dtype=torch.int16, device="cuda")
    sda.splash_verify_attn_splitk_merge(part_o, part_lse, out, prep.dl)
    torch.cuda.synchronize()
    rows = prep.valid_rows()
    got = bf16_to_f64(out.cpu().numpy()[rows[:, 0], rows[:, 1], rows[:, 2]])
    assert_attn_ok(got, prep.oracle_rows(rows), f"partition + merge (v_mag {v_mag})",
                   mag=prep.oracle_rows(rows, abs_v=True), floor=prep.p_floor(rows), v_scale=v_mag)


@pytest.mark.parametrize("shape", [(24, 256), (16, 128), (8, 64)])
def test_merge_matches_oracle(shape):
    """The exported merge on fp32 partials in the oracle's own layout, with NaN in
    the rows of empty splits and splits past a batch of the kernel's loads."""
    Hq, D = shape
    rng = np.random.default_rng(5)
    B, T, S = 3, 16, 37
    po = rng.standard_normal((B, Hq, T, S, D)).astype(np.float32)
    pl = (rng.standard_normal((B, Hq, T, S)) * 3).astype(np.float32)
    pl[rng.random(pl.shape) < 0.2] = -np.inf                # empty splits
    pl[..., 0] = rng.standard_normal((B, Hq, T)).astype(np.float32)   # one live split
    po[np.isneginf(pl)] = np.nan                            # rows of empty splits hold anything
    dl = np.array([16, 3, 0], np.int32)
    ref = oracle.load().splitk_merge(po, pl, dl, T)
    out = torch.full((B, T, Hq, D), BF16_NAN, dtype=torch.int16, device="cuda")
    sda.splash_verify_attn_splitk_merge(up(po), up(pl), out, up(dl))
    got = bf16_to_f64(out.cpu().numpy())
    for b in range(B):
        d = int(dl[b])
        if d:
            assert_attn_ok(got[b, :d], ref[b, :d], f"merge {shape} request {b}")
        assert np.all(out[b, d:].cpu().numpy().view(np.uint16) == BF16_NAN)


def test_merge_is_deterministic_and_order_fixed():
    """Repeated merges give identical bits; a single live split passes its row through."""
    rng = np.random.default_rng(6)
    B, Hq, T, S, D = 2, 24, 16, 64, 256
    po = rng.standard_normal((B, Hq, T, S, D)).astype(np.float32)
    pl = np.full((B, Hq, T, S), -np.inf, np.float32)
    pl[..., 17] = 2.5
    dl = np.array([16, 16], np.int32)
    out = torch.empty((B, T, Hq, D), dtype=torch.int16, device="cuda")
    sda.splash_verify_attn_splitk_merge(up(po), up(pl), out, up(dl))
    a = out.cpu().numpy().copy()
    sda.splash_verify_attn_splitk_merge(up(po), up(pl), out, up(dl))
    assert np.array_equal(a, out.cpu().numpy())
    want = torch.from_numpy(np.ascontiguousarray(po[..., 17, :].transpose(0, 2, 1, 3))).to(torch.bfloat16)
    assert np.array_equal(a, want.view(torch.int16).numpy())


@pytest.mark.parametrize("B,Hkv,ctx,D,cap", [
    (1, 2, 256, 64, 1),           # config 1: 16 pages at D = 64, one split (no merge launch)
    (1, 2, 512, 64, 4),           # 32 pages at D = 64: 8 pages a split
    (1, 4, 256, 256, 4),          # 16 pages at D = 256: one 4-page step a split
    (1, 4, 1024, 256, 16),        # 64 pages at D = 256: still 4 pages a split
    (1, 4, 2048, 256, 16),        # 128 pages: 8 pages a split again
    (1, 4, 32768, 256, 256),      # config 3
    (16, 4, 32768, 256, 256),     # config 5
])
def test_split_preset(B, Hkv, ctx, D, cap):
    """The split preset: one workgroup per compute unit over B * Hkv work items,
    capped by the pages a split must at least hold (the cap column)."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    want = max(1, min(-(-cus // (B * Hkv)), cap))
    assert sda.splash_verify_attn_default_splits(B, Hkv, ctx, 16, D) == want
