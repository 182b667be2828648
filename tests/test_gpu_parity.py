"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Append/quantise: whole pools byte-identical (poison bytes included).
Attention: bf16 rows against the unrounded fp64 oracle, relative L2 <= 2e-3 and
every element within 1e-2 plus half a bf16 ulp.  Full outputs where the oracle
is quick; at the 32K-context sizes a seeded sample of rows, each computed by
the oracle one by one, in the launch configuration the benchmark times (the
split preset).
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

import oracle  # noqa: E402
import speculative_decode_attention_amd as sda  # noqa: E402
from speculative_decode_attention_amd import synth  # noqa: E402
from gpu_util import (BF16_NAN, Prepared, assert_attn_ok, bf16_to_f64, blocks_to_heads,  # noqa: E402
                      heads_to_blocks, log, prepared_config, tile_partials, untile_partials, up)

# rows checked per configuration (None = every row)
SAMPLE = {1: None, 2: None, 3: None, 4: 192, 5: 192}


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
    rows = prep.valid_rows()
    if SAMPLE[cfg] is not None and len(rows) > SAMPLE[cfg]:
        rng = np.random.default_rng(100 + cfg)
        rows = rows[np.sort(rng.choice(len(rows), SAMPLE[cfg], replace=False))]
    ref = prep.oracle_rows(rows)
    got = bf16_to_f64(out[rows[:, 0], rows[:, 1], rows[:, 2]])
    assert_attn_ok(got, ref, f"config {cfg} ({len(rows)} rows)", mag=prep.oracle_rows(rows, abs_v=True))
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
    assert_attn_ok(got, ref, f"config 2, {S} splits", mag=prep.oracle_rows(rows, abs_v=True))


@pytest.mark.parametrize("v_mag", [1.0, 3e4])
def test_partition_partials_match_oracle_split(v_mag):
    """Tiled fp16 partials and log-sum-exps of each split, including empty
    splits; with V scales past 255 the blocks carry an exponent shift k > 0."""
    wl = synth.make_workload("part", 31, B=2, context_lens=[700, 130], T_max=16, draft_lens=[16, 9],
                             Hq=24, Hkv=4, D=256, num_pages=128, v_mag=v_mag)
    prep = Prepared(wl)
    G, S = wl.G, 13
    # documented split length: ceil(pages / S) rounded up to whole 4-page steps
    cdiv = lambda a, b: -(-a // b)
    L = 4 * cdiv(cdiv(cdiv(wl.max_context_len, wl.P), S), 4)   # 4 pages: splits 11, 12 empty
    assert sda.splash_verify_attn_split_pages(wl.max_context_len, wl.P, S) == L
    po_shape, pl_shape = sda.partial_shapes(wl.B, wl.Hq, wl.Hkv, wl.D, S)
    part_o = torch.full(po_shape, 0x7E00, dtype=torch.int16, device="cuda")   # fp16 NaN
    part_lse = torch.full(pl_shape, float("nan"), device="cuda")
    sda.splash_verify_attn_partition(prep.q, *prep.g_pools, prep.bt, prep.ctx, prep.dl,
                                     wl.max_context_len, wl.sm_scale, S, part_o, part_lse)
    torch.cuda.synchronize()
    ro, rl = oracle.load().verify_attn_split(wl.q, *prep.pools, wl.block_table, wl.context_lens,
                                             wl.draft_lens, wl.Hkv, wl.sm_scale, S, L)
    gl_blk = part_lse.cpu().numpy().astype(np.float64)                    # [B][Hkv][S][16G]
    go_blk = untile_partials(part_o.cpu().numpy(), G, wl.D)              # [B][Hkv][S][16G][D]
    # exponent shift per block, read off the log-sum-exps: a whole k >= 0
    rl_blk = heads_to_blocks(rl, wl.Hkv)
    ks = []
    for b in range(wl.B):
        rows = G * int(wl.draft_lens[b])
        r_l, g_l = rl_blk[b, :, :, :rows], gl_blk[b, :, :, :rows]
        assert np.array_equal(np.isneginf(r_l), np.isneginf(g_l)), "empty splits differ"
        assert np.all(np.isnan(gl_blk[b, :, :, rows:])), "rows past the draft written"
        for g in range(wl.Hkv):
            for s in range(S):
                live = ~np.isneginf(r_l[g, s])
                if not live.any():
                    continue
                kk = (g_l[g, s, live] - r_l[g, s, live]) / np.log(2.0)
                k = int(np.rint(kk[0]))
                assert k >= 0 and np.max(np.abs(kk - k)) < 2e-4, f"lse shift not a whole power: {kk[:4]}"
                rows_view = go_blk[b, g, s, :rows]
                rows_view[live] *= 2.0 ** k
                ks.append(k)
    go, gl = blocks_to_heads(go_blk, G, wl.T_max), blocks_to_heads(gl_blk, G, wl.T_max)
    for b in range(wl.B):
        d = int(wl.draft_lens[b])
        live = ~np.isneginf(rl[b, :, :d])
        r_o, g_o = ro[b, :, :d][live], go[b, :, :d][live]
        assert np.all(np.isfinite(g_o))
        rel = np.linalg.norm(g_o - r_o) / np.linalg.norm(r_o)
        log(f"  partials request {b}: rows rel-L2 {rel:.2e}, shifts {sorted(set(ks))}")
        assert rel < 1.5e-3
    assert (max(ks) > 0) == (v_mag > 1.0)


@pytest.mark.parametrize("shape", [(24, 4, 256), (16, 2, 128), (8, 2, 64)])
def test_merge_matches_oracle(shape):
    Hq, Hkv, D = shape
    G = Hq // Hkv
    rng = np.random.default_rng(5)
    B, T, S = 3, 16, 37
    po = rng.standard_normal((B, Hkv, S, 16 * G, D)).astype(np.float16)
    pl = (rng.standard_normal((B, Hkv, S, 16 * G)) * 3).astype(np.float32)
    pl[rng.random(pl.shape) < 0.2] = -np.inf                # empty splits
    pl[:, :, 0] = rng.standard_normal((B, Hkv, 16 * G)).astype(np.float32)   # one live split
    po[np.isneginf(pl)] = np.nan                            # rows of empty splits hold anything
    dl = np.array([16, 3, 0], np.int32)
    ref = oracle.load().splitk_merge(np.nan_to_num(blocks_to_heads(po.astype(np.float64), G, T)),
                                     blocks_to_heads(pl, G, T), dl, T)
    out = torch.full((B, T, Hq, D), BF16_NAN, dtype=torch.int16, device="cuda")
    sda.splash_verify_attn_splitk_merge(up(tile_partials(po, G, D)), up(pl), out, up(dl))
    got = bf16_to_f64(out.cpu().numpy())
    for b in range(B):
        d = int(dl[b])
        if d:
            assert_attn_ok(got[b, :d], ref[b, :d], f"merge {shape} request {b}")
        assert np.all(out[b, d:].cpu().numpy().view(np.uint16) == BF16_NAN)
