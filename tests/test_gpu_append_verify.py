"""GPU parity for splash_verify_attn_append: the append of the drafted block and
the verify call in one launch.  The pools handed in hold every earlier append
but not the block (its slots hold poison, codes 127 with scale 8, so reading
them would move the result).  After the call the pools must equal the oracle's
append byte for byte and the output must equal splash_kv_append_int8 followed by
splash_verify_attn bit for bit, and meet the attention tolerance against the
fp64 oracle.  Blocks that straddle two pages, two steps and two splits, ragged
drafts, bf16 sources, the three compiled shapes, repeated calls (re-appending
is idempotent) and replays of a captured step are covered."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

import speculative_decode_attention_amd as sda  # noqa: E402
from speculative_decode_attention_amd import synth  # noqa: E402
from gpu_util import BF16_NAN, Prepared, assert_attn_ok, bf16_to_f64, log, up  # noqa: E402

NAMES = ("k_pool", "v_pool", "k_scale", "v_scale")


def pools_without_block(prep):
    """GPU pools holding every append phase but the last (the drafted block)."""
    wl = prep.wl
    g = [up(a) for a in (wl.k_pool, wl.v_pool, wl.k_scale, wl.v_scale)]
    for ph in wl.appends[:-1]:
        sda.splash_kv_append_int8(up(ph.k_src), up(ph.v_src), *g, up(ph.block_table), up(ph.context_lens),
                                  up(ph.draft_lens))
    torch.cuda.synchronize()
    return g


def drafts_source(prep, bf16=False):
    ph = prep.wl.appends[-1]
    k, v = up(ph.k_src), up(ph.v_src)
    if bf16:
        k, v = k.to(torch.bfloat16), v.to(torch.bfloat16)
    return k, v


def assert_pools(dev_pools, host_pools, where):
    for name, dev, host in zip(NAMES, dev_pools, host_pools):
        got = dev.cpu().numpy()
        got = got.view(np.uint16) if host.dtype == np.uint16 else got
        bad = np.flatnonzero(got.ravel() != host.ravel())
        assert bad.size == 0, f"{where}: {name} differs from the oracle's append at {bad.size} bytes, first {bad[0]}"


def oracle_pools_bf16(prep, kb, vb):
    """The oracle's pools with the block appended from bf16-rounded source rows."""
    import oracle
    wl = prep.wl
    orc = oracle.load()
    pl = [a.copy() for a in (wl.k_pool, wl.v_pool, wl.k_scale, wl.v_scale)]
    for ph in wl.appends[:-1]:
        orc.kv_append_int8(ph.k_src, ph.v_src, *pl, ph.block_table, ph.context_lens, ph.draft_lens)
    last = wl.appends[-1]
    orc.kv_append_int8(kb, vb, *pl, last.block_table, last.context_lens, last.draft_lens)
    return pl


def check_against_append(prep, S, where, bf16=False):
    wl = prep.wl
    pools = pools_without_block(prep)
    k_new, v_new = drafts_source(prep, bf16)
    out = torch.full(tuple(wl.q.shape), BF16_NAN, dtype=torch.int16, device="cuda")
    sda.splash_verify_attn_append(k_new, v_new, prep.q, out, *pools, prep.bt, prep.ctx, prep.dl, wl.max_context_len,
                                  wl.sm_scale, num_splits=S)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    rows = prep.valid_rows()
    g = bf16_to_f64(got[rows[:, 0], rows[:, 1], rows[:, 2]])
    if bf16:
        # the block's source rounded to bf16 quantises differently: compare with the oracle on those codes
        kb, vb = (x.float().cpu().numpy() for x in (k_new, v_new))
        pl = oracle_pools_bf16(prep, kb, vb)
        assert_pools(pools, pl, where)
        import oracle
        ref = oracle.load().verify_attn_rows(wl.q, *pl, wl.block_table, wl.context_lens, wl.draft_lens, wl.Hkv,
                                             wl.sm_scale, rows)
        assert_attn_ok(g, ref, where)
    else:
        assert_pools(pools, prep.pools, where)
        want = prep.run(num_splits=S).cpu().numpy()      # the oracle-checked pools: append, then verify
        assert np.array_equal(got, want), f"{where}: differs from append + verify"
        assert_attn_ok(g, prep.oracle_rows(rows), where, mag=prep.oracle_rows(rows, abs_v=True),
                       floor=prep.p_floor(rows))
    for b in range(wl.B):
        assert np.all(got[b, int(wl.draft_lens[b]):].view(np.uint16) == BF16_NAN)


_cache = {}


def prepared(name, **kw):
    if name not in _cache:
        _cache.clear()
        _cache[name] = Prepared(synth.make_workload(name, 51, **kw))
    return _cache[name]


STRADDLE = dict(B=3, context_lens=[4104, 1000, 70], T_max=16, draft_lens=[16, 16, 11], Hq=24, Hkv=4, D=256,
                num_pages=400)


@pytest.mark.parametrize("S", [1, 3, 7, 0])
def test_append_verify_blocks_across_pages_steps_and_splits(S):
    """Blocks at 4088..4103 (pages 255 | 256, steps 63 | 64), 984..999 (one
    step) and 59..69 (steps 0 | 1); 3 and 7 splits also cut between them."""
    prep = prepared("drafts_straddle", **STRADDLE)
    check_against_append(prep, S, f"straddling blocks, {S or 'preset'} splits")


def test_append_verify_bf16_source():
    prep = prepared("drafts_straddle", **STRADDLE)
    check_against_append(prep, 3, "bf16 source rows, 3 splits", bf16=True)


@pytest.mark.parametrize("cfg", [2, 3, 5])
def test_append_verify_configs(cfg):
    from gpu_util import prepared_config
    prep = prepared_config(cfg)
    check_against_append(prep, 0, f"config {cfg}, preset splits")


@pytest.mark.parametrize("shape", [(8, 2, 64), (32, 4, 128)])
def test_append_verify_other_shapes(shape):
    Hq, Hkv, D = shape
    prep = Prepared(synth.make_workload("drafts_shape", 52, B=2, context_lens=[300, 77], T_max=16,
                                        draft_lens=[16, 5], Hq=Hq, Hkv=Hkv, D=D, num_pages=40))
    for S in (1, 3):
        check_against_append(prep, S, f"D={D}, {S} splits")


def test_append_verify_step_captured_and_replayed():
    """The step captured in a HIP graph and replayed three times over pools without
    the block, with eager work and synchronisation between the replays: every
    replay appends the block (first time, then again over itself) and returns
    the output of append + verify."""
    prep = prepared("drafts_straddle", **STRADDLE)
    wl = prep.wl
    want = prep.run(num_splits=0).cpu().numpy()
    pools = pools_without_block(prep)
    fresh = [p.clone() for p in pools]
    k_new, v_new = drafts_source(prep)
    out = torch.full(tuple(wl.q.shape), BF16_NAN, dtype=torch.int16, device="cuda")
    S = sda.effective_splits(wl.max_context_len, wl.P, sda.splash_verify_attn_default_splits(
        wl.B, wl.Hkv, wl.max_context_len, wl.P, wl.D))
    ws = torch.empty(sda.splash_verify_attn_workspace_bytes(wl.B, wl.T_max, wl.Hq, wl.D, S), dtype=torch.uint8,
                     device="cuda")

    def step():
        sda.splash_verify_attn_append(k_new, v_new, prep.q, out, *pools, prep.bt, prep.ctx, prep.dl,
                                      wl.max_context_len, wl.sm_scale, num_splits=S, workspace=ws)

    step()                                                # eager: every lazy init done
    torch.cuda.synchronize()
    for p, f in zip(pools, fresh):
        p.copy_(f)
    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        step()
    for rep in range(3):
        if rep == 1:
            for p, f in zip(pools, fresh):                # back to the pools without the block
                p.copy_(f)
        out.fill_(BF16_NAN)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), want), f"replay {rep}: differs from append + verify"
        assert_pools(pools, prep.pools, f"replay {rep}")
    log("  captured append + verify step: 3 replays identical to append + verify, pools equal to the oracle's")


@pytest.mark.parametrize("S", [1, 2, 0])
def test_append_verify_short_contexts_and_empty_blocks(S):
    """A context that is its block (no key before it), a block straddling pages 0
    and 1, a request with no block (a no-op: its pages stay as they were), a
    one-token block, and a block filling page 2 exactly."""
    prep = prepared("drafts_short", B=5, context_lens=[16, 17, 9, 3, 48], T_max=16, draft_lens=[16, 5, 0, 1, 16],
                    Hq=24, Hkv=4, D=256, num_pages=64)
    check_against_append(prep, S, f"short contexts, {S or 'preset'} splits")
