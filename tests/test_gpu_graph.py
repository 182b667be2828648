"""The hot path captured in a HIP graph: every replay, with the program's own
eager work and synchronisations between replays, gives the same bits as the
eager call (the benchmark times such replays)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

import speculative_decode_attention_amd as sda  # noqa: E402
from speculative_decode_attention_amd import synth  # noqa: E402
from gpu_util import BF16_NAN, Prepared, assert_attn_ok, bf16_to_f64, log, up  # noqa: E402


@pytest.mark.parametrize("num_splits", [0, 1, 5])
def test_graph_replays_match_eager(num_splits):
    wl = synth.make_workload("graph", 77, B=3, context_lens=[1500, 260, 33], T_max=16,
                             draft_lens=[16, 7, 1], Hq=24, Hkv=4, D=256, num_pages=256,
                             shared_prefix=16)
    prep = Prepared(wl)
    draft = wl.appends[-1]
    k_new, v_new = up(draft.k_src), up(draft.v_src)
    bt, ctx, dl = prep.bt, prep.ctx, prep.dl
    S = sda.effective_splits(wl.max_context_len, wl.P, num_splits or sda.splash_verify_attn_default_splits(
        wl.B, wl.Hkv, wl.max_context_len, wl.P, wl.D))
    ws = torch.empty(max(sda.splash_verify_attn_workspace_bytes(wl.B, wl.T_max, wl.Hq, wl.D, S), 16),
                     dtype=torch.uint8, device="cuda")
    out = torch.full(tuple(wl.q.shape), BF16_NAN, dtype=torch.int16, device="cuda")

    def step():
        sda.splash_kv_append_int8(k_new, v_new, *prep.g_pools, bt, ctx, dl)
        sda.splash_verify_attn(prep.q, out, *prep.g_pools, bt, ctx, dl, wl.max_context_len,
                               wl.sm_scale, num_splits=num_splits, workspace=ws)

    step()                                   # eager (re-appending the drafts is idempotent)
    torch.cuda.synchronize()
    eager = out.clone()
    pools_eager = [p.clone() for p in prep.g_pools]
    rows = prep.valid_rows()
    got = bf16_to_f64(eager.cpu().numpy()[rows[:, 0], rows[:, 1], rows[:, 2]])
    assert_attn_ok(got, prep.oracle_rows(rows), f"eager, {S} splits")

    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=cap):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        out.fill_(BF16_NAN)                  # eager work between replays
        scratch = torch.randn(1 << 20, device="cuda").sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(scratch)
        assert torch.equal(out, eager), f"replay {rep} differs from the eager call"
        for p, pe in zip(prep.g_pools, pools_eager):
            assert torch.equal(p, pe), f"replay {rep}: pools differ"
    log(f"  {S} splits: 4 replays bit-identical to eager")
    # rows past each request's draft stay untouched
    o = out.cpu().numpy()
    for b in range(wl.B):
        assert np.all(o[b, int(wl.draft_lens[b]):].view(np.uint16) == BF16_NAN)
