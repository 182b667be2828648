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
    assert_attn_ok(got, prep.oracle_rows(rows), f"eager, {S} splits", mag=prep.oracle_rows(rows, abs_v=True), floor=prep.p_floor(rows))

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


def _replays_match(call, outputs, reset, where):
    """Eager call, capture, then 4 replays with eager work between: each replay
    gives the eager bits in every output tensor."""
    reset()
    call()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outputs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=torch.cuda.Stream()):
        call()
    torch.cuda.synchronize()
    for rep in range(4):
        reset()                                               # eager work between replays
        scratch = torch.randn(1 << 20, device="cuda").sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(scratch)
        for o, e in zip(outputs, eager):
            assert torch.equal(o, e), f"{where}: replay {rep} differs from the eager call"
    log(f"  {where}: 4 replays bit-identical to eager")


@pytest.mark.parametrize("kind", ["tree", "window", "prefill"])
def test_graph_replays_other_attention_calls(kind):
    T_max = 40 if kind == "prefill" else 16
    dls = [40, 17, 3] if kind == "prefill" else [16, 7, 1]
    wl = synth.make_workload("graph2", 78, B=3, context_lens=[1500, 260, 33], T_max=T_max, draft_lens=dls,
                             Hq=24, Hkv=4, D=256, num_pages=256)
    prep = Prepared(wl)
    out = torch.full(tuple(wl.q.shape), BF16_NAN, dtype=torch.int16, device="cuda")
    ws = torch.empty(1 << 25, dtype=torch.uint8, device="cuda")
    args = (prep.q, out, *prep.g_pools, prep.bt, prep.ctx, prep.dl)
    if kind == "tree":
        masks = up(synth.tree_block_masks(79, wl.draft_lens, T_max).view(np.int32))
        call = lambda: sda.splash_verify_attn_masked(*args, masks, wl.max_context_len, wl.sm_scale, workspace=ws)
    elif kind == "window":
        call = lambda: sda.splash_verify_attn_window(*args, 100, wl.max_context_len, wl.sm_scale, workspace=ws)
    else:
        call = lambda: sda.splash_prefill_attn(*args, wl.max_context_len, wl.sm_scale, workspace=ws)
    _replays_match(call, [out], lambda: out.fill_(BF16_NAN), kind)


def test_graph_replays_acceptance():
    """Acceptance rolls context_lens back in place: the eager work restores it
    before each replay, and every replay gives the same accepted counts, next
    tokens and rolled-back lengths."""
    case = synth.make_accept_case(21, B=16, T_max=16)
    logits = up(case.logits.view(np.int16))
    bt, dl = up(case.block_tokens), up(case.draft_lens)
    ctx0 = up(case.context_lens)
    ctx = ctx0.clone()
    acc = torch.empty(case.B, dtype=torch.int32, device="cuda")
    nxt = torch.empty(case.B, dtype=torch.int32, device="cuda")
    ws = torch.empty(max(sda.splash_verify_accept_workspace_bytes(case.B, 16, case.V), 16), dtype=torch.uint8,
                     device="cuda")

    def reset():
        ctx.copy_(ctx0)
        acc.fill_(-1)
        nxt.fill_(-1)

    _replays_match(lambda: sda.splash_verify_accept(logits, bt, dl, ctx, acc, nxt, workspace=ws), [acc, nxt, ctx],
                   reset, "acceptance")
