"""GPU parity for sliding-window verify attention (splash_verify_attn_window):
the HIP path through the C ABI against the fp64 oracle with the same window,
with the attention tolerance; a window past the context against the causal
call, bit for bit.  Only the pages inside each request's window are read, so
the windows below also move the first page of every split."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

import oracle  # noqa: E402
import speculative_decode_attention_amd as sda  # noqa: E402
from speculative_decode_attention_amd import synth  # noqa: E402
from gpu_util import BF16_NAN, Prepared, assert_attn_ok, bf16_to_f64, log, prepared_config  # noqa: E402


def run_window(prep, window, num_splits=0):
    wl = prep.wl
    out = torch.full(tuple(wl.q.shape), BF16_NAN, dtype=torch.int16, device="cuda")
    sda.splash_verify_attn_window(prep.q, out, *prep.g_pools, prep.bt, prep.ctx, prep.dl, window,
                                  wl.max_context_len, wl.sm_scale, num_splits=num_splits)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def check_window(prep, window, num_splits, where):
    wl = prep.wl
    out = run_window(prep, window, num_splits)
    ref = oracle.load().verify_attn_window(wl.q, *prep.pools, wl.block_table, wl.context_lens, wl.draft_lens,
                                           wl.Hkv, wl.sm_scale, window)
    rows = prep.valid_rows()
    got = bf16_to_f64(out[rows[:, 0], rows[:, 1], rows[:, 2]])
    mag = oracle.load().verify_attn_window(wl.q, *prep.abs_pools, wl.block_table, wl.context_lens, wl.draft_lens,
                                           wl.Hkv, wl.sm_scale, window)
    assert_attn_ok(got, ref[rows[:, 0], rows[:, 1], rows[:, 2]], where, mag=mag[rows[:, 0], rows[:, 1], rows[:, 2]],
                   floor=prep.p_floor(rows))
    for b in range(wl.B):
        assert np.all(out[b, int(wl.draft_lens[b]):].view(np.uint16) == BF16_NAN)


@pytest.mark.parametrize("cfg,window", [(1, 1), (1, 37), (2, 1), (2, 100), (2, 2048), (3, 4096), (4, 1000)])
def test_window_matches_oracle(cfg, window):
    prep = prepared_config(cfg) if cfg != 1 else Prepared(synth.make_config(1))
    span = sda.splash_verify_attn_window_tokens(prep.wl.max_context_len, prep.wl.T_max, window)
    log(f"  config {cfg}, window {window}: the splits cover {span} tokens")
    check_window(prep, window, 0, f"config {cfg}, window {window}")


@pytest.mark.parametrize("S", [1, 3, 16])
def test_window_split_counts(S):
    check_window(prepared_config(2), 1000, S, f"config 2, window 1000, {S} splits")


def test_window_ragged_requests():
    """Requests whose windows start in different pages (and one inside a page)."""
    wl = synth.make_workload("window", 43, B=3, context_lens=[700, 130, 64], T_max=16, draft_lens=[16, 9, 1],
                             Hq=24, Hkv=4, D=256, num_pages=128)
    prep = Prepared(wl)
    for W in (5, 77, 129):
        check_window(prep, W, 0, f"ragged requests, window {W}")


@pytest.mark.parametrize("cfg", [2, 3])
def test_window_past_the_context_is_causal(cfg):
    prep = prepared_config(cfg)
    causal = prep.run(num_splits=0).cpu().numpy()
    wide = run_window(prep, prep.wl.max_context_len + 5)
    assert np.array_equal(causal, wide), "a window past the context must give the causal rows bit for bit"
