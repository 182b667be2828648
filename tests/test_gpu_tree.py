"""GPU parity for tree-shaped verify masks (splash_verify_attn_masked): the HIP
path through the C ABI against the fp64 oracle given the same masks, with the
attention tolerance; and the chain mask against the causal call, bit for bit.
Random candidate trees: draft t hangs under a drawn earlier draft and sees its
ancestors and itself."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

import oracle  # noqa: E402
import speculative_decode_attention_amd as sda  # noqa: E402
from speculative_decode_attention_amd import synth  # noqa: E402
from gpu_util import (BF16_NAN, Prepared, assert_attn_ok, bf16_to_f64, log,  # noqa: E402
                      prepared_config, up)


def run_masked(prep, masks, num_splits=0):
    wl = prep.wl
    out = torch.full(tuple(wl.q.shape), BF16_NAN, dtype=torch.int16, device="cuda")
    sda.splash_verify_attn_masked(prep.q, out, *prep.g_pools, prep.bt, prep.ctx, prep.dl,
                                  up(masks.view(np.int32)), wl.max_context_len, wl.sm_scale,
                                  num_splits=num_splits)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def check_tree(prep, masks, num_splits, where):
    wl = prep.wl
    out = run_masked(prep, masks, num_splits)
    ref = oracle.load().verify_attn_masked(wl.q, *prep.pools, wl.block_table, wl.context_lens, wl.draft_lens,
                                           wl.Hkv, wl.sm_scale, masks)
    rows = prep.valid_rows()
    got = bf16_to_f64(out[rows[:, 0], rows[:, 1], rows[:, 2]])
    mag = oracle.load().verify_attn_masked(wl.q, *prep.abs_pools, wl.block_table, wl.context_lens, wl.draft_lens,
                                           wl.Hkv, wl.sm_scale, masks)
    assert_attn_ok(got, ref[rows[:, 0], rows[:, 1], rows[:, 2]], where, mag=mag[rows[:, 0], rows[:, 1], rows[:, 2]],
                   floor=prep.p_floor(rows))
    for b in range(wl.B):                                     # rows past the draft stay untouched
        assert np.all(out[b, int(wl.draft_lens[b]):].view(np.uint16) == BF16_NAN)


@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_tree_mask_matches_oracle(cfg):
    prep = prepared_config(cfg) if cfg != 1 else Prepared(synth.make_config(1))
    masks = synth.tree_block_masks(500 + cfg, prep.wl.draft_lens, prep.wl.T_max)
    log(f"  config {cfg}: tree masks {masks[0, :int(prep.wl.draft_lens[0])]}")
    check_tree(prep, masks, 0, f"config {cfg}, tree mask")


@pytest.mark.parametrize("S", [1, 3, 16])
def test_tree_mask_split_counts(S):
    prep = prepared_config(2)
    masks = synth.tree_block_masks(600 + S, prep.wl.draft_lens, prep.wl.T_max)
    check_tree(prep, masks, S, f"config 2, tree mask, {S} splits")


def test_tree_mask_ragged_drafts():
    """Several requests with different block lengths (one of a single draft)."""
    wl = synth.make_workload("tree", 41, B=3, context_lens=[700, 130, 64], T_max=16, draft_lens=[16, 9, 1],
                             Hq=24, Hkv=4, D=256, num_pages=128)
    prep = Prepared(wl)
    check_tree(prep, synth.tree_block_masks(42, wl.draft_lens, wl.T_max), 0, "ragged blocks, tree mask")


@pytest.mark.parametrize("cfg", [2, 3])
def test_chain_mask_is_the_causal_call(cfg):
    prep = prepared_config(cfg)
    causal = prep.run(num_splits=0).cpu().numpy()
    chain = run_masked(prep, synth.chain_block_masks(prep.wl.draft_lens, prep.wl.T_max))
    assert np.array_equal(causal, chain), "the chain mask must give the causal rows bit for bit"
