"""GPU parity at the edges of the sizes the path is used at: a 128K-token
context (the context-scaling benchmark's longest), a batch of 128 ragged
requests, and contexts of exactly one block, every valid row against the fp64
oracle.  Tolerance as in the other attention tests."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

import speculative_decode_attention_amd as sda  # noqa: E402
from speculative_decode_attention_amd import synth  # noqa: E402
from gpu_util import BF16_NAN, Prepared, assert_attn_ok, bf16_to_f64, log  # noqa: E402


def check(prep, S, where):
    wl = prep.wl
    out = prep.run(num_splits=S).cpu().numpy()
    rows = prep.valid_rows()
    got = bf16_to_f64(out[rows[:, 0], rows[:, 1], rows[:, 2]])
    assert_attn_ok(got, prep.oracle_rows(rows), where, mag=prep.oracle_rows(rows, abs_v=True), floor=prep.p_floor(rows))
    for b in range(wl.B):
        assert np.all(out[b, int(wl.draft_lens[b]):].view(np.uint16) == BF16_NAN), f"{where}: row written"


def test_context_128k():
    log("limits: one request, 131072-token context")
    wl = synth.make_workload("limits128k", 91, B=1, context_lens=[131072], T_max=16, Hq=24, Hkv=4, D=256,
                             num_pages=131072 // 16 + 8)
    prep = Prepared(wl)
    check(prep, 0, "128K context, preset splits")
    check(prep, 256, "128K context, 256 splits")


def test_batch_of_128_ragged_requests():
    log("limits: 128 requests, ragged contexts and drafts")
    rng = np.random.default_rng(92)
    ctx = rng.integers(17, 700, size=128).astype(np.int32)
    dl = np.minimum(rng.integers(0, 17, size=128), ctx).astype(np.int32)
    pages = int(sum(-(-c // 16) for c in ctx)) + 8
    wl = synth.make_workload("limits_b128", 93, B=128, context_lens=list(ctx), T_max=16, draft_lens=list(dl),
                             Hq=24, Hkv=4, D=256, num_pages=pages)
    prep = Prepared(wl)
    for S in (0, 1, 3):
        check(prep, S, f"128 requests, {S} splits")


def test_context_of_exactly_one_block():
    """Contexts of exactly 16 tokens that are all drafts: no key before the block."""
    wl = synth.make_workload("limits_one_block", 94, B=3, context_lens=[16, 16, 9], T_max=16, draft_lens=[16, 1, 9],
                             Hq=24, Hkv=4, D=256, num_pages=8)
    prep = Prepared(wl)
    for S in (0, 1, 2):
        check(prep, S, f"one-block contexts, {S} splits")
