"""GPU parity for chunked-prefill attention (splash_prefill_attn): the HIP path
through the C ABI against the fp64 oracle (the verify definition with a long
block), with the attention tolerance, on every valid row.  Chunks of 33 to 512
tokens, a ragged last 16-token block, all three compiled shapes, split counts,
and a 512-token chunk at the end of a 32K context; a 16-token chunk is the
verify call bit for bit."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

import oracle  # noqa: E402
import speculative_decode_attention_amd as sda  # noqa: E402
from speculative_decode_attention_amd import synth  # noqa: E402
from gpu_util import BF16_NAN, Prepared, assert_attn_ok, bf16_to_f64, log  # noqa: E402


def run_prefill(prep, num_splits=0):
    wl = prep.wl
    out = torch.full(tuple(wl.q.shape), BF16_NAN, dtype=torch.int16, device="cuda")
    sda.splash_prefill_attn(prep.q, out, *prep.g_pools, prep.bt, prep.ctx, prep.dl, wl.max_context_len,
                            wl.sm_scale, num_splits=num_splits)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def check_prefill(prep, num_splits, where):
    wl = prep.wl
    out = run_prefill(prep, num_splits)
    rows = prep.valid_rows()
    ref = prep.oracle_rows(rows)
    got = bf16_to_f64(out[rows[:, 0], rows[:, 1], rows[:, 2]])
    assert_attn_ok(got, ref, where, mag=prep.oracle_rows(rows, abs_v=True), floor=prep.p_floor(rows))
    for b in range(wl.B):                                     # rows past each chunk stay untouched
        assert np.all(out[b, int(wl.draft_lens[b]):].view(np.uint16) == BF16_NAN)


def chunk_workload(seed, *, context_lens, chunk_lens, T_max, Hq=24, Hkv=4, D=256):
    pages = sum(-(-c // 16) for c in context_lens) + 8
    return synth.make_workload("prefill", seed, B=len(context_lens), context_lens=context_lens, T_max=T_max,
                               draft_lens=chunk_lens, Hq=Hq, Hkv=Hkv, D=D, num_pages=pages)


@pytest.mark.parametrize("name,kw", [
    ("two_requests_64", dict(context_lens=[300, 700], chunk_lens=[64, 37], T_max=64)),
    ("ragged_last_block_200", dict(context_lens=[2000], chunk_lens=[200], T_max=200)),
    ("chunk_is_the_whole_context", dict(context_lens=[96, 130], chunk_lens=[96, 130], T_max=130)),
    ("d64", dict(context_lens=[500, 90], chunk_lens=[48, 90], T_max=90, Hq=8, Hkv=2, D=64)),
    ("d128", dict(context_lens=[400], chunk_lens=[48], T_max=48, Hq=32, Hkv=4, D=128)),
])
def test_prefill_matches_oracle(name, kw):
    prep = Prepared(chunk_workload(11, **kw))
    check_prefill(prep, 0, name)


@pytest.mark.parametrize("S", [1, 7])
def test_prefill_split_counts(S):
    prep = Prepared(chunk_workload(12, context_lens=[1500, 600], chunk_lens=[80, 33], T_max=80))
    check_prefill(prep, S, f"two requests, {S} splits")


def test_prefill_512_at_32k():
    """A 512-token chunk closing a 32K context: all 12,288 rows."""
    prep = Prepared(chunk_workload(13, context_lens=[32768], chunk_lens=[512], T_max=512))
    log(f"  prefill 512 @ 32K: {sda.splash_prefill_attn_workspace_bytes(1, 512, 24, 4, 256, 32768)} workspace bytes")
    check_prefill(prep, 0, "512-token chunk at 32K")


def test_prefill_of_16_is_the_verify_call():
    prep = Prepared(chunk_workload(14, context_lens=[3000, 500], chunk_lens=[16, 9], T_max=16))
    assert np.array_equal(run_prefill(prep), prep.run(num_splits=0).cpu().numpy())
