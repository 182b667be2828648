"""GPU parity for accepting a verified block: the HIP kernels through the C ABI
against the CPU oracle, bit-exact (accepted counts, next tokens, rolled-back
context lengths are integers), and against the generator's planted values.

Shapes: the verify workloads' request counts and draft lengths (one request
with a 16-token block; 16 requests with ragged blocks of 1..16) at a
151,936-token vocabulary, plus small vocabularies, ties, a vocabulary that ends
just past a chunk of the argmax kernel, the largest block (64) and empty
blocks.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

import oracle  # noqa: E402
import speculative_decode_attention_amd as sda  # noqa: E402
from speculative_decode_attention_amd import synth  # noqa: E402
from gpu_util import log, up  # noqa: E402


def run_gpu(case):
    B = case.B
    logits = up(case.logits)
    bt = up(case.block_tokens)
    dl = up(case.draft_lens)
    ctx = up(case.context_lens)
    acc = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    nxt = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    sda.splash_verify_accept(logits, bt, dl, ctx, acc, nxt)
    torch.cuda.synchronize()
    return acc.cpu().numpy(), nxt.cpu().numpy(), ctx.cpu().numpy()


def check(case, name):
    log(f"  accept {name}: B={case.B} T_max={case.T_max} V={case.V}")
    got = run_gpu(case)
    ref = oracle.load().verify_accept(case.logits, case.block_tokens, case.draft_lens, case.context_lens)
    for g, r, what in zip(got, ref, ("accepted", "next_token", "context_lens")):
        assert np.array_equal(g, r), f"{name}: {what} {g} != oracle {r}"
    acc = got[0]
    for b in range(case.B):                                   # and the construction
        d, a = int(case.draft_lens[b]), int(case.planted_accept[b])
        if d:
            assert acc[b] == a and got[1][b] == case.planted_tokens[b, a - 1], (name, b)


CASES = {
    "one_request_full_vocab": dict(seed=1, B=1, T_max=16, draft_lens=[16]),
    "sixteen_ragged_full_vocab": dict(seed=2, B=16, T_max=16),
    "ties_full_vocab": dict(seed=3, B=4, T_max=16, ties=True),
    "small_vocab": dict(seed=4, B=5, T_max=16, V=1000),
    "vocab_8": dict(seed=5, B=3, T_max=4, V=8),
    "vocab_past_a_chunk": dict(seed=6, B=4, T_max=16, V=8200),
    "edges": dict(seed=7, B=4, T_max=16, V=4096, draft_lens=[16, 16, 1, 0], accept_lens=[1, 16, 1, 0]),
    "block_of_64": dict(seed=8, B=3, T_max=64, V=2048, draft_lens=[64, 64, 33], accept_lens=[64, 40, 1]),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_accept_matches_oracle(name):
    kw = dict(CASES[name])
    seed = kw.pop("seed")
    check(synth.make_accept_case(seed, **kw), name)


def test_accept_chunk_boundary_and_signed_zero():
    """The maximum in the last 8 ids of a chunk, the first id of the next, and a
    row of zeros of both signs (id 0 wins)."""
    V = 3 * 8192
    case = synth.make_accept_case(9, B=3, T_max=2, V=V, draft_lens=[1, 1, 1], accept_lens=[1, 1, 1])
    lg = case.logits.copy()
    lg[0, 0, :] = 0x3F80                                      # 1.0 everywhere ...
    lg[0, 0, 8191] = 0x4000                                   # ... 2.0 at the last id of chunk 0
    lg[1, 0, :] = 0x3F80
    lg[1, 0, 8192] = 0x4000                                   # 2.0 at the first id of chunk 1
    lg[1, 0, 20000] = 0x4000                                  # and an equal value later
    lg[2, 0, :] = 0x8000                                      # -0.0 everywhere
    lg[2, 0, 9000] = 0x0000                                   # +0.0: an equal value
    ref = oracle.load().verify_accept(lg, case.block_tokens, case.draft_lens, case.context_lens)
    assert list(ref[1]) == [8191, 8192, 0]
    case.logits = lg
    got = run_gpu(case)
    assert list(got[1]) == [8191, 8192, 0], got
    assert np.array_equal(got[0], ref[0]) and np.array_equal(got[2], ref[2])


def test_accept_calls_reuse_the_workspace():
    """One uncleared workspace serves several calls in a row, the later ones
    smaller or with empty blocks."""
    cases = [synth.make_accept_case(10, B=8, T_max=16, V=20000),
             synth.make_accept_case(11, B=2, T_max=16, V=9000),
             synth.make_accept_case(12, B=8, T_max=16, V=20000, draft_lens=[0, 3, 16, 0, 1, 9, 2, 16]),
             synth.make_accept_case(13, B=8, T_max=16, V=20000)]
    ws = torch.full((sda.splash_verify_accept_workspace_bytes(8, 16, 20000),), 0x5A, dtype=torch.uint8, device="cuda")
    for case in cases:
        acc = torch.empty(case.B, dtype=torch.int32, device="cuda")
        nxt = torch.empty(case.B, dtype=torch.int32, device="cuda")
        ctx = up(case.context_lens)
        sda.splash_verify_accept(up(case.logits), up(case.block_tokens), up(case.draft_lens), ctx, acc, nxt,
                                 workspace=ws)
        torch.cuda.synchronize()
        ref = oracle.load().verify_accept(case.logits, case.block_tokens, case.draft_lens, case.context_lens)
        assert np.array_equal(acc.cpu().numpy(), ref[0]) and np.array_equal(nxt.cpu().numpy(), ref[1])
        assert np.array_equal(ctx.cpu().numpy(), ref[2])
