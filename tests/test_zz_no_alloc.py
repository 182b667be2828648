"""The entry point that allocates nothing (splash_verify_attn_noalloc), through
the C ABI: its output equals splash_verify_attn's bit for bit (same kernels,
same split count) on two calls in a row, the second with a smaller input, and
both meet the attention tolerance against the fp64 oracle; a call whose
partials exceed the scratch is refused before anything is launched (the
pointers of that call are never dereferenced)."""
import ctypes

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

import speculative_decode_attention_amd as sda  # noqa: E402
from speculative_decode_attention_amd import synth  # noqa: E402
from gpu_util import BF16_NAN, Prepared, assert_attn_ok, bf16_to_f64, log  # noqa: E402


def run_both(prep, S):
    wl = prep.wl
    a = torch.full(tuple(wl.q.shape), BF16_NAN, dtype=torch.int16, device="cuda")
    b = torch.full(tuple(wl.q.shape), BF16_NAN, dtype=torch.int16, device="cuda")
    sda.splash_verify_attn_noalloc(prep.q, a, *prep.g_pools, prep.bt, prep.ctx, prep.dl, wl.max_context_len,
                                   wl.sm_scale, num_splits=S)
    torch.cuda.synchronize()
    got = a.cpu().numpy()
    sda.splash_verify_attn(prep.q, b, *prep.g_pools, prep.bt, prep.ctx, prep.dl, wl.max_context_len,
                           wl.sm_scale, num_splits=S)
    torch.cuda.synchronize()
    return got, b.cpu().numpy()


def check(prep, S, where):
    wl = prep.wl
    got, want = run_both(prep, S)
    assert np.array_equal(got, want), f"{where}: differs from splash_verify_attn"
    rows = prep.valid_rows()
    g = bf16_to_f64(got[rows[:, 0], rows[:, 1], rows[:, 2]])
    assert_attn_ok(g, prep.oracle_rows(rows), where, mag=prep.oracle_rows(rows, abs_v=True),
                   floor=prep.p_floor(rows))
    for b in range(wl.B):
        assert np.all(got[b, int(wl.draft_lens[b]):].view(np.uint16) == BF16_NAN)


def test_two_calls_in_a_row_then_a_smaller_one():
    # first: one request at 32K context with the preset (64 splits, 12.7 MB of partials)
    big = Prepared(synth.make_workload("noalloc_big", 41, B=1, context_lens=[32768], T_max=16, Hq=24, Hkv=4,
                                       D=256, num_pages=32768 // 16 + 8))
    need = sda.splash_verify_attn_workspace_bytes(1, 16, 24, 256, 64)
    log(f"  32K call: {need} bytes of partials in a {sda.NOALLOC_SCRATCH_BYTES}-byte scratch")
    assert 0 < need <= sda.NOALLOC_SCRATCH_BYTES
    check(big, 0, "noalloc, 32K, preset splits")
    # second, smaller: ragged requests, 5 splits, reusing the scratch the first call filled
    small = Prepared(synth.make_workload("noalloc_small", 42, B=3, context_lens=[700, 130, 333], T_max=16,
                                         draft_lens=[16, 9, 4], Hq=24, Hkv=4, D=256, num_pages=96))
    check(small, 5, "noalloc, 3 ragged requests, 5 splits")
    check(small, 1, "noalloc, 3 ragged requests, 1 split (no scratch)")


def test_partials_past_the_scratch_are_refused():
    lib = sda.load_library()
    fake = 0x10000                                          # never dereferenced: refused first
    # 128 requests x 64 splits of 24 heads x 16 drafts x 256 dims: far past 32 MiB
    need = sda.splash_verify_attn_workspace_bytes(128, 16, 24, 256, 64)
    assert need > sda.NOALLOC_SCRATCH_BYTES
    rc = lib.splash_verify_attn_noalloc(fake, fake, fake, fake, fake, fake, fake, 2048, fake, fake, 128, 16, 24,
                                        4, 256, 16, 65536, 32768, ctypes.c_float(0.0625), 64, None)
    assert rc == sda.SPLASH_ERR_WORKSPACE_TOO_SMALL
