"""The C ABI without a GPU: the library loads, exports what the header declares,
and rejects bad arguments synchronously before any HIP call."""
import ctypes
import re
from pathlib import Path

import pytest

import speculative_decode_attention_amd as sda

ROOT = Path(__file__).resolve().parents[1]


@pytest.fixture(scope="module")
def lib():
    if not sda.LIB_PATH.exists():
        from speculative_decode_attention_amd import build
        build.build()
    return sda.load_library()


def header_functions():
    text = (ROOT / "include" / "splash_attn.h").read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(splash_\w+)\s*\(", text)))


def test_header_and_binding_agree():
    assert header_functions() == sorted(sda.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    for name in header_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for code in range(0, 6):
        assert sda.splash_status_string(code) not in ("", None)
    assert sda.splash_status_string(99) == "unknown status"


def test_workspace_and_split_arithmetic(lib):
    # tiled fp16 partials for 16 drafts of every query head per split, then
    # 256-aligned fp32 log-sum-exps, then an int32 exponent per (request, head,
    # split) block (T_max does not change the size)
    assert sda.splash_verify_attn_workspace_bytes(1, 16, 24, 256, 1) == 0
    rows = 1 * 16 * 24 * 64
    want = -(-rows * 256 * 2 // 256) * 256 + -(-rows * 4 // 256) * 256 + -(-24 * 64 * 4 // 256) * 256
    assert sda.splash_verify_attn_workspace_bytes(1, 3, 24, 256, 64) == want
    assert sda.splash_verify_attn_workspace_bytes(1, 16, 24, 256, 64) == want
    # pages per split are whole steps of 4 pages
    assert sda.splash_verify_attn_split_pages(32768, 16, 64) == 32
    assert sda.splash_verify_attn_split_pages(256, 16, 3) == 8
    assert sda.splash_verify_attn_split_pages(17, 16, 8) == 4
    assert sda.effective_splits(32768, 16, 64) == 64
    assert sda.effective_splits(17, 16, 8) == 1
    assert sda.effective_splits(4096, 16, 7) == 7
    with pytest.raises(sda.SplashError):
        sda.splash_verify_attn_split_pages(100, 16, 0)


FAKE = 0x10000        # 16-byte aligned, never dereferenced: every case fails validation first


def _verify(lib, **over):
    args = dict(q=FAKE, out=FAKE, k_pool=FAKE, v_pool=FAKE, k_scale=FAKE, v_scale=FAKE, bt=FAKE,
                maxp=2048, ctx=FAKE, dl=FAKE, B=1, T=16, Hq=24, Hkv=4, D=256, P=16, num_pages=65536,
                max_ctx=32768, sm=0.0625, S=0, ws=None, ws_bytes=0)
    args.update(over)
    a = args
    return lib.splash_verify_attn(a["q"], a["out"], a["k_pool"], a["v_pool"], a["k_scale"],
                                  a["v_scale"], a["bt"], a["maxp"], a["ctx"], a["dl"], a["B"], a["T"],
                                  a["Hq"], a["Hkv"], a["D"], a["P"], a["num_pages"], a["max_ctx"],
                                  ctypes.c_float(a["sm"]), a["S"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("over,status", [
    (dict(q=None), sda.SPLASH_ERR_INVALID_ARGUMENT),
    (dict(out=None), sda.SPLASH_ERR_INVALID_ARGUMENT),
    (dict(k_pool=None), sda.SPLASH_ERR_INVALID_ARGUMENT),
    (dict(bt=None), sda.SPLASH_ERR_INVALID_ARGUMENT),
    (dict(ctx=None), sda.SPLASH_ERR_INVALID_ARGUMENT),
    (dict(Hq=25), sda.SPLASH_ERR_INVALID_ARGUMENT),            # Hq % Hkv != 0
    (dict(B=-1), sda.SPLASH_ERR_INVALID_ARGUMENT),
    (dict(maxp=100), sda.SPLASH_ERR_INVALID_ARGUMENT),         # block table too short
    (dict(q=FAKE + 4), sda.SPLASH_ERR_INVALID_ARGUMENT),       # misaligned
    (dict(sm=float("nan")), sda.SPLASH_ERR_INVALID_ARGUMENT),
    (dict(S=-2), sda.SPLASH_ERR_INVALID_ARGUMENT),
    (dict(T=17), sda.SPLASH_ERR_UNSUPPORTED),                  # more than 16 drafts
    (dict(P=32, maxp=1024), sda.SPLASH_ERR_UNSUPPORTED),
    (dict(D=192), sda.SPLASH_ERR_UNSUPPORTED),
    (dict(Hq=32, Hkv=4), sda.SPLASH_ERR_UNSUPPORTED),          # group of 8 at D = 256
    (dict(S=64, ws=None), sda.SPLASH_ERR_INVALID_ARGUMENT),    # several splits need a workspace
    (dict(S=64, ws=FAKE, ws_bytes=1024), sda.SPLASH_ERR_WORKSPACE_TOO_SMALL),
])
def test_verify_rejects_bad_arguments(lib, over, status):
    assert _verify(lib, **over) == status


def test_verify_empty_batch_is_a_no_op(lib):
    assert _verify(lib, B=0) == sda.SPLASH_OK
    assert _verify(lib, T=0) == sda.SPLASH_OK
    assert _verify(lib, max_ctx=0) == sda.SPLASH_OK


def _append(lib, **over):
    a = dict(k=FAKE, v=FAKE, src=0, k_pool=FAKE, v_pool=FAKE, ks=FAKE, vs=FAKE, bt=FAKE, maxp=4,
             ctx=FAKE, dl=FAKE, B=1, T=16, Hkv=4, D=256, P=16, num_pages=16)
    a.update(over)
    return lib.splash_kv_append_int8(a["k"], a["v"], a["src"], a["k_pool"], a["v_pool"], a["ks"],
                                     a["vs"], a["bt"], a["maxp"], a["ctx"], a["dl"], a["B"], a["T"],
                                     a["Hkv"], a["D"], a["P"], a["num_pages"], None)


@pytest.mark.parametrize("over,status", [
    (dict(k=None), sda.SPLASH_ERR_INVALID_ARGUMENT),
    (dict(vs=None), sda.SPLASH_ERR_INVALID_ARGUMENT),
    (dict(src=2), sda.SPLASH_ERR_INVALID_ARGUMENT),
    (dict(Hkv=0), sda.SPLASH_ERR_INVALID_ARGUMENT),
    (dict(num_pages=0), sda.SPLASH_ERR_INVALID_ARGUMENT),
    (dict(k=FAKE + 4), sda.SPLASH_ERR_INVALID_ARGUMENT),       # fp32 rows need 16-byte alignment
    (dict(D=96), sda.SPLASH_ERR_UNSUPPORTED),
    (dict(P=8), sda.SPLASH_ERR_UNSUPPORTED),
])
def test_append_rejects_bad_arguments(lib, over, status):
    assert _append(lib, **over) == status


def test_append_empty_is_a_no_op(lib):
    assert _append(lib, B=0) == sda.SPLASH_OK
    assert _append(lib, T=0) == sda.SPLASH_OK


def test_merge_rejects_bad_arguments(lib):
    # (part_o, part_lse, out, draft_lens, B, T_max, Hq, D, num_splits, stream)
    m = lib.splash_verify_attn_splitk_merge
    assert m(None, FAKE, FAKE, FAKE, 1, 16, 24, 256, 4, None) == sda.SPLASH_ERR_INVALID_ARGUMENT
    assert m(FAKE, FAKE, FAKE, None, 1, 16, 24, 256, 4, None) == sda.SPLASH_ERR_INVALID_ARGUMENT
    assert m(FAKE, FAKE, FAKE, FAKE, 1, 16, 24, 256, 0, None) == sda.SPLASH_ERR_INVALID_ARGUMENT
    assert m(FAKE + 8, FAKE, FAKE, FAKE, 1, 16, 24, 256, 4, None) == sda.SPLASH_ERR_INVALID_ARGUMENT
    assert m(FAKE, FAKE, FAKE + 4, FAKE, 1, 16, 24, 256, 4, None) == sda.SPLASH_ERR_INVALID_ARGUMENT
    assert m(FAKE, FAKE, FAKE, FAKE, 1, 16, 24, 96, 4, None) == sda.SPLASH_ERR_UNSUPPORTED
    assert m(FAKE, FAKE, FAKE, FAKE, 0, 16, 24, 256, 4, None) == sda.SPLASH_OK
    assert m(FAKE, FAKE, FAKE, FAKE, 1, 0, 24, 256, 4, None) == sda.SPLASH_OK


def test_verify_refuses_merge_grids_it_cannot_launch(lib):
    """More than 65535 requests with several splits is refused before anything is
    launched (the pointers are never dereferenced, so nothing ran)."""
    assert _verify(lib, B=65536, S=64, ws=FAKE, ws_bytes=1 << 40) == sda.SPLASH_ERR_UNSUPPORTED
    assert _verify(lib, B=65536, S=64, ws=None) == sda.SPLASH_ERR_UNSUPPORTED


def test_partition_rejects_bad_arguments(lib):
    p = lib.splash_verify_attn_partition
    base = [FAKE] * 6 + [2048, FAKE, FAKE, 1, 16, 24, 4, 256, 16, 65536, 32768,
                         ctypes.c_float(0.0625), 8, FAKE, FAKE, None]
    args = list(base); args[0] = None
    assert p(*args) == sda.SPLASH_ERR_INVALID_ARGUMENT
    args = list(base); args[18] = 0                              # no preset here: splits >= 1
    assert p(*args) == sda.SPLASH_ERR_INVALID_ARGUMENT
    args = list(base); args[19] = FAKE + 8                       # misaligned partials
    assert p(*args) == sda.SPLASH_ERR_INVALID_ARGUMENT


def test_masked_verify_needs_its_masks(lib):
    args = [FAKE] * 7 + [2048, FAKE, FAKE, None, 1, 16, 24, 4, 256, 16, 65536, 32768,
                         ctypes.c_float(0.0625), 0, FAKE, 1 << 30, None]
    assert lib.splash_verify_attn_masked(*args) == sda.SPLASH_ERR_INVALID_ARGUMENT   # no masks
    args[10] = FAKE
    args[0] = None
    assert lib.splash_verify_attn_masked(*args) == sda.SPLASH_ERR_INVALID_ARGUMENT


def test_accept_workspace_arithmetic(lib):
    ws = lib.splash_verify_accept_workspace_bytes
    # 19 chunks of 8192 logits per row, a (value, id) pair each
    assert ws(16, 16, 151936) == 16 * 16 * 19 * 8
    assert ws(1, 16, 8192) == 16 * 8 and ws(1, 16, 8200) == 16 * 2 * 8
    assert ws(100, 1, 8) == 100 * 8
    assert ws(0, 16, 64) == 0 and ws(2, 3, 4) == 0             # V below 8: no valid size


def test_accept_rejects_bad_arguments(lib):
    a = lib.splash_verify_accept
    ok = [FAKE] * 6 + [4, 16, 151936, FAKE, 1 << 20, None]
    assert a(*ok[:5], None, *ok[6:]) == sda.SPLASH_ERR_INVALID_ARGUMENT       # next_token missing
    args = list(ok); args[8] = 151937                                          # V not a multiple of 8
    assert a(*args) == sda.SPLASH_ERR_INVALID_ARGUMENT
    args = list(ok); args[0] = FAKE + 2                                        # misaligned logits
    assert a(*args) == sda.SPLASH_ERR_INVALID_ARGUMENT
    args = list(ok); args[7] = 65                                              # one wave holds a block
    assert a(*args) == sda.SPLASH_ERR_UNSUPPORTED
    args = list(ok); args[10] = 4 * 16 * 19 * 8 - 1                           # workspace one byte short
    assert a(*args) == sda.SPLASH_ERR_WORKSPACE_TOO_SMALL
    args = list(ok); args[9] = None
    assert a(*args) == sda.SPLASH_ERR_INVALID_ARGUMENT
    args = list(ok); args[6] = 0                                               # empty batch: nothing launched
    assert a(*args) == sda.SPLASH_OK


def test_binding_fails_loudly_without_the_library(tmp_path):
    with pytest.raises(RuntimeError, match="not built"):
        sda.load_library(tmp_path / "missing.so")


def _append_verify(lib, **over):
    a = dict(k=FAKE, v=FAKE, src=0, q=FAKE, out=FAKE, k_pool=FAKE, v_pool=FAKE, ks=FAKE, vs=FAKE, bt=FAKE,
             maxp=2048, ctx=FAKE, dl=FAKE, B=1, T=16, Hq=24, Hkv=4, D=256, P=16, num_pages=65536,
             max_ctx=32768, sm=0.0625, S=0, ws=None, ws_bytes=0)
    a.update(over)
    return lib.splash_verify_attn_append(a["k"], a["v"], a["src"], a["q"], a["out"], a["k_pool"], a["v_pool"],
                                         a["ks"], a["vs"], a["bt"], a["maxp"], a["ctx"], a["dl"], a["B"], a["T"],
                                         a["Hq"], a["Hkv"], a["D"], a["P"], a["num_pages"], a["max_ctx"],
                                         ctypes.c_float(a["sm"]), a["S"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("over,status", [
    (dict(k=None), sda.SPLASH_ERR_INVALID_ARGUMENT),            # no source rows
    (dict(v=None), sda.SPLASH_ERR_INVALID_ARGUMENT),
    (dict(src=2), sda.SPLASH_ERR_INVALID_ARGUMENT),             # unknown source dtype
    (dict(k=FAKE + 4), sda.SPLASH_ERR_INVALID_ARGUMENT),        # fp32 rows read 16 bytes a lane at D = 256
    (dict(src=1, v=FAKE + 2), sda.SPLASH_ERR_INVALID_ARGUMENT),  # bf16 rows read 8 bytes a lane
    (dict(q=None), sda.SPLASH_ERR_INVALID_ARGUMENT),            # then everything the verify call checks
    (dict(maxp=100), sda.SPLASH_ERR_INVALID_ARGUMENT),
    (dict(T=17), sda.SPLASH_ERR_UNSUPPORTED),
    (dict(D=192), sda.SPLASH_ERR_UNSUPPORTED),
    (dict(S=64, ws=None), sda.SPLASH_ERR_INVALID_ARGUMENT),
    (dict(S=64, ws=FAKE, ws_bytes=1024), sda.SPLASH_ERR_WORKSPACE_TOO_SMALL),
])
def test_append_verify_rejects_bad_arguments(lib, over, status):
    assert _append_verify(lib, **over) == status


def test_append_verify_empty_is_a_no_op(lib):
    assert _append_verify(lib, B=0) == sda.SPLASH_OK
    assert _append_verify(lib, T=0) == sda.SPLASH_OK
    assert _append_verify(lib, max_ctx=0) == sda.SPLASH_OK
