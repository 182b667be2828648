"""Block-verify decode attention over an int8 paged KV cache, for MI355X (gfx950).

A thin ctypes binding over the C ABI in ``include/splash_attn.h``
(``libsplash_attn.so``, built from ``csrc/`` by ``build.py``).  Every function
has the name of the C entry point it calls and only marshals arguments: it
checks dtypes, devices and shapes of the torch tensors, passes their device
pointers and the current HIP stream, and raises ``SplashError`` on a non-zero
status.  All computation happens in the library's kernels; there is no other
code path, and a missing library is an error.
"""
from __future__ import annotations

import ctypes
from pathlib import Path

PKG = Path(__file__).resolve().parent
LIB_PATH = PKG / "libsplash_attn.so"

SPLASH_OK = 0
SPLASH_ERR_INVALID_ARGUMENT = 1
SPLASH_ERR_UNSUPPORTED = 2
SPLASH_ERR_WORKSPACE_TOO_SMALL = 3
SPLASH_ERR_LAUNCH = 4
SPLASH_ERR_DEVICE = 5
SPLASH_SRC_F32 = 0
SPLASH_SRC_BF16 = 1
PAGE_SIZE = 16

# every symbol the header declares
EXPORTED = (
    "splash_kv_append_int8",
    "splash_verify_attn_default_splits",
    "splash_verify_attn_workspace_bytes",
    "splash_verify_attn",
    "splash_verify_attn_append",
    "splash_verify_attn_noalloc",
    "splash_verify_attn_masked",
    "splash_verify_attn_window",
    "splash_verify_attn_window_tokens",
    "splash_prefill_attn",
    "splash_prefill_attn_workspace_bytes",
    "splash_verify_attn_partition",
    "splash_verify_attn_split_pages",
    "splash_verify_attn_splitk_merge",
    "splash_verify_accept_workspace_bytes",
    "splash_verify_accept",
    "splash_status_string",
)


class SplashError(RuntimeError):
    """A non-zero status from the library."""

    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {splash_status_string(status)} (status {status})")


_P, _I, _F, _Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
_lib_handle = None


def load_library(path: Path | None = None):
    """dlopen the library (no GPU is touched) and declare its signatures."""
    global _lib_handle
    if path is None and _lib_handle is not None:
        return _lib_handle
    p = Path(path) if path is not None else LIB_PATH
    if not p.exists():
        raise RuntimeError(f"{p} is not built: run `python -m speculative_decode_attention_amd.build`")
    lib = ctypes.CDLL(str(p))
    lib.splash_kv_append_int8.argtypes = [_P, _P, _I, _P, _P, _P, _P, _P, _I, _P, _P,
                                          _I, _I, _I, _I, _I, _I, _P]
    lib.splash_verify_attn_default_splits.argtypes = [_I, _I, _I, _I, _I]
    lib.splash_verify_attn_workspace_bytes.argtypes = [_I, _I, _I, _I, _I]
    lib.splash_verify_attn_workspace_bytes.restype = _Z
    lib.splash_verify_attn.argtypes = [_P, _P, _P, _P, _P, _P, _P, _I, _P, _P,
                                       _I, _I, _I, _I, _I, _I, _I, _I, _F, _I, _P, _Z, _P]
    lib.splash_verify_attn_append.argtypes = [_P, _P, _I, _P, _P, _P, _P, _P, _P, _P, _I, _P, _P,
                                              _I, _I, _I, _I, _I, _I, _I, _I, _F, _I, _P, _Z, _P]
    lib.splash_verify_attn_noalloc.argtypes = [_P, _P, _P, _P, _P, _P, _P, _I, _P, _P,
                                               _I, _I, _I, _I, _I, _I, _I, _I, _F, _I, _P]
    lib.splash_verify_attn_masked.argtypes = [_P, _P, _P, _P, _P, _P, _P, _I, _P, _P, _P,
                                              _I, _I, _I, _I, _I, _I, _I, _I, _F, _I, _P, _Z, _P]
    lib.splash_verify_attn_window.argtypes = [_P, _P, _P, _P, _P, _P, _P, _I, _P, _P, _I,
                                              _I, _I, _I, _I, _I, _I, _I, _I, _F, _I, _P, _Z, _P]
    lib.splash_verify_attn_window_tokens.argtypes = [_I, _I, _I, _I]
    lib.splash_prefill_attn.argtypes = [_P, _P, _P, _P, _P, _P, _P, _I, _P, _P,
                                        _I, _I, _I, _I, _I, _I, _I, _I, _F, _I, _P, _Z, _P]
    lib.splash_prefill_attn_workspace_bytes.argtypes = [_I, _I, _I, _I, _I, _I, _I, _I]
    lib.splash_prefill_attn_workspace_bytes.restype = _Z
    lib.splash_verify_attn_partition.argtypes = [_P, _P, _P, _P, _P, _P, _I, _P, _P,
                                                 _I, _I, _I, _I, _I, _I, _I, _I, _F, _I, _P, _P, _P]
    lib.splash_verify_attn_split_pages.argtypes = [_I, _I, _I]
    lib.splash_verify_attn_splitk_merge.argtypes = [_P, _P, _P, _P, _I, _I, _I, _I, _I, _P]
    lib.splash_verify_accept_workspace_bytes.argtypes = [_I, _I, _I]
    lib.splash_verify_accept_workspace_bytes.restype = _Z
    lib.splash_verify_accept.argtypes = [_P, _P, _P, _P, _P, _P, _I, _I, _I, _P, _Z, _P]
    lib.splash_status_string.argtypes = [_I]
    lib.splash_status_string.restype = ctypes.c_char_p
    for name in EXPORTED:
        if name not in ("splash_verify_attn_workspace_bytes", "splash_verify_accept_workspace_bytes",
                        "splash_prefill_attn_workspace_bytes", "splash_status_string"):
            getattr(lib, name).restype = _I
    if path is None:
        _lib_handle = lib
    return lib


def _lib():
    return load_library()


def splash_status_string(status: int) -> str:
    return _lib().splash_status_string(int(status)).decode()


# ---------------------------------------------------------------------------
# argument marshalling
# ---------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _dev(t, name, dtypes, shape=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must live on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t.data_ptr()


def _stream(stream):
    torch = _torch()
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _check(rc, where):
    if rc != SPLASH_OK:
        raise SplashError(rc, where)


def _pool_dims(k_pool, v_pool, k_scale, v_scale):
    torch = _torch()
    if k_pool.dim() != 4:
        raise ValueError("k_pool must be [num_pages][Hkv][P][D]")
    num_pages, Hkv, P, D = k_pool.shape
    _dev(k_pool, "k_pool", (torch.int8,))
    _dev(v_pool, "v_pool", (torch.int8,), (num_pages, Hkv, P // 8, D, 8))
    _dev(k_scale, "k_scale", (torch.float16, torch.int16), (num_pages, Hkv, P))
    _dev(v_scale, "v_scale", (torch.float16, torch.int16), (num_pages, Hkv, P))
    return num_pages, Hkv, P, D


def _lens(block_table, context_lens, draft_lens, B):
    torch = _torch()
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [B][max_pages_per_seq]")
    _dev(block_table, "block_table", (torch.int32,))
    _dev(context_lens, "context_lens", (torch.int32,), (B,))
    _dev(draft_lens, "draft_lens", (torch.int32,), (B,))
    return block_table.shape[1]


# ---------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------
def splash_kv_append_int8(k_new, v_new, k_pool, v_pool, k_scale, v_scale, block_table,
                          context_lens, draft_lens, stream=None):
    """Quantise k_new/v_new [B][T_max][Hkv][D] (fp32 or bf16) into the int8 pools."""
    torch = _torch()
    if k_new.dim() != 4:
        raise ValueError("k_new must be [B][T_max][Hkv][D]")
    B, T_max, Hkv_src, D_src = k_new.shape
    _dev(k_new, "k_new", (torch.float32, torch.bfloat16))
    _dev(v_new, "v_new", (k_new.dtype,), tuple(k_new.shape))
    num_pages, Hkv, P, D = _pool_dims(k_pool, v_pool, k_scale, v_scale)
    if (Hkv_src, D_src) != (Hkv, D):
        raise ValueError("k_new heads / head dim do not match the pools")
    maxp = _lens(block_table, context_lens, draft_lens, B)
    src = SPLASH_SRC_F32 if k_new.dtype == torch.float32 else SPLASH_SRC_BF16
    rc = _lib().splash_kv_append_int8(
        k_new.data_ptr(), v_new.data_ptr(), src, k_pool.data_ptr(), v_pool.data_ptr(),
        k_scale.data_ptr(), v_scale.data_ptr(), block_table.data_ptr(), maxp,
        context_lens.data_ptr(), draft_lens.data_ptr(), B, T_max, Hkv, D, P, num_pages,
        _stream(stream))
    _check(rc, "splash_kv_append_int8")


def splash_verify_attn_default_splits(B, Hkv, max_context_len, P=PAGE_SIZE, D=256):
    rc = _lib().splash_verify_attn_default_splits(int(B), int(Hkv), int(max_context_len), int(P), int(D))
    if rc < 0:
        _check(-rc, "splash_verify_attn_default_splits")
    return rc


def splash_verify_attn_split_pages(max_context_len, P, num_splits):
    rc = _lib().splash_verify_attn_split_pages(int(max_context_len), int(P), int(num_splits))
    if rc < 0:
        _check(-rc, "splash_verify_attn_split_pages")
    return rc


def splash_verify_attn_workspace_bytes(B, T_max, Hq, D, num_splits):
    return int(_lib().splash_verify_attn_workspace_bytes(int(B), int(T_max), int(Hq), int(D),
                                                         int(num_splits)))


def effective_splits(max_context_len, P, num_splits):
    """Number of splits that hold at least one page for a requested split count."""
    if max_context_len <= 0:
        return 1
    L = splash_verify_attn_split_pages(max_context_len, P, num_splits)
    n_pages = -(-max_context_len // P)
    return -(-n_pages // L)


def splash_verify_attn(q, out, k_pool, v_pool, k_scale, v_scale, block_table, context_lens,
                       draft_lens, max_context_len, sm_scale, num_splits=0, workspace=None,
                       stream=None):
    """Block-verify attention; writes out[b][t][h][:] for t < draft_lens[b].

    workspace: a byte tensor of at least splash_verify_attn_workspace_bytes(...)
    for the splits that run, or None to let this binding allocate one with torch.
    """
    return _verify(q, out, k_pool, v_pool, k_scale, v_scale, block_table, context_lens, draft_lens,
                   max_context_len, sm_scale, num_splits, workspace, stream, None)


def splash_verify_attn_append(k_new, v_new, q, out, k_pool, v_pool, k_scale, v_scale, block_table, context_lens,
                              draft_lens, max_context_len, sm_scale, num_splits=0, workspace=None, stream=None):
    """splash_kv_append_int8 and splash_verify_attn in one call: the drafted block's
    K/V rows come from k_new / v_new ([B][T_max][Hkv][D], fp32 or bf16), are
    quantised in the kernel as the append quantises them, attended, and stored
    into the pools' block slots (the pools end byte-identical to the append's)."""
    torch = _torch()
    if q.dim() != 4:
        raise ValueError("q must be [B][T_max][Hq][D]")
    B, T_max, Hq, Dq = q.shape
    _dev(q, "q", (torch.bfloat16, torch.int16))
    _dev(out, "out", (torch.bfloat16, torch.int16), tuple(q.shape))
    num_pages, Hkv, P, D = _pool_dims(k_pool, v_pool, k_scale, v_scale)
    if Dq != D:
        raise ValueError("q head dim does not match the pools")
    _dev(k_new, "k_new", (torch.float32, torch.bfloat16), (B, T_max, Hkv, D))
    _dev(v_new, "v_new", (k_new.dtype,), (B, T_max, Hkv, D))
    maxp = _lens(block_table, context_lens, draft_lens, B)
    S_req = num_splits if num_splits > 0 else (
        splash_verify_attn_default_splits(B, Hkv, max_context_len, P, D) if B and max_context_len else 1)
    S = effective_splits(max_context_len, P, S_req) if max_context_len else 1
    need = splash_verify_attn_workspace_bytes(B, T_max, Hq, D, S)
    ws_ptr, ws_bytes = None, 0
    if need:
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        _dev(workspace, "workspace", (torch.uint8, torch.int8, torch.float32))
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    src = SPLASH_SRC_F32 if k_new.dtype == torch.float32 else SPLASH_SRC_BF16
    rc = _lib().splash_verify_attn_append(
        k_new.data_ptr(), v_new.data_ptr(), src, q.data_ptr(), out.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(),
        k_scale.data_ptr(), v_scale.data_ptr(), block_table.data_ptr(), maxp, context_lens.data_ptr(),
        draft_lens.data_ptr(), B, T_max, Hq, Hkv, D, P, num_pages, int(max_context_len), float(sm_scale),
        int(S_req), ws_ptr, ws_bytes, _stream(stream))
    _check(rc, "splash_verify_attn_append")
    return out


NOALLOC_SCRATCH_BYTES = 32 << 20                    # SPLASH_NOALLOC_SCRATCH_BYTES


def splash_verify_attn_noalloc(q, out, k_pool, v_pool, k_scale, v_scale, block_table, context_lens, draft_lens,
                               max_context_len, sm_scale, num_splits=0, stream=None):
    """splash_verify_attn with the split partials in the library's own device
    scratch (no workspace, nothing allocated); calls overlapping on one GPU race."""
    torch = _torch()
    if q.dim() != 4:
        raise ValueError("q must be [B][T_max][Hq][D]")
    B, T_max, Hq, Dq = q.shape
    _dev(q, "q", (torch.bfloat16, torch.int16))
    _dev(out, "out", (torch.bfloat16, torch.int16), tuple(q.shape))
    num_pages, Hkv, P, D = _pool_dims(k_pool, v_pool, k_scale, v_scale)
    if Dq != D:
        raise ValueError("q head dim does not match the pools")
    maxp = _lens(block_table, context_lens, draft_lens, B)
    rc = _lib().splash_verify_attn_noalloc(
        q.data_ptr(), out.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(), k_scale.data_ptr(),
        v_scale.data_ptr(), block_table.data_ptr(), maxp, context_lens.data_ptr(), draft_lens.data_ptr(),
        B, T_max, Hq, Hkv, D, P, num_pages, int(max_context_len), float(sm_scale), int(num_splits),
        _stream(stream))
    _check(rc, "splash_verify_attn_noalloc")
    return out


def splash_verify_attn_masked(q, out, k_pool, v_pool, k_scale, v_scale, block_table, context_lens,
                              draft_lens, block_masks, max_context_len, sm_scale, num_splits=0,
                              workspace=None, stream=None):
    """splash_verify_attn with a tree-shaped block mask: block_masks int32/uint32
    [B][T_max], bit u of row t lets draft t see draft u."""
    return _verify(q, out, k_pool, v_pool, k_scale, v_scale, block_table, context_lens, draft_lens,
                   max_context_len, sm_scale, num_splits, workspace, stream, block_masks)


def splash_verify_attn_window_tokens(max_context_len, T_max, window, P=PAGE_SIZE):
    n = int(_lib().splash_verify_attn_window_tokens(int(max_context_len), int(T_max), int(window), int(P)))
    if n < 0:
        raise SplashError(-n, "splash_verify_attn_window_tokens")
    return n


def splash_verify_attn_window(q, out, k_pool, v_pool, k_scale, v_scale, block_table, context_lens,
                              draft_lens, window, max_context_len, sm_scale, num_splits=0,
                              workspace=None, stream=None):
    """splash_verify_attn where each draft sees only the last `window` keys up to itself."""
    return _verify(q, out, k_pool, v_pool, k_scale, v_scale, block_table, context_lens, draft_lens,
                   max_context_len, sm_scale, num_splits, workspace, stream, None, int(window))


def _verify(q, out, k_pool, v_pool, k_scale, v_scale, block_table, context_lens, draft_lens,
            max_context_len, sm_scale, num_splits, workspace, stream, block_masks, window=0):
    torch = _torch()
    if q.dim() != 4:
        raise ValueError("q must be [B][T_max][Hq][D]")
    B, T_max, Hq, Dq = q.shape
    _dev(q, "q", (torch.bfloat16, torch.int16))
    _dev(out, "out", (torch.bfloat16, torch.int16), tuple(q.shape))
    num_pages, Hkv, P, D = _pool_dims(k_pool, v_pool, k_scale, v_scale)
    if Dq != D:
        raise ValueError("q head dim does not match the pools")
    maxp = _lens(block_table, context_lens, draft_lens, B)
    span = (splash_verify_attn_window_tokens(max_context_len, T_max, window, P)
            if window and max_context_len else max_context_len)
    S_req = num_splits if num_splits > 0 else (
        splash_verify_attn_default_splits(B, Hkv, span, P, D) if B and span else 1)
    S = effective_splits(span, P, S_req) if span else 1
    need = splash_verify_attn_workspace_bytes(B, T_max, Hq, D, S)
    ws_ptr, ws_bytes = None, 0
    if need:
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        _dev(workspace, "workspace", (torch.uint8, torch.int8, torch.float32))
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    if window:
        rc = _lib().splash_verify_attn_window(
            q.data_ptr(), out.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(), k_scale.data_ptr(),
            v_scale.data_ptr(), block_table.data_ptr(), maxp, context_lens.data_ptr(),
            draft_lens.data_ptr(), int(window), B, T_max, Hq, Hkv, D, P, num_pages, int(max_context_len),
            float(sm_scale), int(S_req), ws_ptr, ws_bytes, _stream(stream))
        _check(rc, "splash_verify_attn_window")
    elif block_masks is None:
        rc = _lib().splash_verify_attn(
            q.data_ptr(), out.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(), k_scale.data_ptr(),
            v_scale.data_ptr(), block_table.data_ptr(), maxp, context_lens.data_ptr(),
            draft_lens.data_ptr(), B, T_max, Hq, Hkv, D, P, num_pages, int(max_context_len),
            float(sm_scale), int(S_req), ws_ptr, ws_bytes, _stream(stream))
        _check(rc, "splash_verify_attn")
    else:
        _dev(block_masks, "block_masks", (torch.int32,), (B, T_max))
        rc = _lib().splash_verify_attn_masked(
            q.data_ptr(), out.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(), k_scale.data_ptr(),
            v_scale.data_ptr(), block_table.data_ptr(), maxp, context_lens.data_ptr(),
            draft_lens.data_ptr(), block_masks.data_ptr(), B, T_max, Hq, Hkv, D, P, num_pages,
            int(max_context_len), float(sm_scale), int(S_req), ws_ptr, ws_bytes, _stream(stream))
        _check(rc, "splash_verify_attn_masked")
    return out


def partial_shapes(B, Hq, T_max, D, num_splits):
    """Shapes of the exported split partials: part_o fp32 [B][Hq][T_max][S][D] and
    part_lse fp32 [B][Hq][T_max][S]."""
    return (B, Hq, T_max, num_splits, D), (B, Hq, T_max, num_splits)


def splash_verify_attn_partition(q, k_pool, v_pool, k_scale, v_scale, block_table, context_lens,
                                 draft_lens, max_context_len, sm_scale, num_splits, part_o,
                                 part_lse, stream=None):
    """Normalised partial rows and log-sum-exps per context split into part_o and
    part_lse (fp32, shapes from partial_shapes)."""
    torch = _torch()
    B, T_max, Hq, Dq = q.shape
    _dev(q, "q", (torch.bfloat16, torch.int16))
    num_pages, Hkv, P, D = _pool_dims(k_pool, v_pool, k_scale, v_scale)
    maxp = _lens(block_table, context_lens, draft_lens, B)
    S = int(num_splits)
    po_shape, pl_shape = partial_shapes(B, Hq, T_max, D, S)
    _dev(part_o, "part_o", (torch.float32,), po_shape)
    _dev(part_lse, "part_lse", (torch.float32,), pl_shape)
    rc = _lib().splash_verify_attn_partition(
        q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(), k_scale.data_ptr(), v_scale.data_ptr(),
        block_table.data_ptr(), maxp, context_lens.data_ptr(), draft_lens.data_ptr(), B, T_max,
        Hq, Hkv, D, P, num_pages, int(max_context_len), float(sm_scale), S, part_o.data_ptr(),
        part_lse.data_ptr(), _stream(stream))
    _check(rc, "splash_verify_attn_partition")


def splash_verify_attn_splitk_merge(part_o, part_lse, out, draft_lens, stream=None):
    """Merge S splits (fp32 [B][Hq][T_max][S][D] rows and [B][Hq][T_max][S]
    log-sum-exps) -> out [B][T_max][Hq][D] bf16."""
    torch = _torch()
    B, T_max, Hq, D = out.shape
    _dev(out, "out", (torch.bfloat16, torch.int16))
    if part_lse.dim() != 4:
        raise ValueError("part_lse must be [B][Hq][T_max][S]")
    S = int(part_lse.shape[3])
    po_shape, pl_shape = partial_shapes(B, Hq, T_max, D, S)
    _dev(part_o, "part_o", (torch.float32,), po_shape)
    _dev(part_lse, "part_lse", (torch.float32,), pl_shape)
    _dev(draft_lens, "draft_lens", (torch.int32,), (B,))
    rc = _lib().splash_verify_attn_splitk_merge(part_o.data_ptr(), part_lse.data_ptr(),
                                                out.data_ptr(), draft_lens.data_ptr(), B, T_max,
                                                Hq, D, S, _stream(stream))
    _check(rc, "splash_verify_attn_splitk_merge")
    return out


def splash_verify_accept_workspace_bytes(B, T_max, V):
    return int(_lib().splash_verify_accept_workspace_bytes(int(B), int(T_max), int(V)))


def splash_verify_accept(logits, block_tokens, draft_lens, context_lens, accepted, next_token,
                         workspace=None, stream=None):
    """Greedy acceptance of a verified block; context_lens is updated in place.
    logits bf16 [B][T_max][V]; block_tokens int32 [B][T_max]; draft_lens,
    context_lens, accepted, next_token int32 [B].  Returns (accepted, next_token)."""
    torch = _torch()
    if logits.dim() != 3:
        raise ValueError("logits must be [B][T_max][V]")
    B, T_max, V = (int(x) for x in logits.shape)
    _dev(logits, "logits", (torch.bfloat16, torch.int16))
    _dev(block_tokens, "block_tokens", (torch.int32,), (B, T_max))
    for name, t in (("draft_lens", draft_lens), ("context_lens", context_lens), ("accepted", accepted),
                    ("next_token", next_token)):
        _dev(t, name, (torch.int32,), (B,))
    need = splash_verify_accept_workspace_bytes(B, T_max, V)
    if workspace is None:                                     # no need to clear it
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=logits.device)
    _dev(workspace, "workspace", (torch.uint8,))
    rc = _lib().splash_verify_accept(logits.data_ptr(), block_tokens.data_ptr(), draft_lens.data_ptr(),
                                     context_lens.data_ptr(), accepted.data_ptr(), next_token.data_ptr(),
                                     B, T_max, V, workspace.data_ptr(), workspace.numel(), _stream(stream))
    _check(rc, "splash_verify_accept")
    return accepted, next_token


def splash_prefill_attn_workspace_bytes(B, T_max, Hq, Hkv, D, max_context_len, num_splits=0, P=PAGE_SIZE):
    return int(_lib().splash_prefill_attn_workspace_bytes(int(B), int(T_max), int(Hq), int(Hkv), int(D), int(P),
                                                           int(max_context_len), int(num_splits)))


def splash_prefill_attn(q, out, k_pool, v_pool, k_scale, v_scale, block_table, context_lens, chunk_lens,
                        max_context_len, sm_scale, num_splits=0, workspace=None, stream=None):
    """Causal attention of a prefill chunk over the int8 paged cache (the chunk's
    K/V already appended); writes out[b][t][h][:] for t < chunk_lens[b]."""
    torch = _torch()
    if q.dim() != 4:
        raise ValueError("q must be [B][T_max][Hq][D]")
    B, T_max, Hq, Dq = (int(x) for x in q.shape)
    _dev(q, "q", (torch.bfloat16, torch.int16))
    _dev(out, "out", (torch.bfloat16, torch.int16), tuple(q.shape))
    num_pages, Hkv, P, D = _pool_dims(k_pool, v_pool, k_scale, v_scale)
    if Dq != D:
        raise ValueError("q head dim does not match the pools")
    maxp = _lens(block_table, context_lens, chunk_lens, B)
    need = splash_prefill_attn_workspace_bytes(B, T_max, Hq, Hkv, D, max_context_len, num_splits, P)
    ws_ptr, ws_bytes = None, 0
    if need:
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        _dev(workspace, "workspace", (torch.uint8, torch.int8, torch.float32))
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    rc = _lib().splash_prefill_attn(
        q.data_ptr(), out.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(), k_scale.data_ptr(),
        v_scale.data_ptr(), block_table.data_ptr(), maxp, context_lens.data_ptr(), chunk_lens.data_ptr(),
        B, T_max, Hq, Hkv, D, P, num_pages, int(max_context_len), float(sm_scale), int(num_splits),
        ws_ptr, ws_bytes, _stream(stream))
    _check(rc, "splash_prefill_attn")
    return out
