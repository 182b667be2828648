"""CPU oracle for block-verify decode attention over an int8 paged KV cache.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by the smoke check and by the
CPU-baseline leg of the benchmark.  The product path (the HIP library and its
binding in ``speculative_decode_attention_amd``) never imports this package.

The arithmetic lives in ``splash_oracle.c`` (plain C: fp32 quantiser, fp64
attention); ``dense.py`` is an independent numpy brute force used to pin it.
This module only builds the C file with gcc and marshals numpy arrays.

Functions whose result no page prints a value for are pinned by closed forms,
invariants and brute force in ``tests/test_oracle_*.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

HERE = Path(__file__).resolve().parent
SRC = HERE / "splash_oracle.c"
LIB = HERE / "libsplash_oracle.so"

CFLAGS = ["-O2", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
          "-std=c11", "-Wall", "-Wextra", "-Wno-unused-parameter"]


def build(src: Path = SRC, out: Path = LIB, extra_flags=()) -> Path:
    """Compile the oracle with gcc into a shared library (always recompiles)."""
    cmd = ["gcc", *CFLAGS, *extra_flags, "-o", str(out) + ".tmp", str(src), "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    os.replace(str(out) + ".tmp", out)
    return out


_P = ctypes.c_void_p
_I = ctypes.c_int
_D = ctypes.c_double


def _declare(lib):
    lib.splash_ref_kv_append_int8.argtypes = [_P, _P, _I, _P, _P, _P, _P, _P, _I, _P, _P,
                                              _I, _I, _I, _I, _I, _I]
    lib.splash_ref_verify_attn.argtypes = [_P, _P, _P, _P, _P, _P, _P, _I, _P, _P,
                                           _I, _I, _I, _I, _I, _I, _I, _D]
    lib.splash_ref_verify_attn_rows.argtypes = [_P, _P, _P, _P, _P, _P, _I, _P, _P,
                                                _I, _I, _I, _I, _I, _I, _I, _D,
                                                _P, _P, _P, _I, _P]
    lib.splash_ref_verify_attn_split.argtypes = [_P, _P, _P, _P, _P, _P, _I, _P, _P,
                                                 _I, _I, _I, _I, _I, _I, _I, _D, _I, _I,
                                                 _P, _P]
    lib.splash_ref_splitk_merge.argtypes = [_P, _P, _P, _P, _I, _I, _I, _I, _I]
    lib.splash_ref_verify_accept.argtypes = [_P, _P, _P, _P, _P, _P, _I, _I, _I]
    lib.splash_ref_verify_attn_masked.argtypes = [_P, _P, _P, _P, _P, _P, _P, _I, _P, _P,
                                                  _I, _I, _I, _I, _I, _I, _I, _D, _P]
    lib.splash_ref_verify_attn_window.argtypes = [_P, _P, _P, _P, _P, _P, _P, _I, _P, _P,
                                                  _I, _I, _I, _I, _I, _I, _I, _D, _I]
    lib.splash_ref_num_threads.argtypes = []
    lib.splash_ref_num_threads.restype = ctypes.c_int
    lib.ref_quantize_row.argtypes = [_P, _I, _P, _P]
    lib.ref_quantize_row.restype = None
    lib.ref_f32_to_f16_rne.argtypes = [ctypes.c_float]
    lib.ref_f32_to_f16_rne.restype = ctypes.c_uint16
    lib.ref_f16_to_f32.argtypes = [ctypes.c_uint16]
    lib.ref_f16_to_f32.restype = ctypes.c_float
    for f in ("splash_ref_kv_append_int8", "splash_ref_verify_attn", "splash_ref_verify_attn_rows",
              "splash_ref_verify_attn_split", "splash_ref_splitk_merge", "splash_ref_verify_accept",
              "splash_ref_verify_attn_masked", "splash_ref_verify_attn_window"):
        getattr(lib, f).restype = ctypes.c_int
    return lib


class Oracle:
    """ctypes front end over one compiled copy of the oracle."""

    def __init__(self, path: Path):
        self.lib = _declare(ctypes.CDLL(str(path)))

    # -- helpers -----------------------------------------------------------
    @staticmethod
    def _ptr(a: np.ndarray):
        assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
        return a.ctypes.data_as(ctypes.c_void_p)

    # -- quantiser ---------------------------------------------------------
    def num_threads(self) -> int:
        """Threads the oracle's parallel loops run on."""
        return int(self.lib.splash_ref_num_threads())

    def f32_to_f16(self, x: float) -> int:
        return int(self.lib.ref_f32_to_f16_rne(float(x)))

    def f16_to_f32(self, h: int) -> float:
        return float(self.lib.ref_f16_to_f32(int(h)))

    def quantize_rows(self, x: np.ndarray):
        """x: float32 [..., D] -> (int8 codes [..., D], fp16 scale bits uint16 [...])."""
        x = np.ascontiguousarray(x, dtype=np.float32)
        D = x.shape[-1]
        rows = x.reshape(-1, D)
        q = np.empty(rows.shape, dtype=np.int8)
        s = np.empty(rows.shape[0], dtype=np.uint16)
        for i in range(rows.shape[0]):
            self.lib.ref_quantize_row(rows[i].ctypes.data_as(_P), D,
                                      q[i].ctypes.data_as(_P), s[i:i + 1].ctypes.data_as(_P))
        return q.reshape(x.shape), s.reshape(x.shape[:-1])

    # -- entry points ------------------------------------------------------
    def kv_append_int8(self, k_new, v_new, k_pool, v_pool, k_scale, v_scale,
                       block_table, context_lens, draft_lens):
        """In place on the pools.  k_new/v_new: float32 or bf16-bits uint16 [B][T_max][Hkv][D]."""
        src_dtype = 0 if k_new.dtype == np.float32 else 1
        assert k_new.dtype == v_new.dtype and k_new.dtype in (np.float32, np.uint16)
        B, T_max, Hkv, D = k_new.shape
        num_pages, _, P, _ = k_pool.shape
        rc = self.lib.splash_ref_kv_append_int8(
            self._ptr(k_new), self._ptr(v_new), src_dtype, self._ptr(k_pool), self._ptr(v_pool),
            self._ptr(k_scale), self._ptr(v_scale), self._ptr(block_table), block_table.shape[1],
            self._ptr(context_lens), self._ptr(draft_lens), B, T_max, Hkv, D, P, num_pages)
        if rc:
            raise ValueError(f"oracle append rejected its arguments (rc={rc})")

    def verify_accept(self, logits, block_tokens, draft_lens, context_lens):
        """logits: bf16 bits uint16 [B][T_max][V]; block_tokens int32 [B][T_max].
        Returns (accepted int32 [B], next_token int32 [B], new context_lens int32 [B])."""
        logits = np.ascontiguousarray(logits, dtype=np.uint16)
        B, T_max, V = logits.shape
        blk = np.ascontiguousarray(block_tokens, dtype=np.int32)
        dl = np.ascontiguousarray(draft_lens, dtype=np.int32)
        ctx = np.array(context_lens, dtype=np.int32, copy=True)
        acc = np.empty(B, dtype=np.int32)
        nxt = np.empty(B, dtype=np.int32)
        rc = self.lib.splash_ref_verify_accept(self._ptr(logits), self._ptr(blk), self._ptr(dl), self._ptr(ctx),
                                               self._ptr(acc), self._ptr(nxt), B, T_max, V)
        if rc:
            raise ValueError(f"oracle verify_accept rejected its arguments (rc={rc})")
        return acc, nxt, ctx

    def verify_attn(self, q, k_pool, v_pool, k_scale, v_scale, block_table, context_lens,
                    draft_lens, Hkv, sm_scale, out=None):
        """q: bf16 bits uint16 [B][T_max][Hq][D] -> fp64 [B][T_max][Hq][D] (NaN where not written)."""
        B, T_max, Hq, D = q.shape
        num_pages, _, P, _ = k_pool.shape
        if out is None:
            out = np.full(q.shape, np.nan, dtype=np.float64)
        rc = self.lib.splash_ref_verify_attn(
            self._ptr(q), self._ptr(out), self._ptr(k_pool), self._ptr(v_pool),
            self._ptr(k_scale), self._ptr(v_scale), self._ptr(block_table), block_table.shape[1],
            self._ptr(context_lens), self._ptr(draft_lens), B, T_max, Hq, Hkv, D, P, num_pages,
            float(sm_scale))
        if rc:
            raise ValueError(f"oracle verify_attn rejected its arguments (rc={rc})")
        return out

    def verify_attn_masked(self, q, k_pool, v_pool, k_scale, v_scale, block_table, context_lens,
                           draft_lens, Hkv, sm_scale, block_masks, out=None):
        """As verify_attn with block_masks uint32 [B][T_max] (bit u of row t: draft t sees draft u)."""
        B, T_max, Hq, D = q.shape
        num_pages, _, P, _ = k_pool.shape
        masks = np.ascontiguousarray(block_masks, dtype=np.uint32)
        assert masks.shape == (B, T_max)
        if out is None:
            out = np.full(q.shape, np.nan, dtype=np.float64)
        rc = self.lib.splash_ref_verify_attn_masked(
            self._ptr(q), self._ptr(out), self._ptr(k_pool), self._ptr(v_pool),
            self._ptr(k_scale), self._ptr(v_scale), self._ptr(block_table), block_table.shape[1],
            self._ptr(context_lens), self._ptr(draft_lens), B, T_max, Hq, Hkv, D, P, num_pages,
            float(sm_scale), self._ptr(masks))
        if rc:
            raise ValueError(f"oracle verify_attn_masked rejected its arguments (rc={rc})")
        return out

    def verify_attn_window(self, q, k_pool, v_pool, k_scale, v_scale, block_table, context_lens,
                           draft_lens, Hkv, sm_scale, window, out=None):
        """As verify_attn, each draft seeing only the last `window` keys up to itself."""
        B, T_max, Hq, D = q.shape
        num_pages, _, P, _ = k_pool.shape
        if out is None:
            out = np.full(q.shape, np.nan, dtype=np.float64)
        rc = self.lib.splash_ref_verify_attn_window(
            self._ptr(q), self._ptr(out), self._ptr(k_pool), self._ptr(v_pool),
            self._ptr(k_scale), self._ptr(v_scale), self._ptr(block_table), block_table.shape[1],
            self._ptr(context_lens), self._ptr(draft_lens), B, T_max, Hq, Hkv, D, P, num_pages,
            float(sm_scale), int(window))
        if rc:
            raise ValueError(f"oracle verify_attn_window rejected its arguments (rc={rc})")
        return out

    def verify_attn_rows(self, q, k_pool, v_pool, k_scale, v_scale, block_table, context_lens,
                         draft_lens, Hkv, sm_scale, rows):
        """rows: int array [n][3] of (b, t, h) -> fp64 [n][D]."""
        B, T_max, Hq, D = q.shape
        num_pages, _, P, _ = k_pool.shape
        rows = np.ascontiguousarray(rows, dtype=np.int32)
        rb, rt, rh = (np.ascontiguousarray(rows[:, i]) for i in range(3))
        out = np.empty((rows.shape[0], D), dtype=np.float64)
        rc = self.lib.splash_ref_verify_attn_rows(
            self._ptr(q), self._ptr(k_pool), self._ptr(v_pool), self._ptr(k_scale),
            self._ptr(v_scale), self._ptr(block_table), block_table.shape[1],
            self._ptr(context_lens), self._ptr(draft_lens), B, T_max, Hq, Hkv, D, P, num_pages,
            float(sm_scale), self._ptr(rb), self._ptr(rt), self._ptr(rh), rows.shape[0],
            self._ptr(out))
        if rc:
            raise ValueError(f"oracle verify_attn_rows rejected its arguments (rc={rc})")
        return out

    def verify_attn_split(self, q, k_pool, v_pool, k_scale, v_scale, block_table, context_lens,
                          draft_lens, Hkv, sm_scale, num_splits, pages_per_split):
        """Splits of pages_per_split pages -> (part_o fp64 [B][Hq][T_max][S][D],
        part_lse fp64 [B][Hq][T_max][S])."""
        B, T_max, Hq, D = q.shape
        num_pages, _, P, _ = k_pool.shape
        S = num_splits
        part_o = np.full((B, Hq, T_max, S, D), np.nan)
        part_lse = np.full((B, Hq, T_max, S), np.nan)
        rc = self.lib.splash_ref_verify_attn_split(
            self._ptr(q), self._ptr(k_pool), self._ptr(v_pool), self._ptr(k_scale),
            self._ptr(v_scale), self._ptr(block_table), block_table.shape[1],
            self._ptr(context_lens), self._ptr(draft_lens), B, T_max, Hq, Hkv, D, P, num_pages,
            float(sm_scale), S, int(pages_per_split), self._ptr(part_o), self._ptr(part_lse))
        if rc:
            raise ValueError(f"oracle verify_attn_split rejected its arguments (rc={rc})")
        return part_o, part_lse

    def splitk_merge(self, part_o, part_lse, draft_lens, T_max):
        """part_o fp32 [B][Hq][T_max][S][D], part_lse fp32 [B][Hq][T_max][S] -> fp64 [B][T_max][Hq][D]."""
        part_o = np.ascontiguousarray(part_o, dtype=np.float32)
        part_lse = np.ascontiguousarray(part_lse, dtype=np.float32)
        B, Hq, Tm, S, D = part_o.shape
        assert Tm == T_max
        out = np.full((B, T_max, Hq, D), np.nan)
        rc = self.lib.splash_ref_splitk_merge(self._ptr(part_o), self._ptr(part_lse),
                                              self._ptr(out), self._ptr(draft_lens),
                                              B, T_max, Hq, D, S)
        if rc:
            raise ValueError(f"oracle merge rejected its arguments (rc={rc})")
        return out


_default = None


def load(path: Path = LIB) -> Oracle:
    """The oracle built from ``splash_oracle.c`` (built on first use if absent)."""
    global _default
    if path == LIB:
        if _default is None:
            if not LIB.exists() or LIB.stat().st_mtime < SRC.stat().st_mtime:
                build()
            _default = Oracle(LIB)
        return _default
    return Oracle(path)
