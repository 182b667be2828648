"""Dense brute-force attention in numpy -- an independent check of the oracle.

TEST INFRASTRUCTURE ONLY.  No paging, no quantisation, no block table: the
caller hands over the dequantised context as dense fp64 arrays.  It is written
as whole-matrix numpy operations (a matmul, a mask, a row softmax), a route
that shares nothing with the C oracle's per-key loops, so the two can pin each
other on small inputs whose values are exactly representable.

The definition (Splash community summary on discuss.pytorch.kr, sections on
DFlash 2 block verification and on the decode kernel that reuses the 8-bit
cache across query heads and verify tokens): the T drafted tokens of one
request are checked in one pass; draft t sits at position N - T + t of an
N-token context and sees keys 0..N - T + t; query head h reads kv head
h // (Hq // Hkv).
"""
from __future__ import annotations

import numpy as np


def dense_block_attention(q: np.ndarray, k_hat: np.ndarray, v_hat: np.ndarray,
                          sm_scale: float, block_masks=None, window=None) -> np.ndarray:
    """q: [T][Hq][D]; k_hat, v_hat: [N][Hkv][D] (all fp64) -> out [T][Hq][D] fp64.
    block_masks: optional [T] integers; bit u of block_masks[t] lets draft t see
    the key of draft u (a tree of candidates instead of the causal chain).
    window: optional W >= 1; draft t at position p then sees only keys > p - W."""
    q = np.asarray(q, dtype=np.float64)
    k_hat = np.asarray(k_hat, dtype=np.float64)
    v_hat = np.asarray(v_hat, dtype=np.float64)
    T, Hq, D = q.shape
    N, Hkv, _ = k_hat.shape
    group = Hq // Hkv
    visible_last = N - T + np.arange(T)                      # last key each draft sees
    hidden = np.arange(N)[None, :] > visible_last[:, None]   # [T][N] causal mask
    if block_masks is not None:                              # inside the block: the given bits
        bits = (np.asarray(block_masks, dtype=np.int64)[:, None] >> np.arange(T)[None, :]) & 1   # [T][T]
        hidden[:, N - T:] = bits == 0
    if window is not None:                                   # sliding window: keys > p - W
        hidden |= np.arange(N)[None, :] <= (visible_last - window)[:, None]
    out = np.empty((T, Hq, D))
    for h in range(Hq):
        g = h // group
        scores = sm_scale * (q[:, h, :] @ k_hat[:, g, :].T)  # [T][N]
        scores = np.where(hidden, -np.inf, scores)
        scores = scores - scores.max(axis=1, keepdims=True)
        w = np.exp(scores)
        out[:, h, :] = (w @ v_hat[:, g, :]) / w.sum(axis=1, keepdims=True)
    return out
