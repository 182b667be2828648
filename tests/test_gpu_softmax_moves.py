"""GPU parity where the online softmax must move its reference.

The kernel keeps each row's scores relative to a reference that moves only when
a later step of keys beats it by more than a slack of 8 (log2 units); when that
happens the row sums and the output rows already accumulated are rescaled.  A
row's value must not depend on where in the context its largest score falls:
speculative output equals plain autoregressive decoding (discuss.pytorch.kr
summary, section "DFlash 2 speculative decoding as the default path").  With
N(0, 1) keys the scores never jump that far, so these workloads make them:
 * larger keys (k_mag 4 and 16): spread scores, the maximum anywhere;
 * rising K spikes: a shared direction w added to the keys with amplitudes that
   climb inside every 8-page cycle and peak in the draft block, so each split's
   maximum comes after its first step and the row's maximum lies in the last
   split and inside the block;
 * V scales beyond 255 (v_mag 3e4): the slack drops to 0 for such steps.
Every valid row is compared with the fp64 oracle (relative L2, 1e-2 + half a
bf16 ulp, and half an ulp + 2^-8 of the attention of |V| per element), at
split counts 1, 3 and the preset.  For each workload the test also shows, from
the dequantised cache on the host, that the move condition occurs: some row
has a step after the first whose largest score exceeds the first step's by more
than 8.5 log2 units in the split the kernel gives it (a jump past 16 would
overflow binary16 without a move, so a missing move cannot pass).
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

import speculative_decode_attention_amd as sda  # noqa: E402
from speculative_decode_attention_amd import synth  # noqa: E402
from gpu_util import BF16_NAN, Prepared, assert_attn_ok, bf16_to_f64, log  # noqa: E402

SLACK = 8.0          # log2 units the reference may lag a step's maximum


def sawtooth_spikes(pos, ctx):
    """Amplitude climbing 0 -> 24 over each 128-token cycle, 36 in the last 16 tokens."""
    amp = 24.0 * (pos % 128) / 127.0
    return np.where(pos >= ctx - 16, 36.0, amp)


WORKLOADS = {
    "k_mag_4": dict(k_mag=4.0),
    "k_mag_16": dict(k_mag=16.0),
    "rising_spikes": dict(k_spike=sawtooth_spikes),
    "v_mag_3e4": dict(v_mag=3e4),
}

_cache = {}


def prepared(name):
    if name not in _cache:
        _cache.clear()
        wl = synth.make_workload(name, 71, B=2, context_lens=[4096, 1555], T_max=16, draft_lens=[16, 11],
                                 Hq=24, Hkv=4, D=256, num_pages=400, **WORKLOADS[name])
        _cache[name] = Prepared(wl)
    return _cache[name]


def dequant_k(prep, b):
    """fp64 K rows [ctx][Hkv][D] of request b, read through its block table."""
    wl = prep.wl
    kp, _, ks, _ = prep.pools
    ctx = int(wl.context_lens[b])
    pos = np.arange(ctx)
    pages = wl.block_table[b, pos // wl.P]
    codes = kp[pages, :, pos % wl.P, :].astype(np.float64)                    # [ctx][Hkv][D]
    scale = ks[pages, :, pos % wl.P].view(np.float16).astype(np.float64)      # [ctx][Hkv]
    return codes * scale[:, :, None]


_moves = {}


def count_moves(prep, S):
    """(row, split) pairs whose split has a later step beating its first step's
    maximum by more than the slack + 0.5 log2 units, and the largest such jump.
    The slack is 8, or 0 where a V scale exceeds 255 (binary16 then has no room
    for p > 1)."""
    key = (prep.wl.name, S)
    if key not in _moves:
        _moves[key] = _count_moves(prep, S)
    return _moves[key]


def _count_moves(prep, S):
    wl = prep.wl
    slack = 0.0 if prep.pools[3].view(np.float16).astype(np.float64).max() > 255.0 else SLACK
    L = sda.splash_verify_attn_split_pages(wl.max_context_len, wl.P, S)
    q = bf16_to_f64(wl.q)
    moves, top = 0, 0.0
    for b in range(wl.B):
        d, ctx = int(wl.draft_lens[b]), int(wl.context_lens[b])
        k = dequant_k(prep, b)
        for t in range(d):
            pos = ctx - d + t
            # z[h][j] in log2 units for keys 0..pos
            qh = q[b, t].reshape(wl.Hkv, wl.G, wl.D)                          # [g][hh][D]
            z = np.einsum("ghd,jgd->ghj", qh, k[:pos + 1]) * wl.sm_scale / np.log(2.0)
            for s0 in range(0, pos + 1, L * wl.P):
                s1 = min(s0 + L * wl.P, pos + 1)
                step0 = z[:, :, s0:min(s0 + 64, s1)].max(axis=2)
                if s1 <= s0 + 64:
                    continue
                later = z[:, :, s0 + 64:s1].max(axis=2)
                jump = later - step0
                moves += int(np.sum(jump > slack + 0.5))
                top = max(top, float(jump.max()))
    return moves, top


@pytest.mark.parametrize("name", list(WORKLOADS))
@pytest.mark.parametrize("S", [1, 3, 0])
def test_reference_moves_match_oracle(name, S):
    prep = prepared(name)
    wl = prep.wl
    S_eff = S if S else sda.splash_verify_attn_default_splits(wl.B, wl.Hkv, wl.max_context_len, wl.P, wl.D)
    moves, top = count_moves(prep, S_eff)
    log(f"  {name}, splits {S or 'preset'} ({S_eff}): {moves} (row, split) pairs with a move, largest jump "
        f"{top:.1f} log2 units")
    assert moves > 0, "the workload does not make the reference move"
    out = prep.run(num_splits=S).cpu().numpy()
    rows = prep.valid_rows()
    got = bf16_to_f64(out[rows[:, 0], rows[:, 1], rows[:, 2]])
    assert_attn_ok(got, prep.oracle_rows(rows), f"{name}, {S or 'preset'} splits",
                   mag=prep.oracle_rows(rows, abs_v=True), floor=prep.p_floor(rows), v_scale=WORKLOADS[name].get("v_mag", 1.0))
    for b in range(wl.B):
        assert np.all(out[b, int(wl.draft_lens[b]):].view(np.uint16) == BF16_NAN)


def test_spike_maximum_lies_in_the_block():
    """The rising-spike workload puts rows' largest scores in the draft block and
    in the last split (the merge must weigh that split most)."""
    prep = prepared("rising_spikes")
    wl = prep.wl
    q = bf16_to_f64(wl.q)
    in_block = 0
    for b in range(wl.B):
        d, ctx = int(wl.draft_lens[b]), int(wl.context_lens[b])
        k = dequant_k(prep, b)
        t = d - 1
        qh = q[b, t].reshape(wl.Hkv, wl.G, wl.D)
        z = np.einsum("ghd,jgd->ghj", qh, k[:ctx])
        in_block += int(np.sum(z.argmax(axis=2) >= ctx - d))
    log(f"  rows whose largest score is a draft key: {in_block}")
    assert in_block > 0
