"""GPU parity across V magnitudes.

The kernel rounds P' = p * s_v * 2^jv to binary16, with a workgroup-wide
exponent jv that puts the largest V scale seen so far into [64, 128); when a
later step of keys brings a scale in a higher binade, jv drops and the output
rows already accumulated are rescaled by that power of two.  These workloads
take V far from unit scale and make its scales climb inside every split:
 * v_mag 1e-4 and 1e-3: V scales around 3e-6 and 3e-5, below binary16's normal
   range (P' = p * s_v alone would be subnormal);
 * v_mag 3e4: V scales around 800;
 * climbing V: each 128-token cycle multiplies V by up to 2^6, so every split
   of at least 8 pages sees its largest scale rise after its first step.
Every valid row is compared with the fp64 oracle at split counts 1, 3 and the
preset: relative L2 <= 2e-3, every element within 1e-2 * (V's magnitude) plus
half a bf16 ulp, and within half an ulp plus 2^-8 of the attention of |V|.  For
the climbing workload the test shows on the host that the largest V scale of
some split rises by a binade after the split's first step.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

import speculative_decode_attention_amd as sda  # noqa: E402
from speculative_decode_attention_amd import synth  # noqa: E402
from gpu_util import BF16_NAN, Prepared, assert_attn_ok, bf16_to_f64, log  # noqa: E402


def climbing(pos, ctx):
    return np.exp2(6.0 * (pos % 128) / 128.0)


WORKLOADS = {
    "v_mag_1e-4": (dict(v_mag=1e-4), 1e-4),
    "v_mag_1e-3": (dict(v_mag=1e-3), 1e-3),
    "v_mag_3e4": (dict(v_mag=3e4), 3e4),
    "climbing_v": (dict(v_gain=climbing), 64.0),
}

_cache = {}


def prepared(name):
    if name not in _cache:
        _cache.clear()
        wl = synth.make_workload(name, 81, B=2, context_lens=[4096, 1555], T_max=16, draft_lens=[16, 11],
                                 Hq=24, Hkv=4, D=256, num_pages=400, **WORKLOADS[name][0])
        _cache[name] = Prepared(wl)
    return _cache[name]


def binade_rises(prep, S):
    """Splits whose largest V scale, over the keys after the first step, lies in a
    higher binade than the first step's largest."""
    wl = prep.wl
    L = sda.splash_verify_attn_split_pages(wl.max_context_len, wl.P, S)
    vs = prep.pools[3].view(np.float16).astype(np.float64)
    rises = 0
    for b in range(wl.B):
        ctx = int(wl.context_lens[b])
        pos = np.arange(ctx)
        sv = vs[wl.block_table[b, pos // wl.P], :, pos % wl.P]                 # [ctx][Hkv]
        for s0 in range(0, ctx, L * wl.P):
            s1 = min(s0 + L * wl.P, ctx)
            if s1 <= s0 + 64:
                continue
            first = np.floor(np.log2(sv[s0:s0 + 64].max(axis=0)))
            later = np.floor(np.log2(sv[s0 + 64:s1].max(axis=0)))
            rises += int(np.sum(later > first))
    return rises


@pytest.mark.parametrize("name", list(WORKLOADS))
@pytest.mark.parametrize("S", [1, 3, 0])
def test_v_scales_match_oracle(name, S):
    prep = prepared(name)
    wl = prep.wl
    if name == "climbing_v":
        S_eff = S if S else sda.splash_verify_attn_default_splits(wl.B, wl.Hkv, wl.max_context_len, wl.P, wl.D)
        rises = binade_rises(prep, S_eff)
        log(f"  {name}, splits {S_eff}: {rises} (split, kv head) pairs whose V scales rise a binade")
        assert rises > 0
    out = prep.run(num_splits=S).cpu().numpy()
    rows = prep.valid_rows()
    got = bf16_to_f64(out[rows[:, 0], rows[:, 1], rows[:, 2]])
    assert_attn_ok(got, prep.oracle_rows(rows), f"{name}, {S or 'preset'} splits",
                   mag=prep.oracle_rows(rows, abs_v=True), floor=prep.p_floor(rows), v_scale=WORKLOADS[name][1])
    for b in range(wl.B):
        assert np.all(out[b, int(wl.draft_lens[b]):].view(np.uint16) == BF16_NAN)
