"""Planted mistakes in the oracle must each be caught by at least one pin.

Each mutant is a copy of the oracle's C source with one plausible mistake
(a dropped term, a wrong sign, index or operand, an off-by-one), compiled with
gcc on the CPU into a temporary library.  The pins that ran green on the real
oracle must fail on every mutant; a mutant they all pass would mean the pins
cannot see that kind of mistake.
"""
import subprocess
import sys
import tempfile
from pathlib import Path

import pytest

import oracle
import oracle_pins

MUTANTS = {
    # quantiser
    "divisor_128": ("float s32 = amax / 127.0f;", "float s32 = amax / 128.0f;"),
    "truncate_not_round": ("float r = rintf(x[d] / s);", "float r = truncf(x[d] / s);"),
    "ties_away": ("float r = rintf(x[d] / s);", "float r = roundf(x[d] / s);"),
    "fp32_scale_for_codes": ("float s = ref_f16_to_f32(s16);", "float s = s32;"),
    "clamp_minus_128": ("if (r < -127.0f) r = -127.0f;", "if (r < -128.0f) r = -128.0f;"),
    "amax_not_abs": ("float a = fabsf(x[d]);", "float a = x[d];"),
    "f16_ties_up": ("if (rem > 0x1000u || (rem == 0x1000u && (h & 1u)))", "if (rem >= 0x1000u)"),
    "f16_subnormal_shift": ("int shift = -e - 1;", "int shift = -e;"),
    "bf16_widen_shift": ("return bits_f32((uint32_t)b << 16);", "return bits_f32((uint32_t)b << 15);"),
    # append placement
    "append_pos_off_by_one": ("int pos = n - dl + t;", "int pos = n - dl + t + 1;"),
    "v_layout_like_k": ("{ return ((((size_t)page * Hkv + g) * (P / 8) + slot / 8) * D + d) * 8 + slot % 8; }",
                        "{ return (((size_t)page * Hkv + g) * P + slot) * D + d; }"),
    "v_tile_dropped": ("{ return ((((size_t)page * Hkv + g) * (P / 8) + slot / 8) * D + d) * 8 + slot % 8; }",
                       "{ return ((((size_t)page * Hkv + g) * (P / 8)) * D + d) * 8 + slot % 8; }"),
    "append_v_scale_into_k": ("k_scale[s_index(page, g, slot, Hkv, P)] = s16;",
                              "v_scale[s_index(page, g, slot, Hkv, P)] = s16;"),
    # attention
    "causal_excludes_self": (": (pos + 1 < j_hi ? pos + 1 : j_hi);", ": (pos < j_hi ? pos : j_hi);"),
    "causal_sees_next": (": (pos + 1 < j_hi ? pos + 1 : j_hi);", ": (pos + 2 < j_hi ? pos + 2 : j_hi);"),
    "no_sm_scale": ("z[j - j_base] = sm_scale * dot;", "z[j - j_base] = dot;"),
    "k_uses_v_scale": ("double ks = (double)ref_f16_to_f32(k_scale[",
                       "double ks = (double)ref_f16_to_f32(v_scale["),
    "v_uses_k_scale": ("double vs = (double)ref_f16_to_f32(v_scale[",
                       "double vs = (double)ref_f16_to_f32(k_scale["),
    "gqa_modulo": ("context_lens[b], draft_lens[b], t, h / group,", "context_lens[b], draft_lens[b], t, h % Hkv,"),
    "page_slot_swapped": ("int page = bt_row[j / P], slot = j % P;\n        double ks",
                          "int page = bt_row[j % P], slot = j / P;\n        double ks"),
    "no_normalise": ("for (int d = 0; d < D; ++d) out_row[d] /= wsum;", ""),
    "lse_missing_log": ("return zmax + log(wsum);", "return zmax + wsum;"),
    # split and merge
    "split_range_shift": ("long lo = (long)s * L * P, hi", "long lo = (long)s * L * P + 1, hi"),
    "merge_weight_sign": ("double w = exp(l - M);", "double w = exp(M - l);"),
    "merge_no_normalise": ("for (int d = 0; d < D; ++d) o[d] /= wsum;", ""),
    # tree masks
    "tree_mask_ignored": ("    if (!mask) return 1;", "    return 1;"),
    "tree_mask_bit_shift": ("return (int)((*mask >> (j - blk0)) & 1u);", "return (int)((*mask >> (j - blk0 + 1)) & 1u);"),
    "tree_mask_hides_context": ("    if (j < blk0) return 1;", "    if (j < blk0) return j + 1 < blk0;"),
    # sliding windows
    "window_off_by_one": ("if (window > 0 && pos - window + 1 > j_lo) j_lo = pos - window + 1;",
                          "if (window > 0 && pos - window > j_lo) j_lo = pos - window;"),
    "window_ignored": ("if (window > 0 && pos - window + 1 > j_lo) j_lo = pos - window + 1;", ""),
    # acceptance
    "accept_ties_highest": ("if (x > bv) { bv = x; best = v; }", "if (x >= bv) { bv = x; best = v; }"),
    "accept_compares_bits": ("float x = bf16_to_f32(row[v]);", "float x = (float)row[v];"),
    "accept_draft_index": ("while (a < d && blk[a] == y) {", "while (a < d && blk[a - 1] == y) {"),
    "accept_drafts_from_zero": ("int a = 1;\n        int y", "int a = 0;\n        int y"),
    "accept_rollback_wrong": ("context_lens[b] -= d - a;", "context_lens[b] -= a;"),
    "accept_noop_falls_through": ("if (d == 0) { accepted[b] = 0; next_token[b] = -1; continue; }",
                                  "if (d == 0) { accepted[b] = 0; next_token[b] = -1; }"),
}


_CHILD = r"""
import sys
sys.path[:0] = [{root!r}, {tests!r}]
import oracle, oracle_pins
orc = oracle.Oracle({lib!r})
for pin in oracle_pins.ALL_PINS:
    try:
        pin(orc)
    except (AssertionError, ValueError, FloatingPointError):
        print("CAUGHT_BY", pin.__name__)
        sys.exit(0)
print("NOT_CAUGHT")
sys.exit(3)
"""


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    old, new = MUTANTS[name]
    src = oracle.SRC.read_text()
    assert src.count(old) >= 1, f"mutation site for {name} not found in the oracle source"
    mutated = src.replace(old, new)
    root = Path(__file__).resolve().parents[1]
    with tempfile.TemporaryDirectory() as tmp:
        csrc = Path(tmp) / "mutant.c"
        csrc.write_text(mutated)
        lib = oracle.build(csrc, Path(tmp) / "libmutant.so")
        # a child process, so that a mutant which reads out of bounds and
        # crashes (also a visible failure) cannot take the test runner down
        proc = subprocess.run([sys.executable, "-c", _CHILD.format(
            root=str(root), tests=str(root / "tests"), lib=str(lib))],
            capture_output=True, text=True, timeout=600)
        assert proc.returncode != 3, f"no pin fails on mutant {name}"
        assert proc.returncode == 0 or proc.returncode < 0, proc.stderr[-2000:]
