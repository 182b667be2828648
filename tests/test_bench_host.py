"""Host-side checks of bench.py (no GPU): it refuses more than one GPU, and its
algorithmic byte count is the per-token figure times the tokens."""
import subprocess
import sys
from pathlib import Path

ROOT = Path(__file__).resolve().parents[1]
sys.path.insert(0, str(ROOT))

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    proc = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                          timeout=120)
    assert proc.returncode == 2
    assert "one GPU" in proc.stderr


def test_verify_bytes_at_32k():
    # per (token, kv head): int8 K and V rows of 256 plus two fp16 scales = 516 bytes;
    # per call: bf16 q in and out for 16 drafts x 24 heads x 256, the block table, two lengths
    ctx, Hkv, D, T, Hq = 32768, 4, 256, 16, 24
    expect = ctx * Hkv * 516 + T * Hq * D * 2 * 2 + (ctx // 16) * 4 + 8
    assert bench.verify_bytes(ctx, Hkv, D, T, Hq) == expect == 68034568


def test_batch_bytes_of_the_shared_prefix_batch():
    # config 4: 1,536 shared + 4 x 128 private pages = 32,768 distinct tokens, four requests of 26,624
    # tokens with 16 drafts each; the block table counts every request's 1,664 entries
    n = bench.batch_bytes([26624] * 4, [16] * 4, 4, 256, 24, distinct_tokens=2048 * 16)
    assert n == 32768 * 4 * 516 + 4 * 16 * 24 * 256 * 4 + 4 * 1664 * 4 + 4 * 8 == 69232672


def test_batch_bytes_follow_the_drawn_draft_lengths():
    dl = [3, 16, 1]
    n = bench.batch_bytes([32768] * 3, dl, 4, 256, 24)
    assert n == 3 * 32768 * 4 * 516 + sum(dl) * 24 * 256 * 4 + 3 * 2048 * 4 + 3 * 8
    # one request with 16 drafts is the single-request figure
    assert bench.batch_bytes([32768], [16], 4, 256, 24) == bench.verify_bytes(32768, 4, 256, 16, 24)


def test_batch_flops_count_visible_keys():
    # draft t of a block of d at context c sees c - d + t + 1 keys; 4 D flops per (row, key) and q head
    assert bench.batch_flops([10], [2], 1, 1) == 4 * (9 + 10)
    assert bench.batch_flops([26624] * 4, [16] * 4, 24, 256) == 41864134656


def test_phase_slices(tmp_path):
    log = tmp_path / "phases.json"
    ph = bench.Phases()
    ph.add("a", 3)
    ph.add(bench.HEADLINE, 5)
    ph.add("c", 0)
    ph.write(log)
    assert bench._phase_slices(log, 8) == [("a", 0, 3), (bench.HEADLINE, 3, 8), ("c", 8, 8)]
    import pytest
    with pytest.raises(SystemExit):
        bench._phase_slices(log, 9)
