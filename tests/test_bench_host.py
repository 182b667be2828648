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
