"""Host-side checks of bench.py: the one-GPU refusal and the algorithmic byte counts
its GB/s figures divide by (no GPU needed)."""
import subprocess
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
sys.path.insert(0, str(ROOT))

import bench  # noqa: E402
from decode_attention_append_amd.workloads import WORKLOADS  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       cwd=ROOT, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.parametrize("name,kv,total", [
    # 32 sequences x 8 KV heads x 8192 keys x (K + V) x 128 dims x 2 bytes; q and out 32 x 16 x 128 x 2
    # bytes each; the append reads and writes 32 x 8 new K and V rows of 256 bytes
    ("gqa16x8_b32_ctx8192_28l", 32 * 8 * 8192 * 2 * 128 * 2,
     32 * 8 * 8192 * 2 * 128 * 2 + 2 * 32 * 16 * 128 * 2 + 4 * 32 * 8 * 128 * 2),
    # one sequence at 512 keys, 8 KV heads, 16 query heads
    ("qwen3_0p6b_b1_ctx512", 8 * 512 * 2 * 128 * 2, 8 * 512 * 2 * 128 * 2 + 2 * 16 * 128 * 2 + 4 * 8 * 128 * 2),
])
def test_algorithmic_bytes(name, kv, total):
    w = WORKLOADS[name]
    assert bench.algorithmic_bytes(w, [w.seq_pos] * w.batch) == (kv, total)


def test_algorithmic_bytes_gated_head_dim_256():
    """The gated workload also reads the gate (the output's shape); K+V are 1 KB per key."""
    w = WORKLOADS["qwen35_gqa16x2_d256_gated_b16_ctx8192_10l"]
    sp = [8000 + i for i in range(w.batch)]
    ctx = sum(s + 1 for s in sp)
    kv = 2 * ctx * 2 * 256 * 2
    assert bench.algorithmic_bytes(w, sp) == (kv, kv + 3 * 16 * 16 * 256 * 2 + 4 * 16 * 2 * 256 * 2)


def test_counter_staleness_ignores_comments_only():
    """The counters' source hash changes with the code, not with its comments."""
    from decode_attention_append_amd import profiling
    a = "int f(int x) {  // doubles\n    return 2 * x; /* plain */\n}\n"
    b = "// a new comment\nint f(int x) {\n  return 2 * x;\n}\n"
    c = "int f(int x) {\n    return 3 * x;\n}\n"
    assert profiling.code_text(a) == profiling.code_text(b)
    assert profiling.code_text(a) != profiling.code_text(c)
