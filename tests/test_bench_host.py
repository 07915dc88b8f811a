"""Host-side checks of bench.py: the one-GPU contract and the counter summary it reads."""
import os
import subprocess
import sys

import bench_traffic  # noqa: F401  (the summary writer imports cleanly without a GPU)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_counter_summary_is_whole_or_ignored():
    """The committed summary either matches the decode sources and then gives HBM bytes, VALU and
    MFMA instructions per launch, or is ignored as a whole."""
    c = bench.measured_counters("moe30b_gqa_t32768")
    if c:
        assert set(c) == {"hbm_bytes_per_launch", "valu_insts_per_launch", "mfma_insts_per_launch"}
        # at least the packed K and V rows (104 B per token and KV head) are read
        assert c["hbm_bytes_per_launch"] >= 4 * 32768 * 104
        # 24 MFMAs per 32-slot block (16 for the scores of G = 8 query heads, 8 for PV: all 32
        # tokens in one MFMA per 16-dim tile): the 1024 blocks of each of 4 KV heads x 32768 tokens
        assert c["mfma_insts_per_launch"] >= 24 * 4 * 1024
        assert bench.measured_traffic("moe30b_gqa_t32768") == c["hbm_bytes_per_launch"]
    else:
        assert bench.measured_traffic("moe30b_gqa_t32768") is None


def test_unknown_workload_has_no_counters():
    assert bench.measured_counters("no_such_workload") == {}
