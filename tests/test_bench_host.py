"""Host-side checks of bench.py (no GPU): the algorithmic byte counts behind roofline.achieved,
the source-keyed HBM traffic summaries, and the one-GPU refusal."""
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _finalize_dict(T, H, k, per_expert_ids=None):
    d = dict(kind="finalize", T=T, H=H, k=k, expert_gamma=None)
    if per_expert_ids is not None:
        d["expert_gamma"] = np.zeros(1)
        d["expert_ids"] = per_expert_ids
    return d


def test_prefill_algorithmic_bytes():
    # every gathered bf16 row, the fp32 residual in and out, the bf16 out, the int32 indices
    # and fp32 weights once, and gamma once: 186,432 B per token + 14,336 B
    T, H, k = 16384, 7168, 8
    b = bench.algorithmic_bytes(_finalize_dict(T, H, k))
    assert b == T * (k * H * 2 + H * 4 + H * 4 + H * 2 + k * 8) + H * 2 == 3_054_516_224


def test_per_expert_bytes_count_each_used_expert_gamma_once():
    T, H, k = 4, 64, 2
    ids = np.array([[0, 3], [3, 5], [0, 5], [7, 3]], dtype=np.int32)   # 4 distinct experts
    plain = bench.algorithmic_bytes(_finalize_dict(T, H, k))
    per = bench.algorithmic_bytes(_finalize_dict(T, H, k, ids))
    assert per - plain == T * k * 4 + 4 * H * 2


def test_traffic_summaries_are_keyed_to_their_sources():
    # a committed summary whose kernel sources are unchanged gives its bytes; the same file read
    # against another kernel family's sources gives none
    v = bench.read_traffic("finalize_prefill", "finalize")
    if v is None:
        pytest.skip("the prefill traffic summary predates the current finalize sources")
    assert 1.0 <= v / 3_054_516_224 < 1.05
    assert bench.read_traffic("finalize_prefill", "route") is None
    assert bench.read_traffic("no_such_workload", "finalize") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)
