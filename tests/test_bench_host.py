"""Host-side checks of bench.py (no GPU): the algorithmic byte counts behind roofline.achieved,
the source-keyed HBM traffic summaries, the launch shapes it reports, the host CPU report of
the oracle leg, the routing recipe of the named workloads, and the one-GPU refusal."""
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


def test_launch_shape_reported_per_kernel():
    # the combine has its own shape (at most 8 waves per token), not the gated norm's
    comb = bench.launch_config("finalize_ep_combine", dict(kind="ep_combine", T=2048, H=7168))
    gated = bench.launch_config("gated_residual_rmsnorm", dict(kind="gated", T=4096, H=7168))
    fin = bench.launch_config("finalize_prefill", dict(kind="finalize", T=16384, H=7168, k=8,
                                                       expert_gamma=None))
    assert comb["waves_per_token"] == 8 and comb["vectors_per_lane"] == 2
    assert gated["waves_per_token"] == 16 and gated["vectors_per_lane"] == 1
    assert fin["waves_per_token"] == 8 and fin["block"] == 512 and fin["grid"] == 16384
    # the EP partial reports its own shape (one slot per wave at H = 7168)
    part = bench.launch_config("finalize_ep_partial", dict(kind="ep_partial", T=16384, H=7168, k=8))
    assert part == dict(waves_per_token=16, vectors_per_lane=1, block=1024, grid=16384)


def test_cpu_share_and_host_report(monkeypatch):
    monkeypatch.setenv("OMP_NUM_THREADS", "3")
    assert bench.cpu_share() == min(3, len(os.sched_getaffinity(0)))
    monkeypatch.delenv("OMP_NUM_THREADS")
    assert bench.cpu_share() == len(os.sched_getaffinity(0))
    h = bench.host_cpu()
    assert h["logical_cpus"] == os.cpu_count()
    assert h["model"] and h["model"] != "unknown"


def test_named_finalize_workloads_follow_the_logits_recipe():
    import workloads
    for name in ("finalize_tiny", "finalize_decode_per_expert", "finalize_prefill",
                 "finalize_1tok", "finalize_1tok_per_expert", "finalize_ep_partial",
                 "finalize_prefill_mxfp4", "finalize_wide_12288", "finalize_wide_20480",
                 "finalize_wide_32768"):
        assert workloads.WORKLOADS[name]["routing"] == "logits", name
    assert workloads.WORKLOADS["finalize_tiny"]["layout"] == "random"
    assert workloads.WORKLOADS["finalize_prefill"]["layout"] == "expert_sorted"
    # the bench's description of the recipe, and the oracle leg's own routing of the logits
    d = workloads.make_inputs("finalize_prefill", T=64)
    assert "routed on the GPU by mf_moe_route" in bench._routing(d)
    c = bench.oracle_inputs(d)
    assert c["idx"].shape == (64, 8) and c["weights"].dtype == np.float32
    assert np.array_equal(np.sort(c["idx"].ravel()), np.arange(64 * 8))


def test_same_size_copies_move_their_norms_bytes():
    # each copy workload moves exactly the algorithmic bytes of the norm it stands beside, computed
    # here from small instances of the same formulas scaled to the full sizes
    import workloads
    for copy, ref, (T, H) in (("stream_copy_gated", "gated_residual_rmsnorm", (4096, 8192)),
                              ("stream_copy_rmsnorm_mxfp4", "rmsnorm_mxfp4", (4096, 8192))):
        small = bench.algorithmic_bytes(workloads.make_inputs(ref, T=1))
        per_token = bench.algorithmic_bytes(workloads.make_inputs(ref, T=2)) - small
        full = small + (T - 1) * per_token
        assert workloads.make_inputs(ref, T=1)["H"] == H
        assert bench.algorithmic_bytes(bench.make_workload(copy)) == full, copy
    small = bench.algorithmic_bytes(workloads.make_inputs("rmsnorm_sigmoid_gate", T=1))
    per_token = bench.algorithmic_bytes(workloads.make_inputs("rmsnorm_sigmoid_gate", T=2)) - small
    assert bench.algorithmic_bytes(bench.make_workload("stream_copy_per_head")) == small + 4095 * per_token


def test_workload_overrides():
    assert bench.parse_overrides(["H=2048", "k=4"]) == {"H": 2048, "k": 4}
    for bad in (["H"], ["H=2.5"], ["=3"], ["2x=1"]):
        with pytest.raises(SystemExit):
            bench.parse_overrides(bad)
    d = bench.make_workload("finalize_prefill", {"T": 8, "H": 2048, "k": 4})
    assert (d["T"], d["H"], d["k"], d["E"]) == (8, 2048, 4, 256)
    assert d["logits"].shape == (8, 256) and d["routing"] == "logits"
    with pytest.raises(ValueError):
        bench.make_workload("stream_copy", {"T": 8})


def test_run_labels():
    # the names under which runs and their profile summaries are kept
    assert bench.run_label("finalize_prefill", {}) == "finalize_prefill"
    assert bench.run_label("finalize_prefill", {"H": 4096, "k": 2}) == "finalize_prefill_H4096_k2"
    assert bench.run_label("finalize_prefill", {"T": 20480}, 2) == "finalize_prefill_T20480_sets2"
    assert bench.run_label("finalize_prefill", {}, 0, True) == "finalize_prefill_inplace"
    assert (bench.run_label("gated_residual_rmsnorm", {"T": 64}, 3, True)
            == "gated_residual_rmsnorm_T64_sets3_inplace")
