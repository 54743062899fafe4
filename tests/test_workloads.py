"""The seeded input generator: determinism and the structure of each workload (CPU only)."""
import numpy as np
import pytest

import workloads
from tests.helpers import f32


def test_same_seed_same_bytes():
    a = workloads.make_inputs("finalize_tiny")
    b = workloads.make_inputs("finalize_tiny")
    for key in ("logits", "expert_rows", "idx", "residual", "gamma"):
        assert np.array_equal(a[key], b[key]), key
    c = workloads.make_inputs("finalize_tiny", seed=99)
    assert not np.array_equal(a["expert_rows"], c["expert_rows"])
    d = workloads.make_finalize_inputs(9, 16, E=4, k=2, seed=3)      # drawn routing
    e = workloads.make_finalize_inputs(9, 16, E=4, k=2, seed=3)
    for key in ("expert_rows", "idx", "weights", "expert_ids", "residual", "gamma"):
        assert np.array_equal(d[key], e[key]), key


def test_logits_recipe_draws_logits_and_leaves_the_routing_to_the_consumer():
    # C1: N(0,1) logits [T, E], then a drawn random row permutation; the experts and weights are
    # not drawn (the routing computes them)
    d = workloads.make_inputs("finalize_tiny")
    assert d["logits"].shape == (16, 8) and d["logits"].dtype == np.float32
    assert d["expert_ids"] is None and d["weights"] is None
    assert np.array_equal(np.sort(d["idx"].ravel()), np.arange(32))
    # C3 at reduced T: the expert-sorted idx is the routing's too
    p = workloads.make_inputs("finalize_prefill", T=4096)
    assert p["idx"] is None and p["logits"].shape == (4096, 256)
    assert abs(float(p["logits"].std()) - 1.0) < 0.01 and abs(float(p["logits"].mean())) < 0.01
    assert p["expert_rows"].shape == (4096 * 8, 7168)


def test_with_routing_completes_the_workload():
    d = workloads.make_inputs("finalize_decode_per_expert", T=4)
    ids = np.array([[3, 1, 0, 2, 4, 5, 6, 7]] * 4, np.int32)
    w = np.full((4, 8), 0.125, np.float32)
    idx = np.arange(32, dtype=np.int32).reshape(4, 8)[::-1].copy()
    c = workloads.with_routing(d, ids, w, idx)
    assert np.array_equal(c["expert_ids"], ids) and np.array_equal(c["idx"], idx)
    assert d["expert_ids"] is None                                   # d is unchanged
    # the random layout keeps its drawn permutation
    t = workloads.make_inputs("finalize_tiny")
    ct = workloads.with_routing(t, np.zeros((16, 2), np.int32), np.ones((16, 2), np.float32),
                                np.zeros((16, 2), np.int32))
    assert np.array_equal(ct["idx"], t["idx"])
    # an expert-parallel view marks the other ranks' slots (expert e on rank e % 8)
    ep = workloads.make_inputs("finalize_ep_partial", T=4)
    ce = workloads.with_routing(ep, ids, w, idx)
    assert np.array_equal(ce["idx"] >= 0, ids % 8 == 0)
    with pytest.raises(ValueError):
        workloads.with_routing(workloads.make_finalize_inputs(2, 8, E=4, k=2, seed=1), ids, w, idx)


@pytest.mark.parametrize("layout", ["random", "expert_grouped"])
def test_idx_is_a_bijection(layout):
    d = workloads.make_finalize_inputs(37, 16, E=12, k=5, seed=3, layout=layout)
    assert d["idx"].dtype == np.int32 and d["idx"].shape == (37, 5)
    assert np.array_equal(np.sort(d["idx"].ravel()), np.arange(37 * 5))


def test_expert_grouped_rows_are_grouped_by_expert():
    d = workloads.make_finalize_inputs(64, 16, E=32, k=8, seed=4, layout="expert_grouped")
    n = 64 * 8
    expert_of_row = np.empty(n, np.int64)
    expert_of_row[d["idx"].ravel()] = d["expert_ids"].ravel()
    assert np.all(np.diff(expert_of_row) >= 0)


def test_routing_draw_is_distinct_experts_and_simplex_weights():
    d = workloads.make_finalize_inputs(50, 8, E=16, k=4, seed=5)
    w = d["weights"].astype(np.float64)
    assert np.allclose(w.sum(axis=1), 1.0, atol=1e-6)
    assert np.all(w > 0) and np.all(np.diff(w, axis=1) <= 0)   # largest first
    for t in range(50):                                           # distinct experts per token
        assert len(set(d["expert_ids"][t])) == 4
    assert d["expert_ids"].min() >= 0 and d["expert_ids"].max() < 16
    # k == E: every expert once per token
    d = workloads.make_finalize_inputs(6, 8, E=5, k=5, seed=6)
    assert np.array_equal(np.sort(d["expert_ids"], axis=1), np.tile(np.arange(5), (6, 1)))


def test_route_inputs():
    d = workloads.make_inputs("moe_route_prefill", T=32)
    assert d["logits"].shape == (32, 256) and d["logits"].dtype == np.float32
    assert abs(d["logits"].std() - 1.0) < 0.05
    q = workloads.make_inputs("moe_route_decode")
    assert q["logits"].shape == (64, 128) and q["k"] == 8
    # bf16-valued: the low 16 bits are zero, and equal logits occur
    assert np.all(q["logits"].view(np.uint32) & 0xFFFF == 0)
    assert any(len(set(r.tolist())) < len(r) for r in q["logits"])


def test_shapes_and_dtypes_of_named_workloads():
    d = workloads.make_inputs("finalize_decode_per_expert")
    assert d["logits"].shape == (64, 128)
    assert d["expert_rows"].shape == (64 * 8, 4096) and d["expert_rows"].dtype == np.uint16
    assert d["expert_gamma"].shape == (128, 4096) and d["expert_gamma"].dtype == np.uint16
    assert d["residual"].dtype == np.float32 and abs(d["residual"].std() - 2.0) < 0.05
    g = workloads.make_inputs("gated_residual_rmsnorm", T=8)
    assert g["x"].shape == (8, 8192) and abs(f32(g["gate"]).std() - 2.0) < 0.05
    p = workloads.make_inputs("rmsnorm_sigmoid_gate", T=4)
    assert p["x"].shape == (4, 64, 64) and p["gamma"].shape == (64,)


def test_bf16_inputs_are_rounded_to_nearest_even():
    v = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -2.5], np.float32)
    assert list(workloads.to_bf16_bits(v)) == [0x3F80, 0x3F82, 0xC020]
