"""Pins of the CPU oracle to facts outside itself (CPU only).

Each test checks the oracle against something the pages or the mathematics fix: hand
worked examples, float64 brute force written independently with numpy/scipy, closed forms,
special cases that reduce to a library routine (torch's rms_norm, float32 addition), and
invariants (permutation equivariance, exact power-of-two scaling).  The cases are chosen so
that a plausible slip in the oracle (a dropped term, a wrong sign or index, a transposed
operand, a wrong norm axis, a double rounding) fails at least one of them.
"""
import json
import os

import numpy as np
import pytest
import torch
from scipy.special import expit

import oracle
import workloads
from tests.helpers import bf16_ulp_diff, f32, torch_bf16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")
U32 = 2.0 ** -24  # unit roundoff of float32


def _bits(hexes):
    return np.array([[int(h, 16) for h in row] for row in hexes], dtype=np.uint16)


def _rows_bf16(values):
    b = workloads.to_bf16_bits(np.asarray(values, dtype=np.float32))
    assert np.array_equal(f32(b), np.asarray(values, dtype=np.float32)), "fixture not exact in bf16"
    return b


# ----------------------------------------------------------------------------- golden


def test_golden_finalize_hand_example():
    g = json.load(open(GOLDEN))["moe_finalize"]
    r, o = oracle.moe_finalize(_rows_bf16(g["expert_rows"]), np.array(g["idx"], np.int32),
                               np.array(g["weights"], np.float32),
                               np.array(g["residual"], np.float32), _rows_bf16(g["gamma"]),
                               g["eps"])
    assert np.array_equal(r, np.array(g["expected_residual_out"], np.float32))
    assert np.array_equal(o, _bits(g["expected_out_bits"]))


def test_golden_gated_hand_example():
    g = json.load(open(GOLDEN))["gated_residual_rmsnorm"]
    r, o = oracle.gated_residual_rmsnorm(_rows_bf16(g["x"]), _rows_bf16(g["gate"]),
                                         np.array(g["residual"], np.float32),
                                         _rows_bf16(g["gamma"]), g["eps"])
    assert np.array_equal(r, np.array(g["expected_residual_out"], np.float32))
    assert np.array_equal(o, _bits(g["expected_out_bits"]))


def test_golden_gated_next_hand_example():
    g = json.load(open(GOLDEN))["gated_residual_next_rmsnorm"]
    r, o, on = oracle.gated_residual_next_rmsnorm(
        _rows_bf16(g["x"]), _rows_bf16(g["gate"]), np.array(g["residual"], np.float32),
        _rows_bf16(g["gamma"]), _rows_bf16(g["gamma_next"]), g["eps"])
    assert np.array_equal(r, np.array(g["expected_residual_out"], np.float32))
    assert np.array_equal(o, _bits(g["expected_out_bits"]))
    assert np.array_equal(on, _bits(g["expected_out_next_bits"]))


def test_golden_per_head_hand_example():
    g = json.load(open(GOLDEN))["rmsnorm_sigmoid_gate"]
    x = _rows_bf16(np.array(g["x"], np.float32).reshape(-1, g["D"])).reshape(np.shape(g["x"]))
    gt = _rows_bf16(np.array(g["gate"], np.float32).reshape(-1, g["D"])).reshape(x.shape)
    o = oracle.rmsnorm_sigmoid_gate(x, gt, _rows_bf16(g["gamma"]), g["eps"])
    exp = np.array([[[int(h, 16) for h in head] for head in tok] for tok in g["expected_out_bits"]],
                   dtype=np.uint16)
    assert np.array_equal(o, exp)


# ----------------------------------------------------------------------------- bf16 rounding


def test_bf16_round_matches_torch_on_float32_values():
    # On values that are exactly float32 there is only one rounding, so the oracle's
    # double->bf16 rounding must agree bit for bit with torch's float32->bf16 cast (RNE).
    rng = np.random.default_rng(11)
    v = np.concatenate([rng.standard_normal(200000).astype(np.float32),
                        (rng.standard_normal(20000) * 1e30).astype(np.float32),
                        (rng.standard_normal(20000) * 1e-30).astype(np.float32)])
    assert np.array_equal(oracle.bf16_round(v.astype(np.float64)), torch_bf16_bits(v))


def test_bf16_round_special_cases():
    cases = {
        1.0: 0x3F80, -1.0: 0xBF80, 0.0: 0x0000,
        1.0 + 2.0 ** -8: 0x3F80,          # tie between 1 and 1+2^-7: even mantissa (1) wins
        1.0 + 3 * 2.0 ** -8: 0x3F82,      # tie between 1+2^-7 and 1+2^-6: even (1+2^-6) wins
        1.0 + 2.0 ** -8 + 2.0 ** -40: 0x3F81,  # just above the tie: rounds up (no double rounding)
        2.0 ** -130: 0x0008,              # bf16 subnormal, spacing 2^-133
        3.0e38: 0x7F62, 3.5e38: 0x7F80,   # largest finite range, then overflow to +inf
    }
    for v, bits in cases.items():
        assert oracle.bf16_round(np.array([v]))[0] == bits, (v, hex(bits))
    assert oracle.bf16_round(np.array([-0.0]))[0] == 0x8000


# ----------------------------------------------------------------------------- finalize


def _bf_finalize(d):
    """float64 brute force: residual + sum_j w * row[idx]."""
    x = f32(d["expert_rows"]).astype(np.float64)
    terms = d["weights"][..., None].astype(np.float64) * x[d["idx"]]
    return d["residual"].astype(np.float64) + terms.sum(axis=1), np.abs(terms).sum(axis=1)


def _close_bf16(a, b, min_exact=0.999):
    """Within one bf16 ulp everywhere, and bit-identical almost everywhere (the reference
    rounds float64 -> float32 -> bf16, so it may differ from a single rounding at ties)."""
    d = bf16_ulp_diff(a, b)
    return d.max() <= 1 and (d == 0).mean() >= min_exact


def _rmsnorm_bits(r, gamma, eps):
    """Textbook RMSNorm through torch (float64), then to bf16."""
    rt = torch.from_numpy(np.asarray(r, np.float64))
    y = torch.nn.functional.rms_norm(rt, (rt.shape[-1],), weight=torch.from_numpy(
        f32(gamma).astype(np.float64)), eps=eps)
    return torch_bf16_bits(y.numpy())


@pytest.mark.parametrize("T,H,k,layout", [(1, 8, 1, "random"), (3, 24, 2, "random"),
                                          (16, 1024, 8, "expert_grouped"), (5, 40, 3, "random"),
                                          (7, 1024, 2, "expert_grouped")])
def test_finalize_brute_force(T, H, k, layout):
    d = workloads.make_finalize_inputs(T, H, E=max(8, k), k=k, seed=100 + T + H + k, layout=layout)
    r, o = oracle.moe_finalize(d["expert_rows"], d["idx"], d["weights"], d["residual"],
                               d["gamma"], d["eps"])
    exact, mag = _bf_finalize(d)
    bound = (k + 1) * U32 * (np.abs(d["residual"]) + mag) * 1.0001
    assert np.all(np.abs(r - exact) <= bound)
    # out is RMSNorm of the oracle's float32 residual_out, within one bf16 ulp
    assert _close_bf16(o, _rmsnorm_bits(r, d["gamma"], d["eps"]))


def test_finalize_k1_unit_weight_is_add_rmsnorm():
    # k = 1, w = 1: fma(1, x, 0) = x, so residual_out = residual + x exactly (one float32
    # add), and out is the textbook fused add + RMSNorm.
    d = workloads.make_finalize_inputs(9, 520, E=4, k=1, seed=7, layout="random")
    w = np.ones_like(d["weights"])
    r, o = oracle.moe_finalize(d["expert_rows"], d["idx"], w, d["residual"], d["gamma"], d["eps"])
    x = f32(d["expert_rows"])[d["idx"][:, 0]]
    assert np.array_equal(r, d["residual"] + x)
    assert _close_bf16(o, _rmsnorm_bits(r, d["gamma"], d["eps"]))


def test_finalize_zero_weights_keep_residual():
    d = workloads.make_finalize_inputs(6, 256, E=8, k=4, seed=8)
    r, o = oracle.moe_finalize(d["expert_rows"], d["idx"], np.zeros_like(d["weights"]),
                               d["residual"], d["gamma"], d["eps"])
    assert np.array_equal(r, d["residual"])
    assert _close_bf16(o, _rmsnorm_bits(d["residual"], d["gamma"], d["eps"]))


def test_rmsnorm_of_a_given_residual():
    # tests/refs.rmsnorm_of (the GPU tests' reference for the bf16 output of a non-unique fp32
    # residual) is the zero-weight finalize: textbook RMSNorm of the residual it is given, over
    # the rows of any leading shape, also when it runs over token blocks in threads
    from tests import refs
    rng = np.random.default_rng(21)
    for T, H in ((1, 8), (37, 520), (300, 4096)):
        r = rng.standard_normal((T, H), dtype=np.float32) * np.float32(2.0)
        gamma = workloads.to_bf16_bits(1 + 0.1 * rng.standard_normal(H, dtype=np.float32))
        got = refs.rmsnorm_of(r, gamma, 1e-6)
        assert _close_bf16(got, _rmsnorm_bits(r, gamma, 1e-6))
        assert np.array_equal(got, refs.rmsnorm_of(r, gamma, 1e-6, threads=1))
        assert np.array_equal(refs.rmsnorm_of(r.reshape(1, T, H), gamma, 1e-6)[0], got)


def test_finalize_unit_gamma_rms_closed_form():
    # gamma = 1: the RMS of r * (ms + eps)^-1/2 is sqrt(ms / (ms + eps)); bf16 rounding moves
    # each element by at most 2^-9 relative.
    d = workloads.make_finalize_inputs(8, 2048, E=16, k=4, seed=9)
    gamma = workloads.to_bf16_bits(np.ones(2048, np.float32))
    eps = 0.5  # large enough to show in the closed form
    r, o = oracle.moe_finalize(d["expert_rows"], d["idx"], d["weights"], d["residual"], gamma, eps)
    ms = (r.astype(np.float64) ** 2).mean(axis=1)
    want = np.sqrt(ms / (ms + eps))
    got = np.sqrt((f32(o).astype(np.float64) ** 2).mean(axis=1))
    assert np.all(np.abs(got - want) <= 2.0 ** -9 * want)


def test_finalize_integer_rows_exact():
    # Small integers (exact in bf16), power-of-two weights and integer residuals keep every
    # float32 step exact, so residual_out has a closed form; a wrong row, weight or a missing
    # term shows up as a mismatch.
    rng = np.random.default_rng(12)
    T, H, k, n = 11, 72, 5, 11 * 5
    rows = rng.integers(-8, 9, size=(n, H)).astype(np.float32)
    idx = rng.permutation(n).astype(np.int32).reshape(T, k)
    w = (2.0 ** rng.integers(-3, 2, size=(T, k))).astype(np.float32)
    res = rng.integers(-50, 51, size=(T, H)).astype(np.float32)
    gamma = workloads.to_bf16_bits(np.ones(H, np.float32))
    r, _ = oracle.moe_finalize(workloads.to_bf16_bits(rows), idx, w, res, gamma, 1e-6)
    want = res.astype(np.int64) * 8
    for j in range(k):
        want += (w[:, j:j + 1] * 8).astype(np.int64) * rows[idx[:, j]].astype(np.int64)
    assert np.array_equal(r, (want / 8.0).astype(np.float32))


def test_finalize_one_hot_weights_select_a_row():
    d = workloads.make_finalize_inputs(10, 96, E=8, k=4, seed=13, layout="random")
    rng = np.random.default_rng(14)
    jstar = rng.integers(0, 4, size=10)
    w = np.zeros_like(d["weights"])
    w[np.arange(10), jstar] = 1.0
    r, _ = oracle.moe_finalize(d["expert_rows"], d["idx"], w, np.zeros_like(d["residual"]),
                               d["gamma"], d["eps"])
    assert np.array_equal(r, f32(d["expert_rows"])[d["idx"][np.arange(10), jstar]])


def test_finalize_permutation_equivariance():
    d = workloads.make_finalize_inputs(12, 64, E=8, k=3, seed=15, layout="expert_grouped")
    r0, o0 = oracle.moe_finalize(d["expert_rows"], d["idx"], d["weights"], d["residual"],
                                 d["gamma"], d["eps"])
    pi = np.random.default_rng(16).permutation(d["expert_rows"].shape[0])
    rows = np.empty_like(d["expert_rows"])
    rows[pi] = d["expert_rows"]            # row p moves to pi[p]
    r1, o1 = oracle.moe_finalize(rows, pi[d["idx"]].astype(np.int32), d["weights"],
                                 d["residual"], d["gamma"], d["eps"])
    assert np.array_equal(r0, r1) and np.array_equal(o0, o1)


def test_finalize_power_of_two_scaling():
    # Scaling rows and residual by 2^m scales every float32 step exactly, and RMSNorm is
    # scale invariant up to eps.
    d = workloads.make_finalize_inputs(6, 128, E=8, k=4, seed=17)
    r0, o0 = oracle.moe_finalize(d["expert_rows"], d["idx"], d["weights"], d["residual"],
                                 d["gamma"], d["eps"])
    rows4 = workloads.to_bf16_bits(f32(d["expert_rows"]) * 4)
    r1, o1 = oracle.moe_finalize(rows4, d["idx"], d["weights"], d["residual"] * 4, d["gamma"],
                                 d["eps"])
    assert np.array_equal(r1, r0 * 4)
    assert bf16_ulp_diff(o0, o1).max() <= 1


def test_finalize_rejects_out_of_range_index():
    d = workloads.make_finalize_inputs(2, 16, E=4, k=2, seed=18, layout="random")
    bad = d["idx"].copy()
    bad[1, 1] = d["expert_rows"].shape[0]
    with pytest.raises(ValueError):
        oracle.moe_finalize(d["expert_rows"], bad, d["weights"], d["residual"], d["gamma"], 1e-6)


# ----------------------------------------------------------------------------- per-expert


def _bf_per_expert(d):
    x = f32(d["expert_rows"]).astype(np.float64)[d["idx"]]                 # [T,k,H]
    scale = 1.0 / np.sqrt((x * x).mean(axis=2, keepdims=True) + d["eps"])
    y = x * scale * f32(d["expert_gamma"]).astype(np.float64)[d["expert_ids"]]
    terms = d["weights"][..., None].astype(np.float64) * y
    return d["residual"].astype(np.float64) + terms.sum(axis=1), np.abs(terms).sum(axis=1)


@pytest.mark.parametrize("T,H,k", [(1, 16, 1), (4, 96, 3), (16, 1024, 8)])
def test_per_expert_brute_force(T, H, k):
    d = workloads.make_finalize_inputs(T, H, E=16, k=k, seed=200 + T + k, per_expert=True,
                                       residual_std=2.0)
    r, o = oracle.moe_finalize(d["expert_rows"], d["idx"], d["weights"], d["residual"],
                               d["gamma"], d["eps"], d["expert_ids"], d["expert_gamma"])
    exact, mag = _bf_per_expert(d)
    # one rounding of each normalised row to float32, k FMAs and the residual add
    bound = (k + 2) * U32 * (np.abs(d["residual"]) + mag) * 1.0001
    assert np.all(np.abs(r - exact) <= bound)
    assert _close_bf16(o, _rmsnorm_bits(r, d["gamma"], d["eps"]))


def test_per_expert_unit_gammas_ignore_expert_ids():
    d = workloads.make_finalize_inputs(8, 64, E=16, k=4, seed=19, per_expert=True)
    ones = workloads.to_bf16_bits(np.ones((16, 64), np.float32))
    other = np.random.default_rng(20).integers(0, 16, size=d["expert_ids"].shape).astype(np.int32)
    a = oracle.moe_finalize(d["expert_rows"], d["idx"], d["weights"], d["residual"], d["gamma"],
                            d["eps"], d["expert_ids"], ones)
    b = oracle.moe_finalize(d["expert_rows"], d["idx"], d["weights"], d["residual"], d["gamma"],
                            d["eps"], other, ones)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_per_expert_single_row_closed_form():
    # Every slot of a token reads the same row x through expert e, weights sum to 1, residual
    # 0: residual_out = RMSNorm_e(x) = x / rms(x) * gammaE[e].
    H, k = 256, 4
    rng = np.random.default_rng(21)
    x = workloads.to_bf16_bits(rng.standard_normal((1, H)).astype(np.float32))
    ge = workloads.to_bf16_bits((1 + 0.1 * rng.standard_normal((3, H))).astype(np.float32))
    idx = np.zeros((1, k), np.int32)
    eids = np.full((1, k), 2, np.int32)
    w = np.array([[0.5, 0.25, 0.125, 0.125]], np.float32)
    r, _ = oracle.moe_finalize(x, idx, w, np.zeros((1, H), np.float32),
                               workloads.to_bf16_bits(np.ones(H, np.float32)), 1e-6, eids, ge)
    xv = f32(x[0]).astype(np.float64)
    want = xv / np.sqrt((xv ** 2).mean() + 1e-6) * f32(ge[2]).astype(np.float64)
    assert np.all(np.abs(r[0] - want) <= 3 * U32 * np.abs(want))


def test_per_expert_row_scale_invariance():
    # Each gathered row is normalised, so scaling every row by 2^m leaves residual_out
    # unchanged up to the eps term.
    d = workloads.make_finalize_inputs(5, 128, E=8, k=3, seed=22, per_expert=True)
    a, _ = oracle.moe_finalize(d["expert_rows"], d["idx"], d["weights"], d["residual"],
                               d["gamma"], 0.0, d["expert_ids"], d["expert_gamma"])
    rows8 = workloads.to_bf16_bits(f32(d["expert_rows"]) * 8)
    b, _ = oracle.moe_finalize(rows8, d["idx"], d["weights"], d["residual"], d["gamma"], 0.0,
                               d["expert_ids"], d["expert_gamma"])
    assert np.array_equal(a, b)  # with eps = 0 the scale cancels exactly


# ----------------------------------------------------------------------------- expert-parallel split


def _ep_split(d, G):
    """Per-rank idx arrays: expert e lives on rank e % G; other ranks' slots are -1."""
    owner = d["expert_ids"] % G
    return [np.where(owner == g, d["idx"], -1).astype(np.int32) for g in range(G)]


@pytest.mark.parametrize("per_expert", [False, True])
def test_ep_one_rank_is_the_finalize(per_expert):
    d = workloads.make_finalize_inputs(9, 520, E=8, k=4, seed=40, per_expert=per_expert)
    kw = dict(expert_ids=d["expert_ids"], expert_gamma=d["expert_gamma"]) if per_expert else {}
    part = oracle.moe_finalize_ep_partial(d["expert_rows"], d["idx"], d["weights"], d["eps"], **kw)
    r, o = oracle.moe_finalize_ep_combine(part[None], d["residual"], d["gamma"], d["eps"])
    r_ref, o_ref = oracle.moe_finalize(d["expert_rows"], d["idx"], d["weights"], d["residual"],
                                       d["gamma"], d["eps"], **kw)
    assert np.array_equal(r, r_ref) and np.array_equal(o, o_ref)


def test_ep_all_slots_remote_give_zero():
    d = workloads.make_finalize_inputs(5, 64, E=8, k=3, seed=41)
    part = oracle.moe_finalize_ep_partial(d["expert_rows"], np.full_like(d["idx"], -1),
                                          d["weights"], d["eps"])
    assert np.array_equal(part.view(np.uint32), np.zeros_like(part).view(np.uint32))  # +0


@pytest.mark.parametrize("G", [2, 3, 8])
def test_ep_exact_integers_match_the_finalize(G):
    # small-integer rows, power-of-two weights, integer residual: every partial sum and every
    # combine add is exact, so any rank split gives the single-GPU residual_out bit for bit
    rng = np.random.default_rng(42 + G)
    d = workloads.make_finalize_inputs(12, 256, E=16, k=6, seed=42 + G)
    d["expert_rows"] = workloads.to_bf16_bits(rng.integers(-8, 9, d["expert_rows"].shape)
                                              .astype(np.float32))
    d["weights"] = (2.0 ** -rng.integers(0, 4, d["weights"].shape)).astype(np.float32)
    d["residual"] = rng.integers(-16, 17, d["residual"].shape).astype(np.float32)
    parts = np.stack([oracle.moe_finalize_ep_partial(d["expert_rows"], i, d["weights"], d["eps"])
                      for i in _ep_split(d, G)])
    r, o = oracle.moe_finalize_ep_combine(parts, d["residual"], d["gamma"], d["eps"])
    closed = d["residual"].astype(np.float64) + (d["weights"][..., None].astype(np.float64) *
                                                 f32(d["expert_rows"])[d["idx"]]).sum(axis=1)
    assert np.array_equal(r, closed.astype(np.float32))
    r_ref, o_ref = oracle.moe_finalize(d["expert_rows"], d["idx"], d["weights"], d["residual"],
                                       d["gamma"], d["eps"])
    assert np.array_equal(r, r_ref) and np.array_equal(o, o_ref)


def test_ep_brute_force_partials_and_combine():
    G = 4
    d = workloads.make_finalize_inputs(10, 384, E=16, k=8, seed=43)
    X = f32(d["expert_rows"]).astype(np.float64)
    w = d["weights"].astype(np.float64)
    parts = []
    for g, ig in enumerate(_ep_split(d, G)):
        p = oracle.moe_finalize_ep_partial(d["expert_rows"], ig, d["weights"], d["eps"])
        local = (ig >= 0)[..., None]
        terms = np.where(local, w[..., None] * X[np.maximum(ig, 0)], 0.0)
        exact = terms.sum(axis=1)
        assert np.all(np.abs(p - exact) <= 9 * U32 * 2 * np.abs(terms).sum(axis=1) + 1e-30), g
        parts.append(p)
    r, o = oracle.moe_finalize_ep_combine(np.stack(parts), d["residual"], d["gamma"], d["eps"])
    terms = w[..., None] * X[d["idx"]]
    exact = d["residual"].astype(np.float64) + terms.sum(axis=1)
    bound = (8 + G + 2) * U32 * 2 * (np.abs(terms).sum(axis=1) + np.abs(d["residual"]))
    assert np.all(np.abs(r - exact) <= bound)
    assert _close_bf16(o, _rmsnorm_bits(r, d["gamma"], d["eps"]))


def test_ep_combine_adds_ranks_in_ascending_order():
    # partials 1, 2^-24, 2^-24 (ranks 0, 1, 2), residual 0: in rank order (0 + 1) + 2^-24 is a
    # tie that rounds to even, 1, and so does the next add: residual_out is exactly 1.  The
    # reverse order would give 2^-23 + 1 = 1 + 2^-23.
    T, H = 2, 8
    parts = np.stack([np.ones((T, H)), np.full((T, H), 2.0 ** -24), np.full((T, H), 2.0 ** -24)])
    r, _ = oracle.moe_finalize_ep_combine(parts.astype(np.float32), np.zeros((T, H), np.float32),
                                          workloads.to_bf16_bits(np.ones(H, np.float32)), 1e-6)
    assert np.array_equal(r, np.ones((T, H), np.float32))


def test_ep_remote_slots_skip_the_per_expert_norm():
    # a remote slot's expert id and weight are never read: garbage there changes nothing
    d = workloads.make_finalize_inputs(6, 256, E=8, k=4, seed=44, per_expert=True)
    ig = _ep_split(d, 2)[0]
    eids = np.where(ig >= 0, d["expert_ids"], 10 ** 6).astype(np.int32)
    w = np.where(ig >= 0, d["weights"], np.nan).astype(np.float32)
    p1 = oracle.moe_finalize_ep_partial(d["expert_rows"], ig, w, d["eps"], eids, d["expert_gamma"])
    p2 = oracle.moe_finalize_ep_partial(d["expert_rows"], ig, d["weights"], d["eps"],
                                        d["expert_ids"], d["expert_gamma"])
    assert np.array_equal(p1, p2)


# ----------------------------------------------------------------------------- MXFP4

E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _mx_decode(q, sc):
    """Values of MXFP4 codes (float64 [T, H])."""
    lo, hi = q & 0xF, q >> 4
    codes = np.stack([lo, hi], axis=-1).reshape(q.shape[0], -1)
    mag = E2M1[codes & 7]
    val = np.where(codes & 8, -mag, mag)
    return val * np.repeat(np.ldexp(1.0, sc.astype(np.int64) - 127), 32, axis=1)


def test_golden_mxfp4_hand_example():
    g = json.load(open(GOLDEN))["mxfp4_quantize"]
    head = [-0.0 if v == "-0" else float(v) for v in g["values_block0_head"]]
    b0 = np.array(head + [0.0] * 16, np.float32)
    x = np.concatenate([b0, b0 * np.float32(2.0 ** -10), np.zeros(32, np.float32)])[None]
    q, sc = oracle.mxfp4_quantize(x)
    want = [int(h, 16) for h in g["expected_block_bytes"]]
    assert q[0, :16].tolist() == want and q[0, 16:32].tolist() == want
    assert q[0, 32:].tolist() == [0] * 16
    assert sc[0].tolist() == g["expected_scales"]


def test_golden_rmsnorm_mxfp4_hand_example():
    g = json.load(open(GOLDEN))["rmsnorm_mxfp4_quantize"]
    H = g["H"]
    x = workloads.to_bf16_bits(np.tile([1.0, -1.0], H // 2).astype(np.float32))[None]
    for gam, key in ((1.0, "expected_scale_gamma1"), (0.5, "expected_scale_gamma_half")):
        q, sc = oracle.rmsnorm_mxfp4_quantize(x, workloads.to_bf16_bits(np.full(H, gam, np.float32)),
                                              g["eps"])
        assert q[0].tolist() == [int(g["expected_byte"], 16)] * (H // 2)
        assert sc[0].tolist() == [g[key]]


def _nearest_ok(v, dec, sc):
    """Every decoded value is the nearest E2M1 point of v / X (|v / X| above 6 saturates),
    ties to the even code, and X = 2^(floor(log2(max|v|)) - 2) per block."""
    T, H = v.shape
    blocks = np.abs(v.astype(np.float64)).reshape(T, H // 32, 32).max(axis=-1)
    m, e = np.frexp(blocks)
    want = np.where(blocks == 0, 0, np.clip(e - 1 - 2 + 127, 0, 254))
    assert np.array_equal(sc, want.astype(np.uint8))
    X = np.repeat(np.ldexp(1.0, sc.astype(np.int64) - 127), 32, axis=1)
    r = np.abs(v.astype(np.float64)) / X
    d = np.abs(r[..., None] - E2M1)                     # distance to each grid point
    best = d.min(axis=-1, keepdims=True)
    cand = (d == best)
    even = cand & (np.arange(8) % 2 == 0)
    pick = np.where(even.any(axis=-1), np.argmax(even, axis=-1), np.argmax(cand, axis=-1))
    pick = np.where(r >= 6, 7, pick)
    assert np.array_equal(np.abs(dec) / X, E2M1[pick])
    assert np.array_equal(np.signbit(dec), np.signbit(v))


@pytest.mark.parametrize("T,H,spread", [(3, 64, 1.0), (5, 256, 30.0), (2, 4096, 1e-20), (4, 96, 1e20)])
def test_mxfp4_is_the_nearest_grid_point(T, H, spread):
    rng = np.random.default_rng(50 + H)
    x = (rng.standard_normal((T, H)) * spread).astype(np.float32)
    x[:, 5] = -0.0
    x[0, 32:64] = 0.0                                   # an all-zero block
    q, sc = oracle.mxfp4_quantize(x)
    _nearest_ok(x, _mx_decode(q, sc), sc)


def test_mxfp4_scale_equivariance_and_sign_symmetry():
    rng = np.random.default_rng(51)
    x = rng.standard_normal((4, 128)).astype(np.float32)
    q, sc = oracle.mxfp4_quantize(x)
    q2, sc2 = oracle.mxfp4_quantize(x * np.float32(2.0 ** 7))
    assert np.array_equal(q, q2) and np.array_equal(sc2.astype(int), sc.astype(int) + 7)
    qn, scn = oracle.mxfp4_quantize(-x)
    assert np.array_equal(qn, q ^ 0x88) and np.array_equal(scn, sc)


def test_rmsnorm_mxfp4_scale_invariance_and_brute_force():
    d = workloads.make_gated_inputs(6, 512, seed=52)
    x, gamma = d["x"], d["gamma"]
    q, sc = oracle.rmsnorm_mxfp4_quantize(x, gamma, 0.0)
    # RMSNorm with eps = 0 is invariant under x -> 2^m x, so the codes are unchanged
    q2, sc2 = oracle.rmsnorm_mxfp4_quantize(workloads.to_bf16_bits(f32(x) * np.float32(8.0)), gamma,
                                            0.0)
    assert np.array_equal(q, q2) and np.array_equal(sc, sc2)
    # against torch's float64 rms_norm: the decoded value is within half a grid step (or the
    # saturation) of the normalised value
    xt = torch.from_numpy(f32(x).astype(np.float64))
    y = torch.nn.functional.rms_norm(xt, (512,), weight=torch.from_numpy(
        f32(gamma).astype(np.float64)), eps=1e-6).numpy()
    q, sc = oracle.rmsnorm_mxfp4_quantize(x, gamma, 1e-6)
    dec = _mx_decode(q, sc)
    X = np.repeat(np.ldexp(1.0, sc.astype(np.int64) - 127), 32, axis=1)
    step = np.where(np.abs(y) / X < 2, 0.5, np.where(np.abs(y) / X < 4, 1.0, 2.0)) * X
    assert np.all((np.abs(dec - y) <= 0.5 * step * 1.0001) | (np.abs(y) / X > 6))


def test_rmsnorm_f32_mxfp4_agrees_with_the_bf16_form_on_bf16_values():
    # bf16 values widen exactly, so the fp32-row form must give the same codes; and on rows of
    # +-c it gives the saturated closed form of the golden example at any scale c
    d = workloads.make_gated_inputs(5, 1024, seed=53)
    q1, s1 = oracle.rmsnorm_mxfp4_quantize(d["x"], d["gamma"], 1e-6)
    q2, s2 = oracle.rmsnorm_f32_mxfp4_quantize(f32(d["x"]), d["gamma"], 1e-6)
    assert np.array_equal(q1, q2) and np.array_equal(s1, s2)
    g = json.load(open(GOLDEN))["rmsnorm_mxfp4_quantize"]
    r = np.tile([3.0, -3.0], 16).astype(np.float32)[None] * np.float32(1024)
    q, sc = oracle.rmsnorm_f32_mxfp4_quantize(r, workloads.to_bf16_bits(np.ones(32, np.float32)),
                                              0.0)
    # eps = 0: |y| = 1 exactly, floor(log2) = 0, e = -2, y / 2^-2 = 4: code 6 (and 14)
    assert q[0].tolist() == [0xE6] * 16 and sc[0].tolist() == [125]
    q, sc = oracle.rmsnorm_f32_mxfp4_quantize(r, workloads.to_bf16_bits(np.ones(32, np.float32)),
                                              g["eps"])
    assert q[0].tolist() == [0xE6] * 16 and sc[0].tolist() == [125]  # eps 1e-6 is invisible at 3072


# ----------------------------------------------------------------------------- gated


def test_gated_brute_force_with_scipy_expit():
    d = workloads.make_gated_inputs(7, 264, seed=23)
    r, o = oracle.gated_residual_rmsnorm(d["x"], d["gate"], d["residual"], d["gamma"], d["eps"])
    exact = d["residual"].astype(np.float64) + expit(f32(d["gate"]).astype(np.float64)) * \
        f32(d["x"]).astype(np.float64)
    # one rounding to float32 (half an ulp), plus a sliver for the float64 steps
    assert np.all(np.abs(r - exact) <= 0.5001 * U32 * 2 * np.abs(exact) + 1e-30)
    assert _close_bf16(o, _rmsnorm_bits(r, d["gamma"], d["eps"]))


def test_gated_gate_zero_is_half():
    # sigmoid(0) = 1/2 exactly, and x/2 is exact, so residual_out = float32 add.
    d = workloads.make_gated_inputs(5, 128, seed=24)
    zero = np.zeros_like(d["gate"])
    r, _ = oracle.gated_residual_rmsnorm(d["x"], zero, d["residual"], d["gamma"], d["eps"])
    assert np.array_equal(r, d["residual"] + np.float32(0.5) * f32(d["x"]))


def test_gated_large_gate_is_add_rmsnorm():
    d = workloads.make_gated_inputs(5, 512, seed=25)
    g40 = workloads.to_bf16_bits(np.full(d["gate"].shape, 40.0, np.float32))
    r, o = oracle.gated_residual_rmsnorm(d["x"], g40, d["residual"], d["gamma"], d["eps"])
    plain = d["residual"] + f32(d["x"])
    # sigmoid(40) = 1 - 4.2e-18: within one float32 ulp of the plain add
    assert np.all(np.abs(r - plain) <= U32 * 2 * np.abs(plain))
    assert _close_bf16(o, _rmsnorm_bits(plain, d["gamma"], d["eps"]))


def test_gated_very_negative_gate_keeps_residual():
    d = workloads.make_gated_inputs(4, 256, seed=26)
    res = d["residual"].copy()
    res[np.abs(res) < 1e-3] = 1e-3  # sigmoid(-30)*|x| < 4e-13 is below half an ulp here
    gm30 = workloads.to_bf16_bits(np.full(d["gate"].shape, -30.0, np.float32))
    r, _ = oracle.gated_residual_rmsnorm(d["x"], gm30, res, d["gamma"], d["eps"])
    assert np.array_equal(r, res)


# ----------------------------------------------------------------------------- gated, dual output


def test_gated_next_brute_force():
    d = workloads.make_gated_inputs(6, 520, seed=27, dual=True)
    r, o, on = oracle.gated_residual_next_rmsnorm(d["x"], d["gate"], d["residual"], d["gamma"],
                                                  d["gamma_next"], d["eps"])
    exact = d["residual"].astype(np.float64) + expit(f32(d["gate"]).astype(np.float64)) * \
        f32(d["x"]).astype(np.float64)
    assert np.all(np.abs(r - exact) <= 0.5001 * U32 * 2 * np.abs(exact) + 1e-30)
    assert _close_bf16(o, _rmsnorm_bits(r, d["gamma"], d["eps"]))
    assert _close_bf16(on, _rmsnorm_bits(r, d["gamma_next"], d["eps"]))


def test_gated_next_equal_gammas_give_equal_outputs():
    d = workloads.make_gated_inputs(4, 256, seed=28, dual=True)
    r, o, on = oracle.gated_residual_next_rmsnorm(d["x"], d["gate"], d["residual"], d["gamma"],
                                                  d["gamma"], d["eps"])
    assert np.array_equal(o, on)


def test_gated_next_double_gamma_doubles_exactly():
    # gamma_next = 2 * gamma (exact in bf16): every out_next value is exactly twice out's
    d = workloads.make_gated_inputs(4, 256, seed=29, dual=True)
    g2 = workloads.to_bf16_bits(2.0 * f32(d["gamma"]))
    r, o, on = oracle.gated_residual_next_rmsnorm(d["x"], d["gate"], d["residual"], d["gamma"], g2,
                                                  d["eps"])
    assert np.array_equal(f32(on), np.float32(2) * f32(o))


def test_gated_next_gate_zero_and_unit_gamma_next():
    # gate = 0: residual_out = residual + x/2 exactly; gamma_next = 1: the RMS of out_next is
    # sqrt(ms / (ms + eps)) up to bf16 rounding (2^-9 relative per element)
    d = workloads.make_gated_inputs(5, 1024, seed=30, dual=True)
    zero = np.zeros_like(d["gate"])
    one = workloads.to_bf16_bits(np.ones(1024, np.float32))
    r, o, on = oracle.gated_residual_next_rmsnorm(d["x"], zero, d["residual"], d["gamma"], one,
                                                  d["eps"])
    assert np.array_equal(r, d["residual"] + np.float32(0.5) * f32(d["x"]))
    ms = (r.astype(np.float64) ** 2).mean(axis=1)
    rms = np.sqrt((f32(on).astype(np.float64) ** 2).mean(axis=1))
    assert np.allclose(rms, np.sqrt(ms / (ms + d["eps"])), rtol=2.0 ** -8)


# ----------------------------------------------------------------------------- per-head


def _bf_per_head(d):
    x = f32(d["x"]).astype(np.float64)
    scale = 1.0 / np.sqrt((x * x).mean(axis=2, keepdims=True) + d["eps"])
    return x * scale * f32(d["gamma"]).astype(np.float64) * expit(f32(d["gate"]).astype(np.float64))


def test_per_head_brute_force():
    d = workloads.make_per_head_inputs(5, 3, 64, seed=27)  # T, heads and D all differ
    o = oracle.rmsnorm_sigmoid_gate(d["x"], d["gate"], d["gamma"], d["eps"])
    assert _close_bf16(o, torch_bf16_bits(_bf_per_head(d)))


def test_per_head_large_gate_is_rms_norm_over_head_dim():
    d = workloads.make_per_head_inputs(6, 4, 64, seed=28)
    g40 = workloads.to_bf16_bits(np.full(d["gate"].shape, 40.0, np.float32))
    o = oracle.rmsnorm_sigmoid_gate(d["x"], g40, d["gamma"], d["eps"])
    want = _rmsnorm_bits(f32(d["x"]).astype(np.float64), d["gamma"], d["eps"])
    assert _close_bf16(o, want)


def test_per_head_unit_gamma_rms_is_one():
    d = workloads.make_per_head_inputs(4, 8, 64, seed=29)
    ones = workloads.to_bf16_bits(np.ones(64, np.float32))
    g40 = workloads.to_bf16_bits(np.full(d["gate"].shape, 40.0, np.float32))
    o = oracle.rmsnorm_sigmoid_gate(d["x"], g40, ones, 0.0)
    rms = np.sqrt((f32(o).astype(np.float64) ** 2).mean(axis=2))
    assert np.all(np.abs(rms - 1.0) <= 2.0 ** -9)


def test_per_head_heads_are_independent():
    # Permuting the heads of x and gate permutes the output heads: the norm runs over D only.
    d = workloads.make_per_head_inputs(3, 5, 64, seed=30)
    o = oracle.rmsnorm_sigmoid_gate(d["x"], d["gate"], d["gamma"], d["eps"])
    p = np.array([3, 0, 4, 1, 2])
    o2 = oracle.rmsnorm_sigmoid_gate(d["x"][:, p], d["gate"][:, p], d["gamma"], d["eps"])
    assert np.array_equal(o[:, p], o2)


# ----------------------------------------------------------------------------- routing


def test_golden_route_hand_example():
    g = json.load(open(GOLDEN))["moe_route"]
    eids, w, idx, perm, off = oracle.moe_route(np.array(g["logits"], np.float32), g["k"])
    assert eids.tolist() == g["expected_expert_ids"]
    assert w.tolist() == g["expected_weights"]
    assert idx.tolist() == g["expected_idx"]
    assert perm.tolist() == g["expected_perm"]
    assert off.tolist() == g["expected_offsets"]


@pytest.mark.parametrize("T,E,k", [(1, 4, 1), (5, 8, 2), (33, 64, 8), (100, 256, 8), (7, 130, 16),
                                   (3, 16, 16)])
def test_route_matches_numpy_sorts_and_scipy_softmax(T, E, k):
    rng = np.random.default_rng(300 + T + E + k)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    logits[:, ::5] = np.round(logits[:, ::5])  # plenty of exact ties
    eids, w, idx, perm, off = oracle.moe_route(logits, k)
    want = np.argsort(-logits, axis=1, kind="stable")[:, :k]     # ties: lower id first
    assert np.array_equal(eids, want)
    from scipy.special import softmax
    top = np.take_along_axis(logits, want, axis=1).astype(np.float64)
    ref = softmax(top, axis=1).astype(np.float32)
    assert np.all(np.abs(w.astype(np.float64) - ref) <= np.spacing(ref) * 1.0001)
    assert np.array_equal(perm, np.argsort(eids.ravel(), kind="stable"))
    assert np.array_equal(idx.ravel()[perm], np.arange(T * k))
    assert np.array_equal(off, np.concatenate([[0], np.cumsum(np.bincount(eids.ravel(), minlength=E))]))


def test_route_k_equals_e_is_a_full_softmax():
    rng = np.random.default_rng(310)
    logits = rng.standard_normal((6, 12)).astype(np.float32)
    eids, w, _, _, off = oracle.moe_route(logits, 12)
    assert np.array_equal(np.sort(eids, axis=1), np.tile(np.arange(12), (6, 1)))
    full = np.exp(logits.astype(np.float64) - logits.max(axis=1, keepdims=True))
    full /= full.sum(axis=1, keepdims=True)
    assert np.allclose(w, np.take_along_axis(full, eids, axis=1), rtol=2e-7, atol=0)
    assert np.array_equal(off, np.arange(13) * 6)
