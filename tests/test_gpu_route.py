"""Parity of the GPU routing producer (mf_moe_route, through the C ABI) with the CPU oracle.

Bars:
  - expert_ids, idx, perm and expert_offsets: bit-identical (integer results with one correct
    answer: the top-k with ties to the lower id, and the stable sort of the slots by expert);
  - weights: the GPU computes w_j = expf(l_j - l_0) / sum_i expf(l_i - l_0) in fp32, the
    oracle in float64 rounded once to fp32.  With d_j = |l_j - l_0| (d_j * 2^-24 bounds the
    error the rounded fp32 difference puts into the exponential), expf within 2 ulp, k - 1
    additions of positive terms, one division and the oracle's own rounding, the relative
    difference is at most
        (k + 13 + d_j + sum_i w_i d_i) * 2^-24
    plus 2^-126 absolute for weights that fall below the fp32 normal range (zero weights,
    from -inf or far-off logits, carry no relative term).
Each case prints its name and sizes before it runs.
"""
import json
import os

import numpy as np
import pytest
import torch

import finalize_residual_rmsnorm_amd as mf
import oracle
import workloads
from tests import refs
from tests.helpers import bf16_ulp_diff

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_examples.json")


def say(msg):
    print(msg, flush=True)


def route_gpu(logits, k, workspace=None):
    out = mf.mf_moe_route(torch.from_numpy(np.ascontiguousarray(logits)).to(DEV), k,
                          workspace=workspace)
    torch.cuda.synchronize()
    return tuple(t.cpu().numpy() for t in out)


def weight_bound(logits, eids, w_ref):
    T, k = eids.shape
    l = np.take_along_axis(logits.astype(np.float64), eids, axis=1)
    wr = np.abs(w_ref.astype(np.float64))
    with np.errstate(invalid="ignore"):
        d = np.where(wr > 0, np.abs(l - l[:, :1]), 0.0)   # zero weights carry no error
    den = (k - 1) + 4 * wr.sum(axis=1, keepdims=True) + (wr * d).sum(axis=1, keepdims=True)
    rel = (4 + d + den + 2) * 2.0 ** -24
    return rel * wr + 2.0 ** -126


def check_route(logits, k, name, workspace=None):
    T, E = logits.shape
    say(f"{name}: T={T} E={E} k={k} workspace={mf.mf_moe_route_workspace_bytes(T, E, k)} B")
    ge, gw, gi, gp, go = route_gpu(logits, k, workspace)
    oe, ow, oi, op, oo = oracle.moe_route(logits, k)
    assert np.array_equal(ge, oe), f"expert_ids differ at {np.argwhere(ge != oe)[:5].tolist()}"
    assert np.array_equal(go, oo), "expert_offsets differ"
    assert np.array_equal(gp, op), "perm differs"
    assert np.array_equal(gi, oi), "idx differs"
    err = np.abs(gw.astype(np.float64) - ow.astype(np.float64))
    bound = weight_bound(logits, oe, ow)
    assert np.all(err <= bound), f"{(err > bound).sum()} weights beyond the bound"
    say(f"    weights bit-identical fraction {(gw == ow).mean():.5f}")
    return ge, gw, gi, gp, go


def test_route_golden_hand_example():
    g = json.load(open(GOLDEN))["moe_route"]
    logits = np.array(g["logits"], np.float32)
    say("route golden: T=2 E=4 k=2")
    ge, gw, gi, gp, go = route_gpu(logits, g["k"])
    assert ge.tolist() == g["expected_expert_ids"]
    assert gw.tolist() == g["expected_weights"]
    assert gi.tolist() == g["expected_idx"]
    assert gp.tolist() == g["expected_perm"]
    assert go.tolist() == g["expected_offsets"]


@pytest.mark.parametrize("name", ["moe_route_prefill", "moe_route_decode"])
def test_route_named_workloads(name):
    d = workloads.make_inputs(name)
    check_route(d["logits"], d["k"], name)


ROUTE_SHAPES = [
    # (T, E, k, bf16-valued logits): one expert; every logits-per-lane instantiation, on the
    # two-launch path of small calls and the three-launch path
    # (E <= 64, 128, 256, 512, 1024); k from 1 to 16 and k == E; ragged T around the
    # 16-wave blocks and the 64-slot chunks; T large enough for 16 tokens per wave.
    (1, 1, 1, False), (3, 8, 2, False), (37, 8, 8, True), (64, 130, 16, False),
    (300, 64, 1, True), (1000, 256, 8, True), (4097, 16, 4, False), (9000, 5, 3, True),
    (40, 1024, 16, False), (8200, 33, 2, True), (5, 513, 16, False), (2, 65, 1, False),
    (17, 16, 16, True), (100000, 256, 8, False), (70001, 1024, 16, True), (65537, 64, 6, True),
    # either side of the two-launch path's limits (a per-block count table of at most 8192
    # entries: 16 tokens per block below T = 4096; at most 16384 slots)
    (512, 256, 8, False), (600, 256, 8, False), (128, 1024, 16, True), (129, 1024, 16, True),
    (2048, 32, 1, True), (4096, 16, 4, False),
]


@pytest.mark.parametrize("T,E,k,q", ROUTE_SHAPES)
def test_route_shapes(T, E, k, q):
    d = workloads.make_route_inputs(T, E, k, seed=400 + T + E + k, bf16_logits=q)
    check_route(d["logits"], k, "route shape")


def _random_route_cases(n=12, seed=20261211):
    """Seeded random (T, E, k, bf16-valued logits): T from 1 to 20000 and E from 1 to 1024
    (log-uniform), k from 1 to min(E, 16)."""
    g = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        T = int(np.exp(g.uniform(0.0, np.log(20000.0))))
        E = int(np.exp(g.uniform(0.0, np.log(1024.0))))
        k = int(g.integers(1, min(E, 16) + 1))
        cases.append((T, E, k, i % 2 == 1))
    return cases


@pytest.mark.parametrize("T,E,k,q", _random_route_cases())
def test_route_random_shapes(T, E, k, q):
    d = workloads.make_route_inputs(T, E, k, seed=450 + T + E + k, bf16_logits=q)
    check_route(d["logits"], k, "route random shape")


def test_route_special_values():
    # every logit equal (all ties), signed zeros, -inf entries and huge magnitudes
    E, k = 96, 8
    rows = [np.zeros(E), np.full(E, -3.5), np.where(np.arange(E) % 2, 0.0, -0.0),
            np.where(np.arange(E) < 90, -np.inf, 1.0), np.linspace(-1e30, 1e30, E),
            np.where(np.arange(E) % 7 == 0, 2.0, 1.0)]
    logits = np.array(rows * 11, np.float32)
    check_route(logits, k, "route special values")


def test_route_zero_tokens_writes_offsets():
    say("route T=0 E=16 k=2")
    ge, gw, gi, gp, go = route_gpu(np.zeros((0, 16), np.float32), 2)
    assert ge.shape == (0, 2) and gp.shape == (0,)
    assert np.array_equal(go, np.zeros(17, np.int32))


def test_route_workspace_reuse_and_garbage():
    # the workspace's contents on entry do not matter; one workspace serves calls in turn
    ws = torch.full((mf.mf_moe_route_workspace_bytes(5000, 256, 8),), 0xFF, dtype=torch.uint8,
                    device=DEV)
    a = workloads.make_route_inputs(5000, 256, 8, seed=501)["logits"]
    b = workloads.make_route_inputs(333, 200, 4, seed=502, bf16_logits=True)["logits"]
    check_route(a, 8, "route workspace 1st", workspace=ws)
    check_route(b, 4, "route workspace 2nd (smaller)", workspace=ws)


def test_route_per_token_results_do_not_depend_on_the_batch():
    d = workloads.make_route_inputs(6000, 256, 8, seed=503)["logits"]
    say("route batch invariance: 6000 tokens vs tokens 1234..1300 alone")
    ge, gw, _, _, _ = route_gpu(d, 8)
    se, sw, _, _, _ = route_gpu(d[1234:1301], 8)
    assert np.array_equal(ge[1234:1301], se)
    assert np.array_equal(gw[1234:1301], sw)


def test_route_is_deterministic():
    d = workloads.make_route_inputs(20000, 128, 8, seed=504, bf16_logits=True)["logits"]
    say("route determinism: T=20000 E=128 k=8, twice")
    r1 = route_gpu(d, 8)
    r2 = route_gpu(d, 8)
    for a, b in zip(r1, r2):
        assert np.array_equal(a, b)


def test_route_then_finalize_end_to_end():
    """GPU routing feeds the GPU finalize: idx and weights never leave the GPU."""
    T, E, k, H = 512, 64, 8, 1024
    logits = workloads.make_route_inputs(T, E, k, seed=505)["logits"]
    fin = workloads.make_finalize_inputs(T, H, E, k, seed=506)  # rows, residual, gamma
    say(f"route -> finalize: T={T} E={E} k={k} H={H}")
    eids, w, idx, perm, off = mf.mf_moe_route(torch.from_numpy(logits).to(DEV), k)
    rows = torch.from_numpy(fin["expert_rows"].view(np.int16)).view(torch.bfloat16).to(DEV)
    res = torch.from_numpy(fin["residual"]).to(DEV)
    gamma = torch.from_numpy(fin["gamma"].view(np.int16)).view(torch.bfloat16).to(DEV)
    out, r = mf.mf_moe_finalize(rows, idx, w, res, gamma, fin["eps"])
    torch.cuda.synchronize()
    oe, ow, oi, op, oo = oracle.moe_route(logits, k)
    r_ref, o_ref = oracle.moe_finalize(fin["expert_rows"], oi, ow, fin["residual"], fin["gamma"],
                                       fin["eps"])
    assert np.array_equal(idx.cpu().numpy(), oi)
    # residual_out: the weights' bound times |x|, plus both fp32 FMA chains' rounding
    x = workloads.bf16_bits_to_f32(fin["expert_rows"]).astype(np.float64)[oi]   # [T, k, H]
    wb = weight_bound(logits, oe, ow)[:, :, None]
    acc = np.abs(ow.astype(np.float64)[:, :, None] * x).sum(axis=1)
    rr = r_ref.astype(np.float64)
    r_tol = (wb * np.abs(x)).sum(axis=1) + (2 * k + 2) * 2.0 ** -24 * (
        acc + np.abs(fin["residual"]) + np.abs(rr))
    rg = r.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(rg - rr) <= r_tol)
    say(f"    residual_out bit-identical fraction {(rg == rr).mean():.5f}")
    # out: within one bf16 ulp of the oracle's RMSNorm of the GPU's own residual_out (which has
    # just passed the bound above), and at least 99% bit-identical
    og = out.view(torch.int16).cpu().numpy().view(np.uint16)
    d = bf16_ulp_diff(og, refs.rmsnorm_of(r.cpu().numpy(), fin["gamma"], fin["eps"]))
    assert d.max() <= 1, f"max bf16 ulp diff {d.max()}"
    assert (d == 0).mean() >= 0.99
