"""Parity of the expert-parallel finalize split on the GPU (through the C ABI) with the oracle.

One GPU stands in for G ranks: expert e lives on rank e % G, each rank's partial marks the
other ranks' slots -1, and the owner's combine reads the G partials from one [G, T, H] buffer.

Bars:
  - plain partials and every combine's residual_out: bit-identical (an fp32 FMA chain in
    fixed order, then fp32 adds in rank order: one correct result each);
  - per-expert partials: |gpu - ref| <= 4e-6 * sum_j |w_j * y_j| (the GPU's fp32 rsqrt and
    the rounded normalised rows against the oracle's float64, about (k + 6) * 2^-24 of the
    terms' magnitude, with margin);
  - bf16 out: within one ulp, >= 99% bit-identical.
Each case prints its name and sizes before it runs.
"""
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


def say(msg):
    print(msg, flush=True)


def up(a, bf16=False):
    a = np.ascontiguousarray(a)
    t = torch.from_numpy(a.view(np.int16) if bf16 else a)
    if bf16:
        t = t.view(torch.bfloat16)
    return t.to(DEV)


def bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def assert_bf16_close(gpu, ref, min_exact=0.99):
    d = bf16_ulp_diff(gpu, ref)
    assert d.max() <= 1, f"max bf16 ulp diff {d.max()}"
    assert (d == 0).mean() >= min_exact, f"bit-identical fraction {(d == 0).mean():.5f}"


def split(d, G):
    owner = d["expert_ids"] % G
    return [np.where(owner == g, d["idx"], -1).astype(np.int32) for g in range(G)]


def partial_gpu(d, idx, per_expert=False, out=None):
    kw = {}
    if per_expert:
        kw = dict(expert_ids=up(d["expert_ids"]), expert_gamma=up(d["expert_gamma"], True))
    return mf.mf_moe_finalize_ep_partial(up(d["expert_rows"], True), up(idx), up(d["weights"]),
                                         d["eps"], partial=out, **kw)


def partial_ref(d, idx, per_expert=False):
    kw = dict(expert_ids=d["expert_ids"], expert_gamma=d["expert_gamma"]) if per_expert else {}
    return oracle.moe_finalize_ep_partial(d["expert_rows"], idx, d["weights"], d["eps"], **kw)


def per_expert_bound(d, idx):
    x = workloads.bf16_bits_to_f32(d["expert_rows"]).astype(np.float64)
    g = workloads.bf16_bits_to_f32(d["expert_gamma"]).astype(np.float64)
    live = idx >= 0
    xs = x[np.maximum(idx, 0)]                                          # [T, k, H]
    inv = 1.0 / np.sqrt((xs * xs).mean(axis=-1, keepdims=True) + d["eps"])
    y = xs * inv * g[d["expert_ids"]]
    terms = np.where(live[..., None], np.abs(d["weights"][..., None] * y), 0.0)
    return 4e-6 * terms.sum(axis=1) + 1e-30


@pytest.mark.parametrize("T,H,k,G,pe", [
    (17, 1024, 8, 2, False), (33, 4104, 9, 3, False), (100, 7168, 8, 8, False),
    (5, 32768, 3, 2, False), (64, 4096, 8, 4, True), (9, 520, 5, 2, True), (300, 2048, 1, 4, False),
    (9, 776, 5, 2, False), (6, 5000, 8, 3, True),
    # the compiled top-8 without per-expert norm: ragged rows, 1 to 4 slots per wave, and every
    # slot local
    (9, 776, 8, 2, False), (5, 4128, 8, 3, False), (4, 12288, 8, 1, False),
    (7, 16384, 8, 2, False), (4, 16384, 8, 1, False), (3, 20480, 8, 2, False),
])
def test_ep_partial_matches_oracle(T, H, k, G, pe):
    say(f"ep partial T={T} H={H} k={k} G={G} per_expert={pe}")
    d = workloads.make_finalize_inputs(T, H, E=max(16, k), k=k, seed=700 + T + H + k, per_expert=pe)
    for g, idx in enumerate(split(d, G)):
        got = partial_gpu(d, idx, pe)
        torch.cuda.synchronize()
        ref = partial_ref(d, idx, pe)
        got = got.cpu().numpy()
        if pe:
            assert np.all(np.abs(got.astype(np.float64) - ref) <= per_expert_bound(d, idx)), g
        else:
            assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), g


def test_ep_partial_all_remote_is_zero():
    d = workloads.make_finalize_inputs(40, 1024, E=8, k=4, seed=710)
    say("ep partial, every slot remote: T=40 H=1024")
    p = torch.full((40, 1024), 7.0, device=DEV)
    partial_gpu(d, np.full_like(d["idx"], -1), out=p)
    torch.cuda.synchronize()
    assert np.array_equal(p.cpu().numpy().view(np.uint32), np.zeros((40, 1024), np.uint32))


@pytest.mark.parametrize("T,H,G", [(1, 8, 1), (7, 520, 3), (300, 7168, 8), (5, 32768, 2),
                                   (2049, 1024, 16), (33, 12288, 5), (7, 776, 3), (4, 20000, 2),
                                   # two slots per wave, two ranks in flight: an odd rank count
                                   # and a single rank end the rotation part-way
                                   (65, 7168, 5), (3, 7168, 1), (10, 6000, 7),
                                   # a live wave whose second slot lies past the row
                                   (9, 6656, 3)])
def test_ep_combine_matches_oracle(T, H, G):
    say(f"ep combine T={T} H={H} G={G}")
    d = workloads.make_ep_combine_inputs(T, H, G, seed=720 + T + H + G)
    out, r = mf.mf_moe_finalize_ep_combine(up(d["partials"]), up(d["residual"]),
                                           up(d["gamma"], True), d["eps"])
    torch.cuda.synchronize()
    r_ref, o_ref = oracle.moe_finalize_ep_combine(d["partials"], d["residual"], d["gamma"],
                                                  d["eps"])
    assert np.array_equal(r.cpu().numpy(), r_ref)
    assert_bf16_close(bits(out), o_ref)


def _random_ep_cases(n, seed, partial):
    """Seeded random shapes: H a multiple of 8 from 8 to 32768 (log-uniform); the partial with k
    from 1 to 16 (every other case the compiled 8) and 1 to 8 ranks, every third case per-expert;
    the combine with 1 to 16 ranks.  Each small enough for the oracle."""
    g = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        H = 8 * int(np.exp(g.uniform(0.0, np.log(4096.0))))
        T = int(np.exp(g.uniform(0.0, np.log(400.0))))
        if partial:
            k = 8 if len(cases) % 2 else int(g.integers(1, 17))
            G = int(g.integers(1, 9))
            if T * k * H <= 6_000_000:
                cases.append((T, H, k, G, len(cases) % 3 == 2))
        else:
            G = int(g.integers(1, 17))
            if T * G * H <= 8_000_000:
                cases.append((T, H, G))
    return cases


@pytest.mark.parametrize("T,H,k,G,pe", _random_ep_cases(12, 20261207, True))
def test_ep_partial_random_shapes(T, H, k, G, pe):
    test_ep_partial_matches_oracle(T, H, k, G, pe)


@pytest.mark.parametrize("T,H,G", _random_ep_cases(10, 20261208, False))
def test_ep_combine_random_shapes(T, H, G):
    say(f"ep combine random shape T={T} H={H} G={G}")
    d = workloads.make_ep_combine_inputs(T, H, G, seed=730 + T + H + G)
    out, r = mf.mf_moe_finalize_ep_combine(up(d["partials"]), up(d["residual"]),
                                           up(d["gamma"], True), d["eps"])
    torch.cuda.synchronize()
    r_ref, o_ref = oracle.moe_finalize_ep_combine(d["partials"], d["residual"], d["gamma"],
                                                  d["eps"])
    assert np.array_equal(r.cpu().numpy(), r_ref)
    # (the bit-identical fraction is asserted only where there are enough elements for it)
    assert_bf16_close(bits(out), o_ref, min_exact=0.99 if T * H >= 4096 else 0.0)


def test_ep_combine_in_place():
    d = workloads.make_ep_combine_inputs(100, 7168, 8, seed=730)
    say("ep combine in place: T=100 H=7168 G=8")
    res = up(d["residual"])
    out, _ = mf.mf_moe_finalize_ep_combine(up(d["partials"]), res, up(d["gamma"], True),
                                           d["eps"], residual_out=res)
    torch.cuda.synchronize()
    r_ref, o_ref = oracle.moe_finalize_ep_combine(d["partials"], d["residual"], d["gamma"],
                                                  d["eps"])
    assert np.array_equal(res.cpu().numpy(), r_ref)
    assert_bf16_close(bits(out), o_ref)


@pytest.mark.parametrize("G", [1, 2, 8])
def test_ep_pipeline_on_one_gpu(G):
    """Every rank's partial into one [G, T, H] buffer, then the combine: bit-identical to the
    oracle's two steps.  With one rank, residual_out is bit-identical to mf_moe_finalize's (the
    same FMA chain, then one add of +0); out is within one bf16 ulp of it (the two kernels need
    not share a launch shape, so their mean squares may be reduced in different orders)."""
    T, H, k = 257, 7168, 8
    d = workloads.make_finalize_inputs(T, H, E=64, k=k, seed=740 + G)
    say(f"ep pipeline T={T} H={H} k={k} G={G}")
    parts = torch.empty((G, T, H), dtype=torch.float32, device=DEV)
    idxs = split(d, G)
    for g, idx in enumerate(idxs):
        partial_gpu(d, idx, out=parts[g])
    out, r = mf.mf_moe_finalize_ep_combine(parts, up(d["residual"]), up(d["gamma"], True),
                                           d["eps"])
    torch.cuda.synchronize()
    ref_parts = np.stack([partial_ref(d, idx) for idx in idxs])
    assert np.array_equal(parts.cpu().numpy(), ref_parts)
    r_ref, o_ref = oracle.moe_finalize_ep_combine(ref_parts, d["residual"], d["gamma"], d["eps"])
    assert np.array_equal(r.cpu().numpy(), r_ref)
    assert_bf16_close(bits(out), o_ref)
    out1, r1 = mf.mf_moe_finalize(up(d["expert_rows"], True), up(d["idx"]), up(d["weights"]),
                                  up(d["residual"]), up(d["gamma"], True), d["eps"])
    torch.cuda.synchronize()
    if G == 1:
        assert torch.equal(r, r1)
        assert_bf16_close(bits(out), bits(out1))
    else:
        # another grouping of the same sum: within the fp32 rounding of the terms
        x = workloads.bf16_bits_to_f32(d["expert_rows"]).astype(np.float64)[d["idx"]]
        mag = np.abs(d["weights"][..., None] * x).sum(axis=1) + np.abs(d["residual"])
        err = np.abs(r.cpu().numpy().astype(np.float64) - r1.cpu().numpy())
        assert np.all(err <= (2 * k + G + 2) * 2.0 ** -24 * mag)


@pytest.mark.parametrize("G", [1, 3])
def test_ep_pipeline_per_expert(G):
    """Per-expert partials of G simulated ranks, then the combine.  The normalised rows make the
    fp32 result non-unique: residual_out is held to the per-expert finalize's bar against the
    oracle's two steps, and out to one bf16 ulp of the oracle's RMSNorm of the GPU's own
    residual_out."""
    T, H, k = 65, 4096, 8
    d = workloads.make_finalize_inputs(T, H, E=32, k=k, seed=750 + G, per_expert=True,
                                       residual_std=2.0)
    say(f"ep pipeline per-expert T={T} H={H} k={k} G={G}")
    parts = torch.empty((G, T, H), dtype=torch.float32, device=DEV)
    idxs = split(d, G)
    for g, idx in enumerate(idxs):
        partial_gpu(d, idx, per_expert=True, out=parts[g])
    out, r = mf.mf_moe_finalize_ep_combine(parts, up(d["residual"]), up(d["gamma"], True),
                                           d["eps"])
    torch.cuda.synchronize()
    ref_parts = np.stack([partial_ref(d, idx, per_expert=True) for idx in idxs])
    r_ref, _ = oracle.moe_finalize_ep_combine(ref_parts, d["residual"], d["gamma"], d["eps"])
    rg = r.cpu().numpy()
    err = np.abs(rg.astype(np.float64) - r_ref)
    assert np.all(err <= 1e-6 + 1e-5 * np.abs(r_ref.astype(np.float64)))
    # the combine step alone is exact: the oracle's combine of the GPU's own partials
    r_own, _ = oracle.moe_finalize_ep_combine(parts.cpu().numpy(), d["residual"], d["gamma"],
                                              d["eps"])
    assert np.array_equal(rg, r_own)
    assert_bf16_close(bits(out), refs.rmsnorm_of(rg, d["gamma"], d["eps"]))


def test_ep_partial_workload_full_size():
    d = refs.named("finalize_ep_partial")
    say(f"ep partial workload T=16384 H=7168 k=8, rank 0 of 8: {(d['idx'] >= 0).mean():.3f} of slots local")
    got = partial_gpu(d, d["idx"])
    torch.cuda.synchronize()
    ref = partial_ref(d, d["idx"])
    assert np.array_equal(got.cpu().numpy().view(np.uint32), ref.view(np.uint32))


def test_ep_combine_workload_full_size():
    d = workloads.make_inputs("finalize_ep_combine")
    say("ep combine workload T=2048 H=7168 G=8")
    out, r = mf.mf_moe_finalize_ep_combine(up(d["partials"]), up(d["residual"]),
                                           up(d["gamma"], True), d["eps"])
    torch.cuda.synchronize()
    r_ref, o_ref = oracle.moe_finalize_ep_combine(d["partials"], d["residual"], d["gamma"],
                                                  d["eps"])
    assert np.array_equal(r.cpu().numpy(), r_ref)
    assert_bf16_close(bits(out), o_ref)
