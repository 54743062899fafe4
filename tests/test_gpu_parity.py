"""Parity of the HIP path (through the C ABI) with the CPU oracle, on the GPU.

Bars (from the finalize's determinism requirement and the stated tolerances):
  - plain finalize residual_out: bit-identical to the oracle (the fp32 FMA chain in fixed
    order has one correct result);
  - per-expert and gated residual_out: |gpu - ref| <= 1e-6 + 1e-5 * |ref| (rsqrt / exp
    rounding makes the fp32 result non-unique), with a floor on the bit-identical fraction;
  - bf16 outputs: within one bf16 ulp (two neighbours are both correct near a rounding
    midpoint) and at least 99% bit-identical.  Where residual_out is unique (the plain
    finalize) the reference is the oracle's out.  Where it is not, the reference is the
    oracle's final RMSNorm of the GPU's own residual_out (tests/refs.py), which has itself
    just passed the residual bar: the output step is then held to one ulp on its own, and
    no residual tolerance leaks into the bf16 bar;
  - index handling: exact (covered by the bit-identical residual_out).
The named finalize workloads take their idx and weights from the oracle's routing of their
router logits (tests/refs.py).  Each case prints its name and launch shape before it runs.
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


def assert_fp32_tol(gpu, ref, min_exact):
    """The non-unique fp32 residual: within 1e-6 + 1e-5 |ref| everywhere, and at least
    min_exact of it bit-identical (the floor sits below what the GPU measured)."""
    err = np.abs(gpu.astype(np.float64) - ref.astype(np.float64))
    tol = 1e-6 + 1e-5 * np.abs(ref.astype(np.float64))
    assert np.all(err <= tol), f"max err {err.max():.3e} ({(err > tol).sum()} over tolerance)"
    frac = (gpu == ref).mean()
    say(f"    residual_out bit-identical fraction {frac:.5f}")
    assert frac >= min_exact, f"bit-identical fraction {frac:.5f} below {min_exact}"


def assert_out_given_residual(out_gpu, r_gpu, gamma, eps, o_ref=None):
    """bf16 out of a non-unique residual: within one ulp of the oracle's RMSNorm of the GPU's own
    residual_out (and, for information, its distance to the oracle's own out)."""
    want = refs.rmsnorm_of(r_gpu, gamma, eps)
    assert_bf16_close(out_gpu, want)
    if o_ref is not None:
        d = bf16_ulp_diff(out_gpu, o_ref)
        say(f"    out vs the oracle's own out: max {d.max()} ulp, "
            f"{(d == 0).mean():.5f} bit-identical")


def finalize_gpu(d, per_expert=False, residual_out=None, out=None):
    kw = {}
    if per_expert:
        kw = dict(expert_ids=up(d["expert_ids"]), expert_gamma=up(d["expert_gamma"], True))
    return mf.mf_moe_finalize(up(d["expert_rows"], True), up(d["idx"]), up(d["weights"]),
                              up(d["residual"]), up(d["gamma"], True), d["eps"],
                              residual_out=residual_out, out=out, **kw)


def finalize_ref(d, per_expert=False, tokens=None):
    sl = slice(None) if tokens is None else tokens
    args = (d["expert_rows"], d["idx"][sl], d["weights"][sl], d["residual"][sl], d["gamma"],
            d["eps"])
    if per_expert:
        return oracle.moe_finalize(*args, d["expert_ids"][sl], d["expert_gamma"])
    return oracle.moe_finalize(*args)


def finalize_ref_threaded(d, threads=8):
    """The oracle over all tokens, token blocks in parallel host threads (the C call releases
    the GIL; each token's arithmetic is the same whatever block it is in)."""
    from concurrent.futures import ThreadPoolExecutor
    T = d["idx"].shape[0]
    bounds = np.linspace(0, T, threads + 1).astype(int)
    spans = [np.arange(bounds[i], bounds[i + 1]) for i in range(threads) if bounds[i] < bounds[i + 1]]
    with ThreadPoolExecutor(len(spans)) as ex:
        parts = list(ex.map(lambda tok: finalize_ref(d, tokens=tok), spans))
    return (np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts]))


def shape_str(kind, T, H, k=1):
    s = mf.mf_launch_shape(kind, T, H, k)
    return f"wpt={s['waves_per_token']} vpl={s['vectors_per_lane']} block={s['block']} grid={s['grid']}"


# ----------------------------------------------------------------------------- finalize


def test_finalize_tiny_workload():
    d = refs.named("finalize_tiny")
    say(f"finalize_tiny T=16 H=1024 k=2: {shape_str(0, 16, 1024, 2)}")
    out, r = finalize_gpu(d)
    torch.cuda.synchronize()
    r_ref, o_ref = finalize_ref(d)
    assert np.array_equal(r.cpu().numpy(), r_ref)
    assert_bf16_close(bits(out), o_ref)


FINALIZE_SHAPES = [
    (1, 8, 1, "random"), (3, 24, 2, "random"), (5, 520, 3, "random"),
    (17, 1024, 8, "expert_grouped"), (33, 4104, 9, "random"), (100, 7168, 8, "expert_grouped"),
    (2049, 7168, 8, "expert_grouped"), (7, 8192, 16, "random"), (5, 12288, 4, "random"),
    (3000, 12288, 2, "expert_grouped"), (4, 32768, 3, "random"), (2100, 32768, 1, "random"),
    (4097, 2048, 5, "expert_grouped"), (6, 3584, 64, "random"),
    # rows whose last slot ends past its first 256 values (the second 1 KiB residual store is
    # the partial one)
    (9, 776, 4, "random"), (65, 5000, 8, "expert_grouped"),
    # a grid past 65535 workgroups
    (70000, 64, 2, "random"),
    # wide rows at the compiled top-8 (the slot-serial kernel, 8 waves of 3 and of 5 to 8 slots,
    # up to three of them staged in LDS): whole waves of slots (12288, 20480, 24576, 28672,
    # 32768), a spare slot in a live wave (9216, 12800) and a last slot cut inside (12296)
    (600, 12288, 8, "expert_grouped"), (257, 20480, 8, "random"), (130, 32768, 8, "random"),
    (9, 9216, 8, "random"), (5, 12800, 8, "random"), (7, 12296, 8, "random"),
    (3, 16384, 8, "random"), (11, 24576, 8, "random"), (13, 28672, 8, "random"),
    # the plain finalize's shapes: one slot per wave over 4, 8 or 16 waves with spare waves
    # (1536, 3072, 6144), 8 waves of 3 or 4 slots (10240, 13312, 15360 with k = 3)
    (21, 1536, 8, "random"), (19, 3072, 8, "random"), (17, 6144, 8, "expert_grouped"),
    (9, 10240, 8, "random"), (8, 13312, 8, "random"), (6, 15360, 3, "random"),
    # the largest row and the largest top-k together, and the largest top-k with a ragged row
    (2, 32768, 64, "random"), (3, 4104, 64, "expert_grouped"),
]


@pytest.mark.parametrize("T,H,k,layout", FINALIZE_SHAPES)
def test_finalize_matches_oracle(T, H, k, layout):
    say(f"finalize T={T} H={H} k={k} {layout}: {shape_str(0, T, H, k)}")
    d = workloads.make_finalize_inputs(T, H, E=max(16, k), k=k, seed=1000 + T + H + k,
                                       layout=layout)
    out, r = finalize_gpu(d)
    torch.cuda.synchronize()
    r_ref, o_ref = finalize_ref(d)
    assert np.array_equal(r.cpu().numpy(), r_ref)
    assert_bf16_close(bits(out), o_ref)


def _random_finalize_cases(n=24, n_wide=8, seed=20261203):
    """Seeded random shapes across the launch-shape rules, each small enough for the oracle
    (T * k * H <= 8e6): n with H a multiple of 8 from 8 to 32768 (log-uniform), k from 1 to 64
    and T from 1 to 300; then n_wide rows wider than 8192 (every other one a whole number of
    4 KiB, with k = 8 on every other one: the slot-serial kernel's shapes among them), k up to 16.
    Random and expert-grouped layouts alternate; every third case is per-expert."""
    g = np.random.default_rng(seed)
    cases = []
    while len(cases) < n + n_wide:
        i = len(cases)
        if i < n:
            H = 8 * int(np.exp(g.uniform(0.0, np.log(4096.0))))
            k = int(np.exp(g.uniform(0.0, np.log(64.0))))
            T = int(g.integers(1, 301))
        else:
            H = 8 * int(g.integers(1025, 4097)) if i % 2 else 2048 * int(g.integers(5, 17))
            k = 8 if (i // 2) % 2 else int(g.integers(1, 17))
            T = int(g.integers(1, 41))
        if T * k * H > 8_000_000:
            continue
        cases.append((T, H, k, ("random", "expert_grouped")[i % 2], i % 3 == 2))
    return cases


@pytest.mark.parametrize("T,H,k,layout,per_expert", _random_finalize_cases())
def test_finalize_random_shapes(T, H, k, layout, per_expert):
    say(f"finalize random shape T={T} H={H} k={k} {layout} per_expert={per_expert}: "
        f"{shape_str(int(per_expert), T, H, k)}")
    d = workloads.make_finalize_inputs(T, H, E=max(16, k), k=k, seed=5000 + T + H + k,
                                       layout=layout, per_expert=per_expert)
    out, r = finalize_gpu(d, per_expert=per_expert)
    torch.cuda.synchronize()
    r_ref, o_ref = finalize_ref(d, per_expert=per_expert)
    rg = r.cpu().numpy()
    if per_expert:
        assert_fp32_tol(rg, r_ref, min_exact=0.5)
        assert_out_given_residual(bits(out), rg, d["gamma"], d["eps"], o_ref)
    else:
        assert np.array_equal(rg, r_ref)
        assert_bf16_close(bits(out), o_ref)


@pytest.fixture(scope="module")
def prefill():
    say("generating the prefill workload T=16384 H=7168 E=256 k=8 (host, ~20 s)")
    return refs.named("finalize_prefill")


def test_finalize_prefill_full_size(prefill):
    d = prefill
    T, H = d["T"], d["H"]
    say(f"finalize_prefill T={T} H={H} k=8: {shape_str(0, T, H, 8)}")
    rows, idx, w = up(d["expert_rows"], True), up(d["idx"]), up(d["weights"])
    res, gamma = up(d["residual"]), up(d["gamma"], True)
    out, r = mf.mf_moe_finalize(rows, idx, w, res, gamma, d["eps"])
    out2, r2 = mf.mf_moe_finalize(rows, idx, w, res, gamma, d["eps"])
    torch.cuda.synchronize()
    assert torch.equal(r, r2) and torch.equal(out.view(torch.int16), out2.view(torch.int16))
    assert torch.isfinite(r).all() and torch.isfinite(out.float()).all()
    # in place on a copy of the residual stream: same bits
    r3 = res.clone()
    out3, _ = mf.mf_moe_finalize(rows, idx, w, r3, gamma, d["eps"], residual_out=r3)
    torch.cuda.synchronize()
    assert torch.equal(r3, r) and torch.equal(out3.view(torch.int16), out.view(torch.int16))
    # every token against the oracle (run over token blocks in host threads)
    r_ref, o_ref = finalize_ref_threaded(d)
    assert np.array_equal(r.cpu().numpy(), r_ref)
    assert_bf16_close(bits(out), o_ref)
    say(f"    all {T} tokens bit-identical in residual_out")


def test_finalize_batch_invariance():
    # A token's result does not depend on how many tokens share the launch (different
    # token counts pick different waves-per-token; the reduction tree is the same).
    d = workloads.make_finalize_inputs(3000, 7168, E=64, k=8, seed=77)
    say(f"batch invariance H=7168: T=3000 {shape_str(0, 3000, 7168, 8)} vs T=5 {shape_str(0, 5, 7168, 8)}")
    out_big, r_big = finalize_gpu(d)
    small = dict(d, T=5, idx=d["idx"][:5], weights=d["weights"][:5], residual=d["residual"][:5])
    out_small, r_small = finalize_gpu(small)
    torch.cuda.synchronize()
    assert torch.equal(r_big[:5], r_small)
    assert torch.equal(out_big[:5].view(torch.int16), out_small.view(torch.int16))


@pytest.mark.parametrize("H", [12288, 20480, 24576, 28672, 32768])
def test_wide_finalize_batch_invariance_and_in_place(H):
    # the slot-serial kernel of wide rows: a token's bits do not depend on the batch, and the
    # in-place update of the residual stream gives the same bits as a separate output
    d = workloads.make_finalize_inputs(300, H, E=64, k=8, seed=88 + H)
    say(f"wide batch invariance / in place H={H}: {shape_str(0, 300, H, 8)}")
    out_big, r_big = finalize_gpu(d)
    small = dict(d, T=3, idx=d["idx"][-3:], weights=d["weights"][-3:], residual=d["residual"][-3:])
    out_small, r_small = finalize_gpu(small)
    res = up(d["residual"])
    out_ip, _ = mf.mf_moe_finalize(up(d["expert_rows"], True), up(d["idx"]), up(d["weights"]), res,
                                   up(d["gamma"], True), d["eps"], residual_out=res)
    torch.cuda.synchronize()
    assert torch.equal(r_big[-3:], r_small)
    assert torch.equal(out_big[-3:].view(torch.int16), out_small.view(torch.int16))
    assert torch.equal(res, r_big) and torch.equal(out_ip.view(torch.int16), out_big.view(torch.int16))


def test_finalize_guard_bands():
    T, H, k = 37, 520, 3
    say(f"guard bands T={T} H={H} k={k}: {shape_str(0, T, H, k)}")
    d = workloads.make_finalize_inputs(T, H, E=8, k=k, seed=78, layout="random")
    pad = 64
    rbuf = torch.full((T * H + 2 * pad,), 12345.0, dtype=torch.float32, device=DEV)
    obuf = torch.full((T * H + 2 * pad,), 0x7BAD, dtype=torch.int16, device=DEV)
    r_view = rbuf[pad:pad + T * H].view(T, H)
    o_view = obuf[pad:pad + T * H].view(T, H).view(torch.bfloat16)
    finalize_gpu(d, residual_out=r_view, out=o_view)
    torch.cuda.synchronize()
    assert torch.all(rbuf[:pad] == 12345.0) and torch.all(rbuf[-pad:] == 12345.0)
    assert torch.all(obuf[:pad] == 0x7BAD) and torch.all(obuf[-pad:] == 0x7BAD)
    r_ref, o_ref = finalize_ref(d)
    assert np.array_equal(r_view.cpu().numpy(), r_ref)
    assert_bf16_close(bits(o_view), o_ref)


def test_finalize_on_a_side_stream():
    d = workloads.make_finalize_inputs(64, 1024, E=8, k=4, seed=79)
    s = torch.cuda.Stream(device=DEV)
    with torch.cuda.stream(s):
        out, r = finalize_gpu(d)
    s.synchronize()
    r_ref, o_ref = finalize_ref(d)
    assert np.array_equal(r.cpu().numpy(), r_ref)
    assert_bf16_close(bits(out), o_ref)


def test_finalize_on_concurrent_streams():
    # the library keeps no state between calls: two streams running different problems at once
    # each get their own results (the same bits as run alone)
    a = workloads.make_finalize_inputs(700, 7168, E=64, k=8, seed=86)
    b = workloads.make_finalize_inputs(300, 12288, E=64, k=8, seed=87)
    say("concurrent streams: T=700 H=7168 and T=300 H=12288, k=8")
    alone_a = finalize_gpu(a)
    alone_b = finalize_gpu(b)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(device=DEV), torch.cuda.Stream(device=DEV)
    ins_a = (up(a["expert_rows"], True), up(a["idx"]), up(a["weights"]), up(a["residual"]),
             up(a["gamma"], True), a["eps"])
    ins_b = (up(b["expert_rows"], True), up(b["idx"]), up(b["weights"]), up(b["residual"]),
             up(b["gamma"], True), b["eps"])
    torch.cuda.synchronize()
    for _ in range(3):
        with torch.cuda.stream(s1):
            oa, ra = mf.mf_moe_finalize(*ins_a)
        with torch.cuda.stream(s2):
            ob, rb = mf.mf_moe_finalize(*ins_b)
        s1.synchronize()
        s2.synchronize()
        assert torch.equal(ra, alone_a[1]) and torch.equal(oa.view(torch.int16), alone_a[0].view(torch.int16))
        assert torch.equal(rb, alone_b[1]) and torch.equal(ob.view(torch.int16), alone_b[0].view(torch.int16))


def test_zero_tokens_is_a_no_op():
    d = workloads.make_finalize_inputs(1, 64, E=4, k=2, seed=80)
    rows = up(d["expert_rows"], True)
    out, r = mf.mf_moe_finalize(rows, torch.zeros((0, 2), dtype=torch.int32, device=DEV),
                                torch.zeros((0, 2), device=DEV), torch.zeros((0, 64), device=DEV),
                                up(d["gamma"], True))
    assert out.shape == (0, 64) and r.shape == (0, 64)


# ----------------------------------------------------------------------------- per-expert


def test_finalize_decode_per_expert_workload():
    d = refs.named("finalize_decode_per_expert")
    say(f"finalize_decode_per_expert T=64 H=4096 k=8: {shape_str(1, 64, 4096, 8)}")
    out, r = finalize_gpu(d, per_expert=True)
    torch.cuda.synchronize()
    r_ref, o_ref = finalize_ref(d, per_expert=True)
    rg = r.cpu().numpy()
    assert_fp32_tol(rg, r_ref, min_exact=0.5)
    assert_out_given_residual(bits(out), rg, d["gamma"], d["eps"], o_ref)


@pytest.mark.parametrize("T,H,k", [(1, 64, 1), (5, 520, 3), (33, 7168, 8), (2100, 7168, 8),
                                   (3, 4096, 13), (9, 32768, 2), (2500, 1024, 4), (5, 3848, 8),
                                   (2, 2048, 64), (2, 32768, 8)])
def test_per_expert_matches_oracle(T, H, k):
    say(f"per-expert T={T} H={H} k={k}: {shape_str(1, T, H, k)}")
    d = workloads.make_finalize_inputs(T, H, E=max(32, k), k=k, seed=2000 + T + H + k,
                                       per_expert=True, residual_std=2.0)
    out, r = finalize_gpu(d, per_expert=True)
    torch.cuda.synchronize()
    r_ref, o_ref = finalize_ref(d, per_expert=True)
    rg = r.cpu().numpy()
    assert_fp32_tol(rg, r_ref, min_exact=0.5)
    assert_out_given_residual(bits(out), rg, d["gamma"], d["eps"], o_ref)


def test_per_expert_batch_invariance():
    d = workloads.make_finalize_inputs(2500, 4096, E=32, k=8, seed=81, per_expert=True)
    say(f"per-expert batch invariance: T=2500 {shape_str(1, 2500, 4096, 8)} vs T=3 {shape_str(1, 3, 4096, 8)}")
    out_big, r_big = finalize_gpu(d, per_expert=True)
    small = dict(d, T=3, idx=d["idx"][:3], weights=d["weights"][:3], residual=d["residual"][:3],
                 expert_ids=d["expert_ids"][:3])
    out_small, r_small = finalize_gpu(small, per_expert=True)
    torch.cuda.synchronize()
    assert torch.equal(r_big[:3], r_small)
    assert torch.equal(out_big[:3].view(torch.int16), out_small.view(torch.int16))


# ----------------------------------------------------------------------------- gated

# The gated residual is one fp32 FMA of sigmoid(gate) and x onto the residual; the GPU's sigmoid
# (a hardware exp and an IEEE division) is within a few ulp of the exact one, so most elements
# round to the same fp32 value.  Floor on the bit-identical fraction (measured well above it).
GATED_MIN_EXACT = 0.7


def gated_gpu(d, residual_out=None):
    return mf.mf_gated_residual_rmsnorm(up(d["x"], True), up(d["gate"], True), up(d["residual"]),
                                        up(d["gamma"], True), d["eps"], residual_out=residual_out)


def test_gated_workload_full_size():
    d = workloads.make_inputs("gated_residual_rmsnorm")
    say(f"gated T=4096 H=8192: {shape_str(2, 4096, 8192)}")
    out, r = gated_gpu(d)
    torch.cuda.synchronize()
    r_ref, o_ref = oracle.gated_residual_rmsnorm(d["x"], d["gate"], d["residual"], d["gamma"],
                                                 d["eps"])
    rg = r.cpu().numpy()
    assert_fp32_tol(rg, r_ref, min_exact=GATED_MIN_EXACT)
    assert_out_given_residual(bits(out), rg, d["gamma"], d["eps"], o_ref)


@pytest.mark.parametrize("T,H", [(1, 8), (3, 520), (5000, 1024), (7, 32768), (2049, 8192),
                                 (3, 1000), (70000, 72)])
def test_gated_matches_oracle(T, H):
    say(f"gated T={T} H={H}: {shape_str(2, T, H)}")
    d = workloads.make_gated_inputs(T, H, seed=3000 + T + H)
    out, r = gated_gpu(d)
    torch.cuda.synchronize()
    r_ref, o_ref = oracle.gated_residual_rmsnorm(d["x"], d["gate"], d["residual"], d["gamma"],
                                                 d["eps"])
    rg = r.cpu().numpy()
    assert_fp32_tol(rg, r_ref, min_exact=GATED_MIN_EXACT)
    assert_out_given_residual(bits(out), rg, d["gamma"], d["eps"], o_ref)


def test_gated_zero_gate_is_exact():
    # sigmoid(0) = 1/2 exactly, so residual_out = fp32(residual + x/2) bit for bit.
    d = workloads.make_gated_inputs(64, 8192, seed=82)
    d["gate"] = np.zeros_like(d["gate"])
    out, r = gated_gpu(d)
    torch.cuda.synchronize()
    want = d["residual"] + np.float32(0.5) * workloads.bf16_bits_to_f32(d["x"])
    assert np.array_equal(r.cpu().numpy(), want)


def test_gated_in_place():
    d = workloads.make_gated_inputs(100, 8192, seed=83)
    res = up(d["residual"])
    out, _ = mf.mf_gated_residual_rmsnorm(up(d["x"], True), up(d["gate"], True), res,
                                          up(d["gamma"], True), d["eps"], residual_out=res)
    out2, r2 = gated_gpu(d)
    torch.cuda.synchronize()
    assert torch.equal(res, r2) and torch.equal(out.view(torch.int16), out2.view(torch.int16))


# ----------------------------------------------------------------------------- gated, dual output


def gated_next_gpu(d, residual_out=None):
    return mf.mf_gated_residual_next_rmsnorm(
        up(d["x"], True), up(d["gate"], True), up(d["residual"]), up(d["gamma"], True),
        up(d["gamma_next"], True), d["eps"], residual_out=residual_out)


def check_gated_next(d):
    out, on, r = gated_next_gpu(d)
    torch.cuda.synchronize()
    r_ref, o_ref, on_ref = oracle.gated_residual_next_rmsnorm(
        d["x"], d["gate"], d["residual"], d["gamma"], d["gamma_next"], d["eps"])
    rg = r.cpu().numpy()
    assert_fp32_tol(rg, r_ref, min_exact=GATED_MIN_EXACT)
    assert_out_given_residual(bits(out), rg, d["gamma"], d["eps"], o_ref)
    assert_out_given_residual(bits(on), rg, d["gamma_next"], d["eps"], on_ref)
    return out, on, r


def test_gated_next_workload_full_size():
    d = workloads.make_inputs("gated_residual_next_rmsnorm")
    say(f"gated next T=4096 H=8192: {shape_str(2, 4096, 8192)}")
    check_gated_next(d)


@pytest.mark.parametrize("T,H", [(1, 8), (3, 520), (5000, 1024), (7, 32768), (2049, 8192),
                                 (9, 12288), (5, 7000)])
def test_gated_next_matches_oracle(T, H):
    say(f"gated next T={T} H={H}: {shape_str(2, T, H)}")
    check_gated_next(workloads.make_gated_inputs(T, H, seed=3100 + T + H, dual=True))


def test_gated_next_first_output_is_the_single_output_form():
    # the dual form's residual_out and out are bit-identical to mf_gated_residual_rmsnorm's
    d = workloads.make_gated_inputs(333, 8192, seed=84, dual=True)
    say("gated next vs gated: T=333 H=8192")
    out, on, r = gated_next_gpu(d)
    out1, r1 = gated_gpu(d)
    torch.cuda.synchronize()
    assert torch.equal(r, r1) and torch.equal(out.view(torch.int16), out1.view(torch.int16))


def test_gated_next_equal_gammas_and_in_place():
    d = workloads.make_gated_inputs(100, 8192, seed=85, dual=True)
    d["gamma_next"] = d["gamma"]
    say("gated next: gamma_next == gamma, in place, T=100 H=8192")
    res = up(d["residual"])
    out, on, r = mf.mf_gated_residual_next_rmsnorm(
        up(d["x"], True), up(d["gate"], True), res, up(d["gamma"], True), up(d["gamma"], True),
        d["eps"], residual_out=res)
    out2, on2, r2 = gated_next_gpu(d)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), on.view(torch.int16))
    assert torch.equal(res, r2) and torch.equal(on.view(torch.int16), on2.view(torch.int16))


# ----------------------------------------------------------------------------- per-head


def test_per_head_workload_full_size():
    d = workloads.make_inputs("rmsnorm_sigmoid_gate")
    say("per-head T=4096 heads=64 D=64")
    out = mf.mf_rmsnorm_sigmoid_gate(up(d["x"], True), up(d["gate"], True), up(d["gamma"], True),
                                     d["eps"])
    torch.cuda.synchronize()
    o_ref = oracle.rmsnorm_sigmoid_gate(d["x"], d["gate"], d["gamma"], d["eps"])
    assert_bf16_close(bits(out), o_ref)


@pytest.mark.parametrize("T,heads", [(1, 1), (3, 5), (7, 64), (1000, 3)])
def test_per_head_ragged(T, heads):
    say(f"per-head T={T} heads={heads}")
    d = workloads.make_per_head_inputs(T, heads, 64, seed=4000 + T + heads)
    out = mf.mf_rmsnorm_sigmoid_gate(up(d["x"], True), up(d["gate"], True), up(d["gamma"], True),
                                     d["eps"])
    torch.cuda.synchronize()
    o_ref = oracle.rmsnorm_sigmoid_gate(d["x"], d["gate"], d["gamma"], d["eps"])
    assert_bf16_close(bits(out), o_ref, min_exact=0.98)


# ----------------------------------------------------------------------------- random shapes


def _random_norm_cases(n=12, seed=20261204):
    """Seeded random (T, H) for the gated norms: H a multiple of 8 from 8 to 32768 (log-uniform),
    T from 1 to 3000, T * H <= 4e6."""
    g = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        H = 8 * int(np.exp(g.uniform(0.0, np.log(4096.0))))
        T = int(np.exp(g.uniform(0.0, np.log(3000.0))))
        if T * H <= 4_000_000:
            cases.append((T, H))
    return cases


def _floor(n_elements, floor):
    # a bit-identical fraction is only asserted where there are enough elements for it to be
    # stable; the ulp and tolerance bars hold everywhere
    return floor if n_elements >= 4096 else 0.0


@pytest.mark.parametrize("T,H", _random_norm_cases())
def test_gated_random_shapes(T, H):
    say(f"gated random shape T={T} H={H}: {shape_str(2, T, H)}")
    d = workloads.make_gated_inputs(T, H, seed=6000 + T + H)
    out, r = gated_gpu(d)
    torch.cuda.synchronize()
    r_ref, o_ref = oracle.gated_residual_rmsnorm(d["x"], d["gate"], d["residual"], d["gamma"],
                                                 d["eps"])
    rg = r.cpu().numpy()
    assert_fp32_tol(rg, r_ref, min_exact=_floor(T * H, GATED_MIN_EXACT))
    want = refs.rmsnorm_of(rg, d["gamma"], d["eps"])
    assert_bf16_close(bits(out), want, min_exact=_floor(T * H, 0.99))


@pytest.mark.parametrize("T,H", _random_norm_cases(n=8, seed=20261205))
def test_gated_next_random_shapes(T, H):
    say(f"gated dual random shape T={T} H={H}: {shape_str(2, T, H)}")
    d = workloads.make_gated_inputs(T, H, seed=7000 + T + H, dual=True)
    out, on, r = gated_next_gpu(d)
    torch.cuda.synchronize()
    r_ref, _, _ = oracle.gated_residual_next_rmsnorm(
        d["x"], d["gate"], d["residual"], d["gamma"], d["gamma_next"], d["eps"])
    rg = r.cpu().numpy()
    assert_fp32_tol(rg, r_ref, min_exact=_floor(T * H, GATED_MIN_EXACT))
    for o, gm in ((out, d["gamma"]), (on, d["gamma_next"])):
        assert_bf16_close(bits(o), refs.rmsnorm_of(rg, gm, d["eps"]), min_exact=_floor(T * H, 0.99))


def _random_per_head_cases(n=12, seed=20261206):
    g = np.random.default_rng(seed)
    return [(int(np.exp(g.uniform(0.0, np.log(3000.0)))), int(g.integers(1, 129))) for _ in range(n)]


@pytest.mark.parametrize("T,heads", _random_per_head_cases())
def test_per_head_random_shapes(T, heads):
    say(f"per-head random shape T={T} heads={heads}")
    d = workloads.make_per_head_inputs(T, heads, 64, seed=8000 + T + heads)
    out = mf.mf_rmsnorm_sigmoid_gate(up(d["x"], True), up(d["gate"], True), up(d["gamma"], True),
                                     d["eps"])
    torch.cuda.synchronize()
    o_ref = oracle.rmsnorm_sigmoid_gate(d["x"], d["gate"], d["gamma"], d["eps"])
    assert_bf16_close(bits(out), o_ref, min_exact=_floor(T * heads * 64, 0.99))


# ----------------------------------------------------------------------------- copy


@pytest.mark.parametrize("nbytes", [16, 1040, 1 << 22, (1 << 22) + 48])
def test_stream_copy(nbytes):
    # whole and partial last workgroups; the bytes past the copy stay untouched
    n = nbytes // 4
    src = torch.randint(-2**31, 2**31 - 1, (n + 16,), dtype=torch.int32, device=DEV)
    dst = torch.full((n + 16,), 0x5A5A5A5A, dtype=torch.int32, device=DEV)
    mf.mf_stream_copy(src[:n], dst[:n])
    torch.cuda.synchronize()
    assert torch.equal(src[:n], dst[:n])
    assert bool((dst[n:] == 0x5A5A5A5A).all())


@pytest.mark.parametrize("nbytes", [16, 16384, 16384 * 5 + 48, 1 << 24])
def test_stream_read(nbytes):
    # every chunk's xor of its 32-bit words, checked on the host
    g = np.random.default_rng(nbytes)
    host = g.integers(0, 2**32, nbytes // 4, dtype=np.uint32)
    src = torch.from_numpy(host.view(np.int32)).to(DEV)
    sink = mf.mf_stream_read(src)
    torch.cuda.synchronize()
    chunk = mf.MF_STREAM_READ_CHUNK // 4
    want = [np.bitwise_xor.reduce(host[i:i + chunk]) for i in range(0, host.size, chunk)]
    assert np.array_equal(sink.cpu().numpy().view(np.uint32), np.array(want, dtype=np.uint32))
