"""Parity of the MXFP4 kernels on the GPU (through the C ABI) with the oracle.

Bars:
  - mf_mxfp4_quantize (fp32 in): codes and scales bit-identical (the OCP definition has one
    answer for an fp32 value: the scale from the block maximum's exponent, the nearest code
    with ties to even);
  - mf_rmsnorm_mxfp4_quantize: the quantisation decision is taken on the fp32 normalised value,
    which the GPU forms from its own fp32 mean square (a few ulps from the oracle's float64
    one, rounded to fp32).  So every scale must be one the oracle's rule gives for a block
    maximum within a relative band of 2^-20 of the oracle's, and every decoded value one its
    rule gives for a value within that band of the oracle's; and >= 99.9% of all codes and
    scales are bit-identical.
  - mf_moe_finalize_mxfp4: residual_out bit-identical to the oracle's finalize (the same fp32
    FMA chain as mf_moe_finalize); codes and scales to the band bar above, against the oracle's
    RMSNorm + MXFP4 of that fp32 residual.  The prefill workload is checked on every token.
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

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_examples.json")
E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
BAND = 2.0 ** -20


def say(msg):
    print(msg, flush=True)


def quantize_gpu(x):
    q, sc = mf.mf_mxfp4_quantize(torch.from_numpy(np.ascontiguousarray(x)).to(DEV))
    torch.cuda.synchronize()
    return q.cpu().numpy(), sc.cpu().numpy()


def decode(q, sc):
    codes = np.stack([q & 0xF, q >> 4], axis=-1).reshape(q.shape[0], -1)
    mag = E2M1[codes & 7]
    val = np.where(codes & 8, -mag, mag)
    return val * np.repeat(np.ldexp(1.0, sc.astype(np.int64) - 127), 32, axis=1)


def test_mxfp4_golden_hand_example():
    g = json.load(open(GOLDEN))["mxfp4_quantize"]
    head = [-0.0 if v == "-0" else float(v) for v in g["values_block0_head"]]
    b0 = np.array(head + [0.0] * 16, np.float32)
    x = np.concatenate([b0, b0 * np.float32(2.0 ** -10), np.zeros(32, np.float32)])[None]
    say("mxfp4 golden: T=1 H=96")
    q, sc = quantize_gpu(x)
    want = [int(h, 16) for h in g["expected_block_bytes"]]
    assert q[0, :16].tolist() == want and q[0, 16:32].tolist() == want
    assert q[0, 32:].tolist() == [0] * 16 and sc[0].tolist() == g["expected_scales"]


@pytest.mark.parametrize("T,H,spread", [
    (1, 32, 1.0), (3, 64, 1.0), (7, 96, 30.0), (5, 4096, 1e-20), (4, 8192, 1e20),
    (1000, 7168, 1.0), (33, 32768, 0.01), (2, 1024, 1e-38),
])
def test_mxfp4_quantize_matches_oracle(T, H, spread):
    say(f"mxfp4 quantize T={T} H={H} spread={spread}")
    rng = np.random.default_rng(800 + T + H)
    x = (rng.standard_normal((T, H)) * spread).astype(np.float32)
    x[:, 3] = -0.0
    if H >= 64:
        x[0, 32:64] = 0.0                                           # an all-zero block
    # exact ties and saturation inside one block of the first row
    x[0, :16] = np.array([6, 3, 1.5, 0.5, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5, 7, 0.3, 4, -2.5, -5],
                         np.float32) * np.float32(spread)
    q, sc = quantize_gpu(x)
    q_ref, sc_ref = oracle.mxfp4_quantize(x)
    assert np.array_equal(sc, sc_ref), f"{(sc != sc_ref).sum()} scales differ"
    assert np.array_equal(q, q_ref), f"{(q != q_ref).sum()} code bytes differ"


def test_mxfp4_quantize_every_code_and_tie():
    # every E2M1 magnitude and every midpoint between neighbours, both signs, at three scales
    mags = np.concatenate([E2M1, (E2M1[:-1] + E2M1[1:]) / 2, [6.5, 7.9]])
    vals = np.concatenate([mags, -mags])
    blocks = []
    for e in (-100, 0, 100):
        v = np.zeros(64)
        v[:len(vals)] = vals
        v[63] = 7.5                                                  # pins the block maximum
        blocks.append(np.ldexp(v, e))
    x = np.stack(blocks).astype(np.float32)
    say(f"mxfp4 quantize: every code and tie, {x.shape}")
    q, sc = quantize_gpu(x)
    q_ref, sc_ref = oracle.mxfp4_quantize(x)
    assert np.array_equal(sc, sc_ref) and np.array_equal(q, q_ref)


def rms_mx_gpu(x, gamma, eps):
    q, sc = mf.mf_rmsnorm_mxfp4_quantize(
        torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(DEV),
        torch.from_numpy(gamma.view(np.int16)).view(torch.bfloat16).to(DEV), eps)
    torch.cuda.synchronize()
    return q.cpu().numpy(), sc.cpu().numpy()


def nearest(r):
    """Signed E2M1 value nearest to r (ties to the even code, saturating at 6)."""
    m = np.abs(r)
    d = np.abs(m[..., None] - E2M1)
    best = d.min(axis=-1, keepdims=True)
    cand = d == best
    even = cand & (np.arange(8) % 2 == 0)
    pick = np.where(even.any(axis=-1), np.argmax(even, axis=-1), np.argmax(cand, axis=-1))
    pick = np.where(m >= 6, 7, pick)
    return np.where(np.signbit(r), -E2M1[pick], E2M1[pick])


def check_rms_mx(x, gamma, eps, min_exact=0.999):
    q, sc = rms_mx_gpu(x, gamma, eps)
    q_ref, sc_ref = oracle.rmsnorm_mxfp4_quantize(x, gamma, eps)
    check_band(q, sc, q_ref, sc_ref, workloads.bf16_bits_to_f32(x), gamma, eps, min_exact)


def check_band(q, sc, q_ref, sc_ref, xf, gamma, eps, min_exact=0.999):
    """q, sc from the GPU against the oracle's (q_ref, sc_ref) for the RMSNorm of the fp32 rows
    xf with gamma: the band bar of the module docstring (the bit-identical floor min_exact)."""
    T, H = xf.shape
    # the oracle's fp32 normalised value, and a band around it
    xd = xf.astype(np.float64)
    s = 1.0 / np.sqrt((xd * xd).mean(axis=1, keepdims=True) + eps)
    y = (xd * s * workloads.bf16_bits_to_f32(gamma)).astype(np.float32).astype(np.float64)
    lo, hi = y * (1 - BAND), y * (1 + BAND)
    # scales: a code the rule gives for a block maximum inside the band
    amax = np.abs(y).reshape(T, H // 32, 32).max(axis=-1)
    code = lambda a: np.where(a == 0, 0, np.clip(np.frexp(a)[1] - 1 - 2 + 127, 0, 254))
    c_lo, c_hi = code(amax * (1 - BAND)), code(amax * (1 + BAND))
    assert np.all((sc >= c_lo) & (sc <= c_hi)), f"{((sc < c_lo) | (sc > c_hi)).sum()} scales outside"
    # values: with the GPU's scale, the code the rule gives for a value inside the band
    X = np.repeat(np.ldexp(1.0, sc.astype(np.int64) - 127), 32, axis=1)
    dec = decode(q, sc)
    v1, v2 = nearest(lo / X) * X, nearest(hi / X) * X
    ok = (dec >= np.minimum(v1, v2)) & (dec <= np.maximum(v1, v2))
    assert ok.all(), f"{(~ok).sum()} codes outside the band"
    exact = ((q == q_ref).sum() + (sc == sc_ref).sum()) / (q.size + sc.size)
    assert exact >= min_exact, f"bit-identical fraction {exact:.5f}"
    say(f"    bit-identical fraction {exact:.6f}")


def test_rmsnorm_mxfp4_golden():
    g = json.load(open(GOLDEN))["rmsnorm_mxfp4_quantize"]
    H = g["H"]
    x = workloads.to_bf16_bits(np.tile([1.0, -1.0], H // 2).astype(np.float32))[None]
    say("rmsnorm mxfp4 golden: T=1 H=32")
    for gam, key in ((1.0, "expected_scale_gamma1"), (0.5, "expected_scale_gamma_half")):
        q, sc = rms_mx_gpu(x, workloads.to_bf16_bits(np.full(H, gam, np.float32)), g["eps"])
        assert q[0].tolist() == [int(g["expected_byte"], 16)] * (H // 2)
        assert sc[0].tolist() == [g[key]]


@pytest.mark.parametrize("T,H", [(1, 32), (3, 544), (100, 7168), (7, 32768), (2049, 1024),
                                 (5, 12288),
                                 # 1 to 4 slots per wave over 4 to 8 waves, whole and ragged
                                 # last slots
                                 (9, 8192), (5, 4096), (6, 2048), (4, 3072), (3, 4128), (2, 8160),
                                 (33, 1536), (4097, 8192)])
def test_rmsnorm_mxfp4_matches_oracle(T, H):
    say(f"rmsnorm mxfp4 T={T} H={H}")
    d = workloads.make_rmsnorm_mx_inputs(T, H, seed=900 + T + H)
    check_rms_mx(d["x"], d["gamma"], d["eps"])


@pytest.mark.parametrize("H", [8192, 4128, 12288])
def test_rmsnorm_mxfp4_batch_invariance(H):
    # a token's codes and scales do not depend on how many tokens share the launch
    d = workloads.make_rmsnorm_mx_inputs(301, H, seed=950 + H)
    say(f"rmsnorm mxfp4 batch invariance H={H}: T=301 against its last 3 tokens alone")
    q, sc = rms_mx_gpu(d["x"], d["gamma"], d["eps"])
    q3, sc3 = rms_mx_gpu(d["x"][-3:], d["gamma"], d["eps"])
    assert np.array_equal(q[-3:], q3) and np.array_equal(sc[-3:], sc3)


def test_rmsnorm_mxfp4_workload_full_size():
    d = workloads.make_inputs("rmsnorm_mxfp4")
    say("rmsnorm mxfp4 workload T=4096 H=8192")
    check_rms_mx(d["x"], d["gamma"], d["eps"])


def up(a, bf16=False):
    a = np.ascontiguousarray(a)
    t = torch.from_numpy(a.view(np.int16) if bf16 else a)
    if bf16:
        t = t.view(torch.bfloat16)
    return t.to(DEV)


def finalize_mx_gpu(d, in_place=False):
    res = up(d["residual"])
    q, sc, r = mf.mf_moe_finalize_mxfp4(up(d["expert_rows"], True), up(d["idx"]),
                                        up(d["weights"]), res, up(d["gamma"], True), d["eps"],
                                        residual_out=res if in_place else None)
    torch.cuda.synchronize()
    return q.cpu().numpy(), sc.cpu().numpy(), r.cpu().numpy()


def check_finalize_mx(d, rows=None, in_place=False, min_exact=0.999):
    q, sc, r = finalize_mx_gpu(d, in_place)
    sel = slice(None) if rows is None else rows
    r_ref, _ = oracle.moe_finalize(d["expert_rows"], d["idx"][sel], d["weights"][sel],
                                   d["residual"][sel], d["gamma"], d["eps"])
    assert np.array_equal(r[sel].view(np.uint32), r_ref.view(np.uint32)), "residual_out differs"
    q_ref, sc_ref = oracle.rmsnorm_f32_mxfp4_quantize(r_ref, d["gamma"], d["eps"])
    check_band(q[sel], sc[sel], q_ref, sc_ref, r_ref, d["gamma"], d["eps"], min_exact)


@pytest.mark.parametrize("T,H,k,layout", [
    (1, 32, 1, "random"), (17, 1024, 8, "random"), (33, 4128, 9, "random"),
    (100, 7168, 8, "expert_grouped"), (5, 32768, 3, "random"), (64, 4096, 16, "random"),
    (2049, 512, 4, "random"), (7, 12288, 32, "random"), (3, 800, 4, "random"),
    # 8 waves of 3 or 4 slots, and 16 waves of one slot with spare waves
    (6, 16384, 8, "random"), (5, 13312, 8, "random"), (9, 6144, 8, "random"),
])
def test_finalize_mxfp4_matches_oracle(T, H, k, layout):
    say(f"finalize mxfp4 T={T} H={H} k={k} layout={layout}")
    d = workloads.make_finalize_inputs(T, H, E=max(16, k), k=k, seed=950 + T + H + k,
                                       layout=layout)
    check_finalize_mx(d)


def _random_mx_cases(n, seed, finalize):
    """Seeded random shapes: H a multiple of 32 from 32 to 32768 (log-uniform), T up to 400; the
    finalize with k from 1 to 16 (every other case the compiled 8).  Each small enough for the
    oracle."""
    g = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        H = 32 * int(np.exp(g.uniform(0.0, np.log(1024.0))))
        T = int(np.exp(g.uniform(0.0, np.log(400.0))))
        if finalize:
            k = 8 if len(cases) % 2 else int(g.integers(1, 17))
            if T * k * H <= 6_000_000:
                cases.append((T, H, k, ("random", "expert_grouped")[len(cases) % 2]))
        elif T * H <= 4_000_000:
            cases.append((T, H))
    return cases


def _mx_floor(T, H):
    # the bit-identical floor only where there are enough code and scale bytes for it
    return 0.999 if T * (H // 2 + H // 32) >= 4096 else 0.0


@pytest.mark.parametrize("T,H,k,layout", _random_mx_cases(10, 20261209, True))
def test_finalize_mxfp4_random_shapes(T, H, k, layout):
    say(f"finalize mxfp4 random shape T={T} H={H} k={k} layout={layout}")
    d = workloads.make_finalize_inputs(T, H, E=max(16, k), k=k, seed=970 + T + H + k,
                                       layout=layout)
    check_finalize_mx(d, min_exact=_mx_floor(T, H))


@pytest.mark.parametrize("T,H", _random_mx_cases(10, 20261210, False))
def test_rmsnorm_mxfp4_random_shapes(T, H):
    say(f"rmsnorm mxfp4 random shape T={T} H={H}")
    d = workloads.make_rmsnorm_mx_inputs(T, H, seed=980 + T + H)
    check_rms_mx(d["x"], d["gamma"], d["eps"], min_exact=_mx_floor(T, H))


def test_finalize_mxfp4_in_place():
    d = workloads.make_finalize_inputs(100, 7168, E=64, k=8, seed=960)
    say("finalize mxfp4 in place: T=100 H=7168 k=8")
    check_finalize_mx(d, in_place=True)


def test_finalize_mxfp4_agrees_with_two_steps():
    """The fused epilogue's residual_out equals mf_moe_finalize's, bit for bit."""
    d = workloads.make_finalize_inputs(257, 7168, E=64, k=8, seed=961)
    say("finalize mxfp4 vs finalize: T=257 H=7168 k=8")
    _, _, r = finalize_mx_gpu(d)
    _, r1 = mf.mf_moe_finalize(up(d["expert_rows"], True), up(d["idx"]), up(d["weights"]),
                               up(d["residual"]), up(d["gamma"], True), d["eps"])
    torch.cuda.synchronize()
    assert np.array_equal(r.view(np.uint32), r1.cpu().numpy().view(np.uint32))


def test_finalize_mxfp4_workload_full_size():
    """Every one of the 16384 tokens, checked in blocks of 2048; the oracle's finalize and its
    RMSNorm + MXFP4 run over the blocks in host threads (each token's arithmetic is the same in
    any block)."""
    from concurrent.futures import ThreadPoolExecutor
    d = refs.named("finalize_prefill_mxfp4")
    T = d["T"]
    say(f"finalize mxfp4 workload T={T} H=7168 k=8, all tokens")
    q, sc, r = finalize_mx_gpu(d)
    blocks = [np.arange(lo, min(lo + 2048, T)) for lo in range(0, T, 2048)]

    def reference(rows):
        r_ref, _ = oracle.moe_finalize(d["expert_rows"], d["idx"][rows], d["weights"][rows],
                                       d["residual"][rows], d["gamma"], d["eps"])
        q_ref, sc_ref = oracle.rmsnorm_f32_mxfp4_quantize(r_ref, d["gamma"], d["eps"])
        return r_ref, q_ref, sc_ref

    with ThreadPoolExecutor(len(blocks)) as ex:
        expected = list(ex.map(reference, blocks))
    for rows, (r_ref, q_ref, sc_ref) in zip(blocks, expected):
        assert np.array_equal(r[rows].view(np.uint32), r_ref.view(np.uint32)), \
            f"residual_out differs in tokens {rows[0]}..{rows[-1]}"
        check_band(q[rows], sc[rows], q_ref, sc_ref, r_ref, d["gamma"], d["eps"])
