"""Guard bands around every output of every entry point, on the GPU through the C ABI.

Each output is a view into a larger byte buffer whose 512 bytes on either side hold a sentinel
byte pattern; the view itself starts filled with the same pattern.  After the call:
  - the sentinel bytes on both sides are untouched (no store lands outside the output);
  - the output equals, bit for bit, what the same call writes into a fresh unpadded buffer
    (every element is written, and the padding changes nothing).
Shapes are ragged on purpose: rows whose last 512-value slot is cut inside (H = 520, 776,
4128), head counts that are not a multiple of the 8 heads one wave covers, MXFP4 rows whose
code and scale bytes are not a multiple of 4 or 16, and routing sizes on both the two- and the
three-launch paths.  Numerical parity of the same entry points is checked elsewhere.
Each case prints its name and sizes before it runs.
"""
import numpy as np
import pytest
import torch

import finalize_residual_rmsnorm_amd as mf
import workloads

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
PAD = 512          # bytes of sentinel on each side (a multiple of 16: the view stays aligned)
SENTINEL = 0xA5


def say(msg):
    print(msg, flush=True)


def up(a, bf16=False):
    a = np.ascontiguousarray(a)
    t = torch.from_numpy(a.view(np.int16) if bf16 else a)
    if bf16:
        t = t.view(torch.bfloat16)
    return t.to(DEV)


class Guarded:
    """An output tensor of `shape` and `dtype` inside a sentinel-filled byte buffer."""

    def __init__(self, shape, dtype):
        self.nbytes = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        self.buf = torch.full((self.nbytes + 2 * PAD,), SENTINEL, dtype=torch.uint8, device=DEV)
        self.view = self.buf[PAD:PAD + self.nbytes].view(dtype).view(shape)

    def check(self, name, expected):
        head, tail = self.buf[:PAD], self.buf[PAD + self.nbytes:]
        assert torch.all(head == SENTINEL), f"{name}: {int((head != SENTINEL).sum())} bytes before it written"
        assert torch.all(tail == SENTINEL), f"{name}: {int((tail != SENTINEL).sum())} bytes after it written"
        got = self.buf[PAD:PAD + self.nbytes]
        want = expected.contiguous().view(torch.uint8).reshape(-1)
        assert torch.equal(got, want), f"{name}: differs from the unpadded call's output"


def guarded(**outs):
    return {name: Guarded(shape, dtype) for name, (shape, dtype) in outs.items()}


def check_all(g, expected):
    torch.cuda.synchronize()
    for name, t in expected.items():
        g[name].check(name, t)


# ----------------------------------------------------------------------------- finalize


@pytest.mark.parametrize("T,H,k,pe", [(37, 520, 3, False), (9, 776, 8, False), (5, 4128, 8, False),
                                      (3, 7168, 8, True), (11, 520, 5, True),
                                      # wide rows: the slot-serial kernel with slots staged in LDS
                                      (3, 20480, 8, False), (2, 32768, 8, False)])
def test_finalize_guard_bands(T, H, k, pe):
    say(f"guard bands finalize T={T} H={H} k={k} per_expert={pe}")
    d = workloads.make_finalize_inputs(T, H, E=16, k=k, seed=1100 + T + H + k, per_expert=pe,
                                       layout="random")
    kw = dict(expert_ids=up(d["expert_ids"]), expert_gamma=up(d["expert_gamma"], True)) if pe else {}
    args = (up(d["expert_rows"], True), up(d["idx"]), up(d["weights"]), up(d["residual"]),
            up(d["gamma"], True), d["eps"])
    out, r = mf.mf_moe_finalize(*args, **kw)
    g = guarded(out=((T, H), torch.bfloat16), r=((T, H), torch.float32))
    mf.mf_moe_finalize(*args, residual_out=g["r"].view, out=g["out"].view, **kw)
    check_all(g, dict(out=out, r=r))


@pytest.mark.parametrize("T,H,k", [(5, 4128, 8), (37, 544, 3)])
def test_finalize_mxfp4_guard_bands(T, H, k):
    say(f"guard bands finalize mxfp4 T={T} H={H} k={k}")
    d = workloads.make_finalize_inputs(T, H, E=16, k=k, seed=1200 + T + H, layout="random")
    args = (up(d["expert_rows"], True), up(d["idx"]), up(d["weights"]), up(d["residual"]),
            up(d["gamma"], True), d["eps"])
    q, sc, r = mf.mf_moe_finalize_mxfp4(*args)
    g = guarded(q=((T, H // 2), torch.uint8), sc=((T, H // 32), torch.uint8),
                r=((T, H), torch.float32))
    mf.mf_moe_finalize_mxfp4(*args, residual_out=g["r"].view, q=g["q"].view, scales=g["sc"].view)
    check_all(g, dict(q=q, sc=sc, r=r))


# ----------------------------------------------------------------------------- expert parallel


def test_ep_partial_guard_bands():
    T, H, k = 37, 776, 5
    say(f"guard bands ep partial T={T} H={H} k={k}")
    d = workloads.make_finalize_inputs(T, H, E=16, k=k, seed=1300, layout="random")
    idx = workloads.remote_slots_marked(d["idx"], d["expert_ids"], 2, 0)
    args = (up(d["expert_rows"], True), up(idx), up(d["weights"]), d["eps"])
    p = mf.mf_moe_finalize_ep_partial(*args)
    g = guarded(p=((T, H), torch.float32))
    mf.mf_moe_finalize_ep_partial(*args, partial=g["p"].view)
    check_all(g, dict(p=p))


@pytest.mark.parametrize("T,H,G", [(9, 776, 3), (4, 7168, 5)])
def test_ep_combine_guard_bands(T, H, G):
    say(f"guard bands ep combine T={T} H={H} G={G}")
    d = workloads.make_ep_combine_inputs(T, H, G, seed=1400 + T)
    args = (up(d["partials"]), up(d["residual"]), up(d["gamma"], True), d["eps"])
    out, r = mf.mf_moe_finalize_ep_combine(*args)
    g = guarded(out=((T, H), torch.bfloat16), r=((T, H), torch.float32))
    mf.mf_moe_finalize_ep_combine(*args, residual_out=g["r"].view, out=g["out"].view)
    check_all(g, dict(out=out, r=r))


# ----------------------------------------------------------------------------- gated norms


@pytest.mark.parametrize("T,H", [(37, 520), (5, 776), (3, 8192)])
def test_gated_guard_bands(T, H):
    say(f"guard bands gated T={T} H={H}")
    d = workloads.make_gated_inputs(T, H, seed=1500 + T + H)
    args = (up(d["x"], True), up(d["gate"], True), up(d["residual"]), up(d["gamma"], True), d["eps"])
    out, r = mf.mf_gated_residual_rmsnorm(*args)
    g = guarded(out=((T, H), torch.bfloat16), r=((T, H), torch.float32))
    mf.mf_gated_residual_rmsnorm(*args, residual_out=g["r"].view, out=g["out"].view)
    check_all(g, dict(out=out, r=r))


@pytest.mark.parametrize("T,H", [(37, 520), (2, 12288)])
def test_gated_next_guard_bands(T, H):
    say(f"guard bands gated next T={T} H={H}")
    d = workloads.make_gated_inputs(T, H, seed=1600 + T + H, dual=True)
    args = (up(d["x"], True), up(d["gate"], True), up(d["residual"]), up(d["gamma"], True),
            up(d["gamma_next"], True), d["eps"])
    out, on, r = mf.mf_gated_residual_next_rmsnorm(*args)
    g = guarded(out=((T, H), torch.bfloat16), on=((T, H), torch.bfloat16), r=((T, H), torch.float32))
    mf.mf_gated_residual_next_rmsnorm(*args, residual_out=g["r"].view, out=g["out"].view,
                                      out_next=g["on"].view)
    check_all(g, dict(out=out, on=on, r=r))


@pytest.mark.parametrize("T,heads", [(3, 5), (1, 1), (7, 9), (129, 64)])
def test_per_head_guard_bands(T, heads):
    say(f"guard bands per-head T={T} heads={heads}")
    d = workloads.make_per_head_inputs(T, heads, 64, seed=1700 + T + heads)
    args = (up(d["x"], True), up(d["gate"], True), up(d["gamma"], True), d["eps"])
    out = mf.mf_rmsnorm_sigmoid_gate(*args)
    g = guarded(out=((T, heads, 64), torch.bfloat16))
    mf.mf_rmsnorm_sigmoid_gate(*args, out=g["out"].view)
    check_all(g, dict(out=out))


# ----------------------------------------------------------------------------- random shapes


def _random_rows(n, seed, with_k):
    """Seeded random ragged shapes: H a multiple of 8 from 8 to 32768 (log-uniform), T from 1 to
    64, and with_k a top-k from 1 to 64 (every third case per-expert)."""
    g = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        H = 8 * int(np.exp(g.uniform(0.0, np.log(4096.0))))
        T = int(g.integers(1, 65))
        if not with_k:
            cases.append((T, H))
            continue
        k = int(np.exp(g.uniform(0.0, np.log(64.0))))
        if T * k * H <= 4_000_000:
            cases.append((T, H, k, len(cases) % 3 == 2))
    return cases


@pytest.mark.parametrize("T,H,k,pe", _random_rows(16, 20261212, True))
def test_finalize_guard_bands_random_shapes(T, H, k, pe):
    say(f"guard bands finalize random shape T={T} H={H} k={k} per_expert={pe}")
    d = workloads.make_finalize_inputs(T, H, E=max(16, k), k=k, seed=1150 + T + H + k,
                                       per_expert=pe, layout="random")
    kw = dict(expert_ids=up(d["expert_ids"]), expert_gamma=up(d["expert_gamma"], True)) if pe else {}
    args = (up(d["expert_rows"], True), up(d["idx"]), up(d["weights"]), up(d["residual"]),
            up(d["gamma"], True), d["eps"])
    out, r = mf.mf_moe_finalize(*args, **kw)
    g = guarded(out=((T, H), torch.bfloat16), r=((T, H), torch.float32))
    mf.mf_moe_finalize(*args, residual_out=g["r"].view, out=g["out"].view, **kw)
    check_all(g, dict(out=out, r=r))


@pytest.mark.parametrize("T,H", _random_rows(10, 20261213, False))
def test_gated_guard_bands_random_shapes(T, H):
    say(f"guard bands gated random shape T={T} H={H}")
    d = workloads.make_gated_inputs(T, H, seed=1550 + T + H)
    args = (up(d["x"], True), up(d["gate"], True), up(d["residual"]), up(d["gamma"], True), d["eps"])
    out, r = mf.mf_gated_residual_rmsnorm(*args)
    g = guarded(out=((T, H), torch.bfloat16), r=((T, H), torch.float32))
    mf.mf_gated_residual_rmsnorm(*args, residual_out=g["r"].view, out=g["out"].view)
    check_all(g, dict(out=out, r=r))


@pytest.mark.parametrize("T,heads", [(int(t), int(h)) for t, h in
                                     np.random.default_rng(20261214).integers(1, 97, (8, 2))])
def test_per_head_guard_bands_random_shapes(T, heads):
    test_per_head_guard_bands(T, heads)


# ----------------------------------------------------------------------------- MXFP4


@pytest.mark.parametrize("T,H", [(3, 544), (1, 32), (5, 4128)])
def test_mxfp4_guard_bands(T, H):
    say(f"guard bands mxfp4 quantize and rmsnorm + mxfp4 T={T} H={H}")
    x = workloads.make_gated_inputs(T, H, seed=1800 + T + H)["residual"]
    q, sc = mf.mf_mxfp4_quantize(up(x))
    g = guarded(q=((T, H // 2), torch.uint8), sc=((T, H // 32), torch.uint8))
    mf.mf_mxfp4_quantize(up(x), q=g["q"].view, scales=g["sc"].view)
    check_all(g, dict(q=q, sc=sc))
    d = workloads.make_rmsnorm_mx_inputs(T, H, seed=1900 + T + H)
    args = (up(d["x"], True), up(d["gamma"], True), d["eps"])
    q, sc = mf.mf_rmsnorm_mxfp4_quantize(*args)
    g = guarded(q=((T, H // 2), torch.uint8), sc=((T, H // 32), torch.uint8))
    mf.mf_rmsnorm_mxfp4_quantize(*args, q=g["q"].view, scales=g["sc"].view)
    check_all(g, dict(q=q, sc=sc))


# ----------------------------------------------------------------------------- routing


@pytest.mark.parametrize("T,E,k", [(37, 96, 8), (5000, 256, 8), (3, 1024, 16)])
def test_route_guard_bands(T, E, k):
    say(f"guard bands route T={T} E={E} k={k}")
    logits = up(workloads.make_route_inputs(T, E, k, seed=2000 + T + E)["logits"])
    ref = mf.mf_moe_route(logits, k)
    g = guarded(expert_ids=((T, k), torch.int32), weights=((T, k), torch.float32),
                idx=((T, k), torch.int32), perm=((T * k,), torch.int32),
                offsets=((E + 1,), torch.int32))
    mf.mf_moe_route(logits, k, **{n: v.view for n, v in g.items()})
    check_all(g, dict(zip(["expert_ids", "weights", "idx", "perm", "offsets"], ref)))
