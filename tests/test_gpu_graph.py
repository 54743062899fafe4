"""The entry points inside a captured HIP graph (through torch.cuda.CUDAGraph).

The library allocates nothing, never synchronises and records no memset, so a caller can capture
its launches (a decode loop, say) and replay them.  One graph holds a finalize, a gated-residual
norm, a per-head norm and a routing call (three kernels).  It is replayed three times with eager
work between the replays (the outputs wiped, unrelated torch kernels run); every replay must give
the eager results bit for bit.  Then new inputs are copied into the captured buffers and one more
replay must give the eager results for those.
"""
import numpy as np
import pytest
import torch

import finalize_residual_rmsnorm_amd as mf
import workloads

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


def inputs(seed):
    f = workloads.make_finalize_inputs(257, 7168, E=64, k=8, seed=seed)
    g = workloads.make_gated_inputs(100, 8192, seed=seed + 1)
    h = workloads.make_per_head_inputs(50, 64, 64, seed=seed + 2)
    r = workloads.make_route_inputs(300, 256, 8, seed=seed + 3)
    return dict(
        rows=up(f["expert_rows"], True), idx=up(f["idx"]), w=up(f["weights"]),
        res=up(f["residual"]), gamma=up(f["gamma"], True),
        gx=up(g["x"], True), gg=up(g["gate"], True), gres=up(g["residual"]),
        ggamma=up(g["gamma"], True),
        hx=up(h["x"], True), hg=up(h["gate"], True), hgamma=up(h["gamma"], True),
        logits=up(r["logits"]),
    )


def outputs(src):
    e = lambda t, dt=None: torch.empty_like(t, dtype=dt or t.dtype)
    T, k = src["idx"].shape
    Tr = src["logits"].shape[0]
    return dict(
        r=e(src["res"]), out=e(src["res"], torch.bfloat16), gr=e(src["gres"]),
        gout=e(src["gres"], torch.bfloat16), hout=e(src["hx"]),
        eids=torch.empty((Tr, 8), dtype=torch.int32, device=DEV),
        ew=torch.empty((Tr, 8), dtype=torch.float32, device=DEV),
        ridx=torch.empty((Tr, 8), dtype=torch.int32, device=DEV),
        perm=torch.empty((Tr * 8,), dtype=torch.int32, device=DEV),
        offs=torch.empty((257,), dtype=torch.int32, device=DEV),
        ws=torch.empty((mf.mf_moe_route_workspace_bytes(Tr, 256, 8),), dtype=torch.uint8,
                       device=DEV),
    )


def launch_all(src, o):
    mf.mf_moe_finalize(src["rows"], src["idx"], src["w"], src["res"], src["gamma"], 1e-6,
                       residual_out=o["r"], out=o["out"])
    mf.mf_gated_residual_rmsnorm(src["gx"], src["gg"], src["gres"], src["ggamma"], 1e-6,
                                 residual_out=o["gr"], out=o["gout"])
    mf.mf_rmsnorm_sigmoid_gate(src["hx"], src["hg"], src["hgamma"], 1e-6, out=o["hout"])
    mf.mf_moe_route(src["logits"], 8, expert_ids=o["eids"], weights=o["ew"], idx=o["ridx"],
                    perm=o["perm"], offsets=o["offs"], workspace=o["ws"])


def snapshot(o):
    return {k: v.clone() for k, v in o.items() if k != "ws"}


def same(a, b):
    for k in a:
        x, y = a[k], b[k]
        if x.dtype == torch.bfloat16:
            x, y = x.view(torch.int16), y.view(torch.int16)
        if not torch.equal(x, y):
            return k
    return None


def test_graph_replays_match_eager():
    say("graph: finalize T=257 H=7168 k=8, gated T=100 H=8192, per-head T=50x64, route T=300 E=256")
    src = inputs(61)
    o = outputs(src)
    launch_all(src, o)
    torch.cuda.synchronize()
    eager = snapshot(o)

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        launch_all(src, o)
    torch.cuda.synchronize()

    for rep in range(3):
        for v in o.values():
            v.zero_()
        junk = torch.randn(1 << 20, device=DEV).sum()  # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        bad = same(eager, snapshot(o))
        assert bad is None, f"replay {rep}: {bad} differs from the eager result"
        assert torch.isfinite(junk)

    # new inputs copied into the captured buffers: the replay follows them
    src2 = inputs(62)
    o2 = outputs(src2)
    launch_all(src2, o2)
    torch.cuda.synchronize()
    for k2 in src:
        src[k2].copy_(src2[k2])
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    bad = same(snapshot(o2), snapshot(o))
    assert bad is None, f"replay with new inputs: {bad} differs from the eager result"


def test_graph_wide_per_expert_and_noalloc_route():
    """A second captured graph with this library's other launch paths: the slot-serial finalize of
    wide rows (H=12288, k=8), the per-expert finalize, and the routing call on the library's static
    scratch (the allocation-free form made for captured graphs: it looks up its scratch on the
    first, eager, call and allocates nothing).  Replayed three times with eager work between;
    every replay matches the eager results bit for bit."""
    say("graph 2: wide finalize T=40 H=12288 k=8, per-expert finalize T=33 H=4096 k=8, "
        "route_noalloc T=300 E=256 k=8")
    f = workloads.make_finalize_inputs(40, 12288, E=64, k=8, seed=71)
    p = workloads.make_finalize_inputs(33, 4096, E=32, k=8, seed=72, per_expert=True)
    r = workloads.make_route_inputs(300, 256, 8, seed=73)
    src = dict(rows=up(f["expert_rows"], True), idx=up(f["idx"]), w=up(f["weights"]),
               res=up(f["residual"]), gamma=up(f["gamma"], True),
               prows=up(p["expert_rows"], True), pidx=up(p["idx"]), pw=up(p["weights"]),
               pres=up(p["residual"]), pgamma=up(p["gamma"], True), peids=up(p["expert_ids"]),
               pegamma=up(p["expert_gamma"], True), logits=up(r["logits"]))
    e = lambda shape, dt: torch.empty(shape, dtype=dt, device=DEV)
    o = dict(r=e((40, 12288), torch.float32), out=e((40, 12288), torch.bfloat16),
             pr=e((33, 4096), torch.float32), pout=e((33, 4096), torch.bfloat16),
             eids=e((300, 8), torch.int32), ew=e((300, 8), torch.float32),
             ridx=e((300, 8), torch.int32), perm=e((2400,), torch.int32), offs=e((257,), torch.int32))

    def launch():
        mf.mf_moe_finalize(src["rows"], src["idx"], src["w"], src["res"], src["gamma"], 1e-6,
                           residual_out=o["r"], out=o["out"])
        mf.mf_moe_finalize(src["prows"], src["pidx"], src["pw"], src["pres"], src["pgamma"], 1e-6,
                           expert_ids=src["peids"], expert_gamma=src["pegamma"],
                           residual_out=o["pr"], out=o["pout"])
        mf.mf_moe_route_noalloc(src["logits"], 8, expert_ids=o["eids"], weights=o["ew"],
                                idx=o["ridx"], perm=o["perm"], offsets=o["offs"])

    assert mf.mf_launch_shape(0, 40, 12288, 8)["vectors_per_lane"] == 3   # the wide kernel's shape
    launch()
    torch.cuda.synchronize()
    eager = snapshot(o)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        launch()
    torch.cuda.synchronize()
    for rep in range(3):
        for v in o.values():
            v.zero_()
        junk = torch.randn(1 << 20, device=DEV).sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        bad = same(eager, snapshot(o))
        assert bad is None, f"replay {rep}: {bad} differs from the eager result"
        assert torch.isfinite(junk)
