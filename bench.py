"""Throughput of the MoE finalize hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the path over one batch of seeded synthetic inputs already resident
in HBM: for the default workload, one mf_moe_finalize launch at T=16384, H=7168, E=256,
k=8, which gathers the k rows, accumulates them in fp32, adds and stores the residual and
emits the RMSNorm output.  The inputs follow the configured recipe: router logits ~ N(0, 1),
routed on the GPU by mf_moe_route (top-8, softmax over the 8, rows stably sorted by expert id)
before the timed region.  W untimed steps, then exactly K timed steps between device
synchronisations; one JSON line on stdout.

Timing: a calibrated spin kernel first keeps the GPU busy while the K launches are enqueued on
the launch stream, so the GPU runs them back to back, and two HIP events on that stream bracket
the K launches: the kernels' time, not the host's launch gaps.  value, ms_per_step and the
kernel's average launch duration come from that span.  A second pass puts an event pair around
every launch for the spread (p10/median/p90; each pair adds its own few microseconds).
roofline: algorithmic HBM bytes of one launch / the kernel's average launch duration; peak
8 TB/s.  traffic: HBM bytes per launch measured with rocprofv3 counters, read from the
committed summary under profiles/ when it was taken from the current kernel sources, else null.
cpu_baseline: the CPU oracle (with its own routing of the same logits) timed on a bounded
sample of the workload on the host's CPU share; beside it, a sampled parity check of the GPU
path against the oracle on the same inputs.
Other workloads (--workload) time the one-token decode finalizes, the sibling kernels (the
gated norms, single and dual output, and the per-head norm), RMSNorm + MXFP4 quantisation,
the expert-parallel partial and combine steps, the routing producer (one step = one
mf_moe_route call: its kernels, timed together by the events around the call) and the copy
used for calibration.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "finalize tokens/s + achieved HBM GB/s (% of peak) at T=16384,H=7168,k=8"
PEAK_GBPS = 8000.0
MALL_BYTES = 256 << 20
MAX_INPUT_SETS = 8192   # rotated copies of a small workload's inputs (cold data every step)
WORKLOAD_CHOICES = ["finalize_prefill", "finalize_1tok", "finalize_1tok_per_expert",
                    "finalize_wide_12288", "finalize_wide_20480", "finalize_wide_32768",
                    "finalize_decode_per_expert", "finalize_tiny", "gated_residual_rmsnorm",
                    "gated_residual_next_rmsnorm", "rmsnorm_sigmoid_gate", "moe_route_prefill",
                    "finalize_ep_partial", "finalize_ep_combine", "rmsnorm_mxfp4",
                    "finalize_prefill_mxfp4", "moe_route_decode", "stream_copy",
                    "stream_copy_per_head", "empty_grid_per_head", "stream_read", "torch_copy", "stream_copy_gated",
                    "stream_copy_rmsnorm_mxfp4", "empty_grid_1tok"]
CSRC = os.path.join(ROOT, "finalize_residual_rmsnorm_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")


# The sources each kind of kernel is built from (launch code included): a counter summary
# stays valid while these are unchanged.
_NORM_SOURCES = ["mf_device.h", "row_norm.h", "norm_kernels.h", "api_util.h", "row_shape.h",
                 "norm_api.hip"]
KERNEL_SOURCES = {
    "finalize": ["mf_device.h", "row_norm.h", "finalize_kernel.h", "mx_device.h", "api_util.h",
                 "row_shape.h", "mf_api.hip"],
    "ep_partial": ["mf_device.h", "row_norm.h", "finalize_kernel.h", "mx_device.h", "api_util.h",
                   "row_shape.h", "mf_api.hip"],
    "finalize_mx": ["mf_device.h", "row_norm.h", "finalize_kernel.h", "mx_device.h", "api_util.h",
                    "row_shape.h", "mf_api.hip"],
    "ep_combine": ["mf_device.h", "row_norm.h", "finalize_kernel.h", "mx_device.h", "api_util.h",
                   "row_shape.h", "mf_api.hip"],
    "gated": _NORM_SOURCES,
    "gated_next": _NORM_SOURCES,
    "per_head": _NORM_SOURCES,
    "copy": _NORM_SOURCES,
    "read": _NORM_SOURCES,
    "empty_grid": _NORM_SOURCES,
    "route": ["mf_device.h", "route_kernels.h", "api_util.h", "route_api.hip"],
    "rmsnorm_mx": ["mf_device.h", "row_norm.h", "mx_device.h", "mx_kernels.h", "api_util.h",
                   "row_shape.h", "mx_api.hip"],
}


def kernel_source_digest(kind: str = "finalize") -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kind]:
        h.update(name.encode())
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def read_traffic(workload: str, kind: str):
    """HBM bytes per launch from the committed counter summary, if it matches the sources."""
    path = os.path.join(PROFILES, f"traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256") != kernel_source_digest(kind):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# ------------------------------------------------------------------------------ workloads


def algorithmic_bytes(d: dict) -> int:
    """Bytes the method must move once: every input read once, every output written once."""
    kind = d["kind"]
    if kind == "finalize":
        T, H, k = d["T"], d["H"], d["k"]
        b = T * (k * H * 2 + H * 4 + H * 4 + H * 2 + k * 8) + H * 2
        if d.get("expert_gamma") is not None:
            b += T * k * 4 + len(np.unique(d["expert_ids"])) * H * 2
        return b
    if kind == "rmsnorm_mx":
        T, H = d["T"], d["H"]
        return T * H * 2 + H * 2 + T * H // 2 + T * H // 32   # x, gamma in; codes, scales out
    if kind == "finalize_mx":
        T, H, k = d["T"], d["H"], d["k"]
        return T * (k * H * 2 + H * 4 + H * 4 + H // 2 + H // 32 + k * 8) + H * 2
    if kind == "ep_partial":
        # local rows read, every idx read, local weights read, the fp32 partial written
        T, H, k = d["T"], d["H"], d["k"]
        local = int((d["idx"] >= 0).sum())
        return local * (H * 2 + 4) + T * k * 4 + T * H * 4
    if kind == "ep_combine":
        T, H, G = d["T"], d["H"], d["G"]
        return G * T * H * 4 + T * H * (4 + 4 + 2) + H * 2
    if kind == "gated":
        T, H = d["T"], d["H"]
        return T * H * (2 + 2 + 4 + 4 + 2) + H * 2
    if kind == "gated_next":
        T, H = d["T"], d["H"]
        return T * H * (2 + 2 + 4 + 4 + 2 + 2) + 2 * H * 2
    if kind == "per_head":
        n = d["T"] * d["heads"] * d["D"]
        return n * 6 + d["D"] * 2
    if kind in ("copy", "torch_copy"):
        return 2 * d["bytes"]
    if kind == "read":
        return d["bytes"] + -(-d["bytes"] // 16384) * 4   # src read; one sink word per 16 KiB
    if kind == "empty_grid":
        return 0
    if kind == "route":
        T, E, k = d["T"], d["E"], d["k"]
        return T * E * 4 + T * k * 16 + (E + 1) * 4   # logits in; ids, weights, idx, perm out
    raise ValueError(kind)


def tokens_of(d: dict) -> int:
    return d["T"] if "T" in d else 0


# The per-head norm's bytes (4096 tokens x 64 heads x 64 values: x and gate read, out written),
# the gated-residual norm's (4096 x 8192: x, gate, residual read; residual, out written; gamma)
# and RMSNorm + MXFP4's (4096 x 8192: x read; codes and scales written; gamma)
PER_HEAD_BYTES = 4096 * 64 * 64 * 6 + 64 * 2
GATED_BYTES = 4096 * 8192 * 14 + 8192 * 2
RMSNORM_MX_BYTES = 4096 * 8192 * 2 + 8192 * 2 + 4096 * 8192 // 2 + 4096 * 8192 // 32


def make_workload(name: str, overrides: dict | None = None) -> dict:
    """A named workload; `overrides` (integer sizes or seed, e.g. {"H": 2048, "k": 4}) change a
    generated workload's parameters (the measurement aids take none)."""
    import workloads
    if overrides:
        if name not in workloads.WORKLOADS:
            raise ValueError(f"{name} takes no overrides")
        return workloads.make_inputs(name, **overrides)
    if name == "stream_copy":
        return dict(kind="copy", bytes=1 << 30)
    if name == "stream_copy_per_head":
        # a plain copy moving the per-head norm's byte count (half read, half written)
        return dict(kind="copy", bytes=PER_HEAD_BYTES // 2 // 16 * 16)
    if name == "stream_copy_gated":
        return dict(kind="copy", bytes=GATED_BYTES // 2 // 16 * 16)
    if name == "stream_copy_rmsnorm_mxfp4":
        return dict(kind="copy", bytes=RMSNORM_MX_BYTES // 2 // 16 * 16)
    if name == "empty_grid_per_head":
        # an empty kernel of the per-head norm's grid: 8 heads per one-wave workgroup
        return dict(kind="empty_grid", workgroups=4096 * 64 // 8, threads=64)
    if name == "empty_grid_1tok":
        # an empty kernel of the one-token finalize's launch: one workgroup of 16 waves
        return dict(kind="empty_grid", workgroups=1, threads=1024)
    if name == "stream_read":
        return dict(kind="read", bytes=1 << 30)
    # PyTorch's own copy of 1 GiB, an outside reference for the copy rate
    if name == "torch_copy":
        return dict(kind="torch_copy", bytes=1 << 30)
    return workloads.make_inputs(name)


def route_on_gpu(d: dict, dev) -> dict:
    """A finalize workload drawn with router logits, completed by the GPU routing call (expert
    ids, weights and the expert-sorted idx), before any timing.  Other workloads pass through."""
    if d.get("routing") != "logits":
        return d
    import torch

    import finalize_residual_rmsnorm_amd as mf
    import workloads
    eids, w, idx, _, _ = mf.mf_moe_route(torch.from_numpy(d["logits"]).to(dev), d["k"])
    torch.cuda.synchronize()
    return workloads.with_routing(d, eids.cpu().numpy(), w.cpu().numpy(), idx.cpu().numpy())


def upload(d: dict, dev):
    import torch

    def up(a, bf16=False):
        a = np.ascontiguousarray(a)
        t = torch.from_numpy(a.view(np.int16) if bf16 else a)
        return (t.view(torch.bfloat16) if bf16 else t).to(dev)

    kind = d["kind"]
    if kind == "finalize":
        g = dict(rows=up(d["expert_rows"], True), idx=up(d["idx"]), w=up(d["weights"]),
                 res=up(d["residual"]), gamma=up(d["gamma"], True))
        if d.get("expert_gamma") is not None:
            g.update(eids=up(d["expert_ids"]), egamma=up(d["expert_gamma"], True))
        T, H = d["T"], d["H"]
        g["res_out"] = torch.empty((T, H), dtype=torch.float32, device=dev)
        g["out"] = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
        return g
    if kind == "gated":
        T, H = d["T"], d["H"]
        return dict(x=up(d["x"], True), gate=up(d["gate"], True), res=up(d["residual"]),
                    gamma=up(d["gamma"], True),
                    res_out=torch.empty((T, H), dtype=torch.float32, device=dev),
                    out=torch.empty((T, H), dtype=torch.bfloat16, device=dev))
    if kind == "finalize_mx":
        T, H = d["T"], d["H"]
        return dict(rows=up(d["expert_rows"], True), idx=up(d["idx"]), w=up(d["weights"]),
                    res=up(d["residual"]), gamma=up(d["gamma"], True),
                    res_out=torch.empty((T, H), dtype=torch.float32, device=dev),
                    q=torch.empty((T, H // 2), dtype=torch.uint8, device=dev),
                    sc=torch.empty((T, H // 32), dtype=torch.uint8, device=dev))
    if kind == "rmsnorm_mx":
        T, H = d["T"], d["H"]
        return dict(x=up(d["x"], True), gamma=up(d["gamma"], True),
                    q=torch.empty((T, H // 2), dtype=torch.uint8, device=dev),
                    sc=torch.empty((T, H // 32), dtype=torch.uint8, device=dev))
    if kind == "ep_partial":
        T, H = d["T"], d["H"]
        return dict(rows=up(d["expert_rows"], True), idx=up(d["idx"]), w=up(d["weights"]),
                    part=torch.empty((T, H), dtype=torch.float32, device=dev))
    if kind == "ep_combine":
        T, H = d["T"], d["H"]
        return dict(parts=up(d["partials"]), res=up(d["residual"]), gamma=up(d["gamma"], True),
                    res_out=torch.empty((T, H), dtype=torch.float32, device=dev),
                    out=torch.empty((T, H), dtype=torch.bfloat16, device=dev))
    if kind == "gated_next":
        T, H = d["T"], d["H"]
        e = lambda dt: torch.empty((T, H), dtype=dt, device=dev)
        return dict(x=up(d["x"], True), gate=up(d["gate"], True), res=up(d["residual"]),
                    gamma=up(d["gamma"], True), gamma_next=up(d["gamma_next"], True),
                    res_out=e(torch.float32), out=e(torch.bfloat16), out_next=e(torch.bfloat16))
    if kind == "per_head":
        x = up(d["x"], True)
        return dict(x=x, gate=up(d["gate"], True), gamma=up(d["gamma"], True),
                    out=torch.empty_like(x))
    if kind in ("copy", "torch_copy"):
        n = d["bytes"] // 4
        return dict(src=torch.randint(0, 1 << 30, (n,), dtype=torch.int32, device=dev),
                    dst=torch.empty(n, dtype=torch.int32, device=dev))
    if kind == "read":
        n = d["bytes"] // 4
        return dict(src=torch.randint(0, 1 << 30, (n,), dtype=torch.int32, device=dev),
                    sink=torch.empty(-(-d["bytes"] // 16384), dtype=torch.int32, device=dev))
    if kind == "empty_grid":
        return {}
    if kind == "route":
        import finalize_residual_rmsnorm_amd as mf
        T, E, k = d["T"], d["E"], d["k"]
        e = lambda shape, dt: torch.empty(shape, dtype=dt, device=dev)
        return dict(logits=up(d["logits"]), eids=e((T, k), torch.int32),
                    w=e((T, k), torch.float32), idx=e((T, k), torch.int32),
                    perm=e((T * k,), torch.int32), off=e((E + 1,), torch.int32),
                    ws=e((mf.mf_moe_route_workspace_bytes(T, E, k),), torch.uint8))
    raise ValueError(kind)


def launcher(d: dict, g: dict):
    import finalize_residual_rmsnorm_amd as mf
    kind = d["kind"]
    if kind == "finalize":
        kw = {}
        if "egamma" in g:
            kw = dict(expert_ids=g["eids"], expert_gamma=g["egamma"])
        return lambda: mf.mf_moe_finalize(g["rows"], g["idx"], g["w"], g["res"], g["gamma"],
                                          d["eps"], residual_out=g["res_out"], out=g["out"], **kw)
    if kind == "gated":
        return lambda: mf.mf_gated_residual_rmsnorm(g["x"], g["gate"], g["res"], g["gamma"],
                                                    d["eps"], residual_out=g["res_out"],
                                                    out=g["out"])
    if kind == "finalize_mx":
        return lambda: mf.mf_moe_finalize_mxfp4(g["rows"], g["idx"], g["w"], g["res"], g["gamma"],
                                                d["eps"], residual_out=g["res_out"], q=g["q"],
                                                scales=g["sc"])
    if kind == "rmsnorm_mx":
        return lambda: mf.mf_rmsnorm_mxfp4_quantize(g["x"], g["gamma"], d["eps"], q=g["q"],
                                                    scales=g["sc"])
    if kind == "ep_partial":
        return lambda: mf.mf_moe_finalize_ep_partial(g["rows"], g["idx"], g["w"], d["eps"],
                                                     partial=g["part"])
    if kind == "ep_combine":
        return lambda: mf.mf_moe_finalize_ep_combine(g["parts"], g["res"], g["gamma"], d["eps"],
                                                     residual_out=g["res_out"], out=g["out"])
    if kind == "gated_next":
        return lambda: mf.mf_gated_residual_next_rmsnorm(
            g["x"], g["gate"], g["res"], g["gamma"], g["gamma_next"], d["eps"],
            residual_out=g["res_out"], out=g["out"], out_next=g["out_next"])
    if kind == "per_head":
        return lambda: mf.mf_rmsnorm_sigmoid_gate(g["x"], g["gate"], g["gamma"], d["eps"],
                                                  out=g["out"])
    if kind == "copy":
        return lambda: mf.mf_stream_copy(g["src"], g["dst"])
    if kind == "torch_copy":
        return lambda: g["dst"].copy_(g["src"])
    if kind == "read":
        return lambda: mf.mf_stream_read(g["src"], g["sink"])
    if kind == "empty_grid":
        return lambda: mf.mf_empty_grid(d["workgroups"], d["threads"])
    if kind == "route":
        return lambda: mf.mf_moe_route(g["logits"], d["k"], expert_ids=g["eids"], weights=g["w"],
                                       idx=g["idx"], perm=g["perm"], offsets=g["off"],
                                       workspace=g["ws"])
    raise ValueError(kind)


def launch_config(name: str, d: dict) -> dict:
    import finalize_residual_rmsnorm_amd as mf
    kind = d["kind"]
    if kind in ("finalize", "ep_partial", "finalize_mx"):
        pe = d.get("expert_gamma") is not None
        plain = mf.KIND_EP_PARTIAL if kind == "ep_partial" else mf.KIND_FINALIZE
        return mf.mf_launch_shape(mf.KIND_FINALIZE_PER_EXPERT if pe else plain,
                                  d["T"], d["H"], d["k"])
    if kind == "ep_combine":
        return mf.mf_launch_shape(mf.KIND_EP_COMBINE, d["T"], d["H"])
    if kind in ("gated", "gated_next"):
        return mf.mf_launch_shape(mf.KIND_GATED, d["T"], d["H"])
    return {}


# ------------------------------------------------------------------------------ CPU oracle


def cpu_share() -> int:
    """Host threads this process may use: its CPU affinity, capped by OMP_NUM_THREADS when set
    (a host shared by several GPUs may allot each GPU a share of its cores and say so there)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    omp = os.environ.get("OMP_NUM_THREADS", "")
    if omp.isdigit() and int(omp) > 0:
        n = min(n, int(omp))
    return max(1, n)


def oracle_inputs(d: dict) -> dict:
    """The workload as the oracle sees it: a logits-recipe finalize completed with the oracle's
    own routing of the same logits (nothing the GPU computed enters the oracle)."""
    if d.get("routing") != "logits":
        return d
    import oracle
    import workloads
    eids, w, idx, _, _ = oracle.moe_route(d["logits"], d["k"])
    return workloads.with_routing(d, eids, w, idx)


def parity_sample(d_raw: dict, d_gpu: dict, d_cpu: dict, dev, n: int = 256) -> dict:
    """Parity of the timed path with the oracle on the bench's own inputs, before timing:
    - routing (logits recipe): the GPU's expert ids and idx equal the oracle's;
    - finalize: one launch on the oracle-routed inputs; on n sampled tokens (the first and the
      last among them) residual_out bit-identical to the oracle's (plain finalize) or within
      1e-6 + 1e-5 |r| (per-expert), and out within one bf16 ulp of the oracle's out (plain) or
      of the oracle's RMSNorm of the GPU's residual_out (per-expert: the zero-weight finalize).
    Other workloads: None (their parity is the GPU tests')."""
    if d_raw["kind"] != "finalize":
        return None
    import torch

    import oracle
    rep = {}
    if d_raw.get("routing") == "logits":
        same_ids = bool(np.array_equal(d_gpu["expert_ids"], d_cpu["expert_ids"]))
        same_idx = bool(np.array_equal(d_gpu["idx"], d_cpu["idx"]))
        rep["routing_ids_and_idx_bit_identical"] = same_ids and same_idx
    T = d_cpu["T"]
    rng = np.random.default_rng(0)
    tok = np.unique(np.concatenate([[0, T - 1], rng.choice(T, min(n, T), replace=False)]))
    g = upload(d_cpu, dev)
    launcher(d_cpu, g)()
    torch.cuda.synchronize()
    r_gpu = g["res_out"].cpu().numpy()[tok]
    o_gpu = g["out"].view(torch.int16).cpu().numpy().view(np.uint16)[tok]
    pe = d_cpu.get("expert_gamma") is not None
    kw = dict(expert_ids=d_cpu["expert_ids"][tok], expert_gamma=d_cpu["expert_gamma"]) if pe else {}
    r_ref, o_ref = oracle.moe_finalize(d_cpu["expert_rows"], d_cpu["idx"][tok],
                                       d_cpu["weights"][tok], d_cpu["residual"][tok],
                                       d_cpu["gamma"], d_cpu["eps"], **kw)
    if pe:
        r64 = r_ref.astype(np.float64)
        rep["residual_out_within_tolerance"] = bool(
            np.all(np.abs(r_gpu - r64) <= 1e-6 + 1e-5 * np.abs(r64)))
        H = d_cpu["H"]
        _, o_ref = oracle.moe_finalize(np.zeros((1, H), np.uint16),
                                       np.zeros((len(tok), 1), np.int32),
                                       np.zeros((len(tok), 1), np.float32), r_gpu,
                                       d_cpu["gamma"], d_cpu["eps"])
    else:
        rep["residual_out_bit_identical"] = bool(np.array_equal(r_gpu, r_ref))

    def ordered(b):
        v = b.astype(np.int32)
        return np.where(v & 0x8000, -(v & 0x7FFF), v)

    ulp = np.abs(ordered(o_gpu) - ordered(o_ref))
    rep["out_max_bf16_ulp"] = int(ulp.max())
    rep["out_bit_identical_fraction"] = float((ulp == 0).mean())
    rep["tokens_checked"] = int(len(tok))
    rep["ok"] = bool(all(v for k_, v in rep.items() if k_.endswith("identical") or
                         k_.endswith("tolerance")) and ulp.max() <= 1)
    return rep


def cpu_baseline(d: dict, target_cpu_s: float = 20.0) -> dict:
    """The CPU oracle as it stands on a bounded sample (about target_cpu_s of CPU work) of the
    workload's tokens, split into token blocks over the host threads of this process's CPU
    share (the call releases the GIL); and one thread on one such block."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle

    kind = d["kind"]

    def run(lo: int, hi: int):
        if kind == "finalize":
            kw = {}
            if d.get("expert_gamma") is not None:
                kw = dict(expert_ids=d["expert_ids"][lo:hi], expert_gamma=d["expert_gamma"])
            oracle.moe_finalize(d["expert_rows"], d["idx"][lo:hi], d["weights"][lo:hi],
                                d["residual"][lo:hi], d["gamma"], d["eps"], **kw)
        elif kind == "gated":
            oracle.gated_residual_rmsnorm(d["x"][lo:hi], d["gate"][lo:hi], d["residual"][lo:hi],
                                          d["gamma"], d["eps"])
        elif kind == "gated_next":
            oracle.gated_residual_next_rmsnorm(d["x"][lo:hi], d["gate"][lo:hi],
                                               d["residual"][lo:hi], d["gamma"], d["gamma_next"],
                                               d["eps"])
        elif kind == "per_head":
            oracle.rmsnorm_sigmoid_gate(d["x"][lo:hi], d["gate"][lo:hi], d["gamma"], d["eps"])
        elif kind == "route":
            oracle.moe_route(d["logits"][lo:hi], d["k"])
        elif kind == "rmsnorm_mx":
            oracle.rmsnorm_mxfp4_quantize(d["x"][lo:hi], d["gamma"], d["eps"])
        elif kind == "finalize_mx":
            r, _ = oracle.moe_finalize(d["expert_rows"], d["idx"][lo:hi], d["weights"][lo:hi],
                                       d["residual"][lo:hi], d["gamma"], d["eps"])
            oracle.rmsnorm_f32_mxfp4_quantize(r, d["gamma"], d["eps"])
        elif kind == "ep_partial":
            oracle.moe_finalize_ep_partial(d["expert_rows"], d["idx"][lo:hi], d["weights"][lo:hi],
                                           d["eps"])
        elif kind == "ep_combine":
            oracle.moe_finalize_ep_combine(d["partials"][:, lo:hi], d["residual"][lo:hi],
                                           d["gamma"], d["eps"])

    T = d["T"]
    threads = cpu_share()
    probe = min(T, 64)
    t0 = time.perf_counter()
    run(0, probe)
    per_token = (time.perf_counter() - t0) / probe           # one thread
    n = int(min(T, max(threads, target_cpu_s / max(per_token, 1e-9))))
    n = max(threads, (n // threads) * threads) if T >= threads else T
    chunk = max(1, n // threads)
    spans = [(i, min(n, i + chunk)) for i in range(0, n, chunk)]
    # a sample smaller than the target (the whole workload) is run again until about the
    # target amount of CPU work is done, so the timing is not dominated by thread start-up
    with ThreadPoolExecutor(len(spans)) as ex:
        t0 = time.perf_counter()
        list(ex.map(lambda s: run(*s), spans))
        first = time.perf_counter() - t0
        reps = max(1, int(target_cpu_s / threads / max(first, 1e-9)))
        t0 = time.perf_counter()
        for _ in range(reps):
            list(ex.map(lambda s: run(*s), spans))
        dt = time.perf_counter() - t0
    # one thread on one token block of the same size, for about a fifth of the target
    one = spans[0][1] - spans[0][0]
    reps1 = max(1, int(target_cpu_s / 5 / max(one * per_token, 1e-9)))
    t0 = time.perf_counter()
    for _ in range(reps1):
        run(0, one)
    dt1 = time.perf_counter() - t0
    what = f"the first {n} of {T} tokens" if n < T else f"all {T} tokens"
    host = host_cpu()
    return dict(value=n * reps / dt, unit="tokens/s", cores=len(spans), kind="oracle",
                sample=f"{what} of the same inputs (routed by the oracle), {reps} pass(es), "
                       f"{len(spans)} threads over token blocks, {dt:.1f} s wall; the threads are "
                       f"this process's CPU share ({threads} of the host's "
                       f"{host['logical_cpus']} logical CPUs)",
                value_1_thread=one * reps1 / dt1,
                sample_1_thread=f"the first {one} tokens, {reps1} pass(es), {dt1:.1f} s",
                cpu_share=threads, host=host)


def host_cpu() -> dict:
    """The host's CPU as lscpu reports it (model string, sockets, cores, logical CPUs)."""
    info = {"logical_cpus": os.cpu_count()}
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        keys = {"Model name": "model", "Socket(s)": "sockets",
                "Core(s) per socket": "cores_per_socket", "Thread(s) per core": "threads_per_core",
                "CPU(s)": "lscpu_cpus", "Vendor ID": "vendor"}
        for line in out.splitlines():
            if ":" in line:
                k, v = line.split(":", 1)
                if k.strip() in keys:
                    info[keys[k.strip()]] = v.strip()
    except (OSError, ValueError, subprocess.SubprocessError):
        pass
    if "model" not in info:
        try:
            for line in open("/proc/cpuinfo"):
                if line.startswith("model name"):
                    info["model"] = line.split(":", 1)[1].strip()
                    break
        except OSError:
            info["model"] = "unknown"
    try:
        info["physical_cores"] = int(info["sockets"]) * int(info["cores_per_socket"])
    except (KeyError, ValueError):
        pass
    return info


# ------------------------------------------------------------------------------ timing


def spin_cycles_per_us() -> float:
    """Clock cycles torch.cuda._sleep spins per microsecond (measured once with events)."""
    import torch
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(1000)
    cycles = 2_000_000
    a.record()
    torch.cuda._sleep(cycles)
    b.record()
    torch.cuda.synchronize()
    return cycles / max(a.elapsed_time(b) * 1e3, 1.0)


def enqueue_behind_spin(launches, K: int, enqueue_s_per_launch: float, cycles_per_us: float,
                        per_launch_events: bool, stream):
    """K launches enqueued behind a spin kernel long enough to cover the host's enqueue time, so
    the GPU runs them back to back.  Returns (event pairs, host wall seconds, whether the
    enqueue outlasted the spin, i.e. the queue may have run dry)."""
    import torch
    n_ev = K if per_launch_events else 1
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n_ev)]
    spin_us = min(2e6, max(50.0, 3.0 * K * enqueue_s_per_launch * 1e6))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    torch.cuda._sleep(int(spin_us * cycles_per_us))
    if not per_launch_events:
        ev[0][0].record(stream)
    for i in range(K):
        if per_launch_events:
            ev[i][0].record(stream)
        launches[i % len(launches)]()
        if per_launch_events:
            ev[i][1].record(stream)
    if not per_launch_events:
        ev[0][1].record(stream)
    enqueued = time.perf_counter() - t0
    torch.cuda.synchronize()
    return ev, time.perf_counter() - t0, enqueued * 1e6 > spin_us


# ------------------------------------------------------------------------------ main


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="finalize_prefill", choices=WORKLOAD_CHOICES)
    ap.add_argument("--set", action="append", default=[], metavar="KEY=INT",
                    help="change an integer parameter of the workload (T, H, E, k, seed, ...); "
                         "repeatable")
    ap.add_argument("--sets", type=int, default=0, metavar="N",
                    help="rotate the timed launches over N copies of the inputs and outputs "
                         "(default: 1, or enough copies to exceed 1 GiB for small workloads)")
    ap.add_argument("--in-place", action="store_true",
                    help="write residual_out over the residual input (the workloads with a "
                         "residual: the finalize, its MXFP4 form, the gated norms and the combine)")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle leg (its CPU timing and the sampled parity check)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this path has no multi-GPU mode "
              "(use --gpus 1)", file=sys.stderr)
        return 2

    import torch

    import finalize_residual_rmsnorm_amd as mf

    mf.lib()
    dev = torch.device("cuda:0")
    print(f"# {torch.cuda.get_device_name(dev)}; generating {args.workload}", file=sys.stderr,
          flush=True)
    overrides = parse_overrides(args.set)
    d_raw = make_workload(args.workload, overrides)
    if args.sets < 0:
        raise SystemExit("--sets must be at least 1")
    label = run_label(args.workload, overrides, args.sets, args.in_place)
    d = route_on_gpu(d_raw, dev)
    ws = algorithmic_bytes(d)
    # Working sets that fit in the 256 MB Infinity Cache are rotated over enough copies that
    # every step reads cold data; --sets fixes the number of copies instead.
    nsets = 1 if ws == 0 or ws >= 4 * MALL_BYTES else min(MAX_INPUT_SETS, -(-4 * MALL_BYTES // ws))
    if args.sets:
        nsets = args.sets
    sets = [upload(d, dev) for _ in range(nsets)]
    if args.in_place:
        if not all("res" in g and "res_out" in g for g in sets):
            raise SystemExit(f"--in-place: {args.workload} has no residual")
        for g in sets:
            g["res_out"] = g["res"]
    launches = [launcher(d, g) for g in sets]
    stream = torch.cuda.current_stream(dev)
    torch.cuda.synchronize()
    print(f"# uploaded {nsets} input set(s) of {ws / 1e9:.6f} GB; warmup {args.warmup}",
          file=sys.stderr, flush=True)

    parity = None
    d_cpu = None
    if not args.no_cpu_baseline and tokens_of(d):
        d_cpu = oracle_inputs(d_raw)
        parity = parity_sample(d_raw, d, d_cpu, dev)
        print(f"# parity sample: {parity}", file=sys.stderr, flush=True)

    W = max(1, args.warmup)
    cycles_per_us = spin_cycles_per_us()
    t0 = time.perf_counter()
    for i in range(W):
        launches[i % nsets]()
    enqueue_s = (time.perf_counter() - t0) / W
    torch.cuda.synchronize()

    K = args.steps
    # the timed region starts on the set after the warmup's last
    order = launches[W % nsets:] + launches[:W % nsets]
    # The timed region: K launches back to back between two events on the launch stream.
    ev, wall, drained = enqueue_behind_spin(order, K, enqueue_s, cycles_per_us, False, stream)
    span_ms = ev[0][0].elapsed_time(ev[0][1])
    avg_kernel_s = span_ms / K / 1e3
    ms_per_step = span_ms / K
    # The spread over launches, from a second pass with an event pair around every launch (each
    # pair adds the events' own cost, a few microseconds, to every figure).
    ev2, _, drained2 = enqueue_behind_spin(order, K, enqueue_s, cycles_per_us, True, stream)
    kern_ms = [a.elapsed_time(b) for a, b in ev2]

    achieved = ws / avg_kernel_s / 1e9
    traffic = read_traffic(label, d["kind"]) if d["kind"] in KERNEL_SOURCES else None
    tokens = tokens_of(d)
    if tokens:
        value, unit = tokens * K / (span_ms / 1e3), "tokens/s"
    elif ws:
        value, unit = ws * K / (span_ms / 1e3) / 1e9, "GB/s"
    else:
        value, unit = K / (span_ms / 1e3), "launches/s"
    cfg = {k: d[k] for k in ("T", "H", "E", "k", "heads", "D", "bytes", "workgroups", "threads")
           if k in d}
    cfg = dict(workload=label, **cfg, routing=_routing(d_raw),
               algorithmic_bytes_per_step=ws, input_sets=nsets, rotated_bytes=ws * nsets,
               residual_in_place=args.in_place,
               launch=launch_config(args.workload, d),
               kernel_ms_avg_back_to_back=ms_per_step,
               event_pair_ms_median=float(np.median(kern_ms)),
               event_pair_ms_p10=float(np.percentile(kern_ms, 10)),
               event_pair_ms_p90=float(np.percentile(kern_ms, 90)),
               host_wall_ms_per_step=wall * 1e3 / K, queue_ran_dry=drained or drained2)
    res = {
        "metric": METRIC if label == "finalize_prefill" else f"{label} {unit}",
        "value": value, "unit": unit, "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic", "config": cfg,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / PEAK_GBPS, "traffic": traffic},
    }
    if parity is not None:
        res["parity"] = parity
    if d_cpu is not None:
        print("# timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(d_cpu)
    print(json.dumps(res), flush=True)
    return 0 if parity is None or parity["ok"] else 1


def run_label(workload: str, overrides: dict, sets: int = 0, in_place: bool = False) -> str:
    """The name a run's JSON line and profile summaries carry: the workload, then any size
    overrides, the number of rotated input sets and the in-place residual, in that order."""
    label = workload + "".join(f"_{k}{v}" for k, v in overrides.items())
    if sets:
        label += f"_sets{sets}"
    if in_place:
        label += "_inplace"
    return label


def parse_overrides(items: list[str]) -> dict:
    """KEY=INT pairs, in the order given."""
    out = {}
    for item in items:
        key, sep, val = item.partition("=")
        if not sep or not key.isidentifier():
            raise SystemExit(f"--set {item!r}: expected KEY=INT")
        try:
            out[key] = int(val)
        except ValueError:
            raise SystemExit(f"--set {item!r}: {val!r} is not an integer")
    return out


def _routing(d: dict) -> str:
    if d.get("routing") == "logits":
        order = ("rows in a drawn random permutation" if d["layout"] == "random"
                 else "rows stably sorted by expert id")
        return (f"top-{d['k']} of N(0,1) router logits over {d['E']} experts, softmax over the "
                f"{d['k']}, routed on the GPU by mf_moe_route; {order}")
    if d.get("routing") == "drawn":
        return "drawn (uniform distinct experts, simplex weights)"
    return None


if __name__ == "__main__":
    sys.exit(main())
