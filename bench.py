"""Throughput of the MoE finalize hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the path over one batch of seeded synthetic inputs already resident
in HBM: for the default workload, one mf_moe_finalize launch at T=16384, H=7168, E=256,
k=8 (rows grouped by expert), which gathers the k rows, accumulates them in fp32, adds and
stores the residual and emits the RMSNorm output.  W untimed steps, then exactly K timed
steps between device synchronisations; one JSON line on stdout.

roofline: algorithmic HBM bytes of one launch / the kernel's average duration, timed
with HIP events around every launch on the stream the kernel runs on; peak 8 TB/s.
traffic: HBM bytes per launch measured with rocprofv3 counters, read from the committed
summary under profiles/ when it was taken from the current kernel sources, else null.
cpu_baseline: the CPU oracle timed on a bounded sample of the same workload on the host.
Other workloads (--workload) time the sibling kernels (the gated norms, single and dual output,
and the per-head norm), RMSNorm + MXFP4 quantisation, the expert-parallel partial and combine
steps, the routing producer (one step = one
mf_moe_route call: its three kernels, timed together by the events around the call) and the
copy used for calibration.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "finalize tokens/s + achieved HBM GB/s (% of peak) at T=16384,H=7168,k=8"
PEAK_GBPS = 8000.0
MALL_BYTES = 256 << 20
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
    if kind == "copy":
        return 2 * d["bytes"]
    if kind == "route":
        T, E, k = d["T"], d["E"], d["k"]
        return T * E * 4 + T * k * 16 + (E + 1) * 4   # logits in; ids, weights, idx, perm out
    raise ValueError(kind)


def tokens_of(d: dict) -> int:
    return d["T"] if "T" in d else 0


def make_workload(name: str) -> dict:
    import workloads
    if name == "stream_copy":
        return dict(kind="copy", bytes=1 << 30)
    return workloads.make_inputs(name)


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
    if kind == "copy":
        n = d["bytes"] // 4
        return dict(src=torch.randint(0, 1 << 30, (n,), dtype=torch.int32, device=dev),
                    dst=torch.empty(n, dtype=torch.int32, device=dev))
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
        return mf.mf_launch_shape(mf.KIND_FINALIZE_PER_EXPERT if pe else mf.KIND_FINALIZE,
                                  d["T"], d["H"], d["k"])
    if kind in ("ep_combine", "rmsnorm_mx"):
        return mf.mf_launch_shape(mf.KIND_GATED, d["T"], d["H"])  # the same row shape
    if kind in ("gated", "gated_next"):
        return mf.mf_launch_shape(mf.KIND_GATED, d["T"], d["H"])
    if kind == "ep_combine":
        return mf.mf_launch_shape(mf.KIND_EP_COMBINE, d["T"], d["H"])
    return {}


# ------------------------------------------------------------------------------ CPU oracle


def cpu_baseline(d: dict, target_cpu_s: float = 20.0, max_threads: int = 16) -> dict:
    """The CPU oracle on a bounded sample (about target_cpu_s of CPU work) of the workload's
    tokens, split over up to max_threads host threads (the call releases the GIL)."""
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
    try:
        ncpu = len(os.sched_getaffinity(0))
    except AttributeError:
        ncpu = os.cpu_count() or 1
    threads = max(1, min(max_threads, ncpu))
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
    with ThreadPoolExecutor(threads) as ex:
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
    return dict(value=n * reps / dt, unit="tokens/s", cores=min(threads, len(spans)), kind="oracle",
                sample=f"{what} of the same inputs, {reps} pass(es), {len(spans)} threads over "
                       f"token blocks, {dt:.1f} s wall",
                value_1_thread=one * reps1 / dt1,
                sample_1_thread=f"the first {one} tokens, {reps1} pass(es), {dt1:.1f} s",
                cpu_model=cpu_model())


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# ------------------------------------------------------------------------------ main


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="finalize_prefill",
                    choices=["finalize_prefill", "finalize_decode_per_expert", "finalize_tiny",
                             "gated_residual_rmsnorm", "gated_residual_next_rmsnorm",
                             "rmsnorm_sigmoid_gate", "moe_route_prefill", "finalize_ep_partial",
                             "finalize_ep_combine", "rmsnorm_mxfp4", "finalize_prefill_mxfp4",
                             "moe_route_decode", "stream_copy"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
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
    d = make_workload(args.workload)
    ws = algorithmic_bytes(d)
    # Working sets that fit in the 256 MB Infinity Cache are rotated over enough copies that
    # every step reads cold data.
    nsets = 1 if ws >= 4 * MALL_BYTES else min(64, -(-4 * MALL_BYTES // ws))
    sets = [upload(d, dev) for _ in range(nsets)]
    launches = [launcher(d, g) for g in sets]
    stream = torch.cuda.current_stream(dev)
    torch.cuda.synchronize()
    print(f"# uploaded {nsets} input set(s) of {ws / 1e9:.3f} GB; warmup {args.warmup}",
          file=sys.stderr, flush=True)

    for i in range(args.warmup):
        launches[i % nsets]()
    torch.cuda.synchronize()

    K = args.steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        ev[i][0].record(stream)
        launches[i % nsets]()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_ms = [a.elapsed_time(b) for a, b in ev]
    avg_kernel_s = float(np.mean(kern_ms)) / 1e3
    ms_per_step = wall * 1e3 / K

    achieved = ws / avg_kernel_s / 1e9
    traffic = read_traffic(args.workload, d["kind"])
    tokens = tokens_of(d)
    value = tokens * K / wall if tokens else ws * K / wall / 1e9
    unit = "tokens/s" if tokens else "GB/s"
    cfg = {k: d[k] for k in ("T", "H", "E", "k", "heads", "D") if k in d}
    cfg = dict(workload=args.workload, **cfg, layout=_layout(args.workload),
               algorithmic_bytes_per_step=ws, input_sets=nsets,
               launch=launch_config(args.workload, d),
               kernel_ms_median=float(np.median(kern_ms)),
               kernel_ms_p10=float(np.percentile(kern_ms, 10)),
               kernel_ms_p90=float(np.percentile(kern_ms, 90)))
    res = {
        "metric": METRIC if args.workload == "finalize_prefill" else f"{args.workload} {unit}",
        "value": value, "unit": unit, "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic", "config": cfg,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / PEAK_GBPS, "traffic": traffic},
    }
    if not args.no_cpu_baseline and tokens:
        print("# timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(d)
    print(json.dumps(res), flush=True)
    return 0


def _layout(name: str):
    import workloads
    return workloads.WORKLOADS.get(name, {}).get("layout")


if __name__ == "__main__":
    sys.exit(main())
