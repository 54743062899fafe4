"""Expected values and oracle-completed inputs for the GPU tests (the CPU oracle only).

- ``routed(d)`` / ``named(name)``: a finalize workload drawn with its configured recipe
  (router logits ~ N(0, 1)) completed with the oracle's routing of those logits: the top-k
  experts, the softmax over their k logits and the stable expert sort.  The GPU finalize and the
  oracle finalize then read the same idx and weights, so the plain finalize's residual_out is
  still compared bit for bit.
- ``rmsnorm_of(r, gamma, eps)``: the oracle's final RMSNorm, rounded to bf16, of a given fp32
  residual.  It is the oracle's finalize with every routing weight zero, a pinned special case
  (the residual passes through unchanged, then the final RMSNorm).  Where the GPU's fp32
  residual is itself not unique (per-expert and gated variants), its bf16 output is held to one
  ulp of this function applied to the GPU's own residual_out, after that residual has passed
  its own check against the oracle's.
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle
import workloads


def routed(d: dict) -> dict:
    if d.get("routing") != "logits":
        return d
    eids, w, idx, _, _ = oracle.moe_route(d["logits"], d["k"])
    return workloads.with_routing(d, eids, w, idx)


def named(name: str, **overrides) -> dict:
    return routed(workloads.make_inputs(name, **overrides))


def rmsnorm_of(r, gamma, eps, threads: int = 8):
    r = np.ascontiguousarray(r, dtype=np.float32)
    lead = r.shape[:-1]
    r2 = r.reshape(-1, r.shape[-1])
    T, H = r2.shape
    if T == 0:
        return np.empty(r.shape, np.uint16)
    zero_row = np.zeros((1, H), np.uint16)

    def block(lo, hi):
        n = hi - lo
        _, out = oracle.moe_finalize(zero_row, np.zeros((n, 1), np.int32),
                                     np.zeros((n, 1), np.float32), r2[lo:hi], gamma, eps)
        return out

    bounds = np.linspace(0, T, min(threads, T) + 1).astype(int)
    spans = [(bounds[i], bounds[i + 1]) for i in range(len(bounds) - 1) if bounds[i] < bounds[i + 1]]
    with ThreadPoolExecutor(len(spans)) as ex:
        parts = list(ex.map(lambda s: block(*s), spans))
    return np.concatenate(parts).reshape(*lead, H)
