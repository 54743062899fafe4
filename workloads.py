"""Seeded synthetic inputs for the MoE finalize path, its two sibling fused norms and the
routing that feeds the finalize.

This module only draws random inputs.  It holds none of the arithmetic the path computes:
no top-k selection or softmax, no stable permutation, no gather, no accumulation, no
normalisation and no output rounding.  Where a workload's routing comes from router logits
(the configured recipe), the logits are drawn here and the routing itself is left to the
consumer's routing implementation.  The oracle, the GPU tests, ``bench.py`` and
``__graft_entry__.smoke()`` all take their inputs from here, so both sides of every parity
check see the same bytes.

Recipe (numpy ``default_rng(seed)``, PCG64; draws happen in the order listed):

* MoE finalize (``make_finalize_inputs``), with one of two routing sources:

  ``routing="logits"`` (the configured recipe of the named finalize workloads
  ``finalize_tiny``, ``finalize_decode_per_expert``, ``finalize_prefill`` and the workloads
  built on the prefill inputs):
    1. router logits ``[T, E]`` (float32) ~ N(0, 1);
    2. (``layout="random"`` only) the unpermute index ``idx [T, k]`` (int32): a random
       permutation of 0..T*k-1, ``rng.permutation(T*k)``;
    3. expert rows, residual, gamma and expert gammas as in steps 4-7 below.
  The expert ids, routing weights and (``layout="expert_sorted"``) the unpermute index are
  NOT drawn: they are what the routing computes from the logits (the top-k experts, the
  softmax over their k logits, and the stable sort of the slots by expert id), so each
  consumer runs a routing implementation on ``logits``: the tests the CPU oracle, ``bench.py``
  the GPU routing call.  This module returns them as ``None``.

  ``routing="drawn"`` (the default; the many extra shapes of the parity tests):
    1. expert ids ``[T, k]`` (int32): k distinct experts per token, uniformly at random (the
       first k entries of an independent random permutation of the E experts per token);
    2. routing weights ``[T, k]`` (float32): k Exp(1) draws per token divided by their sum
       (a uniform draw from the probability simplex), listed largest first;
    3. the unpermute index ``idx [T, k]`` (int32): the permuted GEMM2 output row that holds
       the output of slot (t, j):
         - ``layout="random"``: ``rng.permutation(T*k)``;
         - ``layout="expert_grouped"``: rows grouped by expert id in ascending expert order
           (the grouped-GEMM layout), in a random order within each expert;
  and then, for both sources:
    4. expert rows ``[T*k, H]`` ~ N(0, 1), drawn as float32 in chunks of 2**24 values and
       rounded to bfloat16 (round-to-nearest-even, by torch's CPU cast);
    5. residual ``[T, H]`` float32 ~ N(0, residual_std);
    6. gamma ``[H]`` = 1 + 0.1 * N(0, 1), rounded to bfloat16;
    7. (per-expert variant only) expert gammas ``[E, H]`` = 1 + 0.1 * N(0, 1), bfloat16.
  Expert-parallel view (``ep_ranks``; no draw): expert e lives on rank e % ep_ranks, and
  ``remote_slots_marked`` gives the slots of other ranks' experts idx -1 once the expert ids
  are known.
* Expert-parallel combine (``make_ep_combine_inputs``): partials ``[G, T, H]`` ~ N(0, std 0.5)
  fp32, residual ``[T, H]`` ~ N(0, 1) fp32, gamma ``[H]`` = 1 + 0.1 * N(0, 1) bf16.
* MoE routing (``make_route_inputs``): router logits ``[T, E]`` ~ N(0, 1) float32, optionally
  rounded to bfloat16 values (``bf16_logits``: the precision of a bf16 router GEMM, which
  makes exactly equal logits common).
* Gated-residual RMSNorm (``make_gated_inputs``): x ``[T, H]`` ~ N(0, 1) bf16,
  gate ``[T, H]`` ~ N(0, 2) bf16 (standard deviation 2), residual ``[T, H]`` ~ N(0, 1) fp32,
  gamma ``[H]`` = 1 + 0.1 * N(0, 1) bf16; with ``dual=True`` then gamma_next ``[H]``, drawn
  the same way.
* RMSNorm + MXFP4 (``make_rmsnorm_mx_inputs``): x ``[T, H]`` ~ N(0, 1) bf16, gamma ``[H]`` =
  1 + 0.1 * N(0, 1) bf16.
* Per-head RMSNorm + sigmoid gate (``make_per_head_inputs``): x ``[T, heads, D]`` ~ N(0, 1)
  bf16, gate ``[T, heads, D]`` ~ N(0, 2) bf16, gamma ``[D]`` = 1 + 0.1 * N(0, 1) bf16.

bfloat16 arrays are returned as ``numpy.uint16`` holding the raw bit patterns.
"""
from __future__ import annotations

import numpy as np
import torch

CHUNK = 1 << 24  # values per draw when filling large arrays

#: The named workloads, with the sizes the MoE finalize pages and their model
#: configurations work at.  ``seed`` fixes every draw.
WORKLOADS = {
    # Tiny finalize: correctness-sized; top-2 softmax routing from N(0,1) logits, the rows in
    # a random permutation.
    "finalize_tiny": dict(kind="finalize", T=16, H=1024, E=8, k=2, seed=1, routing="logits",
                          layout="random", per_expert=False, residual_std=1.0),
    # Decode-sized finalize with a per-expert RMSNorm on every gathered row (tensor-parallel
    # finalize at hidden 4096, top-k 8); top-8 softmax routing, rows sorted by expert.
    "finalize_decode_per_expert": dict(kind="finalize", T=64, H=4096, E=128, k=8, seed=2,
                                       routing="logits", layout="expert_sorted",
                                       per_expert=True, residual_std=2.0),
    # Prefill-sized deterministic finalize: the throughput workload; top-8 of N(0,1) logits,
    # rows sorted by expert id (the contiguous grouped-GEMM layout).
    "finalize_prefill": dict(kind="finalize", T=16384, H=7168, E=256, k=8, seed=3,
                             routing="logits", layout="expert_sorted", per_expert=False,
                             residual_std=1.0),
    # One token (the decode regime where the finalize's launch and latency dominate): the
    # prefill model's shape, and the per-expert decode shape.
    "finalize_1tok": dict(kind="finalize", T=1, H=7168, E=256, k=8, seed=12, routing="logits",
                          layout="expert_sorted", per_expert=False, residual_std=1.0),
    "finalize_1tok_per_expert": dict(kind="finalize", T=1, H=4096, E=128, k=8, seed=13,
                                     routing="logits", layout="expert_sorted", per_expert=True,
                                     residual_std=2.0),
    # Wide rows (hidden sizes past 8192) at top-8, the prefill recipe with fewer tokens: each
    # still moves 2.2-3.5 GB, far past the Infinity Cache.
    "finalize_wide_12288": dict(kind="finalize", T=8192, H=12288, E=256, k=8, seed=14,
                                routing="logits", layout="expert_sorted", per_expert=False,
                                residual_std=1.0),
    "finalize_wide_20480": dict(kind="finalize", T=4096, H=20480, E=256, k=8, seed=15,
                                routing="logits", layout="expert_sorted", per_expert=False,
                                residual_std=1.0),
    "finalize_wide_32768": dict(kind="finalize", T=4096, H=32768, E=256, k=8, seed=16,
                                routing="logits", layout="expert_sorted", per_expert=False,
                                residual_std=1.0),
    # Expert parallelism over 8 GPUs at the prefill size: this GPU's partial (its 32 of the 256
    # experts; the other slots are marked -1) and the owner's combine of 8 partials for its
    # 2048 tokens.
    "finalize_ep_partial": dict(kind="finalize", T=16384, H=7168, E=256, k=8, seed=9,
                                routing="logits", layout="expert_sorted", per_expert=False,
                                residual_std=1.0, ep_ranks=8, ep_rank=0),
    "finalize_ep_combine": dict(kind="ep_combine", T=2048, H=7168, G=8, seed=10),
    # Gated-residual RMSNorm at its fixed hidden size.
    "gated_residual_rmsnorm": dict(kind="gated", T=4096, H=8192, seed=4),
    # The dual-output form: the same gated residual feeding this layer's and the next layer's
    # RMSNorm (two gammas), at the same fixed hidden size.
    "gated_residual_next_rmsnorm": dict(kind="gated", T=4096, H=8192, seed=8, dual=True),
    # The prefill finalize with its output quantised to MXFP4 (same inputs as finalize_prefill).
    "finalize_prefill_mxfp4": dict(kind="finalize", T=16384, H=7168, E=256, k=8, seed=3,
                                   routing="logits", layout="expert_sorted", per_expert=False,
                                   residual_std=1.0, mx_out=True),
    # RMSNorm + MXFP4 quantisation of bf16 rows at hidden size 8192.
    "rmsnorm_mxfp4": dict(kind="rmsnorm_mx", T=4096, H=8192, seed=11),
    # Per-head RMSNorm + sigmoid gate at its fixed head dim.
    "rmsnorm_sigmoid_gate": dict(kind="per_head", T=4096, heads=64, D=64, seed=5),
    # Routing that produces the prefill finalize's gather indices and weights.
    "moe_route_prefill": dict(kind="route", T=16384, E=256, k=8, seed=6, bf16_logits=False),
    # Decode-sized routing with bf16-valued logits (frequent exact ties).
    "moe_route_decode": dict(kind="route", T=64, E=128, k=8, seed=7, bf16_logits=True),
}

EPS = 1e-6


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round a float32 array to bfloat16 (nearest, ties to even) and return the bit patterns."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _normal_f32(rng: np.random.Generator, n: int, std: float = 1.0) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    for s in range(0, n, CHUNK):
        e = min(n, s + CHUNK)
        rng.standard_normal(out=out[s:e], dtype=np.float32)
    if std != 1.0:
        out *= np.float32(std)
    return out


def _normal_bf16(rng: np.random.Generator, n: int, std: float = 1.0) -> np.ndarray:
    out = np.empty(n, dtype=np.uint16)
    buf = np.empty(min(n, CHUNK), dtype=np.float32)
    for s in range(0, n, CHUNK):
        e = min(n, s + CHUNK)
        b = buf[: e - s]
        rng.standard_normal(out=b, dtype=np.float32)
        if std != 1.0:
            b *= np.float32(std)
        out[s:e] = to_bf16_bits(b)
    return out


def draw_routing(rng: np.random.Generator, T: int, E: int, k: int):
    """Random routing decisions: (expert_ids [T,k] int32, weights [T,k] float32).

    k distinct experts per token, uniformly at random; weights uniform on the simplex
    (normalised Exp(1) draws), largest first.
    """
    if not 1 <= k <= E:
        raise ValueError(f"need 1 <= k <= E, got k={k}, E={E}")
    experts = np.tile(np.arange(E, dtype=np.int32), (T, 1))
    expert_ids = np.ascontiguousarray(rng.permuted(experts, axis=1)[:, :k])
    z = rng.exponential(size=(T, k))
    w = -np.sort(-(z / z.sum(axis=1, keepdims=True)), axis=1)
    return expert_ids, w.astype(np.float32)


def unpermute_index(rng: np.random.Generator, expert_ids: np.ndarray, layout: str) -> np.ndarray:
    """idx[t, j] = the permuted row that holds slot (t, j)'s expert output."""
    T, k = expert_ids.shape
    n = T * k
    if layout == "random":
        return rng.permutation(n).astype(np.int32).reshape(T, k)
    if layout == "expert_grouped":
        # rows ordered by (expert id, random key): grouped by expert, shuffled within
        row_slot = np.lexsort((rng.random(n), expert_ids.ravel()))
        idx = np.empty(n, dtype=np.int64)
        idx[row_slot] = np.arange(n)
        return idx.astype(np.int32).reshape(T, k)
    raise ValueError(f"unknown layout {layout!r}")


def make_finalize_inputs(T: int, H: int, E: int, k: int, seed: int, layout: str = "expert_grouped",
                         per_expert: bool = False, residual_std: float = 1.0, ep_ranks: int = 0,
                         ep_rank: int = 0, mx_out: bool = False, routing: str = "drawn") -> dict:
    rng = np.random.default_rng(seed)
    logits = None
    if routing == "logits":
        if not 1 <= k <= E:
            raise ValueError(f"need 1 <= k <= E, got k={k}, E={E}")
        if layout not in ("random", "expert_sorted"):
            raise ValueError(f"routing from logits takes layout 'random' or 'expert_sorted', "
                             f"got {layout!r}")
        logits = _normal_f32(rng, T * E).reshape(T, E)
        expert_ids = w = None
        idx = rng.permutation(T * k).astype(np.int32).reshape(T, k) if layout == "random" else None
    elif routing == "drawn":
        expert_ids, w = draw_routing(rng, T, E, k)
        idx = unpermute_index(rng, expert_ids, layout)
    else:
        raise ValueError(f"unknown routing {routing!r}")
    rows = _normal_bf16(rng, T * k * H).reshape(T * k, H)
    residual = _normal_f32(rng, T * H, residual_std).reshape(T, H)
    gamma = to_bf16_bits(1.0 + 0.1 * _normal_f32(rng, H))
    d = dict(kind="finalize", T=T, H=H, E=E, k=k, eps=EPS, expert_rows=rows, idx=idx,
             weights=w, expert_ids=expert_ids, residual=residual, gamma=gamma,
             expert_gamma=None, routing=routing, layout=layout, logits=logits)
    if per_expert:
        d["expert_gamma"] = to_bf16_bits(1.0 + 0.1 * _normal_f32(rng, E * H)).reshape(E, H)
    if mx_out:
        d["kind"] = "finalize_mx"  # the same inputs; the output is quantised to MXFP4
    if ep_ranks:
        # one GPU's view under expert parallelism (no draw: the same bytes otherwise)
        d["kind"] = "ep_partial"
        d["ep_ranks"], d["ep_rank"] = ep_ranks, ep_rank
        if expert_ids is not None:
            d["idx"] = remote_slots_marked(idx, expert_ids, ep_ranks, ep_rank)
    return d


def with_routing(d: dict, expert_ids: np.ndarray, weights: np.ndarray,
                 sorted_idx: np.ndarray) -> dict:
    """A finalize workload drawn with ``routing="logits"``, completed with the routing results a
    routing implementation computed from its logits: expert ids and weights ``[T, k]``, and the
    expert-sorted unpermute index ``[T, k]`` (used where ``layout="expert_sorted"``; the
    ``"random"`` layout keeps its drawn index).  Expert-parallel views mark the other ranks'
    slots.  Returns a new dict; ``d`` is unchanged."""
    if d.get("routing") != "logits":
        raise ValueError("the workload's routing was drawn, not computed from logits")
    T, k = d["T"], d["k"]
    e = np.ascontiguousarray(expert_ids, dtype=np.int32).reshape(T, k)
    out = dict(d, expert_ids=e, weights=np.ascontiguousarray(weights, dtype=np.float32).reshape(T, k))
    idx = d["idx"] if d["layout"] == "random" else np.ascontiguousarray(sorted_idx, dtype=np.int32).reshape(T, k)
    if d.get("ep_ranks"):
        idx = remote_slots_marked(idx, e, d["ep_ranks"], d["ep_rank"])
    out["idx"] = idx
    return out


def remote_slots_marked(idx: np.ndarray, expert_ids: np.ndarray, ep_ranks: int,
                        ep_rank: int) -> np.ndarray:
    """idx with -1 in every slot whose expert lives on another rank (expert e on rank
    e % ep_ranks): this rank's view of the expert-parallel split."""
    return np.where(expert_ids % ep_ranks == ep_rank, idx, -1).astype(np.int32)


def make_ep_combine_inputs(T: int, H: int, G: int, seed: int) -> dict:
    """The token owner's inputs after the exchange: G partials [G, T, H] ~ N(0, 1/2) fp32 (a
    weighted sum of a few unit rows per rank), residual ~ N(0, 1) fp32, gamma bf16."""
    rng = np.random.default_rng(seed)
    partials = _normal_f32(rng, G * T * H, 0.5).reshape(G, T, H)
    residual = _normal_f32(rng, T * H).reshape(T, H)
    gamma = to_bf16_bits(1.0 + 0.1 * _normal_f32(rng, H))
    return dict(kind="ep_combine", T=T, H=H, G=G, eps=EPS, partials=partials, residual=residual,
                gamma=gamma)


def make_gated_inputs(T: int, H: int, seed: int, dual: bool = False) -> dict:
    rng = np.random.default_rng(seed)
    x = _normal_bf16(rng, T * H).reshape(T, H)
    gate = _normal_bf16(rng, T * H, 2.0).reshape(T, H)
    residual = _normal_f32(rng, T * H).reshape(T, H)
    gamma = to_bf16_bits(1.0 + 0.1 * _normal_f32(rng, H))
    d = dict(kind="gated", T=T, H=H, eps=EPS, x=x, gate=gate, residual=residual, gamma=gamma)
    if dual:
        d["kind"] = "gated_next"
        d["gamma_next"] = to_bf16_bits(1.0 + 0.1 * _normal_f32(rng, H))
    return d


def make_rmsnorm_mx_inputs(T: int, H: int, seed: int) -> dict:
    rng = np.random.default_rng(seed)
    x = _normal_bf16(rng, T * H).reshape(T, H)
    gamma = to_bf16_bits(1.0 + 0.1 * _normal_f32(rng, H))
    return dict(kind="rmsnorm_mx", T=T, H=H, eps=EPS, x=x, gamma=gamma)


def make_per_head_inputs(T: int, heads: int, D: int, seed: int) -> dict:
    rng = np.random.default_rng(seed)
    x = _normal_bf16(rng, T * heads * D).reshape(T, heads, D)
    gate = _normal_bf16(rng, T * heads * D, 2.0).reshape(T, heads, D)
    gamma = to_bf16_bits(1.0 + 0.1 * _normal_f32(rng, D))
    return dict(kind="per_head", T=T, heads=heads, D=D, eps=EPS, x=x, gate=gate, gamma=gamma)


def make_route_inputs(T: int, E: int, k: int, seed: int, bf16_logits: bool = False) -> dict:
    rng = np.random.default_rng(seed)
    logits = _normal_f32(rng, T * E).reshape(T, E)
    if bf16_logits:
        logits = bf16_bits_to_f32(to_bf16_bits(logits))
    return dict(kind="route", T=T, E=E, k=k, logits=logits)


def make_inputs(name: str, **overrides) -> dict:
    """Inputs of a named workload; keyword overrides change its sizes or seed."""
    cfg = dict(WORKLOADS[name])
    cfg.update(overrides)
    kind = cfg.pop("kind")
    if kind == "finalize":
        return make_finalize_inputs(**cfg)
    if kind == "gated":
        return make_gated_inputs(**cfg)
    if kind == "per_head":
        return make_per_head_inputs(**cfg)
    if kind == "route":
        return make_route_inputs(**cfg)
    if kind == "ep_combine":
        return make_ep_combine_inputs(**cfg)
    if kind == "rmsnorm_mx":
        return make_rmsnorm_mx_inputs(**cfg)
    raise ValueError(kind)
