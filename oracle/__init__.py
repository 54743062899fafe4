"""CPU oracle for the MoE finalize path (and its expert-parallel partial and combine steps), the
sibling fused norms (gated residual RMSNorm, its dual-output "next" form, per-head RMSNorm with
a sigmoid gate), the MXFP4 quantisation of a normalised row, and the routing and expert-sorted
permutation the finalize consumes.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg
of ``bench.py`` are the only callers.  The product path never imports this package, and
this package imports nothing from the GPU library.

The arithmetic lives in ``oracle.c`` (plain loops; FP32 FMA where the pages fix the
precision, float64 everywhere else).  This module compiles it with gcc when the shared
object is missing or older than its source, and wraps it for numpy arrays.
bfloat16 arrays are ``numpy.uint16`` bit patterns.

With ``ORACLE_SANITIZE=1`` in the environment the module builds and loads a separate copy,
``liboracle_san.so``, compiled with AddressSanitizer and UndefinedBehaviorSanitizer (any
undefined-behaviour report aborts); the process must then have gcc's ASan runtime preloaded
(``LD_PRELOAD``).  tests/test_sanitizers.py runs the oracle's pins that way.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_DIR = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_DIR, "oracle.c")
LIB = os.path.join(_DIR, "liboracle.so")
LIB_SAN = os.path.join(_DIR, "liboracle_san.so")
# No fast-math and no contraction: every FMA in the source is an explicit fmaf().
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
          "-Wall", "-Wextra"]
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
             "-fno-omit-frame-pointer", "-g"]

_lib = None


def sanitized() -> bool:
    """Whether this process uses the ASan/UBSan build (ORACLE_SANITIZE=1)."""
    return os.environ.get("ORACLE_SANITIZE", "") == "1"


def build(force: bool = False, sanitize: bool | None = None) -> str:
    """Compile oracle.c with gcc (the sanitized copy when asked, or when ORACLE_SANITIZE=1);
    returns the library path."""
    san = sanitized() if sanitize is None else sanitize
    lib = LIB_SAN if san else LIB
    if force or not os.path.exists(lib) or os.path.getmtime(lib) < os.path.getmtime(SRC):
        tmp = lib + f".tmp{os.getpid()}"
        subprocess.run(["gcc", *CFLAGS, *(SAN_FLAGS if san else []), "-o", tmp, SRC, "-lm"],
                       check=True)
        os.replace(tmp, lib)
    return lib


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build())
        p, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float
        lib.oracle_moe_finalize.argtypes = [p, i64, p, p, p, p, i32, p, p, p, f32, p, i64, i32, i32]
        lib.oracle_gated_residual_rmsnorm.argtypes = [p, p, p, p, p, f32, p, i64, i32]
        lib.oracle_moe_finalize_ep_partial.argtypes = [p, i64, p, p, p, p, i32, f32, p, i64, i32, i32]
        lib.oracle_moe_finalize_ep_combine.argtypes = [p, i32, p, p, p, f32, p, i64, i32]
        lib.oracle_gated_residual_next_rmsnorm.argtypes = [p, p, p, p, p, p, f32, p, p, i64, i32]
        lib.oracle_rmsnorm_sigmoid_gate.argtypes = [p, p, p, f32, p, i64, i32, i32]
        lib.oracle_moe_route.argtypes = [p, i64, i32, i32, p, p, p, p, p]
        lib.oracle_mxfp4_quantize.argtypes = [p, i64, i32, p, p]
        lib.oracle_rmsnorm_mxfp4_quantize.argtypes = [p, p, f32, p, p, i64, i32]
        lib.oracle_rmsnorm_f32_mxfp4_quantize.argtypes = [p, p, f32, p, p, i64, i32]
        lib.oracle_bf16_round.argtypes = [p, p, i64]
        lib.oracle_bf16_round.restype = None
        _lib = lib
    return _lib


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data_as(ctypes.c_void_p)


def moe_finalize(expert_rows, idx, weights, residual, gamma, eps, expert_ids=None,
                 expert_gamma=None):
    """Return (residual_out float32 [T,H], out bf16-bits [T,H]).

    expert_rows: bf16 [num_rows, H]; idx: int32 [T, k]; weights: float32 [T, k];
    residual: float32 [T, H]; gamma: bf16 [H]; expert_ids: int32 [T, k] and
    expert_gamma: bf16 [E, H] together select the per-expert RMSNorm variant.
    """
    lib = _load()
    rows, prows = _c(expert_rows, np.uint16)
    idx, pidx = _c(idx, np.int32)
    w, pw = _c(weights, np.float32)
    res, pres = _c(residual, np.float32)
    g, pg = _c(gamma, np.uint16)
    T, k = idx.shape
    H = rows.shape[1]
    if (expert_ids is None) != (expert_gamma is None):
        raise ValueError("expert_ids and expert_gamma go together")
    pe = pge = None
    E = 0
    if expert_gamma is not None:
        eids, pe = _c(expert_ids, np.int32)
        ge, pge = _c(expert_gamma, np.uint16)
        E = ge.shape[0]
    r_out = np.empty((T, H), dtype=np.float32)
    out = np.empty((T, H), dtype=np.uint16)
    st = lib.oracle_moe_finalize(prows, rows.shape[0], pidx, pw, pe, pge, E, pres,
                                 r_out.ctypes.data_as(ctypes.c_void_p), pg, float(eps),
                                 out.ctypes.data_as(ctypes.c_void_p), T, H, k)
    if st != 0:
        raise ValueError(f"oracle_moe_finalize failed with status {st}")
    return r_out, out


def moe_finalize_ep_partial(expert_rows, idx, weights, eps=1e-6, expert_ids=None,
                            expert_gamma=None):
    """This GPU's partial of the expert-parallel finalize: float32 [T, H].

    Slots with idx < 0 belong to another GPU's experts and are skipped; the others are
    accumulated as in moe_finalize (per-expert normalised when expert_gamma is given).
    """
    lib = _load()
    rows, prows = _c(expert_rows, np.uint16)
    idx, pidx = _c(idx, np.int32)
    w, pw = _c(weights, np.float32)
    T, k = idx.shape
    H = rows.shape[1]
    if (expert_ids is None) != (expert_gamma is None):
        raise ValueError("expert_ids and expert_gamma go together")
    pe = pge = None
    E = 0
    if expert_gamma is not None:
        eids, pe = _c(expert_ids, np.int32)
        ge, pge = _c(expert_gamma, np.uint16)
        E = ge.shape[0]
    part = np.empty((T, H), dtype=np.float32)
    st = lib.oracle_moe_finalize_ep_partial(prows, rows.shape[0], pidx, pw, pe, pge, E, float(eps),
                                            part.ctypes.data_as(ctypes.c_void_p), T, H, k)
    if st != 0:
        raise ValueError(f"oracle_moe_finalize_ep_partial failed with status {st}")
    return part


def moe_finalize_ep_combine(partials, residual, gamma, eps):
    """The owner's combine: partials float32 [G, T, H] added in rank order, then the residual
    add and RMSNorm.  Returns (residual_out float32 [T,H], out bf16-bits [T,H])."""
    lib = _load()
    parts, pp = _c(partials, np.float32)
    res, pres = _c(residual, np.float32)
    g, pg = _c(gamma, np.uint16)
    G, T, H = parts.shape
    r_out = np.empty((T, H), dtype=np.float32)
    out = np.empty((T, H), dtype=np.uint16)
    lib.oracle_moe_finalize_ep_combine(pp, G, pres, r_out.ctypes.data_as(ctypes.c_void_p), pg,
                                       float(eps), out.ctypes.data_as(ctypes.c_void_p), T, H)
    return r_out, out


def gated_residual_rmsnorm(x, gate, residual, gamma, eps):
    """Return (residual_out float32 [T,H], out bf16-bits [T,H])."""
    lib = _load()
    x, px = _c(x, np.uint16)
    gt, pgt = _c(gate, np.uint16)
    res, pres = _c(residual, np.float32)
    g, pg = _c(gamma, np.uint16)
    T, H = x.shape
    r_out = np.empty((T, H), dtype=np.float32)
    out = np.empty((T, H), dtype=np.uint16)
    lib.oracle_gated_residual_rmsnorm(px, pgt, pres, r_out.ctypes.data_as(ctypes.c_void_p), pg,
                                      float(eps), out.ctypes.data_as(ctypes.c_void_p), T, H)
    return r_out, out


def gated_residual_next_rmsnorm(x, gate, residual, gamma, gamma_next, eps):
    """Return (residual_out float32 [T,H], out bf16-bits [T,H], out_next bf16-bits [T,H]).

    The gated residual feeding two RMSNorm outputs (gamma and gamma_next) that share one mean
    square: the reading taken of the pages' "gated residual dual norm", which they name only.
    """
    lib = _load()
    x, px = _c(x, np.uint16)
    gt, pgt = _c(gate, np.uint16)
    res, pres = _c(residual, np.float32)
    g, pg = _c(gamma, np.uint16)
    gn, pgn = _c(gamma_next, np.uint16)
    T, H = x.shape
    r_out = np.empty((T, H), dtype=np.float32)
    out = np.empty((T, H), dtype=np.uint16)
    out_next = np.empty((T, H), dtype=np.uint16)
    ptr = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    lib.oracle_gated_residual_next_rmsnorm(px, pgt, pres, ptr(r_out), pg, pgn, float(eps), ptr(out),
                                           ptr(out_next), T, H)
    return r_out, out, out_next


def rmsnorm_sigmoid_gate(x, gate, gamma, eps):
    """Return out bf16-bits with the shape of x ([T, heads, D])."""
    lib = _load()
    x, px = _c(x, np.uint16)
    gt, pgt = _c(gate, np.uint16)
    g, pg = _c(gamma, np.uint16)
    T, heads, D = x.shape
    out = np.empty_like(x)
    lib.oracle_rmsnorm_sigmoid_gate(px, pgt, pg, float(eps), out.ctypes.data_as(ctypes.c_void_p),
                                    T, heads, D)
    return out


def moe_route(logits, k):
    """Top-k softmax routing and the expert-sorted permutation of float32 logits [T, E].

    Returns (expert_ids int32 [T,k], weights float32 [T,k], idx int32 [T,k],
    perm int32 [T*k], offsets int32 [E+1]).
    """
    lib = _load()
    lg, plg = _c(logits, np.float32)
    T, E = lg.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    eids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    idx = np.empty((T, k), np.int32)
    perm = np.empty(T * k, np.int32)
    off = np.empty(E + 1, np.int32)
    ptr = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    st = lib.oracle_moe_route(plg, T, E, k, ptr(eids), ptr(w), ptr(idx), ptr(perm), ptr(off))
    if st != 0:
        raise ValueError(f"oracle_moe_route failed with status {st}")
    return eids, w, idx, perm, off


def mxfp4_quantize(x):
    """MXFP4 of float32 values [T, H] (H % 32 == 0): (codes uint8 [T, H/2], two E2M1 codes per
    byte, the even-indexed value in the low nibble; scale codes uint8 [T, H/32], E8M0)."""
    lib = _load()
    xa, px = _c(x, np.float32)
    T, H = xa.shape
    if H % 32:
        raise ValueError("H must be a multiple of 32")
    q = np.empty((T, H // 2), np.uint8)
    sc = np.empty((T, H // 32), np.uint8)
    lib.oracle_mxfp4_quantize(px, T, H, q.ctypes.data_as(ctypes.c_void_p),
                              sc.ctypes.data_as(ctypes.c_void_p))
    return q, sc


def rmsnorm_mxfp4_quantize(x, gamma, eps):
    """RMSNorm of bf16 rows x [T, H] with gamma, rounded to float32, then MXFP4 (as above)."""
    lib = _load()
    xa, px = _c(x, np.uint16)
    g, pg = _c(gamma, np.uint16)
    T, H = xa.shape
    if H % 32:
        raise ValueError("H must be a multiple of 32")
    q = np.empty((T, H // 2), np.uint8)
    sc = np.empty((T, H // 32), np.uint8)
    lib.oracle_rmsnorm_mxfp4_quantize(px, pg, float(eps), q.ctypes.data_as(ctypes.c_void_p),
                                      sc.ctypes.data_as(ctypes.c_void_p), T, H)
    return q, sc


def rmsnorm_f32_mxfp4_quantize(r, gamma, eps):
    """RMSNorm of float32 rows r [T, H] (the finalize's residual_out) with gamma, rounded to
    float32, then MXFP4: the finalize's MXFP4 epilogue.  Returns (q, scales) as above."""
    lib = _load()
    ra, pr = _c(r, np.float32)
    g, pg = _c(gamma, np.uint16)
    T, H = ra.shape
    if H % 32:
        raise ValueError("H must be a multiple of 32")
    q = np.empty((T, H // 2), np.uint8)
    sc = np.empty((T, H // 32), np.uint8)
    lib.oracle_rmsnorm_f32_mxfp4_quantize(pr, pg, float(eps), q.ctypes.data_as(ctypes.c_void_p),
                                          sc.ctypes.data_as(ctypes.c_void_p), T, H)
    return q, sc


def bf16_round(v):
    """Round float64 values to bfloat16 bit patterns (nearest, ties to even)."""
    lib = _load()
    v, pv = _c(v, np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    lib.oracle_bf16_round(pv, out.ctypes.data_as(ctypes.c_void_p), v.size)
    return out
