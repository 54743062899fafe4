"""Python binding of libmf.so: the MI355X (gfx950) MoE finalize, its sibling fused norms and the
routing producer of the finalize's gather indices.

The functions carry the names of the C entry points in include/mf.h and do argument
marshalling only: they take torch tensors (device memory), optionally allocate the outputs
with torch, and pass raw pointers, sizes and the current HIP stream to the library.  Every
step of the computation runs in the library's HIP kernels.  There is no fallback: if the
library is not built, or a tensor is not on the GPU, the call raises.

bf16 tensors are torch.bfloat16; fp32 tensors torch.float32; indices torch.int32.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import threading

import torch

__all__ = [
    "MFError", "lib", "mf_moe_finalize", "mf_gated_residual_rmsnorm", "mf_rmsnorm_sigmoid_gate",
    "mf_moe_finalize_supported", "mf_gated_residual_rmsnorm_supported",
    "mf_rmsnorm_sigmoid_gate_supported", "mf_launch_shape", "mf_stream_copy", "mf_status_string",
    "mf_moe_route", "mf_moe_route_supported", "mf_moe_route_workspace_bytes",
    "mf_gated_residual_next_rmsnorm", "mf_gated_residual_next_rmsnorm_supported",
    "mf_moe_finalize_ep_partial", "mf_moe_finalize_ep_combine", "mf_mxfp4_quantize",
    "mf_rmsnorm_mxfp4_quantize", "mf_mxfp4_supported", "mf_moe_finalize_mxfp4", "LIB_PATH",
    "mf_moe_route_noalloc", "MF_ROUTE_SCRATCH_BYTES", "mf_empty_grid", "mf_stream_read",
    "MF_STREAM_READ_CHUNK",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmf.so")

MF_OK = 0
MF_ROUTE_SCRATCH_BYTES = 4 << 20   # the static scratch of mf_moe_route_noalloc, per GPU
MF_STREAM_READ_CHUNK = 16384        # bytes of src per word of mf_stream_read's sink
_lib = None


class MFError(RuntimeError):
    """A negative mf_status returned by the library."""

    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {mf_status_string(status)} (status {status})")


def lib() -> ctypes.CDLL:
    """The loaded libmf.so (argument types set).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m finalize_residual_rmsnorm_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        p, i64, i32, f32, ci = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float,
                                ctypes.c_int)
        sig = {
            "mf_moe_finalize": [p, i64, p, p, p, p, i32, p, p, p, f32, p, i64, i32, i32, p],
            "mf_gated_residual_rmsnorm": [p, p, p, p, p, f32, p, i64, i32, p],
            "mf_rmsnorm_sigmoid_gate": [p, p, p, f32, p, i64, i32, i32, p],
            "mf_moe_finalize_supported": [i32, i32, ci],
            "mf_gated_residual_rmsnorm_supported": [i32],
            "mf_rmsnorm_sigmoid_gate_supported": [i32],
            "mf_launch_shape": [ci, i64, i32, i32, p, p, p, p],
            "mf_stream_copy": [p, p, i64, p],
            "mf_stream_read": [p, i64, p, p],
            "mf_empty_grid": [i64, i32, p],
            "mf_status_string": [ci],
            "mf_moe_route": [p, i64, i32, i32, p, p, p, p, p, p, i64, p],
            "mf_gated_residual_next_rmsnorm": [p, p, p, p, p, p, f32, p, p, i64, i32, p],
            "mf_gated_residual_next_rmsnorm_supported": [i32],
            "mf_moe_finalize_ep_partial": [p, i64, p, p, p, p, i32, f32, p, i64, i32, i32, p],
            "mf_moe_finalize_ep_combine": [p, i32, p, p, p, f32, p, i64, i32, p],
            "mf_mxfp4_quantize": [p, i64, i32, p, p, p],
            "mf_rmsnorm_mxfp4_quantize": [p, p, f32, p, p, i64, i32, p],
            "mf_mxfp4_supported": [i32],
            "mf_moe_finalize_mxfp4": [p, i64, p, p, p, p, p, f32, p, p, i64, i32, i32, p],
            "mf_moe_route_supported": [i32, i32],
            "mf_moe_route_workspace_bytes": [i64, i32, i32],
            "mf_moe_route_noalloc": [p, i64, i32, i32, p, p, p, p, p, p],
        }
        for name, args in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        L.mf_status_string.restype = ctypes.c_char_p
        L.mf_moe_route_workspace_bytes.restype = ctypes.c_int64
        _lib = L
    return _lib


def mf_status_string(status: int) -> str:
    return lib().mf_status_string(status).decode()


def _check(fn: str, status: int) -> None:
    if status != MF_OK:
        raise MFError(fn, status)


_call = threading.local()


@contextlib.contextmanager
def _on(device: torch.device):
    """Run one library call with `device` current (the library launches on the current HIP
    device) and require every tensor passed through _dev inside it to live there."""
    if device.type != "cuda":
        raise ValueError(f"expected GPU tensors, got device {device}")
    prev = getattr(_call, "device", None)
    _call.device = device
    try:
        with torch.cuda.device(device):
            yield
    finally:
        _call.device = prev


def _dev(t: torch.Tensor, dtype: torch.dtype, name: str, shape=None) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: must be a GPU tensor, got device {t.device}")
    want = getattr(_call, "device", None)
    if want is not None and t.device != want:
        raise ValueError(f"{name}: on {t.device}, but the call's other tensors are on {want}")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    return t.data_ptr()


def _stream(stream, device) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream if isinstance(stream, torch.cuda.Stream) else int(stream)


def mf_moe_finalize(expert_rows: torch.Tensor, idx: torch.Tensor, weights: torch.Tensor,
                    residual: torch.Tensor, gamma: torch.Tensor, eps: float = 1e-6, *,
                    expert_ids: torch.Tensor | None = None,
                    expert_gamma: torch.Tensor | None = None,
                    residual_out: torch.Tensor | None = None, out: torch.Tensor | None = None,
                    stream=None):
    """MoE finalize + residual add + RMSNorm.  Returns (out bf16 [T,H], residual_out fp32 [T,H]).

    expert_rows bf16 [num_rows, H]; idx int32 [T, k]; weights fp32 [T, k]; residual fp32 [T, H];
    gamma bf16 [H]; optional expert_ids int32 [T, k] + expert_gamma bf16 [E, H] for the
    per-expert RMSNorm variant.  Pass residual_out=residual to update the residual in place.
    """
    T, k = idx.shape
    num_rows, H = expert_rows.shape
    dev = expert_rows.device
    if residual_out is None:
        residual_out = torch.empty((T, H), dtype=torch.float32, device=dev)
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    pe = pg = None
    E = 0
    if (expert_ids is None) != (expert_gamma is None):
        raise ValueError("expert_ids and expert_gamma go together")
    if expert_gamma is not None:
        E = expert_gamma.shape[0]
        pe = _dev(expert_ids, torch.int32, "expert_ids", (T, k))
        pg = _dev(expert_gamma, torch.bfloat16, "expert_gamma", (E, H))
    with _on(dev):
        st = lib().mf_moe_finalize(
            _dev(expert_rows, torch.bfloat16, "expert_rows"), num_rows,
            _dev(idx, torch.int32, "idx"), _dev(weights, torch.float32, "weights", (T, k)),
            pe, pg, E,
            _dev(residual, torch.float32, "residual", (T, H)),
            _dev(residual_out, torch.float32, "residual_out", (T, H)),
            _dev(gamma, torch.bfloat16, "gamma", (H,)), float(eps),
            _dev(out, torch.bfloat16, "out", (T, H)), T, H, k, _stream(stream, dev))
    _check("mf_moe_finalize", st)
    return out, residual_out


def mf_moe_finalize_ep_partial(expert_rows: torch.Tensor, idx: torch.Tensor,
                               weights: torch.Tensor, eps: float = 1e-6, *,
                               expert_ids: torch.Tensor | None = None,
                               expert_gamma: torch.Tensor | None = None,
                               partial: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """This GPU's partial of the expert-parallel finalize (fp32 [T, H]).  idx < 0 marks a slot
    whose expert lives on another GPU: it is skipped."""
    T, k = idx.shape
    num_rows, H = expert_rows.shape
    dev = expert_rows.device
    if partial is None:
        partial = torch.empty((T, H), dtype=torch.float32, device=dev)
    pe = pg = None
    E = 0
    if (expert_ids is None) != (expert_gamma is None):
        raise ValueError("expert_ids and expert_gamma go together")
    if expert_gamma is not None:
        E = expert_gamma.shape[0]
        pe = _dev(expert_ids, torch.int32, "expert_ids", (T, k))
        pg = _dev(expert_gamma, torch.bfloat16, "expert_gamma", (E, H))
    with _on(dev):
        st = lib().mf_moe_finalize_ep_partial(
            _dev(expert_rows, torch.bfloat16, "expert_rows"), num_rows,
            _dev(idx, torch.int32, "idx"),
            _dev(weights, torch.float32, "weights", (T, k)), pe, pg, E, float(eps),
            _dev(partial, torch.float32, "partial", (T, H)), T, H, k, _stream(stream, dev))
    _check("mf_moe_finalize_ep_partial", st)
    return partial


def mf_moe_finalize_ep_combine(partials: torch.Tensor, residual: torch.Tensor, gamma: torch.Tensor,
                               eps: float = 1e-6, *, residual_out: torch.Tensor | None = None,
                               out: torch.Tensor | None = None, stream=None):
    """The token owner's combine: partials fp32 [G, T, H] added in rank order, then the
    residual add and RMSNorm.  Returns (out bf16 [T,H], residual_out fp32 [T,H])."""
    G, T, H = partials.shape
    dev = partials.device
    if residual_out is None:
        residual_out = torch.empty((T, H), dtype=torch.float32, device=dev)
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    with _on(dev):
        st = lib().mf_moe_finalize_ep_combine(
            _dev(partials, torch.float32, "partials"), G,
            _dev(residual, torch.float32, "residual", (T, H)),
            _dev(residual_out, torch.float32, "residual_out", (T, H)),
            _dev(gamma, torch.bfloat16, "gamma", (H,)), float(eps),
            _dev(out, torch.bfloat16, "out", (T, H)), T, H, _stream(stream, dev))
    _check("mf_moe_finalize_ep_combine", st)
    return out, residual_out


def mf_gated_residual_rmsnorm(x: torch.Tensor, gate: torch.Tensor, residual: torch.Tensor,
                              gamma: torch.Tensor, eps: float = 1e-6, *,
                              residual_out: torch.Tensor | None = None,
                              out: torch.Tensor | None = None, stream=None):
    """Gated-residual RMSNorm.  Returns (out bf16 [T,H], residual_out fp32 [T,H])."""
    T, H = x.shape
    dev = x.device
    if residual_out is None:
        residual_out = torch.empty((T, H), dtype=torch.float32, device=dev)
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    with _on(dev):
        st = lib().mf_gated_residual_rmsnorm(
            _dev(x, torch.bfloat16, "x"), _dev(gate, torch.bfloat16, "gate", (T, H)),
            _dev(residual, torch.float32, "residual", (T, H)),
            _dev(residual_out, torch.float32, "residual_out", (T, H)),
            _dev(gamma, torch.bfloat16, "gamma", (H,)), float(eps),
            _dev(out, torch.bfloat16, "out", (T, H)), T, H, _stream(stream, dev))
    _check("mf_gated_residual_rmsnorm", st)
    return out, residual_out


def mf_gated_residual_next_rmsnorm(x: torch.Tensor, gate: torch.Tensor, residual: torch.Tensor,
                                   gamma: torch.Tensor, gamma_next: torch.Tensor,
                                   eps: float = 1e-6, *,
                                   residual_out: torch.Tensor | None = None,
                                   out: torch.Tensor | None = None,
                                   out_next: torch.Tensor | None = None, stream=None):
    """Gated-residual dual RMSNorm.  Returns (out, out_next bf16 [T,H], residual_out fp32 [T,H])."""
    T, H = x.shape
    dev = x.device
    if residual_out is None:
        residual_out = torch.empty((T, H), dtype=torch.float32, device=dev)
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    if out_next is None:
        out_next = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    with _on(dev):
        st = lib().mf_gated_residual_next_rmsnorm(
            _dev(x, torch.bfloat16, "x"), _dev(gate, torch.bfloat16, "gate", (T, H)),
            _dev(residual, torch.float32, "residual", (T, H)),
            _dev(residual_out, torch.float32, "residual_out", (T, H)),
            _dev(gamma, torch.bfloat16, "gamma", (H,)),
            _dev(gamma_next, torch.bfloat16, "gamma_next", (H,)), float(eps),
            _dev(out, torch.bfloat16, "out", (T, H)),
            _dev(out_next, torch.bfloat16, "out_next", (T, H)),
            T, H, _stream(stream, dev))
    _check("mf_gated_residual_next_rmsnorm", st)
    return out, out_next, residual_out


def mf_rmsnorm_sigmoid_gate(x: torch.Tensor, gate: torch.Tensor, gamma: torch.Tensor,
                            eps: float = 1e-6, *, out: torch.Tensor | None = None, stream=None):
    """Per-head RMSNorm + sigmoid gate over x [T, heads, head_dim].  Returns out (bf16)."""
    T, heads, D = x.shape
    dev = x.device
    if out is None:
        out = torch.empty_like(x)
    with _on(dev):
        st = lib().mf_rmsnorm_sigmoid_gate(
            _dev(x, torch.bfloat16, "x"), _dev(gate, torch.bfloat16, "gate", (T, heads, D)),
            _dev(gamma, torch.bfloat16, "gamma", (D,)), float(eps),
            _dev(out, torch.bfloat16, "out", (T, heads, D)), T, heads, D, _stream(stream, dev))
    _check("mf_rmsnorm_sigmoid_gate", st)
    return out


def mf_moe_finalize_supported(H: int, k: int, per_expert: bool = False) -> bool:
    return bool(lib().mf_moe_finalize_supported(H, k, int(per_expert)))


def mf_gated_residual_rmsnorm_supported(H: int) -> bool:
    return bool(lib().mf_gated_residual_rmsnorm_supported(H))


def mf_gated_residual_next_rmsnorm_supported(H: int) -> bool:
    return bool(lib().mf_gated_residual_next_rmsnorm_supported(H))


def mf_rmsnorm_sigmoid_gate_supported(head_dim: int) -> bool:
    return bool(lib().mf_rmsnorm_sigmoid_gate_supported(head_dim))


KIND_FINALIZE, KIND_FINALIZE_PER_EXPERT, KIND_GATED, KIND_EP_COMBINE, KIND_EP_PARTIAL = 0, 1, 2, 3, 4


def mf_launch_shape(kind: int, T: int, H: int, k: int = 1) -> dict:
    """The launch shape the library picks: waves per token, vectors per lane, block, grid."""
    wpt, vpl, blk = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    grid = ctypes.c_int64()
    _check("mf_launch_shape", lib().mf_launch_shape(kind, T, H, k, ctypes.byref(wpt),
                                                    ctypes.byref(vpl), ctypes.byref(blk),
                                                    ctypes.byref(grid)))
    return dict(waves_per_token=wpt.value, vectors_per_lane=vpl.value, block=blk.value,
                grid=grid.value)


def mf_stream_copy(src: torch.Tensor, dst: torch.Tensor, stream=None) -> None:
    """Copy src into dst (same byte size, a multiple of 16) with the library's copy kernel."""
    if src.device.type != "cuda" or dst.device.type != "cuda":
        raise ValueError("mf_stream_copy: GPU tensors required")
    if src.device != dst.device:
        raise ValueError("mf_stream_copy: src and dst on different devices")
    if not (src.is_contiguous() and dst.is_contiguous()):
        raise ValueError("mf_stream_copy: contiguous tensors required")
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != n:
        raise ValueError("mf_stream_copy: size mismatch")
    with _on(src.device):
        _check("mf_stream_copy", lib().mf_stream_copy(src.data_ptr(), dst.data_ptr(), n,
                                                      _stream(stream, src.device)))


def mf_stream_read(src: torch.Tensor, sink: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Read src (contiguous, a multiple of 16 bytes) with the library's read kernel; returns the
    sink: int32 [ceil(bytes / MF_STREAM_READ_CHUNK)], word c the xor of chunk c's 32-bit words."""
    if src.device.type != "cuda":
        raise ValueError("mf_stream_read: a GPU tensor required")
    if not src.is_contiguous():
        raise ValueError("mf_stream_read: a contiguous tensor required")
    n = src.numel() * src.element_size()
    words = -(-n // MF_STREAM_READ_CHUNK)
    if sink is None:
        sink = torch.empty(words, dtype=torch.int32, device=src.device)
    if (sink.device != src.device or sink.dtype != torch.int32 or not sink.is_contiguous()
            or sink.numel() < words):
        raise ValueError(f"mf_stream_read: sink must be int32 [{words}] on {src.device}")
    with _on(src.device):
        _check("mf_stream_read", lib().mf_stream_read(src.data_ptr(), n, sink.data_ptr(),
                                                      _stream(stream, src.device)))
    return sink


def mf_empty_grid(workgroups: int, threads: int, device=None, stream=None) -> None:
    """Launch an empty kernel of `workgroups` x `threads` (a measurement aid: the dispatch floor
    of a grid shape) on the current stream of `device` (default: the current device)."""
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    with _on(dev):
        _check("mf_empty_grid", lib().mf_empty_grid(workgroups, threads, _stream(stream, dev)))


def mf_moe_route_supported(num_experts: int, k: int) -> bool:
    return bool(lib().mf_moe_route_supported(num_experts, k))


def mf_moe_route_workspace_bytes(T: int, num_experts: int, k: int) -> int:
    """Workspace bytes mf_moe_route needs (raises MFError for unsupported arguments)."""
    n = lib().mf_moe_route_workspace_bytes(T, num_experts, k)
    if n < 0:
        raise MFError("mf_moe_route_workspace_bytes", int(n))
    return int(n)


def mf_moe_route(logits: torch.Tensor, k: int, *, expert_ids: torch.Tensor | None = None,
                 weights: torch.Tensor | None = None, idx: torch.Tensor | None = None,
                 perm: torch.Tensor | None = None, offsets: torch.Tensor | None = None,
                 workspace: torch.Tensor | None = None, stream=None):
    """Top-k softmax routing and the expert-sorted permutation of fp32 logits [T, E].

    Returns (expert_ids int32 [T,k], weights fp32 [T,k], idx int32 [T,k], perm int32 [T*k],
    offsets int32 [E+1]).  Outputs and the workspace (a uint8 tensor of at least
    mf_moe_route_workspace_bytes(T, E, k) bytes) are allocated with torch when not given.
    """
    T, E = logits.shape
    dev = logits.device
    ws_bytes = mf_moe_route_workspace_bytes(T, E, k)
    new = lambda shape, dt: torch.empty(shape, dtype=dt, device=dev)
    expert_ids = new((T, k), torch.int32) if expert_ids is None else expert_ids
    weights = new((T, k), torch.float32) if weights is None else weights
    idx = new((T, k), torch.int32) if idx is None else idx
    perm = new((T * k,), torch.int32) if perm is None else perm
    offsets = new((E + 1,), torch.int32) if offsets is None else offsets
    workspace = new((ws_bytes,), torch.uint8) if workspace is None else workspace
    if workspace.dtype != torch.uint8 or workspace.dim() != 1:
        raise TypeError("workspace: expected a 1-d torch.uint8 tensor")
    with _on(dev):
        st = lib().mf_moe_route(
            _dev(logits, torch.float32, "logits"), T, E, k,
            _dev(expert_ids, torch.int32, "expert_ids", (T, k)),
            _dev(weights, torch.float32, "weights", (T, k)), _dev(idx, torch.int32, "idx", (T, k)),
            _dev(perm, torch.int32, "perm", (T * k,)),
            _dev(offsets, torch.int32, "offsets", (E + 1,)),
            _dev(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(stream, dev))
    _check("mf_moe_route", st)
    return expert_ids, weights, idx, perm, offsets


def mf_moe_route_noalloc(logits: torch.Tensor, k: int, *, expert_ids: torch.Tensor,
                         weights: torch.Tensor, idx: torch.Tensor, perm: torch.Tensor,
                         offsets: torch.Tensor, stream=None):
    """mf_moe_route on the library's static scratch: no workspace, and the caller passes every
    output (nothing is allocated).  Returns the outputs it was given."""
    T, E = logits.shape
    dev = logits.device
    with _on(dev):
        st = lib().mf_moe_route_noalloc(
            _dev(logits, torch.float32, "logits"), T, E, k,
            _dev(expert_ids, torch.int32, "expert_ids", (T, k)),
            _dev(weights, torch.float32, "weights", (T, k)), _dev(idx, torch.int32, "idx", (T, k)),
            _dev(perm, torch.int32, "perm", (T * k,)),
            _dev(offsets, torch.int32, "offsets", (E + 1,)), _stream(stream, dev))
    _check("mf_moe_route_noalloc", st)
    return expert_ids, weights, idx, perm, offsets


def mf_mxfp4_supported(H: int) -> bool:
    return bool(lib().mf_mxfp4_supported(H))


def _mx_outputs(T, H, dev, q, scales):
    if q is None:
        q = torch.empty((T, H // 2), dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty((T, H // 32), dtype=torch.uint8, device=dev)
    return q, scales


def mf_mxfp4_quantize(x: torch.Tensor, *, q: torch.Tensor | None = None,
                      scales: torch.Tensor | None = None, stream=None):
    """MXFP4 of fp32 rows x [T, H] (H % 32 == 0).  Returns (q uint8 [T, H/2]: two E2M1 codes per
    byte, even value in the low nibble; scales uint8 [T, H/32]: E8M0 codes)."""
    T, H = x.shape
    q, scales = _mx_outputs(T, H, x.device, q, scales)
    with _on(x.device):
        st = lib().mf_mxfp4_quantize(_dev(x, torch.float32, "x"), T, H,
                                     _dev(q, torch.uint8, "q", (T, H // 2)),
                                     _dev(scales, torch.uint8, "scales", (T, H // 32)),
                                     _stream(stream, x.device))
    _check("mf_mxfp4_quantize", st)
    return q, scales


def mf_rmsnorm_mxfp4_quantize(x: torch.Tensor, gamma: torch.Tensor, eps: float = 1e-6, *,
                              q: torch.Tensor | None = None, scales: torch.Tensor | None = None,
                              stream=None):
    """RMSNorm of bf16 rows x [T, H] with gamma, then MXFP4.  Returns (q, scales) as above."""
    T, H = x.shape
    q, scales = _mx_outputs(T, H, x.device, q, scales)
    with _on(x.device):
        st = lib().mf_rmsnorm_mxfp4_quantize(_dev(x, torch.bfloat16, "x"),
                                             _dev(gamma, torch.bfloat16, "gamma", (H,)), float(eps),
                                             _dev(q, torch.uint8, "q", (T, H // 2)),
                                             _dev(scales, torch.uint8, "scales", (T, H // 32)),
                                             T, H,
                                             _stream(stream, x.device))
    _check("mf_rmsnorm_mxfp4_quantize", st)
    return q, scales


def mf_moe_finalize_mxfp4(expert_rows: torch.Tensor, idx: torch.Tensor, weights: torch.Tensor,
                          residual: torch.Tensor, gamma: torch.Tensor, eps: float = 1e-6, *,
                          residual_out: torch.Tensor | None = None, q: torch.Tensor | None = None,
                          scales: torch.Tensor | None = None, stream=None):
    """MoE finalize + residual add + RMSNorm with the output quantised to MXFP4.
    Returns (q uint8 [T, H/2], scales uint8 [T, H/32], residual_out fp32 [T, H])."""
    T, k = idx.shape
    num_rows, H = expert_rows.shape
    dev = expert_rows.device
    if residual_out is None:
        residual_out = torch.empty((T, H), dtype=torch.float32, device=dev)
    q, scales = _mx_outputs(T, H, dev, q, scales)
    with _on(dev):
        st = lib().mf_moe_finalize_mxfp4(
            _dev(expert_rows, torch.bfloat16, "expert_rows"), num_rows,
            _dev(idx, torch.int32, "idx"),
            _dev(weights, torch.float32, "weights", (T, k)),
            _dev(residual, torch.float32, "residual", (T, H)),
            _dev(residual_out, torch.float32, "residual_out", (T, H)),
            _dev(gamma, torch.bfloat16, "gamma", (H,)), float(eps),
            _dev(q, torch.uint8, "q", (T, H // 2)),
            _dev(scales, torch.uint8, "scales", (T, H // 32)),
            T, H, k, _stream(stream, dev))
    _check("mf_moe_finalize_mxfp4", st)
    return q, scales, residual_out
