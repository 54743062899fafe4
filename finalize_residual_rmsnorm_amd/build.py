"""Ahead-of-time build of libmf.so (the C-ABI library) for gfx950 with hipcc.

    python -m finalize_residual_rmsnorm_amd.build

The library is built in-tree, next to this file, and loaded from there by the binding.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmf.so")
SOURCES = [os.path.join(CSRC, name)
           for name in ("mf_api.hip", "norm_api.hip", "route_api.hip", "mx_api.hip")]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    # Keep the compiler from forming packed-fp32 (v_pk_*_f32) instructions.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(out: str = LIB, extra_flags: list[str] | None = None, verbose: bool = False) -> str:
    """Compile the library (always, even if a built copy exists); returns its path."""
    tmp = f"{out}.tmp{os.getpid()}"
    cmd = [hipcc(), *HIPCC_FLAGS, *(extra_flags or []), *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature; that is expected.
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines()
            if ln.strip() and "packed-fp32-ops" not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), file=sys.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
