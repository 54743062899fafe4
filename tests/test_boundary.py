"""The C-ABI boundary on the CPU: the library loads, exports every symbol the header
declares, and rejects bad arguments with the documented status before any HIP call.
No call here reaches a kernel launch (there is no GPU in this container)."""
import ctypes
import os
import re

import pytest

import finalize_residual_rmsnorm_amd as mf

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "mf.h")

# the status numbering include/mf.h declares, MF_ERR_VALUE and MF_ERR_SCRATCH after MF_ERR_HIP
OK, NULL, SHAPE, UNSUP, ALIGN, ALIAS, HIP, VALUE, SCRATCH = 0, -1, -2, -3, -4, -5, -6, -7, -8

# Fake device addresses: never dereferenced, every call below fails validation first.
A = 0x7F0000000000
B = 0x7F0100000000
C = 0x7F0200000000
D = 0x7F0300000000
E_ = 0x7F0400000000
F = 0x7F0500000000
G = 0x7F0600000000


def declared_functions():
    text = open(HEADER).read()
    return re.findall(r"^(?:int|int64_t|const char\*)\s+(mf_\w+)\(", text, flags=re.M)


def test_header_symbols_are_exported():
    names = declared_functions()
    assert len(names) == 23, names
    L = ctypes.CDLL(mf.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n


def test_status_numbering_matches_the_header():
    text = open(HEADER).read()
    declared = {m[0]: int(m[1]) for m in re.findall(r"(MF_\w+)\s*=\s*(-?\d+)", text)}
    assert declared == dict(MF_OK=OK, MF_ERR_NULL=NULL, MF_ERR_SHAPE=SHAPE,
                            MF_ERR_UNSUPPORTED=UNSUP, MF_ERR_ALIGN=ALIGN, MF_ERR_ALIAS=ALIAS,
                            MF_ERR_HIP=HIP, MF_ERR_VALUE=VALUE, MF_ERR_SCRATCH=SCRATCH)
    assert mf.mf_status_string(HIP).startswith("MF_ERR_HIP")
    assert mf.mf_status_string(VALUE).startswith("MF_ERR_VALUE")


def test_status_strings_cover_every_code():
    for code in (OK, NULL, SHAPE, UNSUP, ALIGN, ALIAS, HIP, VALUE, SCRATCH):
        s = mf.mf_status_string(code)
        assert s.startswith("MF_"), (code, s)
    assert mf.mf_status_string(12345) == "unknown mf_status"


def test_supported_queries():
    assert mf.mf_moe_finalize_supported(7168, 8)
    assert mf.mf_moe_finalize_supported(4096, 8, per_expert=True)
    assert not mf.mf_moe_finalize_supported(7170, 8)       # H % 8 != 0
    assert not mf.mf_moe_finalize_supported(32776, 8)      # beyond the widest row
    assert not mf.mf_moe_finalize_supported(1024, 0)
    assert not mf.mf_moe_finalize_supported(1024, 65)
    assert mf.mf_gated_residual_rmsnorm_supported(8192)
    assert not mf.mf_gated_residual_rmsnorm_supported(8190)
    assert mf.mf_gated_residual_next_rmsnorm_supported(8192)
    assert not mf.mf_gated_residual_next_rmsnorm_supported(32776)
    assert mf.mf_rmsnorm_sigmoid_gate_supported(64)
    assert not mf.mf_rmsnorm_sigmoid_gate_supported(128)
    assert mf.mf_moe_route_supported(256, 8)
    assert mf.mf_moe_route_supported(1, 1)
    assert mf.mf_moe_route_supported(1024, 16)
    assert not mf.mf_moe_route_supported(1025, 8)
    assert not mf.mf_moe_route_supported(0, 1)
    assert not mf.mf_moe_route_supported(256, 17)
    assert not mf.mf_moe_route_supported(4, 5)             # k > E


def fin(rows=A, num_rows=32, idx=B, w=C, eids=None, eg=None, E=0, res=D, res_out=E_,
        gamma=F, eps=1e-6, out=G, T=16, H=1024, k=2):
    return mf.lib().mf_moe_finalize(rows, num_rows, idx, w, eids, eg, E, res, res_out, gamma,
                                    eps, out, T, H, k, None)


@pytest.mark.parametrize("kw,code", [
    (dict(T=-1), SHAPE), (dict(num_rows=-1), SHAPE), (dict(H=1030), UNSUP), (dict(H=0), UNSUP),
    (dict(k=0), UNSUP), (dict(k=65), UNSUP), (dict(rows=None), NULL), (dict(idx=None), NULL),
    (dict(w=None), NULL), (dict(res=None), NULL), (dict(res_out=None), NULL),
    (dict(gamma=None), NULL), (dict(out=None), NULL), (dict(eids=B + 4096), NULL),
    (dict(eg=A + 8192), NULL), (dict(eids=B + 4096, eg=A + 1 << 20, E=0), SHAPE),
    (dict(num_rows=0), SHAPE), (dict(eps=float("nan")), VALUE), (dict(eps=-1e-6), VALUE),
    (dict(eps=float("inf")), VALUE), (dict(rows=A + 8), ALIGN), (dict(res_out=E_ + 4), ALIGN),
    (dict(out=G + 2), ALIGN), (dict(idx=B + 2), ALIGN), (dict(gamma=F + 8), ALIGN),
    (dict(res_out=D + 64), ALIAS), (dict(out=A + 1024), ALIAS), (dict(out=E_ + 4096), ALIAS),
    (dict(res_out=B), ALIAS), (dict(out=F), ALIAS),
    (dict(T=1 << 26), SHAPE),  # 128 threads per token would overflow the 32-bit grid
])
def test_finalize_rejects_bad_arguments(kw, code):
    assert fin(**kw) == code


def ep_part(rows=A, num_rows=32, idx=B, w=C, eids=None, eg=None, E=0, eps=1e-6, part=D, T=16,
            H=1024, k=2):
    return mf.lib().mf_moe_finalize_ep_partial(rows, num_rows, idx, w, eids, eg, E, eps, part, T,
                                               H, k, None)


@pytest.mark.parametrize("kw,code", [
    (dict(T=-1), SHAPE), (dict(num_rows=-1), SHAPE), (dict(H=1030), UNSUP), (dict(k=65), UNSUP),
    (dict(rows=None), NULL), (dict(idx=None), NULL), (dict(w=None), NULL), (dict(part=None), NULL),
    (dict(eids=B + 4096), NULL), (dict(num_rows=0), SHAPE), (dict(eps=-1.0), VALUE),
    (dict(part=D + 4), ALIGN), (dict(rows=A + 2), ALIGN), (dict(part=A + 64), ALIAS),
    (dict(part=B), ALIAS), (dict(T=1 << 26), SHAPE),
])
def test_ep_partial_rejects_bad_arguments(kw, code):
    assert ep_part(**kw) == code
    assert ep_part(T=0) == OK


def ep_comb(parts=A, G=8, res=B, res_out=C, gamma=D, eps=1e-6, out=E_, T=16, H=1024):
    return mf.lib().mf_moe_finalize_ep_combine(parts, G, res, res_out, gamma, eps, out, T, H, None)


@pytest.mark.parametrize("kw,code", [
    (dict(T=-1), SHAPE), (dict(G=0), SHAPE), (dict(G=1025), SHAPE), (dict(H=1020), UNSUP),
    (dict(parts=None), NULL), (dict(res=None), NULL), (dict(res_out=None), NULL),
    (dict(gamma=None), NULL), (dict(out=None), NULL), (dict(eps=float("nan")), VALUE),
    (dict(parts=A + 8), ALIGN), (dict(out=E_ + 2), ALIGN), (dict(res_out=A + 16 * 1024 * 4 * 7), ALIAS),
    (dict(out=A), ALIAS), (dict(res_out=B + 16), ALIAS), (dict(out=C + 64), ALIAS),
])
def test_ep_combine_rejects_bad_arguments(kw, code):
    assert ep_comb(**kw) == code
    assert ep_comb(T=0) == OK
    assert ep_comb(T=0, res_out=B) == OK  # in place is allowed


def test_mxfp4_rejects_bad_arguments():
    L = mf.lib()
    q = L.mf_mxfp4_quantize
    assert q(A, -1, 64, B, C, None) == SHAPE
    assert q(A, 4, 48, B, C, None) == UNSUP          # H % 32 != 0
    assert q(A, 4, 32800, B, C, None) == UNSUP
    assert q(A, 0, 64, B, C, None) == OK
    assert q(None, 4, 64, B, C, None) == NULL
    assert q(A, 4, 64, None, C, None) == NULL
    assert q(A + 8, 4, 64, B, C, None) == ALIGN
    assert q(A, 4, 64, B + 2, C, None) == ALIGN
    assert q(A, 4, 64, A + 64, C, None) == ALIAS
    assert q(A, 4, 64, B, B + 64, None) == ALIAS     # q is 128 bytes
    r = L.mf_rmsnorm_mxfp4_quantize
    assert r(A, D, 1e-6, B, C, -1, 64, None) == SHAPE
    assert r(A, D, 1e-6, B, C, 4, 40, None) == UNSUP
    assert r(A, None, 1e-6, B, C, 4, 64, None) == NULL
    assert r(A, D, -1.0, B, C, 4, 64, None) == VALUE
    assert r(A, D + 4, 1e-6, B, C, 4, 64, None) == ALIGN
    assert r(A, D, 1e-6, D, C, 4, 64, None) == ALIAS
    assert r(A, D, 1e-6, B, A + 100, 4, 64, None) == ALIAS
    assert r(A, D, 1e-6, B, C, 0, 64, None) == OK
    assert mf.mf_mxfp4_supported(7168) and not mf.mf_mxfp4_supported(7176)


def test_finalize_mxfp4_rejects_bad_arguments():
    f = lambda **kw: mf.lib().mf_moe_finalize_mxfp4(*[kw.get(n, v) for n, v in (
        ("rows", A), ("num_rows", 32), ("idx", B), ("w", C), ("res", D), ("res_out", E_),
        ("gamma", F), ("eps", 1e-6), ("q", G), ("sc", H_), ("T", 16), ("H", 1024), ("k", 2))],
        None)
    assert f(T=-1) == SHAPE
    assert f(H=1032) == UNSUP           # a multiple of 8 but not of 32
    assert f(k=0) == UNSUP
    assert f(q=None) == NULL and f(sc=None) == NULL and f(rows=None) == NULL
    assert f(num_rows=0) == SHAPE
    assert f(eps=float("nan")) == VALUE
    assert f(q=G + 2) == ALIGN and f(res_out=E_ + 4) == ALIGN
    assert f(q=A) == ALIAS and f(sc=E_ + 8) == ALIAS and f(sc=G + 100) == ALIAS
    assert f(T=0) == OK


def test_finalize_zero_tokens_is_a_no_op():
    assert fin(T=0, rows=None, idx=None, w=None, res=None, res_out=None, gamma=None,
               out=None) == OK
    assert fin(T=0, H=1001) == UNSUP  # widths are still checked


def test_in_place_residual_passes_validation_up_to_launch():
    # residual_out == residual is legal; stop just short of a launch with an unsupported
    # width at T = 0 to show the alias check itself does not reject it.
    assert fin(T=0, res_out=D) == OK


def gated(x=A, gate=B, res=C, res_out=D, gamma=E_, eps=1e-6, out=F, T=8, H=8192):
    return mf.lib().mf_gated_residual_rmsnorm(x, gate, res, res_out, gamma, eps, out, T, H, None)


@pytest.mark.parametrize("kw,code", [
    (dict(T=-1), SHAPE), (dict(H=8196), UNSUP), (dict(x=None), NULL), (dict(gate=None), NULL),
    (dict(res=None), NULL), (dict(res_out=None), NULL), (dict(gamma=None), NULL),
    (dict(out=None), NULL), (dict(eps=float("nan")), VALUE), (dict(x=A + 2), ALIGN),
    (dict(res_out=C + 16), ALIAS), (dict(out=A), ALIAS), (dict(out=D + 32), ALIAS),
])
def test_gated_rejects_bad_arguments(kw, code):
    assert gated(**kw) == code
    assert gated(T=0) == OK


H_ = 0x7F0700000000


def gated_next(x=A, gate=B, res=C, res_out=D, gamma=E_, gnext=H_, eps=1e-6, out=F, onext=G,
               T=8, H=8192):
    return mf.lib().mf_gated_residual_next_rmsnorm(x, gate, res, res_out, gamma, gnext, eps, out,
                                                   onext, T, H, None)


@pytest.mark.parametrize("kw,code", [
    (dict(T=-1), SHAPE), (dict(H=8196), UNSUP), (dict(gnext=None), NULL), (dict(onext=None), NULL),
    (dict(x=None), NULL), (dict(out=None), NULL), (dict(eps=float("nan")), VALUE),
    (dict(gnext=H_ + 8), ALIGN), (dict(onext=G + 2), ALIGN), (dict(onext=F + 64), ALIAS),
    (dict(onext=A), ALIAS), (dict(onext=D + 16), ALIAS), (dict(onext=H_), ALIAS),
    (dict(res_out=H_), ALIAS), (dict(out=C + 16), ALIAS),
])
def test_gated_next_rejects_bad_arguments(kw, code):
    assert gated_next(**kw) == code
    assert gated_next(T=0) == OK


def per_head(x=A, gate=B, gamma=C, eps=1e-6, out=D, T=4, heads=64, dim=64):
    return mf.lib().mf_rmsnorm_sigmoid_gate(x, gate, gamma, eps, out, T, heads, dim, None)


@pytest.mark.parametrize("kw,code", [
    (dict(T=-1), SHAPE), (dict(heads=0), SHAPE), (dict(dim=128), UNSUP), (dict(x=None), NULL),
    (dict(gate=None), NULL), (dict(gamma=None), NULL), (dict(out=None), NULL),
    (dict(eps=-1.0), VALUE), (dict(out=D + 8), ALIGN), (dict(out=A + 256), ALIAS),
])
def test_per_head_rejects_bad_arguments(kw, code):
    assert per_head(**kw) == code
    assert per_head(T=0) == OK


def test_stream_copy_rejects_bad_arguments():
    L = mf.lib()
    assert L.mf_stream_copy(A, B, -16, None) == SHAPE
    assert L.mf_stream_copy(A, B, 24, None) == SHAPE
    assert L.mf_stream_copy(A, B, 0, None) == OK
    assert L.mf_stream_copy(None, B, 16, None) == NULL
    assert L.mf_stream_copy(A + 8, B, 16, None) == ALIGN
    assert L.mf_stream_copy(A, A + 16, 64, None) == ALIAS
    # one vector per lane in one-wave workgroups: at most 2^32 lanes, 64 GiB
    assert L.mf_stream_copy(A, A + (1 << 40), (64 << 30) + 16, None) == SHAPE


def test_stream_read_rejects_bad_arguments():
    L = mf.lib()
    assert L.mf_stream_read(A, -16, B, None) == SHAPE
    assert L.mf_stream_read(A, 24, B, None) == SHAPE
    assert L.mf_stream_read(A, 0, B, None) == OK
    assert L.mf_stream_read(None, 16, B, None) == NULL
    assert L.mf_stream_read(A, 16, None, None) == NULL
    assert L.mf_stream_read(A + 8, 16, B, None) == ALIGN
    assert L.mf_stream_read(A, 16, B + 2, None) == ALIGN
    # the sink (one word per 16 KiB chunk) may not overlap the source
    assert L.mf_stream_read(A, 3 * 16384, A + 2 * 16384, None) == ALIAS
    assert L.mf_stream_read(A, 3 * 16384, A + 3 * 16384, None) != ALIAS


def test_launch_shapes():
    # One workgroup per token; its waves (a power of two, at most 16) hold slots of 512
    # values.  The shape depends on H only, never on the token count.
    # prefill: 14 slots over 8 waves of 2
    assert mf.mf_launch_shape(mf.KIND_FINALIZE, 16384, 7168, 8) == dict(
        waves_per_token=8, vectors_per_lane=2, block=512, grid=16384)
    # ... while the expert-parallel partial keeps one slot per wave there
    assert mf.mf_launch_shape(mf.KIND_EP_PARTIAL, 16384, 7168, 8) == dict(
        waves_per_token=16, vectors_per_lane=1, block=1024, grid=16384)
    assert mf.mf_launch_shape(mf.KIND_EP_PARTIAL, 3, 6144, 3) == mf.mf_launch_shape(
        mf.KIND_FINALIZE, 3, 6144, 3)
    with pytest.raises(mf.MFError):
        mf.mf_launch_shape(5, 4, 1024, 2)
    assert mf.mf_launch_shape(mf.KIND_FINALIZE, 3, 7168, 8) == dict(
        waves_per_token=8, vectors_per_lane=2, block=512, grid=3)
    # 13 slots (6656): one slot per wave over 16 waves
    assert mf.mf_launch_shape(mf.KIND_FINALIZE, 3, 6656, 8) == dict(
        waves_per_token=16, vectors_per_lane=1, block=1024, grid=3)
    # decode with per-expert norm: 8 waves
    assert mf.mf_launch_shape(mf.KIND_FINALIZE_PER_EXPERT, 64, 4096, 8) == dict(
        waves_per_token=8, vectors_per_lane=1, block=512, grid=64)
    # tiny: H = 1024 is two slots
    assert mf.mf_launch_shape(mf.KIND_FINALIZE, 16, 1024, 2) == dict(
        waves_per_token=2, vectors_per_lane=1, block=128, grid=16)
    assert mf.mf_launch_shape(mf.KIND_GATED, 4096, 8192) == dict(
        waves_per_token=16, vectors_per_lane=1, block=1024, grid=4096)
    # the plain finalize: one slot per wave over a power-of-two count of waves up to 16 slots
    # (6144 = 12 slots: 16 waves, 4 of them spare; 1536: 4 waves, 1 spare; 5000: ragged)
    assert mf.mf_launch_shape(mf.KIND_FINALIZE, 9, 6144, 8) == dict(
        waves_per_token=16, vectors_per_lane=1, block=1024, grid=9)
    assert mf.mf_launch_shape(mf.KIND_FINALIZE, 9, 1536, 5) == dict(
        waves_per_token=4, vectors_per_lane=1, block=256, grid=9)
    assert mf.mf_launch_shape(mf.KIND_FINALIZE, 9, 5000, 8)["waves_per_token"] == 16
    # ... while the gated norm keeps the fewest spare slots (12 slots: 4 waves of 3)
    assert mf.mf_launch_shape(mf.KIND_GATED, 9, 6144) == dict(
        waves_per_token=4, vectors_per_lane=3, block=256, grid=9)
    # 12288 = 24 slots: 8 waves of 3 leave no spare slot (16 waves of 2 would leave 8)
    assert mf.mf_launch_shape(mf.KIND_FINALIZE, 5, 12288, 8) == dict(
        waves_per_token=8, vectors_per_lane=3, block=512, grid=5)
    # the widest row: 64 slots; at the compiled top-8 the slot-serial kernel's 8 waves of 8 slots
    # (three of them staged in LDS), at another k 16 waves of 4
    assert mf.mf_launch_shape(mf.KIND_FINALIZE, 100000, 32768, 8) == dict(
        waves_per_token=8, vectors_per_lane=8, block=512, grid=100000)
    assert mf.mf_launch_shape(mf.KIND_FINALIZE, 7, 32768, 6) == dict(
        waves_per_token=16, vectors_per_lane=4, block=1024, grid=7)
    assert mf.mf_launch_shape(mf.KIND_FINALIZE, 7, 20480, 8)["vectors_per_lane"] == 5
    # whole waves of whole slots only: 13312 = 26 slots keeps the batched kernel, at 8 waves of 4
    assert mf.mf_launch_shape(mf.KIND_FINALIZE, 7, 13312, 8) == dict(
        waves_per_token=8, vectors_per_lane=4, block=512, grid=7)
    # 16384 = 32 slots: 8 waves of 4 (the per-expert variant: its own shape, 8 waves of 4 too)
    assert mf.mf_launch_shape(mf.KIND_FINALIZE, 7, 16384, 8)["vectors_per_lane"] == 4
    assert mf.mf_launch_shape(mf.KIND_FINALIZE, 7, 10240, 3) == dict(
        waves_per_token=8, vectors_per_lane=3, block=512, grid=7)
    # the EP combine runs at most 8 waves per token, 16 when 8 waves of 4 slots cannot hold the row
    assert mf.mf_launch_shape(mf.KIND_EP_COMBINE, 2048, 7168) == dict(
        waves_per_token=8, vectors_per_lane=2, block=512, grid=2048)
    assert mf.mf_launch_shape(mf.KIND_EP_COMBINE, 4, 16384)["waves_per_token"] == 8
    assert mf.mf_launch_shape(mf.KIND_EP_COMBINE, 4, 20000) == dict(
        waves_per_token=16, vectors_per_lane=3, block=1024, grid=4)
    with pytest.raises(mf.MFError):
        mf.mf_launch_shape(mf.KIND_FINALIZE, 4, 1001, 2)


def test_every_supported_width_has_a_kernel():
    # The launch-shape query runs the same kernel lookup as a launch: every width and top-k
    # the capability queries accept must map to a compiled kernel.
    for H in range(8, 32768 + 1, 8):
        for kind, k in ((mf.KIND_FINALIZE, 8), (mf.KIND_FINALIZE, 3),
                        (mf.KIND_FINALIZE_PER_EXPERT, 8), (mf.KIND_FINALIZE_PER_EXPERT, 5),
                        (mf.KIND_GATED, 1), (mf.KIND_EP_COMBINE, 1), (mf.KIND_EP_PARTIAL, 8),
                        (mf.KIND_EP_PARTIAL, 2)):
            s = mf.mf_launch_shape(kind, 1000, H, k)
            assert s["waves_per_token"] * s["vectors_per_lane"] * 512 >= H, (kind, H, k)
            assert s["block"] <= (512 if kind == mf.KIND_FINALIZE_PER_EXPERT else 1024)


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros((4, 16), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        mf.mf_moe_finalize(x, torch.zeros((2, 2), dtype=torch.int32),
                           torch.zeros((2, 2)), torch.zeros((2, 16)),
                           torch.zeros(16, dtype=torch.bfloat16))


def route(logits=A, T=16, E=64, k=4, ids=B, w=C, idx=D, perm=E_, off=F, ws=G, ws_bytes=1 << 20):
    return mf.lib().mf_moe_route(logits, T, E, k, ids, w, idx, perm, off, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(T=-1), SHAPE), (dict(ws_bytes=-1), SHAPE), (dict(E=0), UNSUP), (dict(E=1025), UNSUP),
    (dict(k=0), UNSUP), (dict(k=17), UNSUP), (dict(E=4, k=5), UNSUP),
    (dict(T=1 << 28, k=8), SHAPE),             # T * k slots must fit int32
    (dict(ws_bytes=16), SHAPE),                # workspace smaller than required
    (dict(off=None), NULL), (dict(ws=None), NULL), (dict(logits=None), NULL),
    (dict(ids=None), NULL), (dict(w=None), NULL), (dict(idx=None), NULL), (dict(perm=None), NULL),
    (dict(idx=D + 2), ALIGN), (dict(ws=G + 1), ALIGN), (dict(logits=A + 2), ALIGN),
    (dict(idx=B + 8), ALIAS), (dict(perm=G + 64), ALIAS), (dict(off=A + 4), ALIAS),
    (dict(ws=C), ALIAS),
])
def test_route_rejects_bad_arguments(kw, code):
    assert route(**kw) == code


def test_route_workspace_bytes():
    f = mf.mf_moe_route_workspace_bytes
    # 4 * E * (nblocks + 1); a block is 16 waves of tpw tokens
    assert f(0, 8, 2) == 4 * 8 * 1
    assert f(1, 8, 2) == 4 * 8 * 2
    assert f(16384, 256, 8) == 4 * 256 * (16384 // (16 * 4) + 1)     # tpw 4
    assert f(10 ** 6, 1024, 16) == 4 * 1024 * (-(-10 ** 6 // 256) + 1)  # tpw 16
    assert f(10 ** 6, 64, 32 // 2) == 4 * 64 * (-(-10 ** 6 // 256) + 1)
    assert mf.lib().mf_moe_route_workspace_bytes(-1, 8, 2) == SHAPE
    assert mf.lib().mf_moe_route_workspace_bytes(8, 0, 1) == UNSUP
    with pytest.raises(mf.MFError):
        f(8, 4, 5)


def route_noalloc(logits=A, T=16, E=64, k=4, ids=B, w=C, idx=D, perm=E_, off=F):
    return mf.lib().mf_moe_route_noalloc(logits, T, E, k, ids, w, idx, perm, off, None)


@pytest.mark.parametrize("kw,code", [
    (dict(T=-1), SHAPE), (dict(E=0), UNSUP), (dict(E=1025), UNSUP), (dict(k=17), UNSUP),
    (dict(T=1 << 28, k=8), SHAPE),
    (dict(T=2_000_000, E=256, k=8), SCRATCH),  # 8 MB of counts: beyond the 4 MiB scratch
    (dict(off=None), NULL), (dict(logits=None), NULL), (dict(perm=None), NULL),
    (dict(idx=D + 2), ALIGN), (dict(idx=B + 8), ALIAS), (dict(off=A + 4), ALIAS),
])
def test_route_noalloc_rejects_bad_arguments(kw, code):
    # every check runs before the scratch lookup, the call's only HIP query
    assert route_noalloc(**kw) == code


def test_route_noalloc_scratch_limit():
    f = mf.mf_moe_route_workspace_bytes
    assert f(16384, 256, 8) <= mf.MF_ROUTE_SCRATCH_BYTES
    assert f(1_000_000, 256, 8) <= mf.MF_ROUTE_SCRATCH_BYTES < f(1_100_000, 256, 8)
    hdr = open(HEADER).read()
    assert re.search(r"#define MF_ROUTE_SCRATCH_BYTES \(4 << 20\)", hdr)
    assert mf.MF_ROUTE_SCRATCH_BYTES == 4 << 20


def test_empty_grid_rejects_bad_shapes():
    g = mf.lib().mf_empty_grid
    assert g(0, 64, None) == SHAPE
    assert g(-5, 64, None) == SHAPE
    assert g(8, 0, None) == SHAPE
    assert g(8, 1025, None) == SHAPE
    assert g(1 << 31, 1024, None) == SHAPE        # past the 32-bit work-item count
