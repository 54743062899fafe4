"""mf_moe_route_noalloc (the routing call on the library's static scratch) against
mf_moe_route with a caller workspace, through the C ABI on the GPU.

Both run the same kernels, so every output must be bit-identical: expert ids, idx, perm and
offsets are integers with one correct answer, and the weights come from the same fp32
arithmetic.  Two calls in a row share the one scratch array; the second is smaller (and takes
the two-launch path of small calls), so stale counts left by the first call must not leak into
it.  The outputs start filled with garbage, so every element must be written.
"""
import numpy as np
import pytest
import torch

import finalize_residual_rmsnorm_amd as mf
import oracle
import workloads

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")

# (T, E, k, seed): the prefill routing size (three launches), then a smaller decode-size call
# (two launches) that reuses the scratch the first one left behind
CALLS = [(16384, 256, 8, 601), (300, 128, 8, 602)]


def garbage_outputs(T, E, k):
    fill = lambda shape, dt, v: torch.full(shape, v, dtype=dt, device=DEV)
    return dict(expert_ids=fill((T, k), torch.int32, -7), weights=fill((T, k), torch.float32, -3.5),
                idx=fill((T, k), torch.int32, 0x7FFFFFFF), perm=fill((T * k,), torch.int32, -1),
                offsets=fill((E + 1,), torch.int32, 12345))


def test_noalloc_route_matches_workspace_route_on_two_calls():
    assert mf.mf_moe_route_workspace_bytes(16384, 256, 8) <= mf.MF_ROUTE_SCRATCH_BYTES
    for T, E, k, seed in CALLS:
        print(f"route noalloc vs workspace: T={T} E={E} k={k} "
              f"workspace={mf.mf_moe_route_workspace_bytes(T, E, k)} B", flush=True)
        logits = workloads.make_route_inputs(T, E, k, seed=seed)["logits"]
        lg = torch.from_numpy(logits).to(DEV)
        ref = mf.mf_moe_route(lg, k)
        got = garbage_outputs(T, E, k)
        mf.mf_moe_route_noalloc(lg, k, **got)
        torch.cuda.synchronize()
        names = ["expert_ids", "weights", "idx", "perm", "offsets"]
        for name, r in zip(names, ref):
            assert torch.equal(got[name], r), f"{name} differs (T={T})"
        # the integer outputs also match the oracle
        oe, ow, oi, op, oo = oracle.moe_route(logits, k)
        assert np.array_equal(got["expert_ids"].cpu().numpy(), oe)
        assert np.array_equal(got["idx"].cpu().numpy(), oi)
        assert np.array_equal(got["perm"].cpu().numpy(), op)
        assert np.array_equal(got["offsets"].cpu().numpy(), oo)


def test_noalloc_route_rejects_a_problem_beyond_the_scratch():
    # checked on the host before any launch: nothing is written
    T, E, k = 2_000_000, 256, 8
    assert mf.mf_moe_route_workspace_bytes(T, E, k) > mf.MF_ROUTE_SCRATCH_BYTES
    lg = torch.zeros((T, E), dtype=torch.float32, device=DEV)
    out = garbage_outputs(T, E, k)
    with pytest.raises(mf.MFError) as e:
        mf.mf_moe_route_noalloc(lg, k, **out)
    assert e.value.status == -8
    torch.cuda.synchronize()
    assert torch.all(out["offsets"] == 12345)
