"""The look-back never reads a workspace slot that has not been published in
the same launch.

The library clears only the workspace header and flags before a multi-chunk
scan; the matrix slots keep whatever the memory held.  Here every slot starts
as all-ones bytes, a NaN in fp32 and in fp64, so a matrix read before its
owner wrote it (a missing wait, a flag set before its data, a wrong slot
index) turns the outputs into NaN or changes them.  Each multi-chunk scan is
run twice, once on a NaN-filled and once on a zero-filled workspace: the
outputs must be finite and bitwise the same, and the status word must stay 0.
(Workspaces the binding allocates itself usually come back from torch's cache
holding an earlier call's values, which would hide such a read.)
"""
import numpy as np
import pytest
import torch

from gpu_helpers import dev, host, say
from oracle import build_ref
from workloads import gen_R, gen_x

pytestmark = pytest.mark.gpu

SIGMA = {4: (0.1, 0.05), 8: (0.1, 0.05), 16: (0.05, 0.02), 32: (0.02, 0.01)}

# (n, B, H, T, chunk): every plan cuts each sequence into many chunks and
# several supers, with a ragged last chunk
CASES = [(4, 2, 3, 611, 16), (8, 2, 3, 611, 16), (8, 3, 2, 250, 0), (16, 2, 2, 701, 16),
         (16, 4, 4, 700, 0), (32, 1, 3, 517, 16), (32, 1, 2, 300, 0)]


@pytest.fixture(scope="module")
def mpp():
    import matrix_prefix_product_amd as m
    m.load_library()
    return m


def _ws(mpp, B, H, T, n, direction, chunk, fill):
    nbytes = mpp.workspace_bytes(B, H, T, n, direction, chunk)
    assert nbytes > 0, "the plan must be multi-chunk"
    return torch.full((nbytes,), fill, dtype=torch.uint8, device="cuda")


def _same_and_finite(a, b, what):
    a, b = host(a), host(b)
    assert np.isfinite(a).all(), f"{what}: non-finite outputs from a NaN-filled workspace"
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"{what}: depends on the workspace's old contents"


@pytest.mark.parametrize("n,B,H,T,chunk", CASES)
def test_scans_read_only_published_slots(mpp, n, B, H, T, chunk):
    plan_f = mpp.scan_plan(B, H, T, n, mpp.DIR_FWD, chunk)
    plan_b = mpp.scan_plan(B, H, T, n, mpp.DIR_BWD, chunk)
    say(f"[poisoned workspace] n={n} B={B} H={H} T={T} chunk={chunk} fwd plan {plan_f} bwd plan {plan_b}")
    assert plan_f[1] > plan_f[2] and plan_b[1] > plan_b[2], "several supers per sequence"
    so, sd = SIGMA[n]
    x = gen_x(B, H, T, n, so, sd, seed=T + 101)
    R = gen_R(B, H, T, n, seed=T + 102)
    xd, Rd = dev(x), dev(R)
    Md = dev(build_ref(x, n).astype(np.float32))
    runs = {}
    for fill in (0xFF, 0x00):
        o = {}
        o["fwd"] = mpp.scan_fwd(Md, chunk, workspace=_ws(mpp, B, H, T, n, mpp.DIR_FWD, chunk, fill), check=True)
        o["bwd"] = mpp.scan_bwd(Md, o["fwd"], Rd, chunk,
                                workspace=_ws(mpp, B, H, T, n, mpp.DIR_BWD, chunk, fill), check=True)
        o["fwd_x"] = mpp.scan_fwd_x(xd, n, chunk, workspace=_ws(mpp, B, H, T, n, mpp.DIR_FWD, chunk, fill),
                                    check=True)
        o["bwd_x"] = mpp.scan_bwd_x(xd, o["fwd_x"], Rd, chunk,
                                    workspace=_ws(mpp, B, H, T, n, mpp.DIR_BWD, chunk, fill), check=True)
        o["bwd_dx"] = mpp.scan_bwd_dx(xd, o["fwd_x"], Rd, chunk=chunk,
                                      workspace=_ws(mpp, B, H, T, n, mpp.DIR_BWD, chunk, fill), check=True)
        P, E = mpp.scan_fwd_ex(Md, scaled=True, chunk=chunk,
                               workspace=_ws(mpp, B, H, T, n, mpp.DIR_FWD, chunk, fill), check=True)
        o["fwd_scaled"], o["fwd_scaled_exp"] = P, E.float()
        runs[fill] = o
    for k in runs[0xFF]:
        _same_and_finite(runs[0xFF][k], runs[0x00][k], k)
