"""Tensors of more than 2^31 elements: every offset the kernels form is 64-bit.

Each case fills the raw token vectors x past 2^31 fp32 elements (seeded draws
from torch's generator on the device, scaled per entry), runs the path on the
whole tensor, and compares whole sequences -- the first, one in the middle and
the last, whose offsets are the largest -- with the fp64 oracle run on the same
x.  For n = 4, 8 the scans start from x (the build fused); for n = 16, 32 the
device build is checked on the sampled sequences and then, as in the other
parity tests, those sequences' input matrices are replaced by the oracle's
fp32-rounded build, so that the scan is compared on the same inputs.  The
scales keep the running products far inside the fp32 range over the sequence
lengths used.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import BUILD_TOL, BWD_TOL, FWD_TOL, say
from oracle import build_ref, build_vjp_ref, bwd_ref, rel_fro_err, representable, scan_ref

pytestmark = pytest.mark.gpu

LIMIT = 2 ** 31

# B, H, T, n, sigma_off, sigma_diag, what the automatic plan makes of it
CASES = [
    (8192, 8, 2050, 4, 0.1, 0.05),     # n = 4, one chunk per sequence
    (4096, 8, 1040, 8, 0.1, 0.05),     # n = 8, one chunk per sequence
    (256, 8, 16400, 8, 0.01, 0.01),    # n = 8, several chunks per sequence
    (256, 8, 4100, 16, 0.02, 0.01),    # n = 16: one chunk forward, two backward
    (8, 8, 32800, 32, 0.005, 0.002),   # n = 32, several chunks per sequence
]


@pytest.fixture(scope="module")
def mpp():
    import matrix_prefix_product_amd as m
    m.load_library()
    return m


def make_x(B, H, T, n, s_off, s_diag, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    x = torch.randn((B, H, T, n * n), generator=g, device="cuda")
    scale = torch.full((n, n), s_off, device="cuda")
    scale.fill_diagonal_(s_diag)
    x.mul_(scale.reshape(n * n))
    return x


def make_R(shape, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device="cuda")


def sampled(B, H):
    return [(0, 0), (B // 2, H // 2), (B - 1, H - 1)]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c[0]}H{c[1]}T{c[2]}n{c[3]}")
def test_past_2g_elements(mpp, case):
    B, H, T, n, s_off, s_diag = case
    assert B * H * T * n * n > LIMIT
    fwd_plan = mpp.scan_plan(B, H, T, n, mpp.DIR_FWD)
    bwd_plan = mpp.scan_plan(B, H, T, n, mpp.DIR_BWD)
    say(f"[large] B={B} H={H} T={T} n={n}: {B * H * T * n * n} elements, "
        f"fwd plan {fwd_plan[:3]}, bwd plan {bwd_plan[:3]}")
    x = make_x(B, H, T, n, s_off, s_diag, seed=1000 + n)
    fused = n in mpp.FUSED_N
    samples = sampled(B, H)
    xs = {bh: x[bh].cpu().numpy() for bh in samples}
    Ms = {bh: build_ref(xs[bh], n) for bh in samples}
    M32 = {bh: Ms[bh].astype(np.float32) for bh in samples}
    worst = {"build": 0.0, "fwd": 0.0, "bwd": 0.0, "dx": 0.0}
    if fused:
        P = mpp.scan_fwd_x(x, n)
    else:
        M = mpp.build_inputs(x, n)
        for bh in samples:
            worst["build"] = max(worst["build"], float(rel_fro_err(M[bh].cpu().numpy(), Ms[bh]).max()))
            M[bh] = torch.from_numpy(M32[bh]).to("cuda")
        P = mpp.scan_fwd(M)
    R = make_R(P.shape, seed=2000 + n)
    dM = mpp.scan_bwd_x(x, P, R) if fused else mpp.scan_bwd(M, P, R)
    if fused:
        del P  # room for the build and the layer backward
        torch.cuda.empty_cache()
        P = mpp.scan_fwd_x(x, n)
        dx = mpp.scan_bwd_dx(x, P, R)
        M = mpp.build_inputs(x, n)
        for bh in samples:
            worst["build"] = max(worst["build"], float(rel_fro_err(M[bh].cpu().numpy(), Ms[bh]).max()))
    torch.cuda.synchronize()
    for bh in samples:
        Rs = R[bh].cpu().numpy()
        P_ref = scan_ref(M32[bh])
        assert representable(P_ref).all(), "the scales keep every prefix inside the fp32 range"
        worst["fwd"] = max(worst["fwd"], float(rel_fro_err(P[bh].cpu().numpy(), P_ref).max()))
        dM_ref = bwd_ref(M32[bh], Rs)
        worst["bwd"] = max(worst["bwd"], float(rel_fro_err(dM[bh].cpu().numpy(), dM_ref).max()))
        if fused:
            dx_ref = build_vjp_ref(xs[bh], dM_ref, n)
            e_dx = np.linalg.norm(dx[bh].cpu().numpy() - dx_ref, axis=-1) / np.linalg.norm(dx_ref, axis=-1)
            worst["dx"] = max(worst["dx"], float(e_dx.max()))
    say("  worst relative errors over the sampled sequences: "
        + ", ".join(f"{k} {v:.2e}" for k, v in worst.items()))
    assert worst["build"] <= BUILD_TOL
    assert worst["fwd"] <= FWD_TOL
    assert worst["bwd"] <= BWD_TOL
    assert worst["dx"] <= BWD_TOL
    del x, M, P, R, dM
    if fused:
        del dx
    torch.cuda.empty_cache()
