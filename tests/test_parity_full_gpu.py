"""Full-size workload parity on the GPU, in the launch configuration the
benchmark times (automatic chunk plan), against the fp64 oracle.

Every P_t (and every dM_t for the backward cases) is compared on the
fp32-representable domain: entries of the exact P_t at most 2^125.  Beyond it
the exact products exceed the fp32 range (the running product of det-1
matrices still grows exponentially) and the fp32 output holds +-inf / nan,
as IEEE arithmetic gives it; those matrices are counted and reported, not
graded.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import BWD_TOL, FWD_TOL, dev, host, inputs, say, summary
from oracle import bwd_ref, rel_fro_err, representable, scan_ref
from workloads import WORKLOADS, gen_R

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mpp():
    import matrix_prefix_product_amd as m
    m.load_library()
    return m


@pytest.mark.parametrize("name", ["c1", "c2", "c2l", "c3", "c5"])
def test_full_forward(mpp, name):
    w = WORKLOADS[name]
    say(f"[full fwd] {name}: B={w.B} H={w.H} T={w.T} n={w.n} plan={mpp.scan_plan(w.B, w.H, w.T, w.n)}")
    x, M32, _ = inputs(name)
    Md = dev(M32)
    P = host(mpp.scan_fwd(Md, check=True))
    P_ref = scan_ref(M32)
    dom = representable(P_ref)
    err = rel_fro_err(P, P_ref)
    say("  " + summary(err, dom))
    assert err[dom].max() <= FWD_TOL
    # outside the domain the GPU value is not finite or the exact one is huge
    assert np.all(np.isfinite(P[dom]))


def test_full_forward_c4_streamed(mpp):
    # n=32, T=65536, 8 heads: compared one head at a time to bound host memory.
    w = WORKLOADS["c4"]
    say(f"[full fwd] c4: plan={mpp.scan_plan(w.B, w.H, w.T, w.n)}")
    from workloads import gen_x
    from oracle import build_ref
    M32 = np.empty((w.B, w.H, w.T, w.n, w.n), np.float32)
    for h in range(w.H):
        x = gen_x(w.B, w.H, w.T, w.n, w.sigma_off, w.sigma_diag, w.seed, h_idx=[h])
        M32[:, h:h + 1] = build_ref(x, w.n).astype(np.float32)
    P = mpp.scan_fwd(dev(M32), check=True)
    torch.cuda.synchronize()
    worst = 0.0
    graded = outside = 0
    track = {}
    for h in range(w.H):
        Ph = host(P[:, h])
        Pr = scan_ref(M32[:, h])
        dom = representable(Pr)
        err = rel_fro_err(Ph, Pr)
        worst = max(worst, float(err[dom].max()))
        graded += int(dom.sum())
        outside += int((~dom).sum())
        for t in (1024, 8192, 65536):
            A = Pr[0, t - 1]
            amax = float(np.abs(A).max())
            lnorm = float(np.log(amax) + np.log(np.linalg.norm(A / amax)))  # no overflow
            e = float(err[0, t - 1]) if dom[0, t - 1] else None
            track.setdefault(t, []).append((e, lnorm))
    say(f"  max {worst:.3e} graded {graded} outside-domain {outside}")
    for t, v in track.items():
        es = [e for e, _ in v if e is not None]
        say(f"  t={t}: err max {max(es):.3e}" if es else
            f"  t={t}: unrepresentable in fp32 (oracle ln||P|| {min(l for _, l in v):.1f}..{max(l for _, l in v):.1f})")
    assert worst <= FWD_TOL
    assert graded > 0


@pytest.mark.parametrize("name", ["c5", "c2"])
def test_full_backward(mpp, name):
    w = WORKLOADS[name]
    say(f"[full bwd] {name}: plan={mpp.scan_plan(w.B, w.H, w.T, w.n, mpp.DIR_BWD)}")
    x, M32, R = inputs(name)
    if R is None:
        R = gen_R(w.B, w.H, w.T, w.n, w.seed)
    Md = dev(M32)
    P = mpp.scan_fwd(Md, check=True)
    dM = host(mpp.scan_bwd(Md, P, dev(R), check=True))
    ref = bwd_ref(M32, R)
    assert np.all(np.isfinite(ref))
    err = rel_fro_err(dM, ref)
    say(f"  max {err.max():.3e} p99.9 {np.quantile(err, 0.999):.3e} median {np.median(err):.3e}")
    assert err.max() <= BWD_TOL


def test_full_backward_c2l_sampled(mpp):
    # 8192 sequences: every 64th sequence compared (all of its tokens).
    w = WORKLOADS["c2l"]
    say(f"[full bwd] c2l: plan={mpp.scan_plan(w.B, w.H, w.T, w.n, mpp.DIR_BWD)}")
    x, M32, _ = inputs("c2l")
    R = gen_R(w.B, w.H, w.T, w.n, w.seed)
    Md = dev(M32)
    P = mpp.scan_fwd(Md, check=True)
    dM = mpp.scan_bwd(Md, P, dev(R), check=True)
    torch.cuda.synchronize()
    sel = np.arange(0, w.B, 64)
    got = host(dM[sel])
    ref = bwd_ref(M32[sel], R[sel])
    err = rel_fro_err(got, ref)
    say(f"  sampled {len(sel) * w.H} sequences: max {err.max():.3e}")
    assert err.max() <= BWD_TOL


def test_full_backward_from_x_c5(mpp):
    # the n = 16 training workload from the raw token vectors: forward and
    # backward both form every input matrix on chip, against the oracle's fp64
    # build, forward and backward (every dM_t graded)
    w = WORKLOADS["c5"]
    say(f"[full bwd from x] c5: plan={mpp.scan_plan(w.B, w.H, w.T, w.n, mpp.DIR_BWD)}")
    x, _, R = inputs("c5")
    xd = dev(x)
    P = mpp.scan_fwd_x(xd, w.n, check=True)
    dM = host(mpp.scan_bwd_x(xd, P, dev(R), check=True))
    from oracle import build_ref
    ref = bwd_ref(build_ref(x, w.n), R)
    err = rel_fro_err(dM, ref)
    say(f"  max {err.max():.3e} p99.9 {np.quantile(err, 0.999):.3e} median {np.median(err):.3e}")
    assert err.max() <= BWD_TOL
