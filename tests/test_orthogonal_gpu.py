"""GPU parity of the orthogonal input constructions and of scans over them.

mru_build_orthogonal computes the Cayley map / exponential of A = (X - X^T)/2
in fp64 and rounds once to fp32, so it must match the fp64 oracle
(build_orthogonal_ref) to within fp32 rounding: ORTHO_TOL = 1e-7 relative
Frobenius error per matrix (2^-24 = 6e-8 for the final rounding, plus the
fp64 arithmetic, which is ~1e-14).  Products of orthogonal matrices keep
|P_t|_F = sqrt(n), so long scans are graded at every token with no overflow
domain.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import FWD_TOL, dev, host, say
from oracle import build_orthogonal_ref, rel_fro_err, scan_ref
from workloads import WORKLOADS, gen_x

pytestmark = pytest.mark.gpu

ORTHO_TOL = 1e-7


@pytest.fixture(scope="module")
def mpp():
    import matrix_prefix_product_amd as m
    m.load_library()
    return m


@pytest.mark.parametrize("method", ["cayley", "expm"])
@pytest.mark.parametrize("n", [4, 8, 16, 32])
def test_orthogonal_build_parity(mpp, method, n):
    say(f"[orthogonal build] {method} n={n}")
    for scale in (0.05, 0.5, 3.0):       # exp needs 0, a few and many squarings
        x = gen_x(2, 3, 37, n, scale, scale, seed=n)
        M = host(mpp.build_orthogonal(dev(x), n, method))
        ref = build_orthogonal_ref(x, n, method)
        err = rel_fro_err(M, ref)
        I = np.eye(n)
        orth = np.abs(np.swapaxes(M, -1, -2).astype(np.float64) @ M - I).max()
        say(f"  scale {scale}: max rel err {err.max():.3e}, max |M^T M - I| {orth:.2e}")
        assert err.max() <= ORTHO_TOL
        assert orth <= 4 * n * 2.0 ** -24
    # symmetric tokens give exactly I; an empty batch is a no-op
    xs = gen_x(1, 1, 5, n, 0.3, 0.3, seed=1).reshape(5, n, n)
    xs = (xs + np.swapaxes(xs, -1, -2)).reshape(1, 1, 5, n * n).astype(np.float32)
    assert np.array_equal(host(mpp.build_orthogonal(dev(xs), n, method)),
                          np.broadcast_to(np.eye(n, dtype=np.float32), (1, 1, 5, n, n)))
    assert mpp.build_orthogonal(torch.zeros(0, 2, 3, n * n, device="cuda"), n, method).numel() == 0


def test_orthogonal_bad_method(mpp):
    x = torch.zeros(1, 1, 2, 16, device="cuda")
    with pytest.raises(ValueError):
        mpp.build_orthogonal(x, 4, "qr")
    import ctypes
    M = torch.empty(1, 1, 2, 4, 4, device="cuda")
    st = mpp.load_library().mru_build_orthogonal(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(M.data_ptr()),
                                                 1, 1, 2, 4, 7, None)
    assert st == 2


@pytest.mark.parametrize("method", ["cayley", "expm"])
def test_orthogonal_scan_full_length(mpp, method):
    # the n = 32, 64K-token workload with orthogonal inputs: every prefix is
    # orthogonal, so every token is graded (two of the eight heads)
    w = WORKLOADS["c4"]
    for h in (0, 5):
        x = gen_x(w.B, w.H, w.T, w.n, w.sigma_off, w.sigma_diag, w.seed, b_idx=[0], h_idx=[h])
        M = mpp.build_orthogonal(dev(x), w.n, method)
        P = host(mpp.scan_fwd(M))
        M32 = host(M)
        ref = scan_ref(M32)
        err = rel_fro_err(P, ref)
        nrm = np.linalg.norm(P[0, 0, -1].astype(np.float64))
        say(f"[orthogonal scan {method} head {h}] max err over {w.T} tokens {err.max():.3e}, "
            f"|P_T|_F {nrm:.6f} (sqrt(n) = {np.sqrt(w.n):.6f})")
        assert err.max() <= FWD_TOL
        assert abs(nrm - np.sqrt(w.n)) <= 1e-3


@pytest.mark.parametrize("n", [4, 8, 16, 32])
def test_orthogonal_scan_and_backward_small(mpp, n):
    from gpu_helpers import BWD_TOL
    from oracle import bwd_ref
    from workloads import gen_R
    B, H, T = 2, 3, 700
    x = gen_x(B, H, T, n, 0.3, 0.3, seed=3)
    Md = mpp.build_orthogonal(dev(x), n, "expm")
    M32 = host(Md)
    for chunk in (0, 13):
        P = mpp.scan_fwd(Md, chunk)
        assert rel_fro_err(host(P), scan_ref(M32)).max() <= FWD_TOL
        R = gen_R(B, H, T, n, seed=4)
        dM = host(mpp.scan_bwd(Md, P, dev(R), chunk))
        assert rel_fro_err(dM, bwd_ref(M32, R)).max() <= BWD_TOL
