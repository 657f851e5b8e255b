"""GPU parity of the scans with a carried-in state and of the scaled scan.

mru_scan_fwd_ex: P_t = P_0 M_1 ... M_t, P_0 = 2^carry_exp * carry, optionally
written as 2^E_t times a normalised matrix.  mru_scan_bwd_ex: dM and dL/dP_0.
Graded against the fp64 oracle (scan_ref / bwd_ref with C0, scaled_ref) with
the forward / backward tolerances; bitwise where the arithmetic is the same
(segments and token-by-token streaming of the vector-ALU sizes continue from
the exact fp32 state; a scaled result times its power of two is the unscaled
result).
"""
import numpy as np
import pytest
import torch

from gpu_helpers import BWD_TOL, FWD_TOL, dev, host, random_M, say
from oracle import build_ref, bwd_ref, rel_fro_err, representable, scaled_ref, scan_ref
from workloads import WORKLOADS, gen_R, gen_x

pytestmark = pytest.mark.gpu

SIGMA = {4: (0.1, 0.05), 8: (0.1, 0.05), 16: (0.05, 0.02), 32: (0.02, 0.01)}
SINGLE = 1 << 30  # a chunk longer than any sequence here: one chunk per sequence


@pytest.fixture(scope="module")
def mpp():
    import matrix_prefix_product_amd as m
    m.load_library()
    return m


def _M(B, H, T, n, seed):
    so, sd = SIGMA[n]
    return random_M((B, H, T), n, so, sd, seed)


def _carry(B, H, n, seed):
    # a well-conditioned state with det != 1 and mixed signs
    rng = np.random.default_rng(seed)
    return (np.eye(n) * 1.5 + rng.normal(0, 0.3, size=(B, H, n, n))).astype(np.float32)


CASES = [
    (4, 2, 3, 203, 0), (4, 1, 1, 1024, 0), (4, 2, 2, 97, 1),
    (8, 2, 3, 203, 5), (8, 1, 2, 500, 0), (8, 3, 2, 64, 64),
    (16, 1, 3, 600, 0), (16, 2, 1, 257, 7), (16, 3, 1, 130, SINGLE),
    (32, 1, 2, 400, 0), (32, 2, 1, 150, 13),
]


@pytest.mark.parametrize("n,B,H,T,chunk", CASES)
def test_fwd_carry_parity(mpp, n, B, H, T, chunk):
    say(f"[fwd carry] n={n} B={B} H={H} T={T} chunk={chunk} plan={mpp.scan_plan(B, H, T, n, 0, chunk)}")
    M32 = _M(B, H, T, n, seed=T + n)
    C = _carry(B, H, n, seed=n)
    cexp = np.arange(B * H, dtype=np.int32).reshape(B, H) - 1   # 2^-1, 2^0, 2^1, ...
    P = host(mpp.scan_fwd_ex(dev(M32), carry=dev(C), carry_exp=dev(cexp), chunk=chunk))
    C0 = np.ldexp(C.astype(np.float64), cexp[..., None, None])
    ref = scan_ref(M32, C0)
    err = rel_fro_err(P, ref)
    say(f"  max {err.max():.3e}")
    assert err.max() <= FWD_TOL
    if n <= 8:
        # the same through the x path (factors applied on chip)
        x = gen_x(B, H, T, n, *SIGMA[n], seed=T + n)
        Px = host(mpp.scan_fwd_ex(dev(x), carry=dev(C), from_x=True, n=n, chunk=chunk))
        errx = rel_fro_err(Px, scan_ref(build_ref(x, n), C.astype(np.float64)))
        say(f"  from x: max {errx.max():.3e}")
        assert errx.max() <= FWD_TOL


@pytest.mark.parametrize("n", [4, 8])
def test_segments_and_streaming_are_bitwise(mpp, n):
    # one chunk per sequence: the chain state is the fp32 output itself, so
    # continuing from the last prefix repeats the same arithmetic exactly
    B, H, T, k = 2, 3, 300, 137
    Md = dev(_M(B, H, T, n, seed=3))
    whole = mpp.scan_fwd_ex(Md, chunk=SINGLE)
    head = mpp.scan_fwd_ex(Md[:, :, :k].contiguous(), chunk=SINGLE)
    tail = mpp.scan_fwd_ex(Md[:, :, k:].contiguous(), carry=head[:, :, -1].contiguous(), chunk=SINGLE)
    assert torch.equal(torch.cat([head, tail], dim=2), whole)
    # token-by-token decode
    state = None
    for t in range(40):
        state = mpp.scan_fwd_ex(Md[:, :, t:t + 1].contiguous(), carry=state, chunk=SINGLE)[:, :, 0]
        assert torch.equal(state, whole[:, :, t])
        state = state.contiguous()


@pytest.mark.parametrize("n", [16, 32])
def test_segments_mfma(mpp, n):
    # fp64 chains: the fp32 carry between segments rounds the state once
    B, H, T, k = 1, 2, 400, 150
    M32 = _M(B, H, T, n, seed=5)
    Md = dev(M32)
    head = mpp.scan_fwd_ex(Md[:, :, :k].contiguous())
    tail = mpp.scan_fwd_ex(Md[:, :, k:].contiguous(), carry=head[:, :, -1].contiguous())
    ref = scan_ref(M32)
    err = rel_fro_err(host(torch.cat([head, tail], dim=2)), ref)
    say(f"[segments n={n}] max {err.max():.3e}")
    assert err.max() <= FWD_TOL


SCALED_CASES = [(4, 1, 1, 1024, 0), (4, 2, 2, 300, 7), (8, 2, 3, 203, 5), (8, 1, 2, 500, 0),
                (16, 1, 2, 600, 0), (16, 2, 1, 200, SINGLE), (16, 1, 1, 640, 64),  # register-retained chunks
                (32, 1, 2, 300, 0), (32, 1, 1, 90, 11)]


@pytest.mark.parametrize("n,B,H,T,chunk", SCALED_CASES)
def test_scaled_matches_unscaled_and_oracle(mpp, n, B, H, T, chunk):
    say(f"[scaled] n={n} B={B} H={H} T={T} chunk={chunk}")
    M32 = _M(B, H, T, n, seed=7 * T + n)
    Md = dev(M32)
    C = _carry(B, H, n, seed=n + 1)
    cexp = np.full((B, H), 3, np.int32)
    Pm, E = mpp.scan_fwd_ex(Md, carry=dev(C), carry_exp=dev(cexp), scaled=True, chunk=chunk)
    P = mpp.scan_fwd_ex(Md, carry=dev(C), carry_exp=dev(cexp), chunk=chunk)
    Pm, E, P = host(Pm), host(E), host(P)
    big = np.abs(Pm).max(axis=(-1, -2))
    assert np.all((big >= 0.5) & (big <= 1.0))
    # exact powers of two: 2^E * Pm is the unscaled result bit for bit
    assert np.array_equal(np.ldexp(Pm, E[..., None, None]).astype(np.float32), P)
    ref = scan_ref(M32, np.ldexp(C.astype(np.float64), 3))
    err = rel_fro_err(np.ldexp(Pm.astype(np.float64), E[..., None, None]), ref)
    say(f"  max {err.max():.3e}")
    assert err.max() <= FWD_TOL
    # exponents agree with the oracle's normal form (the mantissa may round up to 1.0)
    _, E_ref = scaled_ref(ref)
    assert np.all(np.abs(E.astype(np.int64) - E_ref) <= 1)


@pytest.mark.parametrize("n", [4, 8])
def test_scaled_beyond_fp32_range(mpp, n):
    # a long n <= 8 sequence whose products overflow fp32: the scaled scan keeps
    # going, graded against the fp64 oracle on the same fp32 inputs everywhere
    so, sd = (0.2, 0.1)
    T = 4096 if n == 8 else 8192
    x = gen_x(1, 1, T, n, so, sd, seed=17)
    M32 = build_ref(x, n).astype(np.float32)
    ref = scan_ref(M32)
    assert not representable(ref).all(), "the case must leave the fp32 range"
    Pm, E = mpp.scan_fwd_ex(dev(M32), scaled=True)
    Pm, E = host(Pm), host(E)
    err = rel_fro_err(np.ldexp(Pm.astype(np.float64), E[..., None, None]), ref)
    say(f"[scaled long n={n}] max log2 |P| {E.max()}, max err {err.max():.3e}")
    assert err.max() <= FWD_TOL


BWD_CASES = [(4, 2, 3, 203, 0), (4, 1, 1, 1024, 0), (8, 2, 2, 300, 7), (8, 3, 1, 64, SINGLE),
             (16, 1, 3, 500, 0), (16, 2, 1, 130, 9), (16, 1, 2, 512, 32), (32, 1, 2, 300, 0),
             (32, 1, 1, 70, 1)]


@pytest.mark.parametrize("n,B,H,T,chunk", BWD_CASES)
def test_bwd_carry_parity(mpp, n, B, H, T, chunk):
    say(f"[bwd carry] n={n} B={B} H={H} T={T} chunk={chunk} plan={mpp.scan_plan(B, H, T, n, 1, chunk)}")
    M32 = _M(B, H, T, n, seed=T + 2 * n)
    R = gen_R(B, H, T, n, seed=T)
    C = _carry(B, H, n, seed=2 * n)
    Md, Cd = dev(M32), dev(C)
    P = mpp.scan_fwd_ex(Md, carry=Cd)
    dM, dC = mpp.scan_bwd_ex(Md, P, dev(R), carry=Cd, want_dcarry=True, chunk=chunk)
    ref_dM, ref_dC = bwd_ref(M32, R, C.astype(np.float64), want_dC0=True)
    e1 = rel_fro_err(host(dM), ref_dM)
    e2 = rel_fro_err(host(dC), ref_dC)
    say(f"  dM max {e1.max():.3e}  dC max {e2.max():.3e}")
    assert e1.max() <= BWD_TOL and e2.max() <= BWD_TOL
    if True:  # from raw token vectors, every n
        x = gen_x(B, H, T, n, *SIGMA[n], seed=T + 2 * n)
        xd = dev(x)
        Px = mpp.scan_fwd_ex(xd, carry=Cd, from_x=True, n=n)
        dMx, dCx = mpp.scan_bwd_ex(xd, Px, dev(R), carry=Cd, want_dcarry=True, from_x=True, chunk=chunk)
        rM, rC = bwd_ref(build_ref(x, n), R, C.astype(np.float64), want_dC0=True)
        ex1, ex2 = rel_fro_err(host(dMx), rM), rel_fro_err(host(dCx), rC)
        say(f"  from x: dM max {ex1.max():.3e}  dC max {ex2.max():.3e}")
        assert ex1.max() <= BWD_TOL and ex2.max() <= BWD_TOL


@pytest.mark.parametrize("n", [8, 16])
def test_bwd_through_two_segments(mpp, n):
    # the documented recipe: the second segment's dcarry joins the first
    # segment's dP at its last token; together they give the whole gradient
    B, H, T, k = 1, 2, 300, 120
    M32 = _M(B, H, T, n, seed=9)
    R = gen_R(B, H, T, n, seed=10)
    Md, Rd = dev(M32), dev(R)
    Pa = mpp.scan_fwd_ex(Md[:, :, :k].contiguous())
    carry = Pa[:, :, -1].contiguous()
    Pb = mpp.scan_fwd_ex(Md[:, :, k:].contiguous(), carry=carry)
    dMb, dC = mpp.scan_bwd_ex(Md[:, :, k:].contiguous(), Pb, Rd[:, :, k:].contiguous(), carry=carry,
                              want_dcarry=True)
    Ra = Rd[:, :, :k].clone()
    Ra[:, :, -1] += dC
    dMa = mpp.scan_bwd_ex(Md[:, :, :k].contiguous(), Pa, Ra)
    err = rel_fro_err(host(torch.cat([dMa, dMb], dim=2)), bwd_ref(M32, R))
    say(f"[bwd segments n={n}] max {err.max():.3e}")
    assert err.max() <= BWD_TOL


def test_carry_without_tokens_writes_nothing(mpp):
    C = dev(_carry(2, 1, 8, seed=1))
    P = mpp.scan_fwd_ex(torch.zeros(2, 1, 0, 8, 8, device="cuda"), carry=C)
    assert P.shape == (2, 1, 0, 8, 8)
    dM, dC = mpp.scan_bwd_ex(torch.zeros(2, 1, 0, 8, 8, device="cuda"), P, P, carry=C,
                             want_dcarry=True)
    assert torch.count_nonzero(dC) == 0


@pytest.mark.parametrize("h", [0, 7])
def test_c4_scaled_full_length(mpp, h):
    # n = 32 at full length: 64K tokens reach |P| ~ e^389, far beyond fp32; the
    # scaled scan is graded against the fp64 oracle at every token, including
    # the 1K / 8K / 64K tracking points (the first and the last head)
    w = WORKLOADS["c4"]
    x = gen_x(w.B, w.H, w.T, w.n, w.sigma_off, w.sigma_diag, w.seed, b_idx=[0], h_idx=[h])
    M32 = build_ref(x, w.n).astype(np.float32)
    Pm, E = mpp.scan_fwd_ex(dev(M32), scaled=True)
    Pm, E = host(Pm), host(E)
    ref = scan_ref(M32)
    got = np.ldexp(Pm.astype(np.float64), E[..., None, None])
    err = rel_fro_err(got, ref)
    for t in (1024, 8192, 65536):
        r = ref[0, 0, t - 1]
        sc = np.abs(r).max()
        ln = float(np.log(sc) + np.log(np.linalg.norm(r / sc)))
        say(f"[c4 scaled head {h}] t={t}: ln||P|| {ln:.1f}  err {err[0, 0, t - 1]:.3e}")
    say(f"  max over all t {err.max():.3e}")
    assert err.max() <= FWD_TOL
