"""GPU parity of the scans that start from raw token vectors (forward n = 4, 8,
16; backward n = 4, 8).

mru_scan_fwd_x / mru_scan_bwd_x multiply by the LDU factors of each input
state matrix instead of forming it (n = 16: form it on chip for the fp64
chain), so they agree with build-then-scan up to rounding order; both are
graded against the fp64 oracle
(scan_ref(build_ref(x)), bwd_ref(build_ref(x), R)) with the forward / backward
tolerances, and must be deterministic run to run.  mru_scan_bwd_dx goes on to
dL/dx in the same pass, graded against build_vjp_ref of the oracle's backward.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import BUILD_TOL, BWD_TOL, FWD_TOL, dev, fwd_errors, host, say, summary
from oracle import build_ref, build_vjp_ref, bwd_ref, rel_fro_err, scaled_ref, scan_ref
from workloads import gen_R, gen_x

pytestmark = pytest.mark.gpu

SIGMA = {4: (0.1, 0.05), 8: (0.1, 0.05), 16: (0.05, 0.02), 32: (0.02, 0.01)}

CASES = [
    (4, 1, 1, 1024, 0), (4, 3, 2, 203, 3), (4, 2, 2, 97, 1), (4, 5, 1, 120, 120),
    (4, 1, 1, 4096, 0),
    (8, 8, 8, 256, 0), (8, 2, 3, 203, 5), (8, 1, 2, 203, 1), (8, 33, 1, 64, 64),
    (8, 2, 2, 500, 16), (8, 1, 1, 1024, 0),
]
# (longer n = 8 sequences at these scales leave the fp32-state domain: by 2048
# tokens the backward error reaches the 5e-4 bound, by ~2900 the products overflow)


@pytest.fixture(scope="module")
def mpp():
    import matrix_prefix_product_amd as m
    m.load_library()
    return m


def _x(B, H, T, n, seed):
    so, sd = SIGMA[n]
    return gen_x(B, H, T, n, so, sd, seed)


@pytest.mark.parametrize("n,B,H,T,chunk", CASES)
def test_fused_fwd(mpp, n, B, H, T, chunk):
    plan = mpp.scan_plan(B, H, T, n, mpp.DIR_FWD, chunk)
    say(f"[fused fwd] n={n} B={B} H={H} T={T} chunk={chunk} plan(K,nch,Z,ws)={plan}")
    x = _x(B, H, T, n, seed=T + n)
    xd = dev(x)
    P = mpp.scan_fwd_x(xd, n, chunk)
    again = mpp.scan_fwd_x(xd, n, chunk)
    assert torch.equal(P.view(torch.int32), again.view(torch.int32)), "not deterministic"
    err, dom, P_ref = fwd_errors(host(P), build_ref(x, n))
    say("  " + summary(err, dom))
    assert err[dom].max() <= FWD_TOL
    # for comparison only: build + scan on the same tokens (its own parity cases
    # are elsewhere; it rounds every M_t to fp32 first, and at n = 8 over 2048
    # tokens that alone costs more than the whole fused error)
    P_two = host(mpp.scan_fwd(mpp.build_inputs(xd, n), chunk))
    say(f"  build + scan: max {rel_fro_err(P_two, P_ref)[dom].max():.3e}")


@pytest.mark.parametrize("n,B,H,T,chunk", CASES)
def test_fused_bwd(mpp, n, B, H, T, chunk):
    plan = mpp.scan_plan(B, H, T, n, mpp.DIR_BWD, chunk)
    say(f"[fused bwd] n={n} B={B} H={H} T={T} chunk={chunk} plan(K,nch,Z,ws)={plan}")
    x = _x(B, H, T, n, seed=T + 3 * n)
    R = gen_R(B, H, T, n, seed=T + 1)
    xd, Rd = dev(x), dev(R)
    P = mpp.scan_fwd_x(xd, n)
    ws = torch.empty(max(plan[3], 256), dtype=torch.uint8, device="cuda")
    dM = mpp.scan_bwd_x(xd, P, Rd, chunk, workspace=ws)
    again = mpp.scan_bwd_x(xd, P, Rd, chunk)
    assert torch.equal(dM.view(torch.int32), again.view(torch.int32)), "not deterministic"
    err = rel_fro_err(host(dM), bwd_ref(build_ref(x, n), R))
    say(f"  max {err.max():.3e} median {np.median(err):.3e}")
    assert err.max() <= BWD_TOL
    if plan[3] > 0:
        assert mpp.ws_status(ws) == 0, "a flag wait timed out"


@pytest.mark.parametrize("n", [4, 8])
def test_fused_zero_input_is_identity(mpp, n):
    # x = 0 builds M_t = I exactly, so every prefix is I and dM is the reverse cumsum of R
    T = 300
    xd = torch.zeros(2, 1, T, n * n, device="cuda")
    for chunk in (0, 7):
        P = host(mpp.scan_fwd_x(xd, n, chunk))
        assert np.array_equal(P, np.broadcast_to(np.eye(n, dtype=np.float32), P.shape))
        R = gen_R(2, 1, T, n, seed=n)
        dM = host(mpp.scan_bwd_x(xd, dev(P), dev(R), chunk))
        expect = np.cumsum(R[:, :, ::-1].astype(np.float64), axis=2)[:, :, ::-1]
        assert rel_fro_err(dM, expect).max() <= BWD_TOL


@pytest.mark.parametrize("n", [4, 8])
def test_fused_edges(mpp, n):
    say(f"[fused edges] n={n}")
    # empty sequences and empty batches are no-ops
    e = mpp.scan_fwd_x(torch.zeros(2, 3, 0, n * n, device="cuda"), n)
    assert e.shape == (2, 3, 0, n, n)
    # one token: P_1 = M_1, dM_1 = R_1
    x = _x(3, 2, 1, n, seed=5)
    P = host(mpp.scan_fwd_x(dev(x), n))
    assert rel_fro_err(P, build_ref(x, n)).max() <= BUILD_TOL
    R = gen_R(3, 2, 1, n, seed=6)
    dM = host(mpp.scan_bwd_x(dev(x), dev(P), dev(R)))
    assert np.array_equal(dM, R)


@pytest.mark.parametrize("n,B,H,T,chunk", CASES)
def test_layer_bwd_dx(mpp, n, B, H, T, chunk):
    # x, P, dL/dP -> dL/dx in one pass, against the oracle's build VJP of its
    # backward scan; and against the two-kernel path (backward to dM, then the
    # build's gradient), which it equals up to rounding order
    plan = mpp.scan_plan(B, H, T, n, mpp.DIR_BWD, chunk)
    say(f"[layer bwd dx] n={n} B={B} H={H} T={T} chunk={chunk} plan(K,nch,Z,ws)={plan}")
    x = _x(B, H, T, n, seed=T + 5 * n)
    R = gen_R(B, H, T, n, seed=T + 2)
    xd, Rd = dev(x), dev(R)
    P = mpp.scan_fwd_x(xd, n)
    ws = torch.empty(max(plan[3], 256), dtype=torch.uint8, device="cuda")
    dx = mpp.scan_bwd_dx(xd, P, Rd, chunk=chunk, workspace=ws)
    again = mpp.scan_bwd_dx(xd, P, Rd, chunk=chunk)
    assert torch.equal(dx.view(torch.int32), again.view(torch.int32)), "not deterministic"
    ref = build_vjp_ref(x, bwd_ref(build_ref(x, n), R), n)
    shape = (B, H, T, n, n)
    err = rel_fro_err(host(dx).reshape(shape), ref.reshape(shape))
    two = build_vjp_ref(x, host(mpp.scan_bwd_x(xd, P, Rd, chunk)), n)  # fp64 build VJP of the GPU dM
    two_gpu = host(mpp.build_inputs_bwd(xd, mpp.scan_bwd_x(xd, P, Rd, chunk)))
    d2 = rel_fro_err(host(dx).reshape(shape), two_gpu.reshape(shape))
    say(f"  max {err.max():.3e} median {np.median(err):.3e}; vs two kernels max {d2.max():.3e}")
    assert err.max() <= BWD_TOL
    assert rel_fro_err(host(dx).reshape(shape), two.reshape(shape)).max() <= 1e-4
    if plan[3] > 0:
        assert mpp.ws_status(ws) == 0, "a flag wait timed out"


@pytest.mark.parametrize("n,chunk", [(4, 0), (8, 0), (8, 7), (4, 16)])
def test_layer_bwd_dx_carry(mpp, n, chunk):
    # a carried-in state and its gradient: dx against the oracle with C0, and
    # dL/dP_0 bitwise as the backward to dM computes it
    B, H, T = 2, 3, 150
    say(f"[layer bwd dx carry] n={n} chunk={chunk}")
    x = _x(B, H, T, n, seed=77 + n)
    R = gen_R(B, H, T, n, seed=78)
    C = gen_R(B, H, 1, n, seed=79)[:, :, 0] * 0.5 + np.eye(n, dtype=np.float32)
    xd, Rd, Cd = dev(x), dev(R), dev(np.ascontiguousarray(C))
    P = mpp.scan_fwd_ex(xd, carry=Cd, from_x=True, n=n)
    dx, dC = mpp.scan_bwd_dx(xd, P, Rd, carry=Cd, want_dcarry=True, chunk=chunk)
    dM_ref, dC_ref = bwd_ref(build_ref(x, n), R, C0=C, want_dC0=True)
    ref = build_vjp_ref(x, dM_ref, n)
    shape = (B, H, T, n, n)
    err = rel_fro_err(host(dx).reshape(shape), ref.reshape(shape))
    say(f"  dx max {err.max():.3e}")
    assert err.max() <= BWD_TOL
    assert rel_fro_err(host(dC), dC_ref).max() <= BWD_TOL
    _, dC_m = mpp.scan_bwd_ex(xd, P, Rd, carry=Cd, want_dcarry=True, from_x=True, chunk=chunk)
    assert torch.equal(dC.view(torch.int32), dC_m.view(torch.int32))


@pytest.mark.parametrize("n", [4, 8])
def test_layer_bwd_dx_edges(mpp, n):
    # empty sequences are no-ops; one token: P_1 = M_1, so dx = build VJP of dP_1
    e = torch.zeros(2, 3, 0, n * n, device="cuda")
    assert mpp.scan_bwd_dx(e, torch.zeros(2, 3, 0, n, n, device="cuda"),
                           torch.zeros(2, 3, 0, n, n, device="cuda")).shape == e.shape
    x = _x(3, 2, 1, n, seed=15)
    R = gen_R(3, 2, 1, n, seed=16)
    xd = dev(x)
    dx = host(mpp.scan_bwd_dx(xd, mpp.scan_fwd_x(xd, n), dev(R)))
    ref = build_vjp_ref(x, R, n)
    assert rel_fro_err(dx.reshape(3, 2, 1, n, n), ref.reshape(3, 2, 1, n, n)).max() <= BWD_TOL
    # x = 0: every M_t = I and every e = 1, so dx is the build VJP at 0 of the
    # reverse cumulative sum of dL/dP
    T = 64
    z = torch.zeros(1, 2, T, n * n, device="cuda")
    R = gen_R(1, 2, T, n, seed=17)
    G = np.cumsum(R[:, :, ::-1].astype(np.float64), axis=2)[:, :, ::-1]
    dx = host(mpp.scan_bwd_dx(z, mpp.scan_fwd_x(z, n), dev(R)))
    ref = build_vjp_ref(np.zeros((1, 2, T, n * n)), G, n)
    assert rel_fro_err(dx.reshape(1, 2, T, n, n), ref.reshape(1, 2, T, n, n)).max() <= BWD_TOL


@pytest.mark.parametrize("n,chunk", [(4, 0), (8, 0), (8, 12)])
def test_bwd_reads_one_prefix_in_four(mpp, n, chunk):
    # The n <= 8 backward reads the stored prefix before each block of 4 tokens
    # (blocks counted from each chunk's end) and recomputes the rest: with every
    # other prefix replaced by NaN the results are unchanged.  Chunk lengths are
    # multiples of 4 here and T is a multiple of the chunk, so the read prefixes
    # are those at t = T-5, T-9, ... (0-based), i.e. t % 4 == 3.
    B, H, T = 2, 2, 96
    x = _x(B, H, T, n, seed=91)
    R = gen_R(B, H, T, n, seed=92)
    xd, Rd = dev(x), dev(R)
    P = mpp.scan_fwd_x(xd, n)
    poisoned = P.clone()
    keep = torch.zeros(T, dtype=torch.bool)
    keep[3::4] = True
    poisoned[:, :, ~keep] = float("nan")
    for fn in (lambda PP: mpp.scan_bwd_x(xd, PP, Rd, chunk), lambda PP: mpp.scan_bwd_dx(xd, PP, Rd, chunk=chunk)):
        a, b = fn(P), fn(poisoned)
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))


@pytest.mark.parametrize("n,chunk", [(4, 0), (8, 0), (8, 12), (16, 0), (32, 7)])
def test_bwd_from_M_uses_every_prefix_as_given(mpp, n, chunk):
    # From M the backward takes P as an input: dM_t = P_{t-1}^T Q_t reads the
    # stored P_{t-1} of every token and Q does not depend on P.  With every
    # other prefix replaced by NaN, exactly the tokens after a poisoned prefix
    # turn NaN and all others keep their bits.
    B, H, T = 2, 2, 96
    say(f"[bwd from M, P as given] n={n} chunk={chunk}")
    x = _x(B, H, T, n, seed=91)
    R = gen_R(B, H, T, n, seed=92)
    M = mpp.build_inputs(dev(x), n)
    Rd = dev(R)
    P = mpp.scan_fwd(M)
    poisoned = P.clone()
    bad = torch.zeros(T, dtype=torch.bool)
    bad[1::2] = True
    poisoned[:, :, bad] = float("nan")
    a = host(mpp.scan_bwd(M, P, Rd, chunk))
    b = host(mpp.scan_bwd(M, poisoned, Rd, chunk))
    after_bad = np.zeros(T, dtype=bool)
    after_bad[1:] = bad.numpy()[:-1]          # token t reads P_{t-1}
    assert np.isnan(b[:, :, after_bad]).all(axis=(-1, -2)).all()
    assert np.array_equal(a[:, :, ~after_bad].view(np.uint32), b[:, :, ~after_bad].view(np.uint32))


@pytest.mark.parametrize("n", [4, 8])
def test_fused_layer_autograd(mpp, n):
    # mru_layer takes the fused path for n = 4, 8: gradient down to x against the oracle
    say(f"[fused layer autograd] n={n}")
    T = 300
    x = _x(1, 2, T, n, seed=41)
    R = gen_R(1, 2, T, n, seed=42)
    xd = dev(x).requires_grad_(True)
    P = mpp.mru_layer(xd, n, chunk=37)
    (P * dev(R)).sum().backward()
    ref = build_vjp_ref(x, bwd_ref(build_ref(x, n), R), n)
    err = rel_fro_err(host(xd.grad).reshape(1, 2, T, n, n), ref.reshape(1, 2, T, n, n))
    say(f"  max rel err {err.max():.3e}")
    assert err.max() <= BWD_TOL


N16_DX_CASES = [(16, 64, 64, 24, 0), (16, 4, 4, 700, 0), (16, 2, 3, 203, 5), (16, 3, 1, 1, 0),
                (32, 32, 32, 12, 0), (32, 1, 4, 500, 0), (32, 2, 1, 301, 37), (32, 2, 1, 1, 0)]


@pytest.mark.parametrize("n,B,H,T,chunk", N16_DX_CASES)
def test_layer_bwd_dx_n16(mpp, n, B, H, T, chunk):
    # the one-pass layer backward at n = 16, 32: bit for bit the build's gradient
    # applied to the backward from x, and against the oracle's build VJP of its
    # fp64 backward
    plan = mpp.scan_plan(B, H, T, n, mpp.DIR_BWD, chunk)
    say(f"[layer bwd dx n={n}] B={B} H={H} T={T} chunk={chunk} plan(K,nch,Z,ws)={plan}")
    x = _x(B, H, T, n, seed=T + 13)
    R = gen_R(B, H, T, n, seed=T + 14)
    xd, Rd = dev(x), dev(R)
    P = mpp.scan_fwd_x(xd, n)
    dx = mpp.scan_bwd_dx(xd, P, Rd, chunk=chunk, check=True)
    two = mpp.build_inputs_bwd(xd, mpp.scan_bwd_x(xd, P, Rd, chunk))
    assert torch.equal(dx.view(torch.int32), two.view(torch.int32)), "differs from the two-kernel path"
    ref = build_vjp_ref(x, bwd_ref(build_ref(x, n), R), n)
    err = rel_fro_err(host(dx).reshape(B, H, T, n, n), ref.reshape(B, H, T, n, n))
    say(f"  max {err.max():.3e} median {np.median(err):.3e}")
    assert err.max() <= BWD_TOL


# n = 16, 32 from raw token vectors: every plan shape of the matrix-core
# forward -- one chunk per sequence (streamed), register-retained chunks (n = 16:
# auto plan, a ragged forced chunk, exactly 64 tokens), streamed chunks (longer
# than the register buffer; every n = 32 chunk), a single token
N16_CASES = [(16, 128, 16, 40, 0), (16, 4, 4, 1000, 0), (16, 2, 3, 203, 5), (16, 2, 2, 130, 64),
             (16, 2, 3, 1000, 32),
             (16, 1, 2, 300, 100), (16, 3, 1, 1, 0),
             (32, 64, 16, 12, 0), (32, 1, 4, 700, 0), (32, 2, 1, 301, 37), (32, 2, 1, 1, 0)]


@pytest.mark.parametrize("n,B,H,T,chunk", N16_CASES)
def test_fused_fwd_n16(mpp, n, B, H, T, chunk):
    plan = mpp.scan_plan(B, H, T, n, mpp.DIR_FWD_X, chunk)
    say(f"[fused fwd n={n}] B={B} H={H} T={T} chunk={chunk} plan(K,nch,Z,ws)={plan}")
    x = _x(B, H, T, n, seed=T + 7)
    xd = dev(x)
    P = mpp.scan_fwd_x(xd, n, chunk)
    again = mpp.scan_fwd_x(xd, n, chunk)
    assert torch.equal(P.view(torch.int32), again.view(torch.int32)), "not deterministic"
    err, dom, P_ref = fwd_errors(host(P), build_ref(x, n))
    say("  " + summary(err, dom))
    assert dom.all() and err.max() <= FWD_TOL
    # against build + scan on the same tokens: the matrix-core build forms each
    # token matrix with the same fp32 products, and the chain is the same, so the
    # outputs are the same bits on the same chunks (the automatic plans may
    # differ: the scan from x's chunk length is passed to the scan from M)
    kx = mpp.scan_plan(B, H, T, n, mpp.DIR_FWD_X, chunk)[0]
    P_two = mpp.scan_fwd(mpp.build_inputs(xd, n), kx)
    assert torch.equal(P.view(torch.int32), P_two.view(torch.int32)), "differs from build + scan"


# The backward from raw token vectors at n = 16, 32 over the plan shapes of the
# matrix-core backward: one chunk per sequence, automatic multi-chunk plans,
# ragged forced chunks, a single token.
N16_BWD_CASES = [(16, 64, 64, 24, 0), (16, 4, 4, 1000, 0), (16, 2, 3, 203, 5), (16, 1, 2, 300, 100),
                 (16, 3, 1, 1, 0), (32, 32, 32, 12, 0), (32, 1, 4, 700, 0), (32, 2, 1, 301, 37),
                 (32, 2, 1, 1, 0)]


@pytest.mark.parametrize("n,B,H,T,chunk", N16_BWD_CASES)
def test_fused_bwd_n16(mpp, n, B, H, T, chunk):
    plan = mpp.scan_plan(B, H, T, n, mpp.DIR_BWD, chunk)
    say(f"[fused bwd n={n}] B={B} H={H} T={T} chunk={chunk} plan(K,nch,Z,ws)={plan}")
    x = _x(B, H, T, n, seed=T + 9)
    R = gen_R(B, H, T, n, seed=T + 10)
    xd, Rd = dev(x), dev(R)
    P = mpp.scan_fwd_x(xd, n)
    ws = torch.empty(max(plan[3], 256), dtype=torch.uint8, device="cuda")
    dM = mpp.scan_bwd_x(xd, P, Rd, chunk, workspace=ws)
    if plan[3] > 0:
        assert mpp.ws_status(ws) == 0, "a flag wait timed out"
    again = mpp.scan_bwd_x(xd, P, Rd, chunk)
    assert torch.equal(dM.view(torch.int32), again.view(torch.int32)), "not deterministic"
    ref = bwd_ref(build_ref(x, n), R)
    err = rel_fro_err(host(dM), ref)
    say(f"  max {err.max():.3e} median {np.median(err):.3e}")
    assert err.max() <= BWD_TOL
    # against build then the backward from M on the same P: each M_{t+1} is
    # formed with the build's own products, so dM carries the same bits
    dM_two = mpp.scan_bwd(mpp.build_inputs(xd, n), P, Rd, chunk)
    assert torch.equal(dM.view(torch.int32), dM_two.view(torch.int32)), "differs from build + backward"


@pytest.mark.parametrize("n", [16, 32])
def test_fused_bwd_n16_zero_input(mpp, n):
    # x = 0: every M_t = I, so Q_t is the reverse cumulative sum of dL/dP and
    # dM_t = P_{t-1}^T Q_t = Q_t (P = I), exactly as the backward from M gives it
    T = 90
    xd = torch.zeros(1, 2, T, n * n, device="cuda")
    R = gen_R(1, 2, T, n, seed=5)
    P = mpp.scan_fwd_x(xd, n)
    for chunk in (0, 7):
        dM = host(mpp.scan_bwd_x(xd, P, dev(R), chunk))
        ref = np.cumsum(R[:, :, ::-1].astype(np.float64), axis=2)[:, :, ::-1]
        assert rel_fro_err(dM, ref).max() <= BWD_TOL
        eye = torch.eye(n, device="cuda").expand(1, 2, T, n, n).contiguous()
        dM_m = host(mpp.scan_bwd(eye, P, dev(R), chunk))
        assert np.array_equal(dM.view(np.uint32), dM_m.view(np.uint32))


@pytest.mark.parametrize("n,chunk", [(16, 0), (16, 9), (16, 100), (32, 0), (32, 21)])
def test_fused_fwd_n16_carry_and_scaled(mpp, n, chunk):
    # a carried-in state, and the scaled form: 2^E * P~ carries the plain scan's
    # bits (exact powers of two), both graded against the oracle
    B, H, T = 2, 2, 400
    x = _x(B, H, T, n, seed=11)
    rng = np.random.default_rng(4)
    C = (np.eye(n) + 0.1 * rng.standard_normal((B, H, n, n))).astype(np.float32)
    xd, Cd = dev(x), dev(C)
    P = host(mpp.scan_fwd_ex(xd, carry=Cd, from_x=True, n=n, chunk=chunk))
    Pm, E = mpp.scan_fwd_ex(xd, carry=Cd, scaled=True, from_x=True, n=n, chunk=chunk)
    Pm, E = host(Pm), host(E)
    assert np.array_equal(np.ldexp(Pm, E[..., None, None]).astype(np.float32), P)
    ref = scan_ref(build_ref(x, n), C.astype(np.float64))
    err = rel_fro_err(np.ldexp(Pm.astype(np.float64), E[..., None, None]), ref)
    say(f"[fused fwd n={n} carry, scaled] chunk={chunk}: max {err.max():.3e}")
    assert err.max() <= FWD_TOL
    _, E_ref = scaled_ref(ref)
    assert np.abs(E - E_ref).max() <= 1


@pytest.mark.parametrize("n", [16, 32])
def test_fused_fwd_n16_zero_input_is_identity(mpp, n):
    # x = 0: mean 0, e = 1, both factors I, so every token matrix and prefix is I exactly
    T = 150
    xd = torch.zeros(2, 2, T, n * n, device="cuda")
    for chunk in (0, 7, 100):
        P = host(mpp.scan_fwd_x(xd, n, chunk))
        assert np.array_equal(P, np.broadcast_to(np.eye(n, dtype=np.float32), P.shape))


@pytest.mark.parametrize("chunk", [8, 5])
def test_n32_fp32_apply_falls_back_past_the_range(mpp, chunk):
    """M_t = diag(2^40, 2^-40, 1, ...): within four steps the fp32 apply chain
    overflows and its chunks are redone by the fp64 pass. Every prefix is an
    exact power of two (inf / 0 once it leaves fp32; 24 tokens keep the fp64
    state finite), from M and, bitwise the same as build then scan, from raw
    token vectors."""
    n, B, H, T = 32, 2, 1, 24
    d = np.ones(n)
    d[0], d[1] = 2.0 ** 40, 2.0 ** -40
    M = np.broadcast_to(np.diag(d).astype(np.float32), (B, H, T, n, n)).copy()
    P = host(mpp.scan_fwd(dev(M), chunk))
    t1 = np.arange(1, T + 1, dtype=np.float64)
    with np.errstate(over="ignore", under="ignore"):
        want = np.broadcast_to(np.eye(n, dtype=np.float32), (B, H, T, n, n)).copy()
        want[..., 0, 0] = (2.0 ** (40 * t1)).astype(np.float32)  # inf from t = 4 on
        want[..., 1, 1] = (2.0 ** (-40 * t1)).astype(np.float32)  # 0 from t = 4 on
    assert np.array_equal(P, want)
    # the same from raw token vectors: X_00 = -X_11 = 40 ln 2, the rest 0
    x = np.zeros((B, H, T, n, n), dtype=np.float32)
    x[..., 0, 0], x[..., 1, 1] = 40 * np.log(2.0), -40 * np.log(2.0)
    xd = dev(x.reshape(B, H, T, n * n))
    Px = mpp.scan_fwd_x(xd, n, chunk)
    Pm = mpp.scan_fwd(mpp.build_inputs(xd, n), chunk)
    assert torch.equal(Px.view(torch.int32), Pm.view(torch.int32))
    Px = host(Px)
    assert np.isinf(Px[:, :, 3:, 0, 0]).all() and (Px[:, :, 3:, 1, 1] == 0).all()
