"""GPU parity of the HIP path (through the C ABI) against the fp64 oracle.

Shapes here are small enough for the oracle to finish in seconds, yet span many
chunks, several supers and ragged tails; full workload sizes are in
test_parity_full_gpu.py.  Tolerances: relative Frobenius error per matrix of
2e-4 (forward) and 5e-4 (backward) on the fp32-representable domain, 1e-6 for
the LDU build; bitwise where the exact result is representable whatever the
association order (identity, Fibonacci shear, triangular zero patterns,
causality zeros).
"""
import numpy as np
import pytest
import torch

from gpu_helpers import (BUILD_TOL, BWD_TOL, FWD_TOL, dev, fwd_errors, host, random_M, say,
                         summary)
from oracle import build_ref, bwd_ref, rel_fro_err, scan_ref
from workloads import gen_R, gen_x

pytestmark = pytest.mark.gpu

SIGMA = {4: (0.1, 0.05), 8: (0.1, 0.05), 16: (0.05, 0.02), 32: (0.02, 0.01)}


@pytest.fixture(scope="module")
def mpp():
    import matrix_prefix_product_amd as m
    m.load_library()
    return m


def _M(B, H, T, n, seed=0):
    so, sd = SIGMA[n]
    return random_M((B, H, T), n, so, sd, seed)


def test_native_library_is_the_one_loaded(mpp):
    x = torch.zeros(1, 1, 2, 16, device="cuda")
    mpp.build_inputs(x, 4)
    torch.cuda.synchronize()
    maps = open("/proc/self/maps").read()
    assert mpp.library_path() in maps
    hip = {ln.split()[-1] for ln in maps.splitlines() if "libamdhip64" in ln}
    assert len(hip) == 1, hip


# ----------------------------------------------------------------------------- build

@pytest.mark.parametrize("n", [4, 8, 16, 32])
def test_build_parity(mpp, n):
    say(f"[build] n={n}")
    so, sd = SIGMA[n]
    for scale in (1.0, 5.0):
        x = gen_x(2, 3, 77, n, so * scale, sd * scale, seed=11)
        M = host(mpp.build_inputs(dev(x), n))
        err = rel_fro_err(M, build_ref(x, n))
        say(f"  scale {scale}: max rel err {err.max():.3e}")
        assert err.max() <= BUILD_TOL
    Mz = host(mpp.build_inputs(torch.zeros(1, 2, 5, n * n, device="cuda"), n))
    assert np.array_equal(Mz, np.broadcast_to(np.eye(n, dtype=np.float32), Mz.shape))


@pytest.mark.parametrize("n", [16, 32])
def test_build_matrix_core_is_correctly_rounded(mpp, n):
    # n = 16, 32 accumulate the LDU product in fp64 and round once: every entry is
    # the fp32 rounding of the oracle's fp64 build, bar entries whose exact value
    # lies within fp64 error of a rounding boundary (none expected at this size;
    # at most one ulp apart in any case)
    so, sd = SIGMA[n]
    x = gen_x(4, 4, 128, n, so, sd, seed=21)
    M = host(mpp.build_inputs(dev(x), n))
    ref32 = build_ref(x, n).astype(np.float32)
    diff = np.abs(M.view(np.int32).astype(np.int64) - ref32.view(np.int32).astype(np.int64))
    say(f"[build rounding] n={n}: entries off by one ulp {int((diff == 1).sum())} of {diff.size}")
    assert diff.max() <= 1
    assert (diff != 0).sum() <= diff.size * 1e-6


@pytest.mark.parametrize("n", [4, 8, 16, 32])
def test_build_fibonacci_exact(mpp, n):
    X = np.zeros((n, n), np.float32)
    X[0, 1] = X[1, 0] = 1.0
    x = np.broadcast_to(X.reshape(n * n), (1, 1, 3, n * n)).copy()
    M = host(mpp.build_inputs(dev(x), n))
    expect = np.eye(n, dtype=np.float32)
    expect[:2, :2] = [[1, 1], [1, 2]]
    assert np.array_equal(M[0, 0, 0], expect)


# ----------------------------------------------------------------------------- forward

FWD_CASES = [
    # (n, B, H, T, chunk)  chunk 0 = automatic plan
    (4, 1, 1, 1024, 0), (4, 3, 2, 203, 3), (4, 5, 1, 300, 300), (4, 2, 2, 97, 1),
    (8, 8, 8, 256, 0), (8, 2, 3, 203, 5), (8, 1, 2, 203, 1), (8, 33, 1, 64, 64), (8, 2, 2, 500, 16),
    (16, 1, 6, 1000, 0), (16, 2, 3, 1000, 7), (16, 3, 1, 257, 257), (16, 1, 2, 130, 1),
    (16, 2, 3, 1024, 32), (16, 1, 2, 96, 32), (16, 3, 1, 4096, 32),  # chunks dividing T
    (16, 2, 3, 1000, 64), (16, 1, 2, 128, 64),  # whole 64-token chunks (registers kept) and a ragged one
    (32, 1, 3, 600, 0), (32, 1, 2, 600, 13), (32, 2, 1, 150, 150), (32, 1, 1, 70, 1),
]


@pytest.mark.parametrize("n,B,H,T,chunk", FWD_CASES)
def test_fwd_parity(mpp, n, B, H, T, chunk):
    plan = mpp.scan_plan(B, H, T, n, mpp.DIR_FWD, chunk)
    say(f"[fwd] n={n} B={B} H={H} T={T} chunk={chunk} plan(K,nch,Z,ws)={plan}")
    M32 = _M(B, H, T, n, seed=T + n)
    ws = torch.empty(max(plan[3], 256), dtype=torch.uint8, device="cuda")
    P = host(mpp.scan_fwd(dev(M32), chunk, workspace=ws))
    err, dom, _ = fwd_errors(P, M32)
    say("  " + summary(err, dom))
    assert dom.all()
    assert err.max() <= FWD_TOL
    if plan[3] > 0:
        assert mpp.ws_status(ws) == 0, "a flag wait timed out"


@pytest.mark.parametrize("n", [4, 8, 16, 32])
@pytest.mark.parametrize("chunk", [0, 1, 4, 1000])
def test_fwd_identity_bitwise(mpp, n, chunk):
    say(f"[fwd identity] n={n} chunk={chunk}")
    M = np.broadcast_to(np.eye(n, dtype=np.float32), (2, 1, 150, n, n)).copy()
    P = host(mpp.scan_fwd(dev(M), chunk))
    assert np.array_equal(P, M)


def _fib_block(t):
    F = [0, 1]
    while len(F) < 2 * t + 2:
        F.append(F[-1] + F[-2])
    return np.array([[F[2 * t - 1], F[2 * t]], [F[2 * t], F[2 * t + 1]]], dtype=np.float64)


@pytest.mark.parametrize("n", [4, 8, 16, 32])
@pytest.mark.parametrize("chunk", [0, 1, 3, 64])
def test_fwd_fibonacci_scattered_bitwise(mpp, n, chunk):
    # 17 Fibonacci-shear tokens scattered among identity tokens over many chunks:
    # every partial product is an integer matrix below 2^24, exact in any order.
    say(f"[fwd fibonacci] n={n} chunk={chunk}")
    T = 700
    rng = np.random.default_rng(5)
    pos = np.sort(rng.choice(T, size=17, replace=False))
    F = np.eye(n, dtype=np.float32)
    F[:2, :2] = [[1, 1], [1, 2]]
    M = np.broadcast_to(np.eye(n, dtype=np.float32), (1, 2, T, n, n)).copy()
    M[:, :, pos] = F
    P = host(mpp.scan_fwd(dev(M), chunk))
    count = np.cumsum(np.isin(np.arange(T), pos))
    for t in range(T):
        expect = np.eye(n)
        if count[t] > 0:
            expect[:2, :2] = _fib_block(int(count[t]))
        assert np.array_equal(P[0, 0, t].astype(np.float64), expect), t
        assert np.array_equal(P[0, 1, t], P[0, 0, t])


@pytest.mark.parametrize("n", [4, 8, 16, 32])
def test_fwd_lower_shear_zero_pattern(mpp, n):
    say(f"[fwd lower shear] n={n}")
    T = 300
    rng = np.random.default_rng(n)
    M = np.broadcast_to(np.eye(n, dtype=np.float32), (1, 1, T, n, n)).copy()
    low = np.tril(rng.normal(0, 0.05, size=(T, n, n)), -1).astype(np.float32)
    M[0, 0] += low
    for chunk in (0, 7):
        P = host(mpp.scan_fwd(dev(M), chunk))[0, 0]
        iu = np.triu_indices(n, 1)
        assert np.all(P[:, iu[0], iu[1]] == 0.0)
        assert np.all(np.diagonal(P, axis1=1, axis2=2) == 1.0)
        err = rel_fro_err(P, scan_ref(M[0, 0]))
        assert err.max() <= FWD_TOL


@pytest.mark.parametrize("n", [4, 8, 16, 32])
def test_fwd_deterministic(mpp, n):
    say(f"[fwd determinism] n={n}")
    M = dev(_M(2, 2, 400, n, seed=3))
    for chunk in (0, 5):
        P1 = host(mpp.scan_fwd(M, chunk))
        P2 = host(mpp.scan_fwd(M, chunk))
        assert np.array_equal(P1, P2)


@pytest.mark.parametrize("n", [8, 16])
def test_fwd_chunk_invariance(mpp, n):
    # different chunkings agree with each other within twice the oracle tolerance
    say(f"[fwd chunk invariance] n={n}")
    M32 = _M(1, 2, 333, n, seed=9)
    Pref = scan_ref(M32)
    Ps = [host(mpp.scan_fwd(dev(M32), c)) for c in (1, 2, 16, 100, 333)]
    for P in Ps:
        assert rel_fro_err(P, Pref).max() <= FWD_TOL
        assert rel_fro_err(P, Ps[-1]).max() <= 2 * FWD_TOL


def test_fwd_edge_shapes(mpp):
    say("[fwd edges]")
    for n in (4, 8, 16, 32):
        P = mpp.scan_fwd(torch.empty(2, 3, 0, n, n, device="cuda"))
        assert P.shape == (2, 3, 0, n, n)
        M32 = _M(1, 1, 1, n, seed=1)
        assert np.array_equal(host(mpp.scan_fwd(dev(M32))), M32)
        M32 = _M(1, 1, 2, n, seed=2)
        P = host(mpp.scan_fwd(dev(M32), 1))
        assert rel_fro_err(P, scan_ref(M32)).max() <= FWD_TOL


def test_flatten_is_row_major_view(mpp):
    from oracle import flatten_ref
    M32 = _M(1, 2, 10, 8, seed=4)
    P = mpp.scan_fwd(dev(M32))
    v = mpp.flatten(P)
    assert v.shape == (1, 2, 10, 64) and v.data_ptr() == P.data_ptr()
    Ph, vh = host(P), host(v)
    # entry (i, j) of P_t is component i*n + j of the vector, by definition
    for i, j in ((0, 0), (0, 7), (3, 5), (7, 0), (7, 7)):
        assert np.array_equal(vh[..., i * 8 + j], Ph[..., i, j])
    # and the vectors are the oracle's flattened prefixes
    ref = flatten_ref(scan_ref(M32.astype(np.float64)))
    assert ref.shape == vh.shape
    err = np.linalg.norm(vh - ref, axis=-1) / np.linalg.norm(ref, axis=-1)
    assert err.max() <= FWD_TOL


# ----------------------------------------------------------------------------- backward

BWD_CASES = [
    (4, 1, 1, 1024, 0), (4, 3, 2, 203, 3), (4, 2, 2, 97, 1), (4, 5, 1, 120, 120),
    (8, 8, 8, 256, 0), (8, 2, 3, 203, 5), (8, 1, 2, 203, 1), (8, 33, 1, 64, 64), (8, 2, 2, 500, 16),
    (16, 1, 6, 1000, 0), (16, 2, 3, 1000, 7), (16, 3, 1, 257, 257), (16, 1, 2, 130, 1),
    (16, 2, 3, 1024, 32), (16, 1, 2, 96, 32), (16, 3, 1, 4096, 32),  # chunks dividing T
    (16, 2, 3, 1000, 64), (16, 1, 2, 128, 64),  # whole 64-token chunks (registers kept) and a ragged one
    (32, 1, 3, 600, 0), (32, 1, 2, 600, 13), (32, 2, 1, 150, 150), (32, 1, 1, 70, 1),
]


@pytest.mark.parametrize("n,B,H,T,chunk", BWD_CASES)
def test_bwd_parity(mpp, n, B, H, T, chunk):
    plan = mpp.scan_plan(B, H, T, n, mpp.DIR_BWD, chunk)
    say(f"[bwd] n={n} B={B} H={H} T={T} chunk={chunk} plan(K,nch,Z,ws)={plan}")
    M32 = _M(B, H, T, n, seed=T + 2 * n)
    R = gen_R(B, H, T, n, seed=T)
    Md = dev(M32)
    P = mpp.scan_fwd(Md)
    ws = torch.empty(max(plan[3], 256), dtype=torch.uint8, device="cuda")
    dM = host(mpp.scan_bwd(Md, P, dev(R), chunk, workspace=ws))
    ref = bwd_ref(M32, R)
    err = rel_fro_err(dM, ref)
    say(f"  max {err.max():.3e} median {np.median(err):.3e}")
    assert err.max() <= BWD_TOL
    if plan[3] > 0:
        assert mpp.ws_status(ws) == 0, "a flag wait timed out"


@pytest.mark.parametrize("n", [4, 8, 16, 32])
def test_bwd_identity_is_reverse_cumsum(mpp, n):
    say(f"[bwd identity] n={n}")
    T = 300
    M = np.broadcast_to(np.eye(n, dtype=np.float32), (1, 2, T, n, n)).copy()
    R = gen_R(1, 2, T, n, seed=7)
    expect = np.cumsum(R[:, :, ::-1].astype(np.float64), axis=2)[:, :, ::-1]
    for chunk in (0, 9):
        dM = host(mpp.scan_bwd(dev(M), dev(M), dev(R), chunk))
        assert rel_fro_err(dM, expect).max() <= BWD_TOL


@pytest.mark.parametrize("n", [4, 8, 16, 32])
def test_bwd_causality_zeros(mpp, n):
    say(f"[bwd causality] n={n}")
    T, t0 = 400, 150
    M32 = _M(1, 1, T, n, seed=12)
    R = np.zeros((1, 1, T, n, n), np.float32)
    R[0, 0, t0] = gen_R(1, 1, 1, n, seed=3)[0, 0, 0]
    Md = dev(M32)
    P = mpp.scan_fwd(Md)
    for chunk in (0, 1, 11):
        dM = host(mpp.scan_bwd(Md, P, dev(R), chunk))
        assert np.all(dM[0, 0, t0 + 1:] == 0.0)
        ref = bwd_ref(M32, R)
        assert rel_fro_err(dM[0, 0, : t0 + 1], ref[0, 0, : t0 + 1]).max() <= BWD_TOL


@pytest.mark.parametrize("n", [4, 8, 16, 32])
def test_bwd_deterministic(mpp, n):
    say(f"[bwd determinism] n={n}")
    M = dev(_M(2, 1, 400, n, seed=4))
    R = dev(gen_R(2, 1, 400, n, seed=4))
    P = mpp.scan_fwd(M)
    for chunk in (0, 6):
        a = host(mpp.scan_bwd(M, P, R, chunk))
        b = host(mpp.scan_bwd(M, P, R, chunk))
        assert np.array_equal(a, b)


def test_autograd_function(mpp):
    say("[autograd]")
    n, T = 8, 120
    M32 = _M(1, 2, T, n, seed=21)
    R = gen_R(1, 2, T, n, seed=21)
    M = dev(M32).requires_grad_(True)
    P = mpp.mru_scan(M)
    (P * dev(R)).sum().backward()
    assert rel_fro_err(host(M.grad), bwd_ref(M32, R)).max() <= BWD_TOL


def test_binding_errors(mpp):
    say("[binding errors]")
    M = torch.zeros(1, 1, 4, 8, 8, device="cuda")
    with pytest.raises(ValueError):
        mpp.scan_fwd(M.double())
    with pytest.raises(ValueError):
        mpp.scan_fwd(torch.zeros(1, 1, 4, 6, 6, device="cuda"))
    flat = torch.zeros(1 + 4 * 64, device="cuda")
    mis = flat[1:].view(1, 1, 4, 8, 8)  # contiguous but 4-byte offset
    with pytest.raises(mpp.MRUError) as e:
        mpp.scan_fwd(mis)
    assert e.value.status == 3
    with pytest.raises(mpp.MRUError) as e:
        mpp.scan_fwd(M, out=M)
    assert e.value.status == 4


# ----------------------------------------------------------------------------- build backward

from oracle import build_vjp_ref  # noqa: E402

BUILD_BWD_TOL = 2e-6  # fp32 sums of <= 2n products per entry (bound ~(2n+3) eps); measured worst 1.6e-7


@pytest.mark.parametrize("n", [4, 8, 16, 32])
def test_build_bwd_parity(mpp, n):
    say(f"[build bwd] n={n}")
    so, sd = SIGMA[n]
    for scale in (1.0, 5.0):
        x = gen_x(2, 3, 77, n, so * scale, sd * scale, seed=13)
        G = gen_R(2, 3, 77, n, seed=14)
        dx = host(mpp.build_inputs_bwd(dev(x), dev(G)))
        ref = build_vjp_ref(x, G, n)
        err = rel_fro_err(dx.reshape(*dx.shape[:-1], n, n), ref.reshape(*ref.shape[:-1], n, n))
        say(f"  scale {scale}: max rel err {err.max():.3e}")
        assert err.max() <= BUILD_BWD_TOL
        # the determinant correction makes every dx traceless
        tr = np.trace(dx.reshape(-1, n, n), axis1=1, axis2=2)
        assert np.abs(tr).max() <= 1e-5 * np.abs(dx).max()


@pytest.mark.parametrize("n", [4, 8, 16, 32])
def test_build_bwd_at_zero(mpp, n):
    G = gen_R(1, 1, 5, n, seed=n)
    dx = host(mpp.build_inputs_bwd(torch.zeros(1, 1, 5, n * n, device="cuda"), dev(G)))
    for t in range(5):
        g = G[0, 0, t].astype(np.float64)
        expect = g - np.diag(np.diag(g)) + np.diag(np.diag(g) - np.diag(g).mean())
        np.testing.assert_allclose(dx[0, 0, t].reshape(n, n), expect, rtol=0, atol=1e-6)


@pytest.mark.parametrize("n", [8, 16])
def test_layer_autograd_to_token_vectors(mpp, n):
    # gradient of sum_t <R_t, P_t> down to x through build, scan and their VJPs
    say(f"[layer autograd] n={n}")
    so, sd = SIGMA[n]
    T = 300
    x = gen_x(1, 2, T, n, so, sd, seed=31)
    R = gen_R(1, 2, T, n, seed=32)
    xd = dev(x).requires_grad_(True)
    P = mpp.mru_layer(xd, n, chunk=37)
    (P * dev(R)).sum().backward()
    M64 = build_ref(x, n)
    ref = build_vjp_ref(x, bwd_ref(M64, R), n)
    g = host(xd.grad)
    err = rel_fro_err(g.reshape(1, 2, T, n, n), ref.reshape(1, 2, T, n, n))
    say(f"  max rel err {err.max():.3e}")
    assert err.max() <= BWD_TOL


def test_ws_status_reports_the_header_word(mpp):
    """The status query returns the word a multi-chunk scan leaves in its
    workspace header (0 when every look-back wait completed), and the binding
    raises MRU_ERR_TIMEOUT when that word carries the timeout bit (set here from
    the host, as a timed-out wait would leave it)."""
    say("[ws_status] n=8 B=1 H=1 T=300 chunk=16")
    B, H, T, n, chunk = 1, 1, 300, 8, 16
    need = mpp.workspace_bytes(B, H, T, n, mpp.DIR_FWD, chunk)
    assert need > 0
    ws = torch.full((need,), 0xAB, dtype=torch.uint8, device="cuda")   # garbage before the scan
    M = dev(_M(B, H, T, n, seed=3))
    mpp.scan_fwd(M, chunk, workspace=ws, check=True)
    assert mpp.ws_status(ws) == 0
    ws[4:8].view(torch.int32).fill_(1)
    assert mpp.ws_status(ws) == 1
    with pytest.raises(mpp.MRUError) as e:
        mpp._after_scan(ws, True, "mru_scan_fwd", (B, H, T), n, mpp.DIR_FWD, chunk)
    assert e.value.status == mpp.MRU_ERR_TIMEOUT
    # no workspace (one chunk per sequence): nothing to wait on, status 0
    assert mpp.ws_status(None) == 0
