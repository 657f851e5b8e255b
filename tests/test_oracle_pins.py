"""Pins for the fp64 oracle: each checks it against something other than itself.

The MRU pages print no worked numeric example, so every pin here comes from
mathematics the pages fix: closed forms of special inputs, library routines,
brute force on tiny inputs, invariants (det = 1 from the determinant-correcting
scalar; associativity, which the pages give as the reason a parallel scan is
possible), central finite differences and an independent autograd library.
The set is chosen so that a dropped term, a wrong sign, an index slip or a
transposed operand anywhere in the oracle fails at least one test.
"""
import itertools
import math

import numpy as np
import pytest

from oracle import build_ref, bwd_ref, flatten_ref, loss_ref, rel_fro_err, representable, scan_ref
from workloads import WORKLOADS, gen_R, gen_x

RNG = np.random.default_rng(12345)


def _x_from_matrix(X):
    X = np.asarray(X, dtype=np.float64)
    return X.reshape(*X.shape[:-2], X.shape[-1] * X.shape[-2])


def _fib(k):
    a, b = 0, 1
    for _ in range(k):
        a, b = b, a + b
    return a


# ----------------------------------------------------------------------------- build

def test_build_zero_is_identity():
    for n in (2, 4, 8, 16, 32):
        M = build_ref(np.zeros((3, n * n), np.float32), n)
        assert np.array_equal(M, np.broadcast_to(np.eye(n), (3, n, n)))


@pytest.mark.parametrize("d1,d2,u,l", [(0.3, -0.1, 0.5, -0.25), (-0.7, 0.2, -1.5, 2.0), (0.0, 0.0, 1.0, 1.0)])
def test_build_n2_closed_form(d1, d2, u, l):
    # Hand derivation: L=[[1,0],[l,1]], D=diag(e^d1,e^d2), U=[[1,u],[0,1]],
    # det(LDU)=e^(d1+d2), c=e^-(d1+d2)/2, so with p=e^((d1-d2)/2):
    # M = [[p, p u], [l p, l p u + 1/p]].
    p = math.exp((d1 - d2) / 2)
    expect = np.array([[p, p * u], [l * p, l * p * u + 1 / p]])
    M = build_ref(np.array([d1, u, l, d2]), 2)
    np.testing.assert_allclose(M, expect, rtol=1e-14, atol=1e-14)


@pytest.mark.parametrize("n", [4, 8, 16, 32])
def test_build_det_is_one(n):
    x = RNG.normal(0, 0.3, size=(64, n * n))
    M = build_ref(x, n)
    np.testing.assert_allclose(np.linalg.det(M), 1.0, rtol=0, atol=1e-12)


@pytest.mark.parametrize("n", [3, 5, 8])
def test_build_triangular_fill(n):
    # Strictly-lower entries alone give exactly L (unit lower); strictly-upper alone give U.
    X = RNG.normal(size=(n, n))
    low = np.tril(X, -1)
    up = np.triu(X, 1)
    np.testing.assert_allclose(build_ref(_x_from_matrix(low), n), low + np.eye(n), rtol=0, atol=1e-15)
    np.testing.assert_allclose(build_ref(_x_from_matrix(up), n), up + np.eye(n), rtol=0, atol=1e-15)


@pytest.mark.parametrize("n", [2, 4, 8])
def test_build_diagonal_only(n):
    d = RNG.normal(0, 0.5, size=n)
    M = build_ref(_x_from_matrix(np.diag(d)), n)
    np.testing.assert_allclose(M, np.diag(np.exp(d - d.mean())), rtol=1e-14, atol=0)


def test_build_factors_recoverable():
    # Undoing the fill with a library LU (no pivoting needed: leading minors > 0
    # for these small perturbations) recovers X: L, U from the factorisation of M/c.
    n = 6
    X = RNG.normal(0, 0.2, size=(n, n))
    M = build_ref(_x_from_matrix(X), n)
    # Doolittle LU of M written out (independent of the oracle's construction).
    A = M.copy()
    Lf = np.eye(n)
    for k in range(n):
        for i in range(k + 1, n):
            Lf[i, k] = A[i, k] / A[k, k]
            A[i, :] -= Lf[i, k] * A[k, :]
    Ud = A
    dvec = np.diag(Ud)
    Uf = Ud / dvec[:, None]
    np.testing.assert_allclose(np.tril(Lf, -1), np.tril(X, -1), atol=1e-12)
    np.testing.assert_allclose(np.triu(Uf, 1), np.triu(X, 1), atol=1e-12)
    np.testing.assert_allclose(np.log(dvec), np.diag(X) - np.diag(X).mean(), atol=1e-12)


def _rotation_x(theta, n):
    X = np.zeros((n, n))
    X[0, 0] = math.log(math.cos(theta))
    X[1, 1] = -math.log(math.cos(theta))
    X[0, 1] = -math.tan(theta)
    X[1, 0] = math.tan(theta)
    return _x_from_matrix(X)


def _rot(phi, n):
    R = np.eye(n)
    R[0, 0] = R[1, 1] = math.cos(phi)
    R[0, 1] = -math.sin(phi)
    R[1, 0] = math.sin(phi)
    return R


@pytest.mark.parametrize("n", [2, 4, 32])
def test_build_rotation(n):
    theta = 0.37
    M = build_ref(_rotation_x(theta, n), n)
    np.testing.assert_allclose(M, _rot(theta, n), atol=1e-15)


# ----------------------------------------------------------------------------- forward scan

def test_scan_identity():
    M = np.broadcast_to(np.eye(5), (2, 7, 5, 5))
    assert np.array_equal(scan_ref(M), M)


def test_scan_order_noncommuting():
    # M_1 lower shear, M_2 upper shear: P_2 = M_1 M_2 = [[1, b], [a, ab + 1]]
    # (M_2 M_1 would be [[1 + ab, b], [a, 1]]).
    a, b = 0.75, -2.0
    M = np.array([[[1, 0], [a, 1]], [[1, b], [0, 1]]], dtype=np.float64)
    P = scan_ref(M)
    np.testing.assert_array_equal(P[0], M[0])
    np.testing.assert_array_equal(P[1], np.array([[1, b], [a, a * b + 1]]))


@pytest.mark.parametrize("n", [2, 4])
def test_scan_fibonacci(n):
    # x[0,1] = x[1,0] = 1 gives M = [[1,1],[1,2]] (+) I, whose t-th power is
    # [[F(2t-1), F(2t)], [F(2t), F(2t+1)]] (+) I.
    X = np.zeros((n, n))
    X[0, 1] = X[1, 0] = 1.0
    M1 = build_ref(_x_from_matrix(X), n)
    T = 30
    P = scan_ref(np.broadcast_to(M1, (T, n, n)))
    for t in range(1, T + 1):
        expect = np.eye(n)
        expect[:2, :2] = [[_fib(2 * t - 1), _fib(2 * t)], [_fib(2 * t), _fib(2 * t + 1)]]
        assert np.array_equal(P[t - 1], expect), t


def test_scan_rotation_long():
    n, theta, T = 4, 0.013, 1000
    M = build_ref(np.broadcast_to(_rotation_x(theta, n), (T, n * n)), n)
    P = scan_ref(M)
    for t in (1, 10, 500, 1000):
        np.testing.assert_allclose(P[t - 1], _rot(t * theta, n), atol=1e-12)


def test_scan_diagonal_closed_form():
    n, T = 6, 50
    d = RNG.normal(0, 0.1, size=(T, n))
    x = np.stack([_x_from_matrix(np.diag(row)) for row in d])
    P = scan_ref(build_ref(x, n))
    cum = np.cumsum(d - d.mean(axis=1, keepdims=True), axis=0)
    for t in range(T):
        np.testing.assert_allclose(P[t], np.diag(np.exp(cum[t])), rtol=1e-13, atol=1e-15)


def test_scan_lower_shear_only():
    n, T = 2, 40
    lows = RNG.normal(size=T)
    M = np.broadcast_to(np.eye(2), (T, 2, 2)).copy()
    M[:, 1, 0] = lows
    P = scan_ref(M)
    np.testing.assert_array_equal(P[:, 0, 1], 0.0)
    np.testing.assert_array_equal(P[:, 0, 0], 1.0)
    np.testing.assert_array_equal(P[:, 1, 1], 1.0)
    np.testing.assert_allclose(P[:, 1, 0], np.cumsum(lows), rtol=1e-14, atol=1e-14)


def test_scan_constant_is_matrix_power():
    n, T = 5, 25
    A = build_ref(RNG.normal(0, 0.2, size=n * n), n)
    P = scan_ref(np.broadcast_to(A, (T, n, n)))
    for t in range(1, T + 1):
        np.testing.assert_allclose(P[t - 1], np.linalg.matrix_power(A, t), rtol=1e-12, atol=1e-13)


def test_scan_bruteforce_multidot_and_loops():
    n, T = 3, 6
    M = RNG.normal(size=(T, n, n))
    P = scan_ref(M)
    for t in range(1, T + 1):
        np.testing.assert_allclose(P[t - 1], np.linalg.multi_dot(list(M[:t])) if t > 1 else M[0],
                                   rtol=1e-13, atol=1e-13)
    # scalar triple loop, no library product at all
    cur = [[1.0 if i == j else 0.0 for j in range(n)] for i in range(n)]
    for t in range(T):
        cur = [[sum(cur[i][k] * M[t, k, j] for k in range(n)) for j in range(n)] for i in range(n)]
        np.testing.assert_allclose(P[t], np.array(cur), rtol=1e-13, atol=1e-13)


def _all_parenthesizations(mats):
    if len(mats) == 1:
        yield mats[0]
        return
    for split in range(1, len(mats)):
        for left in _all_parenthesizations(mats[:split]):
            for right in _all_parenthesizations(mats[split:]):
                yield left @ right


def test_scan_associativity_all_trees():
    n, T = 4, 7
    M = build_ref(RNG.normal(0, 0.3, size=(T, n * n)), n)
    P = scan_ref(M)
    for t in range(1, T + 1):
        trees = list(_all_parenthesizations(list(M[:t])))
        assert len(trees) == math.comb(2 * (t - 1), t - 1) // t     # Catalan(t-1)
        for Y in trees:
            np.testing.assert_allclose(Y, P[t - 1], rtol=1e-13, atol=1e-13)
    # every chunk split carry * local-prefix
    for k in range(1, T):
        carry = P[k - 1]
        local = scan_ref(M[k:])
        np.testing.assert_allclose(carry @ local, P[k:], rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("n", [4, 8])
def test_scan_det_one(n):
    w = WORKLOADS["c2"]
    x = gen_x(1, 1, 256, n, w.sigma_off, w.sigma_diag, seed=77)
    P = scan_ref(build_ref(x[0, 0], n))
    # det(P_t) = 1 exactly; the library determinant of an fp64 P_t is only good
    # to about n * eps * cond(P_t), which grows with t.
    bound = 8 * n * np.finfo(np.float64).eps * np.linalg.cond(P)
    assert np.all(np.abs(np.linalg.det(P) - 1.0) <= np.maximum(bound, 1e-13))
    assert np.all(np.abs(np.linalg.det(P) - 1.0) <= 1e-6)


def test_flatten_row_major():
    P = RNG.normal(size=(2, 3, 4, 4))
    v = flatten_ref(P)
    assert v.shape == (2, 3, 16)
    for i in range(4):
        for j in range(4):
            assert np.array_equal(v[..., 4 * i + j], P[..., i, j])


# ----------------------------------------------------------------------------- backward

def _loss(M, R):
    return loss_ref(scan_ref(M), R)


@pytest.mark.parametrize("n,T", [(2, 5), (3, 4), (4, 6)])
def test_bwd_finite_differences(n, T):
    M = build_ref(RNG.normal(0, 0.3, size=(T, n * n)), n)
    R = RNG.normal(size=(T, n, n))
    g = bwd_ref(M, R)
    h = 1e-6
    fd = np.empty_like(M)
    for idx in np.ndindex(M.shape):
        Mp = M.copy(); Mp[idx] += h
        Mm = M.copy(); Mm[idx] -= h
        fd[idx] = (_loss(Mp, R) - _loss(Mm, R)) / (2 * h)
    np.testing.assert_allclose(g, fd, rtol=0, atol=1e-8)


def test_bwd_quadratic_sum():
    # dM_s = sum_{t >= s} P_{s-1}^T R_t (M_{s+1} ... M_t)^T, written with products
    # of the raw inputs only (no recurrence, no prefix reuse).
    n, T = 3, 7
    M = RNG.normal(0, 0.5, size=(T, n, n))
    R = RNG.normal(size=(T, n, n))
    g = bwd_ref(M, R)
    for s in range(T):
        Pprev = np.eye(n)
        for j in range(s):
            Pprev = Pprev @ M[j]
        acc = np.zeros((n, n))
        for t in range(s, T):
            S = np.eye(n)
            for j in range(s + 1, t + 1):
                S = S @ M[j]
            acc += Pprev.T @ R[t] @ S.T
        np.testing.assert_allclose(g[s], acc, rtol=1e-12, atol=1e-12)


def test_bwd_torch_autograd():
    torch = pytest.importorskip("torch")
    n, T = 4, 9
    M = build_ref(RNG.normal(0, 0.3, size=(2, T, n * n)), n)
    R = RNG.normal(size=(2, T, n, n))
    Mt = torch.tensor(M, dtype=torch.float64, requires_grad=True)
    Rt = torch.tensor(R, dtype=torch.float64)
    state = torch.eye(n, dtype=torch.float64).expand(2, n, n)
    loss = torch.zeros((), dtype=torch.float64)
    for t in range(T):
        state = torch.matmul(state, Mt[:, t])
        loss = loss + (state * Rt[:, t]).sum()
    loss.backward()
    np.testing.assert_allclose(bwd_ref(M, R), Mt.grad.numpy(), rtol=1e-12, atol=1e-12)


def test_bwd_identity_inputs_reverse_cumsum():
    n, T = 4, 20
    M = np.broadcast_to(np.eye(n), (T, n, n))
    R = RNG.normal(size=(T, n, n))
    expect = np.cumsum(R[::-1], axis=0)[::-1]
    np.testing.assert_allclose(bwd_ref(M, R), expect, rtol=1e-13, atol=1e-13)


def test_bwd_causality():
    n, T, t0 = 4, 12, 5
    M = build_ref(RNG.normal(0, 0.3, size=(T, n * n)), n)
    R = np.zeros((T, n, n))
    R[t0] = RNG.normal(size=(n, n))
    g = bwd_ref(M, R)
    assert np.all(g[t0 + 1:] == 0.0)
    assert np.all(np.abs(g[: t0 + 1]).sum(axis=(1, 2)) > 0)


# ----------------------------------------------------------------------------- metrics, inputs

def test_rel_fro_err_and_domain():
    ref = np.ones((2, 3, 3))
    test = ref.copy()
    test[1, 0, 0] += 3.0       # ||diff|| = 3, ||ref|| = 3
    np.testing.assert_allclose(rel_fro_err(test, ref), [0.0, 1.0])
    # the same ratios for references far beyond the range where squares overflow
    np.testing.assert_allclose(rel_fro_err(test * 1e300, ref * 1e300), [0.0, 1.0])
    np.testing.assert_allclose(rel_fro_err(test * 1e-300, ref * 1e-300), [0.0, 1.0])
    assert np.isinf(rel_fro_err(np.ones((2, 2)), np.zeros((2, 2))))
    big = np.full((2, 2), 2.0 ** 126)
    assert list(representable(np.stack([np.eye(2), big]))) == [True, False]


def test_workload_generators():
    x1 = gen_x(2, 3, 40, 4, 0.1, 0.05, seed=9)
    x2 = gen_x(2, 3, 40, 4, 0.1, 0.05, seed=9)
    assert x1.dtype == np.float32 and x1.shape == (2, 3, 40, 16)
    assert np.array_equal(x1, x2)
    # prefix property and subset property
    assert np.array_equal(gen_x(2, 3, 17, 4, 0.1, 0.05, seed=9), x1[:, :, :17])
    assert np.array_equal(gen_x(2, 3, 40, 4, 0.1, 0.05, seed=9, b_idx=[1], h_idx=[2])[0, 0], x1[1, 2])
    # scales: diagonal std sigma_diag, off-diagonal std sigma_off
    big = gen_x(1, 1, 20000, 4, 0.1, 0.05, seed=3).reshape(-1, 4, 4).astype(np.float64)
    diag = np.diagonal(big, axis1=1, axis2=2)
    off = big[:, ~np.eye(4, dtype=bool)]
    assert abs(diag.std() - 0.05) < 0.002 and abs(off.std() - 0.1) < 0.002
    R = gen_R(1, 2, 5, 4, seed=9)
    assert R.shape == (1, 2, 5, 4, 4) and R.dtype == np.float32
    assert not np.array_equal(R[0, 0], R[0, 1])


# ----------------------------------------------------------------------------- golden fixtures

def test_golden_fibonacci_matches_closed_form_and_oracle():
    from golden_io import load_golden
    g = load_golden("fibonacci_n4.txt")
    T, n = g["P"].shape[0], g["P"].shape[-1]
    for t in range(1, T + 1):
        expect = np.eye(n)
        expect[:2, :2] = [[_fib(2 * t - 1), _fib(2 * t)], [_fib(2 * t), _fib(2 * t + 1)]]
        assert np.array_equal(g["P"][t - 1], expect)
    assert np.array_equal(scan_ref(build_ref(g["x"], n)), g["P"])


def test_golden_c1_head_regression():
    from golden_io import load_golden
    g = load_golden("c1_head.txt")
    w = WORKLOADS["c1"]
    T = g["x"].shape[0]
    x = gen_x(w.B, w.H, T, w.n, w.sigma_off, w.sigma_diag, w.seed)[0, 0]
    assert np.array_equal(x.astype(np.float64), g["x"])
    np.testing.assert_allclose(build_ref(x, w.n), g["M"], rtol=1e-15, atol=1e-15)
    np.testing.assert_allclose(scan_ref(g["M"].astype(np.float32)), g["P"], rtol=1e-15, atol=1e-15)


# ----------------------------------------------------------------------------- build backward

from oracle import build_vjp_ref  # noqa: E402


@pytest.mark.parametrize("n", [2, 3, 4])
def test_build_vjp_finite_differences(n):
    x = RNG.normal(0, 0.4, size=(3, n * n))
    G = RNG.normal(size=(3, n, n))
    g = build_vjp_ref(x, G, n)
    h = 1e-6
    fd = np.empty_like(x)
    for idx in np.ndindex(x.shape):
        xp = x.copy(); xp[idx] += h
        xm = x.copy(); xm[idx] -= h
        fd[idx] = (np.sum(G * build_ref(xp, n)) - np.sum(G * build_ref(xm, n))) / (2 * h)
    np.testing.assert_allclose(g, fd, rtol=0, atol=2e-8)


def test_build_vjp_torch_autograd():
    # an independent torch implementation of the construction, determinant included
    torch = pytest.importorskip("torch")
    n = 5
    x = RNG.normal(0, 0.3, size=(4, n * n))
    G = RNG.normal(size=(4, n, n))
    xt = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    X = xt.reshape(4, n, n)
    eye = torch.eye(n, dtype=torch.float64)
    L = torch.tril(X, -1) + eye
    U = torch.triu(X, 1) + eye
    D = torch.diag_embed(torch.exp(torch.diagonal(X, dim1=-2, dim2=-1)))
    LDU = L @ D @ U
    c = torch.abs(torch.linalg.det(LDU)) ** (-1.0 / n)
    M = c[:, None, None] * LDU
    (M * torch.tensor(G)).sum().backward()
    np.testing.assert_allclose(build_vjp_ref(x, G, n), xt.grad.numpy(), rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("n", [4, 8])
def test_build_vjp_at_zero_closed_form(n):
    # X = 0: L = U = I, e = 1, so dX = offdiag(G) + diag(G_kk - mean G_jj)
    G = RNG.normal(size=(n, n))
    dx = build_vjp_ref(np.zeros(n * n), G, n).reshape(n, n)
    expect = G - np.diag(np.diag(G)) + np.diag(np.diag(G) - np.diag(G).mean())
    np.testing.assert_allclose(dx, expect, rtol=0, atol=1e-15)
    assert abs(np.trace(dx)) < 1e-14       # the det correction removes the trace direction


def test_training_gradient_chain():
    # d/dx of sum_t <R_t, P_t(build(x))> by finite differences = build_vjp(bwd_ref)
    n, T = 3, 4
    x = RNG.normal(0, 0.3, size=(T, n * n))
    R = RNG.normal(size=(T, n, n))
    g = build_vjp_ref(x, bwd_ref(build_ref(x, n), R), n)
    h = 1e-6
    fd = np.empty_like(x)
    for idx in np.ndindex(x.shape):
        xp = x.copy(); xp[idx] += h
        xm = x.copy(); xm[idx] -= h
        fd[idx] = (loss_ref(scan_ref(build_ref(xp, n)), R) - loss_ref(scan_ref(build_ref(xm, n)), R)) / (2 * h)
    np.testing.assert_allclose(g, fd, rtol=0, atol=5e-8)


# ----------------------------------------------------------------------------- carried-in state, scaled form

from oracle import scaled_ref  # noqa: E402


def test_scan_carry_brute_force_multidot():
    # P_t = C0 M_1 ... M_t as one library product per t (no recurrence)
    n, T = 3, 6
    M = RNG.normal(0, 0.6, size=(T, n, n))
    C0 = RNG.normal(size=(n, n))
    P = scan_ref(M, C0)
    for t in range(T):
        np.testing.assert_allclose(P[t], np.linalg.multi_dot([C0, *M[: t + 1]]), rtol=1e-12,
                                   atol=1e-12)
    # carry on the left, not the right: the two differ for non-commuting inputs
    assert not np.allclose(P[0], M[0] @ C0)


def test_scan_carry_segments_continue():
    n, T, k = 4, 30, 11
    M = build_ref(RNG.normal(0, 0.3, size=(2, T, n * n)), n)
    whole = scan_ref(M)
    head = scan_ref(M[:, :k])
    tail = scan_ref(M[:, k:], C0=head[:, -1])
    np.testing.assert_allclose(np.concatenate([head, tail], axis=1), whole, rtol=1e-12, atol=1e-12)
    # the identity carry is the plain scan, bit for bit
    assert np.array_equal(scan_ref(M, np.broadcast_to(np.eye(n), (2, n, n))), whole)


def _loss_c(M, R, C0):
    return loss_ref(scan_ref(M, C0), R)


def test_bwd_carry_finite_differences():
    n, T = 3, 5
    M = build_ref(RNG.normal(0, 0.3, size=(T, n * n)), n)
    R = RNG.normal(size=(T, n, n))
    C0 = RNG.normal(size=(n, n))
    dM, dC0 = bwd_ref(M, R, C0, want_dC0=True)
    h = 1e-6
    fdC = np.empty_like(C0)
    for idx in np.ndindex(C0.shape):
        Cp = C0.copy(); Cp[idx] += h
        Cm = C0.copy(); Cm[idx] -= h
        fdC[idx] = (_loss_c(M, R, Cp) - _loss_c(M, R, Cm)) / (2 * h)
    np.testing.assert_allclose(dC0, fdC, rtol=0, atol=1e-8)
    fdM = np.empty_like(M)
    for idx in np.ndindex(M.shape):
        Mp = M.copy(); Mp[idx] += h
        Mm = M.copy(); Mm[idx] -= h
        fdM[idx] = (_loss_c(Mp, R, C0) - _loss_c(Mm, R, C0)) / (2 * h)
    np.testing.assert_allclose(dM, fdM, rtol=0, atol=1e-8)


def test_bwd_carry_explicit_sum_and_torch():
    # dC0 = sum_t R_t (M_1 ... M_t)^T, products of the raw inputs only
    n, T = 4, 7
    M = RNG.normal(0, 0.5, size=(2, T, n, n))
    R = RNG.normal(size=(2, T, n, n))
    C0 = RNG.normal(size=(2, n, n))
    _, dC0 = bwd_ref(M, R, C0, want_dC0=True)
    for b in range(2):
        acc = np.zeros((n, n))
        for t in range(T):
            acc += R[b, t] @ np.linalg.multi_dot([np.eye(n), *M[b, : t + 1]]).T
        np.testing.assert_allclose(dC0[b], acc, rtol=1e-12, atol=1e-12)
    torch = pytest.importorskip("torch")
    Ct = torch.tensor(C0, dtype=torch.float64, requires_grad=True)
    Mt = torch.tensor(M, dtype=torch.float64, requires_grad=True)
    state, loss = Ct, torch.zeros((), dtype=torch.float64)
    for t in range(T):
        state = torch.matmul(state, Mt[:, t])
        loss = loss + (state * torch.tensor(R[:, t])).sum()
    loss.backward()
    dM, dC0 = bwd_ref(M, R, C0, want_dC0=True)
    np.testing.assert_allclose(dC0, Ct.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dM, Mt.grad.numpy(), rtol=1e-12, atol=1e-12)
    # no tokens: no gradient
    _, dz = bwd_ref(M[:, :0], R[:, :0], C0, want_dC0=True)
    assert np.array_equal(dz, np.zeros_like(C0))


def test_scaled_ref_values():
    P = np.array([[[3.0, -0.25], [0.0, 1.0]], [[0.0, 0.0], [0.0, 0.0]],
                  [[1e200, 1.0], [-2e199, 0.0]], [[-0.5, 0.125], [0.25, 0.0]]])
    Pm, E = scaled_ref(P)
    # 3 = 0.75 * 2^2; a zero matrix stays 0 with exponent 0; -0.5 = -0.5 * 2^0
    assert E[0] == 2 and np.array_equal(Pm[0], P[0] / 4)
    assert E[1] == 0 and np.array_equal(Pm[1], P[1])
    assert E[2] == math.frexp(1e200)[1] and E[3] == 0
    for k in range(4):
        assert np.array_equal(np.ldexp(Pm[k], int(E[k])), P[k])       # exact
        big = np.abs(Pm[k]).max()
        assert big == 0 or 0.5 <= big < 1.0


# ----------------------------------------------------------------------------- orthogonal inputs

from oracle import ORTHO_METHODS, build_orthogonal_ref  # noqa: E402


def test_orthogonal_two_by_two_closed_forms():
    # n = 2: A = [[0, a], [-a, 0]] with a = (x01 - x10) / 2; the diagonal of X is ignored
    for x01, x10, d in [(0.3, -0.1, 0.7), (-1.2, 0.4, -2.0), (2.5, 2.5, 0.0)]:
        x = np.array([d, x01, x10, -d])
        a = (x01 - x10) / 2
        E = build_orthogonal_ref(x, 2, "expm")
        np.testing.assert_allclose(E, [[math.cos(a), math.sin(a)], [-math.sin(a), math.cos(a)]],
                                   rtol=0, atol=1e-14)
        C = build_orthogonal_ref(x, 2, "cayley")
        q = 1 + a * a
        np.testing.assert_allclose(C, [[(1 - a * a) / q, 2 * a / q], [-2 * a / q, (1 - a * a) / q]],
                                   rtol=0, atol=1e-14)


@pytest.mark.parametrize("method", ORTHO_METHODS)
@pytest.mark.parametrize("n", [4, 8, 16, 32])
def test_orthogonal_is_orthogonal_with_det_one(method, n):
    x = RNG.normal(0, 0.4, size=(5, n * n))
    M = build_orthogonal_ref(x, n, method)
    I = np.broadcast_to(np.eye(n), M.shape)
    np.testing.assert_allclose(np.swapaxes(M, -1, -2) @ M, I, rtol=0, atol=1e-12)
    np.testing.assert_allclose(np.linalg.det(M), 1.0, rtol=0, atol=1e-11)
    # symmetric X gives A = 0 and M = I; negating A transposes M
    xs = RNG.normal(size=(n, n)); xs = (xs + xs.T).reshape(-1)
    np.testing.assert_allclose(build_orthogonal_ref(xs, n, method), np.eye(n), rtol=0, atol=1e-14)
    Xm = x.reshape(5, n, n)
    np.testing.assert_allclose(build_orthogonal_ref(np.swapaxes(Xm, -1, -2).reshape(5, -1), n, method),
                               np.swapaxes(M, -1, -2), rtol=0, atol=1e-12)


def test_orthogonal_methods_against_series_and_each_other():
    # exp(A) against a plain truncated Taylor series; the Cayley map of the
    # generator of a plane rotation, a times [[0, 1], [-1, 0]], rotates that
    # plane by 2 atan(a) and leaves the rest fixed
    n = 6
    x = RNG.normal(0, 0.2, size=(n * n,))
    X = x.reshape(n, n)
    A = (X - X.T) / 2
    series, term = np.eye(n), np.eye(n)
    for k in range(1, 30):
        term = term @ A / k
        series = series + term
    np.testing.assert_allclose(build_orthogonal_ref(x, n, "expm"), series, rtol=0, atol=1e-14)
    a = 0.37
    x2 = np.zeros((4, 4)); x2[1, 2] = 2 * a     # A = rotation generator in plane (1, 2)
    C = build_orthogonal_ref(x2.reshape(-1), 4, "cayley")
    th = 2 * math.atan(a)
    assert abs(C[1, 1] - math.cos(th)) < 1e-14 and abs(C[1, 2] - math.sin(th)) < 1e-14
    assert np.allclose(C[[0, 3]][:, [0, 3]], np.eye(2), atol=1e-15)


def test_orthogonal_scan_keeps_the_norm():
    n, T = 8, 500
    x = RNG.normal(0, 0.3, size=(T, n * n))
    for method in ORTHO_METHODS:
        P = scan_ref(build_orthogonal_ref(x, n, method))
        np.testing.assert_allclose(np.linalg.norm(P, axis=(-1, -2)), math.sqrt(n), rtol=1e-11)
