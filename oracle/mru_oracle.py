"""Plain fp64 CPU oracle for the MRU prefix-scan path.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  The product path (the
HIP library and its Python binding) never imports, calls or links it, and it
shares no code with that path: it is written from the definitions on the MRU
pages, slowly and obviously, in numpy float64.

Sources (page titles as printed; section names are the pages' own):

* "MRU Update: An independent developer's alternative to Attention is now
  running successfully" (openai-hub.net, English version of the openai-hub.com
  article), section "What MRU Actually Does": each token's vector becomes an
  input state matrix, the matrices are multiplied one after another along the
  sequence to give the output state matrix, and that matrix is turned back
  into a vector.  Each step multiplies the current state matrix by the new
  input matrix (state on the left, input on the right), and associativity of
  the matrix product is what allows a parallel scan.
* "Improving Matrix Recurrent Units as an Attention Alternative"
  (setupai.cc), Key Points: the input state matrix is built by LDU factor
  filling with a determinant-correcting scalar.

Readings taken where the pages are silent:

* The n*n entries of a token vector, viewed row-major as X, fill the strictly
  lower part of a unit lower-triangular L, the strictly upper part of a unit
  upper-triangular U, and log of a positive diagonal D (D_ii = exp X_ii).
* The determinant-correcting scalar is c = |det(L D U)|^(-1/n), so that
  det(M) = 1 for M = c L D U.
* The scan is inclusive with P_0 = I and right multiplication,
  P_t = P_{t-1} M_t; a carried-in state replaces I by a given P_0 (segment
  continuation), and the scaled form writes each P_t as 2^E times a matrix
  whose largest entry lies in [0.5, 1).
* Flattening is the row-major reshape of P_t to an n*n vector, per head.
* The orthogonal variant builds A = (X - X^T) / 2 (the skew-symmetric part of
  the row-major view) and maps it to an orthogonal matrix by the Cayley map
  or the matrix exponential.
* The backward pass is the vector-Jacobian product of L = sum_t <R_t, P_t>_F
  with respect to every M_t (the pages describe training through the product
  but give no formula; the chain rule fixes it), and build_vjp_ref carries a
  gradient dL/dM back to the raw token vectors.

Parity status: every function here is pinned by tests/test_oracle_pins.py
against closed forms, library routines, brute force, finite differences and
an independent autograd library; none is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "build_ref", "build_orthogonal_ref", "ORTHO_METHODS", "build_vjp_ref", "scan_ref", "bwd_ref", "scaled_ref", "flatten_ref", "loss_ref",
    "rel_fro_err", "representable", "FP32_DOMAIN_LIMIT",
]

# Largest |entry| of an exact P_t that the parity comparison grades; fp32
# overflows at 2^128, and 2^125 leaves room for association-order differences.
FP32_DOMAIN_LIMIT = 2.0 ** 125


def _as_matrices(x: np.ndarray, n: int) -> np.ndarray:
    x = np.asarray(x)
    if x.shape[-1] != n * n:
        raise ValueError(f"last axis must be n*n = {n * n}, got {x.shape[-1]}")
    return x.astype(np.float64).reshape(*x.shape[:-1], n, n)


def build_ref(x: np.ndarray, n: int) -> np.ndarray:
    """Input state matrices from raw token vectors (LDU fill + det correction).

    ``x``: ``[..., n*n]`` (any real dtype, promoted to float64).
    Returns ``M``: ``[..., n, n]`` float64 with ``M = c * L @ D @ U``.

    Follows "Improving Matrix Recurrent Units as an Attention Alternative",
    Key Points (LDU factor filling, determinant-correcting scalar), with the
    row-major fill described in the module docstring.  The determinant is
    taken with the library routine, not with any closed form, so that the
    det(M) = 1 pin checks the construction rather than restating it.
    """
    X = _as_matrices(x, n)
    eye = np.eye(n)
    L = np.tril(X, -1) + eye
    U = np.triu(X, 1) + eye
    D = np.diagonal(X, axis1=-2, axis2=-1)
    LDU = (L * np.exp(D)[..., None, :]) @ U          # L @ diag(exp(X_ii)) @ U
    det = np.linalg.det(LDU)
    c = np.abs(det) ** (-1.0 / n)
    return c[..., None, None] * LDU


ORTHO_METHODS = ("cayley", "expm")


def build_orthogonal_ref(x: np.ndarray, n: int, method: str) -> np.ndarray:
    """Orthogonal input state matrices from raw token vectors.

    ``x``: ``[..., n*n]``; returns float64 ``M``: ``[..., n, n]``.  With X the
    row-major n-by-n view and A = (X - X^T) / 2 its skew-symmetric part,
    ``method`` = "cayley" gives M = (I - A)^{-1} (I + A) and "expm" gives
    M = exp(A); both are orthogonal with det(M) = 1.

    Follows "Improving Matrix Recurrent Units as an Attention Alternative",
    Key Points, which names orthogonal constraints through the Cayley map and
    the matrix exponential (the variant it reports hindered learning).  How
    the n*n entries become A is not stated; the skew-symmetric part of X is
    the reading taken.  The steps use library routines: a linear solve for
    the Cayley map and scipy's scaling-and-squaring Pade exponential.
    """
    X = _as_matrices(x, n)
    A = 0.5 * (X - np.swapaxes(X, -1, -2))
    eye = np.broadcast_to(np.eye(n), A.shape)
    if method == "cayley":
        return np.linalg.solve(eye - A, eye + A)
    if method == "expm":
        from scipy.linalg import expm
        flat = A.reshape(-1, n, n)
        out = np.empty_like(flat)
        for i in range(flat.shape[0]):
            out[i] = expm(flat[i])
        return out.reshape(A.shape)
    raise ValueError(f"method must be one of {ORTHO_METHODS}")


def build_vjp_ref(x: np.ndarray, dM: np.ndarray, n: int) -> np.ndarray:
    """Gradient with respect to the raw token vector x of <dM, build_ref(x)>.

    ``x``: ``[..., n*n]``; ``dM``: ``[..., n, n]``; returns float64 ``[..., n*n]``.

    Training through the input construction ("Improving Matrix Recurrent Units
    as an Attention Alternative", Key Points: LDU fill, determinant-correcting
    scalar) needs this step; the pages give no formula, the chain rule fixes it.
    With det L = det U = 1 the scalar is c = exp(-mean_k X_kk), so
    M = L diag(e) U with e_k = exp(X_kk - mean X_jj).  For G = dM:
      through L:  G (diag(e) U)^T, kept on the strictly lower part of X;
      through U:  (L diag(e))^T G, kept on the strictly upper part;
      through e:  g_k = (L^T G U^T)_kk, and X_kk enters every e_j via the mean,
                  so dX_kk = e_k g_k - mean_j(e_j g_j).
    """
    X = _as_matrices(x, n)
    G = np.asarray(dM, dtype=np.float64)
    eye = np.eye(n)
    L = np.tril(X, -1) + eye
    U = np.triu(X, 1) + eye
    d = np.diagonal(X, axis1=-2, axis2=-1)
    e = np.exp(d - d.mean(axis=-1, keepdims=True))
    DU = e[..., :, None] * U                      # diag(e) U
    LD = L * e[..., None, :]                      # L diag(e)
    gL = G @ np.swapaxes(DU, -1, -2)
    gU = np.swapaxes(LD, -1, -2) @ G
    g = np.diagonal(np.swapaxes(L, -1, -2) @ G @ np.swapaxes(U, -1, -2), axis1=-2, axis2=-1)
    eg = e * g
    dX = np.tril(gL, -1) + np.triu(gU, 1)
    dX = dX + (eg - eg.mean(axis=-1, keepdims=True))[..., :, None] * eye
    return dX.reshape(*dX.shape[:-2], n * n)


def _initial_state(C0, batch: tuple, n: int) -> np.ndarray:
    if C0 is None:
        return np.broadcast_to(np.eye(n), batch + (n, n)).copy()    # P_0 = I
    C0 = np.asarray(C0, dtype=np.float64)
    if C0.shape != batch + (n, n):
        raise ValueError(f"C0 must have shape {batch + (n, n)}, got {C0.shape}")
    return C0.copy()


def scan_ref(M: np.ndarray, C0: np.ndarray | None = None) -> np.ndarray:
    """All prefix products P_t = P_0 M_1 M_2 ... M_t, serial, left to right.

    ``M``: ``[..., T, n, n]``; returns float64 of the same shape.  ``C0``
    (``[..., n, n]``) is the state before the first token, I when omitted;
    a sequence cut into segments is scanned by passing each segment the last
    prefix of the one before.

    Follows "MRU Update: ..." (openai-hub.net), section "What MRU Actually
    Does": cumulative multiplication along the sequence, each step being the
    current state matrix times the new input matrix.  No blocking and no
    reassociation: one matrix product per token, in token order.
    """
    M = np.asarray(M, dtype=np.float64)
    T, n = M.shape[-3], M.shape[-1]
    batch = M.shape[:-3]
    P = np.empty(M.shape, dtype=np.float64)
    state = _initial_state(C0, batch, n)
    for t in range(T):
        state = state @ M[..., t, :, :]
        P[..., t, :, :] = state
    return P


def flatten_ref(P: np.ndarray) -> np.ndarray:
    """Output state matrix back to a vector: the row-major reshape ``[..., n*n]``
    ("What MRU Actually Does", dimension reduction step)."""
    P = np.asarray(P)
    return P.reshape(*P.shape[:-2], P.shape[-1] * P.shape[-2])


def loss_ref(P: np.ndarray, R: np.ndarray) -> float:
    """L = sum over (b, h, t) of the Frobenius inner product <R_t, P_t>."""
    return float(np.sum(np.asarray(P, np.float64) * np.asarray(R, np.float64)))


def bwd_ref(M: np.ndarray, R: np.ndarray, C0: np.ndarray | None = None,
            want_dC0: bool = False):
    """Gradient dL/dM_t of L = sum_t <R_t, P_t> with P_t = P_{t-1} M_t.

    ``M``, ``R``: ``[..., T, n, n]``; returns float64 ``dM`` of the same shape,
    or ``(dM, dC0)`` with ``want_dC0``.  ``C0`` is the state P_0 before the
    first token (I when omitted), as in ``scan_ref``.

    Reverse-mode chain rule, serial from the last token to the first: with
    Q_t the total adjoint of P_t (R_t plus what flows back from P_{t+1} =
    P_t M_{t+1}), Q_T = R_T, Q_t = R_t + Q_{t+1} M_{t+1}^T, and since P_t
    depends on M_t only through P_{t-1} M_t, dL/dM_t = P_{t-1}^T Q_t.  P_1 =
    P_0 M_1 also gives dL/dP_0 = Q_1 M_1^T (zero when T = 0).  The prefixes
    come from this module's own fp64 forward.
    """
    M = np.asarray(M, dtype=np.float64)
    R = np.asarray(R, dtype=np.float64)
    if M.shape != R.shape:
        raise ValueError("M and R must have the same shape")
    T, n = M.shape[-3], M.shape[-1]
    batch = M.shape[:-3]
    P = scan_ref(M, C0)
    P0 = _initial_state(C0, batch, n)
    dM = np.empty(M.shape, dtype=np.float64)
    Q = np.zeros(batch + (n, n))
    for t in range(T - 1, -1, -1):
        if t + 1 < T:
            Q = R[..., t, :, :] + Q @ np.swapaxes(M[..., t + 1, :, :], -1, -2)
        else:
            Q = R[..., t, :, :].copy()
        P_prev = P[..., t - 1, :, :] if t > 0 else P0
        dM[..., t, :, :] = np.swapaxes(P_prev, -1, -2) @ Q
    if not want_dC0:
        return dM
    dC0 = Q @ np.swapaxes(M[..., 0, :, :], -1, -2) if T > 0 else np.zeros(batch + (n, n))
    return dM, dC0


def scaled_ref(P: np.ndarray):
    """Power-of-two form of each matrix: ``P = 2^E * Pm`` with ``E`` the frexp
    exponent of the largest |entry| (so max |Pm| lies in [0.5, 1)), and E = 0,
    Pm = 0 for a zero matrix.  ``P``: ``[..., n, n]``; returns float64 ``Pm``
    and int64 ``E`` of shape ``P.shape[:-2]``.

    The exponent side output of a scaled scan; the pages name unbounded states
    as a failure mode ("MRU Update: ...", section "The Two Fatal Issues From a
    Year Ago"), and this form keeps every P_t representable.
    """
    P = np.asarray(P, dtype=np.float64)
    big = np.abs(P).max(axis=(-1, -2))
    _, E = np.frexp(big)
    E = np.where(big > 0, E, 0).astype(np.int64)
    Pm = np.ldexp(P, -E[..., None, None])
    return Pm, E


def rel_fro_err(test: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Per-matrix relative Frobenius error ||test - ref||_F / ||ref||_F in float64.

    Reduces the last two axes.  Both matrices are divided by the reference's
    largest |entry| first (the ratio does not change), so that references far
    beyond 1e154 do not overflow the squares.  A zero reference norm gives inf
    (or nan for 0/0), which every tolerance check treats as a failure.
    """
    test = np.asarray(test, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    scale = np.abs(ref).max(axis=(-2, -1), keepdims=True)
    scale = np.where((scale > 0) & np.isfinite(scale), scale, 1.0)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        num = np.sqrt(np.sum(((test - ref) / scale) ** 2, axis=(-2, -1)))
        den = np.sqrt(np.sum((ref / scale) ** 2, axis=(-2, -1)))
        return num / den


def representable(P_ref: np.ndarray, limit: float = FP32_DOMAIN_LIMIT) -> np.ndarray:
    """Mask of matrices whose exact entries all stay within ``limit`` (fp32 parity domain)."""
    return np.max(np.abs(np.asarray(P_ref)), axis=(-2, -1)) <= limit
