"""Shared helpers for the GPU parity tests: seeded inputs, oracle references and
error statistics.  Inputs to both sides come from workloads/ (random draws) and
oracle/ (the fp64 build), never from the HIP path."""
import sys

import numpy as np
import torch

from oracle import build_ref, bwd_ref, rel_fro_err, representable, scan_ref
from workloads import WORKLOADS, gen_R, gen_x

FWD_TOL = 2e-4     # relative Frobenius error per P_t (fp32 outputs)
BWD_TOL = 5e-4     # relative Frobenius error per dM_t
BUILD_TOL = 1e-6   # relative Frobenius error per M_t (fp32 arithmetic, sums of <= n terms)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def host(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def inputs(name, T=None, B=None, H=None, b_idx=None, h_idx=None):
    """(x fp32, M32 = fp32-rounded oracle build of x, R or None) for a workload."""
    w = WORKLOADS[name]
    T = w.T if T is None else T
    B = w.B if B is None else B
    H = w.H if H is None else H
    bi = list(range(B)) if b_idx is None else b_idx
    hi = list(range(H)) if h_idx is None else h_idx
    x = gen_x(w.B, w.H, T, w.n, w.sigma_off, w.sigma_diag, w.seed, b_idx=bi, h_idx=hi)
    M32 = build_ref(x, w.n).astype(np.float32)
    R = gen_R(w.B, w.H, T, w.n, w.seed, b_idx=bi, h_idx=hi) if w.backward else None
    return x, M32, R


def random_M(shape_bhT, n, sigma_off=0.1, sigma_diag=0.05, seed=0):
    B, H, T = shape_bhT
    x = gen_x(B, H, T, n, sigma_off, sigma_diag, seed)
    return build_ref(x, n).astype(np.float32)


def fwd_errors(P_gpu, M32):
    """Errors of the GPU prefixes against the oracle on the fp32 parity domain."""
    P_ref = scan_ref(M32)
    dom = representable(P_ref)
    err = rel_fro_err(P_gpu, P_ref)
    return err, dom, P_ref


def summary(err, dom):
    e = err[dom]
    if e.size == 0:
        return "empty domain"
    return (f"max {e.max():.3e} p99.9 {np.quantile(e, 0.999):.3e} median {np.median(e):.3e} "
            f"graded {e.size} outside-domain {int((~dom).sum())}")
