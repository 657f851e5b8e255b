"""Write the small text fixtures in this folder.

Every value stored here comes from the fp64 oracle (``oracle/``) applied to
seeded or hand-constructed inputs; nothing comes from the GPU path.  The MRU
pages print no worked numeric example, so there is no page value to store.

Run from the repository root:  python tests/golden/make_golden.py
"""
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

from oracle import build_ref, scan_ref  # noqa: E402
from workloads import WORKLOADS, gen_x  # noqa: E402


def _write(name, header, arrays):
    path = os.path.join(HERE, name)
    with open(path, "w") as f:
        for line in header.strip().splitlines():
            f.write("# " + line + "\n")
        for key, arr in arrays.items():
            arr = np.asarray(arr, dtype=np.float64)
            f.write(f"@ {key} {' '.join(str(d) for d in arr.shape)}\n")
            for v in arr.reshape(-1):
                f.write(repr(float(v)) + "\n")
    print("wrote", path)


def fibonacci(n=4, T=17):
    X = np.zeros((n, n))
    X[0, 1] = X[1, 0] = 1.0
    x = np.broadcast_to(X.reshape(n * n), (T, n * n)).astype(np.float32)
    M = build_ref(x, n)
    P = scan_ref(M)
    _write("fibonacci_n4.txt", f"""
Fibonacci shear input, n={n}, T={T}: every token vector has x[0,1] = x[1,0] = 1
and zeros elsewhere, so the LDU fill gives M = [[1,1],[1,2]] (+) I (unit lower
shear times unit upper shear, D = I, c = 1) and P_t = M^t holds Fibonacci
numbers F(2t-1), F(2t), F(2t+1), all below 2^24 for t <= 17, hence exact in
fp32 under any association order.
Method: "What MRU Actually Does" (cumulative product of per-token input state
matrices) and "Improving Matrix Recurrent Units ..." Key Points (LDU fill with
determinant-correcting scalar).  Values: oracle/ (fp64), by make_golden.py.
""", {"x": x, "M": M, "P": P})


def c1_head(T=8):
    w = WORKLOADS["c1"]
    x = gen_x(w.B, w.H, T, w.n, w.sigma_off, w.sigma_diag, w.seed)[0, 0]
    M = build_ref(x, w.n)
    P = scan_ref(M.astype(np.float32))
    _write("c1_head.txt", f"""
First {T} tokens of the n={w.n} workload (B=1,H=1, seed {w.seed}): raw x (fp32),
M = build_ref(x) in fp64, and P = scan_ref(fp32-rounded M) in fp64.
A regression fixture: it fixes the seeded generator and the oracle's output
on real-sized inputs so that later changes to either are caught.
Values: workloads/ + oracle/ (fp64), by make_golden.py.
""", {"x": x, "M": M, "P": P})


if __name__ == "__main__":
    fibonacci()
    c1_head()
