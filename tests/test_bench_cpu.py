"""Host-side checks of bench.py's contract (no GPU needed)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused():
    for args, env in ((["--gpus", "2"], {}), (["--gpus", "1"], {"WORLD_SIZE": "4"})):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                           capture_output=True, text=True, env={**os.environ, **env}, timeout=120)
        assert r.returncode == 2, r.stderr
        assert "one GPU" in r.stderr
        assert r.stdout == ""


def test_algorithmic_bytes_per_kernel():
    import bench
    S, T, n = 8192, 256, 8
    # n <= 8 backward: x (or M), dP, dM per token plus one stored prefix per 4 tokens
    per_entry = {"fwd_x": 8, "bwd_x": 13, "build": 8, "fwd": 8, "bwd": 13, "build_bwd": 12}
    for kind, b in per_entry.items():
        assert bench.algorithmic_bytes(kind, S, T, n) == b * n * n * S * T
    # one C2L forward launch moves exactly 1 GiB, the backward 1.625 GiB
    assert bench.algorithmic_bytes("fwd_x", S, T, n) == 2 ** 30
    assert bench.algorithmic_bytes("bwd_x", S, T, n) == 13 * 2 ** 27
    # the matrix-core backward (n = 16, 32) reads every prefix
    assert bench.algorithmic_bytes("bwd", 64, 1024, 16) == 16 * 256 * 64 * 1024


def test_traffic_record_is_tied_to_the_sources():
    import bench
    h = bench.source_hash()
    assert len(h) == 16 and h == bench.source_hash()
    # a record taken on other sources is ignored
    assert bench.load_traffic("c2l", "no_such_kernel") is None


def test_counted_sources_exist():
    import bench
    csrc = os.path.join(ROOT, "matrix_prefix_product_amd", "csrc")
    for f in bench.COUNTED_SOURCES:
        assert os.path.isfile(os.path.join(csrc, f)), f


def test_cpu_leg_and_parity_sample():
    import numpy as np

    import bench
    from workloads import WORKLOADS
    w = WORKLOADS["c2"].with_(T=32)
    rec, ref = bench.cpu_leg(w, 0.0, max_workers=2)
    assert rec["kind"] == "oracle" and rec["cores"] == 1 and rec["value"] > 0
    assert rec["parallel"]["cores"] >= 1 and rec["parallel"]["value"] > 0
    P, dM = ref
    assert 1 <= P.shape[0] <= bench.PARITY_ROWS and P.shape[1:] == (w.H, 32, w.n, w.n)
    assert dM.shape == P.shape
    same = bench.cpu_parity(ref, (P.astype(np.float32), dM.astype(np.float32)))
    assert same["P"]["over_bound"] == 0 and same["dM"]["over_bound"] == 0
    assert same["P"]["max"] < 1e-6
    # a wrong row is flagged
    bad = P.astype(np.float32).copy()
    bad[0, 0, 5] *= 1.01
    flagged = bench.cpu_parity(ref, (bad, dM.astype(np.float32)))
    assert flagged["P"]["over_bound"] == 1 and flagged["P"]["max"] > 5e-3
