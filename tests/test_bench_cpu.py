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
    # the definition's bytes per entry and token-head: the backward reads x (or M),
    # P and dP and writes dM (or dx)
    per_entry = {"fwd_x": 8, "bwd_x": 16, "build": 8, "fwd": 8, "bwd": 16, "build_bwd": 12,
                 "bwd_dx": 16}
    for kind, b in per_entry.items():
        assert bench.algorithmic_bytes(kind, S, T, n) == b * n * n * S * T
    # one C2L forward launch moves exactly 1 GiB, the backward 2 GiB
    assert bench.algorithmic_bytes("fwd_x", S, T, n) == 2 ** 30
    assert bench.algorithmic_bytes("bwd_x", S, T, n) == 2 ** 31
    # by design the n <= 8 backwards from x read one stored prefix per 4 tokens
    assert bench.design_bytes("bwd_x", S, T, n) == 13 * 2 ** 27
    assert bench.design_bytes("bwd_dx", S, T, n) == 13 * 2 ** 27
    assert bench.design_bytes("bwd", S, T, n) == 2 ** 31
    # the matrix-core backward (n = 16, 32) reads every prefix
    assert bench.design_bytes("bwd_x", 64, 1024, 16) == 16 * 256 * 64 * 1024


def test_cpu_model_is_named():
    import bench
    assert isinstance(bench.cpu_model(), str) and bench.cpu_model()


def test_traffic_record_is_tied_to_the_sources():
    import bench
    h = bench.source_hash()
    assert len(h) == 16 and h == bench.source_hash()
    # a record taken on other sources is ignored
    assert bench.load_traffic("c2l", "no_such_kernel") is None
    assert bench.load_mfma_util("c3", "no_such_kernel") is None


def test_kernel_kinds():
    import bench
    name = ("void mru::(anonymous namespace)::fwd_mfma_kernel<16, 16, 64, true, false>(float const*, "
            "float*, long, long, long, long, long, unsigned char*, mru::ScanCarry)")
    short = bench.short_kernel(name)
    assert short == "fwd_mfma_kernel<16, 16, 64, true, false>"
    kinds = {
        short: "fwd_x",
        "fwd_mfma_kernel<32, 4, 0, false, true>": "fwd_scaled",
        "fwd_valu_kernel<8, 1, 4, false, false>": "fwd",
        "bwd_valu_kernel<8, 1, 4, true, false>": "bwd_x",
        "bwd_mfma_kernel<16, 2, true, true, 0>": "bwd_dx",
        "bwd_mfma_kernel<16, 4, true, false, 0>": "bwd_x",
        "bwd_mfma_kernel<16, 4, false, false, 64>": "bwd",
        "bwd_valu_kernel<8, 1, 4, true, true>": "bwd_dx",
        "build_mfma_kernel<32>": "build",
        "build_kernel<8, 1>": "build",
        "build_bwd_mfma_kernel<16>": "build_bwd",
        "__amd_rocclr_copyBuffer": "copy",
        "at::native::vectorized_elementwise_kernel<4, at::native::FillFunctor<float>": None,
    }
    for k, v in kinds.items():
        assert bench.kernel_kind(k) == v, k


def test_counter_summary(tmp_path, capsys):
    """The summarizer's arithmetic on a hand-made counter file."""
    import json as js

    import bench
    d = tmp_path / "run"
    d.mkdir()
    hdr = ('"Correlation_Id","Dispatch_Id","Agent_Id","Queue_Id","Process_Id","Thread_Id","Grid_Size",'
           '"Kernel_Id","Kernel_Name","Workgroup_Size","LDS_Block_Size","Scratch_Size","VGPR_Count",'
           '"Accum_VGPR_Count","SGPR_Count","Counter_Name","Counter_Value","Start_Timestamp","End_Timestamp"')
    k = '"void mru::(anonymous namespace)::bwd_mfma_kernel<16, 8, false, false, 0>(float const*)"'
    rows = [hdr]
    for disp, (busy, grbm) in enumerate(((1024e6, 8e6), (512e6, 8e6), (768e6, 8e6)), 1):
        for c, v in (("SQ_VALU_MFMA_BUSY_CYCLES", busy), ("GRBM_GUI_ACTIVE", grbm), ("SQ_INSTS_VALU", busy / 16)):
            rows.append(f'{disp},{disp},"Agent 1",1,1,1,262144,7,{k},64,0,0,256,80,32,"{c}",{v},0,2000000')
    (d / "run_counter_collection.csv").write_text("\n".join(rows) + "\n")
    saved = bench.MFMA_FILE
    bench.MFMA_FILE = str(tmp_path / "mfma.json")
    try:
        bench.summarize("mfma", [str(d)], "c5", ["cmd"])
        rec = js.load(open(bench.MFMA_FILE))["workloads"]["c5"]
        r = rec["kernels"]["bwd"]
        # median busy 768e6 over 1e6 cycles per XCD x 1024 SIMDs
        assert r["mfma_busy"] == round(768e6 / (1e6 * 1024), 4)
        assert r["valu_busy"] == round(4 * 48e6 / (1e6 * 1024), 4)
        assert r["clock_GHz"] == round(1e6 / 2e-3 / 1e9, 3)
        # the 2 ms dispatches at 2.4 GHz
        assert r["mfma_busy_clk"] == round(768e6 / (2e-3 * 2.4e9 * 1024), 4)
        assert rec["source_hash"] == bench.source_hash()
        assert bench._record(bench.MFMA_FILE, "c5", "bwd")["grid"] == 262144
    finally:
        bench.MFMA_FILE = saved
    assert "bwd_mfma_kernel<16, 8, false, false, 0>" in capsys.readouterr().out


def test_counters_summary_per_step(tmp_path, capsys):
    """--summarize counters: medians per dispatch, and per wave-token step for the
    step kernels' grid."""
    import bench
    d = tmp_path / "run"
    d.mkdir()
    hdr = ('"Correlation_Id","Dispatch_Id","Agent_Id","Queue_Id","Process_Id","Thread_Id","Grid_Size",'
           '"Kernel_Id","Kernel_Name","Workgroup_Size","LDS_Block_Size","Scratch_Size","VGPR_Count",'
           '"Accum_VGPR_Count","SGPR_Count","Counter_Name","Counter_Value","Start_Timestamp","End_Timestamp"')
    k = '"void mru::(anonymous namespace)::bwd_valu_kernel<8, 1, 4, true, false>(float const*)"'
    steps = 1024 * 256
    rows = [hdr]
    for disp, lds in enumerate((60.0, 62.5, 70.0), 1):
        rows.append(f'{disp},{disp},"Agent 1",1,1,1,65536,7,{k},64,0,0,238,0,32,"SQ_INSTS_LDS",{lds * steps},0,350000')
    (d / "run_counter_collection.csv").write_text("\n".join(rows) + "\n")
    bench.summarize("counters", [str(d)], "c2l", ["cmd"])
    out = capsys.readouterr().out.splitlines()
    i = next(j for j, ln in enumerate(out) if ln.startswith("bwd_valu_kernel<8, 1, 4, true, false>"))
    assert out[i].split()[-1] == str(int(62.5 * steps))
    assert out[i + 1].split()[-1] == "62.50"


def test_counted_sources_exist():
    import bench
    assert any(f.endswith(".hip") for f in os.listdir(bench.CSRC))


def test_cpu_leg_and_parity_sample():
    import numpy as np

    import bench
    from workloads import WORKLOADS
    w = WORKLOADS["c2"].with_(T=32)
    rec, ref = bench.cpu_leg(w, 0.0, max_workers=2)
    assert rec["kind"] == "oracle" and rec["cores"] == 1 and rec["value"] > 0
    assert rec["cpu_model"] and rec["parallel"]["cpu_model"] == rec["cpu_model"]
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
