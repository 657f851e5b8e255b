"""Host-side checks of libmru.so that need no GPU.

The library must load, export every entry point include/mru.h declares, and
answer its pure host queries (version, status strings, plans).  Argument
validation happens before any HIP call, so invalid calls can be checked here
too; no call in this file launches anything.
"""
import ctypes
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mru.h")


def _declared_functions():
    text = open(HEADER).read()
    return re.findall(r"^\s*(?:mru_status|int32_t|size_t|const char\s*\*)\s*(mru_\w+)\s*\(", text, re.M)


@pytest.fixture(scope="module")
def mpp():
    import matrix_prefix_product_amd as m
    if not os.path.exists(m.library_path()):
        pytest.fail("libmru.so is not built: run python -m matrix_prefix_product_amd.build")
    m.load_library()
    return m


def test_header_declares_the_boundary():
    names = set(_declared_functions())
    assert {"mru_build_inputs", "mru_build_inputs_bwd", "mru_scan_fwd", "mru_scan_bwd",
            "mru_scan_workspace_bytes", "mru_scan_ws_status", "mru_scan_fwd_chunked",
            "mru_scan_bwd_chunked", "mru_scan_workspace_bytes_chunked",
            "mru_scan_chunk", "mru_scan_plan", "mru_status_string", "mru_abi_version"} <= names


def test_library_exports_every_declared_symbol(mpp):
    lib = ctypes.CDLL(mpp.library_path())
    missing = [name for name in _declared_functions() if not hasattr(lib, name)]
    assert not missing, missing


def test_abi_version_and_status_strings(mpp):
    lib = mpp.load_library()
    text = open(HEADER).read()
    assert lib.mru_abi_version() == int(re.search(r"#define MRU_ABI_VERSION (\d+)", text).group(1))
    for code in range(9):
        s = lib.mru_status_string(code).decode()
        assert s.startswith("MRU_")
    assert "unknown" in lib.mru_status_string(99).decode()


def test_plans_single_and_multi(mpp):
    # many sequences: one chunk per sequence, no workspace
    K, nch, Z, ws = mpp.scan_plan(1024, 8, 256, 8, mpp.DIR_FWD)
    assert (K, nch, ws) == (256, 1, 0)
    # one long sequence: chunks, padded to whole waves of chains, with a workspace
    K, nch, Z, ws = mpp.scan_plan(1, 1, 1024, 4, mpp.DIR_FWD)
    assert K >= 16 and nch * K >= 1024 and nch % 16 == 0 and Z % 16 == 0 and ws > 0
    # matrix-core path: one chain per wave, no padding
    K, nch, Z, ws = mpp.scan_plan(1, 8, 65536, 32, mpp.DIR_FWD)
    assert nch == math.ceil(65536 / K) and 1 <= Z <= 64 and ws > 0
    # explicit chunk lengths, ragged tails
    for n in (4, 8, 16, 32):
        for chunk in (1, 5, 64, 10_000):
            K, nch, Z, ws = mpp.scan_plan(2, 3, 203, n, mpp.DIR_BWD, chunk)
            assert K == min(chunk, 203)
            assert nch >= math.ceil(203 / K)
            assert (ws == 0) == (nch == 1)
            assert mpp.workspace_bytes(2, 3, 203, n, mpp.DIR_BWD, chunk) == ws
    assert mpp.scan_chunk(1024, 8, 256, 8) == 256
    # n = 16 from raw token vectors: 24-token chunks (three waves per SIMD) where
    # the scan from M takes 64; one workspace size covers both
    assert mpp.scan_chunk(4, 16, 8192, 16) == 64
    assert mpp.scan_chunk(4, 16, 8192, 16, mpp.DIR_FWD_X) == 24
    Kx, nchx, _, wsx = mpp.scan_plan(4, 16, 8192, 16, mpp.DIR_FWD_X)
    assert (Kx, nchx) == (24, 342)
    # n = 32 from raw token vectors: twice the chains of the scan from M (two
    # waves per SIMD)
    assert mpp.scan_chunk(1, 8, 65536, 32) == 512
    assert mpp.scan_chunk(1, 8, 65536, 32, mpp.DIR_FWD_X) == 256
    assert mpp.workspace_bytes(4, 16, 8192, 16) == wsx > mpp.scan_plan(4, 16, 8192, 16)[3]
    assert mpp.workspace_bytes(4, 16, 8192, 16, mpp.DIR_FWD_X) == wsx
    # the same explicit chunk gives the same chunks and workspace either way; the
    # forward from M at n = 16 groups them into smaller supers (a quarter of
    # sqrt(chunks), at least 5, against a half)
    fx, fm = mpp.scan_plan(2, 3, 203, 16, mpp.DIR_FWD_X, 5), mpp.scan_plan(2, 3, 203, 16, mpp.DIR_FWD, 5)
    assert (fx[0], fx[1], fx[3]) == (fm[0], fm[1], fm[3])
    assert (fx[2], fm[2]) == (round(0.5 * math.sqrt(41)), 5)
    assert mpp.scan_plan(4, 16, 8192, 16)[2] == 5 and mpp.scan_plan(4, 16, 8192, 16, mpp.DIR_BWD)[2] == 4
    assert mpp.scan_plan(8, 8, 4096, 16)[2] == 5 and mpp.scan_plan(4, 16, 65536, 16)[2] == 8


def test_plan_rejects_bad_arguments(mpp):
    with pytest.raises(mpp.MRUError) as e:
        mpp.scan_plan(1, 1, 16, 5)
    assert e.value.status == 2
    with pytest.raises(mpp.MRUError) as e:
        mpp.scan_plan(1, 1, 16, 8, chunk=-1)
    assert e.value.status == 6
    assert mpp.workspace_bytes(-1, 1, 16, 8) == 0
    assert mpp.scan_chunk(1, 1, 16, 6) == 0


def test_validation_before_any_launch(mpp):
    lib = mpp.load_library()
    nul = ctypes.c_void_p(0)
    fake = ctypes.c_void_p(0x10000)       # never dereferenced: every call below fails validation
    odd = ctypes.c_void_p(0x10004)
    # shape errors
    assert lib.mru_scan_fwd(fake, fake, 1, 1, 4, 6, nul, 0, nul) == 2
    assert lib.mru_scan_fwd(fake, fake, -1, 1, 4, 8, nul, 0, nul) == 2
    assert lib.mru_build_inputs(fake, fake, 1, 1, 4, 3, nul) == 2
    # chunk error
    assert lib.mru_scan_fwd_chunked(fake, fake, 1, 1, 4, 8, -2, nul, 0, nul) == 6
    # empty problems are a no-op, even with NULL pointers
    assert lib.mru_scan_fwd(nul, nul, 0, 4, 16, 8, nul, 0, nul) == 0
    assert lib.mru_scan_bwd(nul, nul, nul, nul, 2, 2, 0, 16, nul, 0, nul) == 0
    assert lib.mru_build_inputs(nul, nul, 3, 0, 5, 4, nul) == 0
    # null, alignment, aliasing, workspace
    assert lib.mru_scan_fwd(nul, fake, 1, 1, 4, 8, nul, 0, nul) == 1
    assert lib.mru_scan_bwd(fake, fake, nul, fake, 1, 1, 4, 8, nul, 0, nul) == 1
    assert lib.mru_scan_fwd(odd, fake, 1, 1, 4, 8, nul, 0, nul) == 3
    assert lib.mru_scan_fwd(fake, fake, 1, 1, 4, 8, nul, 0, nul) == 4
    assert lib.mru_build_inputs(fake, ctypes.c_void_p(0x10000 + 16), 1, 1, 4, 4, nul) == 4
    a, b = ctypes.c_void_p(0x100000), ctypes.c_void_p(0x200000)
    # one sequence of 1024 tokens needs a workspace: missing / too small
    assert lib.mru_scan_fwd(a, b, 1, 1, 1024, 4, nul, 0, nul) == 5
    need = mpp.workspace_bytes(1, 1, 1024, 4)
    ws = ctypes.c_void_p(0x400000)
    assert lib.mru_scan_fwd(a, b, 1, 1, 1024, 4, ws, need - 1, nul) == 5
    # workspace overlapping an output
    assert lib.mru_scan_fwd(a, b, 1, 1, 1024, 4, ctypes.c_void_p(0x200000 + 64), need, nul) == 4
    # dM aliasing dP
    assert lib.mru_scan_bwd_chunked(a, b, ws, ws, 1, 1, 8, 8, 1, nul, 0, nul) == 4
    # build gradient: shape, null, alias, empty
    assert lib.mru_build_inputs_bwd(a, b, ws, 1, 1, 4, 5, nul) == 2
    assert lib.mru_build_inputs_bwd(a, nul, ws, 1, 1, 4, 8, nul) == 1
    assert lib.mru_build_inputs_bwd(a, b, a, 1, 1, 4, 8, nul) == 4
    assert lib.mru_build_inputs_bwd(odd, b, ws, 1, 1, 4, 8, nul) == 3
    assert lib.mru_build_inputs_bwd(nul, nul, nul, 0, 1, 4, 8, nul) == 0


def test_fused_entries_validate_before_any_launch(mpp):
    lib = mpp.load_library()
    nul = ctypes.c_void_p(0)
    a, b, c, d = (ctypes.c_void_p(v) for v in (0x100000, 0x200000, 0x300000, 0x400000))
    # both scans start from token vectors for every n (validation still comes first)
    assert lib.mru_scan_bwd_x(a, b, c, c, 1, 1, 16, 16, 0, nul, 0, nul) == 4
    assert lib.mru_scan_bwd_x(a, b, c, c, 1, 1, 16, 32, 0, nul, 0, nul) == 4
    assert lib.mru_scan_bwd_x(a, b, c, d, 1, 1, 16, 6, 0, nul, 0, nul) == 2
    assert lib.mru_scan_fwd_x(a, b, 1, 1, 16, 6, 0, nul, 0, nul) == 2
    # empty, null, alias, workspace, chunk
    assert lib.mru_scan_fwd_x(nul, nul, 0, 1, 16, 8, 0, nul, 0, nul) == 0
    assert lib.mru_scan_fwd_x(nul, b, 1, 1, 16, 8, 0, nul, 0, nul) == 1
    assert lib.mru_scan_fwd_x(a, a, 1, 1, 16, 8, 0, nul, 0, nul) == 4
    assert lib.mru_scan_fwd_x(a, b, 1, 1, 1024, 4, 0, nul, 0, nul) == 5
    assert lib.mru_scan_fwd_x(a, b, 1, 1, 16, 8, -1, nul, 0, nul) == 6
    assert lib.mru_scan_bwd_x(a, b, c, c, 1, 1, 8, 8, 1, nul, 0, nul) == 4
    assert lib.mru_scan_bwd_x(a, b, nul, d, 1, 1, 8, 8, 1, nul, 0, nul) == 1


def test_extended_entries_validate_before_any_launch(mpp):
    lib = mpp.load_library()
    nul = ctypes.c_void_p(0)
    a, b, c, d, e = (ctypes.c_void_p(v) for v in (0x100000, 0x200000, 0x300000, 0x400000, 0x500000))
    odd16 = ctypes.c_void_p(0x300004)
    odd4 = ctypes.c_void_p(0x300002)
    # forward: misaligned carry / exponents, exponents overlapping P, P over the carry
    assert lib.mru_scan_fwd_ex(a, 0, odd16, nul, b, nul, 1, 1, 8, 8, 1 << 20, nul, 0, nul) == 3
    assert lib.mru_scan_fwd_ex(a, 0, c, odd4, b, nul, 1, 1, 8, 8, 1 << 20, nul, 0, nul) == 3
    assert lib.mru_scan_fwd_ex(a, 0, c, nul, b, ctypes.c_void_p(0x200000 + 64), 1, 1, 8, 8, 1 << 20,
                               nul, 0, nul) == 4
    assert lib.mru_scan_fwd_ex(a, 0, ctypes.c_void_p(0x200000 + 256), nul, b, nul, 1, 1, 8, 8,
                               1 << 20, nul, 0, nul) == 4
    # from_x: both directions every n (bad n refused, validation before launch); empty is a no-op
    assert lib.mru_scan_fwd_ex(a, 1, nul, nul, b, nul, 1, 1, 8, 6, 0, nul, 0, nul) == 2
    assert lib.mru_scan_bwd_ex(a, 1, nul, b, c, d, nul, 1, 1, 8, 6, 0, nul, 0, nul) == 2
    assert lib.mru_scan_bwd_ex(a, 1, nul, b, c, c, nul, 1, 1, 8, 16, 0, nul, 0, nul) == 4
    assert lib.mru_scan_fwd_ex(nul, 0, c, nul, nul, nul, 1, 1, 0, 8, 0, nul, 0, nul) == 0
    # backward: dcarry overlapping dM or the carry, misaligned dcarry
    assert lib.mru_scan_bwd_ex(a, 0, c, b, d, e, ctypes.c_void_p(0x500000 + 64), 1, 1, 8, 8, 1 << 20,
                               nul, 0, nul) == 4
    assert lib.mru_scan_bwd_ex(a, 0, c, b, d, e, c, 1, 1, 8, 8, 1 << 20, nul, 0, nul) == 4
    assert lib.mru_scan_bwd_ex(a, 0, c, b, d, e, odd16, 1, 1, 8, 8, 1 << 20, nul, 0, nul) == 3


def test_layer_backward_entry_validates_before_any_launch(mpp):
    lib = mpp.load_library()
    nul = ctypes.c_void_p(0)
    x, C, P, R, dx, dC = (ctypes.c_void_p(v) for v in
                          (0x100000, 0x200000, 0x300000, 0x400000, 0x500000, 0x600000))
    # arguments: x, carry, P, dP, dx, dcarry, B, H, T, n, chunk, ws, ws_bytes, stream
    assert lib.mru_scan_bwd_dx(x, nul, P, R, x, nul, 1, 1, 8, 16, 0, nul, 0, nul) == 4     # n = 16, dx over x
    assert lib.mru_scan_bwd_dx(x, nul, P, R, dx, nul, 1, 1, 8, 6, 0, nul, 0, nul) == 2    # bad n
    assert lib.mru_scan_bwd_dx(nul, nul, nul, nul, nul, nul, 1, 1, 0, 8, 0, nul, 0, nul) == 0  # empty
    assert lib.mru_scan_bwd_dx(x, nul, P, nul, dx, nul, 1, 1, 8, 8, 0, nul, 0, nul) == 1  # null dP
    assert lib.mru_scan_bwd_dx(x, nul, P, R, x, nul, 1, 1, 8, 8, 0, nul, 0, nul) == 4     # dx over x
    assert lib.mru_scan_bwd_dx(x, ctypes.c_void_p(0x200004), P, R, dx, nul, 1, 1, 8, 8, 0, nul, 0,
                               nul) == 3                                                   # carry misaligned
    assert lib.mru_scan_bwd_dx(x, C, P, R, dx, ctypes.c_void_p(0x500000 + 64), 1, 1, 8, 8, 0, nul, 0,
                               nul) == 4                                                   # dcarry over dx
    assert lib.mru_scan_bwd_dx(x, nul, P, R, dx, nul, 1, 1, 8, 8, -1, nul, 0, nul) == 6   # chunk


def test_orthogonal_build_validates(mpp):
    lib = mpp.load_library()
    nul = ctypes.c_void_p(0)
    a, b = ctypes.c_void_p(0x100000), ctypes.c_void_p(0x200000)
    assert lib.mru_build_orthogonal(a, b, 1, 1, 4, 8, 2, nul) == 2     # unknown method
    assert lib.mru_build_orthogonal(a, b, 1, 1, 4, 6, 0, nul) == 2     # bad n
    assert lib.mru_build_orthogonal(a, a, 1, 1, 4, 8, 1, nul) == 4     # alias
    assert lib.mru_build_orthogonal(nul, b, 1, 1, 4, 8, 0, nul) == 1
    assert lib.mru_build_orthogonal(nul, nul, 0, 1, 4, 8, 0, nul) == 0


def _signature(name):
    """Parameter list of a declaration in mru.h, as (type, name) strings."""
    text = open(HEADER).read()
    m = re.search(r"^\s*\w[\w\s\*]*?\b" + name + r"\s*\(([^)]*)\)\s*;", text, re.M)
    assert m, name
    params = [p.strip() for p in m.group(1).replace("\n", " ").split(",")]
    return [re.sub(r"\s+", " ", p) for p in params]


def test_boundary_signatures():
    """The three scan calls of the boundary take exactly (pointers..., B, H, T,
    n, ws, ws_bytes, stream) and (B, H, T, n, direction): no chunk argument."""
    assert _signature("mru_scan_fwd") == [
        "const float* M", "float* P", "int64_t B", "int64_t H", "int64_t T", "int32_t n",
        "void* ws", "size_t ws_bytes", "void* stream"]
    assert _signature("mru_scan_bwd") == [
        "const float* M", "const float* P", "const float* dP", "float* dM", "int64_t B",
        "int64_t H", "int64_t T", "int32_t n", "void* ws", "size_t ws_bytes", "void* stream"]
    assert _signature("mru_scan_workspace_bytes") == [
        "int64_t B", "int64_t H", "int64_t T", "int32_t n", "int32_t direction"]
    assert _signature("mru_build_inputs") == [
        "const float* x", "float* M", "int64_t B", "int64_t H", "int64_t T", "int32_t n",
        "void* stream"]


def test_boundary_calls(mpp):
    """Each boundary signature called through ctypes with its own argument list:
    validation answers before any launch, the workspace query matches the plan."""
    lib = mpp.load_library()
    nul = ctypes.c_void_p(0)
    a, b, c, d = (ctypes.c_void_p(0x10000000 * k) for k in (1, 2, 3, 4))   # 256 MiB apart
    for n in (4, 8, 16, 32):
        for direction in (mpp.DIR_FWD, mpp.DIR_BWD):
            need = lib.mru_scan_workspace_bytes(1, 2, 777, n, direction)
            plans = [mpp.scan_plan(1, 2, 777, n, direction)[3]]
            if direction == mpp.DIR_FWD:
                plans.append(mpp.scan_plan(1, 2, 777, n, mpp.DIR_FWD_X)[3])
            assert need == max(plans)
            assert need == lib.mru_scan_workspace_bytes_chunked(1, 2, 777, n, direction, 0)
            assert need > 0   # two sequences of 777 tokens: several chunks each
        # a missing workspace is reported by the boundary forms themselves
        assert lib.mru_scan_fwd(a, b, 1, 2, 777, n, nul, 0, nul) == 5
        assert lib.mru_scan_bwd(a, b, c, d, 1, 2, 777, n, nul, 0, nul) == 5
        # bad n, empty problem
        assert lib.mru_scan_fwd(a, b, 1, 2, 777, n + 1, nul, 0, nul) == 2
        assert lib.mru_scan_bwd(nul, nul, nul, nul, 1, 2, 0, n, nul, 0, nul) == 0
    # the chunked forms keep the explicit plan
    assert lib.mru_scan_workspace_bytes_chunked(1, 1, 64, 8, 0, 8) == mpp.scan_plan(1, 1, 64, 8, 0, 8)[3]
    assert lib.mru_scan_bwd_chunked(a, b, c, d, 1, 1, 64, 8, -1, nul, 0, nul) == 6


def test_ws_status_validation(mpp):
    lib = mpp.load_library()
    nul = ctypes.c_void_p(0)
    ws = ctypes.c_void_p(0x100000)
    assert lib.mru_scan_ws_status(ws, 4096, nul, nul) == 1                       # no output
    assert lib.mru_scan_ws_status(ws, 4096, ctypes.c_void_p(0x200002), nul) == 3  # misaligned
    assert lib.mru_scan_ws_status(ctypes.c_void_p(0x100008), 4096, ctypes.c_void_p(0x200000), nul) == 3
    assert lib.mru_scan_ws_status(ws, 4096, ctypes.c_void_p(0x100004), nul) == 4  # inside the header
