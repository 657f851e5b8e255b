"""The allocation-free forward scan (mru_scan_fwd_noalloc), called through the C
ABI: bitwise the same prefixes as mru_scan_fwd with a caller workspace, on two
calls in a row (the second smaller, so it runs over the first call's leftover
scratch contents), and its size limit is enforced before any launch."""
import ctypes

import numpy as np
import pytest
import torch

from gpu_helpers import dev, host, random_M, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    import matrix_prefix_product_amd as m
    lib = m.load_library()
    lib.mru_scan_fwd_noalloc.restype = ctypes.c_int32
    lib.mru_scan_fwd_noalloc.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                         ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,
                                         ctypes.c_void_p]
    return lib


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _reference(lib, Md, B, H, T, n):
    """mru_scan_fwd with a workspace of the queried size."""
    need = lib.mru_scan_workspace_bytes(B, H, T, n, 0)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
    P = torch.empty_like(Md)
    assert lib.mru_scan_fwd(_ptr(Md), _ptr(P), B, H, T, n, _ptr(ws), need, _stream()) == 0
    return host(P), need


def test_noalloc_matches_the_workspace_scan_twice(lib):
    # first call: n = 16, several chunks per sequence; second: smaller, n = 8
    for (B, H, T, n, seed) in ((2, 3, 1500, 16, 11), (1, 2, 700, 8, 12)):
        say(f"[noalloc] B={B} H={H} T={T} n={n}")
        Md = dev(random_M((B, H, T), n, seed=seed))
        ref, need = _reference(lib, Md, B, H, T, n)
        assert need > 0   # the plan has a look-back workspace
        P = torch.full_like(Md, float("nan"))
        assert lib.mru_scan_fwd_noalloc(_ptr(Md), _ptr(P), B, H, T, n, _stream()) == 0
        got = host(P)
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_noalloc_single_chunk_and_empty(lib):
    B, H, T, n = 512, 8, 16, 8   # 4096 sequences: one chunk each, no scratch needed
    say(f"[noalloc] single chunk B={B} H={H} T={T} n={n}")
    Md = dev(random_M((B, H, T), n, seed=3))
    ref, need = _reference(lib, Md, B, H, T, n)
    assert need == 0
    P = torch.empty_like(Md)
    assert lib.mru_scan_fwd_noalloc(_ptr(Md), _ptr(P), B, H, T, n, _stream()) == 0
    assert np.array_equal(host(P).view(np.uint32), ref.view(np.uint32))
    nul = ctypes.c_void_p(0)
    assert lib.mru_scan_fwd_noalloc(nul, nul, 0, 4, 16, 8, nul) == 0


def test_noalloc_rejects_plans_beyond_the_scratch(lib):
    # 64 sequences of 65536 tokens at n = 16 need a 256 MiB look-back workspace
    B, H, T, n = 4, 16, 65536, 16
    need = lib.mru_scan_workspace_bytes(B, H, T, n, 0)
    assert need > (64 << 20)
    fake = ctypes.c_void_p(0x10000)   # never dereferenced: rejected before any launch
    assert lib.mru_scan_fwd_noalloc(fake, ctypes.c_void_p(0x40000000), B, H, T, n,
                                    ctypes.c_void_p(0)) == 5
    assert lib.mru_scan_fwd_noalloc(fake, fake, B, H, T, 6, ctypes.c_void_p(0)) == 2
