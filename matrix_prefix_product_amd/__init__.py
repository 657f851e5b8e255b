"""MRU prefix scan on MI355X (gfx950): Python binding of libmru.so.

Matrix Recurrent Units build an n-by-n input state matrix per token (LDU fill
with a determinant-correcting scalar), multiply the matrices along the
sequence, and flatten each running product back to a vector.  Every step of
that runs in the HIP kernels of libmru.so; this module only checks tensor
arguments, allocates outputs and workspaces through torch, and passes device
pointers and the current stream to the C ABI declared in include/mru.h.

Functions (tensors are contiguous fp32 on a ROCm device):
    build_inputs(x, n)        x [B,H,T,n*n] -> M [B,H,T,n,n]
    build_inputs_bwd(x, dM)   gradient through the build: dx [B,H,T,n*n]
    scan_fwd(M, chunk=0)      M -> P, P_t = M_1 ... M_t
    scan_bwd(M, P, dP)        -> dM, gradient of sum_t <dP_t, P_t>
    flatten(P)                P [B,H,T,n,n] -> [B,H,T,n*n] (a view)
    mru_scan(M)               scan_fwd with autograd (backward = scan_bwd)
    mru_layer(x, n)           build + scan with autograd down to the token vectors
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "build_inputs", "build_inputs_bwd", "scan_fwd", "mru_layer", "MRUBuild", "scan_bwd", "flatten", "mru_scan", "MRUScan",
    "scan_fwd_x", "scan_bwd_x", "scan_fwd_ex", "scan_bwd_ex", "scan_bwd_dx", "build_orthogonal",
    "scan_plan", "scan_chunk", "workspace_bytes", "library_path", "load_library",
    "MRUError", "DIR_FWD", "DIR_BWD", "DIR_FWD_X", "SUPPORTED_N", "FUSED_N", "FUSED_FWD_N", "FUSED_BWD_N",
    "set_checking", "ws_status", "MRU_ERR_TIMEOUT",
]

DIR_FWD = 0
DIR_BWD = 1
DIR_FWD_X = 2  # plan queries: the forward from raw token vectors
SUPPORTED_N = (4, 8, 16, 32)
# Sizes whose forward scan can start from raw token vectors (input matrices
# built on chip), whose backward scan to dL/dM can too (FUSED_BWD_N), and whose
# layer backward goes from dL/dP to dL/dx in one pass (FUSED_N).
FUSED_FWD_N = (4, 8, 16, 32)
FUSED_BWD_N = (4, 8, 16, 32)
FUSED_N = (4, 8, 16, 32)
_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libmru.so")
_LIB = None

_STATUS = {
    0: "MRU_OK", 1: "MRU_ERR_NULL", 2: "MRU_ERR_SHAPE", 3: "MRU_ERR_ALIGN", 4: "MRU_ERR_ALIAS",
    5: "MRU_ERR_WORKSPACE", 6: "MRU_ERR_CHUNK", 7: "MRU_ERR_HIP", 8: "MRU_ERR_TIMEOUT",
}
MRU_ERR_TIMEOUT = 8
# Whether every scan checks its workspace status word after the launch (one
# device-to-host read, which synchronises the stream); see set_checking().
_CHECK_ALL = os.environ.get("MRU_CHECK_WS", "0") not in ("", "0")


class MRUError(RuntimeError):
    """A non-OK status from libmru.so."""

    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {_STATUS.get(status, status)} ({_status_string(status)})")


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libmru.so (built in-tree).  Raises if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(
            f"{_LIB_PATH} is missing: build it with `python -m matrix_prefix_product_amd.build` "
            "(there is no CPU fallback)")
    lib = ctypes.CDLL(_LIB_PATH)
    i32, i64, sz, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p
    lib.mru_abi_version.restype = i32
    lib.mru_abi_version.argtypes = []
    lib.mru_status_string.restype = ctypes.c_char_p
    lib.mru_status_string.argtypes = [i32]
    lib.mru_build_inputs.restype = i32
    lib.mru_build_inputs.argtypes = [vp, vp, i64, i64, i64, i32, vp]
    lib.mru_build_orthogonal.restype = i32
    lib.mru_build_orthogonal.argtypes = [vp, vp, i64, i64, i64, i32, i32, vp]
    lib.mru_build_inputs_bwd.restype = i32
    lib.mru_build_inputs_bwd.argtypes = [vp, vp, vp, i64, i64, i64, i32, vp]
    lib.mru_scan_chunk.restype = i32
    lib.mru_scan_chunk.argtypes = [i64, i64, i64, i32, i32]
    lib.mru_scan_plan.restype = i32
    lib.mru_scan_plan.argtypes = [i64, i64, i64, i32, i32, i32, ctypes.POINTER(i64)]
    lib.mru_scan_workspace_bytes.restype = sz
    lib.mru_scan_workspace_bytes.argtypes = [i64, i64, i64, i32, i32]
    lib.mru_scan_workspace_bytes_chunked.restype = sz
    lib.mru_scan_workspace_bytes_chunked.argtypes = [i64, i64, i64, i32, i32, i32]
    lib.mru_scan_ws_status.restype = i32
    lib.mru_scan_ws_status.argtypes = [vp, sz, vp, vp]
    lib.mru_scan_fwd.restype = i32
    lib.mru_scan_fwd.argtypes = [vp, vp, i64, i64, i64, i32, vp, sz, vp]
    lib.mru_scan_fwd_chunked.restype = i32
    lib.mru_scan_fwd_chunked.argtypes = [vp, vp, i64, i64, i64, i32, i32, vp, sz, vp]
    lib.mru_scan_bwd.restype = i32
    lib.mru_scan_bwd.argtypes = [vp, vp, vp, vp, i64, i64, i64, i32, vp, sz, vp]
    lib.mru_scan_bwd_chunked.restype = i32
    lib.mru_scan_bwd_chunked.argtypes = [vp, vp, vp, vp, i64, i64, i64, i32, i32, vp, sz, vp]
    lib.mru_scan_fwd_x.restype = i32
    lib.mru_scan_fwd_x.argtypes = [vp, vp, i64, i64, i64, i32, i32, vp, sz, vp]
    lib.mru_scan_bwd_x.restype = i32
    lib.mru_scan_bwd_x.argtypes = [vp, vp, vp, vp, i64, i64, i64, i32, i32, vp, sz, vp]
    lib.mru_scan_fwd_ex.restype = i32
    lib.mru_scan_fwd_ex.argtypes = [vp, i32, vp, vp, vp, vp, i64, i64, i64, i32, i32, vp, sz, vp]
    lib.mru_scan_bwd_ex.restype = i32
    lib.mru_scan_bwd_ex.argtypes = [vp, i32, vp, vp, vp, vp, vp, i64, i64, i64, i32, i32, vp, sz, vp]
    lib.mru_scan_bwd_dx.restype = i32
    lib.mru_scan_bwd_dx.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i32, i32, vp, sz, vp]
    _LIB = lib
    return lib


def _status_string(status: int) -> str:
    try:
        return load_library().mru_status_string(int(status)).decode()
    except Exception:  # library missing: fall back to the code name
        return _STATUS.get(status, str(status))


def _check(status: int, what: str):
    if status != 0:
        raise MRUError(status, what)


def _stream_handle(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t: torch.Tensor | None):
    return ctypes.c_void_p(t.data_ptr()) if t is not None and t.numel() > 0 else ctypes.c_void_p(0)


def _require(t: torch.Tensor, name: str, ndim: int):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a ROCm GPU device, got {t.device}")
    if t.dtype != torch.float32:
        raise ValueError(f"{name} must be float32, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _mshape(M: torch.Tensor, name: str = "M"):
    _require(M, name, 5)
    B, H, T, n, n2 = M.shape
    if n != n2 or n not in SUPPORTED_N:
        raise ValueError(f"{name} must be [B,H,T,n,n] with n in {SUPPORTED_N}, got {tuple(M.shape)}")
    return B, H, T, n


def scan_chunk(B: int, H: int, T: int, n: int, direction: int = DIR_FWD) -> int:
    """Chunk length the automatic plan uses for this shape."""
    return int(load_library().mru_scan_chunk(B, H, T, n, direction))


def scan_plan(B: int, H: int, T: int, n: int, direction: int = DIR_FWD, chunk: int = 0):
    """(K, chunks per sequence, chunks per super, workspace bytes) of a scan."""
    out = (ctypes.c_int64 * 4)()
    _check(load_library().mru_scan_plan(B, H, T, n, direction, chunk, out), "mru_scan_plan")
    return tuple(int(v) for v in out)


def workspace_bytes(B: int, H: int, T: int, n: int, direction: int = DIR_FWD, chunk: int = 0) -> int:
    lib = load_library()
    if chunk == 0:
        return int(lib.mru_scan_workspace_bytes(B, H, T, n, direction))
    return int(lib.mru_scan_workspace_bytes_chunked(B, H, T, n, direction, chunk))


def set_checking(on: bool = True) -> None:
    """Make every scan of this module read its workspace status word after the
    launch and raise MRUError(MRU_ERR_TIMEOUT) if a look-back wait gave up.
    The read synchronises the stream, so it is off by default; the
    environment variable MRU_CHECK_WS=1 turns it on at import."""
    global _CHECK_ALL
    _CHECK_ALL = bool(on)


def ws_status(workspace: torch.Tensor | None, stream_device: torch.device | None = None) -> int:
    """Status word of a scan workspace (mru_scan_ws_status), read back to the
    host: 0, or MRU_WS_STATUS_SPIN_TIMEOUT (1) when a look-back wait of the
    last multi-chunk scan that used it gave up.  Synchronises the stream."""
    dev = workspace.device if workspace is not None else (stream_device or torch.device("cuda"))
    out = torch.empty(1, dtype=torch.int32, device=dev)
    lib = load_library()
    nbytes = workspace.numel() if workspace is not None else 0
    with torch.cuda.device(dev):
        st = lib.mru_scan_ws_status(_ptr(workspace), nbytes, _ptr(out), _stream_handle(dev))
    _check(st, "mru_scan_ws_status")
    return int(out.item())


def _after_scan(ws, check, what, shape, n, direction, chunk):
    """Raise if the scan that just used ws reported a timed-out look-back (only
    multi-chunk plans wait, and only they write the status word)."""
    if not (check or _CHECK_ALL) or ws is None:
        return
    if workspace_bytes(*shape, n, direction, chunk) == 0:
        return
    if ws_status(ws) != 0:
        raise MRUError(MRU_ERR_TIMEOUT, what)


def _workspace(shape, n, direction, chunk, device, workspace):
    need = workspace_bytes(*shape, n, direction, chunk)
    if workspace is not None:
        if workspace.device != device or workspace.dtype != torch.uint8 or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous uint8 tensor on the same device")
        return workspace, workspace.numel()
    if need == 0:
        return None, 0
    return torch.empty(need, dtype=torch.uint8, device=device), need


def build_inputs(x: torch.Tensor, n: int, out: torch.Tensor | None = None) -> torch.Tensor:
    """[B,H,T,n*n] raw token vectors -> [B,H,T,n,n] input state matrices."""
    _require(x, "x", 4)
    B, H, T, nn = x.shape
    if n not in SUPPORTED_N or nn != n * n:
        raise ValueError(f"x must be [B,H,T,n*n] with n in {SUPPORTED_N}, got {tuple(x.shape)}, n={n}")
    if out is None:
        M = torch.empty((B, H, T, n, n), dtype=torch.float32, device=x.device)
    else:
        _require(out, "out", 5)
        if tuple(out.shape) != (B, H, T, n, n) or out.device != x.device:
            raise ValueError("out must be [B,H,T,n,n] on x's device")
        M = out
    lib = load_library()
    with torch.cuda.device(x.device):
        st = lib.mru_build_inputs(_ptr(x), _ptr(M), B, H, T, n, _stream_handle(x.device))
    _check(st, "mru_build_inputs")
    return M


ORTHO_METHODS = {"cayley": 0, "expm": 1}


def build_orthogonal(x: torch.Tensor, n: int, method: str = "cayley",
                     out: torch.Tensor | None = None) -> torch.Tensor:
    """[B,H,T,n*n] raw token vectors -> [B,H,T,n,n] orthogonal input matrices:
    the Cayley map or the exponential of A = (X - X^T)/2."""
    if method not in ORTHO_METHODS:
        raise ValueError(f"method must be one of {tuple(ORTHO_METHODS)}")
    _require(x, "x", 4)
    B, H, T, nn = x.shape
    if n not in SUPPORTED_N or nn != n * n:
        raise ValueError(f"x must be [B,H,T,n*n] with n in {SUPPORTED_N}, got {tuple(x.shape)}, n={n}")
    if out is None:
        M = torch.empty((B, H, T, n, n), dtype=torch.float32, device=x.device)
    else:
        _require(out, "out", 5)
        if tuple(out.shape) != (B, H, T, n, n) or out.device != x.device:
            raise ValueError("out must be [B,H,T,n,n] on x's device")
        M = out
    lib = load_library()
    with torch.cuda.device(x.device):
        st = lib.mru_build_orthogonal(_ptr(x), _ptr(M), B, H, T, n, ORTHO_METHODS[method],
                                      _stream_handle(x.device))
    _check(st, "mru_build_orthogonal")
    return M


def build_inputs_bwd(x: torch.Tensor, dM: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """Gradient through the LDU build: dx [B,H,T,n*n] from x and dM = dL/dM [B,H,T,n,n]."""
    _require(x, "x", 4)
    B, H, T, n = _mshape(dM, "dM")
    if tuple(x.shape) != (B, H, T, n * n) or x.device != dM.device:
        raise ValueError("x must be [B,H,T,n*n] matching dM on the same device")
    if out is None:
        out = torch.empty_like(x)
    else:
        _require(out, "out", 4)
        if out.shape != x.shape or out.device != x.device:
            raise ValueError("out must match x")
    lib = load_library()
    with torch.cuda.device(x.device):
        st = lib.mru_build_inputs_bwd(_ptr(x), _ptr(dM), _ptr(out), B, H, T, n, _stream_handle(x.device))
    _check(st, "mru_build_inputs_bwd")
    return out


def scan_fwd(M: torch.Tensor, chunk: int = 0, out: torch.Tensor | None = None,
             workspace: torch.Tensor | None = None, check: bool = False) -> torch.Tensor:
    """All prefix products P_t = M_1 ... M_t (P_0 = I), [B,H,T,n,n].

    chunk 0 uses the automatic plan (mru_scan_fwd), a positive chunk forces that
    chunk length (mru_scan_fwd_chunked).  check: read the workspace status word
    afterwards and raise if a look-back wait gave up (synchronises)."""
    B, H, T, n = _mshape(M)
    if out is None:
        out = torch.empty_like(M)
    else:
        _require(out, "out", 5)
        if out.shape != M.shape or out.device != M.device:
            raise ValueError("out must match M")
    ws, ws_bytes = _workspace((B, H, T), n, DIR_FWD, chunk, M.device, workspace)
    lib = load_library()
    with torch.cuda.device(M.device):
        if chunk == 0:
            st = lib.mru_scan_fwd(_ptr(M), _ptr(out), B, H, T, n, _ptr(ws), ws_bytes,
                                  _stream_handle(M.device))
        else:
            st = lib.mru_scan_fwd_chunked(_ptr(M), _ptr(out), B, H, T, n, chunk, _ptr(ws), ws_bytes,
                                          _stream_handle(M.device))
    _check(st, "mru_scan_fwd")
    _after_scan(ws, check, "mru_scan_fwd", (B, H, T), n, DIR_FWD, chunk)
    return out


def scan_bwd(M: torch.Tensor, P: torch.Tensor, dP: torch.Tensor, chunk: int = 0,
             out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
             check: bool = False) -> torch.Tensor:
    """Gradient dM of sum_t <dP_t, P_t> where P = scan_fwd(M), [B,H,T,n,n]
    (chunk and check as for scan_fwd)."""
    B, H, T, n = _mshape(M)
    for name, t in (("P", P), ("dP", dP)):
        _require(t, name, 5)
        if t.shape != M.shape or t.device != M.device:
            raise ValueError(f"{name} must have M's shape and device")
    if out is None:
        out = torch.empty_like(M)
    else:
        _require(out, "out", 5)
        if out.shape != M.shape or out.device != M.device:
            raise ValueError("out must match M")
    ws, ws_bytes = _workspace((B, H, T), n, DIR_BWD, chunk, M.device, workspace)
    lib = load_library()
    with torch.cuda.device(M.device):
        if chunk == 0:
            st = lib.mru_scan_bwd(_ptr(M), _ptr(P), _ptr(dP), _ptr(out), B, H, T, n, _ptr(ws),
                                  ws_bytes, _stream_handle(M.device))
        else:
            st = lib.mru_scan_bwd_chunked(_ptr(M), _ptr(P), _ptr(dP), _ptr(out), B, H, T, n, chunk,
                                          _ptr(ws), ws_bytes, _stream_handle(M.device))
    _check(st, "mru_scan_bwd")
    _after_scan(ws, check, "mru_scan_bwd", (B, H, T), n, DIR_BWD, chunk)
    return out


def _xshape(x: torch.Tensor, n: int, allowed=FUSED_N):
    _require(x, "x", 4)
    B, H, T, nn = x.shape
    if n not in allowed or nn != n * n:
        raise ValueError(f"x must be [B,H,T,n*n] with n in {allowed}, got {tuple(x.shape)}, n={n}")
    return B, H, T


def scan_fwd_x(x: torch.Tensor, n: int, chunk: int = 0, out: torch.Tensor | None = None,
               workspace: torch.Tensor | None = None, check: bool = False) -> torch.Tensor:
    """scan_fwd(build_inputs(x, n)) in one pass that never writes the input
    matrices (n in FUSED_FWD_N)."""
    B, H, T = _xshape(x, n, FUSED_FWD_N)
    if out is None:
        out = torch.empty((B, H, T, n, n), dtype=torch.float32, device=x.device)
    else:
        _require(out, "out", 5)
        if tuple(out.shape) != (B, H, T, n, n) or out.device != x.device:
            raise ValueError("out must be [B,H,T,n,n] on x's device")
    ws, ws_bytes = _workspace((B, H, T), n, DIR_FWD, chunk, x.device, workspace)
    lib = load_library()
    with torch.cuda.device(x.device):
        st = lib.mru_scan_fwd_x(_ptr(x), _ptr(out), B, H, T, n, chunk, _ptr(ws), ws_bytes,
                                _stream_handle(x.device))
    _check(st, "mru_scan_fwd_x")
    _after_scan(ws, check, "mru_scan_fwd_x", (B, H, T), n, DIR_FWD_X, chunk)
    return out


def scan_bwd_x(x: torch.Tensor, P: torch.Tensor, dP: torch.Tensor, chunk: int = 0,
               out: torch.Tensor | None = None, workspace: torch.Tensor | None = None, check: bool = False) -> torch.Tensor:
    """scan_bwd(build_inputs(x, n), P, dP) with the input matrices rebuilt on chip
    (n in FUSED_BWD_N)."""
    _require(P, "P", 5)
    n = P.shape[-1]
    B, H, T = _xshape(x, n, FUSED_BWD_N)
    for name, t in (("P", P), ("dP", dP)):
        _require(t, name, 5)
        if tuple(t.shape) != (B, H, T, n, n) or t.device != x.device:
            raise ValueError(f"{name} must be [B,H,T,n,n] on x's device")
    if out is None:
        out = torch.empty_like(P)
    else:
        _require(out, "out", 5)
        if out.shape != P.shape or out.device != x.device:
            raise ValueError("out must match P")
    ws, ws_bytes = _workspace((B, H, T), n, DIR_BWD, chunk, x.device, workspace)
    lib = load_library()
    with torch.cuda.device(x.device):
        st = lib.mru_scan_bwd_x(_ptr(x), _ptr(P), _ptr(dP), _ptr(out), B, H, T, n, chunk, _ptr(ws),
                                ws_bytes, _stream_handle(x.device))
    _check(st, "mru_scan_bwd_x")
    _after_scan(ws, check, "mru_scan_bwd_x", (B, H, T), n, DIR_BWD, chunk)
    return out


def _inshape(inp: torch.Tensor, from_x: bool, n: int | None, allowed=FUSED_N):
    if from_x:
        if n is None:
            raise ValueError("n is required when the input is raw token vectors")
        return (*_xshape(inp, n, allowed), n)
    return _mshape(inp)


def _carry_arg(carry, B, H, n, dev, name="carry"):
    if carry is None:
        return None
    _require(carry, name, 4)
    if tuple(carry.shape) != (B, H, n, n) or carry.device != dev:
        raise ValueError(f"{name} must be [B,H,n,n] = {(B, H, n, n)} on the input's device")
    return carry


def scan_fwd_ex(inp: torch.Tensor, carry: torch.Tensor | None = None,
                carry_exp: torch.Tensor | None = None, scaled: bool = False,
                from_x: bool = False, n: int | None = None, chunk: int = 0,
                workspace: torch.Tensor | None = None, check: bool = False):
    """P_t = P_0 M_1 ... M_t with P_0 = 2^carry_exp * carry (I when carry is None).

    inp is M [B,H,T,n,n], or x [B,H,T,n*n] with from_x (n in FUSED_FWD_N).
    Returns P, or (P, E) with scaled: P_t = 2^E[t] * P[t], max |P[t]| in
    [0.5, 1].  The last token's (P, E) is the carry into the next segment."""
    B, H, T, n = _inshape(inp, from_x, n, FUSED_FWD_N)
    dev = inp.device
    carry = _carry_arg(carry, B, H, n, dev)
    if carry_exp is not None:
        if (carry_exp.dtype != torch.int32 or tuple(carry_exp.shape) != (B, H)
                or carry_exp.device != dev or not carry_exp.is_contiguous()):
            raise ValueError("carry_exp must be a contiguous int32 [B,H] tensor on the input's device")
    P = torch.empty((B, H, T, n, n), dtype=torch.float32, device=dev)
    E = torch.empty((B, H, T), dtype=torch.int32, device=dev) if scaled else None
    ws, ws_bytes = _workspace((B, H, T), n, DIR_FWD, chunk, dev, workspace)
    lib = load_library()
    with torch.cuda.device(dev):
        st = lib.mru_scan_fwd_ex(_ptr(inp), int(from_x), _ptr(carry), _ptr(carry_exp), _ptr(P),
                                 _ptr(E), B, H, T, n, chunk, _ptr(ws), ws_bytes, _stream_handle(dev))
    _check(st, "mru_scan_fwd_ex")
    _after_scan(ws, check, "mru_scan_fwd_ex", (B, H, T), n, DIR_FWD, chunk)
    return (P, E) if scaled else P


def scan_bwd_ex(inp: torch.Tensor, P: torch.Tensor, dP: torch.Tensor,
                carry: torch.Tensor | None = None, want_dcarry: bool = False,
                from_x: bool = False, chunk: int = 0, workspace: torch.Tensor | None = None, check: bool = False):
    """dM of sum_t <dP_t, P_t> for P_t = P_0 M_1 ... M_t (P_0 = carry, or I),
    and with want_dcarry also dL/dP_0.  P is the plain (unscaled) forward."""
    _require(P, "P", 5)
    n = P.shape[-1]
    B, H, T, n = _inshape(inp, from_x, n, FUSED_BWD_N)
    dev = inp.device
    for name, t in (("P", P), ("dP", dP)):
        _require(t, name, 5)
        if tuple(t.shape) != (B, H, T, n, n) or t.device != dev:
            raise ValueError(f"{name} must be [B,H,T,n,n] on the input's device")
    carry = _carry_arg(carry, B, H, n, dev)
    dM = torch.empty_like(P)
    dC = torch.zeros((B, H, n, n), dtype=torch.float32, device=dev) if want_dcarry else None
    ws, ws_bytes = _workspace((B, H, T), n, DIR_BWD, chunk, dev, workspace)
    lib = load_library()
    with torch.cuda.device(dev):
        st = lib.mru_scan_bwd_ex(_ptr(inp), int(from_x), _ptr(carry), _ptr(P), _ptr(dP), _ptr(dM),
                                 _ptr(dC), B, H, T, n, chunk, _ptr(ws), ws_bytes, _stream_handle(dev))
    _check(st, "mru_scan_bwd_ex")
    _after_scan(ws, check, "mru_scan_bwd_ex", (B, H, T), n, DIR_BWD, chunk)
    return (dM, dC) if want_dcarry else dM


def scan_bwd_dx(x: torch.Tensor, P: torch.Tensor, dP: torch.Tensor,
                carry: torch.Tensor | None = None, want_dcarry: bool = False, chunk: int = 0,
                out: torch.Tensor | None = None, workspace: torch.Tensor | None = None, check: bool = False):
    """dL/dx of sum_t <dP_t, P_t> for P_t = P_0 M_1 ... M_t with M_t built from
    x_t (build_inputs), in one pass: build_inputs_bwd(x, scan_bwd_x(x, P, dP))
    without forming dL/dM.  P is the forward's output on x (scan_fwd_x or
    scan_fwd_ex with the same carry).  With want_dcarry also dL/dP_0."""
    _require(P, "P", 5)
    n = P.shape[-1]
    B, H, T = _xshape(x, n)
    dev = x.device
    for name, t in (("P", P), ("dP", dP)):
        _require(t, name, 5)
        if tuple(t.shape) != (B, H, T, n, n) or t.device != dev:
            raise ValueError(f"{name} must be [B,H,T,n,n] on x's device")
    carry = _carry_arg(carry, B, H, n, dev)
    if out is None:
        out = torch.empty_like(x)
    else:
        _require(out, "out", 4)
        if out.shape != x.shape or out.device != dev:
            raise ValueError("out must match x")
    dC = torch.zeros((B, H, n, n), dtype=torch.float32, device=dev) if want_dcarry else None
    ws, ws_bytes = _workspace((B, H, T), n, DIR_BWD, chunk, dev, workspace)
    lib = load_library()
    with torch.cuda.device(dev):
        st = lib.mru_scan_bwd_dx(_ptr(x), _ptr(carry), _ptr(P), _ptr(dP), _ptr(out), _ptr(dC),
                                 B, H, T, n, chunk, _ptr(ws), ws_bytes, _stream_handle(dev))
    _check(st, "mru_scan_bwd_dx")
    _after_scan(ws, check, "mru_scan_bwd_dx", (B, H, T), n, DIR_BWD, chunk)
    return (out, dC) if want_dcarry else out


def flatten(P: torch.Tensor) -> torch.Tensor:
    """Row-major flatten of each output state matrix: [B,H,T,n,n] -> [B,H,T,n*n] view."""
    return P.view(*P.shape[:-2], P.shape[-2] * P.shape[-1])


class MRUScan(torch.autograd.Function):
    """P = scan_fwd(M) with the exact VJP from scan_bwd."""

    @staticmethod
    def forward(ctx, M: torch.Tensor, chunk: int = 0):
        M = M.contiguous()
        P = scan_fwd(M, chunk)
        ctx.save_for_backward(M, P)
        ctx.chunk = chunk
        return P

    @staticmethod
    def backward(ctx, dP: torch.Tensor):
        M, P = ctx.saved_tensors
        return scan_bwd(M, P, dP.contiguous(), ctx.chunk), None


def mru_scan(M: torch.Tensor, chunk: int = 0) -> torch.Tensor:
    return MRUScan.apply(M, chunk)


class MRUBuild(torch.autograd.Function):
    """M = build_inputs(x, n) with the exact VJP from build_inputs_bwd."""

    @staticmethod
    def forward(ctx, x: torch.Tensor, n: int):
        x = x.contiguous()
        ctx.save_for_backward(x)
        return build_inputs(x, n)

    @staticmethod
    def backward(ctx, dM: torch.Tensor):
        (x,) = ctx.saved_tensors
        return build_inputs_bwd(x, dM.contiguous()), None


class MRULayerFused(torch.autograd.Function):
    """P = scan_fwd_x(x, n); the backward goes from dL/dP to dL/dx in one pass
    (scan_bwd_dx).  Neither the input matrices nor dL/dM are ever stored."""

    @staticmethod
    def forward(ctx, x: torch.Tensor, n: int, chunk: int = 0):
        x = x.contiguous()
        P = scan_fwd_x(x, n, chunk)
        ctx.save_for_backward(x, P)
        ctx.chunk = chunk
        return P

    @staticmethod
    def backward(ctx, dP: torch.Tensor):
        x, P = ctx.saved_tensors
        return scan_bwd_dx(x, P, dP.contiguous(), chunk=ctx.chunk), None, None


def mru_layer(x: torch.Tensor, n: int, chunk: int = 0) -> torch.Tensor:
    """The MRU token mixer up to the output state matrices: x [B,H,T,n*n] ->
    P [B,H,T,n,n] (flatten() gives the output vectors), differentiable in x.
    Both scans form the input matrices on chip (n in FUSED_N: every n), and
    the backward goes from dL/dP straight to dL/dx in one pass."""
    if n in FUSED_N:
        return MRULayerFused.apply(x, n, chunk)
    return MRUScan.apply(MRUBuild.apply(x, n), chunk)
