"""libw4ec Python binding: the W4 + input-adaptive EC linear layer on MI355X.

A thin ctypes layer over the C ABI in ``include/w4ec.h`` with the same
function names.  It only marshals arguments: torch supplies device memory
and the current HIP stream; every step of the layer runs in the library's
HIP kernels.  If ``libw4ec.so`` has not been built, importing the functions
raises -- there is no fallback.

Build: ``python -m w4_gemm_error_amd.build``.
"""
from __future__ import annotations

import ctypes
import os
import re
import threading

__all__ = [
    "W4ECError", "lib", "exported_symbols", "header_symbols",
    "W4EC_OK", "W4EC_ERR_INVALID_ARG", "W4EC_ERR_UNSUPPORTED", "W4EC_ERR_WORKSPACE", "W4EC_ERR_HIP",
    "W4EC_ERR_TIMED_OUT", "W4EC_ERR_BAD_INDEX",
    "w4ec_workspace_status", "w4ec_workspace_reset", "w4ec_set_wait_limit", "w4ec_wait_limit",
    "W4EC_FP16", "W4EC_BF16", "DECODE_MAX_M", "W4EC_WS_STATE_BYTES",
    "w4ec_status_str", "w4ec_packed_bytes", "w4ec_workspace_bytes",
    "w4ec_quantize_rtn", "w4ec_pack", "w4ec_unpack",
    "w4ec_linear_decode", "w4ec_linear_prefill", "w4ec_linear",
    "w4ec_linear_decode_noalloc", "W4EC_NOALLOC_SCRATCH_BYTES",
    "w4ec_linear_decode_vgate", "w4ec_linear_prefill_vgate",
    "w4ec_prefill_ec_workspace_bytes", "w4ec_prefill_ec_gate", "w4ec_prefill_ec_apply",
    "w4ec_linear_decode_serq", "w4ec_linear_prefill_serq",
    "w4ec_pack_xfp", "w4ec_linear_decode_xfp", "w4ec_linear_decode_xfp_lib", "W4EC_XFP_LIB_MAX",
    "w4ec_stream_read",
    "PackedLayer",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libw4ec.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "w4ec.h")

W4EC_OK = 0
W4EC_ERR_INVALID_ARG = -1
W4EC_ERR_UNSUPPORTED = -2
W4EC_ERR_WORKSPACE = -3
W4EC_ERR_HIP = -4
W4EC_ERR_TIMED_OUT = -5
W4EC_ERR_BAD_INDEX = -6
W4EC_FP16 = 0
W4EC_BF16 = 1
DECODE_MAX_M = 16
W4EC_WS_STATE_BYTES = 16 << 20   # leading workspace bytes every call returns to zero
W4EC_NOALLOC_SCRATCH_BYTES = 4 << 20   # the static device array of w4ec_linear_decode_noalloc

_lock = threading.Lock()
_lib = None


class W4ECError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {w4ec_status_str(status)} ({status})")


def lib() -> ctypes.CDLL:
    """Load libw4ec.so (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m w4_gemm_error_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I, F, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        L.w4ec_status_str.argtypes = [I]
        L.w4ec_status_str.restype = ctypes.c_char_p
        L.w4ec_packed_bytes.argtypes = [I, I, I]
        L.w4ec_packed_bytes.restype = Z
        L.w4ec_workspace_bytes.argtypes = [I, I, I, I, I]
        L.w4ec_workspace_bytes.restype = Z
        L.w4ec_workspace_status.argtypes = [P, Z, P]
        L.w4ec_workspace_status.restype = I
        L.w4ec_workspace_reset.argtypes = [P, Z, P]
        L.w4ec_workspace_reset.restype = I
        L.w4ec_stream_read.argtypes = [P, Z, P, P]
        L.w4ec_stream_read.restype = I
        L.w4ec_set_wait_limit.argtypes = [ctypes.c_uint32]
        L.w4ec_set_wait_limit.restype = None
        L.w4ec_wait_limit.argtypes = []
        L.w4ec_wait_limit.restype = ctypes.c_uint32
        L.w4ec_quantize_rtn.argtypes = [P, I, I, I, P, P, P, P]
        L.w4ec_quantize_rtn.restype = I
        L.w4ec_pack.argtypes = [P, P, P, I, I, I, P, P]
        L.w4ec_pack.restype = I
        L.w4ec_unpack.argtypes = [P, I, I, I, P, P, P, P]
        L.w4ec_unpack.restype = I
        for name in ("w4ec_linear_decode", "w4ec_linear_prefill"):
            fn = getattr(L, name)
            fn.argtypes = [P, P, P, P, P, F, P, I, I, I, I, I, I, P, Z, P]
            fn.restype = I
        L.w4ec_linear_decode_noalloc.argtypes = [P, P, P, P, P, F, P, I, I, I, I, I, I, P]
        L.w4ec_linear_decode_noalloc.restype = I
        L.w4ec_prefill_ec_workspace_bytes.argtypes = [I, I, I]
        L.w4ec_prefill_ec_workspace_bytes.restype = Z
        L.w4ec_prefill_ec_gate.argtypes = [P, P, P, F, I, I, I, I, P, Z, P]
        L.w4ec_prefill_ec_gate.restype = I
        L.w4ec_prefill_ec_apply.argtypes = [P, P, I, I, I, I, I, P, Z, P]
        L.w4ec_prefill_ec_apply.restype = I
        for name in ("w4ec_linear_decode_serq", "w4ec_linear_prefill_serq"):
            fn = getattr(L, name)
            fn.argtypes = [P, P, P, P, P, I, I, I, I, I, I, P, Z, P]
            fn.restype = I
        L.w4ec_pack_xfp.argtypes = [P, I, I, P, P]
        L.w4ec_pack_xfp.restype = I
        L.w4ec_linear_decode_xfp.argtypes = [P, P, P, P, P, P, I, P, I, I, I, I, P]
        L.w4ec_linear_decode_xfp.restype = I
        L.w4ec_linear_decode_xfp_lib.argtypes = [P, P, P, I, P, P, P, P, I, P, I, I, I, I, P]
        L.w4ec_linear_decode_xfp_lib.restype = I
        for name in ("w4ec_linear_decode_vgate", "w4ec_linear_prefill_vgate"):
            fn = getattr(L, name)
            fn.argtypes = [P, P, P, P, P, P, P, P, I, P, I, I, I, I, I, I, P, Z, P]
            fn.restype = I
        _lib = L
        return L


def header_symbols() -> list:
    """Function names declared in include/w4ec.h."""
    text = open(HEADER_PATH).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(w4ec_[a-z_]+)\s*\(", text)))


def exported_symbols() -> list:
    L = lib()
    return [s for s in header_symbols() if hasattr(L, s)]


# ---------------------------------------------------------------- host-only calls

def w4ec_status_str(status: int) -> str:
    return lib().w4ec_status_str(int(status)).decode()


def w4ec_packed_bytes(N: int, K: int, group_size: int) -> int:
    return int(lib().w4ec_packed_bytes(N, K, group_size))


def w4ec_workspace_bytes(M: int, N: int, K: int, r: int, group_size: int) -> int:
    return int(lib().w4ec_workspace_bytes(M, N, K, r, group_size))


def w4ec_set_wait_limit(polls: int) -> None:
    """Polls a bounded wait makes before it gives up (0: every wait gives up
    at once, for exercising the failure path)."""
    lib().w4ec_set_wait_limit(int(polls))


def w4ec_wait_limit() -> int:
    return int(lib().w4ec_wait_limit())


# ---------------------------------------------------------------- device calls

def _torch():
    import torch
    return torch


def _stream_handle(stream=None):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(status: int, what: str):
    if status != W4EC_OK:
        raise W4ECError(status, what)


def _need_cuda(t, name, dtype=None):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")


def _act_code(dtype) -> int:
    torch = _torch()
    if dtype == torch.float16:
        return W4EC_FP16
    if dtype == torch.bfloat16:
        return W4EC_BF16
    raise ValueError(f"activation dtype {dtype} is not fp16/bf16")


def w4ec_workspace_status(workspace, *, stream=None) -> int:
    """W4EC_OK, W4EC_ERR_TIMED_OUT or W4EC_ERR_BAD_INDEX: what the calls so
    far on this workspace recorded (synchronizes the stream)."""
    _need_cuda(workspace, "workspace")
    st = lib().w4ec_workspace_status(_ptr(workspace), workspace.numel() * workspace.element_size(),
                                     _stream_handle(stream))
    if st not in (W4EC_OK, W4EC_ERR_TIMED_OUT, W4EC_ERR_BAD_INDEX):
        raise W4ECError(st, "w4ec_workspace_status")
    return int(st)


def w4ec_workspace_reset(workspace, *, stream=None) -> None:
    """Zero the workspace's hand-over state (asynchronous, a kernel)."""
    _need_cuda(workspace, "workspace")
    _check(lib().w4ec_workspace_reset(_ptr(workspace), workspace.numel() * workspace.element_size(),
                                      _stream_handle(stream)), "w4ec_workspace_reset")


def w4ec_stream_read(src, sink, *, nbytes=None, stream=None) -> None:
    """The library's streaming-read reference kernel over the first nbytes
    (default: all) of src; one XOR word per workgroup into sink (uint32 or
    int32, 512 elements).  A measurement hook: the attainable HBM read time."""
    _need_cuda(src, "src")
    _need_cuda(sink, "sink")
    n = src.numel() * src.element_size() if nbytes is None else int(nbytes)
    if sink.numel() * sink.element_size() < 512 * 4:
        raise ValueError("sink holds 512 32-bit words")
    _check(lib().w4ec_stream_read(_ptr(src), n, _ptr(sink), _stream_handle(stream)), "w4ec_stream_read")


def w4ec_quantize_rtn(W, group_size: int, *, stream=None):
    """RTN int4 on the GPU: W float32 [N, K] -> (codes uint8 [N, K/2],
    scale fp16 [N, K/G], zero fp16 [N, K/G])."""
    torch = _torch()
    _need_cuda(W, "W", torch.float32)
    N, K = W.shape
    G = int(group_size)
    q = torch.empty((N, K // 2), dtype=torch.uint8, device=W.device)
    s = torch.empty((N, K // G), dtype=torch.float16, device=W.device)
    z = torch.empty((N, K // G), dtype=torch.float16, device=W.device)
    _check(lib().w4ec_quantize_rtn(_ptr(W), N, K, G, _ptr(q), _ptr(s), _ptr(z), _stream_handle(stream)),
           "w4ec_quantize_rtn")
    return q, s, z


def w4ec_pack(q_canon, scale, zero, N: int, K: int, group_size: int, *, packed=None, stream=None):
    """Canonical codes + fp16 scale/zero -> device blob (uint8 tensor).  Synchronizes the stream."""
    torch = _torch()
    _need_cuda(q_canon, "q_canon", torch.uint8)
    _need_cuda(scale, "scale", torch.float16)
    _need_cuda(zero, "zero", torch.float16)
    nbytes = w4ec_packed_bytes(N, K, group_size)
    if nbytes == 0:
        raise W4ECError(W4EC_ERR_UNSUPPORTED, "w4ec_packed_bytes")
    if packed is None:
        packed = torch.empty(nbytes, dtype=torch.uint8, device=q_canon.device)
    _check(lib().w4ec_pack(_ptr(q_canon), _ptr(scale), _ptr(zero), N, K, group_size, _ptr(packed),
                           _stream_handle(stream)), "w4ec_pack")
    return packed


def w4ec_unpack(packed, N: int, K: int, group_size: int, *, stream=None):
    torch = _torch()
    _need_cuda(packed, "packed", torch.uint8)
    G = int(group_size)
    q = torch.empty((N, K // 2), dtype=torch.uint8, device=packed.device)
    s = torch.empty((N, K // G), dtype=torch.float16, device=packed.device)
    z = torch.empty((N, K // G), dtype=torch.float16, device=packed.device)
    _check(lib().w4ec_unpack(_ptr(packed), N, K, G, _ptr(q), _ptr(s), _ptr(z), _stream_handle(stream)),
           "w4ec_unpack")
    return q, s, z


def _layer_call(name, X, packed, A, B, w_g, b_g, N, group_size, workspace, Y, stream):
    torch = _torch()
    acts = (torch.float16, torch.bfloat16)
    _need_cuda(X, "X", acts)
    act = X.dtype
    M, K = X.shape
    r = 0 if A is None else int(A.shape[1])
    for t, nm in ((A, "A"), (B, "B"), (w_g, "w_g")):
        _need_cuda(t, nm, act)
    _need_cuda(packed, "packed", torch.uint8)
    if Y is None:
        Y = torch.empty((M, N), dtype=act, device=X.device)
    _need_cuda(Y, "Y", act)
    if workspace is None:
        nb = w4ec_workspace_bytes(M, N, K, r, group_size)
        workspace = torch.zeros(max(nb, 256), dtype=torch.uint8, device=X.device)
    fn = getattr(lib(), name)
    st = fn(_ptr(X), _ptr(packed), _ptr(A), _ptr(B), _ptr(w_g), float(b_g), _ptr(Y),
            M, N, K, r, int(group_size), _act_code(act), _ptr(workspace), workspace.numel(),
            _stream_handle(stream))
    _check(st, name)
    return Y


def _layer_call_vgate(name, X, packed, A, B, G1, c1, G2, c2, N, group_size, workspace, Y, stream):
    torch = _torch()
    acts = (torch.float16, torch.bfloat16)
    _need_cuda(X, "X", acts)
    act = X.dtype
    M, K = X.shape
    r = 0 if A is None else int(A.shape[1])
    for t, nm in ((A, "A"), (B, "B"), (G1, "G1"), (c1, "c1"), (G2, "G2"), (c2, "c2")):
        _need_cuda(t, nm, act)
    h = 0 if G1 is None else int(G1.shape[1])
    _need_cuda(packed, "packed", torch.uint8)
    if Y is None:
        Y = torch.empty((M, N), dtype=act, device=X.device)
    _need_cuda(Y, "Y", act)
    if workspace is None:
        nb = w4ec_workspace_bytes(M, N, K, r, group_size)
        workspace = torch.zeros(max(nb, 256), dtype=torch.uint8, device=X.device)
    fn = getattr(lib(), name)
    st = fn(_ptr(X), _ptr(packed), _ptr(A), _ptr(B), _ptr(G1), _ptr(c1), _ptr(G2), _ptr(c2), h,
            _ptr(Y), M, N, K, r, int(group_size), _act_code(act), _ptr(workspace), workspace.numel(),
            _stream_handle(stream))
    _check(st, name)
    return Y


def w4ec_linear_decode_vgate(X, packed, A, B, G1, c1, G2, c2, *, N, group_size, workspace=None, Y=None,
                             stream=None):
    """Y = X Wd^T + (gamma * (X A)) B, gamma = sigmoid(relu((X A) G1 + c1) G2 + c2), 1 <= M <= 16."""
    return _layer_call_vgate("w4ec_linear_decode_vgate", X, packed, A, B, G1, c1, G2, c2, N, group_size,
                             workspace, Y, stream)


def w4ec_linear_prefill_vgate(X, packed, A, B, G1, c1, G2, c2, *, N, group_size, workspace=None, Y=None,
                              stream=None):
    """The vector-gate layer for any M >= 1 (prepass, per-token bottleneck, tiled MFMA GEMM)."""
    return _layer_call_vgate("w4ec_linear_prefill_vgate", X, packed, A, B, G1, c1, G2, c2, N, group_size,
                             workspace, Y, stream)


def _layer_call_serq(name, X, packed, S, R, N, group_size, workspace, Y, stream):
    torch = _torch()
    _need_cuda(X, "X", (torch.float16, torch.bfloat16))
    act = X.dtype
    M, K = X.shape
    s = 0 if R is None else int(R.shape[0])
    _need_cuda(S, "S", torch.int32)
    _need_cuda(R, "R", act)
    _need_cuda(packed, "packed", torch.uint8)
    if Y is None:
        Y = torch.empty((M, N), dtype=act, device=X.device)
    _need_cuda(Y, "Y", act)
    if workspace is None:
        nb = w4ec_workspace_bytes(M, N, K, s, group_size)
        workspace = torch.zeros(max(nb, 256), dtype=torch.uint8, device=X.device)
    st = getattr(lib(), name)(_ptr(X), _ptr(packed), _ptr(S), _ptr(R), _ptr(Y), M, N, K, s, int(group_size),
                              _act_code(act), _ptr(workspace), workspace.numel(), _stream_handle(stream))
    _check(st, name)
    return Y


def w4ec_linear_decode_serq(X, packed, S, R, *, N, group_size, workspace=None, Y=None, stream=None):
    """Y = X Wd^T + X[:, S] R (salient-channel correction), 1 <= M <= 16; S int32 [s], R [s, N]."""
    return _layer_call_serq("w4ec_linear_decode_serq", X, packed, S, R, N, group_size, workspace, Y, stream)


def w4ec_linear_prefill_serq(X, packed, S, R, *, N, group_size, workspace=None, Y=None, stream=None):
    """Y = X Wd^T + X[:, S] R (salient-channel correction) for any M >= 1."""
    return _layer_call_serq("w4ec_linear_prefill_serq", X, packed, S, R, N, group_size, workspace, Y, stream)


def w4ec_pack_xfp(idx_canon, N: int, K: int, *, packed=None, stream=None):
    """Codebook indices, canonical uint8 [N, K/2] (even k in the low nibble)
    -> the codebook blob that w4ec_linear_decode_xfp reads.  Synchronizes."""
    torch = _torch()
    _need_cuda(idx_canon, "idx_canon", torch.uint8)
    nbytes = w4ec_packed_bytes(N, K, K)
    if nbytes == 0:
        raise W4ECError(W4EC_ERR_UNSUPPORTED, "w4ec_packed_bytes")
    if packed is None:
        packed = torch.empty(nbytes, dtype=torch.uint8, device=idx_canon.device)
    _check(lib().w4ec_pack_xfp(_ptr(idx_canon), N, K, _ptr(packed), _stream_handle(stream)), "w4ec_pack_xfp")
    return packed


def w4ec_linear_decode_xfp(X, packed, codebook, row_ptr, col_idx, val, *, N, Y=None, stream=None):
    """Y = X Wh^T with Wh[n,k] = codebook[n][idx[n,k]] plus the sparse residual
    (rows row_ptr, columns col_idx, values val), 1 <= M <= 16.  packed: the
    indices packed by w4ec_pack_xfp;
    codebook fp16 [N, 16]; row_ptr int32 [N + 1]; col_idx int32 [nnz]; val fp16 [nnz]."""
    torch = _torch()
    _need_cuda(X, "X", (torch.float16, torch.bfloat16))
    act = X.dtype
    M, K = X.shape
    _need_cuda(packed, "packed", torch.uint8)
    _need_cuda(codebook, "codebook", torch.float16)
    _need_cuda(row_ptr, "row_ptr", torch.int32)
    _need_cuda(col_idx, "col_idx", torch.int32)
    _need_cuda(val, "val", torch.float16)
    if codebook.shape != (N, 16) or row_ptr.shape != (N + 1,):
        raise ValueError("codebook must be [N, 16] and row_ptr [N + 1]")
    nnz = 0 if col_idx is None else int(col_idx.numel())
    if (val is None and nnz) or (val is not None and int(val.numel()) != nnz):
        raise ValueError("col_idx and val must have the same length")
    if Y is None:
        Y = torch.empty((M, N), dtype=act, device=X.device)
    _need_cuda(Y, "Y", act)
    st = lib().w4ec_linear_decode_xfp(_ptr(X), _ptr(packed), _ptr(codebook), _ptr(row_ptr),
                                      _ptr(col_idx) if nnz else None, _ptr(val) if nnz else None, nnz,
                                      _ptr(Y), M, N, K, _act_code(act), _stream_handle(stream))
    _check(st, "w4ec_linear_decode_xfp")
    return Y


W4EC_XFP_LIB_MAX = 32


def w4ec_linear_decode_xfp_lib(X, packed, library, libid, row_ptr, col_idx, val, *, N, Y=None, stream=None):
    """Y = X Wh^T with Wh[n,k] = library[libid[n, k // 128]][idx[n,k]] plus the
    sparse residual, 1 <= M <= 16.  packed: the indices packed by
    w4ec_pack_xfp; library fp16 [L, 16] (1 <= L <= 32); libid uint8 [N, K/128];
    row_ptr int32 [N + 1]; col_idx int32 [nnz]; val fp16 [nnz]."""
    torch = _torch()
    _need_cuda(X, "X", (torch.float16, torch.bfloat16))
    act = X.dtype
    M, K = X.shape
    _need_cuda(packed, "packed", torch.uint8)
    _need_cuda(library, "library", torch.float16)
    _need_cuda(libid, "libid", torch.uint8)
    _need_cuda(row_ptr, "row_ptr", torch.int32)
    _need_cuda(col_idx, "col_idx", torch.int32)
    _need_cuda(val, "val", torch.float16)
    L = int(library.shape[0])
    if library.dim() != 2 or library.shape[1] != 16 or libid.shape != (N, K // 128) or row_ptr.shape != (N + 1,):
        raise ValueError("library must be [L, 16], libid [N, K/128] and row_ptr [N + 1]")
    nnz = 0 if col_idx is None else int(col_idx.numel())
    if (val is None and nnz) or (val is not None and int(val.numel()) != nnz):
        raise ValueError("col_idx and val must have the same length")
    if Y is None:
        Y = torch.empty((M, N), dtype=act, device=X.device)
    _need_cuda(Y, "Y", act)
    st = lib().w4ec_linear_decode_xfp_lib(_ptr(X), _ptr(packed), _ptr(library), L, _ptr(libid), _ptr(row_ptr),
                                          _ptr(col_idx) if nnz else None, _ptr(val) if nnz else None, nnz,
                                          _ptr(Y), M, N, K, _act_code(act), _stream_handle(stream))
    _check(st, "w4ec_linear_decode_xfp_lib")
    return Y


def w4ec_prefill_ec_workspace_bytes(M: int, K: int, r: int) -> int:
    return int(lib().w4ec_prefill_ec_workspace_bytes(int(M), int(K), int(r)))


def w4ec_prefill_ec_gate(X, A, w_g, b_g, *, workspace, stream=None):
    """T_g = g * (X A) into `workspace` (the EC half of the unfused prefill)."""
    torch = _torch()
    _need_cuda(X, "X", (torch.float16, torch.bfloat16))
    _need_cuda(A, "A", X.dtype)
    _need_cuda(w_g, "w_g", X.dtype)
    M, K = X.shape
    r = int(A.shape[1])
    st = lib().w4ec_prefill_ec_gate(_ptr(X), _ptr(A), _ptr(w_g), float(b_g), M, K, r, _act_code(X.dtype),
                                    _ptr(workspace), workspace.numel(), _stream_handle(stream))
    _check(st, "w4ec_prefill_ec_gate")


def w4ec_prefill_ec_apply(Y, B, *, K, workspace, stream=None):
    """Y += T_g B, with T_g from the last w4ec_prefill_ec_gate on `workspace`."""
    torch = _torch()
    _need_cuda(Y, "Y", (torch.float16, torch.bfloat16))
    _need_cuda(B, "B", Y.dtype)
    M, N = Y.shape
    r = int(B.shape[0])
    st = lib().w4ec_prefill_ec_apply(_ptr(Y), _ptr(B), M, N, int(K), r, _act_code(Y.dtype),
                                     _ptr(workspace), workspace.numel(), _stream_handle(stream))
    _check(st, "w4ec_prefill_ec_apply")


def w4ec_linear_decode(X, packed, A, B, w_g, b_g, *, N, group_size, workspace=None, Y=None, stream=None):
    """Y = X Wd^T + g (X A) B for 1 <= M <= 16 tokens (one kernel launch)."""
    return _layer_call("w4ec_linear_decode", X, packed, A, B, w_g, b_g, N, group_size, workspace, Y, stream)


def w4ec_linear_decode_noalloc(X, packed, A, B, w_g, b_g, *, N, group_size, Y=None, stream=None):
    """w4ec_linear_decode with no workspace and no allocation in the library
    (its state in a static device array; calls on one GPU must not overlap)."""
    torch = _torch()
    acts = (torch.float16, torch.bfloat16)
    _need_cuda(X, "X", acts)
    act = X.dtype
    M, K = X.shape
    r = 0 if A is None else int(A.shape[1])
    for t, nm in ((A, "A"), (B, "B"), (w_g, "w_g")):
        _need_cuda(t, nm, act)
    _need_cuda(packed, "packed", torch.uint8)
    if Y is None:
        Y = torch.empty((M, N), dtype=act, device=X.device)
    _need_cuda(Y, "Y", act)
    st = lib().w4ec_linear_decode_noalloc(_ptr(X), _ptr(packed), _ptr(A), _ptr(B), _ptr(w_g), float(b_g), _ptr(Y),
                                          M, N, K, r, int(group_size), _act_code(act), _stream_handle(stream))
    _check(st, "w4ec_linear_decode_noalloc")
    return Y


def w4ec_linear_prefill(X, packed, A, B, w_g, b_g, *, N, group_size, workspace=None, Y=None, stream=None):
    """Y = X Wd^T + g (X A) B for any M >= 1 (prepass + tiled MFMA GEMM)."""
    return _layer_call("w4ec_linear_prefill", X, packed, A, B, w_g, b_g, N, group_size, workspace, Y, stream)


def w4ec_linear(X, packed, A, B, w_g, b_g, *, N, group_size, workspace=None, Y=None, stream=None):
    """Phase-adaptive dispatch: decode kernel for M <= 16 tokens, prefill otherwise."""
    fn = w4ec_linear_decode if X.shape[0] <= DECODE_MAX_M else w4ec_linear_prefill
    return fn(X, packed, A, B, w_g, b_g, N=N, group_size=group_size, workspace=workspace, Y=Y, stream=stream)


class PackedLayer:
    """A quantized layer held on the GPU: packed weights, EC parameters and a
    reusable (zero-initialised) workspace sized for the largest M seen."""

    def __init__(self, packed, A, B, w_g, b_g, *, N, K, group_size):
        self.packed, self.A, self.B, self.w_g, self.b_g = packed, A, B, w_g, float(b_g)
        self.N, self.K, self.group_size = int(N), int(K), int(group_size)
        self.r = 0 if A is None else int(A.shape[1])
        self._ws = None

    @classmethod
    def from_float(cls, W, A, B, w_g, b_g, *, group_size, stream=None):
        N, K = W.shape
        q, s, z = w4ec_quantize_rtn(W, group_size, stream=stream)
        packed = w4ec_pack(q, s, z, N, K, group_size, stream=stream)
        return cls(packed, A, B, w_g, b_g, N=N, K=K, group_size=group_size)

    def workspace(self, M):
        torch = _torch()
        nb = max(w4ec_workspace_bytes(M, self.N, self.K, self.r, self.group_size), 256)
        if self._ws is None or self._ws.numel() < nb:
            self._ws = torch.zeros(nb, dtype=torch.uint8, device=self.packed.device)
        return self._ws

    def __call__(self, X, *, Y=None, phase=None, stream=None):
        M = X.shape[0]
        ws = self.workspace(M)
        if phase is None:
            phase = "decode" if M <= DECODE_MAX_M else "prefill"
        fn = w4ec_linear_decode if phase == "decode" else w4ec_linear_prefill
        return fn(X, self.packed, self.A, self.B, self.w_g, self.b_g, N=self.N,
                  group_size=self.group_size, workspace=ws, Y=Y, stream=stream)
