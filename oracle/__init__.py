"""Float64 CPU oracle for the W4 + input-adaptive EC linear layer.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import this
package: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` use it.  It shares no code with the HIP library
(``w4_gemm_error_amd``) and imports nothing from it.

The arithmetic lives in ``w4ec_oracle.c`` (plain C, float64, naive loops);
this module builds it with gcc and marshals numpy arrays through ctypes.
Method: SPEAR (gist.science technical summary), section 2.1A, effective
weight W + B diag(gate) A with a per-token scalar gate sigmoid(x.w_g + b_g)
(``forward``), or with one gate per rank component from a bottleneck MLP on
T = X A (``forward_vgate``); the quantizer is the per-channel RTN baseline of
its results section 3.1.  ``forward_serq`` is the single-factor correction
over salient input channels of the SERQ summary (section 2); ``forward_xfp``
the per-channel codebook weights with a sparse outlier residual of the XFP
summary (section 2), and ``forward_xfp_lib`` its shared-library mode (one
library of codebooks per layer, an entry per group of 128 weights).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "w4ec_oracle.c")
_BUILD_DIR = os.path.join(_HERE, "_build")
# W4EC_ORACLE_SANITIZE=1 builds and loads a copy instrumented with
# AddressSanitizer and UndefinedBehaviorSanitizer (the process must then
# preload the ASan runtime; tests/test_sanitizers.py runs the pins that way)
_SANITIZE = os.environ.get("W4EC_ORACLE_SANITIZE") == "1"
_LIB_PATH = os.path.join(_BUILD_DIR, "libw4ec_oracle_san.so" if _SANITIZE else "libw4ec_oracle.so")

_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no fast-math, no FMA contraction)."""
    os.makedirs(_BUILD_DIR, exist_ok=True)
    if not force and os.path.exists(_LIB_PATH) and os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC):
        return _LIB_PATH   # built from the current source
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-std=c11", "-Wall", "-o", tmp, _SRC, "-lm"]
    if _SANITIZE:
        cmd[1:2] = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        build(force=False)    # (only when missing or older than the source)
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        I = ctypes.c_int
        lib.w4o_half_to_double.argtypes = [ctypes.c_uint16]
        lib.w4o_half_to_double.restype = ctypes.c_double
        lib.w4o_bf16_to_double.argtypes = [ctypes.c_uint16]
        lib.w4o_bf16_to_double.restype = ctypes.c_double
        lib.w4o_double_to_half.argtypes = [ctypes.c_double]
        lib.w4o_double_to_half.restype = ctypes.c_uint16
        lib.w4o_unpack_codes.argtypes = [P, I, I, P]
        lib.w4o_unpack_codes.restype = None
        lib.w4o_rtn_quantize.argtypes = [P, I, I, I, P, P, P]
        lib.w4o_rtn_quantize.restype = None
        lib.w4o_forward.argtypes = [I, I, I, I, I, I, P, P, P, P, P, P, P,
                                    ctypes.c_double, P, I, P, P, P, P, P]
        lib.w4o_forward.restype = I
        lib.w4o_forward_vgate.argtypes = [I, I, I, I, I, I, I, P, P, P, P, P, P, P, P, P, P,
                                          P, I, P, P, P, P, P]
        lib.w4o_forward_vgate.restype = I
        lib.w4o_forward_serq.argtypes = [I, I, I, I, I, I, P, P, P, P, P, P, P, I, P, P, P]
        lib.w4o_forward_serq.restype = I
        lib.w4o_forward_xfp.argtypes = [I, I, I, I, P, P, P, P, P, P, P, I, P]
        lib.w4o_forward_xfp.restype = I
        lib.w4o_forward_xfp_lib.argtypes = [I, I, I, I, P, P, P, I, P, P, P, P, P, I, P]
        lib.w4o_forward_xfp_lib.restype = I
        lib.w4o_max_threads.argtypes = []
        lib.w4o_max_threads.restype = I
        _lib = lib
        return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def max_threads() -> int:
    return int(_load().w4o_max_threads())


def half_to_double(bits) -> float:
    return float(_load().w4o_half_to_double(int(bits)))


def bf16_to_double(bits) -> float:
    return float(_load().w4o_bf16_to_double(int(bits)))


def double_to_half(x: float) -> int:
    return int(_load().w4o_double_to_half(float(x)))


def act_to_f64(bits: np.ndarray, act: str) -> np.ndarray:
    """Exact widening of fp16 / bf16 bit patterns (uint16) to float64."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    if act == "fp16":
        return bits.view(np.float16).astype(np.float64)
    if act == "bf16":
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    raise ValueError(act)


def unpack_codes(qc: np.ndarray, N: int, K: int) -> np.ndarray:
    """Canonical codes uint8 [N, K/2] -> one code per element, uint8 [N, K]."""
    qc = _c(qc, np.uint8)
    assert qc.shape == (N, K // 2)
    q = np.empty((N, K), dtype=np.uint8)
    _load().w4o_unpack_codes(_ptr(qc), N, K, _ptr(q))
    return q


def rtn_quantize(W: np.ndarray, group_size: int):
    """RTN asymmetric int4: W float32 [N, K] -> (codes u8 [N, K/2], scale, zero)
    with scale and zero as fp16 bit patterns (uint16) [N, K/G]."""
    W = _c(W, np.float32)
    N, K = W.shape
    G = int(group_size)
    assert K % G == 0 and K % 2 == 0
    qc = np.empty((N, K // 2), dtype=np.uint8)
    s = np.empty((N, K // G), dtype=np.uint16)
    z = np.empty((N, K // G), dtype=np.uint16)
    _load().w4o_rtn_quantize(_ptr(W), N, K, G, _ptr(qc), _ptr(s), _ptr(z))
    return qc, s, z


def forward(X, qc, scale, zero, A, B, w_g, b_g, *, N, K, r, group_size,
            act="fp16", rows=None, want_parts=True):
    """Evaluate the layer in float64 for all tokens or for the listed rows.

    X: act bits uint16 [M, K]; qc: uint8 [N, K/2]; scale/zero: fp16 bits
    uint16 [N, K/G]; A: act bits [K, r]; B: act bits [r, N]; w_g: act bits
    [K] or None; b_g: float.  Returns a dict with Y (and Y0, T, g, C when
    want_parts) as float64 arrays indexed by the evaluated rows.
    """
    lib = _load()
    X = _c(X, np.uint16)
    M = X.shape[0]
    assert X.shape == (M, K)
    qc = _c(qc, np.uint8)
    scale = _c(scale, np.uint16)
    zero = _c(zero, np.uint16)
    G = int(group_size)
    assert qc.shape == (N, K // 2) and scale.shape == (N, K // G) and zero.shape == (N, K // G)
    if r > 0:
        A = _c(A, np.uint16)
        B = _c(B, np.uint16)
        assert A.shape == (K, r) and B.shape == (r, N)
    else:
        A = np.zeros((1,), np.uint16)
        B = np.zeros((1,), np.uint16)
    w_g = _c(w_g, np.uint16)
    if w_g is not None:
        assert w_g.shape == (K,)
    rows_arr = None
    n_rows = M
    if rows is not None:
        rows_arr = np.ascontiguousarray(rows, dtype=np.int32)
        n_rows = int(rows_arr.shape[0])
    Y = np.empty((n_rows, N), np.float64)
    Y0 = np.empty((n_rows, N), np.float64) if want_parts else None
    C = np.empty((n_rows, N), np.float64) if want_parts else None
    T = np.empty((n_rows, max(r, 0)), np.float64) if want_parts else None
    g = np.empty((n_rows,), np.float64) if want_parts else None
    act_bf16 = {"fp16": 0, "bf16": 1}[act]
    rc = lib.w4o_forward(M, N, K, r, G, act_bf16, _ptr(X), _ptr(qc), _ptr(scale),
                         _ptr(zero), _ptr(A), _ptr(B), _ptr(w_g), float(b_g),
                         _ptr(rows_arr), n_rows, _ptr(Y), _ptr(Y0), _ptr(T),
                         _ptr(g), _ptr(C))
    if rc != 0:
        raise RuntimeError("oracle forward failed (bad arguments)")
    out = {"Y": Y}
    if want_parts:
        out.update(Y0=Y0, T=T, g=g, C=C)
    return out



def forward_vgate(X, qc, scale, zero, A, B, G1, c1, G2, c2, *, N, K, r, h, group_size,
                  act="fp16", rows=None, want_parts=True):
    """The layer with a vector gate (one gate per rank component, from a
    bottleneck MLP of width h on T = X A), in float64; see w4o_forward_vgate.

    G1: act bits [r, h]; c1: act bits [h]; G2: act bits [h, r]; c2: act bits
    [r].  Other arguments as forward().  Returns Y (and Y0, T, gamma, C when
    want_parts) indexed by the evaluated rows.
    """
    lib = _load()
    X = _c(X, np.uint16)
    M = X.shape[0]
    assert X.shape == (M, K) and r > 0 and h > 0
    qc = _c(qc, np.uint8)
    scale = _c(scale, np.uint16)
    zero = _c(zero, np.uint16)
    G = int(group_size)
    assert qc.shape == (N, K // 2) and scale.shape == (N, K // G) and zero.shape == (N, K // G)
    A, B = _c(A, np.uint16), _c(B, np.uint16)
    G1, c1, G2, c2 = _c(G1, np.uint16), _c(c1, np.uint16), _c(G2, np.uint16), _c(c2, np.uint16)
    assert A.shape == (K, r) and B.shape == (r, N)
    assert G1.shape == (r, h) and c1.shape == (h,) and G2.shape == (h, r) and c2.shape == (r,)
    rows_arr = None
    n_rows = M
    if rows is not None:
        rows_arr = np.ascontiguousarray(rows, dtype=np.int32)
        n_rows = int(rows_arr.shape[0])
    Y = np.empty((n_rows, N), np.float64)
    Y0 = np.empty((n_rows, N), np.float64) if want_parts else None
    C = np.empty((n_rows, N), np.float64) if want_parts else None
    T = np.empty((n_rows, r), np.float64) if want_parts else None
    gam = np.empty((n_rows, r), np.float64) if want_parts else None
    act_bf16 = {"fp16": 0, "bf16": 1}[act]
    rc = lib.w4o_forward_vgate(M, N, K, r, G, act_bf16, h, _ptr(X), _ptr(qc), _ptr(scale),
                               _ptr(zero), _ptr(A), _ptr(B), _ptr(G1), _ptr(c1), _ptr(G2),
                               _ptr(c2), _ptr(rows_arr), n_rows, _ptr(Y), _ptr(Y0), _ptr(T),
                               _ptr(gam), _ptr(C))
    if rc != 0:
        raise RuntimeError("oracle forward_vgate failed (bad arguments)")
    out = {"Y": Y}
    if want_parts:
        out.update(Y0=Y0, T=T, gamma=gam, C=C)
    return out


def forward_serq(X, qc, scale, zero, S, R, *, N, K, group_size, act="fp16", rows=None, want_parts=True):
    """Y = X Wd^T + X[:, S] R in float64 (see w4o_forward_serq).  S: int32
    [s] input-channel indices in [0, K); R: act bits [s, N]."""
    lib = _load()
    X = _c(X, np.uint16)
    M = X.shape[0]
    assert X.shape == (M, K)
    qc, scale, zero = _c(qc, np.uint8), _c(scale, np.uint16), _c(zero, np.uint16)
    G = int(group_size)
    assert qc.shape == (N, K // 2) and scale.shape == (N, K // G) and zero.shape == (N, K // G)
    S = np.zeros((1,), np.int32) if S is None else _c(S, np.int32)
    s = 0 if R is None else int(np.asarray(R).shape[0])
    R = np.zeros((1,), np.uint16) if R is None else _c(R, np.uint16)
    if s > 0:
        assert S.shape == (s,) and R.shape == (s, N)
    rows_arr = None
    n_rows = M
    if rows is not None:
        rows_arr = np.ascontiguousarray(rows, dtype=np.int32)
        n_rows = int(rows_arr.shape[0])
    Y = np.empty((n_rows, N), np.float64)
    Y0 = np.empty((n_rows, N), np.float64) if want_parts else None
    C = np.empty((n_rows, N), np.float64) if want_parts else None
    act_bf16 = {"fp16": 0, "bf16": 1}[act]
    rc = lib.w4o_forward_serq(M, N, K, s, G, act_bf16, _ptr(X), _ptr(qc), _ptr(scale), _ptr(zero),
                              _ptr(S), _ptr(R), _ptr(rows_arr), n_rows, _ptr(Y), _ptr(Y0), _ptr(C))
    if rc != 0:
        raise RuntimeError("oracle forward_serq failed (bad arguments)")
    out = {"Y": Y}
    if want_parts:
        out.update(Y0=Y0, C=C)
    return out


def forward_xfp(X, qc, cb, row_ptr, col_idx, val, *, N, K, act="fp16", rows=None):
    """Y = X Wh^T with Wh[n,k] = cb[n][idx[n,k]] + (sparse residual)[n,k]
    (see w4o_forward_xfp).  qc: 4-bit indices uint8 [N, K/2]; cb: fp16 bits
    [N, 16]; row_ptr int32 [N+1], col_idx int32 [nnz], val fp16 bits [nnz]."""
    lib = _load()
    X = _c(X, np.uint16)
    M = X.shape[0]
    assert X.shape == (M, K)
    qc, cb = _c(qc, np.uint8), _c(cb, np.uint16)
    row_ptr, col_idx, val = _c(row_ptr, np.int32), _c(col_idx, np.int32), _c(val, np.uint16)
    assert qc.shape == (N, K // 2) and cb.shape == (N, 16) and row_ptr.shape == (N + 1,)
    assert col_idx.shape == val.shape == (int(row_ptr[-1]),)
    if col_idx.size == 0:
        col_idx, val = np.zeros(1, np.int32), np.zeros(1, np.uint16)
    rows_arr = None
    n_rows = M
    if rows is not None:
        rows_arr = np.ascontiguousarray(rows, dtype=np.int32)
        n_rows = int(rows_arr.shape[0])
    Y = np.empty((n_rows, N), np.float64)
    act_bf16 = {"fp16": 0, "bf16": 1}[act]
    rc = lib.w4o_forward_xfp(M, N, K, act_bf16, _ptr(X), _ptr(qc), _ptr(cb), _ptr(row_ptr),
                             _ptr(col_idx), _ptr(val), _ptr(rows_arr), n_rows, _ptr(Y))
    if rc != 0:
        raise RuntimeError("oracle forward_xfp failed (bad arguments)")
    return {"Y": Y}


def forward_xfp_lib(X, qc, library, libid, row_ptr, col_idx, val, *, N, K, act="fp16", rows=None):
    """Y = X Wh^T with Wh[n,k] = library[libid[n, k // 128]][idx[n,k]] +
    (sparse residual)[n,k] (see w4o_forward_xfp_lib).  qc: 4-bit indices
    uint8 [N, K/2]; library: fp16 bits [L, 16]; libid: uint8 [N, K/128];
    row_ptr, col_idx, val as forward_xfp."""
    lib = _load()
    X = _c(X, np.uint16)
    M = X.shape[0]
    assert X.shape == (M, K) and K % 128 == 0
    qc, library, libid = _c(qc, np.uint8), _c(library, np.uint16), _c(libid, np.uint8)
    row_ptr, col_idx, val = _c(row_ptr, np.int32), _c(col_idx, np.int32), _c(val, np.uint16)
    L = int(library.shape[0])
    assert qc.shape == (N, K // 2) and library.shape == (L, 16) and libid.shape == (N, K // 128)
    assert row_ptr.shape == (N + 1,) and col_idx.shape == val.shape == (int(row_ptr[-1]),)
    if col_idx.size == 0:
        col_idx, val = np.zeros(1, np.int32), np.zeros(1, np.uint16)
    rows_arr = None
    n_rows = M
    if rows is not None:
        rows_arr = np.ascontiguousarray(rows, dtype=np.int32)
        n_rows = int(rows_arr.shape[0])
    Y = np.empty((n_rows, N), np.float64)
    act_bf16 = {"fp16": 0, "bf16": 1}[act]
    rc = lib.w4o_forward_xfp_lib(M, N, K, act_bf16, _ptr(X), _ptr(qc), _ptr(library), L, _ptr(libid),
                                 _ptr(row_ptr), _ptr(col_idx), _ptr(val), _ptr(rows_arr), n_rows, _ptr(Y))
    if rc != 0:
        raise RuntimeError("oracle forward_xfp_lib failed (bad arguments)")
    return {"Y": Y}
