"""Host-side checks of the C ABI (CPU only; no kernel is launched).

Every call below fails validation, which happens before any HIP call, so
these run without a GPU.  Device pointers are fake, suitably aligned
addresses that are never dereferenced.
"""
import ctypes
import math

import pytest

import w4_gemm_error_amd as w4


def test_library_exports_every_header_symbol():
    declared = w4.header_symbols()
    assert set(declared) >= {"w4ec_pack", "w4ec_linear_decode", "w4ec_linear_prefill",
                             "w4ec_linear_decode_vgate", "w4ec_linear_prefill_vgate",
                             "w4ec_quantize_rtn", "w4ec_unpack", "w4ec_packed_bytes",
                             "w4ec_workspace_bytes", "w4ec_status_str"}
    assert w4.exported_symbols() == declared


def test_status_strings():
    for code, name in [(0, "W4EC_OK"), (-1, "W4EC_ERR_INVALID_ARG"), (-2, "W4EC_ERR_UNSUPPORTED"),
                       (-3, "W4EC_ERR_WORKSPACE"), (-4, "W4EC_ERR_HIP"), (-5, "W4EC_ERR_TIMED_OUT"),
                       (-6, "W4EC_ERR_BAD_INDEX"), (7, "W4EC_UNKNOWN_STATUS")]:
        assert w4.w4ec_status_str(code) == name


def test_wait_limit_round_trip_and_workspace_checks():
    old = w4.w4ec_wait_limit()
    assert old == 1 << 22
    try:
        w4.w4ec_set_wait_limit(0)
        assert w4.w4ec_wait_limit() == 0
        w4.w4ec_set_wait_limit(123)
        assert w4.w4ec_wait_limit() == 123
    finally:
        w4.w4ec_set_wait_limit(old)
    L = w4.lib()
    P = ctypes.c_void_p
    # no or a misaligned workspace is rejected before any HIP call
    assert L.w4ec_workspace_status(None, 1 << 20, None) == w4.W4EC_ERR_WORKSPACE
    assert L.w4ec_workspace_status(P(FAKE + 16), 1 << 20, None) == w4.W4EC_ERR_WORKSPACE
    assert L.w4ec_workspace_reset(None, 1 << 20, None) == w4.W4EC_ERR_WORKSPACE
    assert L.w4ec_workspace_reset(P(FAKE), 100, None) == w4.W4EC_ERR_WORKSPACE


def test_packed_bytes():
    # header + N/16 * K/128 panels of 1 KB + (K/G) * Npad scale/zero dwords
    assert w4.w4ec_packed_bytes(512, 512, 512) == 256 + 32 * 4 * 1024 + 512 * 4
    assert w4.w4ec_packed_bytes(14336, 4096, 4096) == 256 + 14336 * 4096 // 2 + 14336 * 4
    assert w4.w4ec_packed_bytes(4096, 14336, 128) == 256 + 4096 * 14336 // 2 + 112 * 4096 * 4
    assert w4.w4ec_packed_bytes(20, 256, 256) == 256 + 2 * 2 * 1024 + 32 * 4   # N padded to 32
    assert w4.w4ec_packed_bytes(16, 100, 100) == 0      # K not a multiple of 128
    assert w4.w4ec_packed_bytes(16, 512, 96) == 0       # group not a multiple of 128
    assert w4.w4ec_packed_bytes(0, 512, 512) == 0


def test_workspace_bytes():
    assert w4.w4ec_workspace_bytes(1, 14336, 4096, 64, 4096) > 0
    assert w4.w4ec_workspace_bytes(2048, 4096, 4096, 64, 4096) >= 2048 * 64 * 2   # gated T for every token
    assert w4.w4ec_workspace_bytes(256, 4096, 14336, 128, 128) >= 256 * 4096 * 4  # split-K partial tiles
    assert w4.w4ec_workspace_bytes(1, 512, 512, 300, 512) == 0   # rank above 256
    assert w4.w4ec_workspace_bytes(0, 512, 512, 8, 512) == 0


FAKE = 0x7F0000000000   # 256-byte aligned, never dereferenced


def call(name, X=FAKE, packed=FAKE + 0x100000, A=FAKE + 0x200000, B=FAKE + 0x300000,
         w_g=FAKE + 0x400000, b_g=0.0, Y=FAKE + 0x500000, M=4, N=512, K=512, r=8, G=512,
         act=0, ws=FAKE + 0x600000, ws_bytes=1 << 30):
    fn = getattr(w4.lib(), name)
    P = ctypes.c_void_p
    return fn(P(X) if X else None, P(packed) if packed else None, P(A) if A else None,
              P(B) if B else None, P(w_g) if w_g else None, b_g, P(Y) if Y else None,
              M, N, K, r, G, act, P(ws) if ws else None, ws_bytes, None)


@pytest.mark.parametrize("name", ["w4ec_linear_decode", "w4ec_linear_prefill"])
def test_layer_argument_errors(name):
    E = w4
    assert call(name, M=0) == E.W4EC_ERR_INVALID_ARG
    assert call(name, r=-1) == E.W4EC_ERR_INVALID_ARG
    assert call(name, N=0) == E.W4EC_ERR_INVALID_ARG
    assert call(name, K=500) == E.W4EC_ERR_UNSUPPORTED
    assert call(name, G=96) == E.W4EC_ERR_UNSUPPORTED
    assert call(name, r=257) == E.W4EC_ERR_UNSUPPORTED
    assert call(name, act=5) == E.W4EC_ERR_INVALID_ARG
    assert call(name, X=0) == E.W4EC_ERR_INVALID_ARG
    assert call(name, packed=0) == E.W4EC_ERR_INVALID_ARG
    assert call(name, Y=0) == E.W4EC_ERR_INVALID_ARG
    assert call(name, A=0) == E.W4EC_ERR_INVALID_ARG            # r > 0 needs A and B
    assert call(name, X=FAKE + 8) == E.W4EC_ERR_INVALID_ARG     # misaligned
    assert call(name, packed=FAKE + 0x100010) == E.W4EC_ERR_INVALID_ARG
    assert call(name, Y=FAKE) == E.W4EC_ERR_INVALID_ARG         # aliases X
    assert call(name, ws=0) == E.W4EC_ERR_WORKSPACE
    assert call(name, ws_bytes=64) == E.W4EC_ERR_WORKSPACE
    assert call(name, ws=FAKE + 0x600010) == E.W4EC_ERR_WORKSPACE


def test_decode_rejects_more_than_16_tokens():
    assert call("w4ec_linear_decode", M=17) == w4.W4EC_ERR_UNSUPPORTED


def test_weight_prep_argument_errors():
    L = w4.lib()
    P = ctypes.c_void_p
    f = P(FAKE)
    assert L.w4ec_quantize_rtn(None, 16, 256, 256, f, f, f, None) == w4.W4EC_ERR_INVALID_ARG
    assert L.w4ec_quantize_rtn(f, 16, 256, 100, f, f, f, None) == w4.W4EC_ERR_INVALID_ARG
    assert L.w4ec_pack(f, f, f, 16, 200, 200, f, None) == w4.W4EC_ERR_UNSUPPORTED
    assert L.w4ec_pack(f, f, f, 16, 256, 256, P(FAKE + 16), None) == w4.W4EC_ERR_INVALID_ARG
    assert L.w4ec_pack(None, f, f, 16, 256, 256, f, None) == w4.W4EC_ERR_INVALID_ARG
    assert L.w4ec_unpack(None, 16, 256, 256, f, f, f, None) == w4.W4EC_ERR_INVALID_ARG
    assert L.w4ec_unpack(f, 16, 256, 64, f, f, f, None) == w4.W4EC_ERR_UNSUPPORTED


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(w4, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(w4, "_lib", None)
    with pytest.raises(ImportError):
        w4.lib()


def test_state_region_constant_matches_header():
    """The binding's W4EC_WS_STATE_BYTES mirrors the header's definition."""
    import re
    text = open(w4.HEADER_PATH).read()
    m = re.search(r"#define W4EC_WS_STATE_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m, "W4EC_WS_STATE_BYTES not found in the header"
    assert int(m.group(1)) << int(m.group(2)) == w4.W4EC_WS_STATE_BYTES


def call_vg(name, X=FAKE, packed=FAKE + 0x100000, A=FAKE + 0x200000, B=FAKE + 0x300000,
            G1=FAKE + 0x400000, c1=FAKE + 0x410000, G2=FAKE + 0x420000, c2=FAKE + 0x430000, h=8,
            Y=FAKE + 0x500000, M=4, N=512, K=512, r=8, G=512, act=0, ws=FAKE + 0x600000, ws_bytes=1 << 30):
    fn = getattr(w4.lib(), name)
    P = lambda v: ctypes.c_void_p(v) if v else None
    return fn(P(X), P(packed), P(A), P(B), P(G1), P(c1), P(G2), P(c2), h, P(Y),
              M, N, K, r, G, act, P(ws), ws_bytes, None)


@pytest.mark.parametrize("name", ["w4ec_linear_decode_vgate", "w4ec_linear_prefill_vgate"])
def test_vgate_argument_errors(name):
    E = w4
    assert call_vg(name, h=0) == E.W4EC_ERR_INVALID_ARG
    assert call_vg(name, h=65) == E.W4EC_ERR_UNSUPPORTED
    for arg in ("G1", "c1", "G2", "c2"):
        assert call_vg(name, **{arg: 0}) == E.W4EC_ERR_INVALID_ARG
    assert call_vg(name, G2=FAKE + 0x420001) == E.W4EC_ERR_INVALID_ARG   # not 2-byte aligned
    assert call_vg(name, M=0) == E.W4EC_ERR_INVALID_ARG
    assert call_vg(name, r=257) == E.W4EC_ERR_UNSUPPORTED
    assert call_vg(name, A=0) == E.W4EC_ERR_INVALID_ARG
    assert call_vg(name, ws=0) == E.W4EC_ERR_WORKSPACE
    assert call_vg(name, act=5) == E.W4EC_ERR_INVALID_ARG


def test_vgate_decode_rejects_more_than_16_tokens():
    assert call_vg("w4ec_linear_decode_vgate", M=17) == w4.W4EC_ERR_UNSUPPORTED


def test_prefill_ec_split_argument_errors():
    L = w4.lib()
    P = ctypes.c_void_p
    E = w4
    assert w4.w4ec_prefill_ec_workspace_bytes(2048, 4096, 64) > w4.W4EC_WS_STATE_BYTES
    assert w4.w4ec_prefill_ec_workspace_bytes(16, 100, 8) == 0       # K not a multiple of 128
    assert w4.w4ec_prefill_ec_workspace_bytes(16, 512, 0) == 0       # needs a compensator
    x, a, wg, y, b = (P(FAKE + i * 0x100000) for i in range(5))
    ws = P(FAKE + 0x600000)
    big = 1 << 30
    gate = lambda **k: L.w4ec_prefill_ec_gate(k.get("X", x), k.get("A", a), k.get("w_g", wg), 0.0,
                                              k.get("M", 64), k.get("K", 512), k.get("r", 8),
                                              k.get("act", 0), k.get("ws", ws), k.get("wsb", big), None)
    assert gate(M=0) == E.W4EC_ERR_INVALID_ARG
    assert gate(r=0) == E.W4EC_ERR_INVALID_ARG
    assert gate(K=500) == E.W4EC_ERR_UNSUPPORTED
    assert gate(r=257) == E.W4EC_ERR_UNSUPPORTED
    assert gate(X=None) == E.W4EC_ERR_INVALID_ARG
    assert gate(A=P(FAKE + 8)) == E.W4EC_ERR_INVALID_ARG
    assert gate(act=3) == E.W4EC_ERR_INVALID_ARG
    assert gate(ws=None) == E.W4EC_ERR_WORKSPACE
    assert gate(wsb=64) == E.W4EC_ERR_WORKSPACE
    apply = lambda **k: L.w4ec_prefill_ec_apply(k.get("Y", y), k.get("B", b), k.get("M", 64), k.get("N", 512),
                                                k.get("K", 512), k.get("r", 8), k.get("act", 0),
                                                k.get("ws", ws), k.get("wsb", big), None)
    assert apply(N=0) == E.W4EC_ERR_INVALID_ARG
    assert apply(Y=None) == E.W4EC_ERR_INVALID_ARG
    assert apply(B=y) == E.W4EC_ERR_INVALID_ARG                    # aliases Y
    assert apply(K=96) == E.W4EC_ERR_UNSUPPORTED
    assert apply(ws=P(FAKE + 0x600010)) == E.W4EC_ERR_WORKSPACE


@pytest.mark.parametrize("name", ["w4ec_linear_decode_serq", "w4ec_linear_prefill_serq"])
def test_serq_argument_errors(name):
    fn = getattr(w4.lib(), name)
    P = ctypes.c_void_p
    E = w4

    def c(X=FAKE, packed=FAKE + 0x100000, S=FAKE + 0x200000, R=FAKE + 0x300000, Y=FAKE + 0x500000,
          M=4, N=512, K=512, s=8, G=512, act=0, ws=FAKE + 0x600000, wsb=1 << 30):
        p = lambda v: P(v) if v else None
        return fn(p(X), p(packed), p(S), p(R), p(Y), M, N, K, s, G, act, p(ws), wsb, None)

    assert c(S=0) == E.W4EC_ERR_INVALID_ARG
    assert c(R=0) == E.W4EC_ERR_INVALID_ARG
    assert c(S=FAKE + 0x200002) == E.W4EC_ERR_INVALID_ARG        # not 4-byte aligned
    assert c(R=FAKE + 0x300001) == E.W4EC_ERR_INVALID_ARG
    assert c(s=257) == E.W4EC_ERR_UNSUPPORTED
    assert c(s=-1) == E.W4EC_ERR_INVALID_ARG
    assert c(M=0) == E.W4EC_ERR_INVALID_ARG
    assert c(X=0) == E.W4EC_ERR_INVALID_ARG
    assert c(R=FAKE + 0x500000) == E.W4EC_ERR_INVALID_ARG        # R aliases Y
    assert c(ws=0) == E.W4EC_ERR_WORKSPACE


def test_xfp_argument_errors():
    fn = w4.lib().w4ec_linear_decode_xfp
    P = ctypes.c_void_p
    E = w4

    def c(X=FAKE, packed=FAKE + 0x100000, cb=FAKE + 0x200000, rp=FAKE + 0x300000, ci=FAKE + 0x400000,
          val=FAKE + 0x500000, nnz=10, Y=FAKE + 0x600000, M=1, N=512, K=512, act=0):
        p = lambda v: P(v) if v else None
        return fn(p(X), p(packed), p(cb), p(rp), p(ci), p(val), nnz, p(Y), M, N, K, act, None)

    assert c(M=0) == E.W4EC_ERR_INVALID_ARG
    assert c(M=17) == E.W4EC_ERR_UNSUPPORTED
    assert c(K=500) == E.W4EC_ERR_UNSUPPORTED
    assert c(N=0) == E.W4EC_ERR_INVALID_ARG
    assert c(nnz=-1) == E.W4EC_ERR_INVALID_ARG
    assert c(act=2) == E.W4EC_ERR_INVALID_ARG
    assert c(cb=0) == E.W4EC_ERR_INVALID_ARG
    assert c(rp=0) == E.W4EC_ERR_INVALID_ARG
    assert c(ci=0) == E.W4EC_ERR_INVALID_ARG                    # entries but no columns
    assert c(val=0) == E.W4EC_ERR_INVALID_ARG
    assert c(cb=FAKE + 0x200008) == E.W4EC_ERR_INVALID_ARG      # codebook not 16-byte aligned
    assert c(rp=FAKE + 0x300002) == E.W4EC_ERR_INVALID_ARG
    assert c(val=FAKE + 0x500001) == E.W4EC_ERR_INVALID_ARG
    assert c(packed=FAKE + 0x100010) == E.W4EC_ERR_INVALID_ARG  # blob not 256-byte aligned
    assert c(Y=FAKE) == E.W4EC_ERR_INVALID_ARG                  # Y aliases X
    assert c(X=0) == E.W4EC_ERR_INVALID_ARG


def test_pack_xfp_argument_errors():
    fn = w4.lib().w4ec_pack_xfp
    P = ctypes.c_void_p
    assert fn(None, 512, 512, P(FAKE), None) == w4.W4EC_ERR_INVALID_ARG
    assert fn(P(FAKE), 512, 512, None, None) == w4.W4EC_ERR_INVALID_ARG
    assert fn(P(FAKE), 512, 512, P(FAKE + 0x10), None) == w4.W4EC_ERR_INVALID_ARG   # blob alignment
    assert fn(P(FAKE), 512, 500, P(FAKE), None) == w4.W4EC_ERR_UNSUPPORTED
    assert fn(P(FAKE), 0, 512, P(FAKE), None) == w4.W4EC_ERR_INVALID_ARG
