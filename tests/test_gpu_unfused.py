"""GPU parity of the unfused and semi-fused prefill forms against the
float64 oracle: the EC gate step (T_g into a workspace), the plain W4 GEMM
(w4ec_linear_prefill with r = 0) and the T_g B step, run one after the
other or with the gate step on a second stream beside the GEMM.

Same tolerance as the fused layer (one more rounding of Y to the activation
type stays well inside it).
"""
import numpy as np
import pytest

import oracle
import w4_gemm_error_amd as w4
from w4_gemm_error_amd import synth

from gpu_util import (assert_all_finite, assert_close, dev_act, gpu_layer, gpu_quantize, host_bits, nan_y,
                      new_workspace, oracle_layer, torch)

pytestmark = pytest.mark.gpu


def _print(*a):
    print(*a, flush=True)


def small_layer(act, M, N, K, r, G, seed=5):
    cfg = synth.LAYERS["mlp_70b_bf16"] if act == "bf16" else synth.LAYERS["tiny"]
    return synth.make_layer(cfg, M, seed=seed, N=N, K=K, r=r, group_size=G)


def unfused(d, packed, *, two_streams=False):
    t = torch()
    act = d["act"]
    M, N, K, r, G = d["M"], d["N"], d["K"], d["r"], d["group_size"]
    X, A, B, wg = (dev_act(d[k], act) for k in ("X", "A", "B", "w_g"))
    # the EC workspace holds only per-call data (no hand-over state): all of it poisoned
    ws_ec = t.full((w4.w4ec_prefill_ec_workspace_bytes(M, K, r),), 0xFF, dtype=t.uint8, device="cuda")
    ws_mm = new_workspace(w4.w4ec_workspace_bytes(M, N, K, 0, G))
    Y = nan_y(M, N, act)
    main = t.cuda.current_stream()
    if two_streams:
        side = t.cuda.Stream()
        side.wait_stream(main)
        with t.cuda.stream(side):
            w4.w4ec_prefill_ec_gate(X, A, wg, d["b_g"], workspace=ws_ec)
        w4.w4ec_linear_prefill(X, packed, None, None, None, 0.0, N=N, group_size=G, workspace=ws_mm, Y=Y)
        main.wait_stream(side)
    else:
        w4.w4ec_prefill_ec_gate(X, A, wg, d["b_g"], workspace=ws_ec)
        w4.w4ec_linear_prefill(X, packed, None, None, None, 0.0, N=N, group_size=G, workspace=ws_mm, Y=Y)
    w4.w4ec_prefill_ec_apply(Y, B, K=K, workspace=ws_ec)
    t.cuda.synchronize()
    assert int(t.count_nonzero(ws_mm[: w4.W4EC_WS_STATE_BYTES]).item()) == 0
    assert_all_finite(Y, f"unfused M={M}")
    return host_bits(Y)


CASES = [
    # act, M, N, K, r, G
    ("fp16", 17, 528, 640, 72, 640),
    ("fp16", 300, 512, 512, 8, 512),
    ("fp16", 129, 784, 1024, 64, 128),
    ("bf16", 100, 528, 512, 40, 512),
    ("bf16", 200, 512, 768, 16, 128),
    ("fp16", 64, 1024, 2048, 130, 2048),
]


@pytest.mark.parametrize("act,M,N,K,r,G", CASES)
def test_unfused_prefill_parity(act, M, N, K, r, G):
    _print(f"unfused {act} M={M} N={N} K={K} r={r} G={G}")
    d = small_layer(act, M, N, K, r, G)
    _, _, _, packed = gpu_quantize(d)
    codes = oracle.rtn_quantize(d["W"], G)
    Y = unfused(d, packed)
    ref = oracle_layer(d, codes)
    assert_close(Y, ref, act, f"unfused {act} M={M}")
    Ys = unfused(d, packed, two_streams=True)
    assert np.array_equal(Ys, Y)                       # the same kernels, only overlapped


def test_unfused_matches_fused_at_full_size():
    _print("unfused vs fused, 2048 x 4096 x 4096")
    d = synth.make_layer("prefill_out_proj_8b", 2048, seed=0)
    _, _, _, packed = gpu_quantize(d)
    Yu = unfused(d, packed, two_streams=True)
    Yf = gpu_layer(d, packed, "prefill")
    rows = [0, 1, 77, 1023, 2047]
    codes = oracle.rtn_quantize(d["W"], d["group_size"])
    ref = oracle_layer(d, codes, rows=rows)
    assert_close(Yu[rows], ref, "fp16", "unfused full size")
    a = synth.act_bits_to_f64(Yu, "fp16")
    b = synth.act_bits_to_f64(Yf, "fp16")
    bound = 2e-3 * (np.abs(b).max(axis=1, keepdims=True) + 1.0)
    assert (np.abs(a - b) <= bound).all()
