"""GPU: w4ec_linear_decode_noalloc, the decode entry point that takes no
workspace and allocates nothing (its hand-over state in a static device
array), against w4ec_linear_decode with a caller's workspace.

Two calls in a row on the same array, the second with a smaller input (fewer
tokens, a narrower layer, a lower rank): each must equal the workspace entry
point's output element by element (the same kernels and launch plan), and
the first also matches the oracle within the layer's tolerance.  Also: a
shape whose state would not fit the array is refused, and r = 0 touches no
state.
"""
import numpy as np
import pytest

import oracle
import w4_gemm_error_amd as w4
from w4_gemm_error_amd import synth

from gpu_util import assert_close, dev_act, gpu_quantize, host_bits, nan_y, new_workspace, oracle_layer, torch

pytestmark = pytest.mark.gpu


def _print(*a):
    print(*a, flush=True)


def _both(d, packed):
    t = torch()
    act = d["act"]
    X, A, B, wg = (dev_act(d[k], act) for k in ("X", "A", "B", "w_g"))
    if d["r"] == 0:
        A = B = wg = None
    kw = dict(N=d["N"], group_size=d["group_size"])
    Y_ws = nan_y(d["M"], d["N"], act)
    ws = new_workspace(max(w4.w4ec_workspace_bytes(d["M"], d["N"], d["K"], d["r"], d["group_size"]), 256))
    w4.w4ec_linear_decode(X, packed, A, B, wg, d["b_g"], workspace=ws, Y=Y_ws, **kw)
    Y_na = nan_y(d["M"], d["N"], act)
    w4.w4ec_linear_decode_noalloc(X, packed, A, B, wg, d["b_g"], Y=Y_na, **kw)
    t.cuda.synchronize()
    return host_bits(Y_ws), host_bits(Y_na)


@pytest.mark.parametrize("act", ["fp16", "bf16"])
def test_noalloc_matches_workspace_entry_two_calls(act):
    layer = "tiny" if act == "fp16" else "mlp_70b_bf16"
    cases = [dict(M=16, N=1040, K=4096, r=64, group_size=4096),    # first call: the larger input
             dict(M=3, N=272, K=1024, r=16, group_size=128)]       # second call: smaller in every size
    for i, c in enumerate(cases):
        _print(f"noalloc decode {act} call {i}: {c}")
        d = synth.make_layer(layer, c["M"], seed=31 + i, N=c["N"], K=c["K"], r=c["r"], group_size=c["group_size"])
        _, _, _, packed = gpu_quantize(d)
        y_ws, y_na = _both(d, packed)
        assert np.array_equal(y_ws, y_na), f"call {i}: noalloc differs from the workspace entry point"
        if i == 0:
            ref = oracle_layer(d, oracle.rtn_quantize(d["W"], d["group_size"]))
            assert_close(y_na, ref, act, f"noalloc {act} call {i}")


def test_noalloc_without_rank_and_refusal():
    _print("noalloc decode: r = 0, then a shape too large for the array")
    d = synth.make_layer("tiny", 2, seed=41, N=512, K=512, r=0, group_size=512)
    _, _, _, packed = gpu_quantize(d)
    y_ws, y_na = _both(d, packed)
    assert np.array_equal(y_ws, y_na)
    # 16 tokens, rank 256, K = 16384: 256 EC slices of 64 k hold 16 x 257
    # words each, about 4.2 MB with the control region: more than the array
    t = torch()
    M, N, K, r = 16, 256, 16384, 256
    X = t.zeros((M, K), dtype=t.float16, device="cuda")
    A = t.zeros((K, r), dtype=t.float16, device="cuda")
    B = t.zeros((r, N), dtype=t.float16, device="cuda")
    wg = t.zeros((K,), dtype=t.float16, device="cuda")
    packed = t.zeros((w4.w4ec_packed_bytes(N, K, K),), dtype=t.uint8, device="cuda")
    Y = t.empty((M, N), dtype=t.float16, device="cuda")
    with pytest.raises(w4.W4ECError) as e:
        w4.w4ec_linear_decode_noalloc(X, packed, A, B, wg, 0.0, N=N, group_size=K, Y=Y)
    assert e.value.status == w4.W4EC_ERR_UNSUPPORTED
