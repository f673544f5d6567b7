"""GPU: a bounded wait that gives up is visible to the caller.

The condition is forced from the host with w4ec_set_wait_limit(0): every
wait inside the decode kernel gives up at once, as if it had timed out, and
every kernel still exits normally.  Then:
  * the call's Y is NaN wherever it depended on the hand-over (all of it:
    every output workgroup waits for the gated rank-r activations);
  * w4ec_workspace_status reports W4EC_ERR_TIMED_OUT;
  * later decode calls on that workspace, with the normal limit, write NaN
    into all of Y: its hand-over state is no longer trusted (the prefill
    kernels keep their own hand-over state and stay correct);
  * after w4ec_workspace_reset the same calls match the oracle again.
The same holds, phase for phase, for a prefill call of at most 64 tokens,
whose GEMM workgroups compute the gated rank-r activations themselves and
wait for each other's pieces (a decode call on the workspace stays correct
meanwhile).
A salient-channel index outside [0, K) is reported as W4EC_ERR_BAD_INDEX.
"""
import numpy as np
import pytest

import oracle
import w4_gemm_error_amd as w4
from w4_gemm_error_amd import synth

from gpu_util import assert_close, dev_act, gpu_quantize, host_bits, nan_y, oracle_layer, torch

pytestmark = pytest.mark.gpu


def _print(*a):
    print(*a, flush=True)


def _call(d, packed, phase, ws):
    t = torch()
    act = d["act"]
    X, A, B, wg = (dev_act(d[k], act) for k in ("X", "A", "B", "w_g"))
    Y = nan_y(d["M"], d["N"], act)
    fn = w4.w4ec_linear_decode if phase == "decode" else w4.w4ec_linear_prefill
    fn(X, packed, A, B, wg, d["b_g"], N=d["N"], group_size=d["group_size"], workspace=ws, Y=Y)
    t.cuda.synchronize()
    return Y


def test_forced_timeout_is_visible_sticky_and_reset():
    _print("forced timeout: decode M=4 N=784 K=2048 r=64")
    t = torch()
    d = synth.make_layer("tiny", 4, seed=21, N=784, K=2048, r=64, group_size=2048)
    _, _, _, packed = gpu_quantize(d)
    ref = oracle_layer(d, oracle.rtn_quantize(d["W"], d["group_size"]))
    need = max(w4.w4ec_workspace_bytes(4, d["N"], d["K"], d["r"], d["group_size"]),
               w4.w4ec_workspace_bytes(40, d["N"], d["K"], d["r"], d["group_size"]))
    ws = t.zeros(need, dtype=t.uint8, device="cuda")
    assert w4.w4ec_workspace_status(ws) == w4.W4EC_OK
    old = w4.w4ec_wait_limit()
    try:
        w4.w4ec_set_wait_limit(0)
        Y = _call(d, packed, "decode", ws)             # returns normally
    finally:
        w4.w4ec_set_wait_limit(old)
    assert w4.w4ec_wait_limit() == old
    assert bool(t.isnan(Y.float()).all()), "outputs of a wait that gave up must be NaN"
    assert w4.w4ec_workspace_status(ws) == w4.W4EC_ERR_TIMED_OUT
    # sticky: the normal limit, same workspace -> decode writes NaN everywhere
    Y = _call(d, packed, "decode", ws)
    assert bool(t.isnan(Y.float()).all())
    # the prefill kernels keep their own hand-over state: untouched, and they
    # stay correct on that workspace
    d40 = synth.make_layer("tiny", 40, seed=21, N=784, K=2048, r=64, group_size=2048)
    Y = _call(d40, packed, "prefill", ws)
    assert_close(host_bits(Y), oracle_layer(d40, oracle.rtn_quantize(d40["W"], 2048)), "fp16", "prefill")
    assert w4.w4ec_workspace_status(ws) == w4.W4EC_ERR_TIMED_OUT
    # reset: correct again, nothing recorded, state back at zero after the call
    w4.w4ec_workspace_reset(ws)
    assert w4.w4ec_workspace_status(ws) == w4.W4EC_OK
    Y = _call(d, packed, "decode", ws)
    assert_close(host_bits(Y), ref, "fp16", "after reset")
    assert w4.w4ec_workspace_status(ws) == w4.W4EC_OK
    assert int(t.count_nonzero(ws[: w4.W4EC_WS_STATE_BYTES]).item()) == 0


def test_forced_prefill_fused_ec_timeout_is_visible_sticky_and_reset():
    # M=40, N=784, K=2048: one row of 64-token tiles (4 column tiles, K split
    # in 4): the fused EC
    _print("forced timeout: prefill M=40 N=784 K=2048 r=64 (fused EC)")
    t = torch()
    d = synth.make_layer("tiny", 40, seed=23, N=784, K=2048, r=64, group_size=2048)
    _, _, _, packed = gpu_quantize(d)
    ref = oracle_layer(d, oracle.rtn_quantize(d["W"], d["group_size"]))
    need = max(w4.w4ec_workspace_bytes(4, d["N"], d["K"], d["r"], d["group_size"]),
               w4.w4ec_workspace_bytes(40, d["N"], d["K"], d["r"], d["group_size"]))
    ws = t.zeros(need, dtype=t.uint8, device="cuda")
    old = w4.w4ec_wait_limit()
    try:
        w4.w4ec_set_wait_limit(0)
        Y = _call(d, packed, "prefill", ws)            # returns normally
    finally:
        w4.w4ec_set_wait_limit(old)
    assert bool(t.isnan(Y.float()).all()), "outputs of a wait that gave up must be NaN"
    assert w4.w4ec_workspace_status(ws) == w4.W4EC_ERR_TIMED_OUT
    # sticky for the prefill hand-over
    Y = _call(d, packed, "prefill", ws)
    assert bool(t.isnan(Y.float()).all())
    # the decode hand-over state is separate: decode stays correct
    d4 = synth.make_layer("tiny", 4, seed=23, N=784, K=2048, r=64, group_size=2048)
    Y = _call(d4, packed, "decode", ws)
    assert_close(host_bits(Y), oracle_layer(d4, oracle.rtn_quantize(d4["W"], 2048)), "fp16", "decode")
    # reset: correct again, state back at zero after the call
    w4.w4ec_workspace_reset(ws)
    assert w4.w4ec_workspace_status(ws) == w4.W4EC_OK
    Y = _call(d, packed, "prefill", ws)
    assert_close(host_bits(Y), ref, "fp16", "prefill after reset")
    assert w4.w4ec_workspace_status(ws) == w4.W4EC_OK
    assert int(t.count_nonzero(ws[: w4.W4EC_WS_STATE_BYTES]).item()) == 0


@pytest.mark.parametrize("phase", ["decode", "prefill"])
def test_bad_salient_index_is_reported(phase):
    _print(f"bad salient index reported, {phase}")
    t = torch()
    M = 4 if phase == "decode" else 40
    d = synth.make_layer("tiny", M, seed=9, N=512, K=512, r=8, group_size=512)
    _, _, _, packed = gpu_quantize(d)
    S = np.arange(8, dtype=np.int32)
    S[3] = d["K"] + 5
    R = synth.to_act_bits(np.random.default_rng(2).normal(0.0, 0.01, (8, d["N"])), "fp16")
    ws = t.zeros(w4.w4ec_workspace_bytes(M, d["N"], d["K"], 8, 512), dtype=t.uint8, device="cuda")
    fn = w4.w4ec_linear_decode_serq if phase == "decode" else w4.w4ec_linear_prefill_serq
    Y = fn(dev_act(d["X"], "fp16"), packed, t.from_numpy(S).cuda(), dev_act(R, "fp16"), N=d["N"],
           group_size=512, workspace=ws)
    t.cuda.synchronize()
    assert bool(t.isfinite(Y.float()).all())          # clamped, not poisoned
    assert w4.w4ec_workspace_status(ws) == w4.W4EC_ERR_BAD_INDEX
    w4.w4ec_workspace_reset(ws)
    assert w4.w4ec_workspace_status(ws) == w4.W4EC_OK
