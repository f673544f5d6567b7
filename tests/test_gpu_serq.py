"""GPU parity of the salient-channel correction (Y = X Wd^T + X[:, S] R;
SERQ summary, section 2, in the W4A16 setting) through the C ABI, against
the float64 oracle.  Same tolerance as the layer; the workspace's state
region returns to zero after every call (an out-of-range index is the one
case that leaves a flag there, and is tested as such)."""
import numpy as np
import pytest

import oracle
import w4_gemm_error_amd as w4
from w4_gemm_error_amd import synth

from gpu_util import (assert_all_finite, assert_close, dev_act, gpu_quantize, host_bits, nan_y,
                      new_workspace, poison_workspace, sample_rows, torch)

pytestmark = pytest.mark.gpu


def _print(*a):
    print(*a, flush=True)


def serq_inputs(d, s, seed=0, contiguous=False):
    rng = np.random.default_rng(500 + seed)
    if contiguous:
        S = np.arange(s, dtype=np.int32)
    else:
        S = rng.integers(0, d["K"], size=s).astype(np.int32)
        if s >= 3:
            S[1] = S[0]                                 # a repeated channel
    R = synth.to_act_bits(rng.normal(0.0, 0.01, (s, d["N"])), d["act"])
    return S, R


def gpu_serq(d, packed, phase, S, R, *, workspace=None, check_state=True):
    t = torch()
    act = d["act"]
    s = len(S)
    X = dev_act(d["X"], act)
    Sd = t.from_numpy(S).cuda() if s else None
    Rd = dev_act(R, act) if s else None
    if workspace is None:
        workspace = new_workspace(w4.w4ec_workspace_bytes(d["M"], d["N"], d["K"], s, d["group_size"]))
    else:
        poison_workspace(workspace)
    fn = w4.w4ec_linear_decode_serq if phase == "decode" else w4.w4ec_linear_prefill_serq
    Y = nan_y(d["M"], d["N"], act)
    fn(X, packed, Sd, Rd, N=d["N"], group_size=d["group_size"], workspace=workspace, Y=Y)
    t.cuda.synchronize()
    assert_all_finite(Y, f"serq {phase} M={d['M']}")
    if check_state:
        state = workspace[: w4.W4EC_WS_STATE_BYTES]
        assert int(t.count_nonzero(state).item()) == 0, f"{phase}: state not at zero after the call"
    return host_bits(Y), workspace


def oracle_serq(d, codes, S, R, rows=None):
    qc, s, z = codes
    return oracle.forward_serq(d["X"], qc, s, z, S if len(S) else None, R if len(S) else None,
                               N=d["N"], K=d["K"], group_size=d["group_size"], act=d["act"],
                               rows=rows, want_parts=False)["Y"]


def small_layer(act, M, N, K, G, seed=5):
    cfg = synth.LAYERS["mlp_70b_bf16"] if act == "bf16" else synth.LAYERS["tiny"]
    return synth.make_layer(cfg, M, seed=seed, N=N, K=K, r=8, group_size=G)


SMALL = [
    # phase, act, M, N, K, G, s
    ("decode", "fp16", 1, 512, 512, 512, 8),
    ("decode", "fp16", 3, 528, 640, 640, 41),
    ("decode", "fp16", 16, 512, 512, 128, 64),
    ("decode", "bf16", 5, 272, 384, 384, 40),
    ("decode", "fp16", 2, 512, 20480, 20480, 256),
    ("prefill", "fp16", 17, 528, 640, 640, 41),
    ("prefill", "fp16", 300, 512, 512, 512, 8),
    ("prefill", "bf16", 100, 528, 512, 512, 40),        # per-channel bf16: activation sums too
    ("prefill", "bf16", 200, 512, 768, 128, 16),
    ("prefill", "fp16", 64, 1024, 2048, 2048, 130),
]


@pytest.mark.parametrize("phase,act,M,N,K,G,s", SMALL)
def test_serq_small_parity(phase, act, M, N, K, G, s):
    _print(f"serq small {phase} {act} M={M} N={N} K={K} G={G} s={s}")
    d = small_layer(act, M, N, K, G)
    S, R = serq_inputs(d, s, seed=M + s)
    _, _, _, packed = gpu_quantize(d)
    codes = oracle.rtn_quantize(d["W"], G)
    Y, _ = gpu_serq(d, packed, phase, S, R)
    assert_close(Y, oracle_serq(d, codes, S, R), act, f"serq {phase} {act} M={M}")


@pytest.mark.parametrize("phase", ["decode", "prefill"])
def test_serq_empty_is_plain_w4(phase):
    _print(f"serq s=0 {phase}")
    d = small_layer("fp16", 9 if phase == "decode" else 40, 528, 512, 512, seed=8)
    _, _, _, packed = gpu_quantize(d)
    Y, _ = gpu_serq(d, packed, phase, np.zeros(0, np.int32), None)
    fn = w4.w4ec_linear_decode if phase == "decode" else w4.w4ec_linear_prefill
    plain = host_bits(fn(dev_act(d["X"], "fp16"), packed, None, None, None, 0.0, N=d["N"], group_size=512))
    assert np.array_equal(Y, plain)


@pytest.mark.parametrize("phase", ["decode", "prefill"])
def test_serq_out_of_range_index_is_flagged(phase):
    """The kernel's own bounds check: an index past K is clamped (no access
    out of bounds) and leaves a nonzero word in the state region."""
    _print(f"serq bad index {phase}")
    d = small_layer("fp16", 4 if phase == "decode" else 40, 512, 512, 512, seed=9)
    S, R = serq_inputs(d, 8, seed=1)
    S[5] = d["K"] + 7
    _, _, _, packed = gpu_quantize(d)
    Y, ws = gpu_serq(d, packed, phase, S, R, check_state=False)
    t = torch()
    assert int(t.count_nonzero(ws[: w4.W4EC_WS_STATE_BYTES]).item()) > 0
    assert np.isfinite(synth.act_bits_to_f64(Y, "fp16")).all()


FULL = [
    # cfg, M, phase (oracle rows: sample_rows)
    ("decode_up_proj_8b", 1, "decode"),
    ("decode_up_proj_8b", 16, "decode"),
    ("prefill_out_proj_8b", 2048, "prefill"),
    ("mlp_70b_bf16", 64, "prefill"),
]


@pytest.mark.parametrize("cfg,M,phase", FULL)
def test_serq_full_size_parity(cfg, M, phase):
    """The salient channels are the configs' outlier channels (the ones whose
    activation scale marks them), as an offline permutation would gather."""
    rows = sample_rows(M)
    _print(f"serq full {cfg} M={M} {phase} rows={'all' if rows is None else len(rows)}")
    d = synth.make_layer(cfg, M, seed=0)
    S = np.asarray(d["outlier_channels"], dtype=np.int32)
    R = synth.to_act_bits(np.random.default_rng(synth.SEEDS[cfg]).normal(0.0, 0.01, (len(S), d["N"])), d["act"])
    _, _, _, packed = gpu_quantize(d)
    codes = oracle.rtn_quantize(d["W"], d["group_size"])
    Y, _ = gpu_serq(d, packed, phase, S, R)
    ref = oracle_serq(d, codes, S, R, rows=rows)
    worst = assert_close(Y if rows is None else Y[rows], ref, d["act"], f"serq {cfg} M={M}")
    _print(f"  worst err/tol {worst:.3f}")
