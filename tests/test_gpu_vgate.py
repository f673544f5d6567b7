"""GPU parity of the vector-gate layer (one gate per rank component from a
bottleneck MLP on T = X A) through the C ABI, against the float64 oracle.

Same bar as the scalar-gate tests: codes bit-exact, Y within
2e-3 (fp16) / 1.6e-2 (bf16) * (max_n |Y_oracle[m, n]| + 1) per token; the
hand-over state returns to zero after every call.
"""
import math

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


def vg_params(d, h, seed=0):
    # gates spread over (0, 1) for rows of T of about this size
    t_std = 0.01 * math.sqrt(d["K"]) * 2.0
    return synth.make_vgate(d["r"], h, d["act"], seed=seed, t_std=t_std)


def gpu_vgate(d, packed, phase, p, *, workspace=None, c2=None, G2=None):
    act = d["act"]
    X = dev_act(d["X"], act)
    A, B = dev_act(d["A"], act), dev_act(d["B"], act)
    G1, c1 = dev_act(p["G1"], act), dev_act(p["c1"], act)
    G2d = dev_act(p["G2"] if G2 is None else G2, act)
    c2d = dev_act(p["c2"] if c2 is None else c2, act)
    if workspace is None:
        workspace = new_workspace(w4.w4ec_workspace_bytes(d["M"], d["N"], d["K"], d["r"], d["group_size"]))
    else:
        poison_workspace(workspace)
    fn = w4.w4ec_linear_decode_vgate if phase == "decode" else w4.w4ec_linear_prefill_vgate
    Y = nan_y(d["M"], d["N"], act)
    fn(X, packed, A, B, G1, c1, G2d, c2d, N=d["N"], group_size=d["group_size"], workspace=workspace, Y=Y)
    torch().cuda.synchronize()
    assert_all_finite(Y, f"vgate {phase} M={d['M']}")
    state = workspace[: w4.W4EC_WS_STATE_BYTES]
    assert int(torch().count_nonzero(state).item()) == 0, f"{phase}: hand-over state not at zero after the call"
    return host_bits(Y)


def oracle_vgate(d, codes, p, *, rows=None, c2=None, G2=None):
    qc, s, z = codes
    return oracle.forward_vgate(d["X"], qc, s, z, d["A"], d["B"], p["G1"], p["c1"],
                                p["G2"] if G2 is None else G2, p["c2"] if c2 is None else c2,
                                N=d["N"], K=d["K"], r=d["r"], h=p["h"], group_size=d["group_size"],
                                act=d["act"], rows=rows, want_parts=False)["Y"]


def small_layer(act, M, N, K, r, G, seed=5):
    cfg = synth.LAYERS["mlp_70b_bf16"] if act == "bf16" else synth.LAYERS["tiny"]
    return synth.make_layer(cfg, M, seed=seed, N=N, K=K, r=r, group_size=G)


SMALL = [
    # phase, act, M, N, K, r, G, h
    ("decode", "fp16", 1, 512, 512, 8, 512, 4),
    ("decode", "fp16", 3, 528, 640, 72, 640, 16),
    ("decode", "fp16", 16, 512, 512, 64, 128, 16),
    ("decode", "bf16", 5, 272, 384, 40, 384, 8),
    ("decode", "fp16", 7, 48, 1280, 256, 256, 64),
    ("decode", "fp16", 2, 512, 20480, 256, 20480, 32),    # more slices than reducing workgroups
    ("prefill", "fp16", 17, 528, 640, 72, 640, 16),
    ("prefill", "fp16", 300, 512, 512, 8, 512, 4),
    ("prefill", "bf16", 100, 528, 512, 40, 512, 8),        # per-channel bf16: activation sums too
    ("prefill", "bf16", 200, 512, 768, 16, 128, 16),
    ("prefill", "fp16", 64, 1024, 2048, 130, 2048, 64),
]


@pytest.mark.parametrize("phase,act,M,N,K,r,G,h", SMALL)
def test_vgate_small_parity(phase, act, M, N, K, r, G, h):
    _print(f"vgate small {phase} {act} M={M} N={N} K={K} r={r} G={G} h={h}")
    d = small_layer(act, M, N, K, r, G)
    p = vg_params(d, h, seed=M + r)
    q, s, z, packed = gpu_quantize(d)
    codes = oracle.rtn_quantize(d["W"], G)
    assert np.array_equal(q.cpu().numpy(), codes[0])
    Y = gpu_vgate(d, packed, phase, p)
    assert_close(Y, oracle_vgate(d, codes, p), act, f"vgate {phase} {act} M={M}")


@pytest.mark.parametrize("phase", ["decode", "prefill"])
def test_vgate_closed_and_open(phase):
    _print(f"vgate closed/open {phase}")
    M = 9 if phase == "decode" else 40
    d = small_layer("fp16", M, 528, 512, 24, 512, seed=8)
    p = vg_params(d, 8, seed=3)
    _, _, _, packed = gpu_quantize(d)
    codes = oracle.rtn_quantize(d["W"], 512)
    r = d["r"]
    closed = gpu_vgate(d, packed, phase, p, c2=synth.to_act_bits(np.full(r, -np.inf), "fp16"))
    t = torch()
    fn = w4.w4ec_linear_decode if phase == "decode" else w4.w4ec_linear_prefill
    plain = host_bits(fn(dev_act(d["X"], "fp16"), packed, None, None, None, 0.0, N=d["N"], group_size=512))
    assert np.array_equal(closed, plain)                   # every gate 0: the plain W4 layer
    ones_c2 = synth.to_act_bits(np.full(r, np.inf), "fp16")
    zero_G2 = synth.to_act_bits(np.zeros((p["h"], r)), "fp16")
    opened = gpu_vgate(d, packed, phase, p, c2=ones_c2, G2=zero_G2)
    assert_close(opened, oracle_vgate(d, codes, p, c2=ones_c2, G2=zero_G2), "fp16", "vgate open")


FULL = [
    # cfg, M, phase, h (oracle rows: sample_rows)
    ("decode_up_proj_8b", 1, "decode", 16),
    ("decode_up_proj_8b", 16, "decode", 16),
    ("prefill_out_proj_8b", 2048, "prefill", 16),
    ("mlp_70b_bf16", 64, "prefill", 32),
]


@pytest.mark.parametrize("cfg,M,phase,h", FULL)
def test_vgate_full_size_parity(cfg, M, phase, h):
    rows = sample_rows(M)
    _print(f"vgate full {cfg} M={M} {phase} rows={'all' if rows is None else len(rows)}")
    d = synth.make_layer(cfg, M, seed=0)
    p = vg_params(d, h, seed=synth.SEEDS[cfg])
    q, s, z, packed = gpu_quantize(d)
    codes = oracle.rtn_quantize(d["W"], d["group_size"])
    del q, s, z
    Y = gpu_vgate(d, packed, phase, p)
    qc, s, z = codes
    parts = oracle.forward_vgate(d["X"], qc, s, z, d["A"], d["B"], p["G1"], p["c1"], p["G2"], p["c2"],
                                 N=d["N"], K=d["K"], r=d["r"], h=h, group_size=d["group_size"],
                                 act=d["act"], rows=rows)
    g = parts["gamma"]
    assert np.mean((g > 0.05) & (g < 0.95)) > 0.5, "gates saturated: the case would not test them"
    worst = assert_close(Y if rows is None else Y[rows], parts["Y"], d["act"], f"vgate {cfg} M={M}")
    _print(f"  worst err/tol {worst:.3f}")


def test_vgate_and_scalar_share_a_workspace():
    _print("vgate / scalar shared workspace")
    t = torch()
    d = small_layer("fp16", 4, 512, 1024, 64, 1024, seed=12)
    p = vg_params(d, 16, seed=4)
    _, _, _, packed = gpu_quantize(d)
    codes = oracle.rtn_quantize(d["W"], 1024)
    need = w4.w4ec_workspace_bytes(d["M"], d["N"], d["K"], d["r"], 1024)
    ws = t.zeros(need, dtype=t.uint8, device="cuda")
    ref_v = oracle_vgate(d, codes, p)
    X, A, B, wg = (dev_act(d[k], "fp16") for k in ("X", "A", "B", "w_g"))
    for rep in range(3):
        for phase in ("decode", "prefill"):
            Yv = gpu_vgate(d, packed, phase, p, workspace=ws)
            assert_close(Yv, ref_v, "fp16", f"vgate {phase} rep {rep}")
            fn = w4.w4ec_linear_decode if phase == "decode" else w4.w4ec_linear_prefill
            fn(X, packed, A, B, wg, d["b_g"], N=d["N"], group_size=1024, workspace=ws)
            t.cuda.synchronize()
            assert int(t.count_nonzero(ws[: w4.W4EC_WS_STATE_BYTES]).item()) == 0
