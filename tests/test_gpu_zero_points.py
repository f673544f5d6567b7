"""GPU parity with zero points that are not integers in 0..15.

Quantizers other than round-to-nearest (SPEAR's results list GPTQ, AWQ and
OmniQuant beside RTN) can produce any fp16 zero point.  The blob takes any z
with |z| <= 1024: the kernels offset the codes by floor(z) exactly and
correct for the fractional part (an activation-sum term, or a fused
multiply-add in the grouped dequantization).  A zero point that is not
finite or lies outside that range makes the layer's outputs NaN.
Same tolerance as the layer; every path: decode and prefill, fp16 and bf16,
per channel and grouped, with and without the compensator.  An out-of-range
zero point is stored as NaN, so the column that uses it comes out NaN.
"""
import numpy as np
import pytest

import oracle
import w4_gemm_error_amd as w4
from w4_gemm_error_amd import synth

from gpu_util import (assert_close, dev_act, gpu_layer, host_bits, oracle_layer, sample_rows, torch)

pytestmark = pytest.mark.gpu


def _print(*a):
    print(*a, flush=True)


def frac_codes(d, seed):
    """RTN codes and scales of the layer, with the zero points moved off the
    integers: z + u for u in [-0.75, 0.75) in steps of 1/64, a few pushed
    below 0 and above 15 (codes unchanged, so the weights change with z)."""
    qc, s, z = oracle.rtn_quantize(d["W"], d["group_size"])
    rng = np.random.default_rng(seed)
    zf = z.view(np.float16).astype(np.float64)
    zf = zf + rng.integers(-48, 48, size=zf.shape) / 64.0
    zf.reshape(-1)[:3] = [-2.5, 16.25, 19.0]
    return qc, s, zf.astype(np.float16).view(np.uint16)


def pack_host(qc, s, z, N, K, G):
    t = torch()
    return w4.w4ec_pack(t.from_numpy(qc).cuda(), t.from_numpy(s.view(np.float16)).cuda(),
                        t.from_numpy(z.view(np.float16)).cuda(), N, K, G)


CASES = [
    # phase, act, M, N, K, r, G
    ("decode", "fp16", 1, 528, 1024, 16, 1024),
    ("decode", "fp16", 4, 512, 1024, 0, 128),
    ("decode", "bf16", 3, 272, 768, 32, 768),
    ("decode", "bf16", 9, 512, 512, 8, 128),
    ("decode", "fp16", 16, 512, 2048, 64, 2048),
    ("prefill", "fp16", 200, 528, 640, 16, 640),
    ("prefill", "fp16", 129, 512, 1024, 0, 1024),      # the fp16 per-channel path without a prepass
    ("prefill", "fp16", 64, 784, 1024, 24, 128),
    ("prefill", "bf16", 100, 528, 512, 40, 512),
    ("prefill", "bf16", 70, 512, 768, 0, 128),
]


@pytest.mark.parametrize("phase,act,M,N,K,r,G", CASES)
def test_fractional_zero_point_parity(phase, act, M, N, K, r, G):
    _print(f"fractional z {phase} {act} M={M} N={N} K={K} r={r} G={G}")
    cfg = synth.LAYERS["mlp_70b_bf16"] if act == "bf16" else synth.LAYERS["tiny"]
    d = synth.make_layer(cfg, M, seed=31, N=N, K=K, r=max(r, 8), group_size=G)
    codes = frac_codes(d, seed=M + K)
    packed = pack_host(*codes, N, K, G)
    q2, s2, z2 = w4.w4ec_unpack(packed, N, K, G)             # exact round trip
    torch().cuda.synchronize()
    assert np.array_equal(host_bits(z2), codes[2]) and np.array_equal(host_bits(s2), codes[1])
    assert np.array_equal(q2.cpu().numpy(), codes[0])
    Y = gpu_layer(d, packed, phase, r=r)
    rows = sample_rows(M)
    ref = oracle_layer(d, codes, r=r, rows=rows)
    assert_close(Y if rows is None else Y[rows], ref, act, f"fractional z {phase} {act} M={M}")


@pytest.mark.parametrize("phase,act,G", [("decode", "fp16", 512), ("prefill", "fp16", 128),
                                         ("prefill", "bf16", 512), ("decode", "bf16", 128),
                                         ("prefill", "fp16", 512), ("decode", "fp16", 128)])
def test_out_of_range_zero_point_gives_nan(phase, act, G):
    """A zero point beyond +-1024 (or not finite) is stored as NaN: the
    output column that uses it is NaN for every token, the others are right."""
    _print(f"out-of-range z {phase} {act} G={G}")
    t = torch()
    M = 3 if phase == "decode" else 80
    cfg = synth.LAYERS["mlp_70b_bf16"] if act == "bf16" else synth.LAYERS["tiny"]
    d = synth.make_layer(cfg, M, seed=5, N=272, K=512, r=8, group_size=G)
    qc, s, z = oracle.rtn_quantize(d["W"], G)
    ng = d["K"] // G
    bad_col = 7 // ng
    z2 = z.copy()
    z2.reshape(-1)[7] = np.float16(4096.0).view(np.uint16)
    z2.reshape(-1)[ng * 20] = np.float16(np.inf).view(np.uint16)     # column 20, group 0
    packed = pack_host(qc, s, z2, d["N"], d["K"], G)
    _, _, zu = w4.w4ec_unpack(packed, d["N"], d["K"], G)
    zu = host_bits(zu)
    assert np.isnan(zu.view(np.float16).astype(np.float32).reshape(-1)[[7, ng * 20]]).all()
    Y = gpu_layer(dict(d, M=M), packed, phase, r=0, expect_nan=True)
    Yf = synth.act_bits_to_f64(Y, act)
    assert np.isnan(Yf[:, [bad_col, 20]]).all()
    good = [n for n in range(d["N"]) if n not in (bad_col, 20)]
    ref = oracle_layer(d, (qc, s, z), r=0)
    assert_close(Y[:, good], ref[:, good], act, "columns with valid zero points")


@pytest.mark.parametrize("act,M,N,K,r", [
    ("fp16", 200, 528, 640, 16),       # 64-token tiles, K in one piece
    ("bf16", 100, 528, 512, 40),
    ("fp16", 96, 512, 4096, 64),       # 64-token tiles, K split in eight
    ("bf16", 1280, 2048, 1024, 32),    # 128-token tiles, K split in two
])
def test_zero_scale_columns_prefill(act, M, N, K, r):
    """A zero scale (a constant weight row, or a quantizer's choice) in a few
    columns: those weights are zero and the correction still applies, so
    those output columns hold the gated rank-r term alone.  Per-channel
    prefill tiles in one piece and split in K, 64- and 128-token tiles."""
    _print(f"zero scales prefill {act} M={M} N={N} K={K} r={r}")
    cfg = synth.LAYERS["mlp_70b_bf16"] if act == "bf16" else synth.LAYERS["tiny"]
    d = synth.make_layer(cfg, M, seed=17, N=N, K=K, r=r, group_size=K)
    qc, s, z = oracle.rtn_quantize(d["W"], K)
    s = s.copy()
    s[[5, 300, N - 1], :] = 0                  # tiles 0 and 1 and the last one
    packed = pack_host(qc, s, z, N, K, K)
    Y = gpu_layer(d, packed, "prefill", r=r)
    rows = sample_rows(M)
    ref = oracle_layer(d, (qc, s, z), r=r, rows=rows)
    Ys = Y if rows is None else Y[rows]
    assert_close(Ys, ref, act, f"zero scales {act} M={M}")
    # the zero-scale columns hold the correction alone
    assert np.abs(synth.act_bits_to_f64(Ys, act)[:, [5, 300, N - 1]]).max() > 0
