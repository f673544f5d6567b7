"""GPU parity: the HIP path through the C ABI against the float64 oracle.

Codes are compared bit for bit; Y within
max|err| <= 2e-3 (fp16) / 1.6e-2 (bf16) * (max_n |Y_oracle[m, n]| + 1) per token.
Small cases span several tiles with ragged tails in M and N; the five
workload shapes run at full size with the oracle evaluating sampled tokens.
"""
import math

import numpy as np
import pytest

import oracle
import w4_gemm_error_amd as w4
from w4_gemm_error_amd import synth

from gpu_util import (assert_close, dev_act, gpu_layer, gpu_quantize, host_bits, new_workspace, oracle_layer,
                      sample_rows, torch)

pytestmark = pytest.mark.gpu


def _print(*a):
    print(*a, flush=True)


# ---------------------------------------------------------------- weight prep

@pytest.mark.parametrize("N,K,G", [(512, 512, 512), (300, 1024, 128), (37, 384, 128)])
def test_quantize_bit_exact(N, K, G):
    _print(f"quantize N={N} K={K} G={G}")
    d = synth.make_layer("tiny", 1, seed=3, N=N, K=K, group_size=G)
    q, s, z, _ = gpu_quantize(d)
    oq, os_, oz = oracle.rtn_quantize(d["W"], G)
    assert np.array_equal(q.cpu().numpy(), oq)
    assert np.array_equal(host_bits(s), os_)
    assert np.array_equal(host_bits(z), oz)


@pytest.mark.parametrize("N,K,G", [(37, 384, 128), (512, 512, 512), (64, 1024, 256)])
def test_pack_unpack_round_trip(N, K, G):
    _print(f"pack/unpack N={N} K={K} G={G}")
    t = torch()
    rng = np.random.default_rng(11)
    qc = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    qc.reshape(-1)[:256] = np.arange(256, dtype=np.uint8)        # every byte value
    s = rng.uniform(1e-3, 1e-1, size=(N, K // G)).astype(np.float16)
    z = rng.integers(0, 16, size=(N, K // G)).astype(np.float16)
    packed = w4.w4ec_pack(t.from_numpy(qc).cuda(), t.from_numpy(s).cuda(), t.from_numpy(z).cuda(), N, K, G)
    assert packed.numel() == w4.w4ec_packed_bytes(N, K, G)
    q2, s2, z2 = w4.w4ec_unpack(packed, N, K, G)
    t.cuda.synchronize()
    assert np.array_equal(q2.cpu().numpy(), qc)
    assert np.array_equal(s2.cpu().numpy().view(np.uint16), s.view(np.uint16))
    assert np.array_equal(z2.cpu().numpy().view(np.uint16), z.view(np.uint16))


# ---------------------------------------------------------------- small layers

SMALL = [
    # phase, act, M, N, K, r, G
    ("decode", "fp16", 1, 512, 512, 8, 512),
    ("decode", "fp16", 3, 528, 640, 72, 640),
    ("decode", "fp16", 16, 512, 512, 8, 128),
    ("decode", "bf16", 5, 272, 384, 40, 384),
    ("decode", "bf16", 16, 512, 512, 8, 128),
    ("decode", "fp16", 7, 48, 1280, 256, 256),
    ("decode", "fp16", 16, 512, 20480, 256, 20480),    # more K slices than EC workgroups
    ("decode", "bf16", 3, 512, 20480, 256, 1024),
    # the EC split by column blocks (1-4 tokens, K <= 4096, r a multiple of 16)
    ("decode", "fp16", 1, 512, 640, 16, 640),          # a partial 512-row round; zero words past r
    ("decode", "bf16", 4, 528, 4096, 48, 4096),
    ("decode", "fp16", 2, 272, 1024, 256, 128),
    ("prefill", "fp16", 17, 528, 640, 72, 640),
    ("prefill", "fp16", 300, 512, 512, 8, 512),
    ("prefill", "fp16", 129, 784, 1024, 64, 128),
    ("prefill", "bf16", 100, 528, 512, 40, 512),
    ("prefill", "bf16", 200, 512, 768, 16, 128),
    ("prefill", "fp16", 2, 512, 512, 8, 512),
    ("prefill", "fp16", 64, 1024, 2048, 130, 2048),
    # many tiles, ragged in M and N
    ("prefill", "fp16", 1000, 8000, 256, 16, 256),
    ("prefill", "bf16", 1030, 8008, 384, 24, 384),
    # 128-token tiles without a K split (one row block of tiles per 128
    # tokens, every workgroup a whole K): r = 64; r = 48 with the ranks of
    # r_pad past r and a ragged N; r = 96 over K = 2048
    ("prefill", "fp16", 1000, 4096, 768, 64, 768),
    ("prefill", "fp16", 1100, 4000, 896, 48, 896),
    ("prefill", "fp16", 700, 8192, 2048, 96, 2048),
    # a prepass of more than one round of workgroups: two chunks of K per
    # workgroup, the last one past K
    ("prefill", "fp16", 1100, 256, 8320, 128, 8320),
]


def small_layer(act, M, N, K, r, G, seed=5):
    cfg = synth.LAYERS["mlp_70b_bf16"] if act == "bf16" else synth.LAYERS["tiny"]
    return synth.make_layer(cfg, M, seed=seed, N=N, K=K, r=r, group_size=G)


@pytest.mark.parametrize("phase,act,M,N,K,r,G", SMALL)
def test_small_layer_parity(phase, act, M, N, K, r, G):
    _print(f"small {phase} {act} M={M} N={N} K={K} r={r} G={G}")
    d = small_layer(act, M, N, K, r, G)
    q, s, z, packed = gpu_quantize(d)
    codes = oracle.rtn_quantize(d["W"], G)
    assert np.array_equal(q.cpu().numpy(), codes[0])
    Y = gpu_layer(d, packed, phase)
    ref = oracle_layer(d, codes)
    assert_close(Y, ref, act, f"{phase} {act} M={M}")


@pytest.mark.parametrize("phase,M,r", [("decode", 9, 24), ("decode", 2, 32), ("prefill", 40, 24)])
def test_special_cases(phase, M, r):
    _print(f"special cases {phase} M={M} r={r}")
    d = small_layer("fp16", M, 528, 512, r, 512, seed=8)
    _, _, _, packed = gpu_quantize(d)
    codes = oracle.rtn_quantize(d["W"], 512)
    plain = gpu_layer(d, packed, phase, r=0)
    assert_close(plain, oracle_layer(d, codes, r=0), "fp16", "r=0")
    closed = gpu_layer(d, packed, phase, b_g=-math.inf)
    assert np.array_equal(synth.act_bits_to_f64(closed, "fp16"), synth.act_bits_to_f64(plain, "fp16"))
    opened = gpu_layer(d, packed, phase, b_g=math.inf, with_gate=False)
    assert_close(opened, oracle_layer(d, codes, b_g=math.inf, with_gate=False), "fp16", "g=1")
    nogate = gpu_layer(d, packed, phase, b_g=0.25, with_gate=False)
    assert_close(nogate, oracle_layer(d, codes, b_g=0.25, with_gate=False), "fp16", "w_g=None")


def test_special_cases_many_tiles():
    # M=1000, N=4096, K=768: 128-token tiles without a K split
    _print("special cases prefill M=1000 N=4096 K=768 r=64 (128-token tiles)")
    d = small_layer("fp16", 1000, 4096, 768, 64, 768, seed=8)
    _, _, _, packed = gpu_quantize(d)
    codes = oracle.rtn_quantize(d["W"], 768)
    plain_ref = oracle_layer(d, codes, r=0)
    closed = gpu_layer(d, packed, "prefill", b_g=-math.inf)
    assert_close(closed, plain_ref, "fp16", "g=0")
    opened = gpu_layer(d, packed, "prefill", b_g=math.inf, with_gate=False)
    assert_close(opened, oracle_layer(d, codes, b_g=math.inf, with_gate=False), "fp16", "g=1")
    # repeated calls on one workspace (each leaves the hand-over state at
    # zero, which gpu_layer checks), bit for bit the same
    ws = new_workspace(w4.w4ec_workspace_bytes(d["M"], d["N"], d["K"], d["r"], d["group_size"]))
    nogate = gpu_layer(d, packed, "prefill", b_g=0.25, with_gate=False, workspace=ws)
    assert_close(nogate, oracle_layer(d, codes, b_g=0.25, with_gate=False), "fp16", "w_g=None")
    again = gpu_layer(d, packed, "prefill", b_g=0.25, with_gate=False, workspace=ws)
    assert np.array_equal(again, nogate)


@pytest.mark.parametrize("M,K,G", [(64, 512, 512), (130, 1024, 1024), (40, 768, 256)])
def test_bf16_prefill_plain_w4(M, K, G):
    """bf16 prefill with r = 0: the per-channel path subtracts the zero point
    through each token's activation sum, which the prepass computes even
    without a compensator; the grouped path dequantizes exactly."""
    _print(f"bf16 prefill r=0 M={M} K={K} G={G}")
    d = small_layer("bf16", M, 528, K, 16, G, seed=13)
    _, _, _, packed = gpu_quantize(d)
    codes = oracle.rtn_quantize(d["W"], G)
    Y = gpu_layer(d, packed, "prefill", r=0)
    assert_close(Y, oracle_layer(d, codes, r=0), "bf16", f"bf16 r=0 M={M}")


@pytest.mark.parametrize("phase,M", [("decode", 16), ("prefill", 256)])
def test_deterministic_and_workspace_reuse(phase, M):
    _print(f"determinism {phase} M={M}")
    t = torch()
    d = synth.make_layer("batched_down_proj_8b_g128", M, seed=2, N=1024, K=2048)   # group 128, split-K in prefill
    _, _, _, packed = gpu_quantize(d)
    ws = t.zeros(w4.w4ec_workspace_bytes(M, d["N"], d["K"], d["r"], d["group_size"]),
                 dtype=t.uint8, device="cuda")
    first = gpu_layer(d, packed, phase, workspace=ws)
    for _ in range(5):
        again = gpu_layer(d, packed, phase, workspace=ws)
        assert np.array_equal(again, first)
    # hand-over state (flags, counters, data) is back at zero, no wait timed out
    assert int(t.count_nonzero(ws[: w4.W4EC_WS_STATE_BYTES]).item()) == 0


def test_phase_dispatch_agrees():
    _print("decode vs prefill on the same 16 tokens")
    d = small_layer("fp16", 16, 512, 1024, 32, 1024, seed=9)
    _, _, _, packed = gpu_quantize(d)
    a = synth.act_bits_to_f64(gpu_layer(d, packed, "decode"), "fp16")
    b = synth.act_bits_to_f64(gpu_layer(d, packed, "prefill"), "fp16")
    ref = oracle_layer(d, oracle.rtn_quantize(d["W"], 1024))
    bound = 2e-3 * (np.abs(ref).max(axis=1, keepdims=True) + 1.0)
    assert (np.abs(a - b) <= 2 * bound).all()


def test_special_cases_full_size_decode():
    """The 8B up-projection at one token (N 14336, K 4096, r 64): the plain
    W4 layer (r = 0), a closed gate (b_g = -inf: the plain layer, bitwise),
    and a fully open gate with no gate vector (the static compensation)."""
    _print("special cases, decode_up_proj_8b M=1")
    d = synth.make_layer("decode_up_proj_8b", 1, seed=0)
    _, _, _, packed = gpu_quantize(d)
    codes = oracle.rtn_quantize(d["W"], d["group_size"])
    plain = gpu_layer(d, packed, "decode", r=0)
    assert_close(plain, oracle_layer(d, codes, r=0), "fp16", "r=0")
    closed = gpu_layer(d, packed, "decode", b_g=-math.inf)
    assert np.array_equal(synth.act_bits_to_f64(closed, "fp16"), synth.act_bits_to_f64(plain, "fp16"))
    opened = gpu_layer(d, packed, "decode", b_g=math.inf, with_gate=False)
    assert_close(opened, oracle_layer(d, codes, b_g=math.inf, with_gate=False), "fp16", "g=1")


# ---------------------------------------------------------------- full-size workloads

FULL = [
    # cfg, M, phase (every token of Y must be finite; the oracle checks all
    # tokens up to 64 and a token in every row tile beyond: sample_rows)
    ("tiny", 16, "decode"),
    ("decode_up_proj_8b", 1, "decode"),
    ("decode_up_proj_8b", 4, "decode"),
    ("decode_up_proj_8b", 16, "decode"),
    ("prefill_out_proj_8b", 2048, "prefill"),
    ("batched_down_proj_8b_g128", 256, "prefill"),
    ("mlp_70b_bf16", 64, "prefill"),
    ("mlp_70b_bf16", 4096, "prefill"),
]


@pytest.mark.parametrize("cfg,M,phase", FULL)
def test_full_size_parity(cfg, M, phase):
    rows = sample_rows(M)
    _print(f"full {cfg} M={M} {phase} rows={'all' if rows is None else len(rows)}")
    d = synth.make_layer(cfg, M, seed=0)
    q, s, z, packed = gpu_quantize(d)
    codes = oracle.rtn_quantize(d["W"], d["group_size"])
    assert np.array_equal(q.cpu().numpy(), codes[0])
    assert np.array_equal(host_bits(s), codes[1]) and np.array_equal(host_bits(z), codes[2])
    del q, s, z
    Y = gpu_layer(d, packed, phase)
    ref = oracle_layer(d, codes, rows=rows)
    Ysub = Y if rows is None else Y[rows]
    worst = assert_close(Ysub, ref, d["act"], f"{cfg} M={M}")
    _print(f"  worst err/tol {worst:.3f}")


def test_shared_workspace_across_shapes_and_phases():
    """One workspace serves interleaved decode / prefill calls of different
    ranks and shapes: every call's counters and flags must be back at zero."""
    _print("shared workspace")
    t = torch()
    layers = []
    for (M, N, K, r, G) in [(1, 528, 512, 64, 512), (16, 512, 1024, 128, 128), (40, 512, 512, 8, 512),
                            (3, 256, 768, 256, 256), (200, 784, 1024, 64, 128)]:
        d = small_layer("fp16", M, N, K, r, G, seed=M + r)
        _, _, _, packed = gpu_quantize(d)
        layers.append((d, packed))
    need = max(w4.w4ec_workspace_bytes(d["M"], d["N"], d["K"], d["r"], d["group_size"]) for d, _ in layers)
    ws = t.zeros(need, dtype=t.uint8, device="cuda")
    ref = {}
    for i, (d, packed) in enumerate(layers):
        for phase in ("decode", "prefill"):
            if phase == "decode" and d["M"] > 16:
                continue
            ref[(i, phase)] = gpu_layer(d, packed, phase)          # own fresh workspace
    for rep in range(3):
        for (i, phase), y in ref.items():
            d, packed = layers[i]
            got = gpu_layer(d, packed, phase, workspace=ws)
            assert np.array_equal(got, y), (i, phase, rep)
