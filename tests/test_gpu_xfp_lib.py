"""GPU parity of the shared-library codebook decode (XFP summary, section 2,
shared-library mode: L codebooks of 16 fp16 entries per layer, each group of
128 weights of an output channel naming its entry, plus the sparse fp16
outlier residual), through the C ABI, against the float64 oracle at the
layer's tolerance.  Inputs: the layer's seeded weights with planted
outliers, encoded by synth.make_xfp_lib."""
import numpy as np
import pytest

import oracle
import w4_gemm_error_amd as w4
from w4_gemm_error_amd import synth

from gpu_util import assert_all_finite, assert_close, dev_act, host_bits, nan_y, torch

pytestmark = pytest.mark.gpu


def _print(*a):
    print(*a, flush=True)


def pack_nibbles(idx):
    idx = np.asarray(idx, dtype=np.uint8)
    return (idx[:, 0::2] | (idx[:, 1::2] << 4)).astype(np.uint8)


def lib_layer(act, M, N, K, L, seed=0, frac=0.005):
    cfg = "mlp_70b_bf16" if act == "bf16" else "tiny"
    d = synth.make_layer(cfg, M, seed=seed, N=N, K=K, r=8, group_size=K)
    W = synth.plant_outliers(d["W"], frac=frac, seed=seed)
    # channels of different spreads, so that the groups name many entries
    W = W * np.exp(np.random.default_rng(seed + 1).normal(0.0, 0.5, (N, 1))).astype(np.float32)
    x = synth.make_xfp_lib(W, L=L)
    x["qc"] = pack_nibbles(x["idx"])
    return d, x


def gpu_lib(d, x):
    t = torch()
    N, K = d["N"], d["K"]
    packed = w4.w4ec_pack_xfp(t.from_numpy(x["qc"]).cuda(), N, K)
    library = t.from_numpy(x["lib"].view(np.int16)).view(t.float16).cuda()
    libid = t.from_numpy(x["libid"]).cuda()
    rp = t.from_numpy(x["row_ptr"]).cuda()
    nnz = int(x["row_ptr"][-1])
    ci = t.from_numpy(x["col_idx"]).cuda() if nnz else None
    val = t.from_numpy(x["val"].view(np.int16)).view(t.float16).cuda() if nnz else None
    X = dev_act(d["X"], d["act"])
    Y = nan_y(d["M"], N, d["act"])
    w4.w4ec_linear_decode_xfp_lib(X, packed, library, libid, rp, ci, val, N=N, Y=Y)
    t.cuda.synchronize()
    assert_all_finite(Y, f"xfp lib M={d['M']}")
    return host_bits(Y)


def oracle_lib(d, x):
    return oracle.forward_xfp_lib(d["X"], x["qc"], x["lib"], x["libid"], x["row_ptr"], x["col_idx"], x["val"],
                                  N=d["N"], K=d["K"], act=d["act"])["Y"]


CASES = [
    # act, M, N, K, L      (X in LDS for M <= 4 and M K <= 16384, else from L2)
    ("fp16", 1, 512, 512, 32),
    ("fp16", 3, 528, 640, 32),       # ragged column blocks
    ("fp16", 4, 1024, 4096, 17),     # the largest activations staged in LDS
    ("fp16", 2, 512, 20480, 32),     # one column block per workgroup, X from L2
    ("fp16", 5, 528, 1024, 8),       # more tokens: two column blocks per workgroup, X from L2
    ("fp16", 16, 512, 512, 32),
    ("fp16", 1, 272, 256, 1),        # a single codebook
    ("bf16", 2, 272, 384, 32),
    ("bf16", 8, 528, 1280, 5),
    ("bf16", 1, 1024, 8192, 32),
    ("fp16", 2, 1000, 512, 32),      # a partial last column block
    ("bf16", 7, 1000, 640, 32),
]


@pytest.mark.parametrize("act,M,N,K,L", CASES)
def test_xfp_lib_parity(act, M, N, K, L):
    _print(f"xfp lib parity {act} M={M} N={N} K={K} L={L}")
    d, x = lib_layer(act, M, N, K, L, seed=M + N + L)
    if L > 1:
        assert len(np.unique(x["libid"])) > 1
    assert_close(gpu_lib(d, x), oracle_lib(d, x), act, f"xfp lib {act} M={M} N={N} K={K} L={L}")


def test_xfp_lib_full_size_decode_up_proj():
    """The 8B up-projection (N = 14336, K = 4096), one token, 32 entries."""
    _print("xfp lib full size M=1 N=14336 K=4096 L=32")
    d, x = lib_layer("fp16", 1, 14336, 4096, 32, seed=3)
    assert_close(gpu_lib(d, x), oracle_lib(d, x), "fp16", "xfp lib full size")


def test_xfp_lib_single_shared_codebook_equals_per_channel_mode():
    """One library entry for every group, and the per-channel mode with that
    entry as every channel's codebook: the same weights and the same sums,
    so the two kernels agree bit for bit."""
    _print("xfp lib L=1 vs per-channel, M=2 N=528 K=1024")
    t = torch()
    d, x = lib_layer("fp16", 2, 528, 1024, 1, seed=11)
    N, K = d["N"], d["K"]
    packed = w4.w4ec_pack_xfp(t.from_numpy(x["qc"]).cuda(), N, K)
    cb = np.repeat(x["lib"], N, axis=0)
    cbd = t.from_numpy(np.ascontiguousarray(cb).view(np.int16)).view(t.float16).cuda()
    rp = t.from_numpy(x["row_ptr"]).cuda()
    nnz = int(x["row_ptr"][-1])
    ci = t.from_numpy(x["col_idx"]).cuda() if nnz else None
    val = t.from_numpy(x["val"].view(np.int16)).view(t.float16).cuda() if nnz else None
    Y = nan_y(2, N, "fp16")
    w4.w4ec_linear_decode_xfp(dev_act(d["X"], "fp16"), packed, cbd, rp, ci, val, N=N, Y=Y)
    t.cuda.synchronize()
    assert np.array_equal(host_bits(Y), gpu_lib(d, x))
