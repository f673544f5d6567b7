"""GPU parity of the codebook decode (XFP summary, sections 2 and 3: every
weight an index into its output channel's 16-entry fp16 codebook, plus a
sparse fp16 outlier residual), through the C ABI, against the float64
oracle, at the layer's tolerance.  Inputs: the layer's seeded weights with
planted outliers, turned into codebooks, indices and residual entries by
synth.make_xfp."""
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
    """indices uint8 [N, K] -> [N, K/2], even k in the low nibble (the
    canonical layout that w4ec_pack_xfp takes)."""
    idx = np.asarray(idx, dtype=np.uint8)
    return (idx[:, 0::2] | (idx[:, 1::2] << 4)).astype(np.uint8)


def xfp_layer(act, M, N, K, seed=0, frac=0.005, dense_row=None, k_sigma=4.0):
    cfg = "mlp_70b_bf16" if act == "bf16" else "tiny"
    d = synth.make_layer(cfg, M, seed=seed, N=N, K=K, r=8, group_size=K)
    W = synth.plant_outliers(d["W"], frac=frac, seed=seed)
    max_frac = 0.02
    if dense_row is not None:
        W[dense_row, ::16] = np.float32(0.5)              # one row with many outliers
        max_frac, k_sigma = 0.2, 2.5
    x = synth.make_xfp(W, k_sigma=k_sigma, max_frac=max_frac)
    x["qc"] = pack_nibbles(x["idx"])
    return d, x


def gpu_xfp(d, x):
    t = torch()
    N, K = d["N"], d["K"]
    qc = t.from_numpy(x["qc"]).cuda()
    packed = w4.w4ec_pack_xfp(qc, N, K)
    cb = t.from_numpy(x["cb"].view(np.int16)).view(t.float16).cuda()
    rp = t.from_numpy(x["row_ptr"]).cuda()
    nnz = int(x["row_ptr"][-1])
    ci = t.from_numpy(x["col_idx"]).cuda() if nnz else None
    val = t.from_numpy(x["val"].view(np.int16)).view(t.float16).cuda() if nnz else None
    X = dev_act(d["X"], d["act"])
    Y = nan_y(d["M"], N, d["act"])
    w4.w4ec_linear_decode_xfp(X, packed, cb, rp, ci, val, N=N, Y=Y)
    t.cuda.synchronize()
    assert_all_finite(Y, f"xfp M={d['M']}")
    return host_bits(Y)


def oracle_xfp(d, x):
    return oracle.forward_xfp(d["X"], x["qc"], x["cb"], x["row_ptr"], x["col_idx"], x["val"],
                              N=d["N"], K=d["K"], act=d["act"])["Y"]


CASES = [
    # act, M, N, K           (X in LDS for M <= 4 and M K <= 16384, else from L2)
    ("fp16", 1, 512, 512),
    ("fp16", 3, 528, 640),       # ragged column blocks
    ("fp16", 4, 1024, 4096),     # the largest activations staged in LDS
    ("fp16", 2, 512, 20480),     # one column block per workgroup, X from L2
    ("fp16", 5, 528, 1024),      # four column blocks per workgroup
    ("fp16", 16, 512, 512),
    ("bf16", 2, 272, 384),
    ("bf16", 8, 528, 1280),
    ("bf16", 1, 1024, 8192),
    ("fp16", 2, 1000, 512),      # N not a multiple of 16: a partial last column block
    ("bf16", 7, 1000, 640),
]


@pytest.mark.parametrize("act,M,N,K", CASES)
def test_xfp_decode_parity(act, M, N, K):
    _print(f"xfp decode {act} M={M} N={N} K={K}")
    d, x = xfp_layer(act, M, N, K, seed=M + N)
    assert int(x["row_ptr"][-1]) > 0
    assert_close(gpu_xfp(d, x), oracle_xfp(d, x), act, f"xfp {act} M={M} N={N} K={K}")


def test_xfp_no_outliers_and_a_dense_row():
    _print("xfp decode: no residual entries; one row with many")
    d, x = xfp_layer("fp16", 2, 512, 1024, seed=3, frac=0.0, k_sigma=1e9)
    assert int(x["row_ptr"][-1]) == 0
    assert_close(gpu_xfp(d, x), oracle_xfp(d, x), "fp16", "xfp nnz=0")
    d, x = xfp_layer("fp16", 3, 512, 1024, seed=4, dense_row=77)
    counts = np.diff(x["row_ptr"])
    assert counts[77] >= 64                            # several passes of the residual loop
    assert_close(gpu_xfp(d, x), oracle_xfp(d, x), "fp16", "xfp dense row")


def test_xfp_repeatable():
    _print("xfp decode: two calls, same bits")
    d, x = xfp_layer("fp16", 4, 528, 2048, seed=8)
    a = gpu_xfp(d, x)
    b = gpu_xfp(d, x)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("M", [1, 4, 16])
def test_xfp_decode_up_proj_full_size(M):
    """The 8B up-projection shape (N 14336, K 4096), every output checked."""
    _print(f"xfp decode up_proj M={M}")
    d, x = xfp_layer("fp16", M, 14336, 4096, seed=20 + M)
    assert_close(gpu_xfp(d, x), oracle_xfp(d, x), "fp16", f"xfp up_proj M={M}")
