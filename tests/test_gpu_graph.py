"""GPU: the layer captured into a HIP graph and replayed, as bench.py times it.

Each case runs the layer once eagerly, then captures the same call (into a
NaN-filled output, on a workspace allocated before the capture) into a
torch.cuda.CUDAGraph and replays it several times.  Between replays the
program does eager work of its own -- another layer call on a second
workspace, a torch kernel, a synchronization -- and every replay must give
the eager output bit for bit (the kernels add their partial sums in a fixed
order) and leave the hand-over state at zero.  The eager output itself is
checked against the oracle (SPEAR summary section 2.1A: Y = X Wd^T + g (X A)
B).  The cases cover each launch structure of the timed path: the decode
kernel with its EC role (one token on the full 8B up-projection, the
headline shape), the prefill with the prepass and reduction ahead of the
GEMM (split K and not), and the prefill whose GEMM workgroups compute the
EC themselves.
"""
import numpy as np
import pytest

import oracle
import w4_gemm_error_amd as w4
from w4_gemm_error_amd import synth

from gpu_util import assert_close, dev_act, gpu_quantize, host_bits, new_workspace, oracle_layer, sample_rows, torch

pytestmark = pytest.mark.gpu

REPLAYS = 4

CASES = [
    # name, cfg, phase, M, N, K, r, G (None: the config's own shape)
    ("decode_up_proj_8b_m1", "decode_up_proj_8b", "decode", 1, None, None, None, None),
    ("decode_m4_grouped", "tiny", "decode", 4, 4096, 2048, 64, 128),
    ("prefill_m300", "tiny", "prefill", 300, 1024, 1024, 64, 1024),          # prepass + reduce, split K
    ("prefill_m1000_k768", "tiny", "prefill", 1000, 4096, 768, 64, 768),     # 128-token tiles, no split
    ("prefill_m40_fused", "tiny", "prefill", 40, 784, 2048, 64, 2048),       # the EC inside the GEMM
    ("prefill_bf16_m200", "mlp_70b_bf16", "prefill", 200, 1024, 1024, 32, 1024),
]


def _print(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("name,cfg,phase,M,N,K,r,G", CASES, ids=[c[0] for c in CASES])
def test_graph_replay_matches_eager_and_oracle(name, cfg, phase, M, N, K, r, G):
    _print(f"graph replay {name}: {phase} M={M}")
    t = torch()
    d = synth.make_layer(cfg, M, seed=41, N=N, K=K, r=r, group_size=G)
    act = d["act"]
    N, K, r, G = d["N"], d["K"], d["r"], d["group_size"]
    _, _, _, packed = gpu_quantize(d)
    X, A, B, wg = (dev_act(d[k], act) for k in ("X", "A", "B", "w_g"))
    fn = w4.w4ec_linear_decode if phase == "decode" else w4.w4ec_linear_prefill
    dtype = t.float16 if act == "fp16" else t.bfloat16
    nbytes = w4.w4ec_workspace_bytes(M, N, K, r, G)
    ws = new_workspace(nbytes)
    ws_other = new_workspace(nbytes)

    # eager reference, checked against the oracle
    Ye = t.full((M, N), float("nan"), dtype=dtype, device="cuda")
    fn(X, packed, A, B, wg, d["b_g"], N=N, group_size=G, workspace=ws, Y=Ye)
    t.cuda.synchronize()
    eager = host_bits(Ye)
    rows = sample_rows(M)
    ref = oracle_layer(d, oracle.rtn_quantize(d["W"], G), rows=rows)
    assert_close(eager if rows is None else eager[rows], ref, act, f"{name} eager")

    # capture: the output is NaN-filled inside the graph, then written
    Yg = t.empty((M, N), dtype=dtype, device="cuda")
    side = t.cuda.Stream()
    side.wait_stream(t.cuda.current_stream())
    graph = t.cuda.CUDAGraph()
    with t.cuda.stream(side):
        with t.cuda.graph(graph):
            Yg.fill_(float("nan"))
            fn(X, packed, A, B, wg, d["b_g"], N=N, group_size=G, workspace=ws, Y=Yg)
    t.cuda.current_stream().wait_stream(side)
    t.cuda.synchronize()

    scratch = t.randn(1 << 20, device="cuda")
    for rep in range(REPLAYS):
        graph.replay()
        t.cuda.synchronize()
        got = host_bits(Yg)
        assert np.array_equal(got, eager), f"{name}: replay {rep} differs from the eager call"
        state = ws[: w4.W4EC_WS_STATE_BYTES]
        assert int(t.count_nonzero(state).item()) == 0, f"{name}: hand-over state not at zero after replay {rep}"
        # the program's own eager work between replays
        Yo = t.empty((M, N), dtype=dtype, device="cuda")
        fn(X, packed, A, B, wg, d["b_g"], N=N, group_size=G, workspace=ws_other, Y=Yo)
        scratch.mul_(1.0001).add_(0.5)
        t.cuda.synchronize()
        assert np.array_equal(host_bits(Yo), eager), f"{name}: eager call {rep} between replays differs"
    assert w4.w4ec_workspace_status(ws) == w4.W4EC_OK
