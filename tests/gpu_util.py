"""Shared helpers for the GPU parity tests: move seeded inputs to the GPU,
run the HIP path through the C ABI binding, run the oracle on the same
inputs, and compare to the stated tolerance."""
import numpy as np

import oracle
import w4_gemm_error_amd as w4
from w4_gemm_error_amd import synth

# max |Y_gpu - Y_oracle| <= TOL * (max_n |Y_oracle[m, n]| + 1), per token m.
# fp16: fp32 accumulation, fp16 output rounding.  bf16: 8x wider, the ratio
# of the two formats' unit roundoffs (2^-8 / 2^-11): rounding the exact
# result to bf16 alone already exceeds the fp16 bound.
TOL = {"fp16": 2e-3, "bf16": 1.6e-2}


def torch():
    import torch as t
    return t


def dev_act(bits, act):
    t = torch()
    x = t.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return x.view(t.float16 if act == "fp16" else t.bfloat16).cuda()


def host_bits(tensor):
    t = torch()
    return tensor.detach().cpu().contiguous().view(t.int16).numpy().view(np.uint16)


def act_f64(bits, act):
    return synth.act_bits_to_f64(bits, act)


def gpu_quantize(d):
    t = torch()
    W = t.from_numpy(d["W"]).cuda()
    q, s, z = w4.w4ec_quantize_rtn(W, d["group_size"])
    packed = w4.w4ec_pack(q, s, z, d["N"], d["K"], d["group_size"])
    del W
    return q, s, z, packed


def nan_y(M, N, act):
    """An output buffer filled with NaN, so that an element the kernels never
    write cannot pass as a result left over from an earlier call."""
    t = torch()
    return t.full((M, N), float("nan"), dtype=t.float16 if act == "fp16" else t.bfloat16, device="cuda")


def poison_workspace(ws):
    """Fill the per-call part of a workspace (past the hand-over state,
    which must stay zero between calls) with 0xFF bytes: NaN as fp16, bf16
    and fp32, so that data a kernel reads before writing it shows up."""
    if ws.numel() > w4.W4EC_WS_STATE_BYTES:
        ws[w4.W4EC_WS_STATE_BYTES:].fill_(0xFF)
    return ws


def new_workspace(nbytes):
    t = torch()
    return poison_workspace(t.zeros(max(nbytes, 256), dtype=t.uint8, device="cuda"))


def assert_all_finite(Y, what=""):
    """Every element of Y (device tensor) is finite: no tile left unwritten."""
    t = torch()
    bad = int((~t.isfinite(Y.float())).sum().item())
    assert bad == 0, f"{what}: {bad} non-finite output elements"


def sample_rows(M):
    """Tokens compared against the oracle at full size: every token up to 64;
    one per 16-token MFMA block up to 256; beyond that one per 64 (M <= 2048)
    or 128 tokens -- a token in every GEMM row tile -- placed so that the
    16-token block hit inside a 128-token tile cycles through all eight from
    tile to tile, at a lane row that moves too; plus the last token."""
    if M <= 64:
        return None
    if M <= 256:
        rows = [16 * b + (b * 5) % 16 for b in range((M + 15) // 16)]
    else:
        span = 64 if M <= 2048 else 128
        per = 128 // span
        nb = span // 16
        rows = []
        for T in range((M + 127) // 128):
            for h in range(per):
                blk = h * nb + (T + 2 * h) % nb
                rows.append(T * 128 + 16 * blk + (7 * T + 3 * h) % 16)
    rows.append(M - 1)
    return sorted(set(min(x, M - 1) for x in rows))


def gpu_layer(d, packed, phase, *, r=None, b_g=None, with_gate=True, workspace=None, expect_nan=False):
    act = d["act"]
    r = d["r"] if r is None else r
    X = dev_act(d["X"], act)
    A = dev_act(d["A"][:, :r], act) if r > 0 else None
    B = dev_act(d["B"][:r], act) if r > 0 else None
    wg = dev_act(d["w_g"], act) if (r > 0 and with_gate) else None
    bg = d["b_g"] if b_g is None else b_g
    fn = w4.w4ec_linear_decode if phase == "decode" else w4.w4ec_linear_prefill
    if workspace is None:
        workspace = new_workspace(w4.w4ec_workspace_bytes(d["M"], d["N"], d["K"], r, d["group_size"]))
    else:
        poison_workspace(workspace)
    Y = nan_y(d["M"], d["N"], act)
    fn(X, packed, A, B, wg, bg, N=d["N"], group_size=d["group_size"], workspace=workspace, Y=Y)
    torch().cuda.synchronize()
    if not expect_nan:
        assert_all_finite(Y, f"{phase} M={d['M']}")
    # every call leaves the hand-over state at zero; a nonzero byte there
    # would mean that a bounded wait timed out
    state = workspace[: w4.W4EC_WS_STATE_BYTES]
    assert int(torch().count_nonzero(state).item()) == 0, f"{phase}: hand-over state not at zero after the call"
    return host_bits(Y)


def oracle_layer(d, codes, *, r=None, b_g=None, with_gate=True, rows=None):
    qc, s, z = codes
    r = d["r"] if r is None else r
    A = d["A"][:, :r] if r > 0 else None
    B = d["B"][:r] if r > 0 else None
    wg = d["w_g"] if with_gate else None
    bg = d["b_g"] if b_g is None else b_g
    return oracle.forward(d["X"], qc, s, z, A, B, wg, bg, N=d["N"], K=d["K"], r=r,
                          group_size=d["group_size"], act=d["act"], rows=rows, want_parts=False)["Y"]


def assert_close(Y_bits, Y_ref, act, what=""):
    Yg = act_f64(Y_bits, act)
    assert Yg.shape == Y_ref.shape, (Yg.shape, Y_ref.shape)
    assert np.isfinite(Yg).all(), f"{what}: non-finite output"
    bound = TOL[act] * (np.abs(Y_ref).max(axis=1, keepdims=True) + 1.0)
    ratio = np.abs(Yg - Y_ref) / bound
    worst = np.unravel_index(np.argmax(ratio), ratio.shape)
    assert ratio.max() <= 1.0, (f"{what}: max err/tol {ratio.max():.3f} at {worst}: "
                                f"gpu {Yg[worst]:.6g} oracle {Y_ref[worst]:.6g}")
    return float(ratio.max())
