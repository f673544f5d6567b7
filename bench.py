#!/usr/bin/env python3
"""Benchmark of the W4 + EC linear layer (libw4ec) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-graph]

One step is one call of the layer -- every stage of the hot path: the gate
and X A pass, the int4 weight stream and dequantization, the main
contraction and the gated rank-r epilogue -- over one batch of seeded
synthetic tokens, with all inputs resident in HBM.  The packed weights and
EC parameters are replicated R times (R x layer bytes >= 512 MB, twice the
256 MB Infinity Cache) and the steps cycle through the copies, so every
step streams its weights from HBM.

Prints one JSON line: the whole-job rate (decode: algorithmic HBM GB/s;
prefill: TFLOP/s), the roofline that binds the call (HBM or MFMA, whichever
takes longer at its peak) from the HIP events that bracket the timed region,
and the float64 CPU oracle timed on a bounded sample on the host.  Without
--workload the line is the one-token decode of the 8B up-projection, and its
"prefill" object times the 2048-token prefill of the 8B out-projection in
the same run: the metric's two halves.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
MFMA_PEAK_TFLOPS = {"fp16": 2500.0, "bf16": 2500.0}   # dense fp16 / bf16 MFMA
MALL_BYTES = 256 << 20

# name -> (synthetic layer, tokens, entry point)
WORKLOADS = {
    "decode_up_proj_8b_m1": ("decode_up_proj_8b", 1, "decode"),
    "decode_up_proj_8b_m4": ("decode_up_proj_8b", 4, "decode"),
    "decode_up_proj_8b_m16": ("decode_up_proj_8b", 16, "decode"),
    "tiny_m16": ("tiny", 16, "decode"),
    "prefill_out_proj_8b_m2048": ("prefill_out_proj_8b", 2048, "prefill"),
    "batched_down_proj_8b_g128_m256": ("batched_down_proj_8b_g128", 256, "prefill"),
    "mlp_70b_bf16_m64": ("mlp_70b_bf16", 64, "prefill"),
    "mlp_70b_bf16_m4096": ("mlp_70b_bf16", 4096, "prefill"),
}
DEFAULT_WORKLOAD = "decode_up_proj_8b_m1"
PREFILL_WORKLOAD = "prefill_out_proj_8b_m2048"   # the prefill half of the default line


def layer_bytes(M, N, K, r, G, has_gate=True, h=0):
    """Algorithmic HBM bytes of one call: packed codes, scale/zero, X, Y, A,
    B and the gate parameters (w_g, or with a vector gate of width h its
    G1, c1, G2, c2), each moved once (the dequantized weights are never
    stored)."""
    codes = N * K // 2
    sz = N * (K // G) * 4
    act = 2
    gate = (2 * r * h + h + r) * act if h else (K * act if has_gate else 0)
    return codes + sz + M * K * act + M * N * act + (K * r + r * N) * act + gate


def layer_flops(M, N, K, r, h=0):
    """2MNK main product + 2MK(r+1) gate and X A (with a vector gate of width
    h: 2MKr for X A and 4Mrh for its bottleneck) + 2MrN rank-r product + 2MN
    gating/add."""
    gate = 2 * M * K * r + 4 * M * r * h if h else 2 * M * K * (r + 1)
    return 2 * M * N * K + gate + 2 * M * r * N + 2 * M * N


def roofline(nbytes, flops, seconds, act):
    """The binding roofline of one call: HBM if moving its algorithmic bytes
    at 8 TB/s takes longer than its algorithmic flops at the dense MFMA
    peak, else MFMA; `achieved` is the rate in that roofline's unit."""
    t_hbm = nbytes / (HBM_PEAK_GBS * 1e9)
    t_mfma = flops / (MFMA_PEAK_TFLOPS[act] * 1e12)
    if t_hbm >= t_mfma:
        achieved = nbytes / seconds / 1e9
        return {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4)}
    achieved = flops / seconds / 1e12
    peak = MFMA_PEAK_TFLOPS[act]
    return {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4)}


# the sources each measured kernel is built from (its counters stay valid
# while these are unchanged)
KERNEL_SOURCES = {
    "decode_kernel": ["decode.hip", "ec_tile.h", "w4ec_common.h", "w4ec_launch.h", "api.cpp"],
    "prefill_call": ["prefill.hip", "ec_tile.h", "w4ec_common.h", "w4ec_launch.h", "api.cpp"],
}


def source_digest(kernel):
    """Digest of a kernel's sources' code: line comments and blank lines are
    left out, so that a comment edit does not invalidate measured counters."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "w4_gemm_error_amd", "csrc")
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(csrc, name), encoding="utf-8") as f:
            code = [ln.split("//", 1)[0].rstrip() for ln in f]
        h.update(name.encode() + "\n".join(ln for ln in code if ln).encode())
    return h.hexdigest()[:16]


def traffic_from_profiles(kernel_key):
    """Measured HBM bytes per launch from the committed counter summary, if
    it was taken on the kernel as it is now (same source digest)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            table = json.load(f)
    except (OSError, ValueError):
        return None
    e = table.get(kernel_key)
    if not e or e.get("source_digest") != source_digest(kernel_key.split("/")[0]):
        return None
    return e.get("bytes_per_launch")


def host_cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or "unknown"."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(d, phase, budget_s):
    """The float64 oracle on the host, on a bounded sample of the workload."""
    import oracle
    qc, s, z = oracle.rtn_quantize(d["W"], d["group_size"])   # offline step, untimed
    M, N, K, r, G = d["M"], d["N"], d["K"], d["r"], d["group_size"]
    rows_per_call = M
    rows = None
    if M > 1:
        # evaluate a prefix of the tokens: the oracle's cost is linear in them
        est = N * K * 1.5e-9 / max(oracle.max_threads(), 1)   # ~s per token
        rows_per_call = int(max(1, min(M, budget_s / 3 / max(est, 1e-9))))
        rows = list(range(rows_per_call))
    n, t0 = 0, time.perf_counter()
    while True:
        oracle.forward(d["X"], qc, s, z, d["A"], d["B"], d["w_g"], d["b_g"], N=N, K=K, r=r,
                       group_size=G, act=d["act"], rows=rows, want_parts=False)
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s or n >= 1000:
            break
    per_call = el / n
    frac = rows_per_call / M
    if phase == "decode":
        value = layer_bytes(rows_per_call, N, K, r, G) / per_call / 1e9
        unit = "GB/s"
    else:
        value = layer_flops(rows_per_call, N, K, r) / per_call / 1e12
        unit = "TFLOP/s"
    sample = (f"{n} oracle call(s) of {rows_per_call} of {M} token(s) "
              f"({frac:.3g} of the batch), {el:.1f} s total, weights quantized beforehand, "
              f"host CPU: {host_cpu_model()}")
    return {"value": round(value, 6), "unit": unit, "cores": int(oracle.max_threads()),
            "kind": "oracle", "sample": sample}


def split_prefill_step(torch, w4, path, X, Y, copies, R, b_g, M, N, K, r, G):
    """One call of the unfused ("unfused": one stream) or semi-fused ("semi":
    the gate step on a second stream beside the GEMM) prefill: T_g into an EC
    workspace, the plain W4 GEMM into Y, then Y += T_g B."""
    dev = X.device
    ws_ec = torch.zeros(w4.w4ec_prefill_ec_workspace_bytes(M, K, r), dtype=torch.uint8, device=dev)
    ws_mm = torch.zeros(max(w4.w4ec_workspace_bytes(M, N, K, 0, G), 256), dtype=torch.uint8, device=dev)
    side = torch.cuda.Stream() if path == "semi" else None

    def step(i):
        p, A, B, wg = copies[i % R]
        if side is not None:
            cur = torch.cuda.current_stream()
            side.wait_stream(cur)
            with torch.cuda.stream(side):
                w4.w4ec_prefill_ec_gate(X, A, wg, b_g, workspace=ws_ec)
            w4.w4ec_linear_prefill(X, p, None, None, None, 0.0, N=N, group_size=G, workspace=ws_mm, Y=Y)
            cur.wait_stream(side)
        else:
            w4.w4ec_prefill_ec_gate(X, A, wg, b_g, workspace=ws_ec)
            w4.w4ec_linear_prefill(X, p, None, None, None, 0.0, N=N, group_size=G, workspace=ws_mm, Y=Y)
        w4.w4ec_prefill_ec_apply(Y, B, K=K, workspace=ws_ec)
    return step


def graph_time_us(torch, step, steps, warmup, reps=1):
    """Microseconds per step of `steps` calls captured in one graph (after
    `warmup` eager calls and one untimed replay; the best of `reps` timed
    replays)."""
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            for i in range(steps):
                step(i)
    torch.cuda.current_stream().wait_stream(stream)
    graph.replay()
    torch.cuda.synchronize()
    best = None
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        graph.replay()
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) * 1e3 / steps
        best = t if best is None else min(best, t)
    return best


def latency_table(torch, w4, synth, dev):
    """Per-call latency of the fused, unfused and semi-fused prefill over a
    grid of shapes: the input of an EC-aware scheduler that picks a path per
    (M, r, N, K) (SPEAR summary, section 2.2A)."""
    shapes = [(4096, 4096), (14336, 4096), (4096, 14336)]
    for (N, K) in shapes:
        W = torch.randn(N, K, device=dev) * 0.02
        q, s, z = w4.w4ec_quantize_rtn(W, K)
        packed = w4.w4ec_pack(q, s, z, N, K, K)
        del W, q, s, z
        R = max(2, -(-2 * MALL_BYTES // packed.numel()))
        pk = [packed] + [packed.clone() for _ in range(R - 1)]
        for M in (64, 256, 1024, 4096):
            X = (torch.randn(M, K, device=dev)).half()
            Y = torch.empty((M, N), dtype=torch.float16, device=dev)
            for r in (16, 64, 128):
                A = (torch.randn(K, r, device=dev) * 0.01).half()
                B = (torch.randn(r, N, device=dev) * 0.01).half()
                wg = (torch.randn(K, device=dev) * 0.05).half()
                copies = [(p, A, B, wg) for p in pk]
                ws = torch.zeros(w4.w4ec_workspace_bytes(M, N, K, r, K), dtype=torch.uint8, device=dev)
                steps = 20 if M * N * K > 1e11 else 50
                res = {}
                for path in ("fused", "unfused", "semi"):
                    if path == "fused":
                        def step(i, copies=copies, ws=ws):
                            p, A_, B_, wg_ = copies[i % R]
                            w4.w4ec_linear_prefill(X, p, A_, B_, wg_, 0.0, N=N, group_size=K, workspace=ws, Y=Y)
                    else:
                        step = split_prefill_step(torch, w4, path, X, Y, copies, R, 0.0, M, N, K, r, K)
                    res[path] = round(graph_time_us(torch, step, steps, 5), 2)
                best = min(res, key=res.get)
                print(json.dumps({"M": M, "N": N, "K": K, "r": r, "us": res, "best": best,
                                  "fused_over_best": round(res["fused"] / res[best], 3)}), flush=True)
            del X, Y
        del pk, packed


def xfp_main(args, torch, w4, synth, dev, layer, M):
    """Codebook decode: Y = X Wh^T, Wh = per-channel 16-entry codebook lookups
    plus a sparse fp16 outlier residual.  The layer's weights with 0.5 % of
    them planted as x25 outliers, converted offline (untimed)."""
    d = synth.make_layer(layer, M, seed=args.seed, r=0)
    N, K, act = d["N"], d["K"], d["act"]
    tdt = torch.float16 if act == "fp16" else torch.bfloat16
    L = args.xfp_lib
    W = synth.plant_outliers(d["W"], seed=args.seed)
    if L:
        # shared-library mode: channels of different spreads (so that the
        # groups name many of the L entries)
        W = W * np.exp(np.random.default_rng(args.seed + 1).normal(0.0, 0.5, (N, 1))).astype(np.float32)
        x = synth.make_xfp_lib(W, L=L)
    else:
        x = synth.make_xfp(W)
    idx = x["idx"]
    qc = torch.from_numpy((idx[:, 0::2] | (idx[:, 1::2] << 4)).astype(np.uint8)).to(dev)
    packed0 = w4.w4ec_pack_xfp(qc, N, K)
    del qc
    nnz = int(x["row_ptr"][-1])
    if L:
        cb0 = torch.from_numpy(x["lib"].view(np.int16)).view(torch.float16).to(dev)
        id0 = torch.from_numpy(x["libid"]).to(dev)
        table_bytes = L * 32 + N * (K // 128)
    else:
        cb0 = torch.from_numpy(x["cb"].view(np.int16)).view(torch.float16).to(dev)
        id0 = None
        table_bytes = N * 32
    rp0 = torch.from_numpy(x["row_ptr"]).to(dev)
    ci0 = torch.from_numpy(x["col_idx"]).to(dev)
    val0 = torch.from_numpy(x["val"].view(np.int16)).view(torch.float16).to(dev)
    # algorithmic bytes: indices, codebooks (per channel; or the library and
    # the groups' entry ids), the residual (row pointers, columns, values), X and Y
    nbytes = N * K // 2 + table_bytes + (N + 1) * 4 + nnz * 6 + M * K * 2 + M * N * 2
    weight_bytes = packed0.numel() + table_bytes + (N + 1) * 4 + nnz * 6
    R = max(1, -(-2 * MALL_BYTES // weight_bytes))

    def clone(t):
        return None if t is None else t.clone()

    copies = [(packed0, cb0, id0, rp0, ci0, val0)] + [
        (packed0.clone(), cb0.clone(), clone(id0), rp0.clone(), ci0.clone(), val0.clone()) for _ in range(R - 1)]
    X = torch.from_numpy(np.ascontiguousarray(d["X"]).view(np.int16)).view(tdt).to(dev)
    Y = torch.empty((M, N), dtype=tdt, device=dev)

    def step(i):
        p, cb, lid, rp, ci, val = copies[i % R]
        if L:
            w4.w4ec_linear_decode_xfp_lib(X, p, cb, lid, rp, ci, val, N=N, Y=Y)
        else:
            w4.w4ec_linear_decode_xfp(X, p, cb, rp, ci, val, N=N, Y=Y)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    graph = None
    if not args.no_graph:
        stream = torch.cuda.Stream()
        stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(stream):
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=stream):
                for i in range(args.steps):
                    step(i)
        torch.cuda.current_stream().wait_stream(stream)
        graph.replay()
        torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    torch.cuda._sleep(int(100e6) if graph is None else int(20e6))
    start.record()
    if graph is not None:
        graph.replay()
    else:
        for i in range(args.steps):
            step(i)
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = start.elapsed_time(end) / args.steps
    kdur = ms_per_step * 1e-3
    achieved = nbytes / kdur / 1e9
    roof = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic_from_profiles(f"decode_kernel/{args.workload}/xfp" + (f"_lib{L}" if L else "")),
            "kernel": "decode_kernel (codebook" + (", shared library)" if L else ")"), "kernel_us": round(kdur * 1e6, 3)}
    flops = 2 * M * N * K + 2 * M * nnz
    out = {
        "metric": "W4+EC linear: decode HBM GB/s & prefill TFLOP/s, % of MI355X roofline",
        "value": round(nbytes / kdur / 1e9, 3), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 6), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": act, "data": "synthetic",
        "config": {"workload": args.workload, "M": M, "N": N, "K": K, "act": act, "phase": "decode",
                   "method": "xfp", **({"library_entries": L} if L else {}), "residual_entries": nnz,
                   "weight_copies": R,
                   "launch": "hipgraph" if graph is not None else "eager",
                   "bytes_per_step": nbytes, "flops_per_step": flops},
        "roofline": roof,
        "cpu_baseline": None,
        "wall_s": round(wall, 4),
    }
    print(json.dumps(out), flush=True)


def stream_read_time_us(torch, w4, nbytes, steps, warmup, dev):
    """Microseconds per launch of the library's streaming-read reference
    kernel over nbytes, the launches cycling through copies that together
    exceed twice the 256 MB Infinity Cache (graph replay, events)."""
    nb = -(-nbytes // 256) * 256
    R = max(2, -(-2 * MALL_BYTES // nb))
    buf = torch.ones(R * nb, dtype=torch.uint8, device=dev)
    sink = torch.empty(512, dtype=torch.int32, device=dev)

    def step(i):
        w4.w4ec_stream_read(buf[(i % R) * nb:(i % R) * nb + nbytes // 16 * 16], sink)

    # the attainable time: the best of three timed replays (one that a
    # stall of the machine interrupts says nothing about the read)
    us = graph_time_us(torch, step, steps, warmup, reps=3)
    del buf
    return us, R


def stream_read_main(args, torch, w4, synth, dev):
    """Only the streaming-read reference, over the algorithmic bytes of the
    workload's call: the HBM read time attainable for that byte count."""
    layer, M, phase = WORKLOADS[args.workload]
    c = synth.LAYERS[layer]
    r = c.r if args.rank is None else args.rank
    nbytes = layer_bytes(M, c.N, c.K, r, c.group_size, has_gate=r > 0) // 16 * 16
    us, R = stream_read_time_us(torch, w4, nbytes, args.steps, args.warmup, dev)
    achieved = nbytes / (us * 1e-6) / 1e9
    print(json.dumps({"metric": "streaming-read reference (stream_read_kernel)", "value": round(achieved, 2),
                      "unit": "GB/s", "us_per_launch": round(us, 3), "bytes": nbytes, "copies": R,
                      "frac_of_hbm_peak": round(achieved / HBM_PEAK_GBS, 4), "steps": args.steps,
                      "config": {"workload": args.workload, "bytes_of": "one call's algorithmic bytes"}}),
          flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default=None, choices=sorted(WORKLOADS),
                    help=f"one workload only (default: {DEFAULT_WORKLOAD}, with {PREFILL_WORKLOAD} "
                         "timed in the same run as the line's prefill half)")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches instead of a HIP graph")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work on the host")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB a few times "
                         "(the reference point for the HBM byte counters)")
    ap.add_argument("--rank", type=int, default=None,
                    help="EC rank override (0 = the plain W4 layer, for the EC overhead ratio)")
    ap.add_argument("--gate", choices=["scalar", "vector"], default="scalar",
                    help="scalar: one gate per token, sigmoid(x.w_g + b_g); vector: one gate per "
                         "rank component from a bottleneck MLP on X A")
    ap.add_argument("--gate-width", type=int, default=16, help="bottleneck width h of the vector gate")
    ap.add_argument("--path", choices=["fused", "unfused", "semi"], default="fused",
                    help="prefill only -- fused: the EC inside the GEMM's epilogue (default); unfused: gate "
                         "step, plain W4 GEMM, then a T_g B kernel, on one stream; semi: the gate step on a "
                         "second stream beside the GEMM, then the T_g B kernel")
    ap.add_argument("--method", choices=["spear", "serq", "xfp"], default="spear",
                    help="spear: the input-adaptive EC (default); serq: the single-factor correction over "
                         "the salient input channels (the config's outlier channels), X[:, S] R; xfp "
                         "(decode workloads): per-channel 16-entry codebooks plus a sparse fp16 outlier "
                         "residual, no EC")
    ap.add_argument("--stream-read", action="store_true",
                    help="only time the library's streaming-read reference kernel over the workload's "
                         "algorithmic bytes (the attainable HBM read time for that byte count)")
    ap.add_argument("--xfp-lib", type=int, default=0, metavar="L",
                    help="with --method xfp: the shared-library mode with L codebooks (1..32) instead of "
                         "per-channel codebooks")
    ap.add_argument("--lut", action="store_true",
                    help="prefill latency table: time the three paths over a grid of (M, r, N, K) and print "
                         "one JSON line per point (no roofline / CPU legs)")
    args = ap.parse_args()
    args.default_workload = args.workload is None
    if args.workload is None:
        args.workload = DEFAULT_WORKLOAD

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: measures one GPU only (the layer runs on one MI355X); "
              "--gpus must be 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import w4_gemm_error_amd as w4
    from w4_gemm_error_amd import synth

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        src = torch.ones(args.copy_calibration << 20, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": src.numel(), "launches": 5}), flush=True)
        return
    w4.lib()   # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    if args.lut:
        latency_table(torch, w4, synth, dev)
        return
    if args.stream_read:
        stream_read_main(args, torch, w4, synth, dev)
        return
    if args.path != "fused" and (WORKLOADS[args.workload][2] != "prefill" or args.gate != "scalar"):
        print("bench.py: --path unfused/semi applies to the prefill workloads with the scalar gate",
              file=sys.stderr)
        sys.exit(2)
    layer, M, phase = WORKLOADS[args.workload]
    if args.method == "xfp":
        if phase != "decode" or args.gate != "scalar" or args.path != "fused":
            print("bench.py: --method xfp applies to the decode workloads (no --gate / --path)", file=sys.stderr)
            sys.exit(2)
        xfp_main(args, torch, w4, synth, dev, layer, M)
        return
    out = measure_layer(args, args.workload, torch, w4, synth, dev)
    if args.default_workload and args.method == "spear" and args.gate == "scalar" and args.rank is None:
        # the metric has two halves: decode HBM GB/s (the line's value) and
        # prefill TFLOP/s, timed in the same run on the 2048-token prefill
        pf = measure_layer(args, PREFILL_WORKLOAD, torch, w4, synth, dev)
        out["prefill"] = {k: pf[k] for k in ("value", "unit", "ms_per_step", "dtype", "config",
                                             "roofline", "cpu_baseline")}
    print(json.dumps(out), flush=True)


def measure_layer(args, workload, torch, w4, synth, dev):
    """Time one workload of the W4 + EC layer; returns the JSON record."""
    layer, M, phase = WORKLOADS[workload]
    d = synth.make_layer(layer, M, seed=args.seed, r=args.rank)
    N, K, r, G, act = d["N"], d["K"], d["r"], d["group_size"], d["act"]
    tdt = torch.float16 if act == "fp16" else torch.bfloat16

    def dev_act(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(tdt).to(dev)

    # weights: quantize + pack once (offline, untimed), then replicate
    Wt = torch.from_numpy(d["W"]).to(dev)
    q, s, z = w4.w4ec_quantize_rtn(Wt, G)
    packed0 = w4.w4ec_pack(q, s, z, N, K, G)
    del Wt, q, s, z
    vector = args.gate == "vector" and r > 0
    h = args.gate_width if vector else 0
    serq = args.method == "serq"
    if serq and (vector or args.path != "fused"):
        print("bench.py: --method serq takes no --gate vector or --path", file=sys.stderr)
        sys.exit(2)
    if serq:
        S_host = np.asarray(d["outlier_channels"], dtype=np.int32)
        r = len(S_host)
        R_bits = synth.to_act_bits(np.random.default_rng(args.seed).normal(0.0, 0.01, (r, N)), act)
        A0, B0 = torch.from_numpy(S_host).to(dev), dev_act(R_bits)
        wg0 = None
        ec_elems = B0.numel() + r * 2          # R, and S as int32 (two halves' worth)
    elif r > 0 and vector:
        vg = synth.make_vgate(r, h, act, seed=args.seed, t_std=0.02 * K ** 0.5)
        A0, B0 = dev_act(d["A"]), dev_act(d["B"])
        wg0 = tuple(dev_act(vg[k]) for k in ("G1", "c1", "G2", "c2"))
        ec_elems = A0.numel() + B0.numel() + sum(t.numel() for t in wg0)
    elif r > 0:
        A0, B0, wg0 = dev_act(d["A"]), dev_act(d["B"]), dev_act(d["w_g"])
        ec_elems = A0.numel() + B0.numel() + wg0.numel()
    else:
        A0 = B0 = wg0 = None
        ec_elems = 0
    nbytes = layer_bytes(M, N, K, r, G, has_gate=r > 0, h=h)
    if serq:
        # codes + s/z + X + Y + R [s, N] + S (int32): no A and no gate
        nbytes = N * K // 2 + N * (K // G) * 4 + M * K * 2 + M * N * 2 + r * N * 2 + r * 4
    weight_bytes = packed0.numel() + ec_elems * 2
    R = max(1, -(-2 * MALL_BYTES // weight_bytes))

    def clone(t):
        if isinstance(t, tuple):
            return tuple(x.clone() for x in t)
        return None if t is None else t.clone()

    copies = [(packed0, A0, B0, wg0)] + [(packed0.clone(), clone(A0), clone(B0), clone(wg0))
                                         for _ in range(R - 1)]
    X = dev_act(d["X"])
    Y = torch.empty((M, N), dtype=tdt, device=dev)
    ws = torch.zeros(max(w4.w4ec_workspace_bytes(M, N, K, r, G), 256), dtype=torch.uint8, device=dev)
    b_g = d["b_g"]
    if serq:
        fns = w4.w4ec_linear_decode_serq if phase == "decode" else w4.w4ec_linear_prefill_serq

        def step(i):
            p, Sd, Rd, _ = copies[i % R]
            fns(X, p, Sd, Rd, N=N, group_size=G, workspace=ws, Y=Y)
    elif vector:
        fnv = w4.w4ec_linear_decode_vgate if phase == "decode" else w4.w4ec_linear_prefill_vgate

        def step(i):
            p, A, B, gp = copies[i % R]
            fnv(X, p, A, B, *gp, N=N, group_size=G, workspace=ws, Y=Y)
    elif args.path != "fused" and r > 0:
        step = split_prefill_step(torch, w4, args.path, X, Y, copies, R, b_g, M, N, K, r, G)
    else:
        fn = w4.w4ec_linear_decode if phase == "decode" else w4.w4ec_linear_prefill

        def step(i):
            p, A, B, wg = copies[i % R]
            fn(X, p, A, B, wg, b_g, N=N, group_size=G, workspace=ws, Y=Y)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # ---- timed region: K steps, bracketed by synchronization
    use_graph = not args.no_graph
    graph = None
    if use_graph:
        stream = torch.cuda.Stream()
        stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(stream):
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=stream):
                for i in range(args.steps):
                    step(i)
        torch.cuda.current_stream().wait_stream(stream)
        graph.replay()           # one untimed replay
        torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    # hold the stream while the host submits the work, so that the timed
    # region starts with the first kernel, not with the host's submission
    torch.cuda._sleep(int(100e6) if graph is None else int(20e6))
    start.record()
    if graph is not None:
        graph.replay()
    else:
        for i in range(args.steps):
            step(i)
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    elapsed_ms = start.elapsed_time(end)
    ms_per_step = elapsed_ms / args.steps

    # ---- dominant kernel.  A decode call is one kernel launch, so its
    # average launch duration is the timed region's event time over K (the
    # steps run back to back inside the graph).  A prefill call is up to three
    # launches (gate / X A partial sums, their reduction, then the GEMM); its
    # figure is per call.
    kdur = elapsed_ms * 1e-3 / args.steps
    reduce_name = "ec_reduce_vgate_kernel" if vector else "ec_reduce_kernel"
    kernel_name = "decode_kernel" if phase == "decode" else f"prepass_kernel + {reduce_name} + prefill_gemm_kernel (per call)"
    if phase == "prefill" and M <= 64 and r > 0 and not vector and not serq and args.path == "fused" \
            and -(-N // 256) <= 256:
        # one row of 64-token tiles: the GEMM's workgroups make T_g themselves
        kernel_name = "prefill_gemm_kernel (EC inside; per call)"
    if args.path != "fused" and r > 0:
        kernel_name = (f"prepass_kernel + ec_reduce_kernel, prefill_gemm_kernel (r = 0), ec_apply_kernel "
                       f"({args.path}, per call)")
    if serq and phase == "prefill":
        kernel_name = "serq_gather_kernel + prefill_gemm_kernel (per call)"

    flops = layer_flops(M, N, K, r, h)
    if serq:
        flops = 2 * M * N * K + 2 * M * r * N + 2 * M * N      # main product, X[:, S] R, add
    # the line's value: decode in algorithmic HBM GB/s, prefill in TFLOP/s
    # (the metric's two halves); the roofline takes whichever bound binds
    if phase == "decode":
        value = nbytes / (ms_per_step * 1e-3) / 1e9
        unit = "GB/s"
        kernel_key = f"decode_kernel/{workload}" + ("/vector_gate" if vector else "") + \
            ("/serq" if serq else "")
    else:
        value = flops / (ms_per_step * 1e-3) / 1e12
        unit = "TFLOP/s"
        kernel_key = f"prefill_call/{workload}" + ("/vector_gate" if vector else "") + \
            ("" if args.path == "fused" else f"/{args.path}") + ("/serq" if serq else "")
    roof = roofline(nbytes, flops, kdur, act)
    roof["traffic"] = traffic_from_profiles(kernel_key)
    roof["kernel"] = kernel_name
    roof["kernel_us"] = round(kdur * 1e6, 3)
    if phase == "decode" and roof["bound"] == "hbm":
        # the attainable read time for the same bytes, timed in this run:
        # the library's plain streaming-read kernel
        sus, _ = stream_read_time_us(torch, w4, nbytes // 16 * 16, min(args.steps, 200), 10, dev)
        roof["stream_read"] = {"kernel": "stream_read_kernel", "us": round(sus, 3),
                               "achieved": round(nbytes / (sus * 1e-6) / 1e9, 2),
                               "frac": round(nbytes / (sus * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                               "call_over_read": round(kdur * 1e6 / sus, 3)}

    cpu = None
    if not args.no_cpu and not vector and not serq:
        cpu = cpu_baseline(d, phase, args.cpu_budget)

    return {
        "metric": "W4+EC linear: decode HBM GB/s & prefill TFLOP/s, % of MI355X roofline",
        "value": round(value, 3),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": act,
        "data": "synthetic",
        "config": {"workload": workload, "M": M, "N": N, "K": K, "r": r, "group_size": G,
                   "act": act, "phase": phase, "method": args.method,
                   **({"salient_channels": r} if serq else {"gate": "vector" if vector else "scalar"}),
                   **({"path": args.path} if phase == "prefill" else {}),
                   **({"gate_width": h} if vector else {}), "weight_copies": R,
                   "launch": "hipgraph" if graph is not None else "eager",
                   "bytes_per_step": nbytes, "flops_per_step": flops},
        "roofline": roof,
        "cpu_baseline": cpu,
        "wall_s": round(wall, 4),
    }


if __name__ == "__main__":
    main()
