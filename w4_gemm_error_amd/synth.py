"""Seeded synthetic inputs for the W4 + EC linear layer.

This module only draws random numbers and casts them to the activation
format; it holds none of the layer's arithmetic (no quantizer, no product),
so both the GPU library's tests and the CPU oracle can take their inputs from
it.  The pages measure on trained checkpoints and perplexity / accuracy
datasets that are not available here; seeded tensors shaped like the linear
layers of 8B- and 70B-class decoder models stand in for them.

Draw order per call, from ``numpy.random.default_rng(seed)``:
W, X, outlier channel set, A, B, w_g (or the gate direction w0).

Outliers: ``round(frac * K)`` input channels (columns of X), drawn without
replacement, shared by every token, multiplied after drawing; then X is cast
to the activation format.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class LayerConfig:
    name: str
    Ms: tuple
    K: int
    N: int
    r: int
    group_size: int          # == K means one scale/zero per output channel
    act: str                 # "fp16" or "bf16"
    outlier_frac: float
    outlier_scale: float
    gate: str                # "plain": w_g ~ N(0, 0.05), b_g = 0; "calibrated": g spans (0.05, 0.95)
    w_std: float = 0.02
    ab_std: float = 0.01
    wg_std: float = 0.05


# the synthetic layers, by name; SEEDS gives each a small integer for the
# generators of its extra inputs
LAYERS = {c.name: c for c in (
    LayerConfig("tiny", (16,), 512, 512, 8, 512, "fp16", 0.01, 20.0, "plain"),
    LayerConfig("decode_up_proj_8b", (1, 4, 16), 4096, 14336, 64, 4096, "fp16", 0.01, 20.0, "plain"),
    LayerConfig("prefill_out_proj_8b", (2048,), 4096, 4096, 64, 4096, "fp16", 0.01, 20.0, "calibrated"),
    LayerConfig("batched_down_proj_8b_g128", (256,), 14336, 4096, 128, 128, "fp16", 0.01, 20.0, "plain"),
    LayerConfig("mlp_70b_bf16", (64, 4096), 8192, 28672, 128, 8192, "bf16", 0.005, 30.0, "plain"),
)}
SEEDS = {"tiny": 1, "decode_up_proj_8b": 2, "prefill_out_proj_8b": 3, "batched_down_proj_8b_g128": 4,
         "mlp_70b_bf16": 5}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def to_act_bits(x: np.ndarray, act: str) -> np.ndarray:
    """Round float values to the activation format; return its bit patterns."""
    if act == "fp16":
        return np.ascontiguousarray(np.asarray(x).astype(np.float16)).view(np.uint16)
    if act == "bf16":
        return f32_to_bf16_bits(np.asarray(x, dtype=np.float32))
    raise ValueError(act)


def act_bits_to_f64(bits: np.ndarray, act: str) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    if act == "fp16":
        return bits.view(np.float16).astype(np.float64)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def make_layer(cfg, M: int, seed: int = 0, *, K=None, N=None, r=None,
               group_size=None) -> dict:
    """Inputs for one layer call.  ``cfg`` is a config id or a LayerConfig;
    K, N, r, group_size override its shape (same distributions).

    Returns a dict: X (act bits [M, K]), W (float32 [N, K]), A (act bits
    [K, r]), B (act bits [r, N]), w_g (act bits [K]), b_g (float), the shape,
    ``act`` and the outlier channel indices.
    """
    c = LAYERS[cfg] if isinstance(cfg, str) else cfg
    K = c.K if K is None else int(K)
    N = c.N if N is None else int(N)
    r = c.r if r is None else int(r)
    G = (c.group_size if c.group_size != c.K else K) if group_size is None else int(group_size)
    rng = np.random.default_rng(seed)

    W = rng.standard_normal((N, K), dtype=np.float32) * np.float32(c.w_std)
    X = rng.standard_normal((M, K))
    n_out = int(round(c.outlier_frac * K))
    out_ch = np.sort(rng.choice(K, size=n_out, replace=False)) if n_out > 0 else np.zeros(0, np.int64)
    X[:, out_ch] *= c.outlier_scale
    Xb = to_act_bits(X, c.act)
    A = to_act_bits(rng.normal(0.0, c.ab_std, (K, r)), c.act)
    B = to_act_bits(rng.normal(0.0, c.ab_std, (r, N)), c.act)
    if c.gate == "plain":
        w_g = to_act_bits(rng.normal(0.0, c.wg_std, (K,)), c.act)
        b_g = 0.0
    elif c.gate == "calibrated":
        # A gate direction w0 ~ N(0, 1), rescaled so that the logits of the
        # 1st and 99th percentile tokens land at logit(0.05) and logit(0.95):
        # about 98 % of the tokens then get a gate inside (0.05, 0.95).
        w0 = rng.standard_normal(K)
        l0 = act_bits_to_f64(Xb, c.act) @ w0
        p1, p99 = np.percentile(l0, [1.0, 99.0]) if M > 1 else (l0[0] - 1.0, l0[0] + 1.0)
        span = max(p99 - p1, 1e-12)
        cscale = 2.0 * np.log(0.95 / 0.05) / span
        w_g = to_act_bits(cscale * w0, c.act)
        b_g = float(-cscale * (p99 + p1) / 2.0)
    else:
        raise ValueError(c.gate)
    return dict(X=Xb, W=W, A=A, B=B, w_g=w_g, b_g=b_g, M=M, K=K, N=N, r=r,
                group_size=G, act=c.act, outlier_channels=out_ch, name=c.name)


def make_vgate(r: int, h: int, act: str = "fp16", seed: int = 0, t_std: float = 1.0) -> dict:
    """Seeded parameters of a vector gate (a bottleneck of width h on the
    rank-r projection T): G1 [r, h], c1 [h], G2 [h, r], c2 [r] as act bits.
    Scaled so that, for rows of T with standard deviation about t_std, the
    gates spread over (0, 1) rather than saturating."""
    rng = np.random.default_rng(1_000_003 + seed)
    G1 = rng.normal(0.0, 1.0 / (t_std * np.sqrt(r)), (r, h))
    c1 = rng.normal(0.0, 0.5, (h,))
    G2 = rng.normal(0.0, 2.0 / np.sqrt(h), (h, r))
    c2 = rng.normal(0.0, 1.0, (r,))
    return {"G1": to_act_bits(G1, act), "c1": to_act_bits(c1, act),
            "G2": to_act_bits(G2, act), "c2": to_act_bits(c2, act), "h": h}


def plant_outliers(W: np.ndarray, frac: float = 0.005, scale: float = 25.0, seed: int = 0) -> np.ndarray:
    """A copy of W [N, K] with frac of its entries (chosen uniformly, seeded)
    multiplied by scale: the heavy-tailed weights that the codebook format
    keeps apart."""
    W = np.array(W, dtype=np.float32, copy=True)
    n_out = int(frac * W.size)
    if n_out:
        pos = np.random.default_rng(900 + seed).choice(W.size, size=n_out, replace=False)
        W.reshape(-1)[pos] *= np.float32(scale)
    return W


def make_xfp(W: np.ndarray, k_sigma: float = 4.0, max_frac: float = 0.02) -> dict:
    """Synthetic weights in the codebook-plus-outliers format, built from a
    float32 matrix W [N, K]: per output channel, the weights farther than
    k_sigma standard deviations from the channel mean (at most max_frac of
    the channel, the farthest first) are outliers; the rest keep their value,
    the outlier positions take the channel mean.  The channel's 16 codebook
    entries are quantiles of those values (fp16, ascending), each weight
    takes the nearest entry's index, and the outliers carry the fp16 residual
    w - cb[idx] at their positions (compressed sparse rows).
    Returns idx (uint8 [N, K], 0..15), cb (fp16 bits [N, 16]), row_ptr,
    col_idx (int32) and val (fp16 bits)."""
    W = np.asarray(W, dtype=np.float64)
    N, K = W.shape
    mu = W.mean(axis=1, keepdims=True)
    sd = W.std(axis=1, keepdims=True)
    dev = np.abs(W - mu)
    cap = max(0, int(max_frac * K))
    out = dev > k_sigma * sd
    if cap < K:
        # keep only the cap farthest per row
        kth = -np.partition(-dev, cap, axis=1)[:, cap:cap + 1] if cap > 0 else np.full((N, 1), np.inf)
        out &= dev > kth
    block = np.where(out, mu, W)
    qs = (np.arange(16) + 0.5) / 16.0
    cb = np.ascontiguousarray(np.quantile(block, qs, axis=1).T.astype(np.float16))   # [N, 16], ascending
    cb64 = cb.astype(np.float64)
    mid = (cb64[:, 1:] + cb64[:, :-1]) / 2.0
    idx = np.empty((N, K), np.uint8)
    for n0 in range(0, N, 2048):
        sl = slice(n0, min(N, n0 + 2048))
        idx[sl] = (block[sl, :, None] > mid[sl, None, :]).sum(axis=2).astype(np.uint8)
    rows, cols = np.nonzero(out)
    resid = W[rows, cols] - cb64[rows, idx[rows, cols]]
    row_ptr = np.zeros(N + 1, np.int32)
    np.add.at(row_ptr, rows + 1, 1)
    row_ptr = np.cumsum(row_ptr).astype(np.int32)
    return {"idx": idx, "cb": cb.view(np.uint16), "row_ptr": row_ptr, "col_idx": cols.astype(np.int32),
            "val": resid.astype(np.float16).view(np.uint16)}


def make_xfp_lib(W: np.ndarray, L: int = 32, k_sigma: float = 4.0, max_frac: float = 0.02) -> dict:
    """Synthetic weights in the shared-library codebook format, built from a
    float32 matrix W [N, K] (K a multiple of 128): the outliers are separated
    as in make_xfp; the library holds L codebooks, the 16 quantiles of a
    standard normal scaled by L scales spaced geometrically over the range
    of the groups' standard deviations (fp16); each group of 128 weights of
    a channel takes the entry whose scale is nearest its own (in log), each
    weight the nearest value of that entry, and the outliers carry the fp16
    residual w - entry[idx] at their positions.
    Returns idx (uint8 [N, K]), lib (fp16 bits [L, 16]), libid (uint8
    [N, K/128]), row_ptr, col_idx (int32) and val (fp16 bits)."""
    from math import erf, sqrt
    W = np.asarray(W, dtype=np.float64)
    N, K = W.shape
    assert K % 128 == 0 and 1 <= L <= 256
    mu = W.mean(axis=1, keepdims=True)
    sd = W.std(axis=1, keepdims=True)
    dev = np.abs(W - mu)
    cap = max(0, int(max_frac * K))
    out = dev > k_sigma * sd
    if cap < K:
        kth = -np.partition(-dev, cap, axis=1)[:, cap:cap + 1] if cap > 0 else np.full((N, 1), np.inf)
        out &= dev > kth
    block = np.where(out, mu, W)
    ng = K // 128
    gsd = np.maximum(block.reshape(N, ng, 128).std(axis=2), 1e-8)          # [N, ng]
    lo, hi = np.log(gsd.min()), np.log(gsd.max())
    scales = np.exp(np.linspace(lo, hi, L)) if L > 1 else np.exp(np.array([(lo + hi) / 2]))
    # the 16 quantiles (t + 1/2) / 16 of a standard normal, by bisection on erf
    z = np.empty(16)
    for t in range(16):
        p, a, b = (t + 0.5) / 16.0, -8.0, 8.0
        for _ in range(80):
            m = (a + b) / 2
            a, b = (m, b) if 0.5 * (1 + erf(m / sqrt(2))) < p else (a, m)
        z[t] = (a + b) / 2
    lib = (scales[:, None] * z[None, :]).astype(np.float16)                  # [L, 16], ascending
    libid = np.abs(np.log(gsd)[:, :, None] - np.log(scales)[None, None, :]).argmin(axis=2).astype(np.uint8)
    ent = lib.astype(np.float64)[libid]                                      # [N, ng, 16]
    mid = (ent[:, :, 1:] + ent[:, :, :-1]) / 2.0
    idx = np.empty((N, K), np.uint8)
    for n0 in range(0, N, 1024):
        sl = slice(n0, min(N, n0 + 1024))
        bl = block[sl].reshape(-1, ng, 128)
        idx[sl] = (bl[:, :, :, None] > mid[sl][:, :, None, :]).sum(axis=3).astype(np.uint8).reshape(-1, K)
    rows, cols = np.nonzero(out)
    resid = W[rows, cols] - ent[rows, cols // 128, idx[rows, cols]]
    row_ptr = np.zeros(N + 1, np.int32)
    np.add.at(row_ptr, rows + 1, 1)
    row_ptr = np.cumsum(row_ptr).astype(np.int32)
    return {"idx": idx, "lib": np.ascontiguousarray(lib).view(np.uint16), "libid": libid,
            "row_ptr": row_ptr, "col_idx": cols.astype(np.int32), "val": resid.astype(np.float16).view(np.uint16)}
