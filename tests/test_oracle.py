"""Pins for the float64 CPU oracle (CPU only).

Each test ties the oracle to something other than itself: numpy's IEEE
conversions, exhaustive enumeration, exact rational arithmetic
(``fractions.Fraction``), ``numpy.matmul`` on weights that lie exactly on the
quantization grid, a hand-worked example (tests/golden/hand_example.json),
and the special cases and invariants of the layer definition in SPEAR
(gist.science technical summary, section 2.1A; per-channel RTN baseline from
section 3.1).
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
from scipy.special import expit

import oracle
from w4_gemm_error_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f16bits(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float16)).view(np.uint16)


def pack_canonical(q):
    """codes uint8 [N, K] -> canonical uint8 [N, K/2] (even k in the low nibble)."""
    q = np.asarray(q, dtype=np.uint8)
    return (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)


def on_grid_layer(rng, N, K, G):
    """Random codes (every group holds a 0 and a 15), integer zeros and fp16 scales;
    returns codes, scale/zero bits and the exact weights (q - z) * s."""
    q = rng.integers(0, 16, size=(N, K)).astype(np.uint8)
    ng = K // G
    for n in range(N):
        for gi in range(ng):
            pos = rng.choice(G, size=2, replace=False) + gi * G
            q[n, pos[0]] = 0
            q[n, pos[1]] = 15
    z = rng.integers(0, 16, size=(N, ng)).astype(np.float64)
    s = np.exp2(rng.uniform(-9, -4, size=(N, ng))).astype(np.float16).astype(np.float64)
    W = (q.astype(np.float64) - np.repeat(z, G, 1)) * np.repeat(s, G, 1)
    return q, f16bits(s), f16bits(z), W


# ---------------------------------------------------------------- formats

def test_half_to_double_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.half_to_double(b) for b in bits[::7]])
    r = ref[::7]
    same = (got == r) | (np.isnan(got) & np.isnan(r))
    assert same.all()


def test_double_to_half_matches_numpy_rounding():
    rng = np.random.default_rng(1)
    xs = list(rng.standard_normal(3000) * np.exp2(rng.uniform(-30, 17, 3000)))
    # exact halfway points between neighbouring halves, subnormals, overflow edge
    h = np.arange(0, 0x7bff, 97, dtype=np.uint16).view(np.float16).astype(np.float64)
    h1 = (np.arange(0, 0x7bff, 97, dtype=np.uint16) + 1).view(np.float16).astype(np.float64)
    xs += list((h + h1) / 2) + list(-(h + h1) / 2)
    xs += [0.0, -0.0, 2.0 ** -25, 3 * 2.0 ** -26, 65504.0, 65519.99, 65520.0, 1e6, -1e6]
    for x in xs:
        with np.errstate(over="ignore"):
            want = int(np.array(x, dtype=np.float64).astype(np.float16).view(np.uint16))
        assert oracle.double_to_half(x) == want, x


def test_bf16_widening():
    for b in [0x0000, 0x3F80, 0xC000, 0x4170, 0x0001, 0x7F7F]:
        want = np.array([b << 16], np.uint32).view(np.float32)[0]
        assert oracle.bf16_to_double(b) == float(want)


# ---------------------------------------------------------------- codes

def test_unpack_exhaustive_bytes():
    N, K = 1, 512
    qc = np.arange(256, dtype=np.uint8).reshape(1, 256)
    q = oracle.unpack_codes(qc, N, K)
    for b in range(256):
        assert q[0, 2 * b] == (b & 15) and q[0, 2 * b + 1] == (b >> 4)


# ---------------------------------------------------------------- RTN

@pytest.mark.parametrize("G", [64, 128, 256])
def test_rtn_grid_identity(G):
    rng = np.random.default_rng(2)
    N, K = 12, 256
    q, s, z, W = on_grid_layer(rng, N, K, G)
    W32 = W.astype(np.float32)
    assert np.array_equal(W32.astype(np.float64), W)  # the grid is exact in float32
    qc, s2, z2 = oracle.rtn_quantize(W32, G)
    assert np.array_equal(oracle.unpack_codes(qc, N, K), q)
    assert np.array_equal(s2, s) and np.array_equal(z2, z)


def test_rtn_brute_force_exact():
    rng = np.random.default_rng(3)
    N, K, G = 6, 64, 32
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    W[2, 5:9] = 0.0
    qc, s, z = oracle.rtn_quantize(W, G)
    q = oracle.unpack_codes(qc, N, K)
    sv = s.view(np.float16).astype(np.float64)
    zv = z.view(np.float16).astype(np.float64)
    for n in range(N):
        for gi in range(K // G):
            w = W[n, gi * G:(gi + 1) * G].astype(np.float64)
            lo, hi = min(w.min(), 0.0), max(w.max(), 0.0)
            assert sv[n, gi] == float(np.float16((hi - lo) / 15.0))
            assert zv[n, gi] == float(np.clip(np.rint(-lo / sv[n, gi]), 0, 15))
            S, Z = Fraction(sv[n, gi]), Fraction(zv[n, gi])
            for k in range(G):
                wk = Fraction(float(w[k]))
                errs = [abs(wk - (c - Z) * S) for c in range(16)]
                assert errs[q[n, gi * G + k]] == min(errs)


def test_rtn_degenerate_group():
    W = np.zeros((2, 64), np.float32)
    W[1, :32] = 0.01
    qc, s, z = oracle.rtn_quantize(W, 32)
    q = oracle.unpack_codes(qc, 2, 64)
    assert (q[0] == 0).all() and (s[0] == 0x3C00).all() and (z[0] == 0).all()
    assert (q[1, 32:] == 0).all() and s[1, 1] == 0x3C00
    # a one-sided group: range [0, 0.01] -> z = 0, max code 15
    assert z[1, 0] == 0 and q[1, :32].max() == 15


# ---------------------------------------------------------------- forward

def run(M, N, K, r, G, X, qc, s, z, A, B, wg, bg, act="fp16", rows=None):
    return oracle.forward(X, qc, s, z, A, B, wg, bg, N=N, K=K, r=r, group_size=G,
                          act=act, rows=rows)


def test_hand_worked_example():
    d = json.load(open(os.path.join(GOLDEN, "hand_example.json")))
    M, K, N, r, G = d["M"], d["K"], d["N"], d["r"], d["group_size"]
    qc = pack_canonical(np.array(d["codes"]))
    assert np.array_equal(qc, np.array(d["canonical_bytes"], np.uint8))
    out = run(M, N, K, r, G, f16bits(d["X"]), qc, f16bits(d["scale"]), f16bits(d["zero"]),
              f16bits(d["A"]), f16bits(d["B"]), f16bits(d["w_g"]), d["b_g"])
    e = d["expected"]
    for key in ("Y0", "T", "C", "g", "Y"):
        assert np.array_equal(out[key], np.array(e[key], np.float64)), key


@pytest.mark.parametrize("act", ["fp16", "bf16"])
def test_tiny_exact_rational(act):
    rng = np.random.default_rng(4)
    M, N, K, r, G = 3, 5, 8, 2, 4
    q, s, z, _ = on_grid_layer(rng, N, K, G)
    Xb = synth.to_act_bits(rng.standard_normal((M, K)) * 3, act)
    Ab = synth.to_act_bits(rng.standard_normal((K, r)) * 0.1, act)
    Bb = synth.to_act_bits(rng.standard_normal((r, N)) * 0.1, act)
    wgb = synth.to_act_bits(rng.standard_normal(K) * 0.2, act)
    bg = 0.3
    out = run(M, N, K, r, G, Xb, pack_canonical(q), s, z, Ab, Bb, wgb, bg, act=act)
    F = lambda a: [[Fraction(float(v)) for v in row] for row in np.atleast_2d(a)]
    X = F(synth.act_bits_to_f64(Xb, act))
    A = F(synth.act_bits_to_f64(Ab, act))
    B = F(synth.act_bits_to_f64(Bb, act))
    wg = [Fraction(float(v)) for v in synth.act_bits_to_f64(wgb, act)]
    sv = F(s.view(np.float16).astype(np.float64))
    zv = F(z.view(np.float16).astype(np.float64))
    for m in range(M):
        T = [sum(X[m][k] * A[k][j] for k in range(K)) for j in range(r)]
        lg = sum(X[m][k] * wg[k] for k in range(K)) + Fraction(bg)
        g = float(expit(float(lg)))
        assert out["g"][m] == pytest.approx(g, rel=1e-15, abs=0)
        for j in range(r):
            assert out["T"][m, j] == pytest.approx(float(T[j]), rel=1e-13, abs=1e-300)
        for n in range(N):
            y0 = sum(X[m][k] * (int(q[n, k]) - zv[n][k // G]) * sv[n][k // G] for k in range(K))
            c = sum(T[j] * B[j][n] for j in range(r))
            y = float(y0) + g * float(c)
            assert out["Y0"][m, n] == pytest.approx(float(y0), rel=1e-13, abs=1e-300)
            assert out["C"][m, n] == pytest.approx(float(c), rel=1e-13, abs=1e-300)
            assert out["Y"][m, n] == pytest.approx(y, rel=1e-12, abs=1e-12)


@pytest.mark.parametrize("G", [4, 8])
def test_fractional_zero_points_exact_rational(G):
    """Zero points need not be integers (quantizers other than RTN may learn
    them): with arbitrary fp16 zero points -- fractional, negative, above 15
    -- the plain product matches exact rational arithmetic, and moving every
    zero point of a group by d moves each output by exactly -d s times the
    group's activation sum (the dequantization is affine in z)."""
    rng = np.random.default_rng(17)
    M, N, K = 3, 5, 8
    q, s, _, _ = on_grid_layer(rng, N, K, G)
    z = np.array(rng.choice([-3.5, -0.125, 0.375, 7.25, 7.3125, 15.0, 17.75, 2.0], size=(N, K // G)),
                 np.float16).view(np.uint16)
    Xb = f16bits(rng.standard_normal((M, K)) * 2)
    out = run(M, N, K, 0, G, Xb, pack_canonical(q), s, z, None, None, None, 0.0)
    X = [[Fraction(float(v)) for v in row] for row in Xb.view(np.float16).astype(np.float64)]
    sv = s.view(np.float16).astype(np.float64)
    zv = z.view(np.float16).astype(np.float64)
    for m in range(M):
        for n in range(N):
            y0 = sum(X[m][k] * (int(q[n, k]) - Fraction(zv[n, k // G])) * Fraction(sv[n, k // G])
                     for k in range(K))
            assert out["Y0"][m, n] == pytest.approx(float(y0), rel=1e-13, abs=1e-300)
    d = 0.25
    z2 = (zv + d).astype(np.float16)
    assert np.array_equal(z2.astype(np.float64), zv + d)        # exact shift
    out2 = run(M, N, K, 0, G, Xb, pack_canonical(q), s, z2.view(np.uint16), None, None, None, 0.0)
    xs = Xb.view(np.float16).astype(np.float64).reshape(M, K // G, G).sum(axis=2)   # [M][groups]
    expect = out["Y0"] - d * xs @ sv.T
    np.testing.assert_allclose(out2["Y0"], expect, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("G", [128, 512])
def test_on_grid_weights_reproduce_matmul(G):
    rng = np.random.default_rng(5)
    M, N, K = 7, 48, 512
    q, s, z, W = on_grid_layer(rng, N, K, G)
    Xb = f16bits(rng.standard_normal((M, K)))
    out = run(M, N, K, 0, G, Xb, pack_canonical(q), s, z, None, None, None, 0.0)
    ref = np.matmul(Xb.view(np.float16).astype(np.float64), W.T)
    np.testing.assert_allclose(out["Y0"], ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
    assert np.array_equal(out["Y"], out["Y0"])


def cfg1_inputs(seed=0, M=16):
    d = synth.make_layer("tiny", M, seed)
    qc, s, z = oracle.rtn_quantize(d["W"], d["group_size"])
    return d, qc, s, z


def test_special_cases_reduce_to_plain_w4():
    d, qc, s, z = cfg1_inputs()
    M, N, K, r, G = d["M"], d["N"], d["K"], d["r"], d["group_size"]
    base = run(M, N, K, 0, G, d["X"], qc, s, z, None, None, None, 0.0)
    full = run(M, N, K, r, G, d["X"], qc, s, z, d["A"], d["B"], d["w_g"], d["b_g"])
    assert np.array_equal(full["Y0"], base["Y"])                     # r = 0 is the plain W4 layer
    off = run(M, N, K, r, G, d["X"], qc, s, z, d["A"], d["B"], d["w_g"], -math.inf)
    assert np.array_equal(off["Y"], base["Y"]) and (off["g"] == 0).all()   # gate closed
    zA = run(M, N, K, r, G, d["X"], qc, s, z, np.zeros_like(d["A"]), d["B"], d["w_g"], 0.0)
    zB = run(M, N, K, r, G, d["X"], qc, s, z, d["A"], np.zeros_like(d["B"]), d["w_g"], 0.0)
    assert np.array_equal(zA["Y"], base["Y"]) and np.array_equal(zB["Y"], base["Y"])


def test_open_gate_is_static_low_rank_compensation():
    rng = np.random.default_rng(6)
    M, N, K, r, G = 9, 40, 256, 8, 128
    q, s, z, W = on_grid_layer(rng, N, K, G)
    Xb = f16bits(rng.standard_normal((M, K)))
    Ab = f16bits(rng.standard_normal((K, r)) * 0.05)
    Bb = f16bits(rng.standard_normal((r, N)) * 0.05)
    out = run(M, N, K, r, G, Xb, pack_canonical(q), s, z, Ab, Bb, None, math.inf)
    assert (out["g"] == 1.0).all()
    X = Xb.view(np.float16).astype(np.float64)
    A = Ab.view(np.float16).astype(np.float64)
    B = Bb.view(np.float16).astype(np.float64)
    ref = np.matmul(X, W.T + np.matmul(A, B))
    np.testing.assert_allclose(out["Y"], ref, rtol=1e-11, atol=1e-11 * np.abs(ref).max())


def test_gate_and_low_rank_against_numpy():
    d, qc, s, z = cfg1_inputs()
    M, N, K, r, G = d["M"], d["N"], d["K"], d["r"], d["group_size"]
    out = run(M, N, K, r, G, d["X"], qc, s, z, d["A"], d["B"], d["w_g"], d["b_g"])
    X = synth.act_bits_to_f64(d["X"], "fp16")
    T = np.matmul(X, synth.act_bits_to_f64(d["A"], "fp16"))
    np.testing.assert_allclose(out["T"], T, rtol=1e-12, atol=1e-12 * np.abs(T).max())
    g = expit(np.matmul(X, synth.act_bits_to_f64(d["w_g"], "fp16")) + d["b_g"])
    np.testing.assert_allclose(out["g"], g, rtol=1e-12, atol=1e-15)
    C = np.matmul(out["T"], synth.act_bits_to_f64(d["B"], "fp16"))
    np.testing.assert_allclose(out["C"], C, rtol=1e-12, atol=1e-12 * np.abs(C).max())


def test_gate_invariants():
    d, qc, s, z = cfg1_inputs()
    M, N, K, r, G = d["M"], d["N"], d["K"], d["r"], d["group_size"]
    out = run(M, N, K, r, G, d["X"], qc, s, z, d["A"], d["B"], d["w_g"], d["b_g"])
    dY = out["Y"] - out["Y0"]
    C, g = out["C"], out["g"]
    big = np.abs(C) > 1e-9
    ratio = np.where(big, dY / np.where(big, C, 1.0), np.nan)
    for m in range(M):
        rm = ratio[m][big[m]]
        np.testing.assert_allclose(rm, g[m], rtol=1e-6, atol=1e-9)
        if 0.0 < g[m] < 1.0:
            assert (np.abs(dY[m][big[m]]) < np.abs(C[m][big[m]])).all()
            assert (np.sign(dY[m][big[m]]) == np.sign(C[m][big[m]])).all()


def test_equivariance_and_row_subsets():
    d, qc, s, z = cfg1_inputs()
    M, N, K, r, G = d["M"], d["N"], d["K"], d["r"], d["group_size"]
    args = (d["X"], qc, s, z, d["A"], d["B"], d["w_g"], d["b_g"])
    full = run(M, N, K, r, G, *args)
    rng = np.random.default_rng(7)
    pm = rng.permutation(M)
    tp = run(M, N, K, r, G, d["X"][pm], *args[1:])
    assert np.array_equal(tp["Y"], full["Y"][pm])
    pn = rng.permutation(N)
    cp = run(M, N, K, r, G, d["X"], qc[pn], s[pn], z[pn], d["A"], d["B"][:, pn], d["w_g"], d["b_g"])
    assert np.array_equal(cp["Y"], full["Y"][:, pn])
    B2 = f16bits(2.0 * synth.act_bits_to_f64(d["B"], "fp16"))
    b2 = run(M, N, K, r, G, d["X"], qc, s, z, d["A"], B2, d["w_g"], d["b_g"])
    assert np.array_equal(b2["C"], 2.0 * full["C"])
    rows = [5, 0, 15, 5]
    sub = run(M, N, K, r, G, *args, rows=rows)
    assert np.array_equal(sub["Y"], full["Y"][rows])


def test_synth_shapes_and_outliers():
    d = synth.make_layer("decode_up_proj_8b", 4, seed=0)
    assert d["X"].shape == (4, 4096) and d["W"].shape == (14336, 4096)
    assert len(d["outlier_channels"]) == 41
    d5 = synth.make_layer("mlp_70b_bf16", 2, seed=0, N=256)
    assert d5["act"] == "bf16" and len(d5["outlier_channels"]) == 41
    d3 = synth.make_layer("prefill_out_proj_8b", 256, seed=0, N=64)
    g = expit(synth.act_bits_to_f64(d3["X"], "fp16") @ synth.act_bits_to_f64(d3["w_g"], "fp16") + d3["b_g"])
    inside = np.mean((g > 0.05) & (g < 0.95))
    assert inside > 0.9


# ---------------------------------------------------------------- vector gate

def vg_run(M, N, K, r, G, h, X, qc, s, z, A, B, G1, c1, G2, c2, rows=None):
    return oracle.forward_vgate(X, qc, s, z, A, B, G1, c1, G2, c2, N=N, K=K, r=r, h=h,
                                group_size=G, rows=rows)


def vg_layer(rng, M=9, N=40, K=256, r=8, G=128):
    q, s, z, W = on_grid_layer(rng, N, K, G)
    Xb = f16bits(rng.standard_normal((M, K)))
    Ab = f16bits(rng.standard_normal((K, r)) * 0.05)
    Bb = f16bits(rng.standard_normal((r, N)) * 0.05)
    f = lambda b: b.view(np.float16).astype(np.float64)
    return dict(M=M, N=N, K=K, r=r, G=G, qc=pack_canonical(q), s=s, z=z, W=W, Xb=Xb, Ab=Ab, Bb=Bb,
                X=f(Xb), A=f(Ab), B=f(Bb))


def test_vgate_closed_gate_is_plain_w4():
    L = vg_layer(np.random.default_rng(21))
    h = 4
    p = synth.make_vgate(L["r"], h, seed=1)
    c2 = f16bits(np.full(L["r"], -np.inf))
    out = vg_run(L["M"], L["N"], L["K"], L["r"], L["G"], h, L["Xb"], L["qc"], L["s"], L["z"],
                 L["Ab"], L["Bb"], p["G1"], p["c1"], p["G2"], c2)
    base = run(L["M"], L["N"], L["K"], 0, L["G"], L["Xb"], L["qc"], L["s"], L["z"], None, None, None, 0.0)
    assert (out["gamma"] == 0.0).all() and np.array_equal(out["Y"], base["Y"])


def test_vgate_open_gate_is_static_low_rank_compensation():
    L = vg_layer(np.random.default_rng(22))
    h = 3
    p = synth.make_vgate(L["r"], h, seed=2)
    G2 = f16bits(np.zeros((h, L["r"])))
    c2 = f16bits(np.full(L["r"], np.inf))
    out = vg_run(L["M"], L["N"], L["K"], L["r"], L["G"], h, L["Xb"], L["qc"], L["s"], L["z"],
                 L["Ab"], L["Bb"], p["G1"], p["c1"], G2, c2)
    assert (out["gamma"] == 1.0).all()
    ref = np.matmul(L["X"], L["W"].T + np.matmul(L["A"], L["B"]))
    np.testing.assert_allclose(out["Y"], ref, rtol=1e-11, atol=1e-11 * np.abs(ref).max())


def test_vgate_constant_gate_against_numpy():
    """G1 = 0: the bottleneck sees only its bias, so every token gets the same
    gate vector sigmoid(relu(c1) G2 + c2), and the layer is X (W + A diag(gamma) B)^T."""
    L = vg_layer(np.random.default_rng(23), r=12)
    h = 5
    rng = np.random.default_rng(24)
    G1 = f16bits(np.zeros((L["r"], h)))
    c1b = f16bits(rng.normal(0.0, 1.0, h))          # both signs: the ReLU matters
    G2b = f16bits(rng.normal(0.0, 1.0, (h, L["r"])))
    c2b = f16bits(rng.normal(0.0, 1.0, L["r"]))
    out = vg_run(L["M"], L["N"], L["K"], L["r"], L["G"], h, L["Xb"], L["qc"], L["s"], L["z"],
                 L["Ab"], L["Bb"], G1, c1b, G2b, c2b)
    f = lambda b: b.view(np.float16).astype(np.float64)
    gam = expit(np.matmul(np.maximum(f(c1b), 0.0), f(G2b)) + f(c2b))
    np.testing.assert_allclose(out["gamma"], np.broadcast_to(gam, out["gamma"].shape), rtol=1e-13, atol=1e-15)
    ref = np.matmul(L["X"], L["W"].T + np.matmul(L["A"] * gam[None, :], L["B"]))
    np.testing.assert_allclose(out["Y"], ref, rtol=1e-11, atol=1e-11 * np.abs(ref).max())


def test_vgate_permutation_bottleneck():
    """h = r, G1 a permutation (u_i = relu(T_pi(i))), G2 = beta times the
    inverse permutation: each component's gate is sigmoid(beta relu(T_j) + c2_j).
    A transposed G1 or G2, or a misplaced ReLU, breaks the identity."""
    L = vg_layer(np.random.default_rng(25), r=6)
    r = h = L["r"]
    pi = np.array([1, 2, 3, 4, 5, 0])              # one 6-cycle: no power below 6 is the identity
    beta = 1.5
    G1 = np.zeros((r, h)); G1[pi, np.arange(h)] = 1.0
    G2 = np.zeros((h, r)); G2[np.arange(h), pi] = beta
    c2b = f16bits(np.linspace(-1.0, 1.0, r))
    out = vg_run(L["M"], L["N"], L["K"], r, L["G"], h, L["Xb"], L["qc"], L["s"], L["z"],
                 L["Ab"], L["Bb"], f16bits(G1), f16bits(np.zeros(h)), f16bits(G2), c2b)
    T = np.matmul(L["X"], L["A"])
    assert (T < 0).any() and (T > 0).any()
    gam = expit(beta * np.maximum(T, 0.0) + c2b.view(np.float16).astype(np.float64)[None, :])
    np.testing.assert_allclose(out["T"], T, rtol=1e-12, atol=1e-12 * np.abs(T).max())
    np.testing.assert_allclose(out["gamma"], gam, rtol=1e-12, atol=1e-15)
    C = np.matmul(T * gam, L["B"])
    np.testing.assert_allclose(out["C"], C, rtol=1e-11, atol=1e-11 * np.abs(C).max())
    np.testing.assert_allclose(out["Y"], out["Y0"] + C, rtol=1e-11, atol=1e-11 * np.abs(C).max())


def test_vgate_rows_and_token_permutation():
    L = vg_layer(np.random.default_rng(26))
    h = 4
    p = synth.make_vgate(L["r"], h, seed=3)
    args = (L["qc"], L["s"], L["z"], L["Ab"], L["Bb"], p["G1"], p["c1"], p["G2"], p["c2"])
    full = vg_run(L["M"], L["N"], L["K"], L["r"], L["G"], h, L["Xb"], *args)
    pm = np.random.default_rng(27).permutation(L["M"])
    tp = vg_run(L["M"], L["N"], L["K"], L["r"], L["G"], h, L["Xb"][pm], *args)
    assert np.array_equal(tp["Y"], full["Y"][pm])
    rows = [3, 0, 8, 3]
    sub = vg_run(L["M"], L["N"], L["K"], L["r"], L["G"], h, L["Xb"], *args, rows=rows)
    assert np.array_equal(sub["Y"], full["Y"][rows])


# ---------------------------------------------------------------- salient-channel correction

def sq_run(L, S, Rb, rows=None):
    return oracle.forward_serq(L["Xb"], L["qc"], L["s"], L["z"], S, Rb, N=L["N"], K=L["K"],
                               group_size=L["G"], rows=rows)


def test_serq_empty_or_zero_factor_is_plain_w4():
    L = vg_layer(np.random.default_rng(31))
    base = run(L["M"], L["N"], L["K"], 0, L["G"], L["Xb"], L["qc"], L["s"], L["z"], None, None, None, 0.0)
    none = sq_run(L, None, None)
    assert np.array_equal(none["Y"], base["Y"])
    S = np.array([3, 7, 7, 200], np.int32)
    zero = sq_run(L, S, f16bits(np.zeros((4, L["N"]))))
    assert np.array_equal(zero["Y"], base["Y"])


def test_serq_all_channels_is_a_full_correction():
    """S = every channel in order: Y = X (Wd^T + R) with R a full K x N matrix."""
    L = vg_layer(np.random.default_rng(32))
    rng = np.random.default_rng(33)
    Rb = f16bits(rng.standard_normal((L["K"], L["N"])) * 0.01)
    out = sq_run(L, np.arange(L["K"], dtype=np.int32), Rb)
    ref = np.matmul(L["X"], L["W"].T + Rb.view(np.float16).astype(np.float64))
    np.testing.assert_allclose(out["Y"], ref, rtol=1e-11, atol=1e-11 * np.abs(ref).max())


def test_serq_gather_against_numpy():
    """An unsorted subset with a repeated channel: C = X[:, S] R by numpy
    indexing and matmul; the split Y = Y0 + C; rows of R follow S."""
    L = vg_layer(np.random.default_rng(34))
    rng = np.random.default_rng(35)
    S = np.array([250, 3, 17, 3, 128, 0, 255], np.int32)
    Rb = f16bits(rng.standard_normal((len(S), L["N"])) * 0.05)
    out = sq_run(L, S, Rb)
    C = np.matmul(L["X"][:, S], Rb.view(np.float16).astype(np.float64))
    np.testing.assert_allclose(out["C"], C, rtol=1e-12, atol=1e-12 * np.abs(C).max())
    ref = np.matmul(L["X"], L["W"].T) + C
    np.testing.assert_allclose(out["Y"], ref, rtol=1e-11, atol=1e-11 * np.abs(ref).max())
    # permuting the list and R's rows together changes nothing but the order of the sum
    p = rng.permutation(len(S))
    perm = sq_run(L, S[p], Rb[p])
    np.testing.assert_allclose(perm["Y"], out["Y"], rtol=1e-13, atol=1e-13 * np.abs(out["Y"]).max())
    rows = [4, 0, 4]
    sub = sq_run(L, S, Rb, rows=rows)
    assert np.array_equal(sub["Y"], out["Y"][rows])


def test_serq_rejects_out_of_range_channels():
    L = vg_layer(np.random.default_rng(36))
    with pytest.raises(RuntimeError):
        sq_run(L, np.array([0, L["K"]], np.int32), f16bits(np.zeros((2, L["N"]))))


# ---------------------------------------------------------------- codebook weights + sparse outliers

def xfp_dense(idx, cbb, row_ptr, col_idx, valb):
    """Wh by numpy: fancy indexing into the codebooks, residuals added at their positions."""
    cb = cbb.view(np.float16).astype(np.float64)
    Wh = np.take_along_axis(cb, idx.astype(np.int64), axis=1)
    rows = np.repeat(np.arange(len(row_ptr) - 1), np.diff(row_ptr))
    np.add.at(Wh, (rows, col_idx), valb.view(np.float16).astype(np.float64))
    return Wh


def test_xfp_linear_codebook_is_the_w4_layer():
    """cb[n][q] = (q - z_n) s_n with power-of-two scales (exact in fp16) and
    no outliers: the same weights as the W4 layer, summed in the same order."""
    rng = np.random.default_rng(41)
    M, N, K = 5, 24, 256
    q = rng.integers(0, 16, size=(N, K)).astype(np.uint8)
    z = rng.integers(0, 16, size=(N, 1)).astype(np.float64)
    s = np.exp2(rng.integers(-9, -4, size=(N, 1))).astype(np.float64)
    cb = (np.arange(16)[None, :] - z) * s
    Xb = f16bits(rng.standard_normal((M, K)))
    qc = pack_canonical(q)
    empty = np.zeros(0, np.int32)
    out = oracle.forward_xfp(Xb, qc, f16bits(cb), np.zeros(N + 1, np.int32), empty, np.zeros(0, np.uint16),
                             N=N, K=K)
    w4 = run(M, N, K, 0, K, Xb, qc, f16bits(s), f16bits(z), None, None, None, 0.0)
    assert np.array_equal(out["Y"], w4["Y"])


def test_xfp_against_numpy_dense():
    rng = np.random.default_rng(42)
    M, N, K = 6, 40, 512
    W = rng.standard_normal((N, K)) * 0.02
    W[rng.random((N, K)) < 0.01] *= 12.0                   # heavy tail: outliers to separate
    x = synth.make_xfp(W)
    assert x["row_ptr"][-1] > 0
    Xb = f16bits(rng.standard_normal((M, K)))
    out = oracle.forward_xfp(Xb, pack_canonical(x["idx"]), x["cb"], x["row_ptr"], x["col_idx"], x["val"], N=N, K=K)
    Wh = xfp_dense(x["idx"], x["cb"], x["row_ptr"], x["col_idx"], x["val"])
    ref = np.matmul(Xb.view(np.float16).astype(np.float64), Wh.T)
    np.testing.assert_allclose(out["Y"], ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
    # the residual restores the outliers (to fp16 rounding of the residual)
    rows = np.repeat(np.arange(N), np.diff(x["row_ptr"]))
    np.testing.assert_allclose(Wh[rows, x["col_idx"]], W[rows, x["col_idx"]], rtol=0, atol=1e-3)


def test_xfp_sparse_only_and_repeated_entries():
    """An all-zero codebook leaves the sparse part alone; two entries at one
    position add up."""
    rng = np.random.default_rng(43)
    M, N, K = 3, 8, 128
    Xb = f16bits(rng.standard_normal((M, K)))
    row_ptr = np.array([0, 2, 2, 5, 5, 5, 6, 6, 8], np.int32)
    col_idx = np.array([3, 3, 0, 127, 64, 9, 10, 11], np.int32)
    valb = f16bits(rng.standard_normal(8))
    idx = rng.integers(0, 16, size=(N, K)).astype(np.uint8)
    out = oracle.forward_xfp(Xb, pack_canonical(idx), f16bits(np.zeros((N, 16))), row_ptr, col_idx, valb, N=N, K=K)
    D = xfp_dense(idx, f16bits(np.zeros((N, 16))), row_ptr, col_idx, valb)
    ref = np.matmul(Xb.view(np.float16).astype(np.float64), D.T)
    np.testing.assert_allclose(out["Y"], ref, rtol=1e-13, atol=1e-13 * np.abs(ref).max())
    assert out["Y"][:, 1].tolist() == [0.0] * M
    with pytest.raises(RuntimeError):
        bad = col_idx.copy(); bad[0] = K
        oracle.forward_xfp(Xb, pack_canonical(idx), f16bits(np.zeros((N, 16))), row_ptr, bad, valb, N=N, K=K)


def test_xfp_row_subsets_and_malformed_rows():
    rng = np.random.default_rng(44)
    M, N, K = 5, 16, 256
    W = rng.standard_normal((N, K)) * 0.02
    W[rng.random((N, K)) < 0.02] *= 15.0
    x = synth.make_xfp(W)
    Xb = f16bits(rng.standard_normal((M, K)))
    qc = pack_canonical(x["idx"])
    full = oracle.forward_xfp(Xb, qc, x["cb"], x["row_ptr"], x["col_idx"], x["val"], N=N, K=K)["Y"]
    rows = [3, 0, 3]
    sub = oracle.forward_xfp(Xb, qc, x["cb"], x["row_ptr"], x["col_idx"], x["val"], N=N, K=K, rows=rows)["Y"]
    assert np.array_equal(sub, full[rows])
    bad = x["row_ptr"].copy()
    n = int(np.argmax(np.diff(bad) > 0))                   # a row with entries
    bad[n + 1] = bad[n] - 1                                 # decreasing pointers
    with pytest.raises((RuntimeError, AssertionError)):
        oracle.forward_xfp(Xb, qc, x["cb"], bad, x["col_idx"], x["val"], N=N, K=K)


# ---------------------------------------------------------------- codebook weights from a shared library

def xfp_lib_dense(idx, libb, libid, row_ptr, col_idx, valb):
    """Wh by numpy: each group of 128 weights indexes its library entry."""
    lib = libb.view(np.float16).astype(np.float64)
    N, K = idx.shape
    ent = np.repeat(libid.astype(np.int64), 128, axis=1)                 # [N, K] library entry per weight
    Wh = lib[ent, idx.astype(np.int64)]
    rows = np.repeat(np.arange(N), np.diff(row_ptr))
    np.add.at(Wh, (rows, col_idx), valb.view(np.float16).astype(np.float64))
    return Wh


def test_xfp_lib_with_a_library_entry_per_channel_is_the_per_channel_mode():
    """L = N and every group of channel n naming entry n: the per-channel
    codebooks exactly (same weights, same order)."""
    rng = np.random.default_rng(51)
    M, N, K = 4, 24, 384
    W = rng.standard_normal((N, K)) * 0.02
    W[rng.random((N, K)) < 0.01] *= 10.0
    x = synth.make_xfp(W)
    Xb = f16bits(rng.standard_normal((M, K)))
    qc = pack_canonical(x["idx"])
    libid = np.repeat(np.arange(N, dtype=np.uint8)[:, None], K // 128, axis=1)
    per_ch = oracle.forward_xfp(Xb, qc, x["cb"], x["row_ptr"], x["col_idx"], x["val"], N=N, K=K)["Y"]
    lib = oracle.forward_xfp_lib(Xb, qc, x["cb"], libid, x["row_ptr"], x["col_idx"], x["val"], N=N, K=K)["Y"]
    assert np.array_equal(lib, per_ch)


def test_xfp_lib_against_numpy_dense():
    rng = np.random.default_rng(52)
    M, N, K = 6, 40, 640
    W = rng.standard_normal((N, K)) * 0.02 * np.exp(rng.standard_normal((N, 1)))
    W[rng.random((N, K)) < 0.01] *= 12.0
    x = synth.make_xfp_lib(W, L=32)
    assert len(np.unique(x["libid"])) > 4 and x["row_ptr"][-1] > 0
    Xb = f16bits(rng.standard_normal((M, K)))
    out = oracle.forward_xfp_lib(Xb, pack_canonical(x["idx"]), x["lib"], x["libid"], x["row_ptr"],
                                 x["col_idx"], x["val"], N=N, K=K)
    Wh = xfp_lib_dense(x["idx"], x["lib"], x["libid"], x["row_ptr"], x["col_idx"], x["val"])
    ref = np.matmul(Xb.view(np.float16).astype(np.float64), Wh.T)
    np.testing.assert_allclose(out["Y"], ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
    # the weights it encodes are close to W (4-bit library codebooks; outliers restored)
    rel = np.abs(Wh - W).mean() / np.abs(W).mean()
    assert rel < 0.15, rel


def test_xfp_lib_group_boundaries():
    """Entry 1 holds 1.0 at index 3, entry 0 zero: with every index 3 and
    the groups' entries alternating, each output sums exactly the inputs of
    the groups (128 consecutive k) that name entry 1."""
    rng = np.random.default_rng(53)
    M, N, K = 3, 5, 768
    libv = np.zeros((2, 16))
    libv[1, 3] = 1.0
    idx = np.full((N, K), 3, np.uint8)
    libid = rng.integers(0, 2, size=(N, K // 128)).astype(np.uint8)
    X = rng.integers(-8, 9, size=(M, K)).astype(np.float64)           # small integers: exact sums
    out = oracle.forward_xfp_lib(f16bits(X), pack_canonical(idx), f16bits(libv), libid,
                                 np.zeros(N + 1, np.int32), np.zeros(0, np.int32), np.zeros(0, np.uint16),
                                 N=N, K=K)["Y"]
    for n in range(N):
        want = sum(X[:, g * 128:(g + 1) * 128].sum(axis=1) for g in range(K // 128) if libid[n, g] == 1)
        want = np.zeros(M) if isinstance(want, int) else want
        assert np.array_equal(out[:, n], want)


def test_xfp_lib_relabelled_library_and_bad_ids():
    """Permuting the library and relabelling the groups' entries leaves Y
    unchanged; an entry id past the library is rejected."""
    rng = np.random.default_rng(54)
    M, N, K = 4, 16, 256
    W = rng.standard_normal((N, K)) * 0.02
    x = synth.make_xfp_lib(W, L=8)
    Xb = f16bits(rng.standard_normal((M, K)))
    qc = pack_canonical(x["idx"])
    args = (x["row_ptr"], x["col_idx"], x["val"])
    base = oracle.forward_xfp_lib(Xb, qc, x["lib"], x["libid"], *args, N=N, K=K)["Y"]
    perm = rng.permutation(8)                                           # new entry j holds old entry perm[j]
    inv = np.argsort(perm).astype(np.uint8)
    again = oracle.forward_xfp_lib(Xb, qc, np.ascontiguousarray(x["lib"][perm]), inv[x["libid"]], *args, N=N, K=K)["Y"]
    assert np.array_equal(again, base)
    bad = x["libid"].copy()
    bad[2, 1] = 8
    with pytest.raises(RuntimeError):
        oracle.forward_xfp_lib(Xb, qc, x["lib"], bad, *args, N=N, K=K)
