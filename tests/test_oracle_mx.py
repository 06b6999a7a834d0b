"""Pins of the MXFP8 oracle (OCP Microscaling reading of the Mixture-of-Kittens
notes, section 5: routed experts in MXFP8).

The format facts used here come from the E4M3 and E8M0 definitions, not from
the oracle: an E4M3 code s.eeee.mmm is (-1)^s (1 + m/8) 2^(e-7) for e > 0 and
(-1)^s (m/8) 2^-6 for e = 0, with s.1111.111 not a number; a block's scale is
2^(floor(log2 amax) - 8).
"""
import math

import numpy as np
import pytest

import oracle
from routing_schedule_expert_amd import inputs


def closed_form(code):
    s, e, m = (code >> 7) & 1, (code >> 3) & 15, code & 7
    if e == 15 and m == 7:
        return math.nan
    v = (m / 8) * 2.0 ** -6 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
    return -v if s else v


FINITE = [c for c in range(256) if not math.isnan(closed_form(c))]


def test_e4m3_decode_matches_closed_form():
    t = oracle.e4m3_table()
    for c in range(256):
        ref = closed_form(c)
        assert (math.isnan(ref) and math.isnan(t[c])) or t[c] == ref, hex(c)
    assert t[0x7E] == 448.0 and t[0x01] == 2.0 ** -9 and t[0x38] == 1.0


def test_encode_decode_identity():
    for c in FINITE:
        assert oracle.e4m3_encode(closed_form(c)) == c, hex(c)


def test_ties_to_even_and_nearest():
    mags = sorted({abs(closed_form(c)) for c in FINITE})
    for lo, hi in zip(mags, mags[1:]):
        mid = (lo + hi) / 2
        c_lo, c_hi = oracle.e4m3_encode(lo), oracle.e4m3_encode(hi)
        even = c_lo if c_lo % 2 == 0 else c_hi  # mantissa parity = the code's last bit
        assert oracle.e4m3_encode(mid) == even, (lo, hi)
        assert oracle.e4m3_encode(mid - (hi - lo) / 8) == c_lo
        assert oracle.e4m3_encode(mid + (hi - lo) / 8) == c_hi
        assert oracle.e4m3_encode(-mid) == even | 0x80


def test_saturation():
    for y in (448.0, 449.0, 464.0, 480.0, 1e6):
        assert oracle.e4m3_encode(y) == 0x7E
        assert oracle.e4m3_encode(-y) == 0xFE


def bf16_bits(x):
    return inputs.bf16_bits(np.asarray(x, np.float32))


def test_block_scale_exponent():
    rng = np.random.default_rng(0)
    for k in range(-20, 20):
        x = rng.uniform(-1, 1, 32).astype(np.float32) * 2.0 ** k
        x[rng.integers(32)] = 1.5 * 2.0 ** k  # amax in [2^k, 2^(k+1))
        q, s = oracle.mx_quantize(bf16_bits(x)[None])
        xb = inputs.bf16_to_f32(bf16_bits(x))
        amax = np.abs(xb).max()
        assert s[0, 0] == math.floor(math.log2(amax)) - 8 + 127
    q, s = oracle.mx_quantize(np.zeros((1, 64), np.uint16))
    assert (s == 0).all() and (q == 0).all()


def test_quantization_error_bound():
    rng = np.random.default_rng(1)
    x = inputs.bf16_to_f32(bf16_bits(rng.standard_normal((64, 256)).astype(np.float32) * 3)).astype(np.float64)
    q, s = oracle.mx_quantize(bf16_bits(x))
    d = oracle.mx_dequantize(q, s)
    scale = np.repeat(np.ldexp(1.0, s.astype(np.int64) - 127), 32, axis=-1)
    y = x / scale
    # E4M3 normals carry 3 mantissa bits (relative error <= 2^-4), subnormals
    # a quantum of 2^-9 (absolute error <= 2^-10 in units of the scale), and
    # anything at or above 448 clips to 448
    ok = np.where(np.abs(y) >= 448, np.abs(d) == 448 * scale,
                  np.abs(d - x) <= np.maximum(2.0 ** -4 * np.abs(x), 2.0 ** -10 * scale) * (1 + 1e-12))
    assert ok.all()
    assert np.sign(d)[d != 0].tolist() == np.sign(x)[d != 0].tolist()


def small_mx_layer(seed=3, P=2, Np=96, E=8, K=2, L=4, H=128, I=64):
    h = inputs.make_layer_inputs(seed, P, Np, E, K, L, H, I, routing="topk", x_std=1.0)
    Xq, Xs = oracle.mx_quantize(h["X"])
    W13q, W13s = oracle.mx_quantize(h["W13"])
    W2q, W2s = oracle.mx_quantize(h["W2"])
    return h, (Xq, Xs, W13q, W13s, W2q, W2s), L


def test_mx_ffn_dot_products_vs_numpy():
    h, (Xq, Xs, W13q, W13s, W2q, W2s), L = small_mx_layer()
    s = oracle.schedule(h["routes"], L, 0, 256)
    Xdq, Xds = oracle.mx_dispatch(Xq, Xs, s.phi)
    r = oracle.mx_expert_ffn_rows(s.seg_off, Xdq, Xds, W13q, W13s, W2q, W2s)
    Xd = oracle.mx_dequantize(Xdq, Xds)
    W13 = oracle.mx_dequantize(W13q, W13s)
    W2 = oracle.mx_dequantize(W2q, W2s)
    I = W13.shape[1] // 2
    for l in range(L):
        rows = np.arange(s.seg_off[l], s.seg_off[l + 1])
        if rows.size == 0:
            continue
        hu = Xd[rows] @ W13[l].T
        a = hu[:, :I] / (1 + np.exp(-hu[:, :I])) * hu[:, I:]
        np.testing.assert_allclose(r["A"][rows], a, rtol=1e-9, atol=1e-12)
        aq, as_ = oracle.mx_quantize_f64(a)
        np.testing.assert_array_equal(r["Aq"][rows], aq)
        np.testing.assert_array_equal(r["As"][rows], as_)
        y = oracle.mx_dequantize(aq, as_) @ W2[l].T
        np.testing.assert_allclose(r["Y"][rows], y, rtol=1e-9, atol=1e-12)
    # padding rows read zeros
    pad = s.phi[:, 0] < 0
    assert not r["Y"][pad].any()


def test_mx_token_path_equals_rows_and_combine():
    h, mx, L = small_mx_layer(seed=4)
    s = oracle.schedule(h["routes"], L, 0, 256)
    Xdq, Xds = oracle.mx_dispatch(mx[0], mx[1], s.phi)
    r = oracle.mx_expert_ffn_rows(s.seg_off, Xdq, Xds, *mx[2:])
    via_rows = oracle.combine(s.route_row, h["w"], r["Y"])
    direct = oracle.mx_layer_fwd_tokens(h["routes"], h["w"], *mx, L=L)
    np.testing.assert_allclose(direct, via_rows, rtol=1e-9, atol=1e-12)


def test_mx_forward_close_to_bf16_forward():
    h, mx, L = small_mx_layer(seed=5)
    out_mx = oracle.mx_layer_fwd_tokens(h["routes"], h["w"], *mx, L=L)
    out = oracle.layer_fwd_tokens(h["routes"], h["w"], h["X"], h["W13"], h["W2"], L=L)
    err = np.linalg.norm(out_mx - out) / np.linalg.norm(out)
    assert 1e-3 < err < 0.1  # quantization error of three 3-bit-mantissa operands, not zero


def test_mx_rows_pre_activations():
    """with_hu: a = silu(h) * u from the returned h and u, the returned A and
    codes unchanged, and each magnitude sum at least |h| or |u|; a row whose
    X codes are a single nonzero element has sums equal to |h| and |u|."""
    h = inputs.make_layer_inputs(12, 2, 64, 8, 2, 4, 256, 128, routing="topk", x_std=1.0)
    s = oracle.schedule(h["routes"], 4, 0, 256)
    Xq, Xs = oracle.mx_quantize(h["X"])
    W13q, W13s = oracle.mx_quantize(h["W13"])
    W2q, W2s = oracle.mx_quantize(h["W2"])
    Xdq, Xds = oracle.mx_dispatch(Xq, Xs, s.phi)
    plain = oracle.mx_expert_ffn_rows(s.seg_off, Xdq, Xds, W13q, W13s, W2q, W2s)
    r = oracle.mx_expert_ffn_rows(s.seg_off, Xdq, Xds, W13q, W13s, W2q, W2s, with_hu=True)
    for k in ("A", "Aq", "As", "Y"):
        assert np.array_equal(plain[k], r[k])
    I = 128
    hh, uu = r["HU"][:, :I], r["HU"][:, I:]
    np.testing.assert_allclose(hh / (1 + np.exp(-hh)) * uu, r["A"], rtol=1e-12, atol=1e-300)
    assert np.all(r["HUabs"] >= np.abs(r["HU"]) * (1 - 1e-12))
    one = Xdq.copy()
    real = np.nonzero(s.phi[:, 0] >= 0)[0][0]
    one[real] = 0
    one[real, 5] = Xdq[real, 5] if Xdq[real, 5] & 0x7f else 0x38
    r1 = oracle.mx_expert_ffn_rows(s.seg_off, one, Xds, W13q, W13s, W2q, W2s, rows=[real], with_hu=True)
    np.testing.assert_array_equal(r1["HUabs"], np.abs(r1["HU"]))
