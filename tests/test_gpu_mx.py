"""MXFP8 routed experts on the GPU vs the CPU oracle (OCP microscaling reading
of the Mixture-of-Kittens notes, section 5).

Quantization of bf16 inputs (X, W13, W2) is a fixed function of the input, so
codes and scale bytes must match the oracle bit for bit.  The activation a is
accumulated by the scaled fp8 MFMA in fp32 on the GPU and in fp64 by the
oracle before it is quantized, so where the exact value sits close to a
rounding boundary (or h cancels) the GPU's code may differ: every a code (and
block scale) must be explained by an error in h and u of at most 2^-14 of the
sum of their terms' magnitudes.  Y of every compared row and out of every
compared token must be within rel-L2 1e-2 of the oracle's MX path, plus the
exact effect of the differing codes on the row (the norm of W2 times the code
differences);
padding rows exactly zero; repeated runs bitwise identical.
"""
import numpy as np
import pytest
import torch

import oracle
from routing_schedule_expert_amd import inputs, ops
from tests.helpers import dev, expected_single_route_table, f64, fused_y_rows, on_dev_mask, single_route_terms, up, up_bf16

pytestmark = pytest.mark.gpu
TOL = 1e-2


# Accumulation error allowed in the GPU's h and u, relative to the sum of the
# magnitudes of their terms (the scaled fp8 MFMA accumulates in fp32 with its
# own internal summation; the oracle sums in fp64).
ACC = 2.0 ** -14


def _silu(h):
    return h / (1.0 + np.exp(-h))


def validate_a_codes(name, Aq_g, As_g, A_ref, Aq_ref, As_ref, HU, HUabs):
    """GPU codes of a against the oracle's.  A GPU code (and block scale) is
    valid when some h', u' within ACC * (sum of term magnitudes) of the exact
    h, u give an a' that rounds to it: the exact value of a must lie within
    that error bound of the code's rounding interval.  Returns the value
    difference (GPU - oracle, dequantized) per element."""
    table = oracle.e4m3_table()
    vals = np.unique(table[np.isfinite(table)])
    I = A_ref.shape[1]
    h, u = HU[:, :I], HU[:, I:]
    sh, su = HUabs[:, :I], HUabs[:, I:]
    sg = 1.0 / (1.0 + np.exp(-h))
    bound = ACC * (np.abs(sg * (1.0 + h * (1.0 - sg)) * u) * sh + np.abs(_silu(h)) * su) + 2.0 ** -20 * np.abs(A_ref)
    sc_g = np.repeat(np.ldexp(1.0, np.asarray(As_g, np.int64) - 127), 32, axis=-1)
    sc_r = np.repeat(np.ldexp(1.0, np.asarray(As_ref, np.int64) - 127), 32, axis=-1)
    # a different block scale: the block maximum must sit within its bound of
    # the power of two between the two scales
    bad_blk = np.asarray(As_g) != np.asarray(As_ref)
    if bad_blk.any():
        amax = np.abs(A_ref).reshape(A_ref.shape[0], -1, 32).max(-1)
        bmax = bound.reshape(A_ref.shape[0], -1, 32).max(-1)
        edge = np.ldexp(1.0, np.maximum(As_g, As_ref).astype(np.int64) - 127 + 8)
        ok = np.abs(amax - edge) <= bmax
        print(f"    {name}: {bad_blk.sum()} block scales differ (block maximum within its bound of the "
              f"power of two: {ok[bad_blk].all()})", flush=True)
        assert ok[bad_blk].all(), f"{name}: a block scale differs away from a power of two"
    vg, vr = table[np.asarray(Aq_g, np.int64)], table[np.asarray(Aq_ref, np.int64)]
    diff = (vg * sc_g) != (vr * sc_r)
    if diff.any():
        y = (A_ref / sc_g)[diff]
        v = vg[diff]
        k = np.searchsorted(vals, v)
        lo = np.where(k > 0, 0.5 * (vals[np.maximum(k - 1, 0)] + v), -np.inf)
        hi = np.where(k < len(vals) - 1, 0.5 * (v + vals[np.minimum(k + 1, len(vals) - 1)]), np.inf)
        dist = np.maximum(0.0, np.maximum(lo - y, y - hi))
        need = dist * sc_g[diff] / np.maximum(bound[diff] / ACC, 1e-300)
        print(f"    {name}: {diff.sum()} of {diff.size} codes differ from the oracle's; the accumulation "
              f"error they imply is at most {need.max():.2e} of the terms' magnitudes (allowed {ACC:.2e})",
              flush=True)
        assert need.max() <= ACC, f"{name}: a code is not explained by accumulation error ({need.max():.3e})"
    return np.where(diff, vg * sc_g - vr * sc_r, 0.0)


def assert_rows_allow(name, got, ref, allow, tol, ids=None):
    """Per row: |got - ref| <= tol |ref| + allow (norms over the row)."""
    got = np.asarray(got, np.float64).reshape(len(got), -1)
    ref = np.asarray(ref, np.float64).reshape(len(ref), -1)
    num = np.linalg.norm(got - ref, axis=1)
    den = np.linalg.norm(ref, axis=1)
    excess = num - tol * den - np.asarray(allow)
    i = int(np.argmax(num / np.maximum(tol * den + allow, 1e-300)))
    where = int(ids[i]) if ids is not None else i
    print(f"    {name}: {len(num)} rows, worst row {where}: rel-L2 {num[i] / max(den[i], 1e-300):.2e}, "
          f"near-tie allowance {allow[i] / max(den[i], 1e-300):.2e} of the row", flush=True)
    assert (excess <= 0).all(), f"{name}: row {where} off by {num[i]:.3e} (norm {den[i]:.3e})"


def near_tie_allowance(delta, rows, seg_off, W2q, W2s):
    """Per row, the norm of W2[l] times the row's code differences: exactly
    what the near-tie codes change in Y."""
    out = np.zeros(len(rows))
    experts = np.searchsorted(seg_off, rows, side="right") - 1
    for l in np.unique(experts):
        sel = np.nonzero(experts == l)[0]
        if not delta[sel].any():
            continue
        W = oracle.mx_dequantize(W2q[l], W2s[l])  # [H][I]
        out[sel] = np.linalg.norm(delta[sel] @ W.T, axis=1)
    return out


def bf16_bits(x):
    return inputs.bf16_bits(np.asarray(x, np.float32))


def edge_rows(rng, K):
    """Rows that exercise the quantizer's corner cases, 32-element blocks."""
    rows = [rng.standard_normal(K) * 3]
    z = rng.standard_normal(K)
    z[:32] = 0.0                                   # all-zero block
    z[32:64] = -0.0
    rows.append(z)
    rows.append(rng.standard_normal(K) * 1e-39)   # bf16 subnormals
    s = rng.standard_normal(K)
    s[::32] = 1.9375 * np.sign(s[::32] + 1e-9)    # maxima with mantissa > 1.75: saturation
    rows.append(s)
    m = rng.standard_normal(K) * 1e-4
    m[5::32] = 1e4                                 # tiny elements under a large maximum
    rows.append(m)
    t = np.zeros(K)
    t[:] = 1.0625                                  # ties at 1.0625 * 2^8 after scaling: to even
    t[::32] = 1.0
    rows.append(t)
    return np.stack(rows).astype(np.float32)


@pytest.mark.parametrize("K", [32, 256, 7168])
def test_quantize_bit_exact(K):
    rng = np.random.default_rng(K)
    x = np.concatenate([edge_rows(rng, K), rng.standard_normal((57, K)).astype(np.float32) * 0.02])
    xb = bf16_bits(x)
    q_ref, s_ref = oracle.mx_quantize(xb)
    src = up_bf16(xb)
    q, s = ops.quantize_mx(src)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(q.cpu().numpy(), q_ref)
    np.testing.assert_array_equal(s.cpu().numpy(), s_ref)


def test_quantize_every_bf16_value_at_unit_scale():
    """Every bf16 value below 512 in magnitude (both signs, zeros and
    subnormals included) through the device quantizer at block scale 1: each
    32-element block holds the anchor 256 (scale exponent 0) and 31 of the
    values, so every E4M3 rounding midpoint (all of them bf16 values), every
    subnormal step and the saturation between 448 and 512 is met, in every
    position of a packed code word.  Row codes (moe_quantize_mx) and column
    codes (moe_quantize_mx_t) bit for bit against the oracle."""
    pats = np.arange(0x8000, dtype=np.uint32)
    vals = (pats << 16).view(np.float32)
    vals = vals[np.isfinite(vals) & (np.abs(vals) < 512)]
    vals = np.concatenate([vals, -vals])
    nblk = -(-vals.size // 31)
    blocks = np.zeros((nblk, 32), np.float32)
    flat = np.zeros(nblk * 31, np.float32)
    flat[:vals.size] = vals
    blocks[:, 1:] = flat.reshape(nblk, 31)
    blocks[:, 0] = 256.0
    shift = np.arange(nblk) % 32                        # the anchor in every position
    blocks = blocks[np.arange(nblk)[:, None], (np.arange(32)[None, :] - shift[:, None]) % 32]
    nrow = -(-nblk // 64 // 8) * 8  # a multiple of 8 columns for the transposed call
    x = np.zeros((nrow * 64, 32), np.float32)
    x[:nblk] = blocks
    x[nblk:, 0] = 256.0
    xb = bf16_bits(x.reshape(nrow, 64 * 32))
    q_ref, s_ref = oracle.mx_quantize(xb)
    assert (s_ref == 127).all()
    q, s = ops.quantize_mx(up_bf16(xb))
    np.testing.assert_array_equal(q.cpu().numpy(), q_ref)
    np.testing.assert_array_equal(s.cpu().numpy(), s_ref)
    # the same values as columns: [R = 2048][C = nrow] quantized along R
    xt = np.ascontiguousarray(xb.T)
    qt, st = ops.quantize_mx_t(up_bf16(xt))
    qt_ref, st_ref = oracle.mx_transpose_quantize(xt)
    np.testing.assert_array_equal(qt.cpu().numpy(), qt_ref)
    np.testing.assert_array_equal(st.cpu().numpy(), st_ref)


def test_quantize_large_bit_exact():
    rng = np.random.default_rng(9)
    xb = bf16_bits(rng.standard_normal((2048, 2048)).astype(np.float32))
    q_ref, s_ref = oracle.mx_quantize(xb)
    q, s = ops.quantize_mx(up_bf16(xb))
    np.testing.assert_array_equal(q.cpu().numpy(), q_ref)
    np.testing.assert_array_equal(s.cpu().numpy(), s_ref)


class MxLayer:
    def __init__(self, seed, P, Np, E, K, L, H, I, routing="uniform", s=1.2, base=0):
        self.h = inputs.make_layer_inputs(seed, P, Np, E, K, L, H, I, routing=routing, base=base, x_std=1.0, s=s)
        self.P, self.Np, self.K, self.L, self.H, self.I, self.base = P, Np, K, L, H, I, base
        self.d = ops.make_desc(P, Np, K, E, L, expert_base=base, H=H, I=I)
        self.routes, self.w = up(self.h["routes"]), up(self.h["w"])
        self.X = up_bf16(self.h["X"])
        self.W13q, self.W13s = ops.quantize_mx(up_bf16(self.h["W13"]))
        self.W2q, self.W2s = ops.quantize_mx(up_bf16(self.h["W2"]))

    def fwd(self, ws_fill=None):
        b = ops.alloc_fwd_mx(self.d, dev())
        if ws_fill is not None:  # what an earlier call could have left there
            b.ws.view(torch.int32).fill_(ws_fill)
        ops.layer_fwd_mx(self.d, self.routes, self.w, self.X, self.W13q, self.W13s, self.W2q, self.W2s, b)
        torch.cuda.synchronize()
        return b


def check_mx_full(lay: MxLayer, b):
    h = lay.h
    s = oracle.schedule(h["routes"], lay.L, lay.base, 256)
    np.testing.assert_array_equal(b.phi[: s.npad].cpu().numpy(), s.phi)
    np.testing.assert_array_equal(b.route_row.cpu().numpy(), s.route_row)
    Xq, Xs = oracle.mx_quantize(h["X"])
    np.testing.assert_array_equal(b.Xq.cpu().numpy(), Xq)
    np.testing.assert_array_equal(b.Xs.cpu().numpy(), Xs)
    W13q, W13s = oracle.mx_quantize(h["W13"])
    W2q, W2s = oracle.mx_quantize(h["W2"])
    np.testing.assert_array_equal(lay.W13q.cpu().numpy(), W13q)
    np.testing.assert_array_equal(lay.W2s.cpu().numpy(), W2s)
    Xdq, Xds = oracle.mx_dispatch(Xq, Xs, s.phi)
    r = oracle.mx_expert_ffn_rows(s.seg_off, Xdq, Xds, W13q, W13s, W2q, W2s, with_hu=True)
    real = s.phi[:, 0] >= 0
    ids = np.nonzero(real)[0]
    Aq, As = b.Aq[: s.npad].cpu().numpy(), b.As[: s.npad].cpu().numpy()
    delta = validate_a_codes("[mx] a", Aq[real], As[real], r["A"][real], r["Aq"][real], r["As"][real],
                             r["HU"][real], r["HUabs"][real])
    allow = near_tie_allowance(delta, ids, s.seg_off, W2q, W2s)
    a_gpu = oracle.mx_dequantize(Aq, As)
    # the rows of tokens with one local route go straight to out (checked
    # below); rows are selected on the device, as unwritten ones may hold any bits
    yw = fused_y_rows(h["routes"], lay.L, lay.base, s.phi)[real]
    if yw.any():
        Y = f64(b.Y[torch.from_numpy(ids[yw]).to(dev())])
        assert_rows_allow("[mx] Y", Y, r["Y"][real][yw], allow[yw], TOL, ids[yw])
    assert not f64(b.Y[: s.npad][on_dev_mask(~real)]).any()
    assert not a_gpu[~real].any()
    out = oracle.mx_layer_fwd_tokens(h["routes"], h["w"], Xq, Xs, W13q, W13s, W2q, W2s, L=lay.L, base=lay.base)
    # a token's allowance: its slots' row allowances weighted by |w|
    allow_row = np.zeros(s.npad)
    allow_row[ids] = allow
    rr = s.route_row.reshape(-1, lay.K)
    tok_allow = (np.where(rr >= 0, allow_row[np.maximum(rr, 0)], 0.0) * np.abs(h["w"].reshape(-1, lay.K))).sum(-1)
    assert_rows_allow("[mx] out", f64(b.out).reshape(out.shape), out, tok_allow, TOL)


def test_mx_tiny_forward():
    print("[mx] tiny forward", flush=True)
    lay = MxLayer(1, 2, 256, 8, 2, 4, 256, 128, routing="topk")
    check_mx_full(lay, lay.fwd())


def test_mx_small_forward_multi_tile():
    print("[mx] small forward, several tiles and ragged segments", flush=True)
    lay = MxLayer(3, 4, 700, 12, 3, 6, 512, 256, routing="zipf", s=1.2)
    check_mx_full(lay, lay.fwd())


def test_mx_nonzero_base_and_dropped_ids():
    """Local experts [5, 11) of 24 and dropped (-1) slots: tables, codes and
    outputs against the oracle's MX path with the same expert base."""
    print("[mx] expert base 5, dropped ids", flush=True)
    lay = MxLayer(17, 3, 300, 24, 3, 6, 256, 128, routing="zipf", base=5)
    rt = lay.h["routes"].copy()
    rt[:, ::5, 1] = -1
    lay.h["routes"] = rt
    lay.routes = up(rt)
    check_mx_full(lay, lay.fwd())


def test_mx_widest_rows():
    """H = 65536 codes, the widest MX row (padding rows read the static zero
    row as bytes): full check against the oracle's MX path."""
    print("[mx] H = 65536", flush=True)
    lay = MxLayer(15, 2, 64, 8, 2, 4, 65536, 128, routing="topk")
    check_mx_full(lay, lay.fwd())


def test_mx_repeat_bitwise():
    lay = MxLayer(8, 4, 500, 16, 4, 8, 512, 256, routing="zipf")
    a, b = lay.fwd(), lay.fwd()
    npad = int(a.seg_off[-1])  # rows past Npad are never written
    s = oracle.schedule(lay.h["routes"], lay.L, lay.base, 256)
    yw = on_dev_mask(fused_y_rows(lay.h["routes"], lay.L, lay.base, s.phi))  # nor Y rows of one-route tokens
    assert torch.equal(a.out, b.out)
    assert torch.equal(a.Y[:npad][yw], b.Y[:npad][yw]) and torch.equal(a.Aq[:npad], b.Aq[:npad])
    assert torch.equal(a.As[:npad], b.As[:npad])


def test_mx_single_route_table_bit_exact():
    """The MX forward's per-row table of single-route tokens (the one its down
    epilogue reads) bit for bit against the host's from the oracle schedule."""
    lay = MxLayer(10, 4, 500, 16, 4, 8, 512, 256, routing="zipf")
    b = lay.fwd(ws_fill=0)
    s = oracle.schedule(lay.h["routes"], lay.L, lay.base, 256)
    ref = expected_single_route_table(lay.h["routes"], lay.h["w"], lay.L, lay.base, s.phi)
    assert (ref[:, 0] >= 0).any() and (ref[:, 0] < 0).any()
    off = ops.workspace_field(lay.d, ops.MOE_OP_LAYER_FWD, ops.MOE_WS_SINGLE_ROUTE)
    got = np.array(ops.read_ws_words(b.ws, off, 2 * s.npad), np.int32).reshape(s.npad, 2)
    np.testing.assert_array_equal(got, ref)


def test_mx_stale_workspace():
    """The MX down tiles write the outputs of single-route tokens from a
    per-row table in the workspace: a workspace filled beforehand with words
    that name routes of tokens 0 and 1 (0 and K) must not change the output
    (bitwise a fresh workspace's, and within the oracle's bound)."""
    lay = MxLayer(9, 2, 300, 8, 2, 4, 256, 128, routing="uniform")
    ref = lay.fwd()
    for fill in (0, lay.K):
        print(f"[mx] stale workspace words {fill}", flush=True)
        b = lay.fwd(ws_fill=fill)
        assert torch.equal(b.out, ref.out)
    check_mx_full(lay, b)


def test_mx_kimi_sampled():
    """Kimi-shaped share (8 x 7,168 tokens, 384 experts with 48 local, top-8,
    H=7168, I=2048, balanced routing).  Every input the oracle sees is
    quantized on the host by the oracle itself: the weights of four sampled
    experts (including the largest segment) and the X rows of the sampled rows'
    and tokens' sources.  The GPU's codes of those weights and rows must equal
    them bit for bit; a and Y of sampled rows of the four experts (for a row
    of a token with one local route, that token's output, which the down
    GEMM writes instead of the row), and out of 256 tokens routed to them,
    within rel-L2 1e-2 per row."""
    print("[mx] Kimi shape", flush=True)
    c = dict(P=8, Np=7168, E=384, K=8, L=48, H=7168, I=2048)
    H, I, L = c["H"], c["I"], c["L"]
    h = inputs.make_layer_inputs_device(5, c["P"], c["Np"], c["E"], c["K"], L, H, I, dev(),
                                        routing="balanced", x_std=1.0)
    d = ops.make_desc(c["P"], c["Np"], c["K"], c["E"], L, H=H, I=I)
    W13q, W13s = ops.quantize_mx(h["W13"])
    W2q, W2s = ops.quantize_mx(h["W2"])
    routes, w = torch.from_numpy(h["routes"]).to(dev()), torch.from_numpy(h["w"]).to(dev())
    b = ops.alloc_fwd_mx(d, dev())
    ops.layer_fwd_mx(d, routes, w, h["X"], W13q, W13s, W2q, W2s, b)
    torch.cuda.synchronize()
    s = oracle.schedule(h["routes"], L, 0, 256)
    np.testing.assert_array_equal(b.phi[: s.npad].cpu().numpy(), s.phi)
    host = lambda t: t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    rng = np.random.default_rng(3)
    seg = np.diff(s.seg_off)
    experts = sorted({int(np.argmax(seg)), 0, 17, 47})
    # sampled rows of the four experts and sampled tokens routed to them
    sample = []
    for l in experts:
        real = np.arange(s.seg_off[l], s.seg_off[l + 1])
        real = real[s.phi[real, 0] >= 0]
        sample.append(rng.choice(real, 32, replace=False))
    rows = np.sort(np.concatenate(sample))
    rt = h["routes"].reshape(-1, c["K"])
    to_sampled = np.nonzero(np.isin(rt, experts).any(-1))[0]
    toks = np.sort(rng.choice(to_sampled, 256, replace=False))
    # host quantization (oracle) of the weights of the sampled experts ...
    W13q_h = np.zeros((L, 2 * I, H), np.uint8)
    W13s_h = np.zeros((L, 2 * I, H // 32), np.uint8)
    W2q_h = np.zeros((L, H, I), np.uint8)
    W2s_h = np.zeros((L, H, I // 32), np.uint8)
    for l in experts:
        W13q_h[l], W13s_h[l] = oracle.mx_quantize(host(h["W13"][l]))
        W2q_h[l], W2s_h[l] = oracle.mx_quantize(host(h["W2"][l]))
        np.testing.assert_array_equal(W13q[l].cpu().numpy(), W13q_h[l])
        np.testing.assert_array_equal(W13s[l].cpu().numpy(), W13s_h[l])
        np.testing.assert_array_equal(W2q[l].cpu().numpy(), W2q_h[l])
        np.testing.assert_array_equal(W2s[l].cpu().numpy(), W2s_h[l])
    # ... and of the X rows the sampled rows and tokens read
    src_tok = np.unique(np.concatenate([s.phi[rows, 0].astype(np.int64) * c["Np"] + s.phi[rows, 1], toks]))
    Xq_h = np.zeros((c["P"] * c["Np"], H), np.uint8)
    Xs_h = np.zeros((c["P"] * c["Np"], H // 32), np.uint8)
    tidx = torch.from_numpy(src_tok).to(dev())
    Xq_h[src_tok], Xs_h[src_tok] = oracle.mx_quantize(host(h["X"].view(-1, H)[tidx]))
    np.testing.assert_array_equal(b.Xq.view(-1, H)[tidx].cpu().numpy(), Xq_h[src_tok])
    np.testing.assert_array_equal(b.Xs.view(-1, H // 32)[tidx].cpu().numpy(), Xs_h[src_tok])
    Xq_h = Xq_h.reshape(c["P"], c["Np"], H)
    Xs_h = Xs_h.reshape(c["P"], c["Np"], H // 32)
    Xdq, Xds = oracle.mx_dispatch(Xq_h, Xs_h, s.phi)
    # the sampled rows, then the rows of the sampled tokens (one local slot each)
    rr = s.route_row.reshape(-1, c["K"])[toks]
    assert ((rr >= 0).sum(-1) == 1).all()
    tok_rows = rr.max(-1).astype(np.int64)
    all_rows = np.concatenate([rows, tok_rows])
    r = oracle.mx_expert_ffn_rows(s.seg_off, Xdq, Xds, W13q_h, W13s_h, W2q_h, W2s_h, rows=all_rows, with_hu=True)
    del Xdq, Xds
    aidx = torch.from_numpy(all_rows).to(dev())
    Aq, As = b.Aq[aidx].cpu().numpy(), b.As[aidx].cpu().numpy()
    delta = validate_a_codes("[mx kimi] a", Aq, As, r["A"], r["Aq"], r["As"], r["HU"], r["HUabs"])
    allow = near_tie_allowance(delta, all_rows, s.seg_off, W2q_h, W2s_h)
    n = len(rows)
    # Y where the forward writes it; a row of a token with one local route
    # goes straight to that token's output, times its weight
    single, g, wt = single_route_terms(h["routes"], h["w"], L, 0, s.phi, rows)
    if (~single).any():
        assert_rows_allow("[mx kimi] Y", f64(b.Y[torch.from_numpy(rows[~single]).to(dev())]), r["Y"][:n][~single],
                          allow[:n][~single], TOL, rows[~single])
    if single.any():
        got = f64(b.out.view(-1, H)[torch.from_numpy(g[single]).to(dev())])
        assert_rows_allow("[mx kimi] out of one-route rows", got, wt[single, None] * r["Y"][:n][single],
                          allow[:n][single] * np.abs(wt[single]), TOL, rows[single])
    # out of the sampled tokens: the oracle's combine of its rows
    yidx = np.zeros(s.npad, np.int64)
    yidx[tok_rows] = np.arange(n, len(all_rows))
    out_ref = oracle.combine(s.route_row, h["w"], r["Y"], yidx, tokens=toks)
    tw = np.abs(np.where(rr >= 0, h["w"].reshape(-1, c["K"])[toks], 0.0)).sum(-1)
    assert_rows_allow("[mx kimi] out", f64(b.out.view(-1, H)[torch.from_numpy(toks).to(dev())]), out_ref,
                      allow[n:] * tw, TOL, toks)
