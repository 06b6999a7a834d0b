"""MXFP8 backward on the GPU vs the CPU oracle (reading: every backward product
on MX operands blocked along its own reduction dimension; "Beyond Peak TFLOPs"
section 3 and the Mixture-of-Kittens notes section 6 report the MXFP8
backward).

Column quantizations of bf16 inputs (the backward's weights) are fixed
functions of the input and must match the oracle bit for bit.  The oracle
computes its own forward (h, u, a) and backward from the bf16 inputs alone;
the GPU runs moe_layer_fwd_mx (saving h, u and the codes of a) and then
moe_layer_bwd_mx.  Both quantize the same numbers wherever the operand is a
bf16 input or a bf16 intermediate that both round the same way (Xd and w dO_d
columns: compared bit for bit); codes that depend on an fp32-vs-fp64
accumulation upstream (a, and dHU through the saved bf16 h and u) may differ
by one step, and one step on a large element moves a whole dX row by a few
percent.  So every differing code is checked to lie within one step of the
exact value (at most 1% of them may differ), its exact effect is added to
the oracle's result, and then: every token's dX and every row of dW13 / dW2
within rel-L2 1e-2; every dw and every weight-gradient element within 1e-2
of the sum of its terms' magnitudes; saved h, u and dHU rows within rel-L2
1e-2; tokens without a local route, non-local slots and empty experts
exactly 0; repeated runs bitwise equal.
"""
import numpy as np
import pytest
import torch

import oracle
from routing_schedule_expert_amd import inputs, ops
from tests.helpers import assert_rows, bits, dev, f64, up, up_bf16
from tests.test_gpu_mx import validate_a_codes

pytestmark = pytest.mark.gpu
TOL = 1e-2


def hot_empty(h, base, E):
    """Local expert 1 takes every token's first slot (a segment of several
    256-row tiles); local expert 2 gets no route."""
    r = h["routes"].copy()
    r[r == base + 2] = E - 1
    r[:, :, 0] = base + 1
    h["routes"] = r
    return h


CASES = {
    # H = 256 and 2I = 256: 4-byte scale DMAs; I = 128: a half-width last dgrad tile
    "small_i128": dict(seed=11, P=2, Np=300, E=8, K=2, L=4, H=256, I=128),
    # 16-byte scale DMAs (H, 2I multiples of 512), a nonzero expert base, an
    # empty expert and one of three 256-row tiles
    "hot_empty_base": dict(seed=12, P=2, Np=400, E=16, K=3, L=6, H=512, I=256, base=5, hot=True),
    # I % 256 = 128 with 2I = 768 (4-byte scale DMAs in the gate/up dgrad), top-1
    "k1_i384": dict(seed=13, P=1, Np=700, E=4, K=1, L=4, H=256, I=384),
    # 512 weight-gradient tiles, so every workgroup of the launch takes two:
    # a tile that issues the next one's first stage before its stores, next
    # tiles of the other weight, with a half-width column (I % 256 = 128) or
    # with no rows (an empty expert), and the reverse-dispatch items after them
    "multi_tile": dict(seed=14, P=2, Np=512, E=16, K=2, L=8, H=2048, I=640, hot=True),
}


class MxBwdCase:
    def __init__(self, seed, P, Np, E, K, L, H, I, base=0, hot=False, routing="uniform"):
        h = inputs.make_layer_inputs(seed, P, Np, E, K, L, H, I, routing=routing, base=base, x_std=1.0,
                                     w_std=0.05, with_grad=True)
        self.h = hot_empty(h, base, E) if hot else h
        self.P, self.Np, self.K, self.L, self.H, self.I, self.base = P, Np, K, L, H, I, base
        self.d = ops.make_desc(P, Np, K, E, L, expert_base=base, H=H, I=I)
        self.routes, self.w = up(self.h["routes"]), up(self.h["w"])
        self.X = up_bf16(self.h["X"])
        self.dOut = up_bf16(self.h["dOut"])
        W13, W2 = up_bf16(self.h["W13"]), up_bf16(self.h["W2"])
        self.W13q, self.W13s = ops.quantize_mx(W13)
        self.W2q, self.W2s = ops.quantize_mx(W2)
        self.W13t = ops.quantize_mx_t(W13)
        self.W2t = ops.quantize_mx_t(W2)

    def run(self):
        b = ops.alloc_fwd_mx(self.d, dev(), save_hu=True)
        ops.layer_fwd_mx(self.d, self.routes, self.w, self.X, self.W13q, self.W13s, self.W2q, self.W2s, b)
        g = ops.alloc_bwd_mx(self.d, dev())
        ops.layer_bwd_mx(self.d, self.dOut, self.w, self.X, b, self.W13t, self.W2t, g)
        torch.cuda.synchronize()
        return b, g


def deq(qs):
    return oracle.mx_dequantize(np.asarray(qs[0]), np.asarray(qs[1]))


E4M3_MAX = 448.0


def e4m3_step(y):
    """Spacing of E4M3 values at |y| (scaled domain): 2^(e - 3) for a normal
    binade [2^e, 2^(e+1)), e >= -6; 2^-9 among the subnormals."""
    e = np.frexp(np.abs(y))[1] - 1
    return np.ldexp(1.0, np.maximum(e, -6) - 3)


def check_mx_of(name, g, vals):
    """g = (codes, scales) must be exactly the MX quantization of vals (blocks
    of 32 along the last axis), from the format's closed form: scale byte
    floor(log2 amax) - 8 + 127 (0 for an all-zero block), codes x / scale
    rounded to the nearest E4M3 value, ties to even, saturated at 448."""
    vals = np.asarray(vals, np.float64)
    blk = vals.reshape(vals.shape[:-1] + (-1, 32))
    amax = np.abs(blk).max(-1)
    sb = np.where(amax > 0, np.clip(np.frexp(amax)[1] - 1 - 8, -127, 127) + 127, 0)
    np.testing.assert_array_equal(np.asarray(g[1], np.int64), sb, err_msg=f"{name}: scale bytes")
    y = blk * np.ldexp(1.0, 127 - sb)[..., None]
    st = e4m3_step(y)
    want = np.sign(y) * np.minimum(np.round(np.abs(y) / st) * st, E4M3_MAX)  # numpy rounds half to even
    got = oracle.e4m3_table()[np.asarray(g[0], np.int64)].reshape(y.shape)
    bad = got != want
    assert not bad.any(), f"{name}: {int(bad.sum())} codes are not the MX quantization of their input"


def code_diff(name, g, r):
    """Value difference (GPU - oracle) of two MX encodings, at most 1% of
    whose codes may differ."""
    gv, rv = deq(g), deq(r)
    diff = gv != rv
    n = int(diff.sum())
    if n:
        print(f"    {name}: {n} of {diff.size} codes differ from the oracle's", flush=True)
        assert n <= 0.01 * diff.size, f"{name}: {n} codes differ"
    return np.where(diff, gv - rv, 0.0)


def check_expert(c, l, sg, g, b, v):
    """One expert segment: the saved h, u, dHU and its codes, the a codes, the
    weight gradients' column codes, and every row and element of dW13[l] and
    dW2[l] after adding the exact effect of the differing column codes."""
    r0, r1 = int(sg["rows"][0]), int(sg["rows"][-1]) + 1
    real = b.phi[r0:r1, 0].cpu().numpy() >= 0
    ids = sg["rows"][real]
    assert_rows(f"[mx bwd] saved HU[{l}]", f64(b.HU[r0:r1])[real], sg["HU"][real], TOL, ids)
    dHU_g = f64(v["dHU"][r0:r1])
    assert_rows(f"[mx bwd] dHU[{l}]", dHU_g[real], sg["dHU"][real], TOL, ids)
    # the forward's a: its fp32 value is not kept, so every code that differs
    # from the oracle's must be explained by an accumulation error in h and u
    # (the MX forward test's validator)
    a_g = (b.Aq[r0:r1].cpu().numpy(), b.As[r0:r1].cpu().numpy())
    a_eff = np.zeros_like(sg["a"])
    a_eff[real] = validate_a_codes(f"[mx bwd] a[{l}]", a_g[0][real], a_g[1][real], sg["a_exact"][real],
                                   sg["Aq"][real], sg["As"][real], sg["HU"][real], sg["HUabs"][real])
    assert not deq(a_g)[~real].any()
    code_diff(f"[mx bwd] a[{l}]", a_g, (sg["Aq"], sg["As"]))  # at most 1% differ
    # every other code must be exactly the MX quantization of the GPU's own
    # input, which is itself within rel-L2 1e-2 of the oracle's
    dhu_g = (v["DHU"][0][r0:r1].cpu().numpy(), v["DHU"][1][r0:r1].cpu().numpy())
    check_mx_of(f"[mx bwd] dHU codes[{l}]", dhu_g, dHU_g)
    dhu_eff = code_diff(f"[mx bwd] dHU codes[{l}]", dhu_g, (sg["dHUq"], sg["dHUs"]))

    def col(t):
        q, sc = ops.mx_expert_block(t, r0, r1 - r0)
        return q.cpu().numpy(), sc.cpu().numpy()

    for nm in ("XdT", "dOwT"):  # column codes of bf16 values both sides hold: bit for bit
        gq, gs = col(v[nm.upper()])
        np.testing.assert_array_equal(gq, sg[nm][0], err_msg=f"{nm}[{l}]")
        np.testing.assert_array_equal(gs, sg[nm][1], err_msg=f"{nm}[{l}]")
    aT_g, dhuT_g = col(v["AT"]), col(v["DHUT"])
    check_mx_of(f"[mx bwd] a column codes[{l}]", aT_g, deq(a_g).T)
    check_mx_of(f"[mx bwd] dHU column codes[{l}]", dhuT_g, dHU_g.T)
    aT_eff = code_diff(f"[mx bwd] a column codes[{l}]", aT_g, sg["aT"])
    dhuT_eff = code_diff(f"[mx bwd] dHU column codes[{l}]", dhuT_g, sg["dHUT"])
    XdT, dOwT = deq(sg["XdT"]), deq(sg["dOwT"])
    for nm, got, ref, eff, ab in (
            ("dW13", f64(g.dW13[l]), sg["dW13"], dhuT_eff @ XdT.T, np.abs(deq(sg["dHUT"])) @ np.abs(XdT).T),
            ("dW2", f64(g.dW2[l]), sg["dW2"], dOwT @ aT_eff.T, np.abs(dOwT) @ np.abs(deq(sg["aT"])).T)):
        assert_rows(f"[mx bwd] {nm}[{l}] ({r1 - r0} rows, plus code effects)", got, ref + eff, TOL)
        worst = float(np.max(np.abs(got - ref - eff) / np.maximum(ab, 1e-30)))
        assert worst <= TOL, (nm, l, worst)
    return a_eff, dhu_eff


def check_tokens(c, r, effects, g, toks):
    """dX and dw of the listed tokens (all their local routes in computed
    experts) after adding the exact effect of the GPU's differing a and dHU
    codes on each of their rows."""
    s = r["sched"]
    K, H = c.K, c.H
    rr = s.route_row.reshape(-1, K)[toks]
    dX_ref = r["dX"][toks].copy()
    dw_ref = r["dw"][toks].copy()
    dwabs = np.zeros_like(dw_ref)
    for l, sg in r["seg"].items():
        a_eff, dhu_eff = effects[l]
        r0, r1 = int(sg["rows"][0]), int(sg["rows"][-1]) + 1
        q, j = np.nonzero((rr >= r0) & (rr < r1))
        k = rr[q, j] - r0
        np.add.at(dX_ref, q, dhu_eff[k] @ sg["W13t"].T)
        dw_ref[q, j] += (sg["dAp"][k] * a_eff[k]).sum(1)
        dwabs[q, j] = np.abs(sg["dAp"][k] * (sg["a"][k] + a_eff[k])).sum(1)
    tidx = torch.from_numpy(np.ascontiguousarray(toks)).to(dev())
    assert_rows("[mx bwd] dX (plus code effects)", f64(g.dX.view(-1, H)[tidx]), dX_ref, TOL, toks)
    loc = rr >= 0
    dw = f64(g.dw.view(-1, K)[tidx])
    worst = float(np.max(np.abs(dw[loc] - dw_ref[loc]) / np.maximum(dwabs[loc], 1e-30)))
    print(f"    [mx bwd] dw: {loc.sum()} slots, worst |err| / sum|terms| {worst:.2e}", flush=True)
    assert worst <= TOL and not dw[~loc].any()


@pytest.mark.parametrize("name", sorted(CASES))
def test_mx_bwd_small(name):
    print(f"[mx bwd] {name}: {CASES[name]}", flush=True)
    c = MxBwdCase(**CASES[name])
    h = c.h
    wt = oracle.mx_weights_t(h["W13"], h["W2"])
    # the backward's weights: bit-exact column quantization
    for nm, t in (("W13tq", c.W13t[0]), ("W13ts", c.W13t[1]), ("W2tq", c.W2t[0]), ("W2ts", c.W2t[1])):
        np.testing.assert_array_equal(t.cpu().numpy(), wt[nm], err_msg=nm)
    b, g = c.run()
    r = oracle.mx_layer_bwd(h["routes"], h["w"], h["X"], h["W13"], h["W2"], h["dOut"], c.L, c.base)
    s = r["sched"]
    np.testing.assert_array_equal(b.phi[: s.npad].cpu().numpy(), s.phi)
    v = ops.mx_bwd_views(c.d, g.ws)
    effects = {l: check_expert(c, l, sg, g, b, v) for l, sg in r["seg"].items()}
    for l in range(c.L):
        if l not in r["seg"]:  # an empty expert: zero weight gradients
            assert not g.dW13[l].any() and not g.dW2[l].any(), l
    rt = h["routes"].reshape(-1, c.K)
    has = ((rt >= c.base) & (rt < c.base + c.L)).any(1)
    check_tokens(c, r, effects, g, np.nonzero(has)[0])
    assert not f64(g.dX).reshape(-1, c.H)[~has].any()
    b2, g2nd = c.run()
    for n in ("dX", "dW13", "dW2", "dw"):
        assert torch.equal(getattr(g, n), getattr(g2nd, n)), f"{n} differs between repeated runs"


class HostWeights:
    """Host bf16 bits of the weights with only the listed experts copied from
    the device (the rest stay zero pages the oracle never reads)."""

    def __init__(self, W, experts):
        self.a = np.zeros(tuple(W.shape), np.uint16)
        for l in experts:
            self.a[l] = bits(W[l])


def test_mx_bwd_kimi():
    """The Kimi-shaped share (8 x 7,168 tokens, 384 experts with 48 local,
    top-8, H = 7168, I = 2048, balanced routing) in the benchmark's launch
    configuration: whole experts (the largest segment, the first and the last;
    under balanced routing the first is also the largest): every row of their
    dW13 and dW2, the dX and dw of every token routed to them, their backward
    weight codes bit for bit; a repeat bitwise."""
    P, Np, E, K, L, H, I = 8, 7168, 384, 8, 48, 7168, 2048

    class C:
        pass

    c = C()
    c.K, c.H, c.I = K, H, I
    print("[mx bwd kimi] inputs", flush=True)
    h = inputs.make_layer_inputs_device(21, P, Np, E, K, L, H, I, dev(), routing="balanced", x_std=1.0,
                                        with_grad=True)
    d = ops.make_desc(P, Np, K, E, L, H=H, I=I)
    routes, w = up(h["routes"]), up(h["w"])
    W13q, W13s = ops.quantize_mx(h["W13"])
    W2q, W2s = ops.quantize_mx(h["W2"])
    W13t, W2t = ops.quantize_mx_t(h["W13"]), ops.quantize_mx_t(h["W2"])

    def run():
        b = ops.alloc_fwd_mx(d, dev(), save_hu=True)
        ops.layer_fwd_mx(d, routes, w, h["X"], W13q, W13s, W2q, W2s, b)
        g = ops.alloc_bwd_mx(d, dev())
        ops.layer_bwd_mx(d, h["dOut"], w, h["X"], b, W13t, W2t, g)
        torch.cuda.synchronize()
        return b, g

    print("[mx bwd kimi] forward + backward", flush=True)
    b, g = run()
    s = oracle.schedule(h["routes"], L, 0, 256)
    seg = np.diff(s.seg_off)
    experts = sorted({int(np.argmax(seg)), 0, L - 1})
    W13h, W2h = HostWeights(h["W13"], experts).a, HostWeights(h["W2"], experts).a
    for l in experts:
        wq, ws_ = oracle.mx_transpose_quantize(W13h[l])
        np.testing.assert_array_equal(W13t[0][l].cpu().numpy(), wq, err_msg=f"W13tq[{l}]")
        np.testing.assert_array_equal(W13t[1][l].cpu().numpy(), ws_, err_msg=f"W13ts[{l}]")
        wq, ws_ = oracle.mx_transpose_quantize(W2h[l])
        np.testing.assert_array_equal(W2t[0][l].cpu().numpy(), wq, err_msg=f"W2tq[{l}]")
        np.testing.assert_array_equal(W2t[1][l].cpu().numpy(), ws_, err_msg=f"W2ts[{l}]")
    print(f"[mx bwd kimi] oracle for experts {experts} ({[int(seg[l]) for l in experts]} rows)", flush=True)
    r = oracle.mx_layer_bwd(h["routes"], h["w"], bits(h["X"]), W13h, W2h, bits(h["dOut"]), L, 0, experts=experts)
    np.testing.assert_array_equal(b.phi[: s.npad].cpu().numpy(), s.phi)
    v = ops.mx_bwd_views(d, g.ws)
    effects = {}
    for l in experts:
        print(f"[mx bwd kimi] expert {l}", flush=True)
        effects[l] = check_expert(c, l, r["seg"][l], g, b, v)
    rt = h["routes"].reshape(-1, K)
    loc = (rt >= 0) & (rt < L)
    assert (loc.sum(1) == 1).all()  # balanced: one local route per token
    toks = np.nonzero(np.isin(np.where(loc, rt, -1).max(1), experts))[0]
    check_tokens(c, r, effects, g, toks)
    del b, v
    b2, g2nd = run()
    for n in ("dX", "dW13", "dW2", "dw"):
        assert torch.equal(getattr(g, n), getattr(g2nd, n)), f"{n} differs between repeated runs"
