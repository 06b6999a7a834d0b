"""Full-size parity at the Kimi-shaped share (8 partitions x 7,168 tokens, 384
experts with 48 local, top-8, H=7168, I=2048), in the launch configuration the
benchmark times.

The schedule is compared whole (bit-exact); the dispatched rows, the expert
FFN rows and the combined tokens on samples the oracle computes one by one
(rows of four experts including the largest segment, 256 tokens), every
sampled row and token on its own; the adversarial forward and backward
(Zipf s=1.5 plus four hot local experts taking a quarter of all routes) on
sampled rows of a hot and a cold expert, sampled tokens, and four weight-
gradient elements in every 256 x 256 output tile of the hottest expert's dW13
and dW2 (one cold expert likewise).  Float tolerance: rel-L2 <= 1e-2 per row
against the fp64 oracle; the sampled weight-gradient elements within rel-L2
1e-2 together and each within 1e-2 of the sum of its terms' magnitudes.
"""
import numpy as np
import pytest
import torch

import oracle
from routing_schedule_expert_amd import inputs, ops
from tests.helpers import assert_elems, assert_rows, dev, f64, fused_y_rows, on_dev_mask, rel_l2, single_route_terms

pytestmark = pytest.mark.gpu
TOL = 1e-2
C = dict(P=8, Np=7168, E=384, K=8, L=48, H=7168, I=2048)


def host_bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def int_checksum(t):
    return int(t.contiguous().view(torch.int16).to(torch.int64).sum().item()), \
        int((t.contiguous().view(torch.int16).to(torch.int64) * torch.arange(
            t.numel(), device=t.device, dtype=torch.int64).remainder(65521).view(t.shape)).sum().item())


class Kimi:
    def __init__(self, routing, seed, grad=False):
        c = C
        self.h = inputs.make_layer_inputs_device(seed, c["P"], c["Np"], c["E"], c["K"], c["L"], c["H"], c["I"],
                                                 dev(), routing=routing, x_std=1.0, s=1.5, with_grad=grad)
        self.d = ops.make_desc(c["P"], c["Np"], c["K"], c["E"], c["L"], H=c["H"], I=c["I"])
        self.routes = torch.from_numpy(self.h["routes"]).to(dev())
        self.w = torch.from_numpy(self.h["w"]).to(dev())

    def fwd(self, flags=0, save_xd=True):
        b = ops.alloc_fwd(self.d, dev(), save_hu=True, save_xd=save_xd)
        ops.layer_fwd(self.d, self.routes, self.w, self.h["X"], self.h["W13"], self.h["W2"], b, flags=flags)
        torch.cuda.synchronize()
        return b


@pytest.fixture(scope="module")
def kimi_fwd():
    print("[kimi] forward, balanced routing", flush=True)
    k = Kimi("balanced", 5)
    b = k.fwd()
    return k, b


def check_routed_rows(label, k, b, s, rows, ref):
    """HU and A of sampled table rows vs the oracle; Y where the forward
    writes it, and for rows of tokens with one local route (whose Y row goes
    straight to the output) the token's output against w times the oracle's
    row."""
    ridx = torch.from_numpy(rows).to(dev())
    for name, t in (("HU", b.HU), ("A", b.A)):
        assert_rows(f"{label} {name}", f64(t[ridx]), ref[name], TOL, rows)
    single, g, wt = single_route_terms(k.h["routes"], k.h["w"], C["L"], 0, s.phi, rows)
    if (~single).any():
        sel = rows[~single]
        assert_rows(f"{label} Y", f64(b.Y[torch.from_numpy(sel).to(dev())]), ref["Y"][~single], TOL, sel)
    if single.any():
        got = f64(b.out.view(-1, C["H"])[torch.from_numpy(g[single]).to(dev())])
        assert_rows(f"{label} out of one-route rows", got, wt[single, None] * ref["Y"][single], TOL, rows[single])


def test_kimi_schedule_bit_exact(kimi_fwd):
    k, b = kimi_fwd
    s = oracle.schedule(k.h["routes"], C["L"], 0, 256)
    np.testing.assert_array_equal(b.counts.cpu().numpy(), s.counts)
    np.testing.assert_array_equal(b.seg_off.cpu().numpy(), s.seg_off)
    np.testing.assert_array_equal(b.phi[: s.npad].cpu().numpy(), s.phi)
    np.testing.assert_array_equal(b.route_row.cpu().numpy(), s.route_row)
    assert s.npad == 61440


def test_kimi_forward_sampled(kimi_fwd):
    k, b = kimi_fwd
    s = oracle.schedule(k.h["routes"], C["L"], 0, 256)
    X = host_bits(k.h["X"])
    rng = np.random.default_rng(3)
    # dispatched rows: bit copies (sampled over the whole table, padding included)
    rows = np.sort(rng.choice(s.npad, 1024, replace=False))
    Xd_rows = host_bits(b.Xd[torch.from_numpy(rows).to(dev())])
    Xd_ref = oracle.dispatch(X, s.phi)[rows]
    np.testing.assert_array_equal(Xd_rows, Xd_ref)
    # expert rows of four experts, including the largest segment
    seg = np.diff(s.seg_off)
    experts = sorted({int(np.argmax(seg)), 0, 17, 47})
    W13 = host_bits(k.h["W13"])
    W2 = host_bits(k.h["W2"])
    Xd = oracle.dispatch(X, s.phi)
    sample = []
    for l in experts:
        real = np.arange(s.seg_off[l], s.seg_off[l + 1])
        real = real[s.phi[real, 0] >= 0]
        sample.append(rng.choice(real, 48, replace=False))
    rows = np.sort(np.concatenate(sample))
    ref = oracle.expert_ffn_rows(s.seg_off, Xd, W13, W2, rows=rows)
    check_routed_rows("[kimi]", k, b, s, rows, ref)
    # combined tokens
    toks = np.sort(rng.choice(C["P"] * C["Np"], 256, replace=False))
    out_ref = oracle.layer_fwd_tokens(k.h["routes"], k.h["w"], X, W13, W2, L=C["L"], tokens=toks)
    got = f64(b.out.view(-1, C["H"])[torch.from_numpy(toks).to(dev())])
    assert_rows("[kimi] out", got, out_ref, TOL, toks)


def test_kimi_forward_repeatable_and_persistent_agrees(kimi_fwd):
    k, b = kimi_fwd
    npad = int(b.seg_off[-1])
    s = oracle.schedule(k.h["routes"], C["L"], 0, 256)
    yw = on_dev_mask(fused_y_rows(k.h["routes"], C["L"], 0, s.phi))  # the Y rows the fused forward writes
    ref = (int_checksum(b.out), int_checksum(b.Y[:npad][yw]))
    for flags, save_xd in ((0, True), (ops.MOE_PERSISTENT, True), (0, False)):
        b2 = k.fwd(flags=flags, save_xd=save_xd)
        assert (int_checksum(b2.out), int_checksum(b2.Y[:npad][yw])) == ref, (flags, save_xd)
        assert torch.equal(b.out, b2.out)
        del b2


def test_kimi_adversarial_forward_backward():
    print("[kimi] forward + backward, Zipf 1.5 + 4 hot experts", flush=True)
    k = Kimi("hot", 6, grad=True)
    b = k.fwd()
    c = C
    s = oracle.schedule(k.h["routes"], c["L"], 0, 256)
    np.testing.assert_array_equal(b.phi[: s.npad].cpu().numpy(), s.phi)
    np.testing.assert_array_equal(b.route_row.cpu().numpy(), s.route_row)
    seg = np.diff(s.seg_off)
    hot = int(np.argmax(seg))
    assert seg[hot] >= 28672
    d = k.d
    L, H, I = c["L"], c["H"], c["I"]

    def bwd():
        g = {"dX": torch.empty_like(k.h["X"]),
             "dW13": torch.empty((L, 2 * I, H), dtype=torch.float32, device=dev()),
             "dW2": torch.empty((L, H, I), dtype=torch.float32, device=dev()),
             "dw": torch.empty((c["P"], c["Np"], c["K"]), dtype=torch.float32, device=dev())}
        ws = torch.empty(ops.workspace_bytes(d, ops.MOE_OP_LAYER_BWD), dtype=torch.uint8, device=dev())
        ops.moe_layer_bwd(d, k.h["dOut"], k.routes, k.w, b.phi, b.route_row, b.seg_off, b.Xd, b.HU, b.A,
                          k.h["W13"], k.h["W2"], g["dX"], g["dW13"], g["dW2"], g["dw"], ws)
        torch.cuda.synchronize()
        return g

    X, W13, W2, dOut = (host_bits(k.h[n]) for n in ("X", "W13", "W2", "dOut"))
    rng = np.random.default_rng(4)
    cold = int(np.argsort(seg)[len(seg) // 2])
    # the adversarial forward: rows of the hottest and a middle expert, tokens
    Xd = oracle.dispatch(X, s.phi)
    sample = []
    for l in (hot, cold):
        real = np.arange(s.seg_off[l], s.seg_off[l + 1])
        real = real[s.phi[real, 0] >= 0]
        sample.append(rng.choice(real, min(48, real.size), replace=False))
    rows = np.sort(np.concatenate(sample))
    ref = oracle.expert_ffn_rows(s.seg_off, Xd, W13, W2, rows=rows)
    check_routed_rows("[kimi adv]", k, b, s, rows, ref)
    del Xd
    toks = np.sort(rng.choice(c["P"] * c["Np"], 128, replace=False))
    out_ref = oracle.layer_fwd_tokens(k.h["routes"], k.h["w"], X, W13, W2, L=L, tokens=toks)
    assert_rows("[kimi adv] out", f64(b.out.view(-1, H)[torch.from_numpy(toks).to(dev())]), out_ref, TOL, toks)

    g = bwd()
    toks = np.sort(rng.choice(c["P"] * c["Np"], 48, replace=False))
    dX_ref, dw_ref = oracle.bwd_tokens(k.h["routes"], k.h["w"], X, W13, W2, dOut, L, 0, toks)
    tidx = torch.from_numpy(toks).to(dev())
    assert_rows("[kimi] dX", f64(g["dX"].view(-1, H)[tidx]), dX_ref, TOL, toks)
    rt = k.h["routes"].reshape(-1, c["K"])[toks]
    loc = (rt >= 0) & (rt < L)
    assert_elems("[kimi] dw", f64(g["dw"].view(-1, c["K"])[tidx])[loc], dw_ref[loc], TOL)
    assert not f64(g["dw"].view(-1, c["K"])[tidx])[~loc].any()
    # weight gradients: four elements in every 256 x 256 output tile.  All
    # tiles of one 256-row band share the band's gate/up column n (dW13 gate
    # band t and up band t + I/256 use the same n, and so does dW2's column
    # band t), so the oracle computes each route's column quantities once.
    for l in (hot, cold):
        noff = rng.integers(0, 256, size=I // 256)
        cols = [256 * t + int(noff[t]) for t in range(I // 256)]
        e13 = [(band * 256 + (cols[band % (I // 256)] % 256), 256 * tc + int(rng.integers(0, 256)))
               for band in range(2 * I // 256) for tc in range(H // 256) for _ in range(4)]
        e2 = [(256 * tr + int(rng.integers(0, 256)), cols[tc]) for tr in range(H // 256) for tc in range(I // 256)
              for _ in range(4)]
        r13, r2, a13, a2 = oracle.wgrad_elems(k.h["routes"], k.h["w"], X, W13, W2, dOut, L, 0, l, e13, e2,
                                              with_abs=True)
        i13 = torch.tensor(e13, device=dev())
        i2 = torch.tensor(e2, device=dev())
        g13 = g["dW13"][l][i13[:, 0], i13[:, 1]].double().cpu().numpy()
        g2 = g["dW2"][l][i2[:, 0], i2[:, 1]].double().cpu().numpy()
        print(f"[kimi] expert {l} ({seg[l]} rows): {len(e13)} dW13 and {len(e2)} dW2 elements", flush=True)
        # rel-L2 over the sampled elements, and every element within 1e-2 of
        # the sum of its terms' magnitudes: the GPU's terms carry a few bf16
        # roundings (saved h and u, dHU, dO_d w, a), each at most 2^-9
        # relative, so a wrong tile fails by far while cancellation in a
        # single element's sum does not
        for name, got, ref, ab in (("dW13", g13, r13, a13), ("dW2", g2, r2, a2)):
            err = rel_l2(got, ref)
            worst = float(np.max(np.abs(got - ref) / ab))
            print(f"    [kimi] {name} expert {l}: rel-L2 {err:.2e}, worst |err| / sum|terms| {worst:.2e}", flush=True)
            assert err <= TOL and worst <= TOL, (name, l)
    g2nd = bwd()
    for n in ("dX", "dW13", "dW2", "dw"):
        assert torch.equal(g[n], g2nd[n]), f"{n} differs between repeated runs"
