"""Full-size parity at the Kimi-shaped share (8 partitions x 7,168 tokens, 384
experts with 48 local, top-8, H=7168, I=2048), in the launch configuration the
benchmark times.

The schedule is compared whole (bit-exact); the dispatched rows, the expert
FFN rows and the combined tokens on samples the oracle computes one by one
(rows of four experts including the largest segment, 256 tokens); the
backward (adversarial routing: Zipf s=1.5 plus four hot local experts taking a
quarter of all routes) on sampled tokens and weight-gradient elements of a hot
and a cold expert.  Float tolerance: rel-L2 <= 1e-2 against the fp64 oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from routing_schedule_expert_amd import inputs, ops
from tests.helpers import dev, f64, rel_l2

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
    ridx = torch.from_numpy(rows).to(dev())
    for name, t in (("HU", b.HU), ("A", b.A), ("Y", b.Y)):
        err = rel_l2(f64(t[ridx]), ref[name])
        print(f"[kimi] {name} rel-L2 {err:.2e}", flush=True)
        assert err <= TOL, name
    # combined tokens
    toks = np.sort(rng.choice(C["P"] * C["Np"], 256, replace=False))
    out_ref = oracle.layer_fwd_tokens(k.h["routes"], k.h["w"], X, W13, W2, L=C["L"], tokens=toks)
    got = f64(b.out.view(-1, C["H"])[torch.from_numpy(toks).to(dev())])
    err = rel_l2(got, out_ref)
    print(f"[kimi] out rel-L2 {err:.2e}", flush=True)
    assert err <= TOL


def test_kimi_forward_repeatable_and_persistent_agrees(kimi_fwd):
    k, b = kimi_fwd
    npad = int(b.seg_off[-1])
    ref = (int_checksum(b.out), int_checksum(b.Y[:npad]))
    for flags, save_xd in ((0, True), (ops.MOE_PERSISTENT, True), (0, False)):
        b2 = k.fwd(flags=flags, save_xd=save_xd)
        assert (int_checksum(b2.out), int_checksum(b2.Y[:npad])) == ref, (flags, save_xd)
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

    g = bwd()
    X, W13, W2, dOut = (host_bits(k.h[n]) for n in ("X", "W13", "W2", "dOut"))
    rng = np.random.default_rng(4)
    toks = np.sort(rng.choice(c["P"] * c["Np"], 48, replace=False))
    dX_ref, dw_ref = oracle.bwd_tokens(k.h["routes"], k.h["w"], X, W13, W2, dOut, L, 0, toks)
    tidx = torch.from_numpy(toks).to(dev())
    err = rel_l2(f64(g["dX"].view(-1, H)[tidx]), dX_ref)
    print(f"[kimi] dX rel-L2 {err:.2e}", flush=True)
    assert err <= TOL
    err = rel_l2(f64(g["dw"].view(-1, c["K"])[tidx]), dw_ref)
    print(f"[kimi] dw rel-L2 {err:.2e}", flush=True)
    assert err <= TOL
    cold = int(np.argsort(seg)[len(seg) // 2])
    for l in (hot, cold):
        e13 = [(int(rng.integers(0, 2 * I)), int(rng.integers(0, H))) for _ in range(6)]
        e2 = [(int(rng.integers(0, H)), int(rng.integers(0, I))) for _ in range(6)]
        r13, r2 = oracle.wgrad_elems(k.h["routes"], k.h["w"], X, W13, W2, dOut, L, 0, l, e13, e2)
        g13 = np.array([g["dW13"][l, n, kk].item() for n, kk in e13])
        g2 = np.array([g["dW2"][l, m, n].item() for m, n in e2])
        e1, e2_ = rel_l2(g13, r13), rel_l2(g2, r2)
        print(f"[kimi] expert {l} (rows {seg[l]}): dW13 rel-L2 {e1:.2e}, dW2 rel-L2 {e2_:.2e}", flush=True)
        assert e1 <= TOL and e2_ <= TOL
    g2nd = bwd()
    for n in ("dX", "dW13", "dW2", "dw"):
        assert torch.equal(g[n], g2nd[n]), f"{n} differs between repeated runs"
