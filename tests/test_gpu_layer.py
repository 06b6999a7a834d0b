"""GPU forward/backward of the layer share vs the CPU oracle.

Integer and copy outputs (schedule, dispatched rows) must match bit for bit;
float outputs must be within rel-L2 1e-2 of the fp64 oracle (over real rows
and tokens); the persistent, chunked and multi-launch forward paths must agree
bitwise; repeated runs must be bitwise identical.
"""
import numpy as np
import pytest
import torch

import oracle
from routing_schedule_expert_amd import inputs, ops
from tests.helpers import bits, digest, dev, f64, rel_l2, up, up_bf16

pytestmark = pytest.mark.gpu
TOL = 1e-2


class Layer:
    """Inputs on host (bit patterns) and device, plus the forward buffers."""

    def __init__(self, seed, P, Np, E, K, L, H, I, routing="uniform", base=0, x_std=1.0, s=1.2, grad=True):
        self.h = inputs.make_layer_inputs(seed, P, Np, E, K, L, H, I, routing=routing, base=base, x_std=x_std,
                                          s=s, with_grad=grad)
        self.P, self.Np, self.E, self.K, self.L, self.H, self.I, self.base = P, Np, E, K, L, H, I, base
        self.d = ops.make_desc(P, Np, K, E, L, expert_base=base, H=H, I=I)
        self.routes = up(self.h["routes"])
        self.w = up(self.h["w"])
        self.X = up_bf16(self.h["X"])
        self.W13 = up_bf16(self.h["W13"])
        self.W2 = up_bf16(self.h["W2"])
        self.dOut = up_bf16(self.h["dOut"]) if grad else None

    def fwd(self, flags=0, chunk_rows=0, save_hu=True, save_xd=True):
        b = ops.alloc_fwd(self.d, dev(), save_hu=save_hu, save_xd=save_xd)
        ops.layer_fwd(self.d, self.routes, self.w, self.X, self.W13, self.W2, b, flags=flags, chunk_rows=chunk_rows)
        torch.cuda.synchronize()
        return b

    def bwd(self, b):
        d, L, H, I = self.d, self.L, self.H, self.I
        g = {
            "dX": torch.empty_like(self.X),
            "dW13": torch.empty((L, 2 * I, H), dtype=torch.float32, device=dev()),
            "dW2": torch.empty((L, H, I), dtype=torch.float32, device=dev()),
            "dw": torch.empty((self.P, self.Np, self.K), dtype=torch.float32, device=dev()),
        }
        ws = torch.empty(ops.workspace_bytes(d, ops.MOE_OP_LAYER_BWD), dtype=torch.uint8, device=dev())
        ops.moe_layer_bwd(d, self.dOut, self.routes, self.w, b.phi, b.route_row, b.seg_off, b.Xd, b.HU, b.A,
                          self.W13, self.W2, g["dX"], g["dW13"], g["dW2"], g["dw"], ws)
        torch.cuda.synchronize()
        return g

    def oracle_schedule(self):
        return oracle.schedule(self.h["routes"], self.L, self.base, 256)


def check_fwd_full(lay: Layer, b: ops.FwdBuffers):
    h = lay.h
    s = lay.oracle_schedule()
    np.testing.assert_array_equal(b.counts.cpu().numpy(), s.counts)
    np.testing.assert_array_equal(b.seg_off.cpu().numpy(), s.seg_off)
    np.testing.assert_array_equal(b.phi[: s.npad].cpu().numpy(), s.phi)
    np.testing.assert_array_equal(b.route_row.cpu().numpy(), s.route_row)
    Xd = oracle.dispatch(h["X"], s.phi)
    np.testing.assert_array_equal(bits(b.Xd[: s.npad]), Xd)
    r = oracle.expert_ffn_rows(s.seg_off, Xd, h["W13"], h["W2"])
    real = s.phi[:, 0] >= 0
    assert rel_l2(f64(b.HU[: s.npad])[real], r["HU"][real]) <= TOL
    assert rel_l2(f64(b.A[: s.npad])[real], r["A"][real]) <= TOL
    assert rel_l2(f64(b.Y[: s.npad])[real], r["Y"][real]) <= TOL
    # padding rows are exactly zero in every row output
    for t in (b.HU, b.A, b.Y):
        assert not f64(t[: s.npad])[~real].any()
    out = oracle.layer_fwd_tokens(h["routes"], h["w"], h["X"], h["W13"], h["W2"], L=lay.L, base=lay.base)
    got = f64(b.out).reshape(out.shape)
    assert rel_l2(got, out) <= TOL
    # tokens with no local slot are exactly zero
    none_local = ~((h["routes"] >= lay.base) & (h["routes"] < lay.base + lay.L)).any(-1).reshape(-1)
    assert not got[none_local].any()


@pytest.mark.parametrize("L,E", [(4, 8), (8, 8)])
def test_tiny_forward(L, E):
    print(f"[layer] tiny forward L={L}", flush=True)
    lay = Layer(1, 2, 256, E, 2, L, 256, 128, routing="topk", x_std=0.02)
    check_fwd_full(lay, lay.fwd())


def test_small_forward_multi_tile():
    print("[layer] small forward, several tiles and ragged segments", flush=True)
    lay = Layer(3, 4, 700, 12, 3, 6, 512, 256, routing="zipf", s=1.2)
    check_fwd_full(lay, lay.fwd())


def test_forward_paths_agree_bitwise():
    lay = Layer(4, 4, 900, 16, 4, 8, 512, 384, routing="uniform")
    ref = lay.fwd()
    outs = [ref]
    for flags, chunk in ((ops.MOE_PERSISTENT, 0), (0, 256), (ops.MOE_PERSISTENT, 512), (0, 1024)):
        print(f"[layer] forward flags={flags} chunk_rows={chunk}", flush=True)
        outs.append(lay.fwd(flags=flags, chunk_rows=chunk))
    npad = int(ref.seg_off[-1])
    for b in outs[1:]:
        assert digest(b.out) == digest(ref.out)
        assert digest(b.Y[:npad], b.A[:npad], b.HU[:npad]) == digest(ref.Y[:npad], ref.A[:npad], ref.HU[:npad])
        assert digest(b.phi[:npad], b.route_row, b.seg_off) == digest(ref.phi[:npad], ref.route_row, ref.seg_off)


def test_forward_fused_dispatch_bitwise():
    """Xd = NULL: the gate/up GEMM pulls its rows from X through phi; every
    output must be bitwise the one of the materialised dispatch, on the
    multi-launch, persistent and chunked paths."""
    lay = Layer(9, 4, 900, 16, 4, 8, 512, 384, routing="zipf", s=1.2)
    ref = lay.fwd()
    npad = int(ref.seg_off[-1])
    for flags, chunk in ((0, 0), (ops.MOE_PERSISTENT, 0), (0, 512), (ops.MOE_PERSISTENT, 256)):
        print(f"[layer] fused dispatch flags={flags} chunk_rows={chunk}", flush=True)
        b = lay.fwd(flags=flags, chunk_rows=chunk, save_xd=False)
        assert b.Xd is None
        assert digest(b.out) == digest(ref.out)
        assert digest(b.Y[:npad], b.A[:npad], b.HU[:npad]) == digest(ref.Y[:npad], ref.A[:npad], ref.HU[:npad])
        assert digest(b.phi[:npad], b.route_row, b.seg_off) == digest(ref.phi[:npad], ref.route_row, ref.seg_off)


def test_fused_dispatch_vs_oracle():
    lay = Layer(10, 2, 256, 8, 2, 4, 256, 128, routing="topk", x_std=0.02)
    b = lay.fwd(save_xd=False)
    h = lay.h
    s = lay.oracle_schedule()
    np.testing.assert_array_equal(b.phi[: s.npad].cpu().numpy(), s.phi)
    r = oracle.expert_ffn_rows(s.seg_off, oracle.dispatch(h["X"], s.phi), h["W13"], h["W2"])
    real = s.phi[:, 0] >= 0
    assert rel_l2(f64(b.A[: s.npad])[real], r["A"][real]) <= TOL
    assert not f64(b.Y[: s.npad])[~real].any()  # padding rows read the zero row
    out = oracle.layer_fwd_tokens(h["routes"], h["w"], h["X"], h["W13"], h["W2"], L=lay.L)
    assert rel_l2(f64(b.out).reshape(out.shape), out) <= TOL


def test_fused_dispatch_widest_rows():
    """H = 32768, the widest row the fused dispatch supports (padding rows
    read a static zero row of that many elements): bitwise the materialised
    path, padding rows zero, output vs the oracle."""
    print("[layer] fused dispatch, H = 32768", flush=True)
    lay = Layer(14, 2, 64, 8, 2, 4, 32768, 128, routing="topk", x_std=0.02, grad=False)
    a = lay.fwd(save_xd=True)
    b = lay.fwd(save_xd=False)
    s = lay.oracle_schedule()
    assert torch.equal(a.out, b.out)
    assert torch.equal(a.Y[: s.npad], b.Y[: s.npad])
    real = s.phi[:, 0] >= 0
    assert (~real).any() and not f64(b.Y[: s.npad])[~real].any()
    h = lay.h
    out = oracle.layer_fwd_tokens(h["routes"], h["w"], h["X"], h["W13"], h["W2"], L=lay.L)
    err = rel_l2(f64(b.out).reshape(out.shape), out)
    print(f"[layer] H=32768 out rel-L2 {err:.2e}", flush=True)
    assert err <= TOL


def test_forward_without_saved_hu():
    lay = Layer(5, 2, 300, 8, 2, 4, 256, 128)
    a = lay.fwd(save_hu=True)
    b = lay.fwd(save_hu=False)
    assert digest(a.out) == digest(b.out)


def test_no_local_routes():
    lay = Layer(6, 2, 128, 8, 2, 4, 256, 128, base=4)
    lay.h["routes"][:] = np.where(lay.h["routes"] >= 4, lay.h["routes"] - 4, lay.h["routes"])
    lay.routes = up(lay.h["routes"])
    b = lay.fwd()
    assert int(b.seg_off[-1]) == 0
    assert not f64(b.out).any()


def check_bwd_full(lay: Layer, g):
    h = lay.h
    ref = oracle.layer_bwd(h["routes"], h["w"], h["X"], h["W13"], h["W2"], h["dOut"], L=lay.L, base=lay.base)
    for name in ("dX", "dW13", "dW2", "dw"):
        got = f64(g[name]).reshape(ref[name].shape)
        err = rel_l2(got, ref[name])
        print(f"[layer] bwd {name} rel-L2 {err:.2e}", flush=True)
        assert err <= TOL, name
    local = (h["routes"] >= lay.base) & (h["routes"] < lay.base + lay.L)
    assert not f64(g["dw"])[~local].any()


def test_tiny_backward():
    print("[layer] tiny backward", flush=True)
    lay = Layer(1, 2, 256, 8, 2, 4, 256, 128, routing="topk", x_std=1.0)
    check_bwd_full(lay, lay.bwd(lay.fwd()))


def test_small_backward_skewed():
    print("[layer] small backward, skewed routing", flush=True)
    lay = Layer(7, 4, 600, 16, 4, 8, 512, 256, routing="zipf", s=1.5)
    check_bwd_full(lay, lay.bwd(lay.fwd()))


def test_repeat_runs_bitwise_identical():
    lay = Layer(8, 4, 800, 16, 4, 8, 512, 256, routing="zipf", s=1.2)
    hashes = set()
    for _ in range(3):
        b = lay.fwd()
        g = lay.bwd(b)
        npad = int(b.seg_off[-1])
        hashes.add(digest(b.out, b.Y[:npad], g["dX"], g["dW13"], g["dW2"], g["dw"]))
    assert len(hashes) == 1


def test_mid_forward_sampled():
    """Mid configuration: 8 x 4096 tokens, 64 experts (8 local), top-6, H=2048, I=1024."""
    print("[layer] mid forward (sampled rows and tokens)", flush=True)
    c = inputs.CONFIGS["mid"]
    lay = Layer(4, c["P"], c["Np"], c["E"], c["K"], c["L"], c["H"], c["I"], routing="uniform", grad=False)
    b = lay.fwd()
    s = lay.oracle_schedule()
    np.testing.assert_array_equal(b.phi[: s.npad].cpu().numpy(), s.phi)
    np.testing.assert_array_equal(b.route_row.cpu().numpy(), s.route_row)
    Xd = oracle.dispatch(lay.h["X"], s.phi)
    np.testing.assert_array_equal(bits(b.Xd[: s.npad]), Xd)
    rng = np.random.default_rng(0)
    real = np.nonzero(s.phi[:, 0] >= 0)[0]
    rows = np.sort(rng.choice(real, 192, replace=False))
    r = oracle.expert_ffn_rows(s.seg_off, Xd, lay.h["W13"], lay.h["W2"], rows=rows)
    assert rel_l2(f64(b.A[rows]), r["A"]) <= TOL
    assert rel_l2(f64(b.Y[rows]), r["Y"]) <= TOL
    toks = np.sort(rng.choice(lay.P * lay.Np, 96, replace=False))
    out = oracle.layer_fwd_tokens(lay.h["routes"], lay.h["w"], lay.h["X"], lay.h["W13"], lay.h["W2"], L=lay.L,
                                  tokens=toks)
    assert rel_l2(f64(b.out).reshape(-1, lay.H)[toks], out) <= TOL


def test_random_shapes_forward_backward():
    """Seeded random shapes within the supported constraints (H a multiple of
    256, I of 128), routing kinds, expert bases and dropped slots: the full
    forward checks (tables bit-exact, rows and outputs vs the oracle, padding
    and non-local tokens exactly zero) and the full backward checks."""
    rng = np.random.default_rng(4242)
    for i in range(10):
        P = int(rng.integers(1, 5))
        Np = int(rng.integers(40, 500))
        E = int(rng.integers(4, 24))
        K = int(rng.integers(1, min(4, E) + 1))
        L = int(rng.integers(1, E + 1))
        base = int(rng.integers(0, E - L + 1))
        H = int(rng.choice([256, 512, 768]))
        I = int(rng.choice([128, 256, 384]))
        routing = str(rng.choice(["uniform", "zipf", "topk"]))
        drop = bool(rng.random() < 0.5)
        print(f"[layer] random {i}: P={P} Np={Np} E={E} K={K} L={L} base={base} H={H} I={I} {routing}"
              f"{' dropped slots' if drop else ''}", flush=True)
        lay = Layer(100 + i, P, Np, E, K, L, H, I, routing=routing, base=base, x_std=1.0)
        if drop:
            rt = lay.h["routes"].copy()
            rt[:, ::3, 0] = -1
            lay.h["routes"] = rt
            lay.routes = up(rt)
        b = lay.fwd()
        check_fwd_full(lay, b)
        check_bwd_full(lay, lay.bwd(b))
