"""Macrobatch ring on the GPU ("Beyond Peak TFLOPs" section 2.B; the
Mixture-of-Kittens notes, section 4) vs the oracle and the ring-less path.

The ring changes where rows live and the order macrobatches run, not the
arithmetic of a row: every per-macrobatch table must equal the oracle's
schedule of that token window bit for bit; the layer output must be bitwise
the ring-less forward's (and within rel-L2 1e-2 of the fp64 oracle); the
slots left resident must hold, per route, bitwise the ring-less path's HU and
A rows; the backward's dX and dw must be bitwise the ring-less backward's,
its weight gradients (summed per macrobatch, then in ascending macrobatch
order) within 1e-5 of the single-pass ones and 1e-2 of the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from routing_schedule_expert_amd import inputs, ops
from tests.helpers import bits, dev, f64, rel_l2, up
from tests.test_gpu_layer import Layer, check_bwd_full

pytestmark = pytest.mark.gpu
TOL = 1e-2


def ring_fwd(lay: Layer, B: int, S: int) -> ops.RingBuffers:
    r = ops.alloc_ring(lay.d, B, S, dev())
    ops.layer_fwd_ring(lay.d, lay.routes, lay.w, lay.X, lay.W13, lay.W2, r)
    torch.cuda.synchronize()
    return r


def ring_bwd(lay: Layer, r: ops.RingBuffers, G: int = 1):
    d, L, H, I = lay.d, lay.L, lay.H, lay.I
    g = {
        "dX": torch.empty_like(lay.X),
        "dW13": torch.empty((L, 2 * I, H), dtype=torch.float32, device=dev()),
        "dW2": torch.empty((L, H, I), dtype=torch.float32, device=dev()),
        "dw": torch.empty((lay.P, lay.Np, lay.K), dtype=torch.float32, device=dev()),
    }
    ws = torch.empty(ops.ring_workspace_bytes(d, r.mb_tokens, ops.MOE_OP_LAYER_BWD, G), dtype=torch.uint8,
                     device=dev())
    ops.moe_layer_bwd_ring(d, r.mb_tokens, r.slots, lay.dOut, lay.w, lay.X, lay.W13, lay.W2, r.phi, r.route_row,
                           r.seg_off, r.HU, r.A, g["dX"], g["dW13"], g["dW2"], g["dw"], ws, wgrad_group=G)
    torch.cuda.synchronize()
    return g


def check_tables(lay: Layer, r: ops.RingBuffers, B: int):
    tabs = oracle.macrobatch_schedules(lay.h["routes"], lay.L, B, lay.base)
    counts, seg_off = r.counts.cpu().numpy(), r.seg_off.cpu().numpy()
    phi, rr = r.phi.cpu().numpy(), r.route_row.cpu().numpy()
    for m, t in enumerate(tabs):
        np.testing.assert_array_equal(counts[m], t.counts)
        np.testing.assert_array_equal(seg_off[m], t.seg_off)
        np.testing.assert_array_equal(phi[m, : t.npad], t.phi)
        np.testing.assert_array_equal(rr[:, m * B:(m + 1) * B], t.route_row)


def check_resident_slots(lay: Layer, r: ops.RingBuffers, std: ops.FwdBuffers, B: int, S: int):
    """Per route, a resident slot's HU and A rows are the ring-less path's."""
    M = lay.Np // B
    _, resident, _ = oracle.ring_walk(M, S)
    rr, rr_std = r.route_row.cpu().numpy(), std.route_row.cpu().numpy()
    HU, A = bits(r.HU), bits(r.A)
    HU_std, A_std = bits(std.HU), bits(std.A)
    for m, slot in resident.items():
        win, win_std = rr[:, m * B:(m + 1) * B], rr_std[:, m * B:(m + 1) * B]
        mask = win >= 0
        np.testing.assert_array_equal(HU[slot][win[mask]], HU_std[win_std[mask]])
        np.testing.assert_array_equal(A[slot][win[mask]], A_std[win_std[mask]])


@pytest.mark.parametrize("B,S", [(512, 1), (128, 1), (128, 2), (64, 3), (256, 8)])
def test_ring_forward(B, S):
    print(f"[ring] forward B={B} S={S}", flush=True)
    lay = Layer(11, 4, 512, 16, 4, 8, 256, 256, routing="zipf", x_std=1.0, grad=False)
    r = ring_fwd(lay, B, S)
    check_tables(lay, r, B)
    std = lay.fwd(save_xd=False)
    assert torch.equal(r.out, std.out)
    h = lay.h
    out = oracle.layer_fwd_tokens(h["routes"], h["w"], h["X"], h["W13"], h["W2"], L=lay.L, base=lay.base)
    err = rel_l2(f64(r.out).reshape(out.shape), out)
    print(f"[ring] out rel-L2 {err:.2e}", flush=True)
    assert err <= TOL
    check_resident_slots(lay, r, std, B, S)


def test_ring_forward_ragged_and_nonlocal():
    """Experts with no routes in some windows, a nonzero expert base and
    dropped (-1) ids."""
    print("[ring] forward, expert base 5 and dropped ids", flush=True)
    lay = Layer(13, 3, 384, 24, 3, 6, 256, 128, routing="zipf", base=5, x_std=1.0, s=1.5, grad=False)
    rt = lay.h["routes"].copy()
    rt[:, ::7, 0] = -1
    lay.h["routes"] = rt
    lay.routes = up(rt)
    r = ring_fwd(lay, 96, 2)
    check_tables(lay, r, 96)
    std = lay.fwd(save_xd=False)
    assert torch.equal(r.out, std.out)
    check_resident_slots(lay, r, std, 96, 2)


@pytest.mark.parametrize("B,S,G", [(512, 1, 1), (128, 1, 1), (128, 4, 1), (64, 3, 1), (128, 1, 4), (64, 3, 3),
                                   (64, 2, 16)])
def test_ring_backward(B, S, G):
    print(f"[ring] backward B={B} S={S} G={G}", flush=True)
    lay = Layer(12, 4, 512, 16, 4, 8, 256, 256, routing="zipf", x_std=1.0)
    r = ring_fwd(lay, B, S)
    g = ring_bwd(lay, r, G)
    std = lay.fwd()
    gs = lay.bwd(std)
    assert torch.equal(g["dX"], gs["dX"])
    assert torch.equal(g["dw"], gs["dw"])
    for name in ("dW13", "dW2"):
        err = rel_l2(f64(g[name]), f64(gs[name]))
        print(f"[ring] {name} vs single pass rel-L2 {err:.2e}", flush=True)
        assert err <= 1e-5
    check_bwd_full(lay, g)
    g2 = ring_bwd(lay, r, G)  # the slots are read only: a second backward is bitwise the first
    for name in g:
        assert torch.equal(g[name], g2[name]), name


def test_ring_kimi_shape():
    """Kimi-shaped share (8 x 7,168 tokens, 384 experts with 48 local, top-8,
    H=7168, I=2048, balanced routing) in 7 macrobatches of 1,024 tokens per
    partition through 2 slots: tables bit-exact, output bitwise the ring-less
    forward's, the backward's dX and dw bitwise the ring-less backward's, the
    weight gradients (one pass over all 7 macrobatches) within 1e-5 of the
    single table."""
    print("[ring] Kimi shape, 7 macrobatches, 2 slots", flush=True)
    c = dict(P=8, Np=7168, E=384, K=8, L=48, H=7168, I=2048)
    h = inputs.make_layer_inputs_device(5, c["P"], c["Np"], c["E"], c["K"], c["L"], c["H"], c["I"], dev(),
                                        routing="balanced", x_std=1.0, with_grad=True)
    d = ops.make_desc(c["P"], c["Np"], c["K"], c["E"], c["L"], H=c["H"], I=c["I"])
    routes, w = up(h["routes"]), up(h["w"])
    B, S = 1024, 2
    r = ops.alloc_ring(d, B, S, dev())
    ops.layer_fwd_ring(d, routes, w, h["X"], h["W13"], h["W2"], r)
    torch.cuda.synchronize()
    tabs = oracle.macrobatch_schedules(h["routes"], c["L"], B)
    for m in (0, 3, 6):
        np.testing.assert_array_equal(r.seg_off[m].cpu().numpy(), tabs[m].seg_off)
        np.testing.assert_array_equal(r.phi[m, : tabs[m].npad].cpu().numpy(), tabs[m].phi)
    np.testing.assert_array_equal(r.route_row.cpu().numpy(),
                                  np.concatenate([t.route_row for t in tabs], axis=1))
    std = ops.alloc_fwd(d, dev(), save_hu=True, save_xd=True)
    ops.layer_fwd(d, routes, w, h["X"], h["W13"], h["W2"], std)
    torch.cuda.synchronize()
    assert torch.equal(r.out, std.out)
    dX = torch.empty_like(h["X"])
    dW13 = torch.empty((c["L"], 2 * c["I"], c["H"]), dtype=torch.float32, device=dev())
    dW2 = torch.empty((c["L"], c["H"], c["I"]), dtype=torch.float32, device=dev())
    dw = torch.empty((c["P"], c["Np"], c["K"]), dtype=torch.float32, device=dev())
    ws = torch.empty(ops.ring_workspace_bytes(d, B, ops.MOE_OP_LAYER_BWD, 7), dtype=torch.uint8, device=dev())
    ops.moe_layer_bwd_ring(d, B, S, h["dOut"], w, h["X"], h["W13"], h["W2"], r.phi, r.route_row, r.seg_off, r.HU,
                           r.A, dX, dW13, dW2, dw, ws, wgrad_group=7)
    torch.cuda.synchronize()
    del ws, r
    gs = {"dX": torch.empty_like(dX), "dW13": torch.empty_like(dW13), "dW2": torch.empty_like(dW2),
          "dw": torch.empty_like(dw)}
    ws = torch.empty(ops.workspace_bytes(d, ops.MOE_OP_LAYER_BWD), dtype=torch.uint8, device=dev())
    ops.moe_layer_bwd(d, h["dOut"], routes, w, std.phi, std.route_row, std.seg_off, std.Xd, std.HU, std.A,
                      h["W13"], h["W2"], gs["dX"], gs["dW13"], gs["dW2"], gs["dw"], ws)
    torch.cuda.synchronize()
    assert torch.equal(dX, gs["dX"])
    assert torch.equal(dw, gs["dw"])
    for name, t in (("dW13", dW13), ("dW2", dW2)):
        err = float(torch.linalg.vector_norm(t - gs[name]) / torch.linalg.vector_norm(gs[name]))
        print(f"[ring] Kimi {name} vs single pass rel-L2 {err:.2e}", flush=True)
        assert err <= 1e-5
