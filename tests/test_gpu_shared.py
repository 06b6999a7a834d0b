"""Shared expert on the GPU ("Beyond Peak TFLOPs" section 2.C; the
Mixture-of-Kittens notes, section 5) vs the oracle and the routed-only path.

The shared expert's tiles share the routed GEMM launches, so the routed rows
(HU, A, Y) must stay bitwise those of moe_layer_fwd; the shared activations
and outputs must be within rel-L2 1e-2 of the fp64 oracle, with the padding
rows past the last token exactly zero; the layer output (routed combine plus
the shared output, one rounding) within rel-L2 1e-2 of the oracle; repeated
runs bitwise identical.
"""
import numpy as np
import pytest
import torch

import oracle
from routing_schedule_expert_amd import inputs, ops
from tests.helpers import bits, dev, f64, fused_y_rows, on_dev_mask, rel_l2, up, up_bf16
from tests.test_gpu_layer import Layer

pytestmark = pytest.mark.gpu
TOL = 1e-2


def shared_weights(seed, H, Is):
    rng = np.random.default_rng(seed)
    return inputs.normal_bf16(rng, (2 * Is, H), 0.02), inputs.normal_bf16(rng, (H, Is), 0.02)


def run_shared(lay: Layer, W13s, W2s, Is):
    b = ops.alloc_fwd(lay.d, dev(), save_hu=True, save_xd=False)
    sh = ops.alloc_shared(lay.d, Is, dev(), save_hu=True)
    ops.layer_fwd_shared(lay.d, lay.routes, lay.w, lay.X, lay.W13, lay.W2, W13s, W2s, b, sh)
    torch.cuda.synchronize()
    return b, sh


def assert_routed_rows_equal(b, std, routes, L, base):
    """Routed HU, A and Y of the shared-expert forward against moe_layer_fwd's
    (separate launches), bitwise; Y on the rows moe_layer_fwd writes (the rows
    of tokens with one local route go straight to its output there)."""
    npad = int(std.seg_off[-1])
    yw = on_dev_mask(fused_y_rows(routes, L, base, std.phi[:npad].cpu().numpy()))
    for name in ("HU", "A"):
        assert torch.equal(getattr(b, name)[:npad], getattr(std, name)[:npad]), name
    assert torch.equal(b.Y[:npad][yw], std.Y[:npad][yw]), "Y"


@pytest.mark.parametrize("P,Np,Is", [(2, 200, 256), (3, 256, 128)])
def test_shared_forward(P, Np, Is):
    print(f"[shared] P={P} Np={Np} Is={Is}", flush=True)
    lay = Layer(21, P, Np, 8, 2, 4, 256, 128, routing="topk", x_std=1.0, grad=False)
    w13s, w2s = shared_weights(22, 256, Is)
    W13s, W2s = up_bf16(w13s), up_bf16(w2s)
    b, sh = run_shared(lay, W13s, W2s, Is)
    std = lay.fwd(save_xd=False)
    npad = int(std.seg_off[-1])
    assert_routed_rows_equal(b, std, lay.h["routes"], lay.L, lay.base)
    np.testing.assert_array_equal(b.phi[:npad].cpu().numpy(), std.phi[:npad].cpu().numpy())  # rows past Npad unwritten
    h = lay.h
    ntok = P * Np
    r = oracle.expert_ffn_rows(np.array([0, ntok], np.int32), h["X"].reshape(ntok, -1), w13s[None], w2s[None])
    for name, t in (("HU", sh.HUs), ("A", sh.As), ("Y", sh.Ys)):
        err = rel_l2(f64(t[:ntok]), r[name])
        print(f"[shared] {name}s rel-L2 {err:.2e}", flush=True)
        assert err <= TOL, name
        assert not f64(t[ntok:]).any(), name  # padding rows past the last token
    out = oracle.layer_fwd_tokens_shared(h["routes"], h["w"], h["X"], h["W13"], h["W2"], w13s, w2s, L=lay.L)
    err = rel_l2(f64(b.out).reshape(out.shape), out)
    print(f"[shared] out rel-L2 {err:.2e}", flush=True)
    assert err <= TOL
    b2, sh2 = run_shared(lay, W13s, W2s, Is)
    assert torch.equal(b.out, b2.out) and torch.equal(sh.Ys, sh2.Ys)


def test_shared_nonzero_base_and_dropped_ids():
    """Local experts [6, 10) of 12 with dropped (-1) slots: routed rows bitwise
    the routed-only path's, the output within rel-L2 1e-2 of the oracle."""
    print("[shared] expert base 6, dropped ids", flush=True)
    lay = Layer(25, 3, 200, 12, 3, 4, 256, 128, routing="zipf", base=6, x_std=1.0, grad=False)
    rt = lay.h["routes"].copy()
    rt[:, ::3, 0] = -1
    lay.h["routes"] = rt
    lay.routes = up(rt)
    w13s, w2s = shared_weights(26, 256, 128)
    b, sh = run_shared(lay, up_bf16(w13s), up_bf16(w2s), 128)
    std = lay.fwd(save_xd=False)
    npad = int(std.seg_off[-1])
    assert_routed_rows_equal(b, std, lay.h["routes"], lay.L, lay.base)
    h = lay.h
    out = oracle.layer_fwd_tokens_shared(h["routes"], h["w"], h["X"], h["W13"], h["W2"], w13s, w2s, L=lay.L,
                                         base=lay.base)
    err = rel_l2(f64(b.out).reshape(out.shape), out)
    print(f"[shared] out rel-L2 {err:.2e}", flush=True)
    assert err <= TOL


def test_shared_only_tokens_without_local_routes():
    """No local route anywhere: the output is the shared expert alone."""
    lay = Layer(23, 2, 128, 8, 2, 4, 256, 128, routing="topk", x_std=1.0, grad=False)
    rt = np.full_like(lay.h["routes"], 7)  # every id outside [0, 4)
    lay.h["routes"] = rt
    lay.routes = up(rt)
    w13s, w2s = shared_weights(24, 256, 128)
    b, sh = run_shared(lay, up_bf16(w13s), up_bf16(w2s), 128)
    assert torch.equal(b.out.view(-1, 256), sh.Ys[: 2 * 128])


def test_shared_kimi_sampled():
    """Kimi-shaped share (8 x 7,168 tokens, 384 experts with 48 local, top-8,
    H=7168, I=2048, balanced routing) with a shared expert of Is=2048: routed
    rows bitwise the routed-only path's, sampled tokens vs the oracle."""
    print("[shared] Kimi shape", flush=True)
    c = dict(P=8, Np=7168, E=384, K=8, L=48, H=7168, I=2048)
    Is = 2048
    h = inputs.make_layer_inputs_device(5, c["P"], c["Np"], c["E"], c["K"], c["L"], c["H"], c["I"], dev(),
                                        routing="balanced", x_std=1.0)
    W13s = inputs.normal_bf16_device((2 * Is, c["H"]), 0.02, 91, dev())
    W2s = inputs.normal_bf16_device((c["H"], Is), 0.02, 92, dev())
    d = ops.make_desc(c["P"], c["Np"], c["K"], c["E"], c["L"], H=c["H"], I=c["I"])
    routes, w = up(h["routes"]), up(h["w"])
    b = ops.alloc_fwd(d, dev(), save_hu=True, save_xd=False)
    sh = ops.alloc_shared(d, Is, dev())
    ops.layer_fwd_shared(d, routes, w, h["X"], h["W13"], h["W2"], W13s, W2s, b, sh)
    std = ops.alloc_fwd(d, dev(), save_hu=True, save_xd=False)
    ops.layer_fwd(d, routes, w, h["X"], h["W13"], h["W2"], std)
    torch.cuda.synchronize()
    npad = int(std.seg_off[-1])
    assert_routed_rows_equal(b, std, h["routes"], c["L"], 0)
    rng = np.random.default_rng(4)
    toks = np.sort(rng.choice(c["P"] * c["Np"], 128, replace=False))
    X, W13, W2 = bits(h["X"]), bits(h["W13"]), bits(h["W2"])
    w13s, w2s = bits(W13s), bits(W2s)
    ref = oracle.layer_fwd_tokens_shared(h["routes"], h["w"], X, W13, W2, w13s, w2s, L=c["L"], tokens=toks)
    tk = torch.from_numpy(toks).to(dev())
    err = rel_l2(f64(b.out.view(-1, c["H"])[tk]), ref)
    print(f"[shared] Kimi out rel-L2 {err:.2e}", flush=True)
    assert err <= TOL
    s_ref = oracle.shared_ffn_tokens(X, w13s, w2s, tokens=toks)
    err = rel_l2(f64(sh.Ys[tk]), s_ref)
    print(f"[shared] Kimi Ys rel-L2 {err:.2e}", flush=True)
    assert err <= TOL
